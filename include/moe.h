/*
 * moe.h -- C ABI of libmoe.so: the sparse mixture-of-experts FFN layer
 * forward on AMD MI355X (gfx950).
 *
 * The layer (the method of "Tutorial 11: Mixture of Experts (MoE)",
 * sections 2-4, and of "Small MoE Architecture, in depth", section "A small
 * MoE layer in PyTorch"):
 *
 *   logits  L = x W_r^T (+ b)                                     [T, E]
 *   ids     the top_k experts per token, ties to the lower index,
 *           slots in descending logit order                        [T, k]
 *   gates   MOE_SOFTMAX_ALL:      softmax over all E, gathered at ids,
 *                                 optionally renormalised to sum 1
 *           MOE_SOFTMAX_SELECTED: softmax over the k selected logits
 *           MOE_SIGMOID:          affinities s = sigmoid(L) of the bias-free
 *                                 logits; ids = the top_k of s + b (b: the
 *                                 selection-only balance bias, when given);
 *                                 gates = s at ids, optionally renormalised
 *                                 ("Small MoE Architecture, in depth",
 *                                 sections "A small MoE layer in PyTorch" and
 *                                 "Balancing without fighting the loss")
 *   dispatch  stable counting sort of the P = T*k pairs p = t*k + j by
 *             expert ids[t, j]: counts[E], offsets[E+1], perm[P] (sorted
 *             row -> pair), inv[P] (pair -> sorted row)
 *   expert  y[r] = W_d[e] (silu(W_g[e] x_t) * (W_u[e] x_t)) for sorted row r
 *           of expert e, t = perm[r] / k                           [P, d]
 *   combine out[t] = sum_{j<k} gates[t, j] y[inv[t*k + j]] (+ shared[t])
 *   shared  shared[t] = (sigmoid(w_s . x_t) if gated) *
 *                       Ws_d (silu(Ws_g x_t) * (Ws_u x_t))
 *
 * Conventions for every entry point:
 *  - Tensors are dense row-major device pointers (HBM), 16-byte aligned.
 *    Activation/weight tensors use cfg->dtype (MOE_F32: float, MOE_BF16:
 *    bfloat16 bit patterns); gates, logits and the router bias are float32;
 *    indices and counts are int32.
 *  - The caller owns every buffer; the library allocates nothing and keeps
 *    no state between calls. Inputs are read-only; outputs must not alias
 *    inputs. Scratch memory is the caller's workspace `ws` of at least
 *    moe_workspace_size_entry(cfg, entry) bytes (256-byte aligned).
 *  - `stream` is a hipStream_t (NULL = the default stream). Kernels are
 *    enqueued on it and the library never synchronises; asynchronous faults
 *    surface at the caller's next synchronisation.
 *  - All argument validation happens on the host before any HIP call, so an
 *    error status means nothing was enqueued. T = 0 returns MOE_OK and
 *    enqueues nothing.
 *  - Errors: MOE_ERR_INVALID_ARG (NULL required pointer; T < 0; d, h or
 *    E <= 0; top_k < 1 or top_k > E; bad enum), MOE_ERR_UNSUPPORTED (d, h or
 *    shared_h not a multiple of 8; E > MOE_MAX_EXPERTS; a pointer not 16-byte
 *    aligned; T*k*d, T*k*h, T*d or T*shared_h at least 2^30 elements), MOE_ERR_WORKSPACE (ws too small or not 256-byte aligned),
 *    MOE_ERR_HIP (a launch failed), MOE_ERR_SCRATCH_LIMIT (the no-alloc
 *    entry point's static workspace is too small for the call).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4
#define MOE_MAX_EXPERTS 256
#define MOE_NUM_STAGES 5 /* route, dispatch, gate_up, down, combine */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4,
  MOE_ERR_SCRATCH_LIMIT = 5
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum { MOE_SOFTMAX_ALL = 0, MOE_SOFTMAX_SELECTED = 1, MOE_SIGMOID = 2 } moe_score_mode;

/* Storage of the routed experts' weights (the shared expert stays in
 * cfg->dtype). MOE_QUANT_Q4_G64: 4-bit affine codes in groups of 64 along the
 * reduction axis ("Small MoE Architecture, in depth", sections "Worked
 * example: the batch-1 budget on a device" and "Quantisation fits MoE
 * unusually well": routed experts at about half a byte per weight, the
 * shared expert at higher precision). A weight matrix [.., N, K] becomes
 * codes [.., N, K/2] bytes (position 2i in the low nibble of byte i) and
 * sb [.., N, K/64] uint32 (bf16 scale s in the low half, bf16 bias b in the
 * high half), w = s * q + b. */
typedef enum { MOE_QUANT_NONE = 0, MOE_QUANT_Q4_G64 = 1 } moe_expert_quant;

/* Which entry point a workspace is sized for (moe_workspace_size_entry). */
typedef enum {
  MOE_ENTRY_LAYER_FORWARD = 0,
  MOE_ENTRY_DISPATCH = 1,
  MOE_ENTRY_GATE_UP = 2,
  MOE_ENTRY_DOWN = 3,
  MOE_ENTRY_EXPERT_FFN = 4,
  MOE_ENTRY_SHARED_EXPERT = 5,
  MOE_ENTRY_ROUTING_STATS = 6,
  MOE_ENTRY_LAYER_BACKWARD = 7
} moe_entry;

/* Shapes and options of one layer call. One (E, h) per call: every routed
 * expert has the same hidden width ("Mixture-of-Experts -- more capacity per
 * byte of weight", section "What's wired today": the same N in every block). */
typedef struct {
  int32_t T;               /* tokens (rows of x) */
  int32_t d;               /* model width */
  int32_t E;               /* routed experts, 1..MOE_MAX_EXPERTS */
  int32_t h;               /* hidden width of each routed expert */
  int32_t top_k;           /* experts per token, 1..E */
  int32_t dtype;           /* moe_dtype of x, weights, act, y, out */
  int32_t mode;            /* moe_score_mode */
  int32_t renormalize;     /* 1: divide the k gates by their sum */
  int32_t has_router_bias; /* 1: b_router [E] float32 is added to the logits
                              (softmax modes), or to the affinities for the
                              choice only (MOE_SIGMOID) */
  int32_t shared_h;        /* hidden width of the shared expert, 0 = none */
  int32_t shared_gate;     /* 1: the shared expert is scaled by sigmoid(w_s . x) */
  int32_t expert_quant;    /* moe_expert_quant of the routed experts */
} moe_config;

/* Weights of one layer, in cfg->dtype unless stated otherwise. */
typedef struct {
  const void* w_router;      /* [E, d] */
  const float* b_router;     /* [E] float32, or NULL when !has_router_bias */
  const void* w_gate;        /* [E, h, d]   (MOE_QUANT_Q4_G64: codes [E, h, d/2]) */
  const void* w_up;          /* [E, h, d]   (MOE_QUANT_Q4_G64: codes [E, h, d/2]) */
  const void* w_down;        /* [E, d, h]   (MOE_QUANT_Q4_G64: codes [E, d, h/2]) */
  const void* ws_gate;       /* [shared_h, d]  (shared_h > 0) */
  const void* ws_up;         /* [shared_h, d]  (shared_h > 0) */
  const void* ws_down;       /* [d, shared_h]  (shared_h > 0) */
  const void* w_shared_gate; /* [d]            (shared_gate) */
  const uint32_t* w_gate_sb; /* [E, h, d/64] scale|bias (MOE_QUANT_Q4_G64, else unused) */
  const uint32_t* w_up_sb;   /* [E, h, d/64] */
  const uint32_t* w_down_sb; /* [E, d, h/64] */
} moe_weights;

/* Gradients of one layer call (moe_layer_backward), all float32 and
 * overwritten. Shapes follow the weights: dw_gate / dw_up [E, h, d],
 * dw_down [E, d, h] (zero for experts no token chose), dw_router [E, d],
 * dx [T, d]; the shared expert's dws_gate / dws_up [shared_h, d],
 * dws_down [d, shared_h] and dw_shared_gate [d] are required when the layer
 * has them and ignored otherwise. dgates [T, k] and dlogits [T, E] are
 * optional copies of the intermediate gate and logit gradients (NULL to
 * skip). */
typedef struct {
  float* dx;
  float* dw_router;
  float* dw_gate;
  float* dw_up;
  float* dw_down;
  float* dws_gate;
  float* dws_up;
  float* dws_down;
  float* dw_shared_gate;
  float* dgates;
  float* dlogits;
} moe_grads;

/* Library ABI version (MOE_ABI_VERSION). */
int32_t moe_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(moe_status s);

/* Host-only check of a configuration (no HIP call). */
moe_status moe_validate_config(const moe_config* cfg);

/* Workspace bytes the given entry point needs for cfg (0 on a bad cfg).
 * It is O(T*k*(d+h) + T*(d+shared_h) + E*T/64), never O(T*h*d): per-token
 * gathered weights are never materialised ("Small models, sparse experts",
 * section "Dispatch decides everything"). */
size_t moe_workspace_size_entry(const moe_config* cfg, int32_t entry);

/* Workspace bytes for moe_layer_forward (the largest of all entries). */
size_t moe_workspace_size(const moe_config* cfg);

/* Dispatch tables that moe_layer_forward leaves in its workspace. */
typedef enum { MOE_TABLE_OFFSETS = 0, MOE_TABLE_PERM = 1, MOE_TABLE_INV = 2 } moe_table;

/* Byte offset, inside a MOE_ENTRY_LAYER_FORWARD workspace sized for cfg, of
 * one of the dispatch tables a moe_layer_forward call writes there: offsets
 * (int32 [E+1]), perm and inv (int32 [T*top_k]), the stable counting sort of
 * "Tutorial 11: Mixture of Experts (MoE)", section 3, step 1. Once the call
 * has completed on its stream the tables hold its dispatch until the next
 * call that uses the same workspace; this lets a caller inspect the fused
 * call's routing. Host arithmetic only (no HIP call). Returns SIZE_MAX for an
 * invalid cfg or table. */
size_t moe_workspace_table_offset(const moe_config* cfg, int32_t table);

/* Router: logits, top-k selection and gates ("Tutorial 11: Mixture of
 * Experts (MoE)", section 2 "The Router"; "Small models, sparse experts",
 * section "How it works", step 3 for MOE_SOFTMAX_SELECTED).
 *   x [T, d], w_router [E, d], b_router [E] f32 (iff has_router_bias)
 *   -> ids [T, k] int32, gates [T, k] f32, logits [T, E] f32 (optional, NULL
 *   to skip; they include b_router in the softmax modes and never in
 *   MOE_SIGMOID). Logits are accumulated in float32; the top-k compares
 *   float32 scores (the logits, or sigmoid(L) + b), ties to the lower expert
 *   index. */
moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* b_router, int32_t* ids, float* gates, float* logits,
                     void* stream);

/* Dispatch: stable counting sort of the T*k (token, slot) pairs by expert
 * ("Tutorial 11: Mixture of Experts (MoE)", section 3, step 1).
 *   ids [T, k] int32 (each in [0, E)) -> counts [E], offsets [E+1], perm [P],
 *   inv [P] (all int32). Rows of one expert keep ascending pair order. */
moe_status moe_dispatch(const moe_config* cfg, const int32_t* ids, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                        size_t ws_bytes, void* stream);

/* Grouped gate/up projection with the SiLU-gated product
 * ("Tutorial 11: Mixture of Experts (MoE)", section 3, step 2):
 *   act[r] = silu(W_g[e] x_t) * (W_u[e] x_t), t = perm[r] / k, for every
 *   sorted row r of expert e (offsets[e] <= r < offsets[e+1]).
 *   x [T, d], perm [P], offsets [E+1], w_gate/w_up [E, h, d] -> act [P, h].
 * moe_gate_up, moe_down and moe_expert_ffn take routed weights in
 * cfg->dtype only: a configuration with expert_quant != MOE_QUANT_NONE
 * returns MOE_ERR_UNSUPPORTED (use moe_layer_forward). */
moe_status moe_gate_up(const moe_config* cfg, const void* x, const int32_t* perm,
                       const int32_t* offsets, const void* w_gate, const void* w_up,
                       void* act, void* ws, size_t ws_bytes, void* stream);

/* Grouped down projection: y[r] = W_d[e] act[r] for sorted row r of expert e.
 *   act [P, h], offsets [E+1], w_down [E, d, h] -> y [P, d] (sorted order). */
moe_status moe_down(const moe_config* cfg, const void* act, const int32_t* offsets,
                    const void* w_down, void* y, void* ws, size_t ws_bytes, void* stream);

/* moe_gate_up then moe_down, with act kept in the workspace:
 *   -> y [P, d] in sorted order, not yet scaled by the gates. */
moe_status moe_expert_ffn(const moe_config* cfg, const void* x, const int32_t* perm,
                          const int32_t* offsets, const void* w_gate, const void* w_up,
                          const void* w_down, void* y, void* ws, size_t ws_bytes,
                          void* stream);

/* Always-on shared expert ("Small MoE Architecture, in depth", section "A
 * small MoE layer in PyTorch"), optionally scaled by sigmoid(w_s . x_t):
 *   x [T, d], ws_gate/ws_up [shared_h, d], ws_down [d, shared_h],
 *   w_shared_gate [d] (NULL: ungated) -> s_out [T, d]. Needs shared_h > 0. */
moe_status moe_shared_expert(const moe_config* cfg, const void* x, const void* ws_gate,
                             const void* ws_up, const void* ws_down,
                             const void* w_shared_gate, void* s_out, void* ws,
                             size_t ws_bytes, void* stream);

/* Gate-weighted combine back to token order ("Tutorial 11: Mixture of
 * Experts (MoE)", section 3, step 3): an additive sum in slot order with
 * float32 accumulation, rounded once to cfg->dtype.
 *   y [P, d] (sorted), inv [P], gates [T, k] f32, shared [T, d] or NULL
 *   -> out [T, d]. */
moe_status moe_combine(const moe_config* cfg, const void* y, const int32_t* inv,
                       const float* gates, const void* shared, void* out, void* stream);

/* Routing statistics ("Mixture-of-Experts -- more capacity per byte of
 * weight", section "What's wired today": the Switch load-balance term;
 * "Small MoE Architecture, in depth", section "Fine-tuning a small MoE":
 * per-expert token share and router entropy), from the router logits as
 * moe_route returns them and the per-expert counts:
 *   share[e]     = counts[e] / (T * top_k)
 *   mean_prob[e] = mean over tokens of p[t, e]
 *   scalars[0]   = mean over tokens of -sum_e p[t, e] ln p[t, e] (nats)
 *   scalars[1]   = alpha * E * sum_e share[e] * mean_prob[e]
 * p = softmax(logits) in the softmax modes, sigmoid(logits) normalised to
 * sum 1 in MOE_SIGMOID. logits [T, E] f32, counts [E] int32 -> share [E],
 * mean_prob [E], scalars [2] (all f32). alpha must be finite and >= 0
 * (MOE_ERR_INVALID_ARG otherwise). Float32 arithmetic, summed in a fixed
 * order (deterministic). Workspace: MOE_ENTRY_ROUTING_STATS. */
moe_status moe_routing_stats(const moe_config* cfg, const float* logits, const int32_t* counts,
                             float alpha, float* share, float* mean_prob, float* scalars,
                             void* ws, size_t ws_bytes, void* stream);

/* The whole layer: route, dispatch, gate/up, down, combine (+ shared).
 *   x [T, d] -> out [T, d]. ids [T, k], gates [T, k] and counts [E] are
 *   optional copies of the routing (NULL to skip).
 *   With cfg->expert_quant == MOE_QUANT_Q4_G64 the routed experts are read in
 *   that format (w_gate_sb, w_up_sb, w_down_sb required) by the small-batch
 *   expert kernels, which serve layers of at most 16 routed rows per expert
 *   on average (T * top_k <= 16 * E) with d and h multiples of 64 and at most
 *   4096, in bf16; other quantised shapes return MOE_ERR_UNSUPPORTED. Per
 *   scale group the kernels form s * sum x (128 + q) + (b - 128 s) * sum x
 *   with bf16 products and float32 accumulation (128 + q is exact in bf16);
 *   at one token the down projection forms s * sum a q + b * sum a in
 *   float32 instead. */
moe_status moe_layer_forward(const moe_config* cfg, const moe_weights* w, const void* x,
                             void* out, int32_t* ids, float* gates, int32_t* counts,
                             void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward that also records stage_events[0] before the first
 * launch and stage_events[i + 1] after stage i (MOE_NUM_STAGES stages:
 * route, dispatch, gate_up, down, combine). stage_events holds
 * MOE_NUM_STAGES + 1 hipEvent_t created by the caller; NULL = untraced, and
 * a NULL entry is not recorded (so one stage can be bracketed alone). A
 * stage whose work a neighbouring launch does brackets no launch: the
 * dispatch at one token (made inside gate/up) and, on the small-batch
 * kernels, the combine at one token and, with activation-dtype experts, at
 * up to four (made inside down). */
moe_status moe_layer_forward_traced(const moe_config* cfg, const moe_weights* w,
                                    const void* x, void* out, int32_t* ids, float* gates,
                                    int32_t* counts, void* ws, size_t ws_bytes,
                                    void* const* stage_events, void* stream);

/* Bytes of the static device array moe_layer_forward_noalloc takes its
 * workspace from (one array per GPU the library runs on, held until the
 * process ends). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* moe_layer_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments as moe_layer_forward minus the workspace, same
 * kernels and the same results; the workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU instead of the caller's ws. The call
 * allocates nothing (no hipMalloc, no hipFree, no allocating library
 * routine). A configuration whose workspace (moe_workspace_size(cfg))
 * exceeds the array returns MOE_ERR_SCRATCH_LIMIT and enqueues nothing: the
 * array serves decode- and serving-sized batches, for example up to T = 1024
 * tokens at top_k = 8, d = 2048, h = 1024 (8192 routed rows, about 48 MiB),
 * not the prefill shapes.
 * The first call on each device (with that device current) looks up the
 * device's address of the array (hipGetSymbolAddress; MOE_ERR_HIP if that
 * fails). Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents (every byte a call reads it has written first, so
 * nothing needs clearing): calls that overlap on one GPU (two streams, or
 * host threads without ordering) race and give wrong results; calls in order
 * on one stream are safe. */
moe_status moe_layer_forward_noalloc(const moe_config* cfg, const moe_weights* w, const void* x,
                                     void* out, int32_t* ids, float* gates, int32_t* counts,
                                     void* stream);

/* Backward of moe_layer_forward: the gradients of sum(out * dout) with the
 * selection held fixed (top-k is piecewise constant in the logits), for the
 * training step of "Small models, sparse experts" (section "Tuning the
 * training loop": forward, backward and optimiser compiled together, with
 * activations recomputed in the backward pass instead of stored). x and
 * dout are [T, d] in cfg->dtype, which must be MOE_BF16; quantised routed
 * experts are MOE_ERR_UNSUPPORTED (they are not trained here). The call
 * recomputes the route, the dispatch and each expert's gate and up
 * pre-activations; it differentiates the gates in the configured mode
 * (softmax over all experts with or without renormalisation, softmax over
 * the selected, sigmoid affinities), the router weights, every expert's
 * SwiGLU and the shared expert with its gate. The router bias and the
 * balance bias are constants and get no gradient. Products run in bf16 on
 * MFMA with float32 accumulation; the intermediate gradients that feed a
 * product (the pre-activation gradients, the gated activations, dlogits)
 * are rounded to bf16 there. Workspace: MOE_ENTRY_LAYER_BACKWARD. Every
 * gradient is written by one workgroup in a fixed order (no atomics): the
 * result is deterministic. */
moe_status moe_layer_backward(const moe_config* cfg, const moe_weights* w, const void* x,
                              const void* dout, const moe_grads* grads, void* ws,
                              size_t ws_bytes, void* stream);

/* Stages of moe_layer_backward_traced: route and dispatch (recomputed), the
 * down-projection gradient into the hidden units, the gate/up
 * pre-activations (recomputed, with the pre-activation gradients formed from
 * them), the gate and logit gradients, dW_down, dW_gate|up, the routed and
 * shared dx rows, and the router products with the final dx. */
#define MOE_NUM_BWD_STAGES 8

/* moe_layer_backward that also records stage_events[0] before the first
 * launch and stage_events[i + 1] after stage i (MOE_NUM_BWD_STAGES stages).
 * stage_events holds MOE_NUM_BWD_STAGES + 1 hipEvent_t created by the
 * caller; NULL = untraced, and a NULL entry is not recorded. With T == 0
 * no event is recorded. */
moe_status moe_layer_backward_traced(const moe_config* cfg, const moe_weights* w,
                                     const void* x, const void* dout, const moe_grads* grads,
                                     void* ws, size_t ws_bytes, void* const* stage_events,
                                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
