// Internal interfaces between the host API (moe_api.cpp) and the HIP kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "../../include/moe.h"

namespace moe {

// Route block: tokens per workgroup of the router / top-k kernel; the
// dispatch histogram is kept per route block. 64 tokens when they all fit
// one block (the dispatch then finishes inside it) or when 64-token blocks
// already give every CU (256) a workgroup; otherwise 32, for twice the
// workgroups (each re-reads the router rows, so not beyond that).
constexpr int kRouteTokensMax = 64;
constexpr int kRouteTokensMin = 32;
inline int route_tokens(int T) {
  return (T <= kRouteTokensMax || T >= 256 * kRouteTokensMax) ? kRouteTokensMax : kRouteTokensMin;
}
// Grouped-GEMM M tile (rows of one expert per workgroup): 128, or 256 when
// experts average at least 256 rows (tile_m in the parameter blocks).
constexpr int kTileM = 128;
constexpr int kTileMLarge = 256;
// Gate/up N tile (hidden units per workgroup; gate and up both) and down N
// tile (model-width columns per workgroup).
constexpr int kTileNGateUp = 64;
constexpr int kTileNDown = 128;

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Tokens per partial sum of the shared gate's weight gradient.
constexpr int kSgateTokens = 32;

// Upper bound on the number of M tiles over all experts:
// sum_e ceil(c_e / BM) <= floor(P / BM) + min(E, P).
inline int max_m_tiles(int P, int E, int bm = kTileM) { return P / bm + (E < P ? E : P) + 1; }

// M tile for a call: 256 rows when the routed rows per expert average at
// least 256 (prefill-shaped batches), else 128.
inline int choose_tile_m(int P, int E) { return P >= kTileMLarge * E ? kTileMLarge : kTileM; }

// Short batches (one route block, T <= 64): the router logits are computed
// by a grid of workgroups (route_part_kernel, 16 columns x 16 tokens each)
// into a [T, ncp] fp32 buffer, then one workgroup finishes the route and the
// dispatch. ncp: logit columns (experts, optional shared-gate row) rounded
// up to 16.
inline int route_part_cols(int E, bool sgate) { return ceil_div(E + (sgate ? 1 : 0), 16) * 16; }

// Grouped GEMMs for batches with few rows per expert (gemm_small_kernel):
// a workgroup holds 16 * NT output columns of one expert's weights over the
// whole reduction in registers, split across NW waves of KS 32-deep MFMA
// steps each. A shape exists when K <= NW * KS * 32 for KS <= 16, NW <= 8.
struct SmallShape {
  int nw, ks;  // 0, 0: no shape fits
};
inline SmallShape small_shape(int K) {
  if (K <= 4 * 4 * 32) return {4, 4};
  if (K <= 4 * 8 * 32) return {4, 8};
  if (K <= 4 * 16 * 32) return {4, 16};
  if (K <= 8 * 16 * 32) return {8, 16};
  return {0, 0};
}
// The small-batch GEMMs run the routed experts when every expert averages at
// most 16 rows, the layer is bf16 and both reductions fit a shape (a shared
// expert, if any, goes through the tiled kernel on its own).
inline bool use_small_gemm(const moe_config& c) {
  return c.dtype == MOE_BF16 && static_cast<long long>(c.T) * c.top_k <= 16LL * c.E &&
         small_shape(c.d).nw > 0 && small_shape(c.h).nw > 0;
}
// 4-bit routed experts are read by the small-batch kernels only, with
// reductions and widths in whole 64-wide scale groups.
inline bool q4_supported(const moe_config& c) {
  return use_small_gemm(c) && c.d % 64 == 0 && c.h % 64 == 0;
}

// Workspace carve-up. Offsets are in bytes from the start of ws.
struct WsLayout {
  size_t blk_hist, lrank, counts, offsets, perm, inv, tile_e, exp_tile0, meta, touched, part;
  size_t ids, gates, sgate;
  size_t end_tables;
  size_t act, act_s, end_act;
  size_t y, ys, end;
};
WsLayout ws_layout(const moe_config& c);

// ---------------------------------------------------------------- kernels --

struct RouteParams {
  const void* x;          // [T, d]
  const void* w_router;   // [E, d]
  const float* bias;      // [E] or null
  const void* w_sgate;    // [d] or null: sigmoid(w_s . x) -> sgate
  int T, d, E, k, mode, renorm;
  int rt;                 // tokens per route block (route_tokens(T))
  int32_t* ids;           // [T, k]
  float* gates;           // [T, k]
  float* logits;          // [T, E] or null
  float* sgate;           // [T] or null
  // dispatch partials (null: route only)
  int32_t* blk_hist;      // [NB, E]
  int32_t* lrank;         // [P]
  // single-block finish (NB == 1): full dispatch inline
  int32_t* counts;        // [E]
  int32_t* offsets;       // [E+1]
  int32_t* perm;          // [P]
  int32_t* inv;           // [P]
  int32_t* tile_e;        // [max tiles]
  int32_t* exp_tile0;     // [E+1]
  int32_t* meta;          // [4]: tiles, touched experts
  int32_t* touched;       // [E][4]: non-empty experts in ascending order: {e, first row, rows, 0}
  int max_tiles;
  int tile_m;
  // split router (route_part_kernel / route_finish_kernel)
  float* part;            // [T][ncp] fp32 logits
  int ncp;
};

// Dispatch from given ids (moe_dispatch): histogram + local ranks.
struct RankParams {
  const int32_t* ids;
  int T, E, k, rt;
  int32_t* blk_hist;
  int32_t* lrank;
};

// Per-expert exclusive scan over route blocks (in place) and expert counts.
struct ScanParams {
  int32_t* blk_hist;  // in: per-block counts; out: per-block base row within the expert
  int NB, E;
  int32_t* counts;    // [E]
};

// perm / inv from the per-block bases; every workgroup rebuilds the expert
// offsets from counts, workgroup 0 also writes offsets and the tile table.
struct ScatterParams {
  const int32_t* ids;
  const int32_t* blk_base;
  const int32_t* lrank;
  int T, E, k, rt;
  int32_t* perm;
  int32_t* inv;
  const int32_t* counts;
  int32_t* offsets;
  int max_tiles, tile_m;
  int32_t* tile_e;
  int32_t* exp_tile0;
  int32_t* meta;
  int32_t* touched;
};

// Tile table from offsets alone (standalone gate_up / down / expert_ffn).
struct TilesParams {
  const int32_t* offsets;
  int E, P, max_tiles, tile_m;
  int32_t* tile_e;
  int32_t* exp_tile0;
  int32_t* meta;
  int32_t* touched;
};

// One grouped GEMM launch. Kind 0: gate/up (+ SiLU product) -> act.
// Kind 1: down -> y. Routed rows come from the tile table; an optional
// dense "shared" group (identity rows 0..shared_T-1) rides in the same launch.
struct GemmParams {
  int kind;
  int dtype;
  // A operand
  const void* a;          // gate/up: x [T, d]; down: act [P, h]
  const int32_t* perm;    // gate/up routed rows: sorted row -> pair (token = pair / k)
  int k;
  int K;                  // reduction length (d for gate/up, h for down)
  // B operand, routed experts
  const void* b0;         // gate/up: w_gate [E, h, d]; down: w_down [E, d, h]
  const void* b1;         // gate/up: w_up   [E, h, d]; down: unused
  // 4-bit routed weights (quant == MOE_QUANT_Q4_G64): b0/b1 hold codes
  // [E, N, K/2] and these the per-64 scale|bias words [E, N, K/64]
  const uint32_t* b0_sb;
  const uint32_t* b1_sb;
  int quant;
  int N;                  // output columns: h (gate/up) or d (down)
  void* out;              // act [P, h] or y [P, d]
  // tile table
  const int32_t* offsets;
  const int32_t* tile_e;
  const int32_t* exp_tile0;
  const int32_t* meta;
  const int32_t* touched;  // [E][4] {e, first row, rows, 0} of the non-empty experts (count in
                           // meta[1]): small-batch kernels
  int E, P;
  int max_mtiles;
  int tile_m;             // M tile of the table (128 or 256)
  int a_rows;             // rows of the gathered A operand (T): token indices are clamped to it
  // shared group
  int shared_T;           // 0: none
  const void* sa;         // gate/up: x; down: act_s [T, hs]
  int sK;                 // d or hs
  const void* sb0;        // ws_gate [hs, d] or ws_down [d, hs]
  const void* sb1;        // ws_up or unused
  int sN;                 // hs or d
  void* sout;             // act_s [T, hs] or ys [T, d]
  // kind 2 (the backward's gate/up product): inputs and outputs of its
  // epilogue, routed rows and the shared group
  const uint16_t* zdh;    // da' [P, h], bf16
  const uint16_t* zdh_s;  // [T, hs]
  const float* zgates;    // [T * k] by pair
  const float* zsgate;    // [T] or null (ungated shared expert: 1)
  uint16_t* zga;          // g a [P, h]
  uint16_t* zga_s;        // [T, hs]
  uint16_t* zdz;          // dz [P, 2h]: gate half, then up half
  uint16_t* zdz_s;        // [T, 2 hs]
  float* zpart;           // [P, znpart] partial sums of da' a, 32 hidden units each
  float* zpart_s;         // [T, znpart_s]
  int znpart, znpart_s;
  // kinds 4 and 5 (the backward's weight gradients): output rows M (sM for
  // the shared group); kind 4 writes rows [0, M / 2) to out and the rest to
  // out2 (sout, sout2)
  int M, sM;
  void* out2;
  void* sout2;
  const int32_t* rtok;    // token of each sorted row (perm / k)
};

struct CombineParams {
  const void* y;        // [P, d]
  const int32_t* inv;   // [P]
  const float* gates;   // [T, k]
  const void* shared;   // [T, d] or null
  const float* shared_scale;  // [T] per-token scale of shared (sigmoid gate) or null
  void* out;            // [T, d]
  int T, d, k, dtype;
  int y_rows;           // rows of y (P): row indices are clamped to it
};

// In-place row scaling: rows[t, :] *= scale[t] (rounded once to dtype).
struct ScaleRowsParams {
  void* rows;           // [T, d]
  const float* scale;   // [T]
  int T, d, dtype;
};

struct RowDotSigmoidParams {
  const void* x;  // [T, d]
  const void* w;  // [d]
  int T, d, dtype;
  float* out;     // [T]
};

// Routing statistics (routing_stats.hip).
struct StatsParams {
  const float* logits;    // [T, E]
  const int32_t* counts;  // [E]
  int T, E, k, mode;
  float alpha;
  float* part;            // [nb][E + 1] partial sums (workspace)
  int nb;                 // stats_blocks(T), at most 256
  int tpb;                // stats_tokens_per_block(T): tokens per block
  float* share;           // [E]
  float* mean_prob;       // [E]
  float* scalars;         // [2]: entropy, aux
};
int stats_blocks(int T);
int stats_tokens_per_block(int T);
hipError_t launch_stats(const StatsParams& p, hipStream_t s);

hipError_t launch_route(const RouteParams& p, int dtype, hipStream_t s);
hipError_t launch_rank(const RankParams& p, hipStream_t s);
hipError_t launch_scan(const ScanParams& p, hipStream_t s);
hipError_t launch_scatter(const ScatterParams& p, hipStream_t s);
// The scan and the scatter in one launch (sp.blk_hist is read, not rewritten;
// sp.counts receives the counts), for at most kDispMaxOwn * 64 route blocks
// and kDispHist histogram entries (every workgroup reads the whole
// histogram); larger dispatches take launch_scan then launch_scatter.
constexpr int kDispMaxOwn = 8;
constexpr long long kDispHist = 65536;
bool dispatch_fused(int NB, int E);
hipError_t launch_dispatch(const ScanParams& sp, const ScatterParams& p, hipStream_t s);
hipError_t launch_tiles(const TilesParams& p, hipStream_t s);
// Compute units of the current device (cached per device; 256 if unknown).
int device_cus();

hipError_t launch_gemm(const GemmParams& p, hipStream_t s);
// route != null (gate/up only, T <= 4 tokens, E <= 64): every workgroup
// derives its expert and rows from route->part (the split router's logits)
// instead of the touched table, and workgroup 0 stores the selection and the
// dispatch tables through *route, as the split router's finish would.
hipError_t launch_gemm_small(const GemmParams& p, hipStream_t s,
                             const RouteParams* route = nullptr);
// A few tokens: the routed down projection and the combine in one launch
// (y is never stored). T <= MOE_DOWN_COMBINE_MAX_T, k <= kDownCombineRows,
// T * k <= kDownCombineMaxRows rows, h a multiple of 64 up to
// kDownCombineMaxK, bf16 layers with activation-dtype experts, or 4-bit
// experts at one token; the shared expert's rows, if any, must already be in
// c.shared. Measured on MI355X at d = 2048, h = 1024, 64 experts, top-8:
// bf16 layers gain 4 / 4 / 1.3 us per layer at 1 / 2 / 4 tokens; 4-bit ones
// gain 1.2 us at one token, none at two and lose 4 at four (their
// vector-ALU code expansion then runs row after row in each wave, where the
// separate 4-bit down kernel puts it on MFMA operands).
#ifndef MOE_DOWN_COMBINE_MAX_T
#define MOE_DOWN_COMBINE_MAX_T 4
#endif
constexpr int kDownCombineRows = 8;
constexpr int kDownCombineMaxRows = 32;
constexpr int kDownCombineMaxK = 1024;
inline bool down_combine_fused(const moe_config& c) {
  return c.T <= MOE_DOWN_COMBINE_MAX_T && (c.T == 1 || c.expert_quant == MOE_QUANT_NONE) &&
         use_small_gemm(c) && c.top_k <= kDownCombineRows &&
         c.T * c.top_k <= kDownCombineMaxRows && c.h % 64 == 0 && c.h <= kDownCombineMaxK;
}
hipError_t launch_down_combine(const GemmParams& p, const CombineParams& c, hipStream_t s);
// The split router's logits kernel alone, then with its finish.
hipError_t launch_route_part(const RouteParams& p, int dtype, hipStream_t s);
hipError_t launch_route_split(const RouteParams& p, int dtype, hipStream_t s);
// The split router's finish runs inside the small-batch gate/up GEMM for
// batches of at most MOE_FUSE_ROUTE_MAX_T tokens. Every gate/up workgroup
// then runs the selection before its weight loads can go out, which pays
// only while the grid is one round of resident workgroups (measured on
// MI355X at d = 2048, h = 1024, 64 experts, top-8: 0.9 us per layer gained
// at one token, 1.5 lost at two, 8 at four; the 4-bit layer likewise).
#ifndef MOE_FUSE_ROUTE_MAX_T
#define MOE_FUSE_ROUTE_MAX_T 1
#endif
inline bool route_in_gate_up(const moe_config& c) {
  return use_small_gemm(c) && c.T <= MOE_FUSE_ROUTE_MAX_T && c.E <= 64;
}
hipError_t launch_combine(const CombineParams& p, hipStream_t s);
hipError_t launch_scale_rows(const ScaleRowsParams& p, hipStream_t s);
hipError_t launch_rowdot_sigmoid(const RowDotSigmoidParams& p, hipStream_t s);

// Backward of the layer (backward.hip). Routing tables come from the route
// and dispatch kernels run with 128-row tiles; buffers are workspace.
struct BwdParams {
  int shared;                 // set by launch_backward for the shared expert's products
  int T, d, E, Epad, h, hs, k, mode, renorm, max_mtiles;
  const int32_t *meta, *tile_e, *exp_tile0, *offsets, *perm, *inv, *ids;
  const float* gates;         // [T, k]
  const float* logits;        // [T, E] (biased in the softmax modes, raw in MOE_SIGMOID)
  const float* sgate;         // [T] sigmoid(w_s . x), or null
  const uint16_t *x, *dout, *w_router, *w_gate, *w_up, *w_down;
  const uint16_t *ws_gate, *ws_up, *ws_down, *w_shared_gate;
  int* rtok;                  // [P] token of each sorted row (perm[r] / k)
  uint16_t *dh, *dh_s;        // [P, h], [T, hs] hidden-unit gradients da' (before the gate), bf16
  uint16_t *gact, *gact_s;    // [P, h], [T, hs] gate * silu(z_g) * z_u, bf16
  uint16_t *dz, *dz_s;        // [P, 2h], [T, 2hs] pre-activation gradients, bf16
  float *part, *part_s;       // [P, 2 ceil(h/64)], [T, 2 ceil(hs/64)] dG partial sums (32 hidden units each)
  uint16_t* dxr;              // [P, d] routed dx rows, bf16 (pair order t * k + slot)
  float* dx_s;                // [T, d] shared dx rows, or null
  uint16_t* dlb;              // [T, Epad] dlogits, bf16, zero-padded
  float* dpre;                // [T] shared gate pre-activation gradient, or null
  float* sg_part;             // [ceil(T/kSgateTokens), d] partial sums of dw_shared_gate
  float* rpart;               // [ceil(T/256), E, d] partial sums of dw_router
  float *dx, *dw_router, *dw_gate, *dw_up, *dw_down;
  float *dws_gate, *dws_up, *dws_down, *dw_shared_gate;
  float *dgates, *dlogits;    // optional copies
  int xcd_rows;               // row products: one contiguous tile range per XCD (set per launch)
  const GemmParams* zg;       // host: the z product on the forward's 256-row tiles, or null
  const GemmParams* xg;       // host: the dx rows on the forward's 256-row tiles, or null
  const GemmParams* wgu;      // host: dW_gate|up on 256 x 256 tiles, or null
  const GemmParams* wdn;      // host: dW_down on 256 x 256 tiles, or null
};
hipError_t launch_backward(const BwdParams& p, hipStream_t s, void* const* ev);
// Tokens per partial sum of dW_r in the backward (the workspace holds
// ceil(T / kBwdRouterChunk) partial [E, d] slabs).
constexpr int kBwdRouterChunk = 256;
// n float zeros at p (a fill kernel, not a memset: safe under graph capture).
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s);

}  // namespace moe
