// Backward of the layer forward: the gradients of sum(out * dO) with the
// selection held fixed, for bf16 layers.
//
// The training step on the pages compiles forward, backward and optimiser
// together and recomputes activations in the backward pass instead of
// storing them ("Small models, sparse experts", section "Tuning the training
// loop"); the backward below follows that: it re-runs the route and the
// dispatch (with the logits kept), recomputes each expert's gate and up
// pre-activations, and never materialises the forward's expert outputs.
// With g the gate of a (token, slot) pair, rows r of expert e in sorted order,
// t its token, z_g / z_u its pre-activations and a = silu(z_g) z_u:
//
//   da'[r]      = W_d[e]^T dO[t]                      (bwd_gemm, PROB_DA; stored, bf16)
//   z[r]        = x[t] W_g|u[e]^T                     (PROB_Z, never stored: its
//                 epilogue forms g a, dz and the dG partial sums from z and da')
//   dG[t, slot] = da'[r] . a[r]      (= dO[t] . y[r]; partial sums per 32 units)
//   dz_g, dz_u  = g da' z_u silu'(z_g), g da' silu(z_g)
//   dW_d[e]     = sum_r dO[t] (g a[r])^T              (PROB_DWD)
//   dW_g|u[e]   = sum_r dz_g|u[r] x[t]^T              (PROB_DWGU)
//   dx rows     = dz_g W_g[e] + dz_u W_u[e]           (PROB_DXR)
//   dL          = the gate-to-logit derivative of dG  (router_bwd_kernel)
//   dX[t]       = dL[t] W_r (+ shared gate term)       (PROB_DXROUTER)
//                 + sum_slots dx rows (+ shared dx row)  (dx_finish_kernel)
//   dW_r        = dL^T X                              (PROB_DWROUTER)
//
// The shared expert is the same arithmetic on every token with the gate
// sigmoid(w_s . x) (or 1), and its gate's gradient w_s gets dL_s = dG_s c (1 - c).
//
// With at least 256 rows per expert on average, z and the dx rows instead
// run on the forward's 256 x 256 grouped GEMM as its third and fourth kinds
// (the same epilogues, expert_gemm.hip), from a 256-row tile table of the
// same dispatch.
//
// Every other product is one kernel, bwd_gemm<PROB>: 128 x 128 output tiles per
// 256-thread workgroup (4 waves of 64 x 64 on v_mfma_f32_16x16x32_bf16), K in
// 32-deep stages streamed by direct global->LDS loads through a ring of two or
// three stages (by product). An operand stored with K contiguous is read out of LDS with 16-byte
// reads; one stored with K as its row index (the weight gradients reduce
// over rows; the weights are read along their output dimension for the
// input gradients) lands as it is stored and is transposed by the fragment
// reads themselves (ds_read_b64_tr_b16). Routed rows of x and dO are read
// through their token (rtok[r] = perm[r] / k, one small kernel): once per
// tile where the rows are the output rows, and by scalar loads one stage
// ahead where they are the reduction (the weight gradients). Every epilogue
// stages its outputs through the then idle ring and stores 16 bytes per lane.

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int NT_ = 256;  // threads per workgroup
constexpr int TM = 128, TN = 128, TK = 32;
constexpr int CH = TM * TK / 8 / NT_;       // 16-byte chunks per thread per operand and stage
constexpr int LPS = 2 * CH;                 // DMA loads per thread per stage
static_assert(TM == TN && CH == 2, "the chunk mappings assume 128 x 32 stages");
static_assert(LPS < 64, "vmcnt range");
constexpr int kRouterKChunk = kBwdRouterChunk;  // tokens per partial of dW_r

enum : int {
  PROB_Z = 0,         // z = x W_{g|u}^T (gate/up pre-activations, interleaved 64-wide)
  PROB_DA = 1,        // da' = dO W_d
  PROB_DWD = 2,       // dW_d = dO^T (g a)
  PROB_DWGU = 3,      // dW_{g|u} = dz^T x
  PROB_DXR = 4,       // dx rows = dz W_{g|u}
  PROB_DXROUTER = 5,  // dX = dL W_r + sum of dx rows (+ shared terms)
  PROB_DWROUTER = 6,  // dW_r = dL^T x
};

// Stored-matrix orientation of each operand: true when the operand's K index
// is the contiguous one (A: [M][K], B: [N][K] rows).
template <int PROB> constexpr bool a_kcontig() {
  return PROB == PROB_Z || PROB == PROB_DA || PROB == PROB_DXR || PROB == PROB_DXROUTER;
}
template <int PROB> constexpr bool b_kcontig() { return PROB == PROB_Z; }

struct Tile {
  int e;           // expert, -1 for the shared expert or a dense product
  int m0, n0;      // first output row / column of the tile
  int mlim, nlim;  // valid rows / columns in the tile
  int row0;        // first sorted row (routed row tiles) or first token
  int k0, k1;      // K range (stored-row indices for K-as-row operands)
};

// Workgroup b runs on XCD b mod 8 (workgroups are dispatched round robin
// over the 8 XCDs). For the row products (z, d_hidden, dx rows) whose
// per-expert weight operand fits one XCD's 4 MB L2, each XCD gets one
// contiguous range of the n real tiles, so the column tiles of a row tile
// (which read the same rows) and the row tiles of an expert (which read the
// same weights) share that L2; numbered straight through, column tile k of
// a row tile fell to XCD k mod 8 and every XCD fetched the rows again.
// With larger weights (or for the weight gradients, whose tile work grows
// with the expert's rows) the straight order spreads each expert's weights
// and work over all XCDs and is faster. Returns -1 for workgroups past the
// real tiles of an upper-bound grid.
__device__ __forceinline__ int xcd_tile(int b, int n) {
  if (b >= n) return -1;
  const int x = b & 7, j = b >> 3;
  const int q = n >> 3, rem = n & 7;
  return (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + j;
}

template <int PROB>
__device__ bool decode(const BwdParams& p, Tile& t) {
  int b = blockIdx.x;
  const bool sh = p.shared;
  const int H = sh ? p.hs : p.h;
  if constexpr (PROB == PROB_Z || PROB == PROB_DA || PROB == PROB_DXR) {
    // rows of one expert (routed: through the tile table; shared: all tokens)
    const int ncols = PROB == PROB_Z ? 2 * H : (PROB == PROB_DA ? H : p.d);
    const int NT = (ncols + TN - 1) / TN;
    if (p.xcd_rows) {
      b = xcd_tile(b, NT * (sh ? (p.T + TM - 1) / TM : p.meta[0]));
      if (b < 0) return false;
    }
    const int q = b / NT, nt = b - q * NT;
    t.n0 = nt * TN;
    t.nlim = min(TN, ncols - t.n0);
    t.m0 = 0;
    if (sh) {
      t.e = -1;
      t.row0 = q * TM;
      if (t.row0 >= p.T) return false;
      t.mlim = min(TM, p.T - t.row0);
    } else {
      if (q >= p.meta[0]) return false;
      const int e = p.tile_e[q];
      t.e = e;
      t.row0 = p.offsets[e] + (q - p.exp_tile0[e]) * TM;
      t.mlim = min(TM, p.offsets[e + 1] - t.row0);
      if (t.mlim <= 0) return false;
    }
    t.k0 = 0;
    t.k1 = PROB == PROB_Z ? p.d : (PROB == PROB_DA ? p.d : 2 * H);
    return true;
  } else if constexpr (PROB == PROB_DWD || PROB == PROB_DWGU) {
    const int M = PROB == PROB_DWD ? p.d : 2 * H;
    const int N = PROB == PROB_DWD ? H : p.d;
    const int MT = (M + TM - 1) / TM, NT = (N + TN - 1) / TN;
    const int per = MT * NT;
    const int e = b / per;
    const int r = b - e * per;
    const int mt = r / NT, nt = r - mt * NT;
    t.m0 = mt * TM; t.n0 = nt * TN;
    t.mlim = min(TM, M - t.m0); t.nlim = min(TN, N - t.n0);
    t.row0 = 0;
    if (sh) {
      if (e != 0) return false;
      t.e = -1; t.k0 = 0; t.k1 = p.T;
    } else {
      if (e >= p.E) return false;
      t.e = e; t.k0 = p.offsets[e]; t.k1 = p.offsets[e + 1];
    }
    return true;
  } else if constexpr (PROB == PROB_DXROUTER) {
    // dense product over tokens
    const int NT = (p.d + TN - 1) / TN;
    const int mt = b / NT, nt = b - mt * NT;
    t.m0 = mt * TM; t.n0 = nt * TN;
    if (t.m0 >= p.T) return false;
    t.mlim = min(TM, p.T - t.m0); t.nlim = min(TN, p.d - t.n0);
    t.e = -1; t.row0 = t.m0;
    t.k0 = 0;
    t.k1 = p.Epad;
    return true;
  } else {
    // dW_r: the token reduction split into chunks of kRouterKChunk, each
    // chunk's tile written to its own partial slab (summed in chunk order)
    const int MT = (p.E + TM - 1) / TM, NT = (p.d + TN - 1) / TN;
    const int per = MT * NT;
    const int ch = b / per;
    const int r = b - ch * per;
    const int mt = r / NT, nt = r - mt * NT;
    t.m0 = mt * TM; t.n0 = nt * TN;
    t.mlim = min(TM, p.E - t.m0); t.nlim = min(TN, p.d - t.n0);
    t.e = ch; t.row0 = 0;
    t.k0 = ch * kRouterKChunk;
    if (t.k0 >= p.T) return false;
    t.k1 = min(p.T, t.k0 + kRouterKChunk);
    return true;
  }
}

// ---- operand addressing --------------------------------------------------
// Every address is clamped in bounds (loads past a range reread valid data);
// the A operand's K tail is zeroed in LDS after it lands, so the products
// past K vanish, and rows or columns past M or N are never stored. Routed
// token rows (x, dO) are addressed by issue_op from the tokens it is given;
// a_src / b_src serve every other operand and the shared expert's.
//
// K-contiguous operands: the 16-byte chunk at tile row i, K index k.
// K-as-row operands: the chunk at K index k, tile columns c .. c + 7.

template <int PROB>
__device__ __forceinline__ const uint16_t* a_src(const BwdParams& p, const Tile& t, int i, int k) {
  const bool sh = p.shared;
  const int H = sh ? p.hs : p.h;
  if constexpr (a_kcontig<PROB>()) {
    const int r = t.row0 + (i < t.mlim ? i : 0);
    const int kk = min(k, t.k1 - 8);
    if constexpr (PROB == PROB_DXR) {
      return (sh ? p.dz_s : p.dz) + static_cast<size_t>(r) * (2 * H) + kk;
    } else {  // PROB_DXROUTER
      return p.dlb + static_cast<size_t>(r) * p.Epad + kk;
    }
  } else {
    const int kk = min(k, t.k1 - 1);
    const int c = t.m0 + (i < t.mlim ? i : 0);
    if constexpr (PROB == PROB_DWD) {
      return p.dout + static_cast<size_t>(kk) * p.d + c;  // shared: rows are tokens
    } else if constexpr (PROB == PROB_DWGU) {
      return (sh ? p.dz_s : p.dz) + static_cast<size_t>(kk) * (2 * H) + c;
    } else {  // PROB_DWROUTER: stored rows tokens, columns experts (padded)
      return p.dlb + static_cast<size_t>(kk) * p.Epad + c;
    }
  }
}

template <int PROB>
__device__ __forceinline__ const uint16_t* b_src(const BwdParams& p, const Tile& t, int j, int k) {
  const bool sh = p.shared;
  const int H = sh ? p.hs : p.h;
  if constexpr (PROB == PROB_Z) {
    // tile column j -> hidden unit and projection: 64 hidden units per tile,
    // wave half w = j / 64 takes 32 of them, gate then up
    const int w = j >> 6, c = j & 63;
    const int hu = min((t.n0 >> 1) + w * 32 + (c & 31), H - 1);
    const uint16_t* W = c < 32 ? (sh ? p.ws_gate : p.w_gate) : (sh ? p.ws_up : p.w_up);
    const size_t eoff = sh ? 0 : static_cast<size_t>(t.e) * H * p.d;
    return W + eoff + static_cast<size_t>(hu) * p.d + min(k, t.k1 - 8);
  } else {
    const int n = t.n0 + (j < t.nlim ? j : 0);
    if constexpr (PROB == PROB_DA) {
      // W_d [d, H]: stored rows k (model dim), columns hidden units
      const uint16_t* W = sh ? p.ws_down : p.w_down;
      const size_t eoff = sh ? 0 : static_cast<size_t>(t.e) * p.d * H;
      return W + eoff + static_cast<size_t>(min(k, t.k1 - 1)) * H + n;
    } else if constexpr (PROB == PROB_DWD) {
      // g a rows: stored rows sorted rows / tokens, columns hidden units
      return (sh ? p.gact_s : p.gact) + static_cast<size_t>(min(k, t.k1 - 1)) * H + n;
    } else if constexpr (PROB == PROB_DWGU) {
      return p.x + static_cast<size_t>(min(k, t.k1 - 1)) * p.d + n;  // shared: rows are tokens
    } else if constexpr (PROB == PROB_DWROUTER) {
      return p.x + static_cast<size_t>(min(k, t.k1 - 1)) * p.d + n;
    } else if constexpr (PROB == PROB_DXR) {
      // [W_g; W_u] rows k (2H of them), columns model dim
      const int kk = min(k, t.k1 - 1);
      const bool up = kk >= H;
      const uint16_t* W = up ? (sh ? p.ws_up : p.w_up) : (sh ? p.ws_gate : p.w_gate);
      const size_t eoff = sh ? 0 : static_cast<size_t>(t.e) * H * p.d;
      return W + eoff + static_cast<size_t>(up ? kk - H : kk) * p.d + n;
    } else {  // PROB_DXROUTER: W_r rows (experts; the padded ones reread row E - 1)
      return p.w_router + static_cast<size_t>(min(k, p.E - 1)) * p.d + n;
    }
  }
}

// LDS stage: A then B, TM x TK each. K-contiguous operand: row i (M or N
// index) holds 4 chunks of 8 K values, chunk c at physical position
// c ^ ((i >> 1) & 3). K-as-row operand: row k holds 16 chunks of 8 M (or N)
// values, chunk c at physical position c ^ kr_swz(k); the fragment reads
// then transpose it (ds_read_b64_tr_b16), two reads of four K values per lane.
constexpr int SEL = (TM + TN) * TK;  // bf16 per stage
__device__ __forceinline__ int kr_swz(int k) { return ((k & 3) << 2) | ((k >> 2) & 3); }

// LDS destination of a DMA, hidden from the compiler's load-counter
// tracking: every wait on the ring is explicit and followed by a barrier.
__device__ __forceinline__ lds_void_t* lds_untracked(uint16_t* q) {
  lds_void_t* r = (lds_void_t*)q;
  asm volatile("" : "+s"(r));
  return r;
}

// Products whose operand rows are routed token rows of x or dO: z and the
// hidden-unit gradient (A rows = output rows, fixed per tile), and dW_down
// (A) and dW_gate|up (B), whose K index is the sorted row.
template <int PROB> constexpr bool tok_out_rows() { return PROB == PROB_Z || PROB == PROB_DA; }
template <int PROB> constexpr bool tok_k_rows() { return PROB == PROB_DWD || PROB == PROB_DWGU; }

// Tokens of the 8 sorted rows this wave's lanes load in the stage at K base
// kb (rows kb + 16 i + 4 wave + j), clamped into the expert's range. The
// addresses are wave-uniform: scalar loads, waited by the next stage wait.
typedef int int4v_t __attribute__((ext_vector_type(4)));
struct StageToks {
  int4v_t lo, hi;  // rows kb + 4 wave + j and kb + 16 + 4 wave + j, j = 0..3
};

template <int PROB>
__device__ __forceinline__ void load_toks(const BwdParams& p, const Tile& t, int kb, StageToks& tk) {
  if constexpr (tok_k_rows<PROB>()) {
    if (!p.shared) {
      const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      typedef __attribute__((address_space(4))) const int const_int_t;
      const const_int_t* rt = (const const_int_t*)p.rtok;
      const int r0 = kb + 4 * w, last = t.k1 - 1;
      tk.lo = int4v_t{rt[min(r0, last)], rt[min(r0 + 1, last)], rt[min(r0 + 2, last)],
                      rt[min(r0 + 3, last)]};
      tk.hi = int4v_t{rt[min(r0 + 16, last)], rt[min(r0 + 17, last)], rt[min(r0 + 18, last)],
                      rt[min(r0 + 19, last)]};
    }
  }
}

// Two 16-byte DMA loads per thread per operand and stage: slot q = tid and
// tid + 256 of the stage's 512 chunks. arow: this thread's two A rows (token
// rows of x or dO) of z and the hidden-unit gradient; tk: the stage's tokens
// of dW_down and dW_gate|up (routed experts).
template <int PROB, bool A>
__device__ __forceinline__ void issue_op(const BwdParams& p, const Tile& t, int kbase, uint16_t* st,
                                         const uint16_t* const (&arow)[CH], const StageToks& tk) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr bool KC = A ? a_kcontig<PROB>() : b_kcontig<PROB>();
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int q = i * NT_ + tid;
    const uint16_t* src;
    if constexpr (KC) {
      const int row = q >> 2, c = (q & 3) ^ ((row >> 1) & 3);
      if constexpr (A && tok_out_rows<PROB>())
        src = arow[i] + min(kbase + 8 * c, t.k1 - 8);
      else
        src = A ? a_src<PROB>(p, t, row, kbase + 8 * c) : b_src<PROB>(p, t, row, kbase + 8 * c);
    } else {
      const int kr = q >> 4, c = (q & 15) ^ kr_swz(kr);
      constexpr bool tok_op = tok_k_rows<PROB>() && (A == (PROB == PROB_DWD));
      if (tok_op && !p.shared) {
        // lane's row kr = 16 i + 4 wave + j
        const int jj = (tid >> 4) & 3;
        const int4v_t v = i == 0 ? tk.lo : tk.hi;
        const int t01 = (jj & 1) ? v.y : v.x, t23 = (jj & 1) ? v.w : v.z;
        const int tok = (jj & 2) ? t23 : t01;
        const int col = A ? t.m0 + (8 * c < t.mlim ? 8 * c : 0) : t.n0 + (8 * c < t.nlim ? 8 * c : 0);
        src = (PROB == PROB_DWD ? p.dout : p.x) + static_cast<size_t>(tok) * p.d + col;
      } else {
        src = A ? a_src<PROB>(p, t, 8 * c, kbase + kr) : b_src<PROB>(p, t, 8 * c, kbase + kr);
      }
    }
    __builtin_amdgcn_global_load_lds((gbl_void_t*)src, lds_untracked(st + (i * NT_ + wave * 64) * 8),
                                     16, 0, 0);
  }
}

// The A operand's K positions at or past k1 in the stage of K base kbase:
// zeroed (this thread's two chunks).
template <int PROB>
__device__ __forceinline__ void zero_a_tail(const Tile& t, int kbase, uint16_t* st) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int q = i * NT_ + tid;
    bool past;
    if constexpr (a_kcontig<PROB>()) {
      const int row = q >> 2, c = (q & 3) ^ ((row >> 1) & 3);
      past = kbase + 8 * c >= t.k1;
    } else {
      past = kbase + (q >> 4) >= t.k1;
    }
    if (past) *reinterpret_cast<u32x4_t*>(st + q * 8) = u32x4_t{0u, 0u, 0u, 0u};
  }
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// MFMA operand (16 rows or columns x 32 K, lane l: row l % 16, K values
// 8 (l / 16) .. + 7) of the 16 rows starting at r0.
template <bool KC>
__device__ __forceinline__ bf16x8_t frag(const uint16_t* op, int r0) {
  const int lane = threadIdx.x & 63;
  if constexpr (KC) {
    const int row = r0 + (lane & 15), c = lane >> 4;
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                            op + row * TK + ((c ^ ((row >> 1) & 3)) << 3)));
  } else {
    // transposing reads: in each group of 16 lanes, lane 4 q + r supplies
    // K row 8 g + 4 h + q at columns r0 + 4 r .. + 3, and lane j receives
    // column r0 + j of K rows 8 g + 4 h .. + 3
    const int g = lane >> 4, q = (lane >> 2) & 3, r = lane & 3;
    const int col = r0 + 4 * r;
    v4i16_t v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 8 * g + 4 * h + q;
      const int e = k * TM + (((col >> 3) ^ kr_swz(k)) << 3) + (col & 7);
      v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(op + e));
    }
    struct { v4i16_t lo, hi; } pair = {v[0], v[1]};
    return __builtin_bit_cast(bf16x8_t, pair);
  }
}

__device__ __forceinline__ float row16_sum_x(float v) {
  v += __shfl_xor(v, 1, kWave);
  v += __shfl_xor(v, 2, kWave);
  v += __shfl_xor(v, 4, kWave);
  v += __shfl_xor(v, 8, kWave);
  return v;
}

// Partial sums of the gate gradient per row: one per 32 hidden units (a
// wave's share of a z tile, 2 waves x 64 hidden units per 128-column tile).
__device__ __forceinline__ int bwd_npart(int H) { return 2 * ((2 * H + TN - 1) / TN); }

__device__ __forceinline__ float silu_grad_f32(float z) {
  const float s = sigmoid_f32(z);
  return s * (1.0f + z * (1.0f - s));
}

// LDS stages and workgroups per CU by product: the weight gradients and the
// dx rows run faster with more workgroups per CU than with deeper rings
// (two 16 KB stages, four workgroups); the others keep three stages and
// three workgroups (z stages its bf16 outputs in the 48 KB ring; dW_r's
// registers do not fit four workgroups).
template <int PROB>
constexpr bool bwd_wide() { return PROB == PROB_DWD || PROB == PROB_DWGU || PROB == PROB_DXR; }
template <int PROB>
constexpr int bwd_stages() { return bwd_wide<PROB>() ? 2 : 3; }
template <int PROB>
constexpr int bwd_occupancy() { return bwd_wide<PROB>() ? 4 : 3; }

template <int PROB>
__global__ __launch_bounds__(NT_, bwd_occupancy<PROB>()) void bwd_gemm(BwdParams p) {
  constexpr int S = bwd_stages<PROB>();
  Tile t;
  if (!decode<PROB>(p, t)) return;
  __shared__ __align__(16) uint16_t Ring[S * SEL];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int fr = lane & 15, fq = lane >> 4;
  floatx4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int nsteps = t.k1 > t.k0 ? (t.k1 - t.k0 + TK - 1) / TK : 0;
  const bool ktail = ((t.k1 - t.k0) % TK) != 0;
  const uint16_t* arow[CH] = {};
  if constexpr (tok_out_rows<PROB>()) {
    const uint16_t* X = PROB == PROB_Z ? p.x : p.dout;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int row = (i * NT_ + tid) >> 2;
      const int r = t.row0 + (row < t.mlim ? row : 0);
      arow[i] = X + static_cast<size_t>(p.shared ? r : p.rtok[r]) * p.d;
    }
  }
  StageToks tk{};
  auto issue = [&](uint16_t* st, int kb) {
    issue_op<PROB, true>(p, t, kb, st, arow, tk);
    issue_op<PROB, false>(p, t, kb, st + TM * TK, arow, tk);
  };
  // S stages of DMA in flight ahead of the MFMAs; every thread issues LPS
  // loads per stage (clamped past the end), so each wave's count of
  // outstanding loads is uniform and one vmcnt wait covers a stage. The
  // tokens of a stage's sorted rows are loaded one stage before its issue.
  if (nsteps > 0) {
#pragma unroll
    for (int st = 0; st < S - 1; ++st) {
      load_toks<PROB>(p, t, t.k0 + st * TK, tk);
      issue(Ring + st * SEL, t.k0 + st * TK);
    }
    load_toks<PROB>(p, t, t.k0 + (S - 1) * TK, tk);
  }
  int cur = 0, nxt = S - 1;
  for (int s = 0; s < nsteps; ++s) {
    wait_stage<(S - 2) * LPS>();
    stage_barrier();
    issue(Ring + nxt * SEL, t.k0 + (s + S - 1) * TK);
    load_toks<PROB>(p, t, t.k0 + (s + S) * TK, tk);
    nxt = nxt + 1 == S ? 0 : nxt + 1;
    uint16_t* st = Ring + cur * SEL;
    cur = cur + 1 == S ? 0 : cur + 1;
    if (ktail && s == nsteps - 1) {
      zero_a_tail<PROB>(t, t.k0 + s * TK, st);
      wait_stage<63>();
      stage_barrier();
    }
    bf16x8_t af[4], bfr[4];
#pragma unroll
    for (int mf = 0; mf < 4; ++mf) af[mf] = frag<a_kcontig<PROB>()>(st, wm * 64 + mf * 16);
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) bfr[nf] = frag<b_kcontig<PROB>()>(st + TM * TK, wn * 64 + nf * 16);
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
        acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mf], bfr[nf], acc[mf][nf], 0, 0, 0);
  }
  // the clamped loads past the last stage land before the workgroup's LDS goes
  __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogues: acc[mf][nf][i] is tile row wm*64 + mf*16 + fq*4 + i,
  // tile column wn*64 + nf*16 + fr ----
  const bool sh = p.shared;
  const int H = sh ? p.hs : p.h;
  if constexpr (PROB == PROB_Z) {
    // nf 0, 1: gate of hidden unit hu; nf 2, 3: up of the same unit. With
    // da' of the row (stored by the hidden-unit product, which runs first)
    // and the gate g: g a (bf16, for dW_down), the pre-activation gradients
    // g da' z_u silu'(z_g) and g da' silu(z_g) (bf16), and this wave's
    // partial sum of da' . a over its 32 hidden units (the gate gradient).
    // g a and dz are staged in this wave's 12 KB of the (now idle) stage ring
    // ([64][32] and [64][64] bf16) and stored 16 bytes per lane.
    const uint16_t* dh = sh ? p.dh_s : p.dh;
    uint16_t* ga = sh ? p.gact_s : p.gact;
    uint16_t* dz = sh ? p.dz_s : p.dz;
    float* part = sh ? p.part_s : p.part;
    const int npart = bwd_npart(H);
    const int hu0 = (t.n0 >> 1) + wn * 32;  // first hidden unit of the wave
    const int pcol = (t.n0 >> 6) + wn;      // its 32-unit group
    static_assert(S * SEL >= 4 * 6144, "staging fits the ring");
    uint16_t* gaS = Ring + wave * 6144;  // [64][32]
    uint16_t* dzS = gaS + 2048;          // [64][64]: gate units, then up units
    __syncthreads();  // every wave is done with the ring
    float c[4][4][2];
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
          const int ir = min(wm * 64 + mf * 16 + fq * 4 + i, t.mlim - 1);
          const int hu = min(hu0 + nf * 16 + fr, H - 1);
          c[mf][i][nf] = bf16_to_f32(dh[static_cast<size_t>(t.row0 + ir) * H + hu]);
        }
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = mf * 16 + fq * 4 + i;  // row within the wave
        const int ir = wm * 64 + lr;
        const bool rok = ir < t.mlim;
        const int r = t.row0 + (rok ? ir : 0);
        float g;
        if (sh) g = p.sgate != nullptr ? p.sgate[r] : 1.0f;
        else g = p.gates[p.perm[r]];
        float dot = 0.f;
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
          const int hu = hu0 + nf * 16 + fr;
          const float zg = acc[mf][nf][i], zu = acc[mf][nf + 2][i];
          const float sgm = 1.0f / (1.0f + expf(-zg));  // sigmoid(z_g)
          const float sg = zg * sgm;                     // silu(z_g)
          const float a = sg * zu;
          const float cv = (rok && hu < H) ? c[mf][i][nf] : 0.f;
          dot += cv * a;
          const float da = g * cv;
          const int col = nf * 16 + fr;
          gaS[lr * 32 + col] = f32_to_bf16(g * a);
          dzS[lr * 64 + col] = f32_to_bf16(da * zu * (sgm * (1.0f + zg * (1.0f - sgm))));
          dzS[lr * 64 + 32 + col] = f32_to_bf16(da * sg);
        }
        dot = row16_sum_x(dot);
        if (rok && fr == 0) part[static_cast<size_t>(r) * npart + pcol] = dot;
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // g a: 64 rows x 4 chunks; dz: 64 rows x 8 chunks (4 gate, 4 up)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = j * 64 + lane, lr = q >> 2, ch = q & 3;
      const int ir = wm * 64 + lr;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(gaS + lr * 32 + ch * 8);
      if (ir < t.mlim && hu0 + ch * 8 < H)
        *reinterpret_cast<u32x4_t*>(ga + static_cast<size_t>(t.row0 + ir) * H + hu0 + ch * 8) = v;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = j * 64 + lane, lr = q >> 3, ch = q & 7;
      const int ir = wm * 64 + lr;
      const int u = hu0 + (ch & 3) * 8;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(dzS + lr * 64 + ch * 8);
      if (ir < t.mlim && u < H)
        *reinterpret_cast<u32x4_t*>(dz + static_cast<size_t>(t.row0 + ir) * (2 * H) + (ch < 4 ? 0 : H) + u) = v;
    }
  } else {
    // float32 outputs (da', in bf16; dW_down; dW_gate|up; the dx rows, in pair
    // order so that a token's k rows are adjacent, bf16 for the routed rows like
    // the forward's y rows; dW_r partials; dL W_r plus the shared gate's term, to
    // which dx_finish_kernel adds the dx rows). This wave's 64 x 64 block goes
    // through its 8 KB of the (now idle) stage ring, 32 rows at a time, and
    // out 16 bytes per lane (8 for bf16). In the staging rows,
    // 16-column blocks are XOR-swizzled by bits 2..3 of the row, so the four
    // row groups of a fragment write to distinct banks.
    static_assert(S * SEL * 2 >= 4 * 32 * 64 * 4, "staging fits the ring");
    float* Sw = reinterpret_cast<float*>(Ring) + wave * (32 * 64);
    auto dst_row = [&](int ir) -> float* {
      const int m = t.m0 + ir;
      if constexpr (PROB == PROB_DA) {  // stored in bf16, below
        return nullptr;
      } else if constexpr (PROB == PROB_DWD) {
        float* o = sh ? p.dws_down : p.dw_down + static_cast<size_t>(t.e) * p.d * H;
        return o + static_cast<size_t>(m) * H;
      } else if constexpr (PROB == PROB_DWGU) {
        const bool up = m >= H;
        float* o = up ? (sh ? p.dws_up : p.dw_up) : (sh ? p.dws_gate : p.dw_gate);
        if (!sh) o += static_cast<size_t>(t.e) * H * p.d;
        return o + static_cast<size_t>(up ? m - H : m) * p.d;
      } else if constexpr (PROB == PROB_DXR) {  // the shared expert's rows (routed: bf16, below)
        return p.dx_s + static_cast<size_t>(t.row0 + ir) * p.d;
      } else if constexpr (PROB == PROB_DWROUTER) {
        return p.rpart + (static_cast<size_t>(t.e) * p.E + m) * p.d;
      } else {  // PROB_DXROUTER
        return p.dx + static_cast<size_t>(m) * p.d;
      }
    };
    __syncthreads();  // every wave is done with the ring
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int nf = 0; nf < 4; ++nf)
            Sw[(mm * 16 + fq * 4 + i) * 64 + ((nf ^ fq) << 4) + fr] = acc[2 * pass + mm][nf][i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = j * 64 + lane, row = q >> 4, ch = q & 15;
        float4 v = *reinterpret_cast<const float4*>(
            Sw + row * 64 + ((((ch >> 2) ^ (row >> 2)) & 3) << 4) + (ch & 3) * 4);
        const int ir = wm * 64 + pass * 32 + row, col = wn * 64 + ch * 4;
        if (ir < t.mlim && col < t.nlim) {
          if constexpr (PROB == PROB_DXROUTER) {
            if (p.dpre != nullptr) {
              const float dp = p.dpre[t.m0 + ir];
              const uint16_t* w = p.w_shared_gate + t.n0 + col;
              v.x += dp * bf16_to_f32(w[0]); v.y += dp * bf16_to_f32(w[1]);
              v.z += dp * bf16_to_f32(w[2]); v.w += dp * bf16_to_f32(w[3]);
            }
          }
          if constexpr (PROB == PROB_DA) {  // da' in bf16
            const uint2 o = {static_cast<uint32_t>(f32_to_bf16(v.x)) |
                                 (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16),
                             static_cast<uint32_t>(f32_to_bf16(v.z)) |
                                 (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16)};
            *reinterpret_cast<uint2*>((sh ? p.dh_s : p.dh) + static_cast<size_t>(t.row0 + ir) * H +
                                      t.n0 + col) = o;
            continue;
          }
          if constexpr (PROB == PROB_DXR) {
            if (!sh) {  // routed dx rows in bf16 at the pair's row
              const uint2 o = {static_cast<uint32_t>(f32_to_bf16(v.x)) |
                                   (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16),
                               static_cast<uint32_t>(f32_to_bf16(v.z)) |
                                   (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16)};
              *reinterpret_cast<uint2*>(p.dxr + static_cast<size_t>(p.perm[t.row0 + ir]) * p.d +
                                        t.n0 + col) = o;
              continue;
            }
          }
          if constexpr (PROB == PROB_DWD || PROB == PROB_DWGU) {
            // weight gradients are written once and not read here: past the caches
            __builtin_nontemporal_store(floatx4_t{v.x, v.y, v.z, v.w},
                                        reinterpret_cast<floatx4_t*>(dst_row(ir) + t.n0 + col));
          } else {
            *reinterpret_cast<float4*>(dst_row(ir) + t.n0 + col) = v;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// dx[t] += the token's k routed dx rows (bf16, adjacent, pair order) + its
// shared dx row, in float32: four columns per thread, all loads issued before
// the sum.
__global__ __launch_bounds__(256) void dx_finish_kernel(BwdParams p) {
  const int cq = p.d / 4;
  const size_t i = blockIdx.x * 256ull + threadIdx.x;
  if (i >= static_cast<size_t>(p.T) * cq) return;
  const size_t t = i / cq;
  const int c = static_cast<int>(i - t * cq) * 4;
  float4 v = *reinterpret_cast<const float4*>(p.dx + t * p.d + c);
  const uint16_t* rows = p.dxr + t * p.k * p.d + c;  // bf16, added in float32
  for (int s0 = 0; s0 < p.k; s0 += 8) {
    uint2 r[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s0 + s < p.k) {  // each dx row is read once: past the caches
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t q = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2_t*>(rows + static_cast<size_t>(s0 + s) * p.d));
        r[s] = uint2{q.x, q.y};
      }
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s0 + s < p.k) {
        v.x += __uint_as_float(r[s].x << 16); v.y += __uint_as_float(r[s].x & 0xFFFF0000u);
        v.z += __uint_as_float(r[s].y << 16); v.w += __uint_as_float(r[s].y & 0xFFFF0000u);
      }
  }
  if (p.dx_s != nullptr) {
    const float4 u = *reinterpret_cast<const float4*>(p.dx_s + t * p.d + c);
    v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
  }
  __builtin_nontemporal_store(floatx4_t{v.x, v.y, v.z, v.w},
                              reinterpret_cast<floatx4_t*>(p.dx + t * p.d + c));
}

// One wave per token: the gate gradients dG from the per-tile partial sums,
// then the gate-to-logit derivative of the gate mode, written as a bf16 row
// (zero-padded to Epad) for the two router products; and the shared gate's
// pre-activation gradient.
__global__ __launch_bounds__(256) void router_bwd_kernel(BwdParams p) {
  // per wave (token): each slot's gate gradient, and the slot of each expert
  __shared__ float sdg[4][MOE_MAX_EXPERTS];
  __shared__ int slot_of[4][MOE_MAX_EXPERTS];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tok = blockIdx.x * 4 + w;
  if (tok >= p.T) return;
  const int k = p.k, E = p.E;
  const int npart = bwd_npart(p.h);
  // slot s's gate gradient in lane s mod 64 (k <= E <= MOE_MAX_EXPERTS)
  for (int e = lane; e < E; e += 64) slot_of[w][e] = -1;
  __builtin_amdgcn_wave_barrier();
  float inner = 0.f;
  for (int s = lane; s < k; s += 64) {
    const int r = p.inv[tok * k + s];
    float dg = 0.f;
    for (int q = 0; q < npart; ++q) dg += p.part[static_cast<size_t>(r) * npart + q];
    inner += dg * p.gates[tok * k + s];
    sdg[w][s] = dg;
    slot_of[w][p.ids[tok * k + s]] = s;
    if (p.dgates != nullptr) p.dgates[tok * k + s] = dg;
  }
  inner = wave_sum(inner);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float* L = p.logits + static_cast<size_t>(tok) * E;
  const bool soft_all = p.mode == MOE_SOFTMAX_ALL && !p.renorm;
  float m = -INFINITY, ssum = 0.f;
  if (soft_all) {
    for (int e = lane; e < E; e += 64) m = fmaxf(m, L[e]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    for (int e = lane; e < E; e += 64) ssum += expf(L[e] - m);
    ssum = wave_sum(ssum);
  }
  float ssel = 0.f;  // sigmoid renorm: sum of the chosen affinities
  if (p.mode == MOE_SIGMOID && p.renorm)
    for (int s = 0; s < k; ++s) ssel += sigmoid_f32(L[p.ids[tok * k + s]]);
  for (int e = lane; e < p.Epad; e += 64) {
    float v = 0.f;
    if (e < E) {
      // the slot that chose e, if any (experts of a token are distinct)
      const int s = slot_of[w][e];
      const bool chosen = s >= 0;
      const float dge = chosen ? sdg[w][s] : 0.f;
      const float ge = chosen ? p.gates[tok * k + s] : 0.f;
      if (soft_all) {
        const float pe = expf(L[e] - m) / ssum;
        v = pe * (dge - inner);
      } else if (p.mode == MOE_SIGMOID) {
        if (chosen) {
          const float se = sigmoid_f32(L[e]);
          const float ds = p.renorm ? (dge - inner) / ssel : dge;
          v = ds * se * (1.0f - se);
        }
      } else if (chosen) {
        v = ge * (dge - inner);
      }
      if (p.dlogits != nullptr) p.dlogits[static_cast<size_t>(tok) * E + e] = v;
    }
    p.dlb[static_cast<size_t>(tok) * p.Epad + e] = f32_to_bf16(v);
  }
  if (p.dpre != nullptr && lane == 0) {
    const int nps = bwd_npart(p.hs);
    float dc = 0.f;
    for (int q = 0; q < nps; ++q) dc += p.part_s[static_cast<size_t>(tok) * nps + q];
    const float c = p.sgate[tok];
    p.dpre[tok] = dc * c * (1.0f - c);
  }
}

// dw_router = the dW_r partials summed in chunk order.
// Four adjacent elements per thread (E*d is a multiple of 8, the slabs and
// dw_router 16-byte aligned), the slabs' 16-byte loads issued 8 at a time,
// each element still summed in slab order.
__global__ __launch_bounds__(256) void router_grad_sum_kernel(BwdParams p, int nch) {
  const size_t n = static_cast<size_t>(p.E) * p.d;
  const size_t i = (blockIdx.x * 256ull + threadIdx.x) * 4;
  if (i >= n) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < nch; c0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = *reinterpret_cast<const float4*>(p.rpart + static_cast<size_t>(min(c0 + u, nch - 1)) * n + i);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (c0 + u < nch) {
        s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
      }
    }
  }
  *reinterpret_cast<float4*>(p.dw_router + i) = s;
}

// dw_shared_gate[c] = sum_t dpre[t] x[t, c]: column partial sums over token
// blocks of kSgateTokens (8 columns per thread, 16-byte loads, a block's 8
// rows of loads issued before their products), then their sum in block order.
__global__ __launch_bounds__(256) void sgate_grad_part_kernel(BwdParams p) {
  const int c = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (c >= p.d) return;  // d is a multiple of 8
  const int t0 = blockIdx.y * kSgateTokens, t1 = min(p.T, t0 + kSgateTokens);
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int tb = t0; tb < t1; tb += 8) {
    u32x4_t v[8];
    float w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = min(tb + u, t1 - 1);  // past the block: reread its last row (weight 0)
      v[u] = *reinterpret_cast<const u32x4_t*>(p.x + static_cast<size_t>(t) * p.d + c);
      w[u] = tb + u < t1 ? p.dpre[t] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[2 * j] += w[u] * __uint_as_float(v[u][j] << 16);
        s[2 * j + 1] += w[u] * __uint_as_float(v[u][j] & 0xFFFF0000u);
      }
  }
  float* o = p.sg_part + static_cast<size_t>(blockIdx.y) * p.d + c;
  *reinterpret_cast<float4*>(o) = float4{s[0], s[1], s[2], s[3]};
  *reinterpret_cast<float4*>(o + 4) = float4{s[4], s[5], s[6], s[7]};
}
__global__ __launch_bounds__(256) void sgate_grad_final_kernel(BwdParams p, int nb) {
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= p.d) return;
  float4 s = {0.f, 0.f, 0.f, 0.f};
  for (int b0 = 0; b0 < nb; b0 += 8) {
    float4 v[8];  // eight partials in flight, then added in block order
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = *reinterpret_cast<const float4*>(p.sg_part + static_cast<size_t>(min(b0 + u, nb - 1)) * p.d + c);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (b0 + u < nb) { s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w; }
  }
  *reinterpret_cast<float4*>(p.dw_shared_gate + c) = s;
}

template <int PROB>
hipError_t launch_prob(const BwdParams& p, hipStream_t s) {
  const int H = p.shared ? p.hs : p.h;
  long long nblk = 0;
  if constexpr (PROB == PROB_Z || PROB == PROB_DA || PROB == PROB_DXR) {
    const int ncols = PROB == PROB_Z ? 2 * H : (PROB == PROB_DA ? H : p.d);
    const long long NT = (ncols + TN - 1) / TN;
    const long long MT = p.shared ? (p.T + TM - 1) / TM : p.max_mtiles;
    nblk = NT * MT;
  } else if constexpr (PROB == PROB_DWD || PROB == PROB_DWGU) {
    const int M = PROB == PROB_DWD ? p.d : 2 * H;
    const int N = PROB == PROB_DWD ? H : p.d;
    nblk = static_cast<long long>((M + TM - 1) / TM) * ((N + TN - 1) / TN) * (p.shared ? 1 : p.E);
  } else if constexpr (PROB == PROB_DXROUTER) {
    nblk = static_cast<long long>((p.T + TM - 1) / TM) * ((p.d + TN - 1) / TN);
  } else {
    nblk = static_cast<long long>((p.E + TM - 1) / TM) * ((p.d + TN - 1) / TN) *
           ((p.T + kRouterKChunk - 1) / kRouterKChunk);
  }
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  BwdParams q = p;
  q.xcd_rows = 0;
  if constexpr (PROB == PROB_Z || PROB == PROB_DA || PROB == PROB_DXR) {
    // the expert's weight operand: [d, 2H] (z), [H, d] (d_hidden), [2H, d] (dx rows)
    const long long wbytes = 2LL * p.d * (PROB == PROB_DA ? H : 2 * H);
    q.xcd_rows = wbytes <= (4LL << 20) ? 1 : 0;
  }
  bwd_gemm<PROB><<<static_cast<unsigned>(nblk), NT_, 0, s>>>(q);
  return hipGetLastError();
}

}  // namespace

// Token of each sorted row: rtok[r] = perm[r] / k.
__global__ __launch_bounds__(256) void row_token_kernel(BwdParams p) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r < p.T * p.k) p.rtok[r] = p.perm[r] / p.k;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, size_t n) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += static_cast<size_t>(gridDim.x) * 256)
    p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t nb = (n + 255) / 256;
  fill_zero_kernel<<<static_cast<unsigned>(nb < 4096 ? nb : 4096), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

// The backward after the route and the dispatch: see the sequence at the
// top of this file. p.shared selects nothing here; the shared expert's
// products are launched with a copy whose shared flag is set. ev: null, or
// the caller's stage events (ev[1..7] are recorded here).
hipError_t launch_backward(const BwdParams& p0, hipStream_t s, void* const* ev) {
  BwdParams p = p0;
  p.shared = 0;
  BwdParams q = p0;
  q.shared = 1;
  const bool has_sh = p0.hs > 0;
  hipError_t err;
#define BWD_TRY(x) do { if ((err = (x)) != hipSuccess) return err; } while (0)
  // ev[i]: recorded after backward stage i (ev[0] closes the route stage)
  auto mark = [&](int i) -> hipError_t {
    return (ev == nullptr || ev[i] == nullptr) ? hipSuccess
                                             : hipEventRecord(reinterpret_cast<hipEvent_t>(ev[i]), s);
  };
  row_token_kernel<<<(p.T * p.k + 255) / 256, 256, 0, s>>>(p);
  BWD_TRY(hipGetLastError());
  BWD_TRY(launch_prob<PROB_DA>(p, s));
  if (has_sh) BWD_TRY(launch_prob<PROB_DA>(q, s));
  BWD_TRY(mark(1));
  if (p0.zg != nullptr) {
    BWD_TRY(launch_gemm(*p0.zg, s));  // routed and shared rows in one launch
  } else {
    BWD_TRY(launch_prob<PROB_Z>(p, s));
    if (has_sh) BWD_TRY(launch_prob<PROB_Z>(q, s));
  }
  BWD_TRY(mark(2));
  router_bwd_kernel<<<(p.T + 3) / 4, 256, 0, s>>>(p);
  BWD_TRY(hipGetLastError());
  BWD_TRY(mark(3));
  if (p0.wdn != nullptr) {
    BWD_TRY(launch_gemm(*p0.wdn, s));  // routed and shared in one launch
  } else {
    BWD_TRY(launch_prob<PROB_DWD>(p, s));
    if (has_sh) BWD_TRY(launch_prob<PROB_DWD>(q, s));
  }
  BWD_TRY(mark(4));
  if (p0.wgu != nullptr) {
    BWD_TRY(launch_gemm(*p0.wgu, s));
  } else {
    BWD_TRY(launch_prob<PROB_DWGU>(p, s));
    if (has_sh) BWD_TRY(launch_prob<PROB_DWGU>(q, s));
  }
  BWD_TRY(mark(5));
  if (p0.xg != nullptr) {
    BWD_TRY(launch_gemm(*p0.xg, s));  // routed and shared rows in one launch
  } else {
    BWD_TRY(launch_prob<PROB_DXR>(p, s));
    if (has_sh) BWD_TRY(launch_prob<PROB_DXR>(q, s));
  }
  BWD_TRY(mark(6));
  BWD_TRY(launch_prob<PROB_DXROUTER>(p, s));
  {
    const size_t n = static_cast<size_t>(p.T) * (p.d / 4);
    dx_finish_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(p);
    BWD_TRY(hipGetLastError());
  }
  BWD_TRY(launch_prob<PROB_DWROUTER>(p, s));
  {
    const int nch = (p.T + kRouterKChunk - 1) / kRouterKChunk;
    const size_t n = static_cast<size_t>(p.E) * p.d;
    if (n % 4 != 0) return hipErrorInvalidValue;  // d is a multiple of 8
    router_grad_sum_kernel<<<static_cast<unsigned>((n / 4 + 255) / 256), 256, 0, s>>>(p, nch);
    BWD_TRY(hipGetLastError());
  }
  if (p.dpre != nullptr) {
    const int nb = (p.T + kSgateTokens - 1) / kSgateTokens;
    sgate_grad_part_kernel<<<dim3((p.d / 8 + 255) / 256, nb), 256, 0, s>>>(p);
    BWD_TRY(hipGetLastError());
    sgate_grad_final_kernel<<<(p.d / 4 + 255) / 256, 256, 0, s>>>(p, nb);
    BWD_TRY(hipGetLastError());
  }
  BWD_TRY(mark(7));
#undef BWD_TRY
  return hipSuccess;
}

}  // namespace moe
