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
//   da'[r]      = W_d[e]^T dO[t]                      (bwd_gemm, PROB_DA)
//   dG[t, slot] = da'[r] . a[r]      (= dO[t] . y[r]; partial sums per tile)
//   dz_g, dz_u  = g da' z_u silu'(z_g), g da' silu(z_g)
//   dW_d[e]     = sum_r dO[t] (g a[r])^T              (PROB_DWD)
//   dW_g|u[e]   = sum_r dz_g|u[r] x[t]^T              (PROB_DWGU)
//   dx rows     = dz_g W_g[e] + dz_u W_u[e]           (PROB_DXR)
//   dL          = the gate-to-logit derivative of dG  (router_bwd_kernel)
//   dX[t]       = sum_slots dx rows + dL[t] W_r (+ shared expert terms)  (PROB_DXROUTER)
//   dW_r        = dL^T X                              (PROB_DWROUTER)
//
// The shared expert is the same arithmetic on every token with the gate
// sigmoid(w_s . x) (or 1), and its gate's gradient w_s gets dL_s = dG_s c (1 - c).
//
// Every product is one kernel, bwd_gemm<PROB>: 128 x 128 output tiles per
// 256-thread workgroup (4 waves of 64 x 64 on v_mfma_f32_16x16x32_bf16), K in
// steps of 32 staged through two LDS buffers by ordinary loads into registers
// (issued before the current step's MFMAs, written to LDS after them). An
// operand stored with K contiguous goes to LDS with 16-byte writes; one stored
// with K as its row index (the weight gradients, and the weights read along
// their output dimension) is loaded two K rows at a time and written as
// 32-bit (k, k+1) pairs, which transposes it on the way into LDS. Everything
// out of range loads as zero.

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int NT_ = 256;  // threads per workgroup
constexpr int TM = 128, TN = 128, TK = 32;
constexpr int KS = TK / 32;                 // MFMA K steps per stage
constexpr int CH = TM * TK / 8 / NT_;       // 16-byte chunks per thread per operand and stage
static_assert(TM == TN && CH % 2 == 0, "square tiles, whole chunk pairs");
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

// LDS tile: TM rows of TK bf16 (TK / 8 chunks of 16 bytes, swizzled so the
// 8 rows LDS serves together read 8 distinct bank groups).
__device__ __forceinline__ int lds_off(int row, int chunk) {
  if constexpr (TK == 64) return row * TK + ((chunk ^ (row & 7)) << 3);
  else return row * TK + ((chunk ^ ((row >> 1) & 3)) << 3);
}

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p, bool ok) {
  return ok ? *reinterpret_cast<const u32x4_t*>(p) : u32x4_t{0u, 0u, 0u, 0u};
}

// Row of the shared or routed expert's token for sorted row r.
__device__ __forceinline__ int tok_of(const BwdParams& p, int r) { return p.perm[r] / p.k; }

template <int PROB>
__device__ bool decode(const BwdParams& p, Tile& t) {
  const int b = blockIdx.x;
  const bool sh = p.shared;
  const int H = sh ? p.hs : p.h;
  if constexpr (PROB == PROB_Z || PROB == PROB_DA || PROB == PROB_DXR) {
    // rows of one expert (routed: through the tile table; shared: all tokens)
    const int ncols = PROB == PROB_Z ? 2 * H : (PROB == PROB_DA ? H : p.d);
    const int NT = (ncols + TN - 1) / TN;
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
// K-contiguous operands: pointer to the 16-byte chunk (row i of the tile,
// K index k) or null when out of range. K-as-row operands: pointer to the
// chunk (K index k, tile column c .. c + 7) or null.

template <int PROB>
__device__ __forceinline__ const uint16_t* a_chunk(const BwdParams& p, const Tile& t, int i, int k) {
  const bool sh = p.shared;
  const int H = sh ? p.hs : p.h;
  if constexpr (PROB == PROB_Z || PROB == PROB_DA) {
    if (i >= t.mlim || k >= t.k1) return nullptr;
    const int r = t.row0 + i;
    const int tok = sh ? r : tok_of(p, r);
    const uint16_t* base = PROB == PROB_Z ? p.x : p.dout;
    return base + static_cast<size_t>(tok) * p.d + k;
  } else if constexpr (PROB == PROB_DXR) {
    if (i >= t.mlim || k >= t.k1) return nullptr;
    const uint16_t* dz = sh ? p.dz_s : p.dz;
    return dz + static_cast<size_t>(t.row0 + i) * (2 * H) + k;
  } else if constexpr (PROB == PROB_DXROUTER) {
    if (i >= t.mlim || k >= t.k1) return nullptr;
    return p.dlb + static_cast<size_t>(t.row0 + i) * p.Epad + k;
  } else if constexpr (PROB == PROB_DWD) {
    // stored rows: sorted rows (routed) or tokens (shared); columns: d
    if (k >= t.k1 || i >= t.mlim) return nullptr;
    const int tok = sh ? k : tok_of(p, k);
    return p.dout + static_cast<size_t>(tok) * p.d + t.m0 + i;
  } else if constexpr (PROB == PROB_DWGU) {
    if (k >= t.k1 || i >= t.mlim) return nullptr;
    const uint16_t* dz = sh ? p.dz_s : p.dz;
    return dz + static_cast<size_t>(k) * (2 * H) + t.m0 + i;
  } else {  // PROB_DWROUTER: stored rows tokens, columns experts (padded)
    if (k >= t.k1 || i >= t.mlim) return nullptr;
    return p.dlb + static_cast<size_t>(k) * p.Epad + t.m0 + i;
  }
}

template <int PROB>
__device__ __forceinline__ const uint16_t* b_chunk(const BwdParams& p, const Tile& t, int j, int k) {
  const bool sh = p.shared;
  const int H = sh ? p.hs : p.h;
  if constexpr (PROB == PROB_Z) {
    // tile column j -> hidden unit and projection: 64 hidden units per tile,
    // wave half w = j / 64 takes 32 of them, gate then up
    if (k >= t.k1) return nullptr;
    const int w = j >> 6, c = j & 63;
    const int hu = (t.n0 >> 1) + w * 32 + (c & 31);
    if (hu >= H) return nullptr;
    const uint16_t* W = c < 32 ? (sh ? p.ws_gate : p.w_gate) : (sh ? p.ws_up : p.w_up);
    const size_t eoff = sh ? 0 : static_cast<size_t>(t.e) * H * p.d;
    return W + eoff + static_cast<size_t>(hu) * p.d + k;
  } else if constexpr (PROB == PROB_DA) {
    // W_d [d, H]: stored rows k (model dim), columns hidden units
    if (k >= t.k1 || j >= t.nlim) return nullptr;
    const uint16_t* W = sh ? p.ws_down : p.w_down;
    const size_t eoff = sh ? 0 : static_cast<size_t>(t.e) * p.d * H;
    return W + eoff + static_cast<size_t>(k) * H + t.n0 + j;
  } else if constexpr (PROB == PROB_DWD) {
    // g a rows: stored rows sorted rows / tokens, columns hidden units
    if (k >= t.k1 || j >= t.nlim) return nullptr;
    const uint16_t* ga = sh ? p.gact_s : p.gact;
    return ga + static_cast<size_t>(k) * H + t.n0 + j;
  } else if constexpr (PROB == PROB_DWGU || PROB == PROB_DWROUTER) {
    if (k >= t.k1 || j >= t.nlim) return nullptr;
    const int tok = (PROB == PROB_DWROUTER || sh) ? k : tok_of(p, k);
    return p.x + static_cast<size_t>(tok) * p.d + t.n0 + j;
  } else if constexpr (PROB == PROB_DXR) {
    // [W_g; W_u] rows k (2H of them), columns model dim
    if (k >= t.k1 || j >= t.nlim) return nullptr;
    const bool up = k >= H;
    const uint16_t* W = up ? (sh ? p.ws_up : p.w_up) : (sh ? p.ws_gate : p.w_gate);
    const size_t eoff = sh ? 0 : static_cast<size_t>(t.e) * H * p.d;
    return W + eoff + static_cast<size_t>(up ? k - H : k) * p.d + t.n0 + j;
  } else {  // PROB_DXROUTER: W_r rows (experts), columns model dim
    if (k >= p.E || j >= t.nlim) return nullptr;
    return p.w_router + static_cast<size_t>(k) * p.d + t.n0 + j;
  }
}

// Staging of one K step into registers and from there into LDS.
// K-contiguous: thread q loads chunks q + 256 i (i < CH) of the TM x TK/8
// chunk tile. K-as-row: thread q loads K rows 2 (q % 16 + 16 j) and the next
// one (j < CH / 2) at tile columns 8 (q / 16) .. + 7, and writes them as 8
// (k, k + 1) pairs each.
struct Stage {
  u32x4_t v[CH];
};

template <int PROB, bool A>
__device__ __forceinline__ void load_stage(const BwdParams& p, const Tile& t, int kbase, Stage& s) {
  const int tid = threadIdx.x;
  constexpr bool KC = A ? a_kcontig<PROB>() : b_kcontig<PROB>();
  constexpr int CPR = TK / 8;
  if constexpr (KC) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int q = tid + i * NT_;
      const uint16_t* ptr = A ? a_chunk<PROB>(p, t, q / CPR, kbase + (q % CPR) * 8)
                              : b_chunk<PROB>(p, t, q / CPR, kbase + (q % CPR) * 8);
      s.v[i] = ld16(ptr, ptr != nullptr);
    }
  } else {
    const int c8 = (tid >> 4) * 8;
#pragma unroll
    for (int j = 0; j < CH / 2; ++j) {
      const int k = kbase + 2 * ((tid & 15) + 16 * j);
      const uint16_t* p0 = A ? a_chunk<PROB>(p, t, c8, k) : b_chunk<PROB>(p, t, c8, k);
      const uint16_t* p1 = A ? a_chunk<PROB>(p, t, c8, k + 1) : b_chunk<PROB>(p, t, c8, k + 1);
      s.v[2 * j] = ld16(p0, p0 != nullptr);
      s.v[2 * j + 1] = ld16(p1, p1 != nullptr);
    }
  }
}

template <int PROB, bool A>
__device__ __forceinline__ void store_stage(uint16_t* lds, const Stage& s) {
  const int tid = threadIdx.x;
  constexpr bool KC = A ? a_kcontig<PROB>() : b_kcontig<PROB>();
  constexpr int CPR = TK / 8;
  if constexpr (KC) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int q = tid + i * NT_;
      *reinterpret_cast<u32x4_t*>(lds + lds_off(q / CPR, q % CPR)) = s.v[i];
    }
  } else {
    const int c8 = (tid >> 4) * 8;
#pragma unroll
    for (int j = 0; j < CH / 2; ++j) {
      const int k = 2 * ((tid & 15) + 16 * j);  // even: the pair is one aligned 32-bit word
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // element i of each chunk: bf16 i of the 16 bytes
        const uint32_t lo = (s.v[2 * j][i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
        const uint32_t hi = (s.v[2 * j + 1][i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
        const int row = c8 + i;
        *reinterpret_cast<uint32_t*>(lds + lds_off(row, k >> 3) + (k & 7)) = lo | (hi << 16);
      }
    }
  }
}

__device__ __forceinline__ float row16_sum_x(float v) {
  v += __shfl_xor(v, 1, kWave);
  v += __shfl_xor(v, 2, kWave);
  v += __shfl_xor(v, 4, kWave);
  v += __shfl_xor(v, 8, kWave);
  return v;
}

__device__ __forceinline__ float silu_grad_f32(float z) {
  const float s = sigmoid_f32(z);
  return s * (1.0f + z * (1.0f - s));
}

// Four workgroups per CU where the product fits 128 VGPRs without spilling
// (measured: the z and dx-row products gain 10-15%); the hidden-unit
// gradient and the final dx, whose epilogues need more, keep three.
template <int PROB>
constexpr int bwd_occupancy() { return PROB == PROB_DA || PROB == PROB_DXROUTER ? 3 : 4; }

template <int PROB>
__global__ __launch_bounds__(NT_, bwd_occupancy<PROB>()) void bwd_gemm(BwdParams p) {
  Tile t;
  if (!decode<PROB>(p, t)) return;
  __shared__ __align__(16) uint16_t As[2][TM * TK];
  __shared__ __align__(16) uint16_t Bs[2][TN * TK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int fr = lane & 15, fq = lane >> 4;
  floatx4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int nsteps = t.k1 > t.k0 ? (t.k1 - t.k0 + TK - 1) / TK : 0;
  auto compute = [&](const uint16_t* as, const uint16_t* bs) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int mf = 0; mf < 4; ++mf)
        af[mf] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                  as + lds_off(wm * 64 + mf * 16 + fr, ks * 4 + fq)));
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
        bfr[nf] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                   bs + lds_off(wn * 64 + nf * 16 + fr, ks * 4 + fq)));
#pragma unroll
      for (int mf = 0; mf < 4; ++mf)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
          acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mf], bfr[nf], acc[mf][nf], 0, 0, 0);
    }
  };
  // One K step of loads in flight: step s + 1 loads into registers while
  // step s is multiplied out of one LDS buffer, then goes to the other one.
  Stage sa, sb;
  if (nsteps > 0) {
    load_stage<PROB, true>(p, t, t.k0, sa);
    load_stage<PROB, false>(p, t, t.k0, sb);
    store_stage<PROB, true>(As[0], sa);
    store_stage<PROB, false>(Bs[0], sb);
  }
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    const bool more = s + 1 < nsteps;
    if (more) {
      load_stage<PROB, true>(p, t, t.k0 + (s + 1) * TK, sa);
      load_stage<PROB, false>(p, t, t.k0 + (s + 1) * TK, sb);
    }
    compute(As[cur], Bs[cur]);
    if (more) {
      store_stage<PROB, true>(As[cur ^ 1], sa);
      store_stage<PROB, false>(Bs[cur ^ 1], sb);
    }
    __syncthreads();
  }

  // ---- epilogues: acc[mf][nf][i] is tile row wm*64 + mf*16 + fq*4 + i,
  // tile column wn*64 + nf*16 + fr ----
  const bool sh = p.shared;
  const int H = sh ? p.hs : p.h;
  if constexpr (PROB == PROB_Z) {
    // nf 0, 1: gate of hidden unit hu; nf 2, 3: up of the same unit
    float* z = sh ? p.z_s : p.z;
    uint16_t* ga = sh ? p.gact_s : p.gact;
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ir = wm * 64 + mf * 16 + fq * 4 + i;
        if (ir >= t.mlim) continue;
        const int r = t.row0 + ir;
        float g;
        if (sh) g = p.sgate != nullptr ? p.sgate[r] : 1.0f;
        else g = p.gates[p.perm[r]];
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
          const int hu = (t.n0 >> 1) + wn * 32 + nf * 16 + fr;
          if (hu >= H) continue;
          const float zg = acc[mf][nf][i], zu = acc[mf][nf + 2][i];
          z[static_cast<size_t>(r) * (2 * H) + hu] = zg;
          z[static_cast<size_t>(r) * (2 * H) + H + hu] = zu;
          ga[static_cast<size_t>(r) * H + hu] = f32_to_bf16(g * (silu_f32(zg) * zu));
        }
      }
  } else if constexpr (PROB == PROB_DA) {
    const float* z = sh ? p.z_s : p.z;
    uint16_t* dz = sh ? p.dz_s : p.dz;
    float* part = sh ? p.part_s : p.part;
    const int npart = 2 * ((H + TN - 1) / TN);
    const int pcol = 2 * (t.n0 / TN) + wn;
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ir = wm * 64 + mf * 16 + fq * 4 + i;
        const bool rok = ir < t.mlim;
        const int r = t.row0 + (rok ? ir : 0);
        float g = 1.0f;
        if (sh) g = p.sgate != nullptr ? p.sgate[r] : 1.0f;
        else g = p.gates[p.perm[r]];
        float dot = 0.f;
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          const int j = wn * 64 + nf * 16 + fr;
          if (rok && j < t.nlim) {
            const int hu = t.n0 + j;
            const float zg = z[static_cast<size_t>(r) * (2 * H) + hu];
            const float zu = z[static_cast<size_t>(r) * (2 * H) + H + hu];
            const float c = acc[mf][nf][i];
            const float sg = silu_f32(zg);
            dot += c * (sg * zu);
            const float da = g * c;
            dz[static_cast<size_t>(r) * (2 * H) + hu] = f32_to_bf16(da * zu * silu_grad_f32(zg));
            dz[static_cast<size_t>(r) * (2 * H) + H + hu] = f32_to_bf16(da * sg);
          }
        }
        dot = row16_sum_x(dot);
        if (rok && fr == 0) part[static_cast<size_t>(r) * npart + pcol] = dot;
      }
  } else if constexpr (PROB == PROB_DWD || PROB == PROB_DWGU || PROB == PROB_DXR ||
                       PROB == PROB_DWROUTER) {
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ir = wm * 64 + mf * 16 + fq * 4 + i;
        if (ir >= t.mlim) continue;
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          const int j = wn * 64 + nf * 16 + fr;
          if (j >= t.nlim) continue;
          const float v = acc[mf][nf][i];
          const int m = t.m0 + ir, n = t.n0 + j;
          if constexpr (PROB == PROB_DWD) {
            float* o = sh ? p.dws_down : p.dw_down + static_cast<size_t>(t.e) * p.d * H;
            o[static_cast<size_t>(m) * H + n] = v;
          } else if constexpr (PROB == PROB_DWGU) {
            const bool up = m >= H;
            float* o = up ? (sh ? p.dws_up : p.dw_up) : (sh ? p.dws_gate : p.dw_gate);
            if (!sh) o += static_cast<size_t>(t.e) * H * p.d;
            o[static_cast<size_t>(up ? m - H : m) * p.d + n] = v;
          } else if constexpr (PROB == PROB_DXR) {
            // routed rows go to their (token, slot) pair's row, so that a
            // token's k rows are adjacent for the final sum
            const int orow = sh ? t.row0 + ir : p.perm[t.row0 + ir];
            float* o = sh ? p.dx_s : p.dxr;
            o[static_cast<size_t>(orow) * p.d + n] = v;
          } else {
            p.rpart[(static_cast<size_t>(t.e) * p.E + m) * p.d + n] = v;
          }
        }
      }
  } else {  // PROB_DXROUTER: the final dX rows
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ir = wm * 64 + mf * 16 + fq * 4 + i;
        if (ir >= t.mlim) continue;
        const int tok = t.m0 + ir;
        const float dpre = p.dpre != nullptr ? p.dpre[tok] : 0.f;
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          const int j = wn * 64 + nf * 16 + fr;
          if (j >= t.nlim) continue;
          const int c = t.n0 + j;
          float v = acc[mf][nf][i];
          const float* rows = p.dxr + static_cast<size_t>(tok) * p.k * p.d + c;
#pragma unroll 8
          for (int s = 0; s < p.k; ++s) v += rows[static_cast<size_t>(s) * p.d];
          if (p.dx_s != nullptr) v += p.dx_s[static_cast<size_t>(tok) * p.d + c];
          if (p.dpre != nullptr) v += dpre * bf16_to_f32(p.w_shared_gate[c]);
          p.dx[static_cast<size_t>(tok) * p.d + c] = v;
        }
      }
  }
}

// One wave per token: the gate gradients dG from the per-tile partial sums,
// then the gate-to-logit derivative of the gate mode, written as a bf16 row
// (zero-padded to Epad) for the two router products; and the shared gate's
// pre-activation gradient.
__global__ __launch_bounds__(256) void router_bwd_kernel(BwdParams p) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= p.T) return;
  const int k = p.k, E = p.E;
  const int npart = 2 * ((p.h + TN - 1) / TN);
  // slot s's gate gradient in lane s (k <= 64 is not required: loop)
  float inner = 0.f;
  for (int s = 0; s < k; ++s) {
    const int r = p.inv[tok * k + s];
    float dg = 0.f;
    for (int q = 0; q < npart; ++q) dg += p.part[static_cast<size_t>(r) * npart + q];
    inner += dg * p.gates[tok * k + s];
    if (p.dgates != nullptr && lane == 0) p.dgates[tok * k + s] = dg;
  }
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
      // dG summed over the slots that chose e (at most one: experts are distinct)
      float dge = 0.f, ge = 0.f;
      bool chosen = false;
      for (int s = 0; s < k; ++s) {
        if (p.ids[tok * k + s] == e) {
          const int r = p.inv[tok * k + s];
          float dg = 0.f;
          for (int q = 0; q < npart; ++q) dg += p.part[static_cast<size_t>(r) * npart + q];
          dge = dg;
          ge = p.gates[tok * k + s];
          chosen = true;
        }
      }
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
    const int nps = 2 * ((p.hs + TN - 1) / TN);
    float dc = 0.f;
    for (int q = 0; q < nps; ++q) dc += p.part_s[static_cast<size_t>(tok) * nps + q];
    const float c = p.sgate[tok];
    p.dpre[tok] = dc * c * (1.0f - c);
  }
}

// dw_router = the dW_r partials summed in chunk order.
__global__ __launch_bounds__(256) void router_grad_sum_kernel(BwdParams p, int nch) {
  const size_t n = static_cast<size_t>(p.E) * p.d;
  const size_t i = blockIdx.x * 256ull + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int c = 0; c < nch; ++c) s += p.rpart[static_cast<size_t>(c) * n + i];
  p.dw_router[i] = s;
}

// dw_shared_gate[c] = sum_t dpre[t] x[t, c]: column partial sums over token
// blocks of 256, then their sum in block order.
__global__ __launch_bounds__(256) void sgate_grad_part_kernel(BwdParams p) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= p.d) return;
  const int t0 = blockIdx.y * 256, t1 = min(p.T, t0 + 256);
  float s = 0.f;
  for (int t = t0; t < t1; ++t) s += p.dpre[t] * bf16_to_f32(p.x[static_cast<size_t>(t) * p.d + c]);
  p.sg_part[static_cast<size_t>(blockIdx.y) * p.d + c] = s;
}
__global__ __launch_bounds__(256) void sgate_grad_final_kernel(BwdParams p, int nb) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= p.d) return;
  float s = 0.f;
  for (int b = 0; b < nb; ++b) s += p.sg_part[static_cast<size_t>(b) * p.d + c];
  p.dw_shared_gate[c] = s;
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
  bwd_gemm<PROB><<<static_cast<unsigned>(nblk), NT_, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

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
    return ev == nullptr ? hipSuccess : hipEventRecord(reinterpret_cast<hipEvent_t>(ev[i]), s);
  };
  BWD_TRY(launch_prob<PROB_Z>(p, s));
  if (has_sh) BWD_TRY(launch_prob<PROB_Z>(q, s));
  BWD_TRY(mark(1));
  BWD_TRY(launch_prob<PROB_DA>(p, s));
  if (has_sh) BWD_TRY(launch_prob<PROB_DA>(q, s));
  BWD_TRY(mark(2));
  router_bwd_kernel<<<(p.T + 3) / 4, 256, 0, s>>>(p);
  BWD_TRY(hipGetLastError());
  BWD_TRY(mark(3));
  BWD_TRY(launch_prob<PROB_DWD>(p, s));
  if (has_sh) BWD_TRY(launch_prob<PROB_DWD>(q, s));
  BWD_TRY(mark(4));
  BWD_TRY(launch_prob<PROB_DWGU>(p, s));
  if (has_sh) BWD_TRY(launch_prob<PROB_DWGU>(q, s));
  BWD_TRY(mark(5));
  BWD_TRY(launch_prob<PROB_DXR>(p, s));
  if (has_sh) BWD_TRY(launch_prob<PROB_DXR>(q, s));
  BWD_TRY(mark(6));
  BWD_TRY(launch_prob<PROB_DXROUTER>(p, s));
  BWD_TRY(launch_prob<PROB_DWROUTER>(p, s));
  {
    const int nch = (p.T + kRouterKChunk - 1) / kRouterKChunk;
    const size_t n = static_cast<size_t>(p.E) * p.d;
    router_grad_sum_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(p, nch);
    BWD_TRY(hipGetLastError());
  }
  if (p.dpre != nullptr) {
    const int nb = (p.T + 255) / 256;
    sgate_grad_part_kernel<<<dim3((p.d + 255) / 256, nb), 256, 0, s>>>(p);
    BWD_TRY(hipGetLastError());
    sgate_grad_final_kernel<<<(p.d + 255) / 256, 256, 0, s>>>(p, nb);
    BWD_TRY(hipGetLastError());
  }
  BWD_TRY(mark(7));
#undef BWD_TRY
  return hipSuccess;
}

}  // namespace moe
