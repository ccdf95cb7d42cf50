// Route and dispatch kernels for the sparse MoE layer forward (gfx950).
//
// route: router logits (bf16 MFMA with fp32 accumulation, or fp32 VALU),
//   top-k per token with ties to the lower expert index and slots in
//   descending logit order, softmax gates ("Tutorial 11: Mixture of Experts
//   (MoE)", section 2 "The Router"; "Small models, sparse experts", section
//   "How it works", step 3), and the first half of the counting sort:
//   per-route-block expert histograms and stable in-block ranks.
// scan: per-expert exclusive scan over route blocks -> counts, offsets,
//   per-block base rows and the grouped-GEMM tile table.
// scatter: perm[base + rank] = pair, inv[pair] = row.
// A launch of one route block (T <= 64) finishes the whole dispatch inline.

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int RT = kRouteTokens;  // tokens per route block
constexpr int RK = 64;            // K chunk of the router GEMM
constexpr int RLD = RK + 8;       // padded LDS row (bf16 elements)
constexpr int kMaxE = MOE_MAX_EXPERTS;

// ---------------------------------------------------------------------------
// wave-0 exclusive scan of n <= 256 ints: out[0..n-1] exclusive, out[n] total.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wave_exclusive_scan256(const int* in, int* out, int n) {
  const int lane = lane_id();
  const int b = lane * 4;
  int v0 = b + 0 < n ? in[b + 0] : 0;
  int v1 = b + 1 < n ? in[b + 1] : 0;
  int v2 = b + 2 < n ? in[b + 2] : 0;
  int v3 = b + 3 < n ? in[b + 3] : 0;
  int s = v0 + v1 + v2 + v3;
  int incl = s;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int t = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += t;
  }
  int ex = incl - s;
  if (b + 0 < n) out[b + 0] = ex;
  if (b + 1 < n) out[b + 1] = ex + v0;
  if (b + 2 < n) out[b + 2] = ex + v0 + v1;
  if (b + 3 < n) out[b + 3] = ex + v0 + v1 + v2;
  if (lane == kWave - 1) out[n] = incl;
}

__device__ __forceinline__ int bits_for(int E) { return E > 1 ? 32 - __clz(E - 1) : 0; }

// ---------------------------------------------------------------------------
// Stable ranks of the block's pairs (pair order), block histogram in run[].
// sel[q] = expert of local pair q, q < npairs. Must be called by all NTHR
// threads; wh has one row per wave.
// ---------------------------------------------------------------------------
template <int NTHR>
__device__ void block_rank(const uint8_t* sel, int npairs, int E, int32_t* lrank_out,
                           int (*wh)[kMaxE], int* run) {
  constexpr int NW = NTHR / kWave;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int nbits = bits_for(E);
  for (int e = tid; e < E; e += NTHR) run[e] = 0;
  for (int base = 0; base < npairs; base += NTHR) {
    for (int e = tid; e < E; e += NTHR) {
#pragma unroll
      for (int w = 0; w < NW; ++w) wh[w][e] = 0;
    }
    __syncthreads();
    const int q = base + tid;
    const bool valid = q < npairs;
    const int e = valid ? static_cast<int>(sel[q]) : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(valid && bit);
      peers &= bit ? bb : ~bb;
    }
    const int rank = __popcll(peers & lanemask_lt());
    if (valid && rank == 0) wh[wave][e] = __popcll(peers);
    __syncthreads();
    for (int x = tid; x < E; x += NTHR) {
      int r = run[x];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int c = wh[w][x];
        wh[w][x] = r;
        r += c;
      }
      run[x] = r;
    }
    __syncthreads();
    if (valid) lrank_out[q] = wh[wave][e] + rank;
    __syncthreads();
  }
}

// Tile table writes shared by the scan, tiles and single-block paths:
// mt[e] = ceil(cnt[e] / kTileM) scanned into tp[]; tile_e[i] = owning expert.
__device__ void write_tile_table(const int* tp, int E, int max_tiles, int32_t* tile_e,
                                 int32_t* exp_tile0, int32_t* meta) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int total = min(tp[E], max_tiles);
  for (int e = tid; e <= E; e += nthr) exp_tile0[e] = tp[e];
  for (int i = tid; i < total; i += nthr) {
    int lo = 0, hi = E - 1;  // last e with tp[e] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tp[mid] <= i) lo = mid; else hi = mid - 1;
    }
    tile_e[i] = lo;
  }
  if (tid == 0) meta[0] = total;
}

// ---------------------------------------------------------------------------
// route kernel: 512 threads, 64 tokens. Logits: 8 waves as 4 token groups of
// 16 x 2 column halves; router rows staged through LDS in 64-deep K chunks,
// double-buffered with the next chunk's loads issued before the MFMAs.
// ---------------------------------------------------------------------------
constexpr int RTHR = 512;
constexpr int RNW = RTHR / kWave;

template <int NCH>
struct RouteSmem {
  static constexpr int NC = NCH * 64;  // padded logit columns (E experts + optional shared gate)
  static constexpr int LDL = NC + 1;   // fp32 logit row stride
  static constexpr int kStageBytes = 2 * NC * RLD * 2;  // two K-chunk buffers
  static constexpr int kLogitBytes = RT * LDL * 4;
  static constexpr int kRawBytes = kStageBytes > kLogitBytes ? kStageBytes : kLogitBytes;
  static constexpr int kLoads = NC * 8 / RTHR;  // 16-byte staging loads per thread per chunk
};

template <int NCH>
__device__ void route_logits_bf16(const RouteParams& p, int t0, unsigned char* raw) {
  using S = RouteSmem<NCH>;
  constexpr int NF = NCH * 2;  // 16-column fragments per wave (half of NC)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 3, wn = wave >> 2;
  const uint16_t* X = static_cast<const uint16_t*>(p.x);
  const uint16_t* W = static_cast<const uint16_t*>(p.w_router);
  const uint16_t* WS = static_cast<const uint16_t*>(p.w_sgate);
  uint16_t* stage = reinterpret_cast<uint16_t*>(raw);
  floatx4_t acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const int arow = t0 + wm * 16 + (lane & 15);
  const bool arow_ok = arow < p.T;
  const int kq = (lane >> 4) * 8;

  // staging rows handled by this thread: c = tid + i * RTHR -> row c / 8, chunk c % 8
  const uint16_t* srow[S::kLoads];
#pragma unroll
  for (int i = 0; i < S::kLoads; ++i) {
    const int r = (tid + i * RTHR) >> 3;
    srow[i] = r < p.E ? W + static_cast<size_t>(r) * p.d : (r == p.E ? WS : nullptr);
  }
  const int sch = (tid & 7) * 8;
  u32x4_t pre[S::kLoads];
  u32x4_t apre[2];
  auto gload = [&](int k0) {
    const int kk = k0 + sch;
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) {
      pre[i] = (srow[i] != nullptr && kk < p.d)
                   ? *reinterpret_cast<const u32x4_t*>(srow[i] + kk) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int ka = k0 + s * 32 + kq;
      apre[s] = (arow_ok && ka < p.d)
                    ? *reinterpret_cast<const u32x4_t*>(X + static_cast<size_t>(arow) * p.d + ka)
                    : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
    uint16_t* st = stage + buf * S::NC * RLD;
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) {
      const int r = (tid + i * RTHR) >> 3;
      *reinterpret_cast<u32x4_t*>(st + r * RLD + sch) = pre[i];
    }
  };
  const int nk = (p.d + RK - 1) / RK;
  gload(0);
  sstore(0);
  u32x4_t acur[2] = {apre[0], apre[1]};
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nk) gload((kc + 1) * RK);
    const uint16_t* st = stage + buf * S::NC * RLD;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, acur[s]);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int col = wn * (S::NC / 2) + f * 16 + (lane & 15);
        const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(st + col * RLD + s * 32 + kq);
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, bv), acc[f], 0, 0, 0);
      }
    }
    if (kc + 1 < nk) {
      sstore(buf ^ 1);
      acur[0] = apre[0];
      acur[1] = apre[1];
    }
    __syncthreads();
  }
  float* lg = reinterpret_cast<float*>(raw);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lg[(wm * 16 + (lane >> 4) * 4 + i) * S::LDL + wn * (S::NC / 2) + f * 16 + (lane & 15)] = acc[f][i];
    }
  }
  __syncthreads();
}

template <int NCH>
__device__ void route_logits_f32(const RouteParams& p, int t0, unsigned char* raw) {
  using S = RouteSmem<NCH>;
  const int tid = threadIdx.x;
  const float* X = static_cast<const float*>(p.x);
  const float* W = static_cast<const float*>(p.w_router);
  const float* WS = static_cast<const float*>(p.w_sgate);
  float* lg = reinterpret_cast<float*>(raw);
  for (int idx = tid; idx < RT * S::NC; idx += RTHR) {
    const int r = idx / S::NC, e = idx - r * S::NC, t = t0 + r;
    float s = 0.f;
    const float* wr = e < p.E ? W + static_cast<size_t>(e) * p.d : (e == p.E ? WS : nullptr);
    if (t < p.T && wr != nullptr) {
      const float* xr = X + static_cast<size_t>(t) * p.d;
      for (int i = 0; i < p.d; ++i) s = fmaf(xr[i], wr[i], s);
    }
    lg[r * S::LDL + e] = s;
  }
  __syncthreads();
}

// Top-k, gates, logits and shared-gate outputs for the block's tokens (one
// wave per token, 8 tokens per wave); the selection also goes to sel[] for
// the rank pass.
template <int NCH>
__device__ void route_select(const RouteParams& p, int t0, const float* lg, uint8_t* sel) {
  using S = RouteSmem<NCH>;
  constexpr int TPW = RT / RNW;  // tokens per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E, k = p.k;
  for (int rr = 0; rr < TPW; ++rr) {
    const int r = wave * TPW + rr, t = t0 + r;
    if (t >= p.T) break;
    float v[NCH], ov[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e = c * 64 + lane;
      float val = -INFINITY;
      if (e < E) {
        val = lg[r * S::LDL + e];
        if (p.bias != nullptr) val += p.bias[e];
        if (p.logits != nullptr) p.logits[static_cast<size_t>(t) * E + e] = val;
      }
      v[c] = val;
      ov[c] = val;
    }
    if (p.sgate != nullptr && lane == 0) p.sgate[t] = sigmoid_f32(lg[r * S::LDL + E]);
    float sv[4] = {0.f, 0.f, 0.f, 0.f};
    int si[4] = {0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
      float bv = v[0];
      int bi = lane;
#pragma unroll
      for (int c = 1; c < NCH; ++c) {
        if (v[c] > bv) { bv = v[c]; bi = c * 64 + lane; }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float ovv = __shfl_xor(bv, off, kWave);
        const int oi = __shfl_xor(bi, off, kWave);
        if (ovv > bv || (ovv == bv && oi < bi)) { bv = ovv; bi = oi; }
      }
      if ((bi & 63) == lane) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) if (c == (bi >> 6)) v[c] = -INFINITY;
      }
      if ((j & 63) == lane) {
#pragma unroll
        for (int q = 0; q < 4; ++q) if (q == (j >> 6)) { sv[q] = bv; si[q] = bi; }
      }
    }
    const float m = __shfl(sv[0], 0, kWave);  // slot 0 holds the largest logit
    float es[4];
    float ssel = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      es[q] = 0.f;
      if (q * 64 + lane < k) { es[q] = expf(sv[q] - m); ssel += es[q]; }
    }
    ssel = wave_sum(ssel);
    float denom = ssel;
    if (p.mode == MOE_SOFTMAX_ALL && !p.renorm) {
      float sall = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) if (c * 64 + lane < E) sall += expf(ov[c] - m);
      denom = wave_sum(sall);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = q * 64 + lane;
      if (j < k) {
        p.ids[static_cast<size_t>(t) * k + j] = si[q];
        p.gates[static_cast<size_t>(t) * k + j] = es[q] / denom;
        sel[r * k + j] = static_cast<uint8_t>(si[q]);
      }
    }
  }
}

template <int NCH, bool BF16>
__global__ __launch_bounds__(RTHR) void route_kernel(RouteParams p) {
  using S = RouteSmem<NCH>;
  __shared__ __align__(16) unsigned char raw[S::kRawBytes];
  __shared__ uint8_t sel[RT * kMaxE];
  __shared__ int wh[RNW][kMaxE];
  __shared__ int run[kMaxE + 1];
  __shared__ int scan_a[kMaxE + 1];
  __shared__ int scan_b[kMaxE + 1];
  const int t0 = blockIdx.x * RT;
  if constexpr (BF16) route_logits_bf16<NCH>(p, t0, raw);
  else route_logits_f32<NCH>(p, t0, raw);
  route_select<NCH>(p, t0, reinterpret_cast<const float*>(raw), sel);
  if (p.blk_hist == nullptr && p.counts == nullptr) return;
  __syncthreads();
  const int nt = min(RT, p.T - t0);
  const int npairs = nt * p.k;
  int32_t* lrank = p.lrank + static_cast<size_t>(t0) * p.k;
  block_rank<RTHR>(sel, npairs, p.E, lrank, wh, run);
  const int tid = threadIdx.x;
  if (p.counts == nullptr) {
    for (int e = tid; e < p.E; e += RTHR) p.blk_hist[blockIdx.x * p.E + e] = run[e];
    return;
  }
  // One route block covers every token: finish the dispatch here.
  __syncthreads();
  if (tid < kWave) wave_exclusive_scan256(run, scan_a, p.E);  // offsets
  for (int e = tid; e < p.E; e += RTHR) scan_b[e] = (run[e] + p.tile_m - 1) / p.tile_m;
  __syncthreads();
  if (tid < kWave) wave_exclusive_scan256(scan_b, scan_b, p.E);  // tile prefix (in place per lane)
  __syncthreads();
  for (int e = tid; e < p.E; e += RTHR) { p.counts[e] = run[e]; p.offsets[e] = scan_a[e]; }
  if (tid == 0) p.offsets[p.E] = scan_a[p.E];
  write_tile_table(scan_b, p.E, p.max_tiles, p.tile_e, p.exp_tile0, p.meta);
  for (int q = tid; q < npairs; q += RTHR) {
    const int pos = scan_a[sel[q]] + lrank[q];
    p.perm[pos] = q;
    p.inv[q] = pos;
  }
}

// ---------------------------------------------------------------------------
// rank kernel: the histogram / rank half of dispatch from given ids
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rank_kernel(RankParams p) {
  __shared__ uint8_t sel[RT * kMaxE];
  __shared__ int wh[4][kMaxE];
  __shared__ int run[kMaxE + 1];
  const int t0 = blockIdx.x * RT;
  const int nt = min(RT, p.T - t0);
  const int npairs = nt * p.k;
  const int32_t* ids = p.ids + static_cast<size_t>(t0) * p.k;
  // caller-provided ids are clamped into [0, E) (the scatter clamps the same
  // way), so a bad id gives a wrong but in-bounds permutation
  for (int q = threadIdx.x; q < npairs; q += 256)
    sel[q] = static_cast<uint8_t>(min(max(ids[q], 0), p.E - 1));
  __syncthreads();
  block_rank<256>(sel, npairs, p.E, p.lrank + static_cast<size_t>(t0) * p.k, wh, run);
  if (static_cast<int>(threadIdx.x) < p.E) p.blk_hist[blockIdx.x * p.E + threadIdx.x] = run[threadIdx.x];
}

// ---------------------------------------------------------------------------
// scan kernel (one workgroup of 1024 threads). The per-block histogram is
// pulled into LDS with batched loads when it fits (NB * E <= kScanLdsInts),
// so the column scans run at LDS latency instead of one HBM round trip per
// block.
// ---------------------------------------------------------------------------
constexpr int kScanLdsInts = 32768;  // 128 KiB

__global__ __launch_bounds__(1024) void scan_kernel(ScanParams p) {
  extern __shared__ int hl[];  // [NB * E] when it fits
  __shared__ int part[1024];
  __shared__ int cnt[kMaxE + 1];
  __shared__ int off[kMaxE + 1];
  __shared__ int tp[kMaxE + 1];
  const int tid = threadIdx.x, E = p.E, NB = p.NB;
  const int n = NB * E;
  const bool in_lds = n <= kScanLdsInts;
  int* h = in_lds ? hl : p.blk_hist;
  if (in_lds) {
    for (int base = tid; base < n; base += 8 * 1024) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * 1024;
        v[u] = i < n ? p.blk_hist[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * 1024;
        if (i < n) hl[i] = v[u];
      }
    }
    __syncthreads();
  }
  int G = 1024 / E;
  if (G > NB) G = NB;
  const int g = tid / E, e = tid - g * E;
  const bool active = g < G;
  const int chunk = (NB + G - 1) / G;
  const int b0 = g * chunk, b1 = min(NB, b0 + chunk);
  if (active) {
    int s = 0;
    for (int b = b0; b < b1; ++b) s += h[b * E + e];
    part[g * E + e] = s;
  }
  __syncthreads();
  if (tid < E) {
    int r = 0;
    for (int gg = 0; gg < G; ++gg) {
      const int c = part[gg * E + tid];
      part[gg * E + tid] = r;
      r += c;
    }
    cnt[tid] = r;
  }
  __syncthreads();
  if (tid < kWave) wave_exclusive_scan256(cnt, off, E);
  if (tid < E) tp[tid] = (cnt[tid] + p.tile_m - 1) / p.tile_m;
  __syncthreads();
  if (tid < kWave) wave_exclusive_scan256(tp, tp, E);
  __syncthreads();
  if (active) {
    int base = off[e] + part[g * E + e];
    for (int b = b0; b < b1; ++b) {
      const int c = h[b * E + e];
      p.blk_hist[b * E + e] = base;
      base += c;
    }
  }
  if (tid < E) { p.counts[tid] = cnt[tid]; p.offsets[tid] = off[tid]; }
  if (tid == 0) p.offsets[E] = off[E];
  write_tile_table(tp, E, p.max_tiles, p.tile_e, p.exp_tile0, p.meta);
}

// ---------------------------------------------------------------------------
// scatter kernel
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scatter_kernel(ScatterParams p) {
  const int P = p.T * p.k;
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= P) return;
  const int t = q / p.k;
  const int b = t / RT;
  const int e = min(max(p.ids[q], 0), p.E - 1);
  const int pos = p.blk_base[b * p.E + e] + p.lrank[q];
  p.perm[pos] = q;
  p.inv[q] = pos;
}

// ---------------------------------------------------------------------------
// tile table from offsets (one workgroup)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tiles_kernel(TilesParams p) {
  __shared__ int tp[kMaxE + 1];
  const int tid = threadIdx.x;
  if (tid < p.E) {
    // caller-provided offsets: counts clamped to [0, P] so the table stays in bounds
    const int c = min(max(p.offsets[tid + 1] - p.offsets[tid], 0), p.P);
    tp[tid] = (c + p.tile_m - 1) / p.tile_m;
  }
  __syncthreads();
  if (tid < kWave) wave_exclusive_scan256(tp, tp, p.E);
  __syncthreads();
  write_tile_table(tp, p.E, p.max_tiles, p.tile_e, p.exp_tile0, p.meta);
}

// ---------------------------------------------------------------------------
// sigmoid(w . x_t) for the standalone shared expert
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rowdot_sigmoid_kernel(RowDotSigmoidParams p) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int lane = lane_id();
  float s = 0.f;
  if (p.dtype == MOE_BF16) {
    const uint16_t* x = static_cast<const uint16_t*>(p.x) + static_cast<size_t>(t) * p.d;
    const uint16_t* w = static_cast<const uint16_t*>(p.w);
    for (int i = lane; i < p.d; i += kWave) s = fmaf(bf16_to_f32(x[i]), bf16_to_f32(w[i]), s);
  } else {
    const float* x = static_cast<const float*>(p.x) + static_cast<size_t>(t) * p.d;
    const float* w = static_cast<const float*>(p.w);
    for (int i = lane; i < p.d; i += kWave) s = fmaf(x[i], w[i], s);
  }
  s = wave_sum(s);
  if (lane == 0) p.out[t] = sigmoid_f32(s);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int NCH>
static void launch_route_nch(const RouteParams& p, int dtype, int nb, hipStream_t s) {
  if (dtype == MOE_BF16) route_kernel<NCH, true><<<nb, RTHR, 0, s>>>(p);
  else route_kernel<NCH, false><<<nb, RTHR, 0, s>>>(p);
}

hipError_t launch_route(const RouteParams& p, int dtype, hipStream_t s) {
  const int nb = ceil_div(p.T, RT);
  const int cols = p.E + (p.w_sgate != nullptr ? 1 : 0);
  const int nch = ceil_div(cols, 64);
  switch (nch) {
    case 1: launch_route_nch<1>(p, dtype, nb, s); break;
    case 2: launch_route_nch<2>(p, dtype, nb, s); break;
    case 3: launch_route_nch<3>(p, dtype, nb, s); break;
    case 4: launch_route_nch<4>(p, dtype, nb, s); break;
    case 5: launch_route_nch<5>(p, dtype, nb, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rank(const RankParams& p, hipStream_t s) {
  rank_kernel<<<ceil_div(p.T, RT), 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanParams& p, hipStream_t s) {
  const int n = p.NB * p.E;
  const size_t lds = n <= kScanLdsInts ? static_cast<size_t>(n) * 4 : 0;
  scan_kernel<<<1, 1024, lds, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_scatter(const ScatterParams& p, hipStream_t s) {
  scatter_kernel<<<ceil_div(p.T * p.k, 256), 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_tiles(const TilesParams& p, hipStream_t s) {
  tiles_kernel<<<1, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_rowdot_sigmoid(const RowDotSigmoidParams& p, hipStream_t s) {
  rowdot_sigmoid_kernel<<<ceil_div(p.T, 4), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
