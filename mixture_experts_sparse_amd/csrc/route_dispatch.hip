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

#include <utility>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

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
// route kernel: 256 threads (4 waves), 64 tokens per workgroup.
//
// Logits: wave w computes its 16 tokens x all NC columns (E experts, the
// optional shared-gate row, padding) on bf16 MFMA, keeping them in the MFMA
// accumulators. x rows and router rows stream through an S-stage pipeline
// of 32-deep K slices loaded straight into LDS (every thread issues one x
// load and NCH router loads per stage, clamped in bounds).
//
// Select: lane l holds column f * 16 + (l & 15) of token rows (l >> 4) * 4 + i
// of its wave; each 16-lane group therefore owns one token per round i and
// runs the top-k with xor-shuffles inside the group.
// ---------------------------------------------------------------------------
constexpr int RTHR = 256;
constexpr int RNW = RTHR / kWave;
constexpr int RBK = 32;

template <int NCH>
struct RouteCfg {
  static constexpr int NC = NCH * 64;            // padded logit columns
  static constexpr int NF = NC / 16;             // 16-column MFMA fragments
  static constexpr int S = NCH <= 2 ? 8 : 4;     // pipeline stages
  static constexpr int SX = RT * RBK;            // x elements per stage
  static constexpr int SEL = SX + NC * RBK;      // elements per stage
  static constexpr int LPS = 1 + NCH;            // 16-byte loads per thread per stage
};

// Router logits on bf16 MFMA into acc[f] (fp32), rows/cols as above.
template <int NCH>
__device__ void route_logits_bf16(const RouteParams& p, int t0, floatx4_t* acc) {
  using C = RouteCfg<NCH>;
  constexpr int S = C::S, SEL = C::SEL, LPS = C::LPS, NF = C::NF;
  __shared__ __align__(16) uint16_t L0[SEL];
  __shared__ __align__(16) uint16_t L1[SEL];
  __shared__ __align__(16) uint16_t L2[SEL];
  __shared__ __align__(16) uint16_t L3[SEL];
  __shared__ __align__(16) uint16_t L4[S > 4 ? SEL : 8];
  __shared__ __align__(16) uint16_t L5[S > 5 ? SEL : 8];
  __shared__ __align__(16) uint16_t L6[S > 6 ? SEL : 8];
  __shared__ __align__(16) uint16_t L7[S > 7 ? SEL : 8];
  auto buf = [&]<int I>() -> uint16_t* {
    if constexpr (I == 0) return L0;
    else if constexpr (I == 1) return L1;
    else if constexpr (I == 2) return L2;
    else if constexpr (I == 3) return L3;
    else if constexpr (I == 4) return L4;
    else if constexpr (I == 5) return L5;
    else if constexpr (I == 6) return L6;
    else return L7;
  };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wbase = tid & ~63;
  const uint16_t* X = static_cast<const uint16_t*>(p.x);
  const uint16_t* W = static_cast<const uint16_t*>(p.w_router);
  const uint16_t* WS = static_cast<const uint16_t*>(p.w_sgate);
  const int d = p.d;
  // x slot: row tid / 4 of the block, physical chunk tid % 4
  const int xr = tid >> 2;
  const int xchunk = swz_phys_to_logical<RBK>(xr, tid & 3) * 8;
  const uint16_t* xsrc = X + static_cast<size_t>(t0 + xr < p.T ? t0 + xr : t0) * d;
  // router slots: rows i * 64 + tid / 4
  const uint16_t* wsrc[NCH];
  int wchunk[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int r = i * 64 + xr;
    wchunk[i] = swz_phys_to_logical<RBK>(r, tid & 3) * 8;
    const uint16_t* row = W;  // padding columns reload row 0 (never read back)
    if (r < p.E) row = W + static_cast<size_t>(r) * d;
    else if (r == p.E && WS != nullptr) row = WS;
    wsrc[i] = row;
  }
  const int nk = (d + RBK - 1) / RBK;
  const bool ktail = (d % RBK) != 0;
  auto issue = [&](uint16_t* st, int kc) {
    const int k0 = min(kc, nk - 1) * RBK;
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(xsrc + min(k0 + xchunk, d - 8)),
                                     (lds_void_t*)(st + wbase * 8), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(wsrc[i] + min(k0 + wchunk[i], d - 8)),
                                       (lds_void_t*)(st + C::SX + (i * RTHR + wbase) * 8), 16, 0, 0);
    }
  };
  const int fr = lane & 15, fq = lane >> 4;
  const int aoff = swz<RBK>(wave * 16 + fr, fq);
  const int boff = C::SX + swz<RBK>(fr, fq);  // + f * 16 rows
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  auto step = [&](int kc, uint16_t* cur, uint16_t* nxt) {
    wait_stage<(S - 2) * LPS>();
    stage_barrier();
    issue(nxt, kc + S - 1);
    if (kc < nk) {
      if (ktail && kc == nk - 1) {
        // zero x's columns past d (the router's clamped duplicates then multiply zeros)
        if (kc * RBK + xchunk >= d)
          *reinterpret_cast<u32x4_t*>(cur + tid * 8) = u32x4_t{0u, 0u, 0u, 0u};
        __syncthreads();
      }
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(cur + aoff));
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const bf16x8_t b = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(cur + boff + f * 16 * RBK));
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[f], 0, 0, 0);
      }
    }
  };
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((I < S - 1 ? issue(buf.template operator()<I>(), I) : void()), ...);
    for (int kb = 0; kb < nk; kb += S) {
      (step(kb + I, buf.template operator()<I>(), buf.template operator()<(I + S - 1) % S>()), ...);
    }
  }(std::make_integer_sequence<int, S>{});
  __syncthreads();  // drain the clamped loads past the last stage
}

// fp32 router logits by VALU into the same register layout (small layers);
// the K loop is outermost so every accumulator index is static.
template <int NCH>
__device__ void route_logits_f32(const RouteParams& p, int t0, floatx4_t* acc) {
  constexpr int NF = RouteCfg<NCH>::NF;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* X = static_cast<const float*>(p.x);
  const float* W = static_cast<const float*>(p.w_router);
  const float* WS = static_cast<const float*>(p.w_sgate);
  const float* wr[NF];
  const float* xr[4];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int e = f * 16 + (lane & 15);
    // columns without a router row read row 0 (their logits are never used)
    wr[f] = e < p.E ? W + static_cast<size_t>(e) * p.d : (e == p.E && WS != nullptr ? WS : W);
    acc[f] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + wave * 16 + (lane >> 4) * 4 + i;
    xr[i] = X + static_cast<size_t>(t < p.T ? t : t0) * p.d;
  }
  for (int c = 0; c < p.d; ++c) {
    float xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = xr[i][c];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const float w = wr[f][c];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[f][i] = fmaf(xv[i], w, acc[f][i]);
    }
  }
}

// Top-k, gates, logits and shared-gate outputs from the accumulator layout;
// the selection also goes to sel[] for the rank pass. Within a 16-lane
// group, lane c holds columns f * 16 + c (ascending with f), so a strict >
// over f keeps the lower index among equal values.
template <int NCH>
__device__ void route_select(const RouteParams& p, int t0, const floatx4_t* acc, uint8_t* sel) {
  constexpr int NF = RouteCfg<NCH>::NF;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int E = p.E, k = p.k;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 16 + (lane >> 4) * 4 + i;  // token row in the block
    const int t = t0 + r;
    const bool live = t < p.T;                       // uniform across the 16-lane group
    float v[NF], ov[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int e = f * 16 + c;
      float val = -INFINITY;
      if (e < E) {
        val = acc[f][i];
        if (p.bias != nullptr) val += p.bias[e];
        if (live && p.logits != nullptr) p.logits[static_cast<size_t>(t) * E + e] = val;
      }
      v[f] = val;
      ov[f] = val;
    }
    if (live && p.sgate != nullptr && c == (E & 15)) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
        if (f == (E >> 4)) p.sgate[t] = sigmoid_f32(acc[f][i]);
    }
    float m = 0.f, ssel = 0.f;
    for (int j = 0; j < k; ++j) {
      float bv = v[0];
      int bi = c;
#pragma unroll
      for (int f = 1; f < NF; ++f) {
        if (v[f] > bv) { bv = v[f]; bi = f * 16 + c; }
      }
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) {
        const float ovv = __shfl_xor(bv, off, kWave);
        const int oi = __shfl_xor(bi, off, kWave);
        if (ovv > bv || (ovv == bv && oi < bi)) { bv = ovv; bi = oi; }
      }
      if ((bi & 15) == c) {
#pragma unroll
        for (int f = 0; f < NF; ++f) if (f == (bi >> 4)) v[f] = -INFINITY;
      }
      if (j == 0) m = bv;  // the largest logit
      const float ej = expf(bv - m);
      ssel += ej;
      if (live && (j & 15) == c) {
        // un-normalised gate; divided by the denominator below
        p.ids[static_cast<size_t>(t) * k + j] = bi;
        p.gates[static_cast<size_t>(t) * k + j] = ej;
        sel[r * k + j] = static_cast<uint8_t>(bi);
      }
    }
    float denom = ssel;
    if (p.mode == MOE_SOFTMAX_ALL && !p.renorm) {
      float sall = 0.f;
#pragma unroll
      for (int f = 0; f < NF; ++f) if (f * 16 + c < E) sall += expf(ov[f] - m);
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) sall += __shfl_xor(sall, off, kWave);
      denom = sall;
    }
    const float inv = 1.0f / denom;
    if (live) {
      for (int j = c; j < k; j += 16) {
        float* g = p.gates + static_cast<size_t>(t) * k + j;
        *g = *g * inv;
      }
    }
  }
}

template <int NCH, bool BF16>
__global__ __launch_bounds__(RTHR) void route_kernel(RouteParams p) {
  __shared__ uint8_t sel[RT * kMaxE];
  __shared__ int wh[RNW][kMaxE];
  __shared__ int run[kMaxE + 1];
  __shared__ int scan_a[kMaxE + 1];
  __shared__ int scan_b[kMaxE + 1];
  const int t0 = blockIdx.x * RT;
  floatx4_t acc[RouteCfg<NCH>::NF];
  if constexpr (BF16) route_logits_bf16<NCH>(p, t0, acc);
  else route_logits_f32<NCH>(p, t0, acc);
  route_select<NCH>(p, t0, acc, sel);
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
  extern __shared__ __align__(16) int hl[];  // [NB * E] when it fits
  __shared__ int part[1024];
  __shared__ int cnt[kMaxE + 1];
  __shared__ int off[kMaxE + 1];
  __shared__ int tp[kMaxE + 1];
  const int tid = threadIdx.x, E = p.E, NB = p.NB;
  const int n = NB * E;
  const bool in_lds = n <= kScanLdsInts;
  int* h = in_lds ? hl : p.blk_hist;
  if (in_lds) {
    // 16-byte loads, all issued before any is used (one round trip when
    // n <= 4 * 8 * 1024), then the scalar tail
    const int n4 = n >> 2;
    const int4* src4 = reinterpret_cast<const int4*>(p.blk_hist);
    for (int base = tid; base < n4; base += 8 * 1024) {
      int4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * 1024;
        v[u] = i < n4 ? src4[i] : int4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * 1024;
        if (i < n4) reinterpret_cast<int4*>(hl)[i] = v[u];
      }
    }
    for (int i = (n4 << 2) + tid; i < n; i += 1024) hl[i] = p.blk_hist[i];
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
