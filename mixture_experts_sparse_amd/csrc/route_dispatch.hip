// Route and dispatch kernels for the sparse MoE layer forward (gfx950).
//
// route: router logits (bf16 MFMA with fp32 accumulation, or fp32 VALU),
//   top-k per token with ties to the lower expert index and slots in
//   descending logit order, softmax gates ("Tutorial 11: Mixture of Experts
//   (MoE)", section 2 "The Router"; "Small models, sparse experts", section
//   "How it works", step 3), and the first half of the counting sort:
//   per-route-block expert histograms and stable in-block ranks.
// scan: per-expert exclusive scan over route blocks -> counts and each
//   block's first row inside its expert's group.
// scatter: offsets (exclusive scan of counts), the grouped-GEMM tile table,
//   perm[offset + block base + rank] = pair, inv[pair] = row.
// A launch of one route block (T <= 64) finishes the whole dispatch inline.

#include <utility>

#include "device_common.h"
#include "moe_internal.h"
#include "tiny_route.h"

namespace moe {

constexpr int RTM = kRouteTokensMax;  // most tokens per route block
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
// tile_e[i] = the expert owning tile i < total (tp: tile prefix in LDS).
__device__ void fill_tile_e(const int* tp, int E, int total, int32_t* tile_e) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  for (int i = tid; i < total; i += nthr) {
    int lo = 0, hi = E - 1;  // last e with tp[e] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tp[mid] <= i) lo = mid; else hi = mid - 1;
    }
    tile_e[i] = lo;
  }
}

__device__ void write_tile_table(const int* tp, int E, int max_tiles, int32_t* tile_e,
                                 int32_t* exp_tile0, int32_t* meta) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int total = min(tp[E], max_tiles);
  for (int e = tid; e <= E; e += nthr) exp_tile0[e] = tp[e];
  fill_tile_e(tp, E, total, tile_e);
  if (tid == 0) meta[0] = total;
}

// Non-empty experts in ascending order -> touched[i] = {e, first row, rows,
// 0} for i < n, and n -> meta[1] (the small-batch GEMMs launch one
// workgroup row per touched expert and read its whole entry in one load).
// cnt(e) / first(e) are expert e's row count and first sorted row; flag and
// pos are LDS scratch of kMaxE + 1 ints. Called by every thread.
template <typename F, typename G>
__device__ void write_touched(F cnt, G first, int E, int* flag, int* pos, int32_t* touched,
                              int32_t* meta) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  for (int e = tid; e < E; e += nthr) flag[e] = cnt(e) > 0 ? 1 : 0;
  __syncthreads();
  if (tid < kWave) wave_exclusive_scan256(flag, pos, E);
  __syncthreads();
  for (int e = tid; e < E; e += nthr)
    if (flag[e])
      *reinterpret_cast<int4*>(touched + 4 * pos[e]) = make_int4(e, first(e), cnt(e), 0);
  if (tid == 0) meta[1] = pos[E];
}

// ---------------------------------------------------------------------------
// route kernel: 512 threads (8 waves), 64 tokens per workgroup.
//
// Logits: wave w computes token rows 16 * (w % 4) .. + 15 against one half of
// the NC columns (E experts, the optional shared-gate row, padding), half
// w / 4, on bf16 MFMA. K is streamed in 32-deep slices by direct
// global->LDS loads through two rings: waves 0-3 stream the block's x rows
// (read once, from HBM) RX - 1 slices ahead, waves 4-7 stream the router
// rows (shared by every workgroup, so mostly L2 hits) RR - 1 slices ahead.
// A wave's outstanding-load counter retires in issue order, so giving each
// stream its own waves lets the HBM stream run far ahead of the L2 one.
//
// The logits then go through LDS (one padded fp32 row per token) and the
// selection runs on 16-lane groups, one token per group and round: lane c
// holds columns f * 16 + c.
// ---------------------------------------------------------------------------
constexpr int RTHR = 512;
constexpr int RNW = RTHR / kWave;

template <int NCH, int RT>
struct RouteCfg {
  static_assert(RT == 32 || RT == 64, "route blocks of 32 or 64 tokens");
  static constexpr int NC = NCH * 64;            // padded logit columns
  static constexpr int NF = NC / 16;             // 16-column fragments of a row
  static constexpr int NTG = RT / 16;            // token groups of 16 (waves along tokens)
  static constexpr int NCG = RNW / NTG;          // column groups (waves along columns)
  static constexpr int NH = NC / NCG;            // columns per wave
  static constexpr int NF2 = NH / 16;            // fragments per wave
  // K slice depth: 64 (128-byte row segments, which stream out of L2 at
  // about 1.6x the rate of 64-byte ones) wherever the two rings fit in LDS
  static constexpr int RBK = (NCH == 5 && RT == 64) ? 32 : 64;
  static constexpr int CPR = RBK / 8;            // 16-byte chunks per LDS row
  static constexpr int KS = RBK / 32;            // MFMA steps per slice
  static constexpr int SX = RT * RBK;            // x elements per slice
  static constexpr int SW = NC * RBK;            // router elements per slice
  static constexpr int RX = RBK == 64 ? 6 : 16;  // x ring slots
  // router ring slots: as many as the LDS left by the x ring holds, 3 to 8
  // (deeper rings measured 1-3 us faster for 60 and 64 experts, no change
  // for 128 and 256)
  static constexpr int RRB = (163840 - 1024 - RX * RT * RBK * 2) / (NCH * 64 * RBK * 2);
  static constexpr int RR = RRB > 8 ? 8 : (RRB < 3 ? 3 : RRB);
  static constexpr int XCH = RT * CPR;           // x chunks per slice
  static constexpr int LX = XCH <= 256 ? 1 : XCH / 256;  // x loads per x-wave lane per slice
  static constexpr int XW = XCH <= 256 ? XCH / 64 : 4;    // x-stream waves
  static constexpr int LW = NC * CPR / 256;      // router loads per router-wave thread per slice
  static_assert(XW * 64 * LX == XCH && LW * 256 == NC * CPR, "whole loads per slice");
  static_assert((RR - 2) * LW < 64 && (RX - 2) * LX < 64, "vmcnt range");
  static constexpr int LGLD = NC + 4;            // logit row stride in LDS (floats)
  // LDS after the logits: selections, per-wave histograms, running counts
  static constexpr int CARVE = RT * kMaxE + RNW * kMaxE * 4 + 3 * (kMaxE + 1) * 4;
  static constexpr int XBYTES = RX * SX * 2 > CARVE ? RX * SX * 2 : CARVE;
  static constexpr int LGBYTES = RT * LGLD * 4;
  static constexpr int WBYTES = RR * SW * 2 > LGBYTES ? RR * SW * 2 : LGBYTES;
};

// LDS destination of a direct global->LDS load, hidden from the compiler's
// load-counter tracking: every wait on these loads is explicit and followed
// by a workgroup barrier before any wave reads the data.
__device__ __forceinline__ lds_void_t* lds_untracked(uint16_t* q) {
  lds_void_t* r = (lds_void_t*)q;
  asm volatile("" : "+s"(r));
  return r;
}

// Router logits on bf16 MFMA: acc[f][i] = logit of token row
// 16 * (w % NTG) + 4 * (lane / 16) + i, column NH * (w / NTG) + 16 * f + lane % 16.
// Waves 0 .. XW-1 stream x, waves 4-7 the router rows (waves XW..3 load nothing).
template <int NCH, int RT>
__device__ void route_logits_bf16(const RouteParams& p, int t0, floatx4_t* acc, uint16_t* Xr,
                                  uint16_t* Wr) {
  using C = RouteCfg<NCH, RT>;
  constexpr int RX = C::RX, RR = C::RR, LW = C::LW, NF2 = C::NF2, NTG = C::NTG;
  constexpr int LX = C::LX, RBK = C::RBK, CPR = C::CPR, KS = C::KS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool xw = wave < C::XW;              // x-stream waves
  const bool ww = wave >= 4;                 // router-stream waves
  const int lt = tid & 255;                  // thread index within the stream
  const int lwb = (wave & 3) * 64;
  const uint16_t* X = static_cast<const uint16_t*>(p.x);
  const uint16_t* W = static_cast<const uint16_t*>(p.w_router);
  const uint16_t* WS = static_cast<const uint16_t*>(p.w_sgate);
  const int d = p.d;
  constexpr int LM = LX > LW ? LX : LW;
  // load i of a stream thread fills slot chunk q = i * 256 + lt: row
  // q / CPR, physical chunk q % CPR (the swizzle picks the logical K chunk);
  // waves that stream nothing keep a valid address they never use
  const uint16_t* src[LM];
  int chunk[LM];
#pragma unroll
  for (int i = 0; i < LM; ++i) {
    const int q = i * 256 + lt;
    const int r = q / CPR;
    chunk[i] = swz_phys_to_logical<RBK>(r, q % CPR) * 8;
    if (xw) {
      src[i] = X + static_cast<size_t>(t0 + r < p.T ? t0 + r : t0) * d;
    } else {
      const uint16_t* row = W;  // padding columns reload row 0 (never read back)
      if (r < p.E) row = W + static_cast<size_t>(r) * d;
      else if (r == p.E && WS != nullptr) row = WS;
      src[i] = row;
    }
  }
  const int nk = (d + RBK - 1) / RBK;
  const bool ktail = (d % RBK) != 0;
  // every lane issues every load (clamped in bounds), so each wave's count
  // of outstanding loads is the same on every path
  auto issue = [&]<int L>(uint16_t* slot, int kc) {
    const int k0 = min(kc, nk - 1) * RBK;
#pragma unroll
    for (int i = 0; i < L; ++i)
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(src[i] + min(k0 + chunk[i], d - 8)),
                                       lds_untracked(slot + (i * 256 + lwb) * 8), 16, 0, 0);
  };
  const int fr = lane & 15, fq = lane >> 4;
  int aoff[KS], boff[KS];  // MFMA step j reads logical chunk 4 j + fq
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    aoff[j] = swz<RBK>((wave % NTG) * 16 + fr, 4 * j + fq);
    boff[j] = swz<RBK>((wave / NTG) * C::NH + fr, 4 * j + fq);  // + f * 16 rows
  }
#pragma unroll
  for (int f = 0; f < NF2; ++f) acc[f] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  if (xw) {
#pragma unroll
    for (int st = 0; st < RX - 1; ++st) issue.template operator()<LX>(Xr + st * C::SX, st);
  } else if (ww) {
#pragma unroll
    for (int st = 0; st < RR - 1; ++st) issue.template operator()<LW>(Wr + st * C::SW, st);
  }
  int cx = 0, cw = 0, ix = RX - 1, iw = RR - 1;
  for (int kc = 0; kc < nk; ++kc) {
    // slice kc is in x slot cx / router slot cw once this wave's own loads
    // of it are done (all but the newer slices') and every wave has passed
    // the barrier
    if (xw) wait_stage<(RX - 2) * LX>();
    else if (ww) wait_stage<(RR - 2) * LW>();
    else wait_stage<0>();
    stage_barrier();
    if (xw) issue.template operator()<LX>(Xr + ix * C::SX, kc + RX - 1);
    else if (ww) issue.template operator()<LW>(Wr + iw * C::SW, kc + RR - 1);
    ix = ix + 1 == RX ? 0 : ix + 1;
    iw = iw + 1 == RR ? 0 : iw + 1;
    uint16_t* xs = Xr + cx * C::SX;
    const uint16_t* ws = Wr + cw * C::SW;
    if (ktail && kc == nk - 1) {
      // zero x's columns past d (the router's clamped duplicates then multiply zeros)
      if (xw) {
#pragma unroll
        for (int i = 0; i < LX; ++i)
          if (kc * RBK + chunk[i] >= d)
            *reinterpret_cast<u32x4_t*>(xs + (i * 256 + lt) * 8) = u32x4_t{0u, 0u, 0u, 0u};
      }
      wait_stage<63>();
      stage_barrier();
    }
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const bf16x8_t a =
          __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(xs + aoff[j]));
#pragma unroll
      for (int f = 0; f < NF2; ++f) {
        const bf16x8_t b = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(ws + boff[j] + f * 16 * RBK));
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[f], 0, 0, 0);
      }
    }
    cx = cx + 1 == RX ? 0 : cx + 1;
    cw = cw + 1 == RR ? 0 : cw + 1;
  }
  // the clamped loads past the last slice are drained before the rings'
  // LDS is reused
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// fp32 router logits by VALU into the same register layout (small layers);
// the K loop is outermost so every accumulator index is static.
template <int NCH, int RT>
__device__ void route_logits_f32(const RouteParams& p, int t0, floatx4_t* acc) {
  using C = RouteCfg<NCH, RT>;
  constexpr int NF2 = C::NF2, NTG = C::NTG;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* X = static_cast<const float*>(p.x);
  const float* W = static_cast<const float*>(p.w_router);
  const float* WS = static_cast<const float*>(p.w_sgate);
  const float* wr[NF2];
  const float* xr[4];
#pragma unroll
  for (int f = 0; f < NF2; ++f) {
    const int e = (wave / NTG) * C::NH + f * 16 + (lane & 15);
    // columns without a router row read row 0 (their logits are never used)
    wr[f] = e < p.E ? W + static_cast<size_t>(e) * p.d : (e == p.E && WS != nullptr ? WS : W);
    acc[f] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + (wave % NTG) * 16 + (lane >> 4) * 4 + i;
    xr[i] = X + static_cast<size_t>(t < p.T ? t : t0) * p.d;
  }
  for (int c = 0; c < p.d; ++c) {
    float xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = xr[i][c];
#pragma unroll
    for (int f = 0; f < NF2; ++f) {
      const float w = wr[f][c];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[f][i] = fmaf(xv[i], w, acc[f][i]);
    }
  }
}

// Accumulators -> one padded fp32 row of logits per token in LDS.
template <int NCH, int RT>
__device__ __forceinline__ void store_logits(const floatx4_t* acc, float* Lg) {
  using C = RouteCfg<NCH, RT>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int f = 0; f < C::NF2; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (wave % C::NTG) * 16 + (lane >> 4) * 4 + i;
      Lg[r * C::LGLD + (wave / C::NTG) * C::NH + f * 16 + (lane & 15)] = acc[f][i];
    }
}

// Selection keys: the float's bits mapped to an unsigned integer of the same
// order in the high word, the bitwise complement of the expert index in the
// low word, so the largest key is the largest logit and, among equal
// logits, the lower expert index. 0 (below every key) marks no candidate.
__device__ __forceinline__ uint64_t sel_key(float v, int e) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(o) << 32) | static_cast<uint32_t>(~e);
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t o = static_cast<uint32_t>(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int key_index(uint64_t key) {
  return static_cast<int>(~static_cast<uint32_t>(key));
}
// max of a 64-bit key with its DPP partner inside each row of 16 lanes
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max(uint64_t a) {
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(a)), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(a >> 32)), CTRL, 0xF, 0xF, false);
  const uint64_t b = (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
  return b > a ? b : a;
}
// Maximum over the 16 lanes of each row: swap neighbours, swap pairs
// (quad permutations), then mirror within 8 lanes and within 16 lanes;
// every lane ends with the row's maximum.
__device__ __forceinline__ uint64_t row16_max(uint64_t a) {
  a = dpp_max<0xB1>(a);   // quad_perm [1,0,3,2]
  a = dpp_max<0x4E>(a);   // quad_perm [2,3,0,1]
  a = dpp_max<0x141>(a);  // row_half_mirror
  a = dpp_max<0x140>(a);  // row_mirror
  return a;
}
// Largest of a lane's NF keys by a pairwise tree (depth log2 NF instead of
// a chain of NF - 1 dependent steps).
template <int NF>
__device__ __forceinline__ uint64_t max_keys(const uint64_t* key) {
  uint64_t t[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) t[f] = key[f];
#pragma unroll
  for (int w = 1; w < NF; w *= 2)
#pragma unroll
    for (int f = 0; f + w < NF; f += 2 * w) t[f] = t[f + w] > t[f] ? t[f + w] : t[f];
  return t[0];
}
// Drops the winner (expert idx) from further rounds: lane c holds expert
// f * 16 + c in key[f]. Only the value word is cleared; a cleared key still
// beats the all-zero keys of columns past E, but never a live key (whose
// value word is at least 1), and at most k <= E keys are ever taken.
template <int NF>
__device__ __forceinline__ void drop_key(uint64_t* key, int idx, int c) {
#pragma unroll
  for (int f = 0; f < NF; ++f)
    if (idx == f * 16 + c) key[f] &= 0xFFFFFFFFull;
}
template <int CTRL>
__device__ __forceinline__ float dpp_add(float a) {
  return a + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of each row, every lane ending with it: after the
// two quad permutations each quad holds its sum in all four lanes, so each
// mirror then adds a partner block of equal values. Same order on every
// lane, so the result is identical across the row.
__device__ __forceinline__ float row16_sum(float a) {
  a = dpp_add<0xB1>(a);
  a = dpp_add<0x4E>(a);
  a = dpp_add<0x141>(a);
  a = dpp_add<0x140>(a);
  return a;
}

// Router bias of this lane's columns (f * 16 + lane % 16), loaded before
// the logits so that no load is outstanding in the selection.
template <int NCH>
__device__ __forceinline__ void load_bias(const RouteParams& p, float* bias) {
  constexpr int NF = NCH * 4;
  const int c = threadIdx.x & 15;
#pragma unroll
  for (int f = 0; f < NF; ++f) bias[f] = 0.f;
  if (p.bias != nullptr) {
#pragma unroll
    // columns past E read bias[E - 1]; their logits are never used
    for (int f = 0; f < NF; ++f) bias[f] = p.bias[min(f * 16 + c, p.E - 1)];
  }
}

// Top-k, gates, logits and shared-gate outputs from the logit rows in LDS;
// the selection also goes to sel[] for the rank pass. 16-lane group g of the
// workgroup owns token rows g, g + 32, ...; rounds of 32 rows past the last
// token are skipped.
//
// Each of the k selection steps is a 16-lane maximum of 64-bit keys (one
// candidate per lane, the lane's best remaining key) followed by removing
// the winner: a chain of dependent instructions with no memory access and no
// branch. For k <= 16, lane c keeps slot c's winner in registers and the
// exponentials, sums and stores run once after the loop, in parallel over
// the slots.
template <int NCH, int RT>
__device__ void route_select(const RouteParams& p, int t0, const float* Lg, const float* bias,
                             uint8_t* sel) {
  using C = RouteCfg<NCH, RT>;
  constexpr int NF = C::NF;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int E = p.E, k = p.k;
  const bool sig = p.mode == MOE_SIGMOID;
#pragma unroll
  for (int rnd = 0; rnd < RT / 32; ++rnd) {
    if (t0 + rnd * 32 >= p.T) break;  // uniform: no live token in this or later rounds
    const int r = rnd * 32 + wave * 4 + (lane >> 4);  // token row in the block
    const int t = t0 + r;
    const bool live = t < p.T;                          // uniform across the 16-lane group
    const float* row = Lg + r * C::LGLD;
    // every column of the padded row is readable and finite: all reads go
    // out together, columns past E are masked afterwards
    float v[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) v[f] = row[f * 16 + c];
    if (live && p.logits != nullptr) {
      // sigmoid scoring keeps the logits output bias-free
#pragma unroll
      for (int f = 0; f < NF; ++f)
        if (f * 16 + c < E)
          p.logits[static_cast<size_t>(t) * E + f * 16 + c] = sig ? v[f] : v[f] + bias[f];
    }
    if (live && p.sgate != nullptr && c == 0) p.sgate[t] = sigmoid_f32(row[E]);
    // the score that selects: the bias steers the choice only
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const float val = (sig ? sigmoid_f32(v[f]) : v[f]) + bias[f];
      v[f] = f * 16 + c < E ? val + 0.0f : -INFINITY;  // -0 -> +0: equal scores, equal keys
    }
    uint64_t key[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) key[f] = f * 16 + c < E ? sel_key(v[f], f * 16 + c) : 0ull;
    // softmax-all without renormalisation divides by the sum over every expert
    const bool all = p.mode == MOE_SOFTMAX_ALL && !p.renorm;
    if (k <= 16) {
      uint64_t mine = 0ull;  // lane c: slot c's key
      for (int j = 0; j < k; ++j) {
        const uint64_t b = row16_max(max_keys<NF>(key));
        drop_key<NF>(key, key_index(b), c);
        mine = j == c ? b : mine;
      }
      const float m = __shfl(key_value(mine), lane & 48, kWave);  // slot 0: the largest logit
      const int mi = c < k ? key_index(mine) : 0;
      // gate numerators: exp(L - max) in the softmax modes; in the sigmoid
      // mode the raw affinity of the chosen expert (its bias left out)
      const float ej = c < k ? (sig ? sigmoid_f32(row[mi]) : expf(key_value(mine) - m)) : 0.f;
      float denom = row16_sum(ej);
      if (sig && !p.renorm) denom = 1.0f;
      if (all) {
        float sall = 0.f;
#pragma unroll
        for (int f = 0; f < NF; ++f) if (f * 16 + c < E) sall += expf(v[f] - m);
        denom = row16_sum(sall);
      }
      if (c < k) {
        sel[r * k + c] = static_cast<uint8_t>(mi);
        if (live) {
          p.ids[static_cast<size_t>(t) * k + c] = mi;
          p.gates[static_cast<size_t>(t) * k + c] = ej * (1.0f / denom);
        }
      }
    } else {
      // k > 16: each slot's id and un-normalised gate are stored as it is found
      float m = 0.f, ssel = 0.f;
      for (int j = 0; j < k; ++j) {
        const uint64_t b = row16_max(max_keys<NF>(key));
        drop_key<NF>(key, key_index(b), c);
        const float bv = key_value(b);
        const int bi = key_index(b);
        if (j == 0) m = bv;  // the largest logit
        const float ej = sig ? sigmoid_f32(row[bi]) : expf(bv - m);
        ssel += ej;
        if ((j & 15) == c) {
          if (live) {
            p.ids[static_cast<size_t>(t) * k + j] = bi;
            p.gates[static_cast<size_t>(t) * k + j] = ej;
          }
          sel[r * k + j] = static_cast<uint8_t>(bi);
        }
      }
      float denom = ssel;
      if (sig && !p.renorm) denom = 1.0f;
      if (all) {
        float sall = 0.f;
#pragma unroll
        for (int f = 0; f < NF; ++f) if (f * 16 + c < E) sall += expf(v[f] - m);
        denom = row16_sum(sall);
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
}

// The same selection by rank counting, for blocks where T_block * E^2 is
// small (few tokens): every (token, expert) item counts the experts whose
// key beats its own -- a larger logit, or an equal logit at a lower index --
// and an item of rank j < k is slot j. The items run in parallel over the
// workgroup, so the cost is E compares per item instead of k dependent
// 16-lane maximum steps. The logit rows in LDS are rewritten in place as
// order-preserving 32-bit keys; gates then follow per token on 16-lane
// groups (lane c: slots c, c + 16, ...). Called by every thread.
__device__ __forceinline__ uint32_t order_key32(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_value32(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int NCH, int RT>
__device__ void route_select_rank(const RouteParams& p, int t0, float* Lg, const float* bias,
                                  uint8_t* sel) {
  using C = RouteCfg<NCH, RT>;
  constexpr int NF = C::NF;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15;
  const int E = p.E, k = p.k;
  const int nt = min(RT, p.T - t0);
  uint32_t* K32 = reinterpret_cast<uint32_t*>(Lg);
  // keys (and the optional logits / shared-gate outputs)
  for (int r0 = 0; r0 < nt; r0 += 32) {
    const int r = r0 + wave * 4 + (lane >> 4);
    if (r < nt) {
      const int t = t0 + r;
      float* row = Lg + r * C::LGLD;
      if (p.sgate != nullptr && c == 0) p.sgate[t] = sigmoid_f32(row[E]);
      float val[NF];  // the padded row is readable: all reads go out together
#pragma unroll
      for (int f = 0; f < NF; ++f) val[f] = row[f * 16 + c] + bias[f];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int e = f * 16 + c;
        if (e < E) {
          if (p.logits != nullptr) p.logits[static_cast<size_t>(t) * E + e] = val[f];
          K32[r * C::LGLD + e] = order_key32(val[f] + 0.0f);  // -0 -> +0
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < nt * E; i += RTHR) {
    const int r = i / E, e = i - r * E;
    const uint32_t* row = K32 + r * C::LGLD;  // 16-byte aligned rows
    const uint32_t o = row[e];
    // four keys per LDS read, four independent counts
    int n4[4] = {0, 0, 0, 0};
    int q = 0;
#pragma unroll 4
    for (; q + 4 <= E; q += 4) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + q);
#pragma unroll
      for (int u = 0; u < 4; ++u) n4[u] += (v[u] > o || (v[u] == o && q + u < e)) ? 1 : 0;
    }
    for (; q < E; ++q) n4[0] += (row[q] > o || (row[q] == o && q < e)) ? 1 : 0;
    const int rank = (n4[0] + n4[1]) + (n4[2] + n4[3]);
    if (rank < k) {
      sel[r * k + rank] = static_cast<uint8_t>(e);
      p.ids[static_cast<size_t>(t0 + r) * k + rank] = e;
    }
  }
  __syncthreads();
  const bool all = p.mode == MOE_SOFTMAX_ALL && !p.renorm;
  for (int r0 = 0; r0 < nt; r0 += 32) {
    const int r = r0 + wave * 4 + (lane >> 4);
    if (r < nt) {  // uniform across the 16-lane group
      const int t = t0 + r;
      const uint32_t* row = K32 + r * C::LGLD;
      const float m = order_value32(row[sel[r * k]]);  // slot 0: the largest logit
      float sum = 0.f;
      for (int j = c; j < k; j += 16) sum += expf(order_value32(row[sel[r * k + j]]) - m);
      if (all) {
        sum = 0.f;
#pragma unroll
        for (int f = 0; f < NF; ++f)
          if (f * 16 + c < E) sum += expf(order_value32(row[f * 16 + c]) - m);
      }
      sum = row16_sum(sum);
      const float inv = 1.0f / sum;
      for (int j = c; j < k; j += 16)
        p.gates[static_cast<size_t>(t) * k + j] = expf(order_value32(row[sel[r * k + j]]) - m) * inv;
    }
  }
}

// One wave finishes the counting sort's tables for a single route block:
// from the per-expert counts (run) it writes counts, offsets (also to
// scan_a, total at E), the tile prefix (exp_tile0 and scan_b, total at E),
// the tile count and the touched table; lane l owns experts 4l .. 4l + 3.
// The three prefix sums share one pass of shuffles.
__device__ void finish_scan(const RouteParams& p, const int* run, int* scan_a, int* scan_b) {
  const int lane = lane_id();
  const int E = p.E, b = lane * 4;
  int v[4], tl[4], fl[4];
  int sv = 0, st = 0, sf = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = b + i < E ? run[b + i] : 0;
    tl[i] = (v[i] + p.tile_m - 1) / p.tile_m;
    fl[i] = v[i] > 0 ? 1 : 0;
    sv += v[i]; st += tl[i]; sf += fl[i];
  }
  int iv = sv, it = st, jf = sf;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int a = __shfl_up(iv, off, kWave), c = __shfl_up(it, off, kWave),
              d = __shfl_up(jf, off, kWave);
    if (lane >= off) { iv += a; it += c; jf += d; }
  }
  int ev = iv - sv, et = it - st, ef = jf - sf;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = b + i;
    if (e < E) {
      scan_a[e] = ev; scan_b[e] = et;
      p.counts[e] = v[i]; p.offsets[e] = ev; p.exp_tile0[e] = et;
      if (fl[i] && p.touched != nullptr)
        *reinterpret_cast<int4*>(p.touched + 4 * ef) = make_int4(e, ev, v[i], 0);
    }
    ev += v[i]; et += tl[i]; ef += fl[i];
  }
  if (lane == kWave - 1) {
    scan_a[E] = iv; scan_b[E] = it;
    p.offsets[E] = iv; p.exp_tile0[E] = it;
    p.meta[0] = min(it, p.max_tiles);
    p.meta[1] = jf;
  }
}

// Selection, then the block's histogram and ranks (several route blocks) or
// the whole dispatch (one route block), from the logit rows in LDS. The
// selections, histograms and scans live in the LDS at carve (CARVE bytes).
template <int NCH, int RT>
__device__ void route_tail(const RouteParams& p, int t0, float* Lg, const float* bias,
                           void* carve) {
  uint8_t* sel = static_cast<uint8_t*>(carve);                             // [RT * kMaxE]
  int (*wh)[kMaxE] = reinterpret_cast<int (*)[kMaxE]>(sel + RT * kMaxE);  // [RNW][kMaxE]
  int* run = reinterpret_cast<int*>(wh + RNW);                             // [kMaxE + 1]
  int* scan_a = run + (kMaxE + 1);
  int* scan_b = scan_a + (kMaxE + 1);
  const int nt = min(RT, p.T - t0);
  // rank counting costs E compares per (token, expert) item, spread over the
  // workgroup; the 16-lane maximum steps cost a fixed dependent chain per 32
  // tokens: the first is cheaper while the block's T * E^2 stays small
  // (the sigmoid mode keeps the raw logits for its gates: the second path)
  if (p.mode != MOE_SIGMOID && static_cast<long long>(nt) * p.E * p.E <= (1LL << 17))
    route_select_rank<NCH, RT>(p, t0, Lg, bias, sel);
  else
    route_select<NCH, RT>(p, t0, Lg, bias, sel);
  if (p.blk_hist == nullptr && p.counts == nullptr) return;
  __syncthreads();
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
  if (tid < kWave) finish_scan(p, run, scan_a, scan_b);
  __syncthreads();
  // the grouped GEMMs' tile table (not needed by the small-batch GEMMs)
  if (p.tile_e != nullptr) fill_tile_e(scan_b, p.E, min(scan_b[p.E], p.max_tiles), p.tile_e);
  for (int q = tid; q < npairs; q += RTHR) {
    const int pos_q = scan_a[sel[q]] + lrank[q];
    p.perm[pos_q] = q;
    p.inv[q] = pos_q;
  }
}

template <int NCH, bool BF16, int RT>
__global__ __launch_bounds__(RTHR) void route_kernel(RouteParams p) {
  using C = RouteCfg<NCH, RT>;
  // x ring during the logits, then the selections and histograms; router
  // ring during the logits, then the logit rows
  __shared__ __align__(16) uint16_t Xr[(BF16 ? C::XBYTES : C::CARVE) / 2];
  __shared__ __align__(16) uint16_t Wr[(BF16 ? C::WBYTES : C::LGBYTES) / 2];
  float* Lg = reinterpret_cast<float*>(Wr);  // [RT][LGLD]
  const int t0 = blockIdx.x * RT;
  float bias[C::NF];
  load_bias<NCH>(p, bias);
  {
    floatx4_t acc[C::NF2];
    if constexpr (BF16) route_logits_bf16<NCH, RT>(p, t0, acc, Xr, Wr);
    else route_logits_f32<NCH, RT>(p, t0, acc);
    store_logits<NCH, RT>(acc, Lg);
  }
  __syncthreads();
  route_tail<NCH, RT>(p, t0, Lg, bias, Xr);
}

// ---------------------------------------------------------------------------
// Split router for one route block (T <= 64). A single workgroup streaming
// the whole router matrix is bound by its own load latency, so the logits
// are spread over workgroups: workgroup (c, g) computes logit columns
// 16 c .. 16 c + 15 (router rows, then the shared-gate row, then padding) for
// tokens 16 g .. 16 g + 15 over the whole of K, its 8 waves each taking one
// eighth of K with every load of its share issued at once; the eight partial
// tiles are added in wave order through LDS and the logits go to a [T, ncp]
// fp32 buffer. route_finish_kernel then runs the selection and the dispatch.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(RTHR) void route_part_kernel(RouteParams p) {
  __shared__ float red[RNW][16][16];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = blockIdx.x * 16 + (lane & 15);
  const int tok = min(static_cast<int>(blockIdx.y) * 16 + (lane & 15), p.T - 1);
  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  // K in batches of 8 steps: the batch's loads are all issued, then used
  constexpr int KB = 8;
  if constexpr (BF16) {
    const int kw = (p.d + RNW * 32 - 1) / (RNW * 32) * 32;  // K per wave, whole 32-deep steps
    const int k0 = wave * kw, k1 = min(p.d, k0 + kw);
    const uint16_t* W = static_cast<const uint16_t*>(p.w_router);
    const uint16_t* WS = static_cast<const uint16_t*>(p.w_sgate);
    // padding columns reread router row 0; their sums are never used
    const uint16_t* wrow = col < p.E ? W + static_cast<size_t>(col) * p.d
                                     : (col == p.E && WS != nullptr ? WS : W);
    const uint16_t* xrow = static_cast<const uint16_t*>(p.x) + static_cast<size_t>(tok) * p.d;
    const int g = (lane >> 4) * 8;
    for (int kk = k0; kk < k1; kk += 32 * KB) {
      u32x4_t av[KB], bv[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int kq = min(kk + 32 * u + g, p.d - 8);
        av[u] = *reinterpret_cast<const u32x4_t*>(xrow + kq);
        bv[u] = *reinterpret_cast<const u32x4_t*>(wrow + kq);
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) { pin(av[u]); pin(bv[u]); }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        // d and k0 are multiples of 8: the 8 values are all in range or none is
        const bool in = kk + 32 * u + g < k1;
        const u32x4_t z = {0u, 0u, 0u, 0u};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, in ? av[u] : z),
                                                      __builtin_bit_cast(bf16x8_t, in ? bv[u] : z),
                                                      acc, 0, 0, 0);
      }
    }
  } else {
    const int kw = (p.d + RNW * 16 - 1) / (RNW * 16) * 16;
    const int k0 = wave * kw, k1 = min(p.d, k0 + kw);
    const float* W = static_cast<const float*>(p.w_router);
    const float* WS = static_cast<const float*>(p.w_sgate);
    const float* wrow = col < p.E ? W + static_cast<size_t>(col) * p.d
                                  : (col == p.E && WS != nullptr ? WS : W);
    const float* xrow = static_cast<const float*>(p.x) + static_cast<size_t>(tok) * p.d;
    const int g = (lane >> 4) * 4;
    for (int kk = k0; kk < k1; kk += 16 * KB) {
      floatx4_t av[KB], bv[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int kq = min(kk + 16 * u + g, p.d - 4);
        av[u] = *reinterpret_cast<const floatx4_t*>(xrow + kq);
        bv[u] = *reinterpret_cast<const floatx4_t*>(wrow + kq);
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) { pin(av[u]); pin(bv[u]); }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const bool in = kk + 16 * u + g < k1;
        const floatx4_t z = {0.f, 0.f, 0.f, 0.f};
        const floatx4_t a = in ? av[u] : z, b = in ? bv[u] : z;
        // step i covers K indices kk + 16 u + 4 (lane / 16) + i
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
      }
    }
  }
  // this lane: column lane % 16, token rows 4 (lane / 16) + i of the group
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][(lane >> 4) * 4 + i][lane & 15] = acc[i];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < RNW; ++w) v += red[w][r][c];
    const int t = blockIdx.y * 16 + r;
    if (t < p.T) p.part[static_cast<size_t>(t) * p.ncp + blockIdx.x * 16 + c] = v;
  }
}

template <int NCH>
__global__ __launch_bounds__(RTHR) void route_finish_kernel(RouteParams p) {
  using C = RouteCfg<NCH, RTM>;
  constexpr int IPT = RTM * C::NC / RTHR;  // logit slots per thread
  __shared__ __align__(16) uint8_t carve[C::CARVE];
  __shared__ __align__(16) float Lg[C::LGBYTES / 4];
  float bias[C::NF];
  load_bias<NCH>(p, bias);
  const int tid = threadIdx.x;
  // every load issued before the first use (clamped addresses, no branches)
  float v[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int i = tid + j * RTHR;
    const int r = i / C::NC, c = i - (i / C::NC) * C::NC;
    v[j] = p.part[static_cast<size_t>(min(r, p.T - 1)) * p.ncp + min(c, p.ncp - 1)];
  }
#pragma unroll
  for (int j = 0; j < IPT; ++j) pin(v[j]);
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int i = tid + j * RTHR;
    const int r = i / C::NC, c = i - (i / C::NC) * C::NC;
    Lg[r * C::LGLD + c] = (r < p.T && c < p.ncp) ? v[j] : 0.f;
  }
  __syncthreads();
  route_tail<NCH, RTM>(p, 0, Lg, bias, carve);
}

// ---------------------------------------------------------------------------
// Finish of the split router for the smallest batches (T <= 4 tokens, at most
// 64 experts), one workgroup: wave t takes token t, lane e expert e. A lane's
// rank is the number of selection keys that beat its own, counted over
// broadcast LDS reads; the gates follow from wave reductions, and wave 0
// builds the dispatch tables with wave prefix sums (tiny_route). The outputs
// are those of route_finish_kernel.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kTinyT * kWave) void route_tiny_kernel(RouteParams p) {
  __shared__ TinyRouteLds S;
  tiny_route(p, S, true, false);
}

// ---------------------------------------------------------------------------
// rank kernel: the histogram / rank half of dispatch from given ids
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rank_kernel(RankParams p) {
  __shared__ uint8_t sel[RTM * kMaxE];
  __shared__ int wh[4][kMaxE];
  __shared__ int run[kMaxE + 1];
  const int t0 = blockIdx.x * p.rt;
  const int nt = min(p.rt, p.T - t0);
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
// scan kernel: 16 experts per workgroup of 256 threads. Thread (c, j) owns
// expert 16 * blockIdx.x + j over the c-th sixteenth of the route blocks:
// it sums its blocks, the 16 chunk sums of each expert are scanned in LDS,
// and the blocks are rewritten in place with their exclusive prefix (the
// first row of the block's pairs inside the expert's group).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scan_kernel(ScanParams p) {
  __shared__ int part[16][17];
  const int tid = threadIdx.x, j = tid & 15, c = tid >> 4;
  const int e = blockIdx.x * 16 + j;
  const int NB = p.NB, E = p.E;
  const int per = (NB + 15) / 16;
  const int b0 = min(c * per, NB), b1 = min(b0 + per, NB);
  int s = 0;
  if (e < E) {
#pragma unroll 8
    for (int b = b0; b < b1; ++b) s += p.blk_hist[static_cast<size_t>(b) * E + e];
  }
  part[c][j] = s;
  __syncthreads();
  if (tid < 16) {
    int r = 0;
    for (int cc = 0; cc < 16; ++cc) {
      const int v = part[cc][tid];
      part[cc][tid] = r;
      r += v;
    }
    if (e < E) p.counts[e] = r;
  }
  __syncthreads();
  if (e < E) {
    int base = part[c][j];
    for (int b = b0; b < b1; b += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = b + u < b1 ? p.blk_hist[static_cast<size_t>(b + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (b + u < b1) {
          p.blk_hist[static_cast<size_t>(b + u) * E + e] = base;
          base += v[u];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// scatter kernel: perm[offsets[e] + block base + local rank] = pair, inv[pair]
// = that row. Each workgroup scans the E counts itself; workgroup 0 also
// writes offsets and the grouped-GEMM tile table.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scatter_kernel(ScatterParams p) {
  __shared__ int offs[kMaxE + 1];
  __shared__ int tp[kMaxE + 1];
  __shared__ int flag[kMaxE + 1];
  __shared__ int tpos[kMaxE + 1];
  const int tid = threadIdx.x, E = p.E;
  if (tid < kWave) wave_exclusive_scan256(p.counts, offs, E);
  if (blockIdx.x == 0) {
    for (int e = tid; e < E; e += 256) tp[e] = (p.counts[e] + p.tile_m - 1) / p.tile_m;
    __syncthreads();
    if (tid < kWave) wave_exclusive_scan256(tp, tp, E);
    __syncthreads();
    for (int e = tid; e <= E; e += 256) p.offsets[e] = offs[e];
    write_tile_table(tp, E, p.max_tiles, p.tile_e, p.exp_tile0, p.meta);
    if (p.touched != nullptr)
      write_touched([&](int e) { return p.counts[e]; }, [&](int e) { return offs[e]; }, E, flag,
                    tpos, p.touched, p.meta);
  }
  __syncthreads();
  const int P = p.T * p.k;
  const int q = blockIdx.x * 256 + tid;
  if (q >= P) return;
  const int t = q / p.k;
  const int b = t / p.rt;
  const int e = min(max(p.ids[q], 0), E - 1);
  const int pos = offs[e] + p.blk_base[static_cast<size_t>(b) * E + e] + p.lrank[q];
  p.perm[pos] = q;
  p.inv[q] = pos;
}

// ---------------------------------------------------------------------------
// dispatch kernel: the scan and the scatter in one launch, for histograms of
// at most kDispHist entries. Each 1024-thread workgroup owns route blocks
// [bs, bs + bpw) and reads the whole [NB, E] block histogram once itself
// (thread (slice, e) sums blocks slice, slice + nsl, ... of expert e, all
// loads of a batch of 32 in flight): the sum over all blocks is the expert's
// count, the sum over blocks before bs the base of its first block (four
// experts per thread with 16-byte loads when E is a multiple of 4). Offsets
// are the exclusive scan of the counts; each owned block's base follows in
// block order; every owned pair gets perm[offs[e] + base + rank] = pair and
// inv[pair] = that row, as the scan and scatter kernels give. Workgroup 0
// also writes counts, offsets, the tile table and the touched table.
// ---------------------------------------------------------------------------
constexpr int DTHR = 1024;
__global__ __launch_bounds__(DTHR) void dispatch_kernel(ScanParams sp, ScatterParams p, int bpw) {
  // per (slice, expert) partial sums: nsl slices of W entries
  __shared__ int pre_s[4 * DTHR];
  __shared__ int tot_s[4 * DTHR];
  __shared__ int tot[kMaxE + 1];
  __shared__ int offs[kMaxE + 1];
  __shared__ int tp[kMaxE + 1];
  __shared__ int flag[kMaxE + 1];
  __shared__ int tpos[kMaxE + 1];
  __shared__ int base[kDispMaxOwn][kMaxE];
  const int tid = threadIdx.x, E = p.E, NB = sp.NB;
  const int bs = blockIdx.x * bpw, be = min(bs + bpw, NB);
  const int32_t* hist = sp.blk_hist;
  constexpr int BB = 32;  // loads of a batch, all in flight
  int nsl, W;
  if (E % 4 == 0) {
    // four experts per thread, 16-byte loads (rows of E ints stay aligned);
    // 16 in flight (1024 threads leave 128 registers a lane)
    constexpr int BV = 16;
    const int Eq = E / 4;
    const int Eqp = Eq <= 16 ? 16 : (Eq <= 32 ? 32 : 64);  // a power of two >= Eq
    nsl = DTHR / Eqp;
    W = 4 * Eqp;
    const int eq = tid & (Eqp - 1), sl = tid / Eqp;
    i32x4_t sum_pre = {0, 0, 0, 0}, sum_tot = {0, 0, 0, 0};
    if (eq < Eq) {
      for (int b0 = sl; b0 < NB; b0 += BV * nsl) {
        i32x4_t v[BV];
#pragma unroll
        for (int u = 0; u < BV; ++u) {
          const int b = min(b0 + u * nsl, NB - 1);
          v[u] = *reinterpret_cast<const i32x4_t*>(hist + static_cast<size_t>(b) * E + 4 * eq);
        }
#pragma unroll
        for (int u = 0; u < BV; ++u) pin(v[u]);
#pragma unroll
        for (int u = 0; u < BV; ++u) {
          const int b = b0 + u * nsl;
          if (b < NB) {
            sum_tot += v[u];
            if (b < bs) sum_pre += v[u];
          }
        }
      }
    }
    *reinterpret_cast<i32x4_t*>(&pre_s[sl * W + 4 * eq]) = sum_pre;
    *reinterpret_cast<i32x4_t*>(&tot_s[sl * W + 4 * eq]) = sum_tot;
  } else {
    const int Ep = E <= 64 ? 64 : (E <= 128 ? 128 : 256);  // a power of two >= E
    nsl = DTHR / Ep;
    W = Ep;
    const int e = tid & (Ep - 1), sl = tid / Ep;
    int sum_pre = 0, sum_tot = 0;
    if (e < E) {
      for (int b0 = sl; b0 < NB; b0 += BB * nsl) {
        int v[BB];
#pragma unroll
        for (int u = 0; u < BB; ++u) {
          const int b = min(b0 + u * nsl, NB - 1);
          v[u] = hist[static_cast<size_t>(b) * E + e];
        }
#pragma unroll
        for (int u = 0; u < BB; ++u) pin(v[u]);
#pragma unroll
        for (int u = 0; u < BB; ++u) {
          const int b = b0 + u * nsl;
          if (b < NB) {
            sum_tot += v[u];
            if (b < bs) sum_pre += v[u];
          }
        }
      }
    }
    pre_s[sl * W + e] = sum_pre;
    tot_s[sl * W + e] = sum_tot;
  }
  // the owned blocks' own counts
  for (int i = tid; i < (be - bs) * E; i += DTHR) {
    const int j = i / E, ee = i - j * E;
    base[j][ee] = hist[static_cast<size_t>(bs + j) * E + ee];
  }
  __syncthreads();
  if (tid < E) {
    int a = 0, t = 0;
    for (int q = 0; q < nsl; ++q) {
      a += pre_s[q * W + tid];
      t += tot_s[q * W + tid];
    }
    tot[tid] = t;
    for (int j = 0; j < be - bs; ++j) {
      const int v = base[j][tid];
      base[j][tid] = a;
      a += v;
    }
  }
  __syncthreads();
  if (tid < kWave) wave_exclusive_scan256(tot, offs, E);
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int ee = tid; ee < E; ee += DTHR) {
      sp.counts[ee] = tot[ee];
      tp[ee] = (tot[ee] + p.tile_m - 1) / p.tile_m;
    }
    __syncthreads();
    if (tid < kWave) wave_exclusive_scan256(tp, tp, E);
    __syncthreads();
    for (int ee = tid; ee <= E; ee += DTHR) p.offsets[ee] = offs[ee];
    write_tile_table(tp, E, p.max_tiles, p.tile_e, p.exp_tile0, p.meta);
    if (p.touched != nullptr)
      write_touched([&](int x) { return tot[x]; }, [&](int x) { return offs[x]; }, E, flag, tpos,
                    p.touched, p.meta);
  }
  const int q0 = bs * p.rt * p.k, q1 = min(be * p.rt, p.T) * p.k;
  for (int q = q0 + tid; q < q1; q += DTHR) {
    const int t = q / p.k;
    const int j = min(max(t / p.rt - bs, 0), bpw - 1);
    const int ex = min(max(p.ids[q], 0), E - 1);
    const int pos = offs[ex] + base[j][ex] + p.lrank[q];
    p.perm[pos] = q;
    p.inv[q] = pos;
  }
}

// ---------------------------------------------------------------------------
// tile table from offsets (one workgroup)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tiles_kernel(TilesParams p) {
  __shared__ int tp[kMaxE + 1];
  __shared__ int cnt[kMaxE + 1];
  __shared__ int first[kMaxE + 1];
  __shared__ int flag[kMaxE + 1];
  __shared__ int pos[kMaxE + 1];
  const int tid = threadIdx.x;
  if (tid < p.E) {
    // caller-provided offsets: counts clamped to [0, P] so the table stays in
    // bounds; the touched entries clamp rows the way the GEMMs do
    const int c = min(max(p.offsets[tid + 1] - p.offsets[tid], 0), p.P);
    const int r0 = min(max(p.offsets[tid], 0), p.P);
    first[tid] = r0;
    cnt[tid] = min(max(p.offsets[tid + 1], r0), p.P) - r0;
    tp[tid] = (c + p.tile_m - 1) / p.tile_m;
  }
  __syncthreads();
  if (tid < kWave) wave_exclusive_scan256(tp, tp, p.E);
  __syncthreads();
  write_tile_table(tp, p.E, p.max_tiles, p.tile_e, p.exp_tile0, p.meta);
  if (p.touched != nullptr)
    write_touched([&](int e) { return cnt[e]; }, [&](int e) { return first[e]; }, p.E, flag, pos,
                  p.touched, p.meta);
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
  if (p.rt == kRouteTokensMax) {
    if (dtype == MOE_BF16) route_kernel<NCH, true, kRouteTokensMax><<<nb, RTHR, 0, s>>>(p);
    else route_kernel<NCH, false, kRouteTokensMax><<<nb, RTHR, 0, s>>>(p);
  } else {
    if (dtype == MOE_BF16) route_kernel<NCH, true, kRouteTokensMin><<<nb, RTHR, 0, s>>>(p);
    else route_kernel<NCH, false, kRouteTokensMin><<<nb, RTHR, 0, s>>>(p);
  }
}

hipError_t launch_route(const RouteParams& p, int dtype, hipStream_t s) {
  if (p.rt != kRouteTokensMax && p.rt != kRouteTokensMin) return hipErrorInvalidValue;
  const int nb = ceil_div(p.T, p.rt);
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

template <int NCH>
static void launch_finish_nch(const RouteParams& p, hipStream_t s) {
  route_finish_kernel<NCH><<<1, RTHR, 0, s>>>(p);
}

hipError_t launch_route_part(const RouteParams& p, int dtype, hipStream_t s) {
  const int cols = p.E + (p.w_sgate != nullptr ? 1 : 0);
  if (p.T < 1 || p.T > RTM || p.part == nullptr || p.ncp != ceil_div(cols, 16) * 16)
    return hipErrorInvalidValue;
  const dim3 grid(p.ncp / 16, ceil_div(p.T, 16));
  if (dtype == MOE_BF16) route_part_kernel<true><<<grid, RTHR, 0, s>>>(p);
  else route_part_kernel<false><<<grid, RTHR, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_route_split(const RouteParams& p, int dtype, hipStream_t s) {
  const hipError_t err = launch_route_part(p, dtype, s);
  if (err != hipSuccess) return err;
  const int cols = p.E + (p.w_sgate != nullptr ? 1 : 0);
  if (p.T <= kTinyT && p.E <= kWave) {
    route_tiny_kernel<<<1, kTinyT * kWave, 0, s>>>(p);
    return hipGetLastError();
  }
  switch (ceil_div(cols, 64)) {
    case 1: launch_finish_nch<1>(p, s); break;
    case 2: launch_finish_nch<2>(p, s); break;
    case 3: launch_finish_nch<3>(p, s); break;
    case 4: launch_finish_nch<4>(p, s); break;
    case 5: launch_finish_nch<5>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rank(const RankParams& p, hipStream_t s) {
  if (p.rt < 1 || p.rt > RTM) return hipErrorInvalidValue;
  rank_kernel<<<ceil_div(p.T, p.rt), 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanParams& p, hipStream_t s) {
  scan_kernel<<<ceil_div(p.E, 16), 256, 0, s>>>(p);
  return hipGetLastError();
}

int dispatch_blocks_per_wg(int NB) { return min(kDispMaxOwn, max(1, ceil_div(NB, 64))); }

bool dispatch_fused(int NB, int E) {
  return NB <= 64 * kDispMaxOwn && static_cast<long long>(NB) * E <= kDispHist;
}

hipError_t launch_dispatch(const ScanParams& sp, const ScatterParams& p, hipStream_t s) {
  if (!dispatch_fused(sp.NB, p.E) || sp.NB != ceil_div(p.T, p.rt) || sp.E != p.E)
    return hipErrorInvalidValue;
  const int bpw = dispatch_blocks_per_wg(sp.NB);
  dispatch_kernel<<<ceil_div(sp.NB, bpw), DTHR, 0, s>>>(sp, p, bpw);
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
