// Grouped expert GEMMs for the sparse MoE layer forward (gfx950), and two
// products of the layer backward on the same 256-row tiles: the recomputed
// gate/up product (kind 2) and the dx rows (kind 3).
//
// Each workgroup computes one (expert, M tile, N tile) block of
//   gate/up: act[r, n] = silu(sum_i x[t_r, i] W_g[e, n, i]) * (sum_i x[t_r, i] W_u[e, n, i])
//   down:    y[r, n]   = sum_j act[r, j] W_d[e, n, j]
// for the sorted rows r of expert e ("Tutorial 11: Mixture of Experts (MoE)",
// section 3, step 2: each expert's SwiGLU runs on its own rows only). Rows
// of x are read in place through the sorted dispatch table (t_r = perm[r] / k),
// so no per-token copy of x or of the weights is ever built.
//
// bf16 path: v_mfma_f32_16x16x32_bf16 with fp32 accumulation; each wave owns
// a 64-row x 16*NFW-column block of a workgroup tile of NWM x NWN waves. K is
// streamed through an S-stage LDS pipeline of direct global->LDS loads, each
// stage a 32- or 64-deep K slice of the tile's A rows and weight rows (LDS
// rows XOR-swizzled so the fragment reads are bank-conflict free). 64-deep
// slices read 128 contiguous bytes of every row per stage, which the L2
// delivers at about 1.6x the rate of 64-byte segments; they pay when a
// workgroup has 8 waves to cover the larger stages. The gate/up epilogue
// applies the SiLU product before the single rounding to bf16.
// fp32 path: one thread per output element (small fp32 layers only).
//
// The launch grid is sized from an upper bound on the tile count; the true
// count is read on the device, so no host synchronisation is needed. Tiles
// are numbered expert-major, in blocks of 4 M tiles x all N tiles, and each
// XCD (block b runs on XCD b mod 8) takes one contiguous eighth of them:
// consecutive logical tiles (the M tiles that share one weight slab) land on
// the same XCD and its L2. The shared group, whose down-projection tiles
// carry a longer reduction than the routed ones, is divided into eighths of
// its own and scheduled first, so every XCD gets the same share of it.

#include <utility>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

struct TileInfo {
  int e;          // expert, or -1 for the shared group
  int row0, nrows;
  int n0;
};

// Local tile index -> (n, m) for a group of mt M tiles x NT N tiles, in
// blocks of up to 4 M tiles: within a block N runs slowest and M fastest, so
// ~32 consecutive tiles (the ones an XCD runs at the same time) touch at most
// 4 distinct A slabs and 8 distinct B slabs.
__device__ __forceinline__ void grouped_nm(int l, int mt, int NT, int& n, int& m) {
  constexpr int G = 4;
  const int full = mt / G;
  const int in_full = full * G * NT;
  if (l < in_full) {
    const int g = l / (G * NT);
    const int r = l - g * G * NT;
    n = r / G;
    m = g * G + (r - n * G);
  } else {
    const int r = l - in_full;
    const int g2 = mt - full * G;
    n = r / g2;
    m = full * G + (r - n * g2);
  }
}

// Decodes the logical tile of this workgroup; returns false for surplus blocks.
// Blocks [0, 8 * ceil(nsh / 8)) run the nsh shared-group tiles, the rest the
// routed ones; each region is split into per-XCD eighths.
template <int BN>
__device__ __forceinline__ bool decode_tile(const GemmParams& p, TileInfo& ti) {
  const int BM = p.tile_m;
  const int ntiles = p.meta != nullptr ? p.meta[0] : 0;  // null: shared group only
  const int NT = (p.N + BN - 1) / BN;
  const int routed = NT * ntiles;
  int MTs = 0, NTs = 0;
  if (p.shared_T > 0) {
    MTs = (p.shared_T + BM - 1) / BM;
    NTs = (p.sN + BN - 1) / BN;
  }
  const int nsh = MTs * NTs;
  const int pers = (nsh + 7) >> 3;
  int b = blockIdx.x;
  int n, m;
  if (b < 8 * pers) {
    const int L = (b & 7) * pers + (b >> 3);
    if (L >= nsh) return false;
    grouped_nm(L, MTs, NTs, n, m);
    ti.e = -1;
    ti.row0 = m * BM;
    ti.nrows = min(BM, p.shared_T - ti.row0);
    ti.n0 = n * BN;
    return ti.nrows > 0;
  }
  b -= 8 * pers;
  const int per = (routed + 7) >> 3;
  const int j = b >> 3;
  if (j >= per) return false;
  const int L = (b & 7) * per + j;
  if (L >= routed) return false;
  const int q = L / NT;
  const int e = p.tile_e[q];
  const int tp0 = p.exp_tile0[e];
  const int mt = p.exp_tile0[e + 1] - tp0;
  grouped_nm(L - NT * tp0, mt, NT, n, m);
  // offsets clamped to [0, P]: caller-provided tables cannot push rows out of bounds
  const int o0 = min(max(p.offsets[e], 0), p.P), o1 = min(max(p.offsets[e + 1], 0), p.P);
  ti.e = e;
  ti.row0 = o0 + m * BM;
  ti.nrows = min(BM, o1 - ti.row0);
  ti.n0 = n * BN;
  return ti.nrows > 0;
}

// KIND 2, the layer backward's gate/up product: z = x W_{g|u}^T recomputed
// (never stored). With the hidden-unit gradient da' (bf16, written by the
// backward's earlier product) and the gate g of each row -- the routed
// pair's gate, or the shared expert's sigmoid gate -- the epilogue forms,
// per (row, hidden unit),
//   g a = g silu(z_g) z_u                                 (bf16, for dW_down),
//   dz_g = g da' z_u silu'(z_g),  dz_u = g da' silu(z_g)   (bf16),
// and per 32 hidden units the partial sum of da' a (the gate gradient): the
// arithmetic of the backward's own z product, on 256-row tiles. The bf16
// outputs of each wave's 16-row blocks go through its 6 KB slice of the
// idle first stage buffer and out 16 bytes per lane.
__device__ __forceinline__ float zrow16_sum(float v) {
  v += __shfl_xor(v, 1, kWave);
  v += __shfl_xor(v, 2, kWave);
  v += __shfl_xor(v, 4, kWave);
  v += __shfl_xor(v, 8, kWave);
  return v;
}

template <int NWM, int NWN, int NFW>
__device__ __forceinline__ void z_epilogue(const GemmParams& p, const TileInfo& ti,
                                           floatx4_t (&acc)[4][NFW], uint16_t* L0) {
  static_assert(NFW == 8, "a wave holds 64 hidden units: 4 gate and 4 up fragments");
  static_assert(NWM * NWN * 3072 * 2 <= (NWM * 64 + NWN * NFW * 16) * 64 * 2, "slices fit L0");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % NWM, wn = wave / NWM;
  const int fr = lane & 15, fq = lane >> 4;
  const bool sh = ti.e < 0;
  const int H = sh ? p.sN : p.N;
  const uint16_t* dh = sh ? p.zdh_s : p.zdh;
  uint16_t* ga = sh ? p.zga_s : p.zga;
  uint16_t* dz = sh ? p.zdz_s : p.zdz;
  float* part = sh ? p.zpart_s : p.zpart;
  const int npart = sh ? p.znpart_s : p.znpart;
  const int hu0 = ti.n0 + wn * 64;   // first hidden unit of the wave
  uint16_t* gaS = L0 + wave * 3072;  // [16][64]
  uint16_t* dzS = gaS + 1024;        // [16][128]: gate units, then up units
  // the wave's da' values and gates, all loads issued together (rows past
  // the group reread the last row, units past H the last unit: never used)
  float c[4][4][4];
  float g[4][4];
#pragma unroll
  for (int mf = 0; mf < 4; ++mf)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rt = min(wm * 64 + mf * 16 + fq * 4 + i, ti.nrows - 1);
      const int r = ti.row0 + rt;
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
        c[mf][i][nf] = bf16_to_f32(dh[static_cast<size_t>(r) * H + min(hu0 + nf * 16 + fr, H - 1)]);
      if (sh) g[mf][i] = p.zsgate != nullptr ? p.zsgate[r] : 1.0f;
      else g[mf][i] = p.zgates[min(max(p.perm[r], 0), p.P - 1)];
    }
#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = fq * 4 + i;  // row within the 16-row block
      const int rt = wm * 64 + mf * 16 + lr;
      const bool rok = rt < ti.nrows;
      float dot0 = 0.f, dot1 = 0.f;
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const int hu = hu0 + nf * 16 + fr;
        const float zg = acc[mf][nf][i], zu = acc[mf][nf + 4][i];
        const float sgm = 1.0f / (1.0f + expf(-zg));  // sigmoid(z_g)
        const float sg = zg * sgm;                     // silu(z_g)
        const float a = sg * zu;
        const float cv = (rok && hu < H) ? c[mf][i][nf] : 0.f;
        if (nf < 2) dot0 += cv * a;
        else dot1 += cv * a;
        const float da = g[mf][i] * cv;
        const int col = nf * 16 + fr;
        gaS[lr * 64 + col] = f32_to_bf16(g[mf][i] * a);
        dzS[lr * 128 + col] = f32_to_bf16(da * zu * (sgm * (1.0f + zg * (1.0f - sgm))));
        dzS[lr * 128 + 64 + col] = f32_to_bf16(da * sg);
      }
      dot0 = zrow16_sum(dot0);
      dot1 = zrow16_sum(dot1);
      const int grp = hu0 / 32;
      if (rok && fr == 0) {
        const size_t pr = static_cast<size_t>(ti.row0 + rt) * npart;
        if (grp < npart) part[pr + grp] = dot0;
        if (grp + 1 < npart) part[pr + grp + 1] = dot1;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
    // g a: 16 rows x 8 chunks; dz: 16 rows x 16 chunks (8 gate, 8 up)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = j * 64 + lane, lr = q >> 3, ch = q & 7;
      const int rt = wm * 64 + mf * 16 + lr;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(gaS + lr * 64 + ch * 8);
      if (rt < ti.nrows && hu0 + ch * 8 < H)
        *reinterpret_cast<u32x4_t*>(ga + static_cast<size_t>(ti.row0 + rt) * H + hu0 + ch * 8) = v;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = j * 64 + lane, lr = q >> 4, c16 = q & 15;
      const int rt = wm * 64 + mf * 16 + lr;
      const int u = hu0 + (c16 & 7) * 8;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(dzS + lr * 128 + c16 * 8);
      if (rt < ti.nrows && u < H)
        *reinterpret_cast<u32x4_t*>(dz + static_cast<size_t>(ti.row0 + rt) * (2 * H) + (c16 < 8 ? 0 : H) + u) = v;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the slice is rewritten
  }
}

// KIND 3, the layer backward's dx rows: dx_r = dz_g[r] W_g[e] + dz_u[r] W_u[e]
// (K = 2H: the gate units, then the up units; N = d), each row written at its
// pair's row in bf16 (routed; like the forward's y rows, they are added in
// float32 by the final sum) or at its token's row in float32 (shared), so
// that a token's rows sit together for the final sum. B is stored with K as its row
// index (W_g and W_u rows are hidden units, contiguous along d): a stage
// holds 64 K rows of the tile's 256 columns as stored, 16-byte chunk c of K
// row k at position c ^ kar_swz(k), and the MFMA operand is built with two
// transposing reads (ds_read_b64_tr_b16) per fragment. A fragment read takes
// K rows 8 g + 4 h + q (lane group g, lane quad q) of 32 consecutive K; their
// chunk positions differ in the low four bits, so the read meets each bank
// twice (the minimum for 512 bytes).
__device__ __forceinline__ int kar_swz(int k) { return (k & 3) | (((k >> 3) & 3) << 2); }
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
// Workgroup barrier for LDS traffic alone (no fence: loads stay in flight).
__device__ __forceinline__ void lds_barrier_g() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The dx rows' epilogue: each wave stages its 64 x 128 float32 block 16 rows
// at a time through its 8 KB slice of the idle first stage buffer (16-byte
// chunks XOR-swizzled by bits 2..3 of the row: conflict-free writes) and
// stores 16 bytes per lane.
template <int NWM, int NWN, int NFW>
__device__ __forceinline__ void dxr_epilogue(const GemmParams& p, const TileInfo& ti,
                                             floatx4_t (&acc)[4][NFW], uint16_t* L0) {
  constexpr int WC = NFW * 16;  // output columns per wave
  static_assert(NWM * NWN * 16 * WC * 4 <= (NWM * 64 + NWN * NFW * 16) * 64 * 2, "slices fit L0");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % NWM, wn = wave / NWM;
  const int fr = lane & 15, fq = lane >> 4;
  const bool sh = ti.e < 0;
  const int N = sh ? p.sN : p.N;
  float* Cw = reinterpret_cast<float*>(L0) + wave * 16 * WC;
  const int c0 = ti.n0 + wn * WC;
#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rc = fq * 4 + i;
#pragma unroll
      for (int nf = 0; nf < NFW; ++nf) {
        const int ch = nf * 4 + (fr >> 2);
        Cw[rc * WC + ((ch ^ (fq << 2)) << 2) + (fr & 3)] = acc[mf][nf][i];
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
#pragma unroll
    for (int pass = 0; pass < 16 * WC / 4 / 64; ++pass) {
      const int idx = pass * 64 + lane;
      const int rc = idx / (WC / 4), ch = idx % (WC / 4);
      const int rt = wm * 64 + mf * 16 + rc;
      const float4 v = *reinterpret_cast<const float4*>(Cw + rc * WC + ((ch ^ (((rc >> 2) & 3) << 2)) << 2));
      if (rt < ti.nrows && c0 + ch * 4 < N) {
        const int r = ti.row0 + rt;
        if (sh) {
          *reinterpret_cast<float4*>(static_cast<float*>(p.sout) + static_cast<size_t>(r) * N + c0 +
                                     ch * 4) = v;
        } else {
          const int orow = min(max(p.perm[r], 0), p.P - 1);
          const uint2 o = {static_cast<uint32_t>(f32_to_bf16(v.x)) |
                               (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16),
                           static_cast<uint32_t>(f32_to_bf16(v.z)) |
                               (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16)};
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + static_cast<size_t>(orow) * N +
                                    c0 + ch * 4) = o;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the slice is rewritten
  }
}

// KIND 0: gate/up: B rows [0, GBR / 2) are gate rows n0.., [GBR / 2, GBR)
//   the up rows of the same hidden units; N tile GBR / 2 hidden units.
// KIND 1: down: B rows [0, GBR) are output columns n0..; N tile GBR.
// NWM x NWN waves of 64 rows x 16 * NFW B rows each (BM = 64 * NWM,
// GBR = 16 * NFW * NWN); S-stage pipeline of 32-deep K slices loaded by
// direct global->LDS loads (global_load_lds_dwordx4), one stage per LDS
// array so the compiler tracks each stage's loads separately. Every lane
// issues every load (addresses clamped into the operand) so the wave's
// outstanding-load count is the same on every path, and a stage is known to
// have landed once at most (S - 2) stages' loads are outstanding.
// LDS destination of a direct global->LDS load of 4-byte words, hidden from
// the compiler's load-counter tracking: the one wave that issues these loads
// reads them back after an explicit wait.
__device__ __forceinline__ lds_void_t* lds_untracked_i32(int32_t* q) {
  lds_void_t* r = (lds_void_t*)q;
  asm volatile("" : "+s"(r));
  return r;
}

template <int KIND, int NWM, int NWN, int NFW, int S, int BK>
__global__ __launch_bounds__(NWM * NWN * 64) void gemm_bf16_kernel(GemmParams p) {
  static_assert(BK == 32 || BK == 64, "K slice of 32 or 64 (64- or 128-byte row segments)");
  constexpr int CPR = BK / 8;                   // 16-byte chunks per LDS row
  constexpr int KS = BK / 32;                   // MFMA K steps per stage
  constexpr int NTHR = NWM * NWN * 64;
  constexpr int BM = NWM * 64;
  constexpr int GBR = NWN * NFW * 16;           // B rows per tile
  constexpr int HB = GBR / 2;                   // gate/up: hidden units per tile
  constexpr bool GU = KIND == 0 || KIND == 2;   // gate and up rows (gate/up, backward z)
  constexpr bool KAR = KIND == 3;               // B with K as its row index (backward dx rows)
  static_assert(!KAR || (BK == 64 && NWN == 2 && NFW == 8), "K-as-row stages of 64 x 256");
  constexpr int BN = GU ? HB : GBR;             // output columns per tile
  constexpr int SA = BM * BK;                   // A elements per stage
  constexpr int SEL = SA + GBR * BK;            // elements per stage
  constexpr int LA = SA / 8 / NTHR;             // 16-byte A loads per thread per stage
  constexpr int LB = GBR * BK / 8 / NTHR;       // B loads per thread per stage
  constexpr int LPS = LA + LB;
  static_assert(LA * NTHR * 8 == SA && LB * NTHR * 8 == GBR * BK, "whole loads per thread");
  static_assert(!GU || NFW % 2 == 0, "gate/up pairs gate and up fragments");
  static_assert(S >= 2 && S <= 8, "stages");
  static_assert((S - 2) * LPS < 64, "vmcnt range");
  __shared__ __align__(16) uint16_t L0[SEL];
  __shared__ __align__(16) uint16_t L1[SEL];
  __shared__ __align__(16) uint16_t L2[S > 2 ? SEL : 8];
  __shared__ __align__(16) uint16_t L3[S > 3 ? SEL : 8];
  __shared__ __align__(16) uint16_t L4[S > 4 ? SEL : 8];
  __shared__ __align__(16) uint16_t L5[S > 5 ? SEL : 8];
  __shared__ __align__(16) uint16_t L6[S > 6 ? SEL : 8];
  __shared__ __align__(16) uint16_t L7[S > 7 ? SEL : 8];
  __shared__ __align__(16) int32_t Pg[NTHR / 64 * LA * 64];  // perm words of each wave's A rows
  // stage i lives in its own LDS array (static index after unrolling), so the
  // compiler can tell one stage's DMA from another stage's fragment reads
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

  TileInfo ti;
  if (!decode_tile<BN>(p, ti)) return;
  const bool shared = ti.e < 0;
  const int K = shared ? p.sK : p.K;
  const int N = shared ? p.sN : p.N;
  const uint16_t* A = static_cast<const uint16_t*>(shared ? p.sa : p.a);
  const uint16_t* B0 = static_cast<const uint16_t*>(shared ? p.sb0 : p.b0);
  const uint16_t* B1 = static_cast<const uint16_t*>(shared ? p.sb1 : p.b1);
  uint16_t* OUT = static_cast<uint16_t*>(shared ? p.sout : p.out);
  if (!shared) {
    // dx rows: W_g and W_u are [H, N] each with K = 2H
    const size_t wstride = static_cast<size_t>(N) * (KAR ? K / 2 : K);
    B0 += static_cast<size_t>(ti.e) * wstride;
    if (GU || KAR) B1 += static_cast<size_t>(ti.e) * wstride;
  }

  const int tid = threadIdx.x;
  const int wbase = tid & ~63;  // first thread of this wave
  // Load i of this thread fills LDS slot q = i * NTHR + tid: row q / CPR,
  // physical chunk tid % CPR (the swizzle decides which logical chunk).
  // A source rows: gate/up gathers x rows through perm. The perm entries go
  // out first (direct-to-LDS, one 4-byte word per lane into this wave's
  // block of Pg), the weight slices of the prologue are issued while they
  // are in flight, and only then are the A addresses formed.
  const uint16_t* asrc[LA];
  int achunk[LA], asrow[LA];
  const bool gather = GU && !shared;
  const int uwave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = (i * NTHR + tid) / CPR;
    achunk[i] = swz_phys_to_logical<BK>(r, tid % CPR) * 8;
    const int rr = r < ti.nrows ? r : 0;  // rows past the group reload row 0 (never stored)
    asrow[i] = ti.row0 + rr;
    if (gather) {
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(p.perm + asrow[i]),
                                       lds_untracked_i32(&Pg[(uwave * LA + i) * 64]), 4, 0, 0);
    }
  }
  auto form_a = [&]() {
    if (gather) {
      // this wave's perm words are in: all its loads but the prologue's
      // weight halves are done
      wait_stage<(S - 1) * LB>();
#pragma unroll
      for (int i = 0; i < LA; ++i) asrow[i] = Pg[(uwave * LA + i) * 64 + (tid & 63)];
    }
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int src = gather ? min(max(asrow[i] / p.k, 0), p.a_rows - 1) : asrow[i];
      asrc[i] = A + static_cast<size_t>(src) * K;
    }
  };
  const uint16_t* bsrc[KAR ? 1 : LB];
  int bchunk[KAR ? 1 : LB];
  if constexpr (!KAR) {
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int r = (i * NTHR + tid) / CPR;
      bchunk[i] = swz_phys_to_logical<BK>(r, tid % CPR) * 8;
      int n;
      const uint16_t* base;
      if (GU) { n = ti.n0 + (r < HB ? r : r - HB); base = r < HB ? B0 : B1; }
      else { n = ti.n0 + r; base = B0; }
      n = n < N ? n : N - 1;  // columns past N reload a valid row (never stored)
      bsrc[i] = base + static_cast<size_t>(n) * K;
    }
  }

  const int nk = (K + BK - 1) / BK;
  const bool ktail = (K % BK) != 0;
  auto issue_a = [&](uint16_t* st, int kc) __attribute__((always_inline)) {
    const int k0 = min(kc, nk - 1) * BK;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int kk = min(k0 + achunk[i], K - 8);
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(asrc[i] + kk),
                                       (lds_void_t*)(st + (i * NTHR + wbase) * 8), 16, 0, 0);
    }
  };
  auto issue_b = [&](uint16_t* st, int kc) __attribute__((always_inline)) {
    const int k0 = min(kc, nk - 1) * BK;
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const uint16_t* src;
      if constexpr (KAR) {
        // slot i * NTHR + tid: K row kr = its index / 32 (256 columns per K
        // row), physical chunk tid % 32; K row k is gate unit k or up unit
        // k - K / 2 (rows past K reread the last; columns past N a valid one)
        const int kr = i * (NTHR / 32) + (tid >> 5);
        const int col = min(ti.n0 + (((tid & 31) ^ kar_swz(kr)) << 3), N - 8);
        const int k = min(k0 + kr, K - 1);
        const int HK = K / 2;
        const bool up = k >= HK;
        src = (up ? B1 : B0) + static_cast<size_t>(up ? k - HK : k) * N + col;
      } else {
        src = bsrc[i] + min(k0 + bchunk[i], K - 8);
      }
      __builtin_amdgcn_global_load_lds((gbl_void_t*)src,
                                       (lds_void_t*)(st + SA + (i * NTHR + wbase) * 8), 16, 0, 0);
    }
  };
  auto issue = [&](uint16_t* st, int kc) __attribute__((always_inline)) {
    issue_a(st, kc);
    issue_b(st, kc);
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % NWM, wn = wave / NWM;
  const int fr = lane & 15, fq = lane >> 4;
  floatx4_t acc[4][NFW];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NFW; ++b) acc[a][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // fragment offsets within a stage (the same for every stage), per MFMA K step
  int aoff[KS][4], boff[KAR ? 1 : KS][NFW];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int mf = 0; mf < 4; ++mf) aoff[ks][mf] = swz<BK>(wm * 64 + mf * 16 + fr, ks * 4 + fq);
    if constexpr (!KAR) {
#pragma unroll
      for (int nf = 0; nf < NFW; ++nf) {
        int r;
        if (GU) {
          constexpr int H = NFW / 2;  // gate fragments per wave (the up ones follow)
          r = (nf < H ? 0 : HB) + wn * H * 16 + (nf % H) * 16 + fr;
        } else {
          r = wn * NFW * 16 + nf * 16 + fr;
        }
        boff[ks][nf] = SA + swz<BK>(r, ks * 4 + fq);
      }
    }
  }
  // K-as-row B: lane (group g, quad q, r) reads K row 32 ks + 8 g + 4 h + q
  // at columns 16 nf + 4 r .. + 3 of the wave's 128; with s = kar_swz of
  // that row (the same for every ks and h), the chunk position is
  // (wn * 16 + 2 nf + r / 2) ^ s = wn * 16 + 2 (nf ^ (s >> 1)) + (r / 2 ^ (s & 1))
  int kbase = 0, ksw = 0;  // K row 8 g + q, h = 0, ks = 0; the rest are constant offsets
  if constexpr (KAR) {
    const int g = lane >> 4, q = (lane >> 2) & 3, r = lane & 3;
    const int sw = q | (g << 2);
    ksw = sw >> 1;
    kbase = SA + (8 * g + q) * GBR + wn * 128 + (((r >> 1) ^ (sw & 1)) << 3) + 4 * (r & 1);
  }

  auto compute = [&](const uint16_t* st) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t af[4], bf[NFW];
#pragma unroll
      for (int mf = 0; mf < 4; ++mf)
        af[mf] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(st + aoff[ks][mf]));
#pragma unroll
      for (int nf = 0; nf < NFW; ++nf) {
        if constexpr (KAR) {
          const uint16_t* b = st + kbase + ((nf ^ ksw) << 4) + ks * 32 * GBR;
          struct { v4i16_t lo, hi; } pr = {
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)b),
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(b + 4 * GBR))};
          bf[nf] = __builtin_bit_cast(bf16x8_t, pr);
        } else {
          bf[nf] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(st + boff[ks][nf]));
        }
      }
#pragma unroll
      for (int mf = 0; mf < 4; ++mf)
#pragma unroll
        for (int nf = 0; nf < NFW; ++nf)
          acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mf], bf[nf], acc[mf][nf], 0, 0, 0);
    }
  };

  // Wait for this wave's loads of stage kc. The prologue issues the weight
  // halves of stages 0..S-2 first and their A halves after, so before step
  // S - 2 the loads newer than A(kc) are A(kc+1..S-2) and the kc earlier
  // steps' stages; from step S - 2 on, S - 2 whole stages.
  auto wait_for = [&](int kc) {
    if (kc >= S - 2) {
      wait_stage<(S - 2) * LPS>();
      return;
    }
    [&]<int... J>(std::integer_sequence<int, J...>) {
      ((kc == J ? wait_stage<(S - 2 - J) * LA + J * LPS>() : void()), ...);
    }(std::make_integer_sequence<int, S - 2>{});
  };
  // One pipeline step: stage kc lives in `cur`; `nxt` receives stage kc + S - 1.
  auto step = [&](int kc, uint16_t* cur, uint16_t* nxt) __attribute__((always_inline)) {
    wait_for(kc);
    stage_barrier();
    issue(nxt, kc + S - 1);
    if (kc < nk) {
      if (ktail && kc == nk - 1) {
        // last, partial K chunk: zero A's columns past K (B's clamped
        // duplicates then multiply zeros)
        const int k0 = kc * BK;
#pragma unroll
        for (int i = 0; i < LA; ++i) {
          if (k0 + achunk[i] >= K)
            *reinterpret_cast<u32x4_t*>(cur + (i * NTHR + tid) * 8) = u32x4_t{0u, 0u, 0u, 0u};
        }
        __syncthreads();
      }
      compute(cur);
    }
  };

  [&]<int... I>(std::integer_sequence<int, I...>) {
    // prologue: weight halves of stages 0 .. S-2, then (perm in hand) their A halves
    ((I < S - 1 ? issue_b(buf.template operator()<I>(), I) : void()), ...);
    form_a();
    ((I < S - 1 ? issue_a(buf.template operator()<I>(), I) : void()), ...);
    for (int kb = 0; kb < nk; kb += S) {
      (step(kb + I, buf.template operator()<I>(), buf.template operator()<(I + S - 1) % S>()), ...);
    }
  }(std::make_integer_sequence<int, S>{});
  // drain the clamped loads past the last stage before L0 is reused
  __syncthreads();
  if constexpr (KIND == 2) {
    z_epilogue<NWM, NWN, NFW>(p, ti, acc, L0);
    return;
  }
  if constexpr (KIND == 3) {
    dxr_epilogue<NWM, NWN, NFW>(p, ti, acc, L0);
    return;
  }

  // epilogue: each wave stages its own sub-tile through a private slice of
  // L0, 16 rows at a time, so every lane stores 16 contiguous bytes of an
  // output row; no block barrier is needed (a wave reads only what it wrote).
  constexpr int WC = KIND == 0 ? NFW * 8 : NFW * 16;  // output columns per wave
  constexpr int WLD = WC + 8;
  constexpr int LPR = WC / 8;      // lanes per output row
  constexpr int NPASS = (16 * LPR + 63) / 64;
  // the waves' slices fill one stage buffer, or the first two
  constexpr bool SPLIT = NWM * NWN * 16 * WLD > SEL;
  constexpr int NWH = SPLIT ? NWM * NWN / 2 : NWM * NWN;
  static_assert(NWH * 16 * WLD <= SEL, "epilogue slices must fit in two stage buffers");
  uint16_t* Cw = (SPLIT && wave >= NWH ? L1 : L0) + (wave % NWH) * 16 * WLD;
  const int c0 = ti.n0 + wn * WC;  // first output column of this wave
#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rc = fq * 4 + i;
      if (KIND == 0) {
#pragma unroll
        for (int nf = 0; nf < NFW / 2; ++nf)
          Cw[rc * WLD + nf * 16 + fr] = f32_to_bf16(silu_fast(acc[mf][nf][i]) * acc[mf][nf + NFW / 2][i]);
      } else {
#pragma unroll
        for (int nf = 0; nf < NFW; ++nf) Cw[rc * WLD + nf * 16 + fr] = f32_to_bf16(acc[mf][nf][i]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
      const int idx = pass * 64 + lane;
      const int rc = idx / LPR, ch = (idx % LPR) * 8;
      const int rt = wm * 64 + mf * 16 + rc;
      if (idx < 16 * LPR && rt < ti.nrows && c0 + ch < N) {
        *reinterpret_cast<u32x4_t*>(OUT + static_cast<size_t>(ti.row0 + rt) * N + c0 + ch) =
            *reinterpret_cast<const u32x4_t*>(Cw + rc * WLD + ch);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the slice is rewritten
  }
}

// ---------------------------------------------------------------------------
// Weight gradients of the layer backward on 256 x 256 tiles:
//   KIND 4: dW_{g|u}[e][m][n] = sum_r dz[r][m] x[t_r][n]  (M = 2H: the gate
//           rows, then the up rows; N = d),
//   KIND 5: dW_d[e][i][j]    = sum_r dO[t_r][i] (g a)[r][j]  (M = d; N = H),
// summed over the sorted rows r of expert e (t_r = perm[r] / k; the shared
// expert: every token; the row tokens come from the rtok table). Both
// operands are rows indexed by the reduction, so both land in LDS as stored,
// BK rows of the tile's 256 columns per stage of an S-stage ring, in the
// layout of the dx rows' B operand (chunk c of row k at c ^ kar_swz(k)), and
// both MFMA operands are built by transposing reads. The gathered operand's
// tokens (x for KIND 4, dO for KIND 5) are scalar loads made one stage
// ahead. Rows past the expert's count reread its last row and are zeroed in
// A after they land; experts without rows write zeros. Tiles run shared ones
// first, then routed ones expert by expert (grouping an M tile's column tiles
// on one XCD measured the same); the float32 outputs leave through the dx
// rows' staging.
// ---------------------------------------------------------------------------
template <int KIND, int S, int BK>
__global__ __launch_bounds__(512) void gemm_wgrad_kernel(GemmParams p) {
  constexpr int NWM = 4, NFW = 8, KS = BK / 32, NTHR = 512;  // 4 x 2 waves of 64 x 128
  constexpr int BM = 256, BN = 256;
  constexpr int SA = BK * BM, SEL = SA + BK * BN;  // bf16 per stage
  constexpr int LA = SA / 8 / NTHR;                 // 16-byte loads per thread per operand and stage
  constexpr int LPS = 2 * LA;
  static_assert(BK == 32 || BK == 64, "K slices of 32 or 64 rows");
  static_assert(S >= 2 && S <= 4 && (S - 2) * LPS < 64, "stages");
  constexpr bool GATHER_A = KIND == 5, GATHER_B = KIND == 4;
  // one LDS array per stage (static indices after unrolling), so the
  // compiler can tell one stage's direct loads from another's reads
  __shared__ __align__(16) uint16_t L0[SEL];
  __shared__ __align__(16) uint16_t L1[SEL];
  __shared__ __align__(16) uint16_t L2[S > 2 ? SEL : 8];
  __shared__ __align__(16) uint16_t L3[S > 3 ? SEL : 8];
  auto buf = [&]<int I>() -> uint16_t* {
    if constexpr (I == 0) return L0;
    else if constexpr (I == 1) return L1;
    else if constexpr (I == 2) return L2;
    else return L3;
  };

  // ---- tile: shared tiles first, then E x MT x NT routed ones
  const bool has_sh = p.shared_T > 0;
  const int MTs = has_sh ? (p.sM + BM - 1) / BM : 0, NTs = has_sh ? (p.sN + BN - 1) / BN : 0;
  const int nsh = MTs * NTs;
  const int MT = (p.M + BM - 1) / BM, NT = (p.N + BN - 1) / BN;
  int b = blockIdx.x;
  bool sh;
  int e, mt, nt;
  if (b < nsh) {
    sh = true; e = -1; mt = b / NTs; nt = b - mt * NTs;
  } else {
    b -= nsh;
    sh = false; e = b / (MT * NT);
    if (e >= p.E) return;
    const int r = b - e * (MT * NT);
    mt = r / NT; nt = r - mt * NT;
  }
  const int M = sh ? p.sM : p.M, N = sh ? p.sN : p.N;
  const int rows = sh ? p.shared_T : p.P;  // rows of the row-indexed operands
  int row0 = 0, cnt = p.shared_T;
  if (!sh) {
    row0 = min(max(ldc(p.offsets, e), 0), p.P);
    cnt = min(max(ldc(p.offsets, e + 1), 0), p.P) - row0;
    cnt = max(cnt, 0);
  }
  const int m0 = mt * BM, n0 = nt * BN;
  const uint16_t* A = static_cast<const uint16_t*>(sh ? p.sa : p.a);
  const uint16_t* B = static_cast<const uint16_t*>(sh ? p.sb0 : p.b0);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wbase = wave * 64;
  const int wm = wave % NWM, wn = wave / NWM;
  const int fr = lane & 15, fq = lane >> 4;
  // the reduction row of stage-local K row kr, clamped into the operand
  auto row_of = [&](int k) __attribute__((always_inline)) {
    return min(max(row0 + min(k, cnt - 1), 0), rows - 1);
  };
  // tokens of this wave's K rows of a stage (rows i * 16 + 2 wave + j):
  // wave-uniform scalar loads, issued one stage before the loads that use them
  int tk[LA][2];
  auto load_toks = [&](int kbase) __attribute__((always_inline)) {
    if constexpr (GATHER_A || GATHER_B) {
#pragma unroll
      for (int i = 0; i < LA; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = row_of(kbase + i * 16 + 2 * wave + j);
          tk[i][j] = sh ? r : min(max(ldc(p.rtok, r), 0), p.a_rows - 1);
        }
    }
  };
  const int pc = tid & 31;  // physical chunk of every load of this thread
  auto issue = [&](uint16_t* st, int kbase) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int kr = i * (NTHR / 32) + (tid >> 5);
      const int c = pc ^ kar_swz(kr);
      const int gk = lane < 32 ? tk[i][0] : tk[i][1];  // gathered row of this lane
      const int dk = row_of(kbase + kr);               // direct row
      const int ra = GATHER_A ? gk : dk, rb = GATHER_B ? gk : dk;
      const uint16_t* sa_ = A + static_cast<size_t>(ra) * M + min(m0 + 8 * c, M - 8);
      const uint16_t* sb_ = B + static_cast<size_t>(rb) * N + min(n0 + 8 * c, N - 8);
      __builtin_amdgcn_global_load_lds((gbl_void_t*)sa_, (lds_void_t*)(st + (i * NTHR + wbase) * 8),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_void_t*)sb_,
                                       (lds_void_t*)(st + SA + (i * NTHR + wbase) * 8), 16, 0, 0);
    }
  };

  floatx4_t acc[4][NFW];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < NFW; ++c) acc[a][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  // transposing fragment reads: lane (group g, quad q, r) reads K row
  // 32 ks + 8 g + 4 h + q at columns 4 r .. + 3 of a 16-column fragment; with
  // s = kar_swz of the row, A's chunk (wm * 8 + 2 mf + r / 2) ^ s and B's
  // (wn * 16 + 2 nf + r / 2) ^ s split into a base and a per-fragment XOR
  const int g = lane >> 4, q = (lane >> 2) & 3, r4 = lane & 3;
  const int sw = q | (g << 2);
  const int sA = (sw >> 1) & 3, sB = sw >> 1;
  const int klane = (8 * g + q) * BM + (((r4 >> 1) ^ (sw & 1)) << 3) + 4 * (r4 & 1);
  const int abase = klane + (((wm * 8) ^ (sw & 8)) << 3);
  const int bbase = SA + klane + wn * 128;
  auto compute = [&](const uint16_t* st) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t af[4], bf[NFW];
#pragma unroll
      for (int mf = 0; mf < 4; ++mf) {
        const uint16_t* a = st + abase + ((mf ^ sA) << 4) + ks * 32 * BM;
        struct { v4i16_t lo, hi; } pr = {__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)a),
                                         __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(a + 4 * BM))};
        af[mf] = __builtin_bit_cast(bf16x8_t, pr);
      }
#pragma unroll
      for (int nf = 0; nf < NFW; ++nf) {
        const uint16_t* bb = st + bbase + ((nf ^ sB) << 4) + ks * 32 * BN;
        struct { v4i16_t lo, hi; } pr = {__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)bb),
                                         __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(bb + 4 * BN))};
        bf[nf] = __builtin_bit_cast(bf16x8_t, pr);
      }
#pragma unroll
      for (int mf = 0; mf < 4; ++mf)
#pragma unroll
        for (int nf = 0; nf < NFW; ++nf)
          acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mf], bf[nf], acc[mf][nf], 0, 0, 0);
    }
  };
  const int nk = (cnt + BK - 1) / BK;
  // one step: stage kc in cur (once at most S - 2 newer stages' loads are
  // outstanding), kc + S - 1 issued into nxt
  auto step = [&](int kc, uint16_t* cur, uint16_t* nxt) __attribute__((always_inline)) {
    wait_stage<(S - 2) * LPS>();
    stage_barrier();
    issue(nxt, (kc + S - 1) * BK);  // past the last stage: clamped rereads, never used
    load_toks((kc + S) * BK);
    if (kc < nk) {
      if ((kc + 1) * BK > cnt) {
        // rows past the expert's count: zero them in A (B's rereads then multiply zeros)
#pragma unroll
        for (int i = 0; i < LA; ++i) {
          const int kr = i * (NTHR / 32) + (tid >> 5);
          if (kc * BK + kr >= cnt)
            *reinterpret_cast<u32x4_t*>(cur + (i * NTHR + tid) * 8) = u32x4_t{0u, 0u, 0u, 0u};
        }
        lds_barrier_g();
      }
      compute(cur);
    }
  };
  [&]<int... I>(std::integer_sequence<int, I...>) {
    // prologue: stages 0 .. S - 2, each with the tokens loaded before it
    ((I < S - 1 ? (load_toks(I * BK), issue(buf.template operator()<I>(), I * BK)) : void()), ...);
    load_toks((S - 1) * BK);
    for (int kc = 0; kc < nk; kc += S) {
      (step(kc + I, buf.template operator()<I>(), buf.template operator()<(I + S - 1) % S>()), ...);
    }
  }(std::make_integer_sequence<int, S>{});
  // the clamped loads past the last stage land before L0 is reused
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- epilogue: float32 rows through each wave's 8 KB slice of L0
  constexpr int WC = NFW * 16;
  float* Cw = reinterpret_cast<float*>(L0) + wave * 16 * WC;
  const int c0 = n0 + wn * WC;
  const int H = M / 2;
  float* O1 = static_cast<float*>(sh ? p.sout : p.out);
  float* O2 = static_cast<float*>(sh ? p.sout2 : p.out2);
#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rc = fq * 4 + i;
#pragma unroll
      for (int nf = 0; nf < NFW; ++nf) {
        const int ch = nf * 4 + (fr >> 2);
        Cw[rc * WC + ((ch ^ (fq << 2)) << 2) + (fr & 3)] = acc[mf][nf][i];
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
#pragma unroll
    for (int pass = 0; pass < 16 * WC / 4 / 64; ++pass) {
      const int idx = pass * 64 + lane;
      const int rc = idx / (WC / 4), ch = idx % (WC / 4);
      const int m = m0 + wm * 64 + mf * 16 + rc;
      const float4 v = *reinterpret_cast<const float4*>(Cw + rc * WC + ((ch ^ (((rc >> 2) & 3) << 2)) << 2));
      if (m < M && c0 + ch * 4 < N) {
        float* row;
        if constexpr (KIND == 4) {
          // gate rows [0, H), up rows [H, 2H) of expert e
          const size_t eoff = sh ? 0 : static_cast<size_t>(e) * H * N;
          row = (m < H ? O1 + eoff + static_cast<size_t>(m) * N
                       : O2 + eoff + static_cast<size_t>(m - H) * N);
        } else {
          row = O1 + (sh ? 0 : static_cast<size_t>(e) * M * N) + static_cast<size_t>(m) * N;
        }
        // written once and not read here: past the caches
        __builtin_nontemporal_store(floatx4_t{v.x, v.y, v.z, v.w},
                                    reinterpret_cast<floatx4_t*>(row + c0 + ch * 4));
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the slice is rewritten
  }
}

// ---------------------------------------------------------------------------
// Persistent variant for 128-row tiles (short K per tile). The grid holds as
// many workgroups as are resident at once (XCD x = id mod 8 owns the x-th
// eighth of the tile order and its workgroups stride through it), and the
// stage ring runs across tile boundaries: while the last slices of one tile
// are multiplied the loads already stream the next tile, whose tile-table
// lookups happen on the scalar unit and whose perm words were fetched into
// LDS one tile ahead. The epilogue stages through its own LDS slice and uses
// buffer stores (every lane issues every store; the buffer range check drops
// the ones past the output), so each wave knows exactly how many stores sit
// in its load counter behind the slices it waits for.
// ---------------------------------------------------------------------------


struct Sched {
  int x, j, W;      // XCD, slot on the XCD, workgroups per XCD
  int per, routed;  // routed tiles per XCD, routed tiles in all
  int sh0, nshx;    // this XCD's first shared tile and its count of them
  int NT;           // routed N tiles per M tile
  int nsh, NTs;     // shared-group tiles, shared N tiles per M tile
};

template <int BN>
__device__ __forceinline__ Sched make_sched(const GemmParams& p) {
  Sched s;
  const int BM = p.tile_m;
  int ntiles = p.meta != nullptr ? ldc(p.meta, 0) : 0;  // null: shared group only
  ntiles = min(max(ntiles, 0), p.max_mtiles);
  s.NT = (p.N + BN - 1) / BN;
  s.nsh = 0;
  s.NTs = 1;
  if (p.shared_T > 0) {
    s.NTs = (p.sN + BN - 1) / BN;
    s.nsh = ((p.shared_T + BM - 1) / BM) * s.NTs;
  }
  s.routed = s.NT * ntiles;
  s.per = (s.routed + 7) >> 3;
  s.x = blockIdx.x & 7;
  s.j = blockIdx.x >> 3;
  s.W = gridDim.x >> 3;
  // XCD x walks its eighth of the shared group, then its eighth of the
  // routed tiles
  const int pers = (s.nsh + 7) >> 3;
  s.sh0 = s.x * pers;
  s.nshx = min(max(s.nsh - s.sh0, 0), pers);
  return s;
}

// The i-th tile of this workgroup; false past its last one. (nrows <= 0 only
// with inconsistent caller tables: such a tile is computed and not stored.)
template <int BN>
__device__ __forceinline__ bool tile_at(const GemmParams& p, const Sched& s, int i, TileInfo& ti) {
  const int jj = s.j + i * s.W;
  const int BM = p.tile_m;
  int n, m;
  if (jj < s.nshx) {
    grouped_nm(s.sh0 + jj, s.nsh / s.NTs, s.NTs, n, m);
    ti.e = -1;
    ti.row0 = m * BM;
    ti.nrows = min(BM, p.shared_T - ti.row0);
    ti.n0 = n * BN;
    return true;
  }
  const int jr = jj - s.nshx;
  if (jr >= s.per) return false;
  const int L = s.x * s.per + jr;
  if (L >= s.routed) return false;
  const int q = L / s.NT;
  const int e = min(max(ldc(p.tile_e, q), 0), p.E - 1);
  const int tp0 = ldc(p.exp_tile0, e);
  grouped_nm(L - s.NT * tp0, ldc(p.exp_tile0, e + 1) - tp0, s.NT, n, m);
  const int o0 = min(max(ldc(p.offsets, e), 0), p.P);
  const int o1 = min(max(ldc(p.offsets, e + 1), 0), p.P);
  ti.e = e;
  ti.row0 = o0 + m * BM;
  ti.nrows = min(BM, o1 - ti.row0);
  ti.n0 = n * BN;
  return true;
}

// LDS destination of a stage load, hidden from the compiler's load-counter
// tracking (all waits on the ring are explicit and followed by a barrier).
__device__ __forceinline__ lds_void_t* lds_untracked(uint16_t* q) {
  lds_void_t* r = (lds_void_t*)q;
  asm volatile("" : "+s"(r));
  return r;
}

template <int N, int X>
__device__ __forceinline__ void wait_relaxed(bool relax) {
  if (relax) wait_stage<N + X>();
  else wait_stage<N>();
}

template <int KIND, int NWM, int NWN, int NFW, int S, int BK>
__global__ __launch_bounds__(NWM * NWN * 64) void gemm_bf16_pers(GemmParams p) {
  static_assert(BK == 32 || BK == 64, "K slice of 32 or 64");
  constexpr int CPR = BK / 8, KS = BK / 32;
  constexpr int NTHR = NWM * NWN * 64, NW = NWM * NWN;
  constexpr int BM = NWM * 64;
  constexpr int GBR = NWN * NFW * 16, HB = GBR / 2;
  constexpr int BN = KIND == 0 ? HB : GBR;
  constexpr int SA = BM * BK, SEL = SA + GBR * BK;
  constexpr int LA = SA / 8 / NTHR, LB = GBR * BK / 8 / NTHR, LPS = LA + LB;
  constexpr int WC = KIND == 0 ? NFW * 8 : NFW * 16;  // output columns per wave
  constexpr int WLD = WC + 8, LPR = WC / 8;
  constexpr int NPASS = (16 * LPR + 63) / 64;
  constexpr int ES = 4 * NPASS;                       // stores per wave per epilogue
  static_assert(LA * NTHR * 8 == SA && LB * NTHR * 8 == GBR * BK, "whole loads per thread");
  static_assert(KIND == 1 || NFW % 2 == 0, "gate/up pairs gate and up fragments");
  static_assert(S >= 3 && (S - 2) * LPS + ES < 64, "vmcnt range");
  __shared__ __align__(16) uint16_t Ring[S * SEL];
  __shared__ __align__(16) uint16_t Cs[NW * 16 * WLD];
  // perm words of the next routed tile's A rows (one 64-word block per wave
  // and load): written by DMA one tile ahead, read back by the same wave at
  // that tile's setup, which completes before the next prefetch is issued
  __shared__ __align__(16) int32_t Pg[NW * LA * 64];

  const Sched sc = make_sched<BN>(p);
  TileInfo ct;  // tile being multiplied
  if (!tile_at<BN>(p, sc, 0, ct)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wbase = wave * 64;
  int achunk[LA], bchunk[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i)
    achunk[i] = swz_phys_to_logical<BK>((i * NTHR + tid) / CPR, tid % CPR) * 8;
#pragma unroll
  for (int i = 0; i < LB; ++i)
    bchunk[i] = swz_phys_to_logical<BK>((i * NTHR + tid) / CPR, tid % CPR) * 8;

  // ---- load cursor ----
  const uint16_t* asrc[LA];
  const uint16_t* bsrc[LB];
  int lK = BK, lnk = 1, lk = 0, li = 0;
  bool lpending = false;  // the next issue starts tile lnext
  TileInfo lnext;
  int gstep = 0, pf_step = -2;  // loop step; step of the last perm prefetch
  // gate/up, routed tile: the perm words of this thread's A rows into Pg
  auto pf_issue = [&](const TileInfo& t) {
    if (KIND == 0 && t.e >= 0) {
#pragma unroll
      for (int i = 0; i < LA; ++i) {
        const int r = (i * NTHR + tid) / CPR;
        const int srow = min(max(t.row0 + (r < t.nrows ? r : 0), 0), p.P - 1);
        lds_void_t* d = (lds_void_t*)(Pg + (wave * LA + i) * 64);
        asm volatile("" : "+s"(d));
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(p.perm + srow), d, 4, 0, 0);
      }
      pf_step = gstep;
    }
  };
  auto setup = [&](const TileInfo& t) {
    const bool sh = t.e < 0;
    lK = sh ? p.sK : p.K;
    lnk = (lK + BK - 1) / BK;
    const int N = sh ? p.sN : p.N;
    const uint16_t* A = static_cast<const uint16_t*>(sh ? p.sa : p.a);
    const uint16_t* B0 = static_cast<const uint16_t*>(sh ? p.sb0 : p.b0);
    const uint16_t* B1 = static_cast<const uint16_t*>(sh ? p.sb1 : p.b1);
    if (!sh) {
      const size_t wstride = static_cast<size_t>(N) * lK;
      B0 += static_cast<size_t>(t.e) * wstride;
      if (KIND == 0) B1 += static_cast<size_t>(t.e) * wstride;
    }
    const int rows = sh ? p.shared_T : (KIND == 0 ? p.a_rows : p.P);
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = (i * NTHR + tid) / CPR;
      int src = t.row0 + (r < t.nrows ? r : 0);  // rows past the tile reload its first row
      if (KIND == 0 && !sh) src = Pg[(wave * LA + i) * 64 + lane] / p.k;
      src = min(max(src, 0), rows - 1);
      asrc[i] = A + static_cast<size_t>(src) * lK;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int r = (i * NTHR + tid) / CPR;
      int n;
      const uint16_t* base;
      if (KIND == 0) { n = t.n0 + (r < HB ? r : r - HB); base = r < HB ? B0 : B1; }
      else { n = t.n0 + r; base = B0; }
      n = min(n, N - 1);  // columns past N reload a valid row (never stored)
      bsrc[i] = base + static_cast<size_t>(n) * lK;
    }
  };
  // Issues the cursor's next K slice into stage st and advances the cursor;
  // every lane issues every load (clamped in bounds).
  auto issue = [&](uint16_t* st) {
    if (lpending) {
      lpending = false;
      // this tile's perm words went out one step ago (previous tile of a
      // single slice): not yet covered by the per-step waits
      if (pf_step >= gstep - 1) wait_stage<0>();
      setup(lnext);
      TileInfo t2;
      if (tile_at<BN>(p, sc, li + 1, t2)) pf_issue(t2);
    }
    const int k0 = min(lk, lnk - 1) * BK;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(asrc[i] + min(k0 + achunk[i], lK - 8)),
                                       lds_untracked(st + (i * NTHR + wbase) * 8), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < LB; ++i)
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(bsrc[i] + min(k0 + bchunk[i], lK - 8)),
                                       lds_untracked(st + SA + (i * NTHR + wbase) * 8), 16, 0, 0);
    if (lk < lnk && ++lk == lnk) {
      if (tile_at<BN>(p, sc, li + 1, lnext)) {
        ++li;
        lk = 0;
        lpending = true;
      }  // else: exhausted; the last slice is re-issued (never multiplied)
    }
  };

  // ---- prologue ----
  pf_issue(ct);
  wait_stage<0>();
  setup(ct);
  {
    TileInfo t1;
    if (tile_at<BN>(p, sc, 1, t1)) pf_issue(t1);
  }
#pragma unroll
  for (int st = 0; st < S - 1; ++st) issue(Ring + st * SEL);

  // ---- compute ----
  const int wm = wave % NWM, wn = wave / NWM;
  const int fr = lane & 15, fq = lane >> 4;
  floatx4_t acc[4][NFW];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NFW; ++b) acc[a][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  int aoff[KS][4], boff[KS][NFW];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int mf = 0; mf < 4; ++mf) aoff[ks][mf] = swz<BK>(wm * 64 + mf * 16 + fr, ks * 4 + fq);
#pragma unroll
    for (int nf = 0; nf < NFW; ++nf) {
      int r;
      if (KIND == 0) {
        constexpr int H = NFW / 2;
        r = (nf < H ? 0 : HB) + wn * H * 16 + (nf % H) * 16 + fr;
      } else {
        r = wn * NFW * 16 + nf * 16 + fr;
      }
      boff[ks][nf] = SA + swz<BK>(r, ks * 4 + fq);
    }
  }
  int cK = ct.e < 0 ? p.sK : p.K;
  int cnk = (cK + BK - 1) / BK;
  int ci = 0, ca = 0, ia = S - 1;
  int win = 0;  // waits still covering the last epilogue's stores
  const bool ktail_any = (p.K % BK) != 0 || (p.shared_T > 0 && (p.sK % BK) != 0);
  uint16_t* Cw = Cs + wave * 16 * WLD;

  for (;;) {
    for (int ck = 0; ck < cnk; ++ck) {
      // slice ck of tile ct is in stage ca once this wave's loads of it are
      // done (all but the newer S - 2 slices' loads, plus the stores of an
      // epilogue issued after it) and every wave has passed the barrier
      const bool relax = win > 0;
      win = win > 0 ? win - 1 : 0;
      wait_relaxed<(S - 2) * LPS, ES>(relax);
      stage_barrier();
      issue(Ring + ia * SEL);
      ia = ia + 1 == S ? 0 : ia + 1;
      uint16_t* st = Ring + ca * SEL;
      if (ktail_any && ck == cnk - 1 && (cK % BK) != 0) {
        // last, partial K slice: zero A's columns past K (B's clamped
        // duplicates then multiply zeros)
#pragma unroll
        for (int i = 0; i < LA; ++i)
          if (ck * BK + achunk[i] >= cK)
            *reinterpret_cast<u32x4_t*>(st + (i * NTHR + tid) * 8) = u32x4_t{0u, 0u, 0u, 0u};
        wait_stage<63>();
        stage_barrier();
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8_t af[4], bf[NFW];
#pragma unroll
        for (int mf = 0; mf < 4; ++mf)
          af[mf] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(st + aoff[ks][mf]));
#pragma unroll
        for (int nf = 0; nf < NFW; ++nf)
          bf[nf] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(st + boff[ks][nf]));
#pragma unroll
        for (int mf = 0; mf < 4; ++mf)
#pragma unroll
          for (int nf = 0; nf < NFW; ++nf)
            acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mf], bf[nf], acc[mf][nf], 0, 0, 0);
      }
      ca = ca + 1 == S ? 0 : ca + 1;
      ++gstep;
    }
    // epilogue: this wave's sub-tile through its LDS slice, 16 rows at a time
    {
      const bool sh = ct.e < 0;
      const int N = sh ? p.sN : p.N;
      const int rows = sh ? p.shared_T : p.P;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          sh ? p.sout : p.out, 0, static_cast<int>(static_cast<unsigned>(rows) * N * 2u), 0x00020000);
      const int c0 = ct.n0 + wn * WC;
#pragma unroll
      for (int mf = 0; mf < 4; ++mf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rc = fq * 4 + i;
          if (KIND == 0) {
#pragma unroll
            for (int nf = 0; nf < NFW / 2; ++nf)
              Cw[rc * WLD + nf * 16 + fr] = f32_to_bf16(silu_fast(acc[mf][nf][i]) * acc[mf][nf + NFW / 2][i]);
          } else {
#pragma unroll
            for (int nf = 0; nf < NFW; ++nf) Cw[rc * WLD + nf * 16 + fr] = f32_to_bf16(acc[mf][nf][i]);
          }
        }
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) {
          const int idx = pass * 64 + lane;
          const int rc = min(idx / LPR, 15), ch = (idx % LPR) * 8;
          const int rt = wm * 64 + mf * 16 + rc;
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(Cw + rc * WLD + ch);
          const bool ok = idx < 16 * LPR && rt < ct.nrows && c0 + ch < N;
          const unsigned off = ok ? (static_cast<unsigned>(ct.row0 + rt) * N + c0 + ch) * 2u : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b128(v, rs, static_cast<int>(off), 0, 0);
        }
      }
    }
    win = S - 1;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < NFW; ++b) acc[a][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    if (!tile_at<BN>(p, sc, ++ci, ct)) break;
    cK = ct.e < 0 ? p.sK : p.K;
    cnk = (cK + BK - 1) / BK;
  }
  // no load may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0);
}

// ---------------------------------------------------------------------------
// fp32 path: one thread per output element.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E - 1;  // last e with offsets[e] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int KIND>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const long long nrouted = static_cast<long long>(p.P) * p.N;
  const long long nshared = static_cast<long long>(p.shared_T) * p.sN;
  if (idx >= nrouted + nshared) return;
  bool shared = idx >= nrouted;
  const long long li = shared ? idx - nrouted : idx;
  const int N = shared ? p.sN : p.N;
  const int K = shared ? p.sK : p.K;
  const int r = static_cast<int>(li / N), c = static_cast<int>(li % N);
  const float* A = static_cast<const float*>(shared ? p.sa : p.a);
  const float* B0 = static_cast<const float*>(shared ? p.sb0 : p.b0);
  const float* B1 = static_cast<const float*>(shared ? p.sb1 : p.b1);
  float* OUT = static_cast<float*>(shared ? p.sout : p.out);
  if (!shared) {
    const int e = expert_of_row(p.offsets, p.E, r);
    if (r < min(max(p.offsets[e], 0), p.P) || r >= min(max(p.offsets[e + 1], 0), p.P)) return;
    B0 += static_cast<size_t>(e) * N * K;
    if (KIND == 0) B1 += static_cast<size_t>(e) * N * K;
  }
  const int src = (KIND == 0 && !shared) ? min(max(p.perm[r] / p.k, 0), p.a_rows - 1) : r;
  const float* a = A + static_cast<size_t>(src) * K;
  if (KIND == 0) {
    const float* wg = B0 + static_cast<size_t>(c) * K;
    const float* wu = B1 + static_cast<size_t>(c) * K;
    float g = 0.f, u = 0.f;
    for (int i = 0; i < K; ++i) { g = fmaf(a[i], wg[i], g); u = fmaf(a[i], wu[i], u); }
    OUT[static_cast<size_t>(r) * N + c] = silu_f32(g) * u;
  } else {
    const float* wd = B0 + static_cast<size_t>(c) * K;
    float s = 0.f;
    for (int i = 0; i < K; ++i) s = fmaf(a[i], wd[i], s);
    OUT[static_cast<size_t>(r) * N + c] = s;
  }
}

// Tile shapes (waves along M, waves along N, B fragments per wave, stages).
template <int KIND, int NWM, int NWN, int NFW, int S, int BK>
struct GemmShape {
  static constexpr int BM = NWM * 64;
  static constexpr int BN = (KIND == 0 || KIND == 2) ? NWN * NFW * 8 : NWN * NFW * 16;
  static void launch(const GemmParams& p, unsigned nblk, hipStream_t s) {
    gemm_bf16_kernel<KIND, NWM, NWN, NFW, S, BK><<<nblk, NWM * NWN * 64, 0, s>>>(p);
  }
};

template <int KIND, int NWM, int NWN, int NFW, int S, int BK>
struct PersShape {
  static constexpr int BM = NWM * 64;
  static constexpr int BN = KIND == 0 ? NWN * NFW * 8 : NWN * NFW * 16;
  static constexpr int OCC = NWM * NWN == 4 ? 2 : 1;  // resident workgroups per CU
  static void launch(const GemmParams& p, unsigned nblk, hipStream_t s) {
    gemm_bf16_pers<KIND, NWM, NWN, NFW, S, BK><<<nblk, NWM * NWN * 64, 0, s>>>(p);
  }
};

// Compute units of the current device (cached per device).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <class Sh>
static hipError_t launch_pers(const GemmParams& p, hipStream_t s) {
  if (p.tile_m != Sh::BM) return hipErrorInvalidValue;
  long long ub = static_cast<long long>(ceil_div(p.N, Sh::BN)) * p.max_mtiles;
  if (p.shared_T > 0) ub += static_cast<long long>(ceil_div(p.shared_T, Sh::BM)) * ceil_div(p.sN, Sh::BN);
  if (ub <= 0) return hipSuccess;
  const long long resident = static_cast<long long>(device_cus()) * Sh::OCC;
  long long nblk = ub < resident ? ub : resident;
  nblk = (nblk + 7) / 8 * 8;
  Sh::launch(p, static_cast<unsigned>(nblk), s);
  return hipGetLastError();
}

template <class Sh>
static hipError_t launch_shape(const GemmParams& p, hipStream_t s) {
  if (p.tile_m != Sh::BM) return hipErrorInvalidValue;
  // the shared and routed regions each take a multiple of 8 blocks
  long long nblk = (static_cast<long long>(ceil_div(p.N, Sh::BN)) * p.max_mtiles + 7) / 8 * 8;
  if (p.shared_T > 0)
    nblk += (static_cast<long long>(ceil_div(p.shared_T, Sh::BM)) * ceil_div(p.sN, Sh::BN) + 7) / 8 * 8;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  Sh::launch(p, static_cast<unsigned>(nblk), s);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  if (p.dtype == MOE_BF16) {
    // 256-row tiles (prefill-sized experts): 4 x 2 waves, 64-deep K slices
    // (128-byte row segments: twice the L2->LDS rate of 64-byte ones).
    if (p.tile_m == 256) {
      if (p.kind == 0) return launch_shape<GemmShape<0, 4, 2, 8, 2, 64>>(p, s);
      if (p.kind == 2) return launch_shape<GemmShape<2, 4, 2, 8, 2, 64>>(p, s);
      if (p.kind == 4 || p.kind == 5) {
        if (p.M % 8 != 0 || p.N % 8 != 0 || (p.shared_T > 0 && (p.sM % 8 != 0 || p.sN % 8 != 0)) ||
            (p.kind == 4 && (p.M % 2 != 0 || (p.shared_T > 0 && p.sM % 2 != 0))))
          return hipErrorInvalidValue;
        long long nblk = static_cast<long long>(p.E) * ceil_div(p.M, 256) * ceil_div(p.N, 256);
        if (p.shared_T > 0) nblk += static_cast<long long>(ceil_div(p.sM, 256)) * ceil_div(p.sN, 256);
        if (nblk <= 0) return hipSuccess;
        if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
        if (p.kind == 4) gemm_wgrad_kernel<4, 3, 32><<<static_cast<unsigned>(nblk), 512, 0, s>>>(p);
        else gemm_wgrad_kernel<5, 3, 32><<<static_cast<unsigned>(nblk), 512, 0, s>>>(p);
        return hipGetLastError();
      }
      if (p.kind == 3) {
        if (p.K % 2 != 0 || p.N % 8 != 0 || (p.shared_T > 0 && (p.sK % 2 != 0 || p.sN % 8 != 0)))
          return hipErrorInvalidValue;
        return launch_shape<GemmShape<3, 4, 2, 8, 2, 64>>(p, s);
      }
      return launch_shape<GemmShape<1, 4, 2, 8, 2, 64>>(p, s);
    }
    // the backward's z and dx-row products exist on the 256-row tiles only
    if (p.tile_m != 128 || p.kind >= 2) return hipErrorInvalidValue;
    // gate/up with at least 32 rows per expert on average: 2 x 4 waves over
    // 128 hidden units, 64-deep K slices, persistent (one workgroup per CU,
    // so tile changes are hidden by the pipeline running across them);
    // otherwise (decode-sized experts, and the down projection) 2 x 2 waves
    // with 32-deep slices and two workgroups per CU.
    if (p.kind == 0) {
      if (p.P >= 32 * p.E) return launch_pers<PersShape<0, 2, 4, 4, 3, 64>>(p, s);
      return launch_shape<GemmShape<0, 2, 2, 4, 4, 32>>(p, s);
    }
    // down: output widths that are multiples of 160 (gemma's d = 640) in
    // 160-column tiles of 5 fragments per wave and 64-deep slices: a fifth
    // fewer re-reads of each row tile than 128-column tiles, and no column
    // tail; other widths in 128-column tiles with 32-deep slices
    if (p.N % 160 == 0 && (p.shared_T == 0 || p.sN % 160 == 0))
      return launch_shape<GemmShape<1, 2, 2, 5, 2, 64>>(p, s);
    return launch_shape<GemmShape<1, 2, 2, 4, 4, 32>>(p, s);
  }
  if (p.kind >= 2) return hipErrorInvalidValue;
  const long long n = static_cast<long long>(p.P) * p.N + static_cast<long long>(p.shared_T) * p.sN;
  const long long nblk = (n + 255) / 256;
  if (nblk <= 0) return hipSuccess;
  if (p.kind == 0) gemm_f32_kernel<0><<<static_cast<unsigned>(nblk), 256, 0, s>>>(p);
  else gemm_f32_kernel<1><<<static_cast<unsigned>(nblk), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
