// Grouped expert GEMMs for the sparse MoE layer forward (gfx950).
//
// Each workgroup computes one (expert, M tile, N tile) block of
//   gate/up: act[r, n] = silu(sum_i x[t_r, i] W_g[e, n, i]) * (sum_i x[t_r, i] W_u[e, n, i])
//   down:    y[r, n]   = sum_j act[r, j] W_d[e, n, j]
// for the sorted rows r of expert e ("Tutorial 11: Mixture of Experts (MoE)",
// section 3, step 2: each expert's SwiGLU runs on its own rows only). Rows
// of x are read in place through the sorted dispatch table (t_r = perm[r] / k),
// so no per-token copy of x or of the weights is ever built.
//
// bf16 path: v_mfma_f32_16x16x32_bf16 with fp32 accumulation, 256 threads as
// 2x2 waves, 128-row M tiles, 64-deep K chunks double-buffered in LDS (rows
// padded by 16 bytes so the MFMA fragment reads are bank-conflict free).
// fp32 path: one thread per output element (small fp32 layers only).
//
// The launch grid is sized from an upper bound on the tile count; the true
// count is read on the device, so no host synchronisation is needed. Tiles
// are numbered expert-major, then N tile, then M tile, and block b runs
// logical tile (b mod 8) * ceil(n/8) + b / 8: consecutive logical tiles (the
// M tiles that share one weight slab) land on the same XCD and its L2.

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int GBM = kTileM;     // 128
constexpr int GBK = 64;
constexpr int GLD = GBK + 8;    // padded LDS row, bf16 elements
constexpr int GBR = 128;        // B rows staged per K chunk

struct TileInfo {
  int e;          // expert, or -1 for the shared group
  int row0, nrows;
  int n0;
};

// Decodes the logical tile of this workgroup; returns false for surplus blocks.
template <int BN>
__device__ __forceinline__ bool decode_tile(const GemmParams& p, TileInfo& ti) {
  const int ntiles = p.meta != nullptr ? p.meta[0] : 0;  // null: shared group only
  const int NT = (p.N + BN - 1) / BN;
  const int routed = NT * ntiles;
  int MTs = 0, NTs = 0;
  if (p.shared_T > 0) {
    MTs = (p.shared_T + GBM - 1) / GBM;
    NTs = (p.sN + BN - 1) / BN;
  }
  const int total = routed + MTs * NTs;
  const int b = blockIdx.x;
  const int per = (total + 7) >> 3;
  const int j = b >> 3;
  if (j >= per) return false;
  const int L = (b & 7) * per + j;
  if (L >= total) return false;
  if (L < routed) {
    const int q = L / NT;
    const int e = p.tile_e[q];
    const int tp0 = p.exp_tile0[e];
    const int mt = p.exp_tile0[e + 1] - tp0;
    const int local = L - NT * tp0;
    const int n = local / mt;
    const int m = local - n * mt;
    // offsets clamped to [0, P]: caller-provided tables cannot push rows out of bounds
    const int o0 = min(max(p.offsets[e], 0), p.P), o1 = min(max(p.offsets[e + 1], 0), p.P);
    ti.e = e;
    ti.row0 = o0 + m * GBM;
    ti.nrows = min(GBM, o1 - ti.row0);
    ti.n0 = n * BN;
  } else {
    const int Ls = L - routed;
    const int n = Ls / MTs;
    const int m = Ls - n * MTs;
    ti.e = -1;
    ti.row0 = m * GBM;
    ti.nrows = min(GBM, p.shared_T - ti.row0);
    ti.n0 = n * BN;
  }
  return ti.nrows > 0;
}

// KIND 0: gate/up (B rows 0..63 gate, 64..127 up; N tile 64).
// KIND 1: down (B rows 0..127; N tile 128).
template <int KIND>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmParams p) {
  constexpr int BN = KIND == 0 ? kTileNGateUp : kTileNDown;
  __shared__ __align__(16) uint16_t As[2][GBM * GLD];
  __shared__ __align__(16) uint16_t Bs[2][GBR * GLD];

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
    const size_t wstride = static_cast<size_t>(N) * K;
    B0 += static_cast<size_t>(ti.e) * wstride;
    if (KIND == 0) B1 += static_cast<size_t>(ti.e) * wstride;
  }

  const int tid = threadIdx.x;
  const int lr = tid >> 3;         // staging row (plus 32 * i)
  const int lc = (tid & 7) * 8;    // staging column (bf16 elements)

  const uint16_t* arow[4];
  const uint16_t* brow[4];
  bool aok[4], bok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = lr + 32 * i;
    aok[i] = r < ti.nrows;
    arow[i] = A;
    if (aok[i]) {
      const int srow = ti.row0 + r;
      int src = srow;
      if (KIND == 0 && !shared) src = min(max(p.perm[srow] / p.k, 0), p.a_rows - 1);
      arow[i] = A + static_cast<size_t>(src) * K;
    }
    int n;
    const uint16_t* base;
    if (KIND == 0) {
      n = ti.n0 + (r & 63);
      base = r < 64 ? B0 : B1;
    } else {
      n = ti.n0 + r;
      base = B0;
    }
    bok[i] = n < N;
    brow[i] = base + static_cast<size_t>(bok[i] ? n : 0) * K;
  }

  u32x4_t ra[4], rb[4];
  auto gload = [&](int k0) {
    const int kk = k0 + lc;
    const bool kok = kk < K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = (aok[i] && kok) ? *reinterpret_cast<const u32x4_t*>(arow[i] + kk) : u32x4_t{0u, 0u, 0u, 0u};
      rb[i] = (bok[i] && kok) ? *reinterpret_cast<const u32x4_t*>(brow[i] + kk) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4_t*>(&As[buf][(lr + 32 * i) * GLD + lc]) = ra[i];
      *reinterpret_cast<u32x4_t*>(&Bs[buf][(lr + 32 * i) * GLD + lc]) = rb[i];
    }
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 15, fk = (lane >> 4) * 8;

  constexpr int NF = KIND == 0 ? 4 : 4;  // B fragments per wave (gate 2 + up 2, or 4)
  floatx4_t acc[4][NF];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NF; ++b) acc[a][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + GBK - 1) / GBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nk) gload((kc + 1) * GBK);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8_t af[4], bf[NF];
#pragma unroll
      for (int mf = 0; mf < 4; ++mf) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&As[buf][(wm * 64 + mf * 16 + fr) * GLD + s * 32 + fk]);
        af[mf] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        int brw;
        if (KIND == 0) brw = (nf < 2 ? 0 : 64) + wn * 32 + (nf & 1) * 16 + fr;
        else brw = wn * 64 + nf * 16 + fr;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&Bs[buf][brw * GLD + s * 32 + fk]);
        bf[nf] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int mf = 0; mf < 4; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
          acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mf], bf[nf], acc[mf][nf], 0, 0, 0);
    }
    if (kc + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue
#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + mf * 16 + (lane >> 4) * 4 + i;
      if (r >= ti.nrows) continue;
      const size_t orow = static_cast<size_t>(ti.row0 + r) * N;
      if (KIND == 0) {
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
          const int c = ti.n0 + wn * 32 + nf * 16 + fr;
          if (c < N) {
            const float g = acc[mf][nf][i];
            const float u = acc[mf][nf + 2][i];
            OUT[orow + c] = f32_to_bf16(silu_f32(g) * u);
          }
        }
      } else {
        const float sc = (shared && p.srow_scale != nullptr) ? p.srow_scale[ti.row0 + r] : 1.0f;
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
          const int c = ti.n0 + wn * 64 + nf * 16 + fr;
          if (c < N) OUT[orow + c] = f32_to_bf16(acc[mf][nf][i] * sc);
        }
      }
    }
  }
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
    if (shared && p.srow_scale != nullptr) s *= p.srow_scale[r];
    OUT[static_cast<size_t>(r) * N + c] = s;
  }
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  if (p.dtype == MOE_BF16) {
    const int BN = p.kind == 0 ? kTileNGateUp : kTileNDown;
    long long nblk = static_cast<long long>(ceil_div(p.N, BN)) * p.max_mtiles;
    if (p.shared_T > 0) nblk += static_cast<long long>(ceil_div(p.shared_T, GBM)) * ceil_div(p.sN, BN);
    nblk = (nblk + 7) / 8 * 8;
    if (nblk <= 0) return hipSuccess;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    if (p.kind == 0) gemm_bf16_kernel<0><<<static_cast<unsigned>(nblk), 256, 0, s>>>(p);
    else gemm_bf16_kernel<1><<<static_cast<unsigned>(nblk), 256, 0, s>>>(p);
  } else {
    const long long n = static_cast<long long>(p.P) * p.N + static_cast<long long>(p.shared_T) * p.sN;
    const long long nblk = (n + 255) / 256;
    if (nblk <= 0) return hipSuccess;
    if (p.kind == 0) gemm_f32_kernel<0><<<static_cast<unsigned>(nblk), 256, 0, s>>>(p);
    else gemm_f32_kernel<1><<<static_cast<unsigned>(nblk), 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace moe
