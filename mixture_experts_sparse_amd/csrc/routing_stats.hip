// Routing statistics from the router logits and the per-expert counts
// ("Mixture-of-Experts -- more capacity per byte of weight", section "What's
// wired today": the Switch load-balance term alpha * N * sum_e f_e P_e;
// "Small MoE Architecture, in depth", section "Fine-tuning a small MoE":
// per-expert token share and router entropy):
//   share_e     = counts_e / (T k)
//   mean_prob_e = (1/T) sum_t p[t, e]
//   entropy     = (1/T) sum_t -sum_e p[t, e] ln p[t, e]        (nats)
//   aux         = alpha * E * sum_e share_e mean_prob_e
// p is the router's distribution over the E experts: softmax(L) in the
// softmax modes, sigmoid(L) normalised to sum 1 in the sigmoid mode.
//
// stats_partial_kernel: at most 256 workgroups of 8 waves, each over tpb
// tokens (a multiple of 32, at least 32; tpb/8 per wave). A wave loads the
// logits of 4 tokens at once (lane l holds experts l, l + 64, l + 128,
// l + 192) and then reduces them; absent experts are masked by selects, not
// branches, and the reciprocals use the hardware's (1 ulp) instruction. Per-expert probability
// sums and the entropy sum go to a [blocks][E + 1] partial table.
// stats_final_kernel: one 1024-thread workgroup; thread (q, c) adds column c
// over the q-th quarter of the blocks in order, then the quarters are added
// in a fixed order, so the results are deterministic.

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int kStatsMaxBlocks = 256;
constexpr int kStatsChunk = 4;  // tokens a wave loads before reducing them
constexpr int kStatsWaves = 8;  // waves per partial workgroup
constexpr int kStatsThreads = kStatsWaves * 64;
static_assert(kStatsWaves == 8, "the partial workgroup sums its waves in a fixed 8-way tree");

template <bool SIG>
__global__ __launch_bounds__(kStatsThreads) void stats_partial_kernel(StatsParams p) {
  __shared__ float red[kStatsWaves][MOE_MAX_EXPERTS + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = p.E;
  const int wt = p.tpb / kStatsWaves;
  const int t0 = blockIdx.x * p.tpb + wave * wt;
  const int tend = min(t0 + wt, p.T);
  bool ok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ok[q] = lane + 64 * q < E;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float pl = 0.f;  // this lane's sum over tokens of sum_e p ln z
  float lz = 0.f;  // sum over tokens of ln Z (the same in every lane)
  for (int tc = t0; tc < tend; tc += kStatsChunk) {
    float L[kStatsChunk][4];
#pragma unroll
    for (int u = 0; u < kStatsChunk; ++u) {
      // rows past the end re-read the last row; their results are dropped
      const float* row = p.logits + static_cast<size_t>(min(tc + u, p.T - 1)) * E;
#pragma unroll
      for (int q = 0; q < 4; ++q) L[u][q] = ok[q] ? row[lane + 64 * q] : 0.f;
    }
    float m[kStatsChunk];
    if (!SIG) {
#pragma unroll
      for (int u = 0; u < kStatsChunk; ++u) {
        m[u] = -INFINITY;
#pragma unroll
        for (int q = 0; q < 4; ++q) m[u] = ok[q] ? fmaxf(m[u], L[u][q]) : m[u];
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1)
#pragma unroll
        for (int u = 0; u < kStatsChunk; ++u) m[u] = fmaxf(m[u], __shfl_xor(m[u], off, kWave));
    }
    // z: unnormalised probability, lnz: its logarithm (0 for absent experts)
    float z[kStatsChunk][4], lnz[kStatsChunk][4], Z[kStatsChunk];
#pragma unroll
    for (int u = 0; u < kStatsChunk; ++u) {
      Z[u] = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float zz, lg;
        if (SIG) {
          zz = __builtin_amdgcn_rcpf(1.0f + expf(-L[u][q]));
          lg = zz > 0.f ? logf(zz) : 0.f;  // p ln p -> 0 as p -> 0
        } else {
          lg = L[u][q] - m[u];
          zz = expf(lg);
        }
        z[u][q] = ok[q] ? zz : 0.f;
        lnz[u][q] = ok[q] ? lg : 0.f;
        Z[u] += z[u][q];
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
#pragma unroll
      for (int u = 0; u < kStatsChunk; ++u) Z[u] += __shfl_xor(Z[u], off, kWave);
    // -sum p ln p = ln Z - sum p ln z
#pragma unroll
    for (int u = 0; u < kStatsChunk; ++u) {
      if (tc + u < tend) {  // uniform across the wave
        const float inv = __builtin_amdgcn_rcpf(Z[u]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float pq = z[u][q] * inv;
          acc[q] += pq;
          pl += pq * lnz[u][q];
        }
        lz += logf(Z[u]);
      }
    }
  }
  const float hsum = lz - wave_sum(pl);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (ok[q]) red[wave][lane + 64 * q] = acc[q];
  if (lane == 0) red[wave][MOE_MAX_EXPERTS] = hsum;
  __syncthreads();
  // waves added in a fixed tree order
  auto wsum = [&](int c) {
    return ((red[0][c] + red[1][c]) + (red[2][c] + red[3][c])) +
           ((red[4][c] + red[5][c]) + (red[6][c] + red[7][c]));
  };
  float* out = p.part + static_cast<size_t>(blockIdx.x) * (E + 1);
  for (int e = threadIdx.x; e < E; e += kStatsThreads) out[e] = wsum(e);
  if (threadIdx.x == 0) out[E] = wsum(MOE_MAX_EXPERTS);
}

__global__ __launch_bounds__(1024) void stats_final_kernel(StatsParams p) {
  __shared__ float col[4][MOE_MAX_EXPERTS + 1];
  __shared__ float prod[256];
  const int tid = threadIdx.x, q = tid >> 8, c = tid & 255;
  const int E = p.E, nb = p.nb;
  const int per = (nb + 3) / 4;
  const int b_lo = min(nb, q * per), b_hi = min(nb, b_lo + per);
  // columns c and c + 256 (the entropy column when E = 256)
#pragma unroll 1
  for (int j = 0; j < 2; ++j) {
    const int cc = c + 256 * j;
    if (cc > E) continue;
    // a thread's (at most 64) loads in rounds of 32 in flight at once;
    // rows past its range read a valid row (clamped to the table) and are
    // dropped. The table is under 2^32 bytes (at most 256 x 257 floats).
    float s = 0.f;
    for (int b0 = b_lo; b0 < b_hi; b0 += 32) {
      float v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u)
        v[u] = p.part[static_cast<unsigned>(min(b0 + u, nb - 1) * (E + 1) + cc)];
#pragma unroll
      for (int u = 0; u < 32; ++u) s += b0 + u < b_hi ? v[u] : 0.f;
    }
    col[q][cc] = s;
  }
  __syncthreads();
  const float invT = 1.0f / static_cast<float>(p.T);
  if (tid < 256) {
    float mine = 0.f;
    if (tid < E) {
      const float P = ((col[0][tid] + col[1][tid]) + (col[2][tid] + col[3][tid])) * invT;
      const float share = static_cast<float>(p.counts[tid]) /
                          (static_cast<float>(p.T) * static_cast<float>(p.k));
      p.mean_prob[tid] = P;
      p.share[tid] = share;
      mine = share * P;
    }
    prod[tid] = mine;
  }
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) prod[tid] += prod[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    p.scalars[0] = ((col[0][E] + col[1][E]) + (col[2][E] + col[3][E])) * invT;
    p.scalars[1] = p.alpha * static_cast<float>(E) * prod[0];
  }
}

int stats_tokens_per_block(int T) { return max(32, ceil_div(ceil_div(T, kStatsMaxBlocks), 32) * 32); }

int stats_blocks(int T) { return ceil_div(T, stats_tokens_per_block(T)); }

hipError_t launch_stats(const StatsParams& p, hipStream_t s) {
  if (p.E > MOE_MAX_EXPERTS || p.nb != stats_blocks(p.T) || p.tpb != stats_tokens_per_block(p.T) ||
      p.nb > kStatsMaxBlocks)
    return hipErrorInvalidValue;
  if (p.mode == MOE_SIGMOID)
    stats_partial_kernel<true><<<p.nb, kStatsThreads, 0, s>>>(p);
  else
    stats_partial_kernel<false><<<p.nb, kStatsThreads, 0, s>>>(p);
  stats_final_kernel<<<1, 1024, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
