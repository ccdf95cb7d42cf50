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
// stats_partial_kernel: 256 tokens per workgroup, one token at a time per
// wave with lane l holding experts l, l + 64, l + 128, l + 192; per-expert
// probability sums and the entropy sum go to a [blocks][E + 1] partial
// table, added in fixed order (waves, then blocks), so results are
// deterministic. stats_final_kernel: one workgroup.

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int kStatsTokens = 256;
constexpr int kStatsWaveTokens = kStatsTokens / 4;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__global__ __launch_bounds__(256) void stats_partial_kernel(StatsParams p) {
  __shared__ float red[4][MOE_MAX_EXPERTS + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = p.E;
  const bool sig = p.mode == MOE_SIGMOID;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float hsum = 0.f;
  const int tb = blockIdx.x * kStatsTokens + wave * kStatsWaveTokens;
  for (int i = 0; i < kStatsWaveTokens; ++i) {
    const int t = tb + i;
    if (t >= p.T) break;  // uniform across the wave
    const float* row = p.logits + static_cast<size_t>(t) * E;
    float L[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      L[q] = e < E ? row[e] : -INFINITY;
    }
    float z[4], Zl = 0.f;
    float m = 0.f;
    if (sig) {
#pragma unroll
      for (int q = 0; q < 4; ++q) z[q] = lane + 64 * q < E ? sigmoid_f32(L[q]) : 0.f;
    } else {
      m = wave_max(fmaxf(fmaxf(L[0], L[1]), fmaxf(L[2], L[3])));
#pragma unroll
      for (int q = 0; q < 4; ++q) z[q] = lane + 64 * q < E ? expf(L[q] - m) : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) Zl += z[q];
    const float Z = wave_sum(Zl);
    const float inv = 1.0f / Z;
    // -sum p ln p = ln Z - sum p ln z, with ln z = L - m (softmax) or ln s
    float pl = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (lane + 64 * q < E) {
        const float pq = z[q] * inv;
        acc[q] += pq;
        pl += pq * (sig ? logf(z[q]) : (L[q] - m));
      }
    }
    hsum += logf(Z) - wave_sum(pl);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (lane + 64 * q < E) red[wave][lane + 64 * q] = acc[q];
  if (lane == 0) red[wave][MOE_MAX_EXPERTS] = hsum;
  __syncthreads();
  float* out = p.part + static_cast<size_t>(blockIdx.x) * (E + 1);
  for (int e = threadIdx.x; e < E; e += 256) out[e] = (red[0][e] + red[1][e]) + (red[2][e] + red[3][e]);
  if (threadIdx.x == 0)
    out[E] = (red[0][MOE_MAX_EXPERTS] + red[1][MOE_MAX_EXPERTS]) +
             (red[2][MOE_MAX_EXPERTS] + red[3][MOE_MAX_EXPERTS]);
}

__global__ __launch_bounds__(256) void stats_final_kernel(StatsParams p) {
  __shared__ float prod[256];
  __shared__ float hpart[256];
  const int tid = threadIdx.x, E = p.E, nb = p.nb;
  const float invT = 1.0f / static_cast<float>(p.T);
  float mine = 0.f;
  if (tid < E) {
    // blocks in order, in batches of 8 loads
    float s = 0.f;
    for (int b0 = 0; b0 < nb; b0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p.part[static_cast<size_t>(min(b0 + u, nb - 1)) * (E + 1) + tid];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += b0 + u < nb ? v[u] : 0.f;
    }
    const float P = s * invT;
    const float share = static_cast<float>(p.counts[tid]) /
                        (static_cast<float>(p.T) * static_cast<float>(p.k));
    p.mean_prob[tid] = P;
    p.share[tid] = share;
    mine = share * P;
  }
  prod[tid] = mine;
  // entropy: thread b sums blocks b, b + 256, ... in order
  float h = 0.f;
  for (int b = tid; b < nb; b += 256) h += p.part[static_cast<size_t>(b) * (E + 1) + E];
  hpart[tid] = h;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      prod[tid] += prod[tid + w];
      hpart[tid] += hpart[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    p.scalars[0] = hpart[0] * invT;
    p.scalars[1] = p.alpha * static_cast<float>(E) * prod[0];
  }
}

int stats_blocks(int T) { return ceil_div(T, kStatsTokens); }

hipError_t launch_stats(const StatsParams& p, hipStream_t s) {
  if (p.E > MOE_MAX_EXPERTS || p.nb != stats_blocks(p.T)) return hipErrorInvalidValue;
  stats_partial_kernel<<<p.nb, 256, 0, s>>>(p);
  stats_final_kernel<<<1, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
