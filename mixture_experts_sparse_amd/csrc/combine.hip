// Gate-weighted combine back to token order (gfx950):
//   out[t] = sum_{j<k} gates[t, j] * y[inv[t*k + j]] (+ s_t * shared[t])
// where s_t is the shared expert's sigmoid gate (1 when ungated)
// ("Tutorial 11: Mixture of Experts (MoE)", section 3, step 3, and section 4,
// step 5). An additive gather in fixed slot order with fp32 accumulation,
// rounded once to the activation dtype; each thread owns 16 contiguous bytes
// of one output row, so every y row read is a coalesced 16-byte-per-lane
// stream.

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

// Slots are taken in batches of CKB (4 for top_k <= 4, else 8): a batch's
// inv words and gates are loaded together, then its y rows together, then
// added in slot order, so a thread waits on two load latencies per batch
// rather than two per slot.
template <int CKB>
__global__ __launch_bounds__(256) void combine_bf16_kernel(CombineParams p) {
  const int cpr = p.d >> 3;  // 8-element chunks per row
  const long long item = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (item >= static_cast<long long>(p.T) * cpr) return;
  const int t = static_cast<int>(item / cpr);
  const int c = static_cast<int>(item - static_cast<long long>(t) * cpr) * 8;
  const uint16_t* y = static_cast<const uint16_t*>(p.y);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  // the shared row does not depend on the tables: its load goes out first
  u32x4_t sv = {0u, 0u, 0u, 0u};
  float sc = 0.f;
  if (p.shared != nullptr) {
    sc = p.shared_scale != nullptr ? p.shared_scale[t] : 1.0f;
    sv = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p.shared) +
                                           static_cast<size_t>(t) * p.d + c);
  }
  for (int j0 = 0; j0 < p.k; j0 += CKB) {
    int r[CKB];
    float g[CKB];
#pragma unroll
    for (int u = 0; u < CKB; ++u) {
      const size_t q = static_cast<size_t>(t) * p.k + min(j0 + u, p.k - 1);
      r[u] = p.inv[q];
      g[u] = p.gates[q];
    }
#pragma unroll
    for (int u = 0; u < CKB; ++u) { pin(r[u]); pin(g[u]); }
    u32x4_t v[CKB];
#pragma unroll
    for (int u = 0; u < CKB; ++u) {
      const int rr = min(max(r[u], 0), p.y_rows - 1);
      // y is read once: streamed past the caches (measured on MI355X at the
      // skewed prefill shape, 537 MB of y: 118 -> 100 us)
      v[u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(y + static_cast<size_t>(rr) * p.d + c));
    }
#pragma unroll
    for (int u = 0; u < CKB; ++u) pin(v[u]);
#pragma unroll
    for (int u = 0; u < CKB; ++u) {
      if (j0 + u < p.k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(g[u], __uint_as_float(v[u][i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(g[u], __uint_as_float(v[u][i] & 0xFFFF0000u), acc[2 * i + 1]);
        }
      }
    }
  }
  if (p.shared != nullptr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(sc, __uint_as_float(sv[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(sc, __uint_as_float(sv[i] & 0xFFFF0000u), acc[2 * i + 1]);
    }
  }
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[i] = static_cast<uint32_t>(f32_to_bf16(acc[2 * i])) |
           (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
  }
  __builtin_nontemporal_store(
      o, reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p.out) + static_cast<size_t>(t) * p.d + c));
}

template <int CKB>
__global__ __launch_bounds__(256) void combine_f32_kernel(CombineParams p) {
  const int cpr = p.d >> 2;  // 4-element chunks per row
  const long long item = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (item >= static_cast<long long>(p.T) * cpr) return;
  const int t = static_cast<int>(item / cpr);
  const int c = static_cast<int>(item - static_cast<long long>(t) * cpr) * 4;
  const float* y = static_cast<const float*>(p.y);
  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  floatx4_t sv = {0.f, 0.f, 0.f, 0.f};
  float sc = 0.f;
  if (p.shared != nullptr) {
    sc = p.shared_scale != nullptr ? p.shared_scale[t] : 1.0f;
    sv = *reinterpret_cast<const floatx4_t*>(static_cast<const float*>(p.shared) +
                                             static_cast<size_t>(t) * p.d + c);
  }
  for (int j0 = 0; j0 < p.k; j0 += CKB) {
    int r[CKB];
    float g[CKB];
#pragma unroll
    for (int u = 0; u < CKB; ++u) {
      const size_t q = static_cast<size_t>(t) * p.k + min(j0 + u, p.k - 1);
      r[u] = p.inv[q];
      g[u] = p.gates[q];
    }
#pragma unroll
    for (int u = 0; u < CKB; ++u) { pin(r[u]); pin(g[u]); }
    floatx4_t v[CKB];
#pragma unroll
    for (int u = 0; u < CKB; ++u) {
      const int rr = min(max(r[u], 0), p.y_rows - 1);
      v[u] = *reinterpret_cast<const floatx4_t*>(y + static_cast<size_t>(rr) * p.d + c);
    }
#pragma unroll
    for (int u = 0; u < CKB; ++u) pin(v[u]);
#pragma unroll
    for (int u = 0; u < CKB; ++u)
      if (j0 + u < p.k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(g[u], v[u][i], acc[i]);
      }
  }
  if (p.shared != nullptr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc, sv[i], acc[i]);
  }
  *reinterpret_cast<floatx4_t*>(static_cast<float*>(p.out) + static_cast<size_t>(t) * p.d + c) = acc;
}

// rows[t, :] *= scale[t]: one thread per 16 bytes, product rounded once.
__global__ __launch_bounds__(256) void scale_rows_kernel(ScaleRowsParams p) {
  const int per = p.dtype == MOE_BF16 ? 8 : 4;
  const int cpr = p.d / per;
  const long long item = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (item >= static_cast<long long>(p.T) * cpr) return;
  const int t = static_cast<int>(item / cpr);
  const float sc = p.scale[t];
  u32x4_t* q = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.rows) + item * 16);
  u32x4_t v = *q;
  if (p.dtype == MOE_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = sc * __uint_as_float(v[i] << 16);
      const float hi = sc * __uint_as_float(v[i] & 0xFFFF0000u);
      v[i] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(sc * __uint_as_float(v[i]));
  }
  *q = v;
}

hipError_t launch_scale_rows(const ScaleRowsParams& p, hipStream_t s) {
  const int per = p.dtype == MOE_BF16 ? 8 : 4;
  const long long items = static_cast<long long>(p.T) * (p.d / per);
  const long long nblk = (items + 255) / 256;
  if (nblk <= 0) return hipSuccess;
  scale_rows_kernel<<<static_cast<unsigned>(nblk), 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  const int per = p.dtype == MOE_BF16 ? 8 : 4;
  const long long items = static_cast<long long>(p.T) * (p.d / per);
  const long long nblk = (items + 255) / 256;
  if (nblk <= 0) return hipSuccess;
  const unsigned g = static_cast<unsigned>(nblk);
  if (p.dtype == MOE_BF16) {
    if (p.k <= 4) combine_bf16_kernel<4><<<g, 256, 0, s>>>(p);
    else combine_bf16_kernel<8><<<g, 256, 0, s>>>(p);
  } else {
    if (p.k <= 4) combine_f32_kernel<4><<<g, 256, 0, s>>>(p);
    else combine_f32_kernel<8><<<g, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace moe
