// Grouped expert GEMMs for batches with few rows per expert (decode-shaped
// layers), gfx950.
//
// Same arithmetic as the tiled grouped GEMMs -- gate/up with the fused SwiGLU
// product, act[r] = silu(W_g[e] x_t) * (W_u[e] x_t), and down,
// y[r] = W_d[e] act[r] ("Tutorial 11: Mixture of Experts (MoE)", section 3,
// step 2; "Small MoE Architecture, in depth", the SwiGLU expert) -- laid out
// for the case where the weights are the whole cost: every touched expert's
// weights are read once from HBM and each expert has a handful of rows.
//
// A workgroup owns 16 * NT output columns of one touched expert (gate and up
// both for the gate/up kind). Its NW waves split the reduction: wave w holds
// K range [w * KS * 32, (w + 1) * KS * 32) of those weight rows in registers
// in the MFMA B-operand layout (lane l: column l % 16, 8 consecutive K values
// at 8 * (l / 16) of every 32-deep step), all loads issued at once. The
// expert's rows then pass through in blocks of 16 (A operand in the same K
// layout, loaded straight into registers), the per-wave partial sums meet in
// LDS and are added in wave order, and the epilogue writes bf16 rows.
// The grid is (touched-expert slots) x (column slices); slots past the
// number of touched experts exit at once.

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

// 16 bytes at row + kq, or zeros when kq is past K. The load is always
// issued (at a clamped address), so there is no branch around it and the
// compiler's count of outstanding loads stays exact.
__device__ __forceinline__ u32x4_t load_k8(const uint16_t* row, int kq, int K) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + min(kq, K - 8));
  return kq < K ? v : u32x4_t{0u, 0u, 0u, 0u};
}
// Weights past K: the clamped load rereads real (finite) weights and the x
// operand is zero there, so the products vanish without a select -- and
// with no select a weight register set can stay in flight across loop
// iterations (a select would wait for the load where it stands).
__device__ __forceinline__ u32x4_t load_k8_w(const uint16_t* row, int kq, int K) {
  return *reinterpret_cast<const u32x4_t*>(row + min(kq, K - 8));
}

// One 16-row block's epilogue: each wave's partial tiles (acc, MFMA C layout:
// lane holds rows 4 (lane / 16) + i of column 16 t + lane % 16) go to LDS,
// the NW partials are added in wave order, and the bf16 results (SiLU
// product for gate/up) are stored for rows rb .. rb + 15 < cnt of the
// expert's range starting at r0, columns n0 .. n0 + 16 NT - 1 < N.
// Two workgroup barriers; called by every thread.
template <int KIND, int NW, int NB, int NT>
__device__ __forceinline__ void small_block_epilogue(const GemmParams& p,
                                                     float (*red)[NB][16][16 * NT],
                                                     const floatx4_t (&acc)[NB][NT], int r0,
                                                     int rb, int cnt, int n0) {
  constexpr int NCOL = 16 * NT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = p.N;
#pragma unroll
  for (int m = 0; m < NB; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][m][(lane >> 4) * 4 + i][t * 16 + (lane & 15)] = acc[m][t][i];
  __syncthreads();
  for (int it = threadIdx.x; it < 16 * NCOL / 2; it += NW * 64) {
    const int row = it / (NCOL / 2);
    const int c = (it - row * (NCOL / 2)) * 2;
    const int n = n0 + c;
    if (rb + row < cnt && n < N) {  // N is a multiple of 8: n + 1 < N too
      float v[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float g = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) g += red[w][0][row][c + j];
        if constexpr (KIND == 0) {
          float u = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) u += red[w][NB - 1][row][c + j];
          v[j] = silu_fast(g) * u;
        } else {
          v[j] = g;
        }
      }
      const uint32_t o = static_cast<uint32_t>(f32_to_bf16(v[0])) |
                         (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.out) +
                                   static_cast<size_t>(r0 + rb + row) * N + n) = o;
    }
  }
  __syncthreads();
}

template <int KIND, int NW, int KS, int NT>
__global__ __launch_bounds__(NW * 64) void gemm_small_kernel(GemmParams p) {
  constexpr int NB = KIND == 0 ? 2 : 1;  // weight matrices: gate and up, or down
  constexpr int NCOL = 16 * NT;          // output columns per workgroup
  __shared__ float red[NW][NB][16][NCOL];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int N = p.N, K = p.K;
  const int ncs = (N + NCOL - 1) / NCOL;
  const int slot = blockIdx.x / ncs;
  const int n0 = (blockIdx.x - slot * ncs) * NCOL;
  // one load gives the slot's expert and rows (slot < E: always in the table)
  int ntouched = p.meta[1];
  int4 ti = *reinterpret_cast<const int4*>(p.touched + 4 * slot);
  // both loads in flight together, ahead of the exit test
  pin_s(ntouched); pin_s(ti.x); pin_s(ti.y); pin_s(ti.z);
  if (slot >= ntouched) return;
  const int e = min(max(ti.x, 0), p.E - 1);
  // rows are clamped so every row index stays in [0, P)
  const int r0 = min(max(ti.y, 0), p.P);
  const int cnt = min(max(ti.z, 0), p.P - r0);
  const int kb = wave * KS * 32 + (lane >> 4) * 8;  // this lane's first K index
  const uint16_t* A = static_cast<const uint16_t*>(p.a);

  // the first row block's perm words go out before the weights, so the
  // x rows' addresses are known while the weights are still in flight
  int first_pair = 0;
  if constexpr (KIND == 0) first_pair = p.perm[min(max(r0 + min(lane & 15, cnt - 1), 0), p.P - 1)];

  u32x4_t bq[NB][NT][KS];
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const uint16_t* B = static_cast<const uint16_t*>(m == 0 ? p.b0 : p.b1) +
                        static_cast<size_t>(e) * N * K;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // columns past N reread column N - 1; their sums are never stored
      const uint16_t* brow = B + static_cast<size_t>(min(n0 + t * 16 + (lane & 15), N - 1)) * K;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        bq[m][t][s] = load_k8_w(brow, kb + s * 32, K);
      }
    }
  }
  // every weight load is issued before anything waits on the perm word
  asm volatile("" ::: "memory");

  for (int rb = 0; rb < cnt; rb += 16) {
    // rows past the expert's last reread its last row; never stored
    const int rr = min(rb + (lane & 15), cnt - 1);
    const uint16_t* arow;
    if constexpr (KIND == 0) {
      const int pair = rb == 0 ? first_pair : p.perm[r0 + rr];
      const int tok = min(max(pair / p.k, 0), p.a_rows - 1);
      arow = A + static_cast<size_t>(tok) * K;
    } else {
      arow = A + static_cast<size_t>(r0 + rr) * K;
    }
    u32x4_t aq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      aq[s] = load_k8(arow, kb + s * 32, K);  // K is a multiple of 8: all 8 in range or none
    }
    floatx4_t acc[NB][NT];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[m][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, aq[s]);
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a, __builtin_bit_cast(bf16x8_t, bq[m][t][s]), acc[m][t], 0, 0, 0);
    }
    small_block_epilogue<KIND, NW, NB, NT>(p, red, acc, r0, rb, cnt, n0);
  }
}

// ---------------------------------------------------------------------------
// 4-bit routed weights (MOE_QUANT_Q4_G64): codes [E, N, K/2] (position 2i in
// the low nibble of byte i) and scale|bias words [E, N, K/64], w = s q + b.
// Every MFMA step must lie inside one 64-wide scale group, so the K layout
// is: scale group G of a wave's range, half h in {0, 1}; lane group g holds
// K values kb + 64 G + 16 g + 8 h .. + 7 (x and weights alike). A lane then
// reads its 16 codes of a group as one 8-byte load and the group's scale and
// bias as one 4-byte word.
//
// The weights are never dequantised one by one. Within a group,
//   sum_k x_k (s q_k + b) = s sum_k x_k (128 + q_k) + (b - 128 s) sum_k x_k,
// and 128 + q (q < 16) is an exact bf16 whose bit pattern is 0x4300 | q, so
// the codes become MFMA operands with two integer operations per pair; each
// group's two MFMA steps accumulate on their own, the x row sums of the group
// come from two MFMAs against ones, and the scale and bias are applied to the
// group's accumulator with two FMAs per output.
// ---------------------------------------------------------------------------

// bf16 pairs (128 + q_2j, 128 + q_2j+1), j = 0..3, of the 8 codes of D (code
// i in nibble i), exact.
__device__ __forceinline__ u32x4_t codes_bf16(uint32_t D) {
  const uint32_t lo = D & 0x0F0F0F0Fu;          // codes 0, 2, 4, 6 (one per byte)
  const uint32_t hi = (D >> 4) & 0x0F0F0F0Fu;   // codes 1, 3, 5, 7
  u32x4_t r;
  // byte j of lo -> bits 0..7, byte j of hi -> bits 16..23 (selector 0x0C: zero)
  r[0] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x43004300u;
  r[1] = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x43004300u;
  r[2] = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x43004300u;
  r[3] = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x43004300u;
  return r;
}

template <int KIND, int NW, int KS, int NT>
__global__ __launch_bounds__(NW * 64) void gemm_small_q4_kernel(GemmParams p) {
  constexpr int NB = KIND == 0 ? 2 : 1;
  constexpr int NCOL = 16 * NT;
  constexpr int KG = KS / 2;  // scale groups per wave
  static_assert(KS % 2 == 0, "whole scale groups per wave");
  __shared__ float red[NW][NB][16][NCOL];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int N = p.N, K = p.K;
  const int ncs = (N + NCOL - 1) / NCOL;
  const int slot = blockIdx.x / ncs;
  const int n0 = (blockIdx.x - slot * ncs) * NCOL;
  int ntouched = p.meta[1];
  int4 ti = *reinterpret_cast<const int4*>(p.touched + 4 * slot);
  pin_s(ntouched); pin_s(ti.x); pin_s(ti.y); pin_s(ti.z);
  if (slot >= ntouched) return;
  const int e = min(max(ti.x, 0), p.E - 1);
  const int r0 = min(max(ti.y, 0), p.P);
  const int cnt = min(max(ti.z, 0), p.P - r0);
  const int kb = wave * KS * 32 + (lane >> 4) * 16;  // lane's first K index in group 0
  const uint16_t* A = static_cast<const uint16_t*>(p.a);

  int first_pair = 0;
  if constexpr (KIND == 0) first_pair = p.perm[min(max(r0 + min(lane & 15, cnt - 1), 0), p.P - 1)];

  uint2 qc[NB][NT][KG];
  uint32_t sb[NB][NT][KG];
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const uint8_t* Q = static_cast<const uint8_t*>(m == 0 ? p.b0 : p.b1) +
                       static_cast<size_t>(e) * N * (K / 2);
    const uint32_t* S = (m == 0 ? p.b0_sb : p.b1_sb) + static_cast<size_t>(e) * N * (K / 64);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // columns past N reread column N - 1; their sums are never stored
      const int n = min(n0 + t * 16 + (lane & 15), N - 1);
#pragma unroll
      for (int G = 0; G < KG; ++G) {
        // groups past K reread the last one: the x operand is zero there
        const int kq = min(kb + 64 * G, K - 16);
        qc[m][t][G] = *reinterpret_cast<const uint2*>(Q + (static_cast<size_t>(n) * K + kq) / 2);
        sb[m][t][G] = S[static_cast<size_t>(n) * (K / 64) + kq / 64];
      }
    }
  }
  asm volatile("" ::: "memory");

  for (int rb = 0; rb < cnt; rb += 16) {
    const int rr = min(rb + (lane & 15), cnt - 1);
    const uint16_t* arow;
    if constexpr (KIND == 0) {
      const int pair = rb == 0 ? first_pair : p.perm[r0 + rr];
      const int tok = min(max(pair / p.k, 0), p.a_rows - 1);
      arow = A + static_cast<size_t>(tok) * K;
    } else {
      arow = A + static_cast<size_t>(r0 + rr) * K;
    }
    u32x4_t aq[KS];
#pragma unroll
    for (int G = 0; G < KG; ++G)
#pragma unroll
      for (int h = 0; h < 2; ++h) aq[2 * G + h] = load_k8(arow, kb + 64 * G + 8 * h, K);
    floatx4_t acc[NB][NT];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[m][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
    const floatx4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int G = 0; G < KG; ++G) {
      // one group at a time: its codes are taken (pinned) only after the
      // previous group's accumulators are final, so the compiler forms each
      // group's bf16 operands next to their MFMAs instead of all groups'
      // at once (4x the registers of the packed codes, hoisted out of the
      // row loop)
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) { pin(qc[m][t][G].x); pin(qc[m][t][G].y); }
      const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, aq[2 * G]);
      const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, aq[2 * G + 1]);
      // x row sums over the group (every column of the tile holds its row's)
      floatx4_t xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          a0, __builtin_bit_cast(bf16x8_t, ones), zero, 0, 0, 0);
      xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8_t, ones), xs, 0,
                                                   0, 0);
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          floatx4_t ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a0, __builtin_bit_cast(bf16x8_t, codes_bf16(qc[m][t][G].x)), zero, 0, 0, 0);
          ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a1, __builtin_bit_cast(bf16x8_t, codes_bf16(qc[m][t][G].y)), ag, 0, 0, 0);
          // this lane's column: its own scale word
          const float sc = bf16_to_f32(static_cast<uint16_t>(sb[m][t][G] & 0xFFFFu));
          const float b2 =
              fmaf(-128.0f, sc, bf16_to_f32(static_cast<uint16_t>(sb[m][t][G] >> 16)));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][t][i] = fmaf(sc, ag[i], fmaf(b2, xs[i], acc[m][t][i]));
        }
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) pin(acc[m][t]);
    }
    small_block_epilogue<KIND, NW, NB, NT>(p, red, acc, r0, rb, cnt, n0);
  }
}

// ---------------------------------------------------------------------------
// Persistent form: one 8-wave workgroup per CU walks the items blockIdx.x,
// blockIdx.x + G, ... (item = touched-expert slot x column slice, slice
// fastest), with two register sets for weight slices. While item n waits on
// its x rows and computes, item n + 1's perm word and weights are already in
// flight; since a wave's vector loads complete in issue order, item n + 1's
// perm word goes out before its weights (so waiting on it does not wait on
// them) and the weights after item n's x rows (so waiting on those does not
// wait on the weights). Past the last item the "next" item is the current
// one again (its lines are in L2), which keeps the code free of branches
// around loads.
// ---------------------------------------------------------------------------
template <int KIND, int KS, int NT>
__global__ __launch_bounds__(512) void gemm_small_pers(GemmParams p) {
  constexpr int NW = 8;
  constexpr int NB = KIND == 0 ? 2 : 1;
  constexpr int NCOL = 16 * NT;
  __shared__ float red[NW][NB][16][NCOL];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int N = p.N, K = p.K;
  const int ncs = (N + NCOL - 1) / NCOL;
  const int total = min(ldc(p.meta, 1), p.E) * ncs;
  const int G = gridDim.x;
  int i = blockIdx.x;
  if (i >= total) return;
  const int kb = wave * KS * 32 + (lane >> 4) * 8;
  const uint16_t* A = static_cast<const uint16_t*>(p.a);

  struct Item {
    int e, r0, cnt, n0;
  };
  auto fetch = [&](int it) -> Item {
    const int slot = __builtin_amdgcn_readfirstlane(it / ncs);
    const i32x4_t ti = ldc(reinterpret_cast<const i32x4_t*>(p.touched), slot);
    Item r;
    r.e = min(max(ti[0], 0), p.E - 1);
    r.r0 = min(max(ti[1], 0), p.P);
    r.cnt = min(max(ti[2], 0), p.P - r.r0);
    r.n0 = __builtin_amdgcn_readfirstlane((it - slot * ncs) * NCOL);
    return r;
  };
  auto load_b = [&](u32x4_t (&bq)[NB][NT][KS], const Item& it) {
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      const uint16_t* B = static_cast<const uint16_t*>(m == 0 ? p.b0 : p.b1) +
                          static_cast<size_t>(it.e) * N * K;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint16_t* brow =
            B + static_cast<size_t>(min(it.n0 + t * 16 + (lane & 15), N - 1)) * K;
#pragma unroll
        for (int s = 0; s < KS; ++s) bq[m][t][s] = load_k8_w(brow, kb + s * 32, K);
      }
    }
  };
  // perm word of row rb + lane % 16 of the item (clamped into the table)
  auto load_pair = [&](const Item& it, int rb) -> int {
    return p.perm[min(max(it.r0 + min(rb + (lane & 15), it.cnt - 1), 0), p.P - 1)];
  };
  auto a_row = [&](const Item& it, int rb, int pair) -> const uint16_t* {
    if constexpr (KIND == 0) {
      const int tok = min(max(pair / p.k, 0), p.a_rows - 1);
      return A + static_cast<size_t>(tok) * K;
    } else {
      return A + static_cast<size_t>(it.r0 + min(rb + (lane & 15), it.cnt - 1)) * K;
    }
  };
  // one 16-row block: MFMAs, the cross-wave sum and the bf16 stores
  auto block = [&](const Item& it, int rb, const u32x4_t (&aq)[KS],
                   const u32x4_t (&bq)[NB][NT][KS]) {
    floatx4_t acc[NB][NT];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[m][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, aq[s]);
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a, __builtin_bit_cast(bf16x8_t, bq[m][t][s]), acc[m][t], 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[wave][m][(lane >> 4) * 4 + q][t * 16 + (lane & 15)] = acc[m][t][q];
    __syncthreads();
    for (int x = threadIdx.x; x < 16 * NCOL / 2; x += NW * 64) {
      const int row = x / (NCOL / 2);
      const int c = (x - row * (NCOL / 2)) * 2;
      const int n = it.n0 + c;
      if (rb + row < it.cnt && n < N) {  // N is a multiple of 8: n + 1 < N too
        float v[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float g = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) g += red[w][0][row][c + j];
          if constexpr (KIND == 0) {
            float u = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) u += red[w][NB - 1][row][c + j];
            v[j] = silu_fast(g) * u;
          } else {
            v[j] = g;
          }
        }
        const uint32_t o = static_cast<uint32_t>(f32_to_bf16(v[0])) |
                           (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.out) +
                                     static_cast<size_t>(it.r0 + rb + row) * N + n) = o;
      }
    }
    __syncthreads();
  };
  // item `it` (weights in bc, first perm word pc) while the next item's perm
  // word (-> pn) and weights (-> bn) go out; the item after that is fetched
  auto run = [&](const Item& it, const u32x4_t (&bc)[NB][NT][KS], int pc, const Item& nx,
                 u32x4_t (&bn)[NB][NT][KS], int& pn, Item& nx2, int i2) {
    u32x4_t aq[KS];
    {
      const uint16_t* arow = a_row(it, 0, pc);
#pragma unroll
      for (int s = 0; s < KS; ++s) aq[s] = load_k8(arow, kb + s * 32, K);
    }
    if constexpr (KIND == 0) pn = load_pair(nx, 0);
    load_b(bn, nx);
    // issue order is the point: the x rows are pinned only after the next
    // item's loads are out, so the MFMAs (which use the pinned values)
    // cannot be scheduled above those loads
    asm volatile("" ::: "memory");
#pragma unroll
    for (int s = 0; s < KS; ++s) pin(aq[s]);
    nx2 = fetch(i2);
    block(it, 0, aq, bc);
    for (int rb = 16; rb < it.cnt; rb += 16) {
      const int pr = KIND == 0 ? load_pair(it, rb) : 0;
      const uint16_t* arow = a_row(it, rb, pr);
#pragma unroll
      for (int s = 0; s < KS; ++s) aq[s] = load_k8(arow, kb + s * 32, K);
      block(it, rb, aq, bc);
    }
  };

  u32x4_t b0[NB][NT][KS], b1[NB][NT][KS];
  Item cur = fetch(i);
  int p0 = KIND == 0 ? load_pair(cur, 0) : 0, p1 = 0;
  load_b(b0, cur);
  Item nxt = fetch(min(i + G, total - 1));
  Item nx2;
  for (;;) {
    run(cur, b0, p0, nxt, b1, p1, nx2, min(i + 2 * G, total - 1));
    i += G;
    if (i >= total) break;
    cur = nxt;
    nxt = nx2;
    run(cur, b1, p1, nxt, b0, p0, nx2, min(i + 2 * G, total - 1));
    i += G;
    if (i >= total) break;
    cur = nxt;
    nxt = nx2;
  }
}

// One launch of the small-batch GEMM. The persistent form keeps the weight
// stream running across items, which pays when every CU has several items;
// measured on MI355X it helps the down projection (one weight matrix, 32
// columns per item) and not gate/up, whose one-shot workgroups already
// stream its two matrices at about 5.8 TB/s.
template <int KIND, int NT>
static hipError_t launch_small_kind(const GemmParams& p, int slots, hipStream_t s) {
  const SmallShape sh = small_shape(p.K);
  const int ncs = ceil_div(p.N, 16 * NT);
  const long long nblk = static_cast<long long>(slots) * ncs;
  if (nblk <= 0) return hipSuccess;
  const unsigned g = static_cast<unsigned>(nblk);
  const int cus = device_cus();
  if constexpr (KIND == 1) {
    if (nblk >= 4LL * cus && p.K <= 8 * 8 * 32) {
      // persistent: one workgroup per CU; two register sets of at most 8 steps
      const unsigned gp = static_cast<unsigned>(cus);
      if (p.K <= 8 * 2 * 32) gemm_small_pers<KIND, 2, NT><<<gp, 512, 0, s>>>(p);
      else if (p.K <= 8 * 4 * 32) gemm_small_pers<KIND, 4, NT><<<gp, 512, 0, s>>>(p);
      else gemm_small_pers<KIND, 8, NT><<<gp, 512, 0, s>>>(p);
      return hipGetLastError();
    }
  }
  if (sh.nw == 4 && sh.ks == 4) gemm_small_kernel<KIND, 4, 4, NT><<<g, 256, 0, s>>>(p);
  else if (sh.nw == 4 && sh.ks == 8) gemm_small_kernel<KIND, 4, 8, NT><<<g, 256, 0, s>>>(p);
  else if (sh.nw == 4 && sh.ks == 16) gemm_small_kernel<KIND, 4, 16, NT><<<g, 256, 0, s>>>(p);
  else if (sh.nw == 8 && sh.ks == 16) gemm_small_kernel<KIND, 8, 16, NT><<<g, 512, 0, s>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int KIND, int NT>
static hipError_t launch_small_q4(const GemmParams& p, int slots, hipStream_t s) {
  const SmallShape sh = small_shape(p.K);
  const long long nblk = static_cast<long long>(slots) * ceil_div(p.N, 16 * NT);
  if (nblk <= 0) return hipSuccess;
  const unsigned g = static_cast<unsigned>(nblk);
  if (sh.nw == 4 && sh.ks == 4) gemm_small_q4_kernel<KIND, 4, 4, NT><<<g, 256, 0, s>>>(p);
  else if (sh.nw == 4 && sh.ks == 8) gemm_small_q4_kernel<KIND, 4, 8, NT><<<g, 256, 0, s>>>(p);
  else if (sh.nw == 4 && sh.ks == 16) gemm_small_q4_kernel<KIND, 4, 16, NT><<<g, 256, 0, s>>>(p);
  else if (sh.nw == 8 && sh.ks == 16) gemm_small_q4_kernel<KIND, 8, 16, NT><<<g, 512, 0, s>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemm_small(const GemmParams& p, hipStream_t s) {
  if (p.dtype != MOE_BF16 || p.touched == nullptr || p.shared_T != 0 || p.N % 8 != 0 ||
      p.K % 8 != 0 || small_shape(p.K).nw == 0)
    return hipErrorInvalidValue;
  // at most min(P, E) experts hold rows
  const int slots = p.P < p.E ? p.P : p.E;
  if (p.quant == MOE_QUANT_Q4_G64) {
    if (p.K % 64 != 0 || p.b0_sb == nullptr || (p.kind == 0 && p.b1_sb == nullptr))
      return hipErrorInvalidValue;
    if (p.kind == 0) return launch_small_q4<0, 1>(p, slots, s);
    return launch_small_q4<1, 2>(p, slots, s);
  }
  if (p.kind == 0) return launch_small_kind<0, 1>(p, slots, s);
  return launch_small_kind<1, 2>(p, slots, s);
}

}  // namespace moe
