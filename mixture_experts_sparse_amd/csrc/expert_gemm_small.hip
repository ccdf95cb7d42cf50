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
#include "tiny_route.h"

#include <type_traits>

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

// The slot's expert, first row and rows, from the touched table, or with FR
// (route in gate/up) from the split router's logits through tiny_route.
template <bool FR>
__device__ __forceinline__ void small_slot(const GemmParams& p, const RouteParams& rp,
                                           std::conditional_t<FR, TinyRouteLds, int>& S,
                                           int slot, int& ntouched, int4& ti) {
  if constexpr (FR) {
    tiny_route(rp, S, blockIdx.x == 0, true);
    ntouched = S.ntouched;
    ti = S.touched[min(slot, kWave - 1)];
  } else {
    // one load gives the slot's expert and rows (slot < E: always in the table)
    ntouched = p.meta[1];
    ti = *reinterpret_cast<const int4*>(p.touched + 4 * slot);
    // both loads in flight together, ahead of the exit test
    pin_s(ntouched); pin_s(ti.x); pin_s(ti.y); pin_s(ti.z);
  }
}

// The word that names sorted row r's token (r in [0, P)): its perm entry
// (the pair), or with FR the token tiny_route left in LDS; and the token it
// names. The division waits for the load, so it stays apart from it.
template <bool FR>
__device__ __forceinline__ int small_row_word(const GemmParams& p,
                                              const std::conditional_t<FR, TinyRouteLds, int>& S,
                                              int r) {
  if constexpr (FR) return S.row_token[min(r, kTinyT * kWave - 1)];
  else return p.perm[r];
}
template <bool FR>
__device__ __forceinline__ int small_word_token(const GemmParams& p, int w) {
  return min(max(FR ? w : w / p.k, 0), p.a_rows - 1);
}

template <int KIND, int NW, int KS, int NT, bool FR>
__global__ __launch_bounds__(NW * 64) void gemm_small_kernel(GemmParams p, RouteParams rp) {
  static_assert(!FR || (KIND == 0 && NW >= kTinyT), "the route runs in gate/up workgroups");
  constexpr int NB = KIND == 0 ? 2 : 1;  // weight matrices: gate and up, or down
  constexpr int NCOL = 16 * NT;          // output columns per workgroup
  __shared__ float red[NW][NB][16][NCOL];
  __shared__ std::conditional_t<FR, TinyRouteLds, int> S;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int N = p.N, K = p.K;
  const int ncs = (N + NCOL - 1) / NCOL;
  const int slot = blockIdx.x / ncs;
  const int n0 = (blockIdx.x - slot * ncs) * NCOL;
  int ntouched;
  int4 ti;
  small_slot<FR>(p, rp, S, slot, ntouched, ti);
  if (slot >= ntouched) return;
  const int e = min(max(ti.x, 0), p.E - 1);
  // rows are clamped so every row index stays in [0, P)
  const int r0 = min(max(ti.y, 0), p.P);
  const int cnt = min(max(ti.z, 0), p.P - r0);
  const int kb = wave * KS * 32 + (lane >> 4) * 8;  // this lane's first K index
  const uint16_t* A = static_cast<const uint16_t*>(p.a);

  // the first row block's perm words go out before the weights, so the
  // x rows' addresses are known while the weights are still in flight
  int first_word = 0;
  if constexpr (KIND == 0)
    first_word = small_row_word<FR>(p, S, min(max(r0 + min(lane & 15, cnt - 1), 0), p.P - 1));

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
      const int tok = small_word_token<FR>(p, rb == 0 ? first_word : small_row_word<FR>(p, S, r0 + rr));
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
// K values kb + 64 G + 16 g + 8 h .. + 7 (x and weights alike, each 8 in the
// order codes_bf16 gives them). A lane then
// reads its 16 codes of a group as one 8-byte load and the group's scale and
// bias as one 4-byte word.
//
// The weights are never dequantised one by one. Within a group,
//   sum_k x_k (s q_k + b) = s sum_k x_k (128 + q_k) + (b - 128 s) sum_k x_k,
// and 128 + q (q < 16) is an exact bf16 whose bit pattern is 0x4300 | q, so
// the codes become MFMA operands at under one integer operation each; each
// group's two MFMA steps accumulate on their own, the x row sums of the group
// come from two MFMAs against ones, and the scale and bias are applied to the
// group's accumulator with two FMAs per output.
// ---------------------------------------------------------------------------

// The 8 codes of D (code i in nibble i) as exact bf16 values 128 + q, in 7
// integer operations: each 32-bit output takes one nibble from bytes 0 and 2
// (or 1 and 3) of D, so a shift and one and-or make the pair. The K order is
// then q0 q4 q2 q6 q1 q5 q3 q7, and the x operand is loaded in the same order
// (x_perm8); an MFMA's sum over its K positions does not depend on their order.
__device__ __forceinline__ u32x4_t codes_bf16(uint32_t D) {
  // the exponent bytes as a register operand, so that each pair is one
  // and-or (a 3-operand instruction takes at most one constant)
  uint32_t e = 0x43004300u;
  asm("" : "+v"(e));
  u32x4_t r;
  r[0] = (D & 0x000F000Fu) | e;          // q0, q4
  r[1] = ((D >> 8) & 0x000F000Fu) | e;   // q2, q6
  r[2] = ((D >> 4) & 0x000F000Fu) | e;   // q1, q5
  r[3] = ((D >> 12) & 0x000F000Fu) | e;  // q3, q7
  return r;
}
// 8 consecutive bf16 values x0..x7 (pairs in 32-bit words, low half first)
// in the K order of codes_bf16: x0 x4 x2 x6 x1 x5 x3 x7.
__device__ __forceinline__ u32x4_t x_perm8(u32x4_t w) {
  u32x4_t r;
  r[0] = __builtin_amdgcn_perm(w[2], w[0], 0x05040100u);  // x0, x4
  r[1] = __builtin_amdgcn_perm(w[3], w[1], 0x05040100u);  // x2, x6
  r[2] = __builtin_amdgcn_perm(w[2], w[0], 0x07060302u);  // x1, x5
  r[3] = __builtin_amdgcn_perm(w[3], w[1], 0x07060302u);  // x3, x7
  return r;
}

// A workgroup's codes and scale words are staged in LDS first. A column's
// codes are K/2 contiguous bytes and the workgroup's columns are adjacent
// rows of the expert's matrix, so direct global->LDS loads of 16 bytes per
// lane read whole cache lines (1 KB per wave instruction); loading each
// lane's 8 bytes of a group straight into registers instead touches 16 lines
// per instruction for 32 bytes each, and the L2's request rate, not the
// bytes, then sets the kernel's time (measured on MI355X: 4-bit decode at
// T = 64 took 142 us per layer that way, 108 us staged).
// Codes sit in LDS as rows of K/2 bytes with each row's 16-byte chunks
// XOR-swizzled by the row (chunk c of row r at c ^ (r mod Z)), so the 16 rows
// one MFMA fragment reads fall in different bank groups; scale words sit as
// rows of (K/64 | 1) words (an odd stride: conflict-free word reads).
template <int KIND, int NW, int KS, int NT, bool FR>
__global__ __launch_bounds__(NW * 64) void gemm_small_q4_lds(GemmParams p, RouteParams rp) {
  static_assert(!FR || (KIND == 0 && NW >= kTinyT), "the route runs in gate/up workgroups");
  constexpr int NB = KIND == 0 ? 2 : 1;
  constexpr int NCOL = 16 * NT;
  constexpr int KG = KS / 2;
  constexpr int NTHR = NW * 64;
  constexpr int KMAX = NW * KS * 32;
  static_assert(KS % 2 == 0, "whole scale groups per wave");
  constexpr int CODE_ROUND = (NB * NCOL * (KMAX / 2) + NTHR * 16 - 1) / (NTHR * 16) * (NTHR * 16);
  constexpr int SW_MAX = (KMAX / 64) | 1;
  constexpr int SC_ROUND = (NB * NCOL * SW_MAX + NTHR - 1) / NTHR * NTHR;
  // the wide shapes (gate/up with 32 columns, down with 128): the cross-wave
  // partial sums reuse the code buffer once a row block's products are done
  // (the codes are staged again for a further row block), so two such
  // workgroups fit a CU; the narrow ones, limited by registers rather than
  // LDS, keep a buffer of their own
  constexpr bool ALIAS = KIND == 0 ? NT == 2 : NT == 8;
  constexpr int RED_BYTES = NW * NB * 16 * NCOL * 4;
  constexpr int LC_BYTES = ALIAS && RED_BYTES > CODE_ROUND ? RED_BYTES : CODE_ROUND;
  __shared__ __align__(16) uint8_t Lc[LC_BYTES];
  __shared__ __align__(16) uint32_t Ls[SC_ROUND];
  __shared__ __align__(16) float red_own[ALIAS ? 1 : NW][NB][16][NCOL];
  auto red = ALIAS ? reinterpret_cast<float (*)[NB][16][NCOL]>(Lc) : red_own;
  // the route's LDS lies over red_own: its last read (the slot's first row
  // tokens) comes before the staging barrier, the first write to red_own
  // after it, and no other buffer has room to spare when two wide
  // workgroups share a CU
  using RouteLds = std::conditional_t<FR, TinyRouteLds, int>;
  static_assert(sizeof(RouteLds) <= sizeof(red_own), "route LDS fits the partial-sum buffer");
  RouteLds& S = *reinterpret_cast<RouteLds*>(&red_own[0][0][0][0]);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int N = p.N, K = p.K;
  const int ncs = (N + NCOL - 1) / NCOL;
  const int slot = blockIdx.x / ncs;
  const int n0 = (blockIdx.x - slot * ncs) * NCOL;
  int ntouched;
  int4 ti;
  small_slot<FR>(p, rp, S, slot, ntouched, ti);
  if (slot >= ntouched) return;
  const int e = min(max(ti.x, 0), p.E - 1);
  const int r0 = min(max(ti.y, 0), p.P);
  const int cnt = min(max(ti.z, 0), p.P - r0);
  const uint16_t* A = static_cast<const uint16_t*>(p.a);
  int first_word = 0;
  if constexpr (KIND == 0)
    first_word = small_row_word<FR>(p, S, min(max(r0 + min(lane & 15, cnt - 1), 0), p.P - 1));

  // codes: rows R = m * NCOL + r (matrix m, column n0 + r), RB bytes each
  const int RB = K / 2;
  const int CPR = RB / 16;  // 16-byte chunks per row (even: K is a multiple of 64)
  const int Z = (CPR % 8 == 0) ? 8 : ((CPR % 4 == 0) ? 4 : 2);
  const int nchunk = NB * NCOL * CPR;
  const int crounds = (nchunk + NTHR - 1) / NTHR;
  const uint8_t* Q0 = static_cast<const uint8_t*>(p.b0) + static_cast<size_t>(e) * N * RB;
  const uint8_t* Q1 = static_cast<const uint8_t*>(KIND == 0 ? p.b1 : p.b0) + static_cast<size_t>(e) * N * RB;
  // load i of this thread stages chunk i * NTHR + tid = row R, chunk pc of
  // the row; (R, pc) advance by (NTHR / CPR, NTHR % CPR) per load, with no
  // division in the loop. Past the last row: reload the last chunk (never read).
  constexpr int NROWS = NB * NCOL;
  const int qa = NTHR / CPR, ra = NTHR - qa * CPR;
  const int R00 = tid / CPR, pc00 = tid - R00 * CPR;
  auto stage_codes = [&]() {
    int R = R00, pc = pc00;
    for (int i = 0; i < crounds; ++i) {
      const bool past = R >= NROWS;
      const int Rc = past ? NROWS - 1 : R, pcc = past ? CPR - 1 : pc;
      const int lc = pcc ^ (Rc & (Z - 1));
      const int m = Rc / NCOL, r = Rc - m * NCOL;
      const int n = min(n0 + r, N - 1);
      const uint8_t* src = (m == 0 ? Q0 : Q1) + static_cast<size_t>(n) * RB + lc * 16;
      lds_void_t* dst = (lds_void_t*)(Lc + (i * NTHR + wave * 64) * 16);
      __builtin_amdgcn_global_load_lds((gbl_void_t*)src, dst, 16, 0, 0);
      pc += ra;
      R += qa;
      if (pc >= CPR) { pc -= CPR; ++R; }
    }
  };
  stage_codes();
  // scale words: rows of SW = (K / 64) | 1 words (the pad word reloads the
  // last), word i * NTHR + tid = (row R, word g) advanced the same way
  const int NG = K / 64;
  const int SW = NG | 1;
  const int nword = NB * NCOL * SW;
  const int srounds = (nword + NTHR - 1) / NTHR;
  const uint32_t* S0 = p.b0_sb + static_cast<size_t>(e) * N * NG;
  const uint32_t* S1 = (KIND == 0 ? p.b1_sb : p.b0_sb) + static_cast<size_t>(e) * N * NG;
  {
    const int qs = NTHR / SW, rs = NTHR - qs * SW;
    int R = tid / SW, g = tid - (tid / SW) * SW;
    for (int i = 0; i < srounds; ++i) {
      const bool past = R >= NROWS;
      const int Rc = past ? NROWS - 1 : R, gc = past ? NG - 1 : min(g, NG - 1);
      const int m = Rc / NCOL, r = Rc - m * NCOL;
      const int n = min(n0 + r, N - 1);
      const uint32_t* src = (m == 0 ? S0 : S1) + static_cast<size_t>(n) * NG + gc;
      lds_void_t* dst = (lds_void_t*)(Ls + i * NTHR + wave * 64);
      __builtin_amdgcn_global_load_lds((gbl_void_t*)src, dst, 4, 0, 0);
      g += rs;
      R += qs;
      if (g >= SW) { g -= SW; ++R; }
    }
  }
  const int kb = wave * KS * 32 + (lane >> 4) * 16;  // lane's first K index in the wave's group 0
  const int j = lane >> 4;
  bool staged = false;

  for (int rb = 0; rb < cnt; rb += 16) {
    const int rr = min(rb + (lane & 15), cnt - 1);
    const uint16_t* arow;
    if constexpr (KIND == 0) {
      const int tok = small_word_token<FR>(p, rb == 0 ? first_word : small_row_word<FR>(p, S, r0 + rr));
      arow = A + static_cast<size_t>(tok) * K;
    } else {
      arow = A + static_cast<size_t>(r0 + rr) * K;
    }
    u32x4_t aq[KS];
#pragma unroll
    for (int G = 0; G < KG; ++G)
#pragma unroll
      for (int h = 0; h < 2; ++h) aq[2 * G + h] = x_perm8(load_k8(arow, kb + 64 * G + 8 * h, K));
    if (!staged) {
      // every wave's staging loads have landed (the x rows are behind them)
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      staged = true;
    }
    floatx4_t acc[NB][NT];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[m][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
    const floatx4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int G = 0; G < KG; ++G) {
      // groups past K read the last group (the x operand is zero there)
      const int Gw = min(wave * KG + G, NG - 1);
      const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, aq[2 * G]);
      const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, aq[2 * G + 1]);
      floatx4_t xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          a0, __builtin_bit_cast(bf16x8_t, ones), zero, 0, 0, 0);
      xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8_t, ones), xs, 0,
                                                   0, 0);
      const int lc = 2 * Gw + (j >> 1);
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int R = m * NCOL + t * 16 + (lane & 15);
          const uint2 qc = *reinterpret_cast<const uint2*>(
              Lc + R * RB + ((lc ^ (R & (Z - 1))) * 16) + (j & 1) * 8);
          const uint32_t sb = Ls[R * SW + Gw];
          floatx4_t ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a0, __builtin_bit_cast(bf16x8_t, codes_bf16(qc.x)), zero, 0, 0, 0);
          ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a1, __builtin_bit_cast(bf16x8_t, codes_bf16(qc.y)), ag, 0, 0, 0);
          const float sc = bf16_to_f32(static_cast<uint16_t>(sb & 0xFFFFu));
          const float b2 = fmaf(-128.0f, sc, bf16_to_f32(static_cast<uint16_t>(sb >> 16)));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][t][i] = fmaf(sc, ag[i], fmaf(b2, xs[i], acc[m][t][i]));
        }
    }
    if constexpr (ALIAS) __syncthreads();  // every wave is done with the codes: the sums overwrite them
    small_block_epilogue<KIND, NW, NB, NT>(p, red, acc, r0, rb, cnt, n0);
    if (ALIAS && rb + 16 < cnt) {  // uniform: another row block needs the codes again
      stage_codes();
      staged = false;
    }
  }
  // no staging load may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0);
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

// ---------------------------------------------------------------------------
// One token (T = 1): the down projection and the combine in one launch.
// With one token each chosen expert holds one row, sorted row w being the
// w-th touched expert. A workgroup owns kDcCols output columns of every
// row: wave w takes row w, lane l column n0 + l / 8, and load i of a lane
// reads K values 64 i + 8 (l % 8) .. + 7 of its column's weight row and of
// the act row -- one whole 128-byte line of each of the 8 columns per load
// instruction. The lane's dot product is summed over the 8 lanes of its
// column by DPP moves and rounded to bf16, the value the down kernel would
// store as y; after a barrier 8 threads add the rows in slot order with
// their gates, then the gated shared row, and round once, as the combine
// kernel does ("Tutorial 11: Mixture of Experts (MoE)", section 3, steps
// 2 and 3).
// ---------------------------------------------------------------------------
constexpr int kDcCols = 8;  // output columns per workgroup (8 lanes each)

// A lane's share of one column's product, bf16 weights: load i holds K
// values 64 i + sub .. + 7 of the weight row and of the act row.
template <int NL>
__device__ __forceinline__ float dc_dot_bf16(const GemmParams& p, int e, int col, int row, int sub) {
  const int K = p.K, nk = K / 64;
  const uint16_t* wrow = static_cast<const uint16_t*>(p.b0) +
                         (static_cast<size_t>(e) * p.N + col) * K + sub;
  const uint16_t* arow = static_cast<const uint16_t*>(p.a) + static_cast<size_t>(row) * K + sub;
  u32x4_t wq[NL], aq[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    // loads past K reread the last line (their products are skipped)
    const int ki = min(i, nk - 1) * 64;
    wq[i] = *reinterpret_cast<const u32x4_t*>(wrow + ki);
    aq[i] = *reinterpret_cast<const u32x4_t*>(arow + ki);
  }
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    if (i < nk) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s0 = fmaf(__uint_as_float(aq[i][q] << 16), __uint_as_float(wq[i][q] << 16), s0);
        s1 = fmaf(__uint_as_float(aq[i][q] & 0xFFFF0000u), __uint_as_float(wq[i][q] & 0xFFFF0000u), s1);
      }
    }
  }
  return s0 + s1;
}

// The same for 4-bit weights (codes [E, N, K/2], scale|bias words
// [E, N, K/64], w = s q + b): load i holds the 16 code bytes of chunk
// ch = sub8 + 8 i (K values 32 ch .. + 31, one scale group), the group's
// word and the 32 act values; per chunk s * sum(a q) + b * sum(a).
template <int NQ>
__device__ __forceinline__ float dc_dot_q4(const GemmParams& p, int e, int col, int row, int sub8) {
  const int K = p.K, nch = K / 32, NG = K / 64;
  const uint8_t* crow = static_cast<const uint8_t*>(p.b0) +
                        (static_cast<size_t>(e) * p.N + col) * (K / 2);
  const uint32_t* srow = p.b0_sb + (static_cast<size_t>(e) * p.N + col) * NG;
  const uint16_t* arow = static_cast<const uint16_t*>(p.a) + static_cast<size_t>(row) * K;
  u32x4_t cq[NQ], aq[NQ][4];
  uint32_t sb[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    // chunks past K reread the last (their products are skipped)
    const int ch = min(sub8 + 8 * i, nch - 1);
    cq[i] = *reinterpret_cast<const u32x4_t*>(crow + ch * 16);
    sb[i] = srow[ch >> 1];
#pragma unroll
    for (int w = 0; w < 4; ++w) aq[i][w] = *reinterpret_cast<const u32x4_t*>(arow + ch * 32 + w * 8);
  }
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    if (sub8 + 8 * i < nch) {
      float saq = 0.f, sa = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // code word w: byte m holds K values 8 w + 2 m (low nibble) and + 1
        // (high nibble), act dword m the same two values (low, high half)
        const uint32_t lo = cq[i][w] & 0x0F0F0F0Fu, hi = (cq[i][w] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float a0 = __uint_as_float(aq[i][w][m] << 16);
          const float a1 = __uint_as_float(aq[i][w][m] & 0xFFFF0000u);
          saq = fmaf(a0, static_cast<float>((lo >> (8 * m)) & 0xFFu), saq);
          saq = fmaf(a1, static_cast<float>((hi >> (8 * m)) & 0xFFu), saq);
          sa += a0 + a1;
        }
      }
      const float sc = bf16_to_f32(static_cast<uint16_t>(sb[i] & 0xFFFFu));
      const float bi = bf16_to_f32(static_cast<uint16_t>(sb[i] >> 16));
      acc = fmaf(sc, saq, fmaf(bi, sa, acc));
    }
  }
  return acc;
}

template <bool Q4>
__global__ __launch_bounds__(kDownCombineRows * 64) void down_combine_t1_kernel(GemmParams p,
                                                                              CombineParams c) {
  __shared__ float yv[kDownCombineRows][kDcCols];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * kDcCols;
  const int P = p.P;
  // the combine's inputs do not depend on the products: they go out first
  int rj[kDownCombineRows];
  float gj[kDownCombineRows];
  float sh = 0.f, sc = 0.f;
  if (tid < kDcCols) {
#pragma unroll
    for (int j = 0; j < kDownCombineRows; ++j) {
      rj[j] = c.inv[min(j, c.k - 1)];
      gj[j] = c.gates[min(j, c.k - 1)];
    }
    if (c.shared != nullptr) {
      sh = bf16_to_f32(static_cast<const uint16_t*>(c.shared)[n0 + tid]);
      sc = c.shared_scale != nullptr ? c.shared_scale[0] : 1.0f;
    }
  }
  // this wave's row: its expert from the touched table
  const int r = min(__builtin_amdgcn_readfirstlane(wave), P - 1);  // wave-uniform
  int4 ti = *reinterpret_cast<const int4*>(p.touched + 4 * r);
  pin_s(ti.x); pin_s(ti.y);
  const int e = min(max(ti.x, 0), p.E - 1);
  const int row = min(max(ti.y, 0), P - 1);
  const int col = min(n0 + (lane >> 3), p.N - 1);
  float v;
  if constexpr (Q4) v = dc_dot_q4<kDownCombineMaxK / 256>(p, e, col, row, lane & 7);
  else v = dc_dot_bf16<kDownCombineMaxK / 64>(p, e, col, row, (lane & 7) * 8);
  // the 8 lanes of a column: pairs, quads, then the two quads of the 8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  if ((lane & 7) == 0) yv[wave][lane >> 3] = wave < P ? bf16_to_f32(f32_to_bf16(v)) : 0.f;
  __syncthreads();
  if (tid < kDcCols) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kDownCombineRows; ++j)
      if (j < c.k) acc = fmaf(gj[j], yv[min(max(rj[j], 0), P - 1)][tid], acc);
    if (c.shared != nullptr) acc = fmaf(sc, sh, acc);
    static_cast<uint16_t*>(c.out)[n0 + tid] = f32_to_bf16(acc);
  }
}

// A few tokens (2 <= T <= MOE_DOWN_COMBINE_MAX_T, at most kDownCombineMaxRows
// rows, k <= kDownCombineRows; bf16 experts): the same launch with each wave
// taking rows wave, wave + 8, ..., a row's expert read from a row -> expert
// table the workgroup first builds in LDS from the touched table (an expert
// may hold several rows now), and thread (t, column) combining token t.
__global__ __launch_bounds__(kDownCombineRows * 64) void down_combine_few_kernel(GemmParams p,
                                                                               CombineParams c) {
  __shared__ float yv[kDownCombineMaxRows][kDcCols];
  __shared__ int rowexp[kDownCombineMaxRows];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * kDcCols;
  const int P = p.P, T = c.T, k = c.k;
  // the combine's inputs first: thread (ct, cc) combines token ct, column n0 + cc
  const int ct = tid / kDcCols, cc = tid - (tid / kDcCols) * kDcCols;
  int rj[kDownCombineRows];
  float gj[kDownCombineRows];
  float sh = 0.f, sc = 0.f;
  if (ct < T) {
#pragma unroll
    for (int j = 0; j < kDownCombineRows; ++j) {
      const int q = ct * k + min(j, k - 1);
      rj[j] = c.inv[q];
      gj[j] = c.gates[q];
    }
    if (c.shared != nullptr) {
      sh = bf16_to_f32(static_cast<const uint16_t*>(c.shared)[static_cast<size_t>(ct) * c.d + n0 + cc]);
      sc = c.shared_scale != nullptr ? c.shared_scale[ct] : 1.0f;
    }
  }
  // row -> expert: touched entry i covers rows [first, first + rows)
  if (tid < min(P, p.E) && tid < p.meta[1]) {
    const int4 ti = *reinterpret_cast<const int4*>(p.touched + 4 * tid);
    const int r0 = min(max(ti.y, 0), P), r1 = min(r0 + max(ti.z, 0), P);
    for (int r = r0; r < r1; ++r) rowexp[r] = ti.x;
  }
  __syncthreads();
  const int col = min(n0 + (lane >> 3), p.N - 1);
#pragma unroll 1
  for (int r = wave; r < P; r += kDownCombineRows) {
    const int e = min(max(__builtin_amdgcn_readfirstlane(rowexp[r]), 0), p.E - 1);
    float v = dc_dot_bf16<kDownCombineMaxK / 64>(p, e, col, r, (lane & 7) * 8);
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    if ((lane & 7) == 0) yv[r][lane >> 3] = bf16_to_f32(f32_to_bf16(v));
  }
  __syncthreads();
  if (ct < T) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kDownCombineRows; ++j)
      if (j < k) acc = fmaf(gj[j], yv[min(max(rj[j], 0), P - 1)][cc], acc);
    if (c.shared != nullptr) acc = fmaf(sc, sh, acc);
    static_cast<uint16_t*>(c.out)[static_cast<size_t>(ct) * c.d + n0 + cc] = f32_to_bf16(acc);
  }
}

hipError_t launch_down_combine(const GemmParams& p, const CombineParams& c, hipStream_t s) {
  const bool q4 = p.quant == MOE_QUANT_Q4_G64;
  if (p.dtype != MOE_BF16 || (!q4 && p.quant != MOE_QUANT_NONE) || (q4 && p.b0_sb == nullptr) ||
      p.kind != 1 || c.T < 1 || c.T > MOE_DOWN_COMBINE_MAX_T || (q4 && c.T != 1) || c.k < 1 ||
      c.k > kDownCombineRows || c.T * c.k != p.P || p.P > kDownCombineMaxRows ||
      p.K % 64 != 0 || p.K > kDownCombineMaxK || p.N != c.d || p.N % kDcCols != 0 ||
      p.touched == nullptr || p.meta == nullptr)
    return hipErrorInvalidValue;
  const unsigned g = static_cast<unsigned>(p.N / kDcCols);
  if (c.T == 1) {
    if (q4) down_combine_t1_kernel<true><<<g, kDownCombineRows * 64, 0, s>>>(p, c);
    else down_combine_t1_kernel<false><<<g, kDownCombineRows * 64, 0, s>>>(p, c);
  } else {
    down_combine_few_kernel<<<g, kDownCombineRows * 64, 0, s>>>(p, c);
  }
  return hipGetLastError();
}

// One launch of the small-batch GEMM. The persistent form keeps the weight
// stream running across items, which pays when every CU has several items;
// measured on MI355X it helps the down projection (one weight matrix, 32
// columns per item) and not gate/up, whose one-shot workgroups already
// stream its two matrices at about 5.8 TB/s.
template <int KIND, int NT, bool FR>
static hipError_t launch_small_kind(const GemmParams& p, const RouteParams& rp, int slots,
                                    hipStream_t s) {
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
  if (sh.nw == 4 && sh.ks == 4) gemm_small_kernel<KIND, 4, 4, NT, FR><<<g, 256, 0, s>>>(p, rp);
  else if (sh.nw == 4 && sh.ks == 8) gemm_small_kernel<KIND, 4, 8, NT, FR><<<g, 256, 0, s>>>(p, rp);
  else if (sh.nw == 4 && sh.ks == 16) gemm_small_kernel<KIND, 4, 16, NT, FR><<<g, 256, 0, s>>>(p, rp);
  else if (sh.nw == 8 && sh.ks == 16) gemm_small_kernel<KIND, 8, 16, NT, FR><<<g, 512, 0, s>>>(p, rp);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int KIND, int NT, bool FR>
static hipError_t launch_small_q4(const GemmParams& p, const RouteParams& rp, int slots,
                                  hipStream_t s) {
  // eight waves split reductions above 512 (half the registers per wave of
  // four, so twice the workgroups per CU)
  SmallShape sh;
  if (p.K <= 4 * 4 * 32) sh = {4, 4};
  else if (p.K <= 8 * 4 * 32) sh = {8, 4};
  else if (p.K <= 8 * 8 * 32) sh = {8, 8};
  else sh = {8, 16};
  const long long nblk = static_cast<long long>(slots) * ceil_div(p.N, 16 * NT);
  if (nblk <= 0) return hipSuccess;
  const unsigned g = static_cast<unsigned>(nblk);
  if (sh.nw == 4) gemm_small_q4_lds<KIND, 4, 4, NT, FR><<<g, 256, 0, s>>>(p, rp);
  else if (sh.ks == 4) gemm_small_q4_lds<KIND, 8, 4, NT, FR><<<g, 512, 0, s>>>(p, rp);
  else if constexpr (NT <= 2) {  // the widest shapes' codes do not fit LDS above K = 1024
    if (sh.ks == 8) gemm_small_q4_lds<KIND, 8, 8, NT, FR><<<g, 512, 0, s>>>(p, rp);
    else gemm_small_q4_lds<KIND, 8, 16, NT, FR><<<g, 512, 0, s>>>(p, rp);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NT>
static hipError_t launch_q4_gate_up(const GemmParams& p, const RouteParams* route, int slots,
                                    hipStream_t s) {
  if (route != nullptr) return launch_small_q4<0, NT, true>(p, *route, slots, s);
  return launch_small_q4<0, NT, false>(p, RouteParams{}, slots, s);
}

hipError_t launch_gemm_small(const GemmParams& p, hipStream_t s, const RouteParams* route) {
  if (p.dtype != MOE_BF16 || p.touched == nullptr || p.shared_T != 0 || p.N % 8 != 0 ||
      p.K % 8 != 0 || small_shape(p.K).nw == 0)
    return hipErrorInvalidValue;
  // the route inside gate/up: at most kTinyT tokens and kWave experts, from
  // the split router's logits, with the dispatch tables to store
  if (route != nullptr &&
      (p.kind != 0 || route->T < 1 || route->T > kTinyT || route->E > kWave ||
       route->T != p.a_rows || route->E != p.E || route->T * route->k != p.P ||
       route->part == nullptr || route->counts == nullptr || route->touched == nullptr))
    return hipErrorInvalidValue;
  // at most min(P, E) experts hold rows
  const int slots = p.P < p.E ? p.P : p.E;
  if (p.quant == MOE_QUANT_Q4_G64) {
    if (p.K % 64 != 0 || p.b0_sb == nullptr || (p.kind == 0 && p.b1_sb == nullptr))
      return hipErrorInvalidValue;
    // gate/up: 32 columns per workgroup once the grid has more than four
    // workgroups of 16 columns per CU (two of them then fit a CU), else 16
    if (p.kind == 0) {
      if (static_cast<long long>(slots) * ceil_div(p.N, 16) > 4LL * device_cus())
        return launch_q4_gate_up<2>(p, route, slots, s);
      return launch_q4_gate_up<1>(p, route, slots, s);
    }
    // down: 128 columns per workgroup on the same condition, for reductions
    // up to 1024 (32 columns otherwise)
    if (p.K <= 1024 && static_cast<long long>(slots) * ceil_div(p.N, 32) > 4LL * device_cus())
      return launch_small_q4<1, 8, false>(p, RouteParams{}, slots, s);
    return launch_small_q4<1, 2, false>(p, RouteParams{}, slots, s);
  }
  if (p.kind == 0) {
    if (route != nullptr) return launch_small_kind<0, 1, true>(p, *route, slots, s);
    return launch_small_kind<0, 1, false>(p, RouteParams{}, slots, s);
  }
  return launch_small_kind<1, 2, false>(p, RouteParams{}, slots, s);
}

}  // namespace moe
