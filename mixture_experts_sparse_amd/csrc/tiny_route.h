// Selection, gates and dispatch tables of the smallest batches (at most
// kTinyT tokens, at most kWave experts) from the split router's float32
// logits, as one workgroup-level device function.
//
// Top-k per token with ties to the lower expert index and slots in
// descending score order, then gates: softmax over all experts gathered at
// the selection (renormalised or not), softmax over the selected logits, or
// the raw sigmoid affinities ("Tutorial 11: Mixture of Experts (MoE)",
// section 2 "The Router"; "Small models, sparse experts", How it works,
// step 3; "Small MoE Architecture, in depth", A small MoE layer in PyTorch).
// Dispatch is the stable counting sort of the pairs by expert (Tutorial 11,
// section 3, step 1): with one row per (token, expert) at most, an expert's
// rows are the tokens that chose it, in token order.
//
// Two callers share it so that their tables agree bit for bit: the
// one-launch finish of the split router, and the small-batch gate/up GEMM,
// whose every workgroup derives its expert and rows from the logits itself
// (one launch fewer per layer; workgroup 0 also stores the tables for the
// kernels after it).

#pragma once

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int kTinyT = 4;  // most tokens of the one-launch selection (one wave each)

// order-preserving 32-bit key of a float (finite values; -0 and +0 equal
// once the caller adds +0.0)
__device__ __forceinline__ uint32_t tiny_key32(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_excl_scan(int v, int& total) {
  const int lane = threadIdx.x & 63;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  total = __shfl(x, kWave - 1, kWave);
  return x - v;
}

// Sum of v over the wave, the same in every lane: each 16-lane row is summed
// by DPP moves (pairs, quads, the 8- and 16-lane mirrors; IEEE addition
// commutes, so every lane of a row holds the same bits), then the four row
// sums are read out and added in row order. No LDS round trips.
__device__ __forceinline__ float wave_total(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  const int b = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

struct TinyRouteLds {
  uint32_t keys[kTinyT][kWave];
  uint64_t chose[kTinyT];         // token t's chosen experts as a lane mask
  int8_t slot_of[kTinyT][kWave];  // slot of (token, expert) when chosen
  // filled when the caller asks for the tables in LDS
  int4 touched[kWave];            // {e, first row, rows, 0}, ascending e
  int8_t row_token[kTinyT * kWave];  // token of each sorted row
  int ntouched;
};

// Called by every thread of a workgroup of at least kTinyT waves (wave t
// takes token t, lane e expert e; further waves only keep the barriers).
// store: write ids, gates, the shared gate, logits (when given) and, when
// p.counts is set, counts, offsets, exp_tile0, touched, tile_e, perm, inv
// and meta -- the outputs of route_finish_kernel. to_lds: also leave the
// touched table, its count and each sorted row's token in S.
// Three workgroup barriers when to_lds, two otherwise. The path is short
// on purpose (one batch of LDS reads for the ranks, DPP sums, ballots
// instead of scans): the small-batch gate/up GEMM runs it before its
// weight loads can go out.
__device__ __forceinline__ void tiny_route(const RouteParams& p, TinyRouteLds& S, bool store,
                                           bool to_lds) {
  const int e = threadIdx.x & 63;  // expert of this lane
  const int t = threadIdx.x >> 6;  // token of this wave
  const int E = p.E, k = p.k, T = p.T;
  const bool sw = t < kTinyT;      // a selecting wave
  const bool valid = e < E;
  const bool live = sw && t < T;   // uniform across the wave
  const bool sig = p.mode == MOE_SIGMOID;
  // every load before the first use, clamped: the bias, this (token,
  // expert) logit and the token's shared-gate logit
  float b = 0.f;
  if (p.bias != nullptr) b = p.bias[min(e, E - 1)];
  const size_t row = static_cast<size_t>(min(t, T - 1)) * p.ncp;
  float raw = p.part[row + min(e, E - 1)];
  float sgl = 0.f;
  if (p.sgate != nullptr) sgl = p.part[row + E];
  pin(b);
  pin(raw);
  pin(sgl);
  if (!valid) b = 0.f;
  // logits (in the softmax modes with the bias) and the selection score;
  // a valid lane's key is never 0 (finite scores), a lane past E has key 0
  const float v = sig ? raw : raw + b;
  const float score = sig ? sigmoid_f32(raw) + b : v;
  const uint32_t key = valid ? tiny_key32(score + 0.0f) : 0u;  // -0 -> +0
  if (sw) S.keys[t][e] = key;
  __syncthreads();
  if (sw) {
    // rank: the keys that beat this one (larger, or equal at a lower
    // index), all 64 read in one batch (the zero keys past E beat none)
    u32x4_t kq[kWave / 4];
#pragma unroll
    for (int i = 0; i < kWave / 4; ++i) kq[i] = *reinterpret_cast<const u32x4_t*>(&S.keys[t][4 * i]);
    int n4[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < kWave / 4; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u) n4[u] += (kq[i][u] > key || (kq[i][u] == key && 4 * i + u < e)) ? 1 : 0;
    const int rank = (n4[0] + n4[1]) + (n4[2] + n4[3]);
    const bool sel = live && valid && rank < k;
    // gate numerators: exp(L - max) in the softmax modes, where the largest
    // logit is the rank-0 lane's (its score), or the raw sigmoid affinity
    float ej;
    if (sig) {
      ej = valid ? sigmoid_f32(raw) : 0.f;
    } else {
      const uint64_t top = __ballot(valid && rank == 0);
      const int l0 = top != 0 ? __ffsll(static_cast<unsigned long long>(top)) - 1 : 0;
      const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l0));
      ej = valid ? expf(v - m) : 0.f;
    }
    float denom = 1.0f;
    if (p.mode == MOE_SOFTMAX_ALL && !p.renorm) denom = wave_total(ej);
    else if (!sig || p.renorm) denom = wave_total(sel ? ej : 0.f);
    if (store && live) {
      if (p.logits != nullptr && valid) p.logits[static_cast<size_t>(t) * E + e] = v;
      if (p.sgate != nullptr && e == 0) p.sgate[t] = sigmoid_f32(sgl);
      if (sel) {
        p.ids[static_cast<size_t>(t) * k + rank] = e;
        p.gates[static_cast<size_t>(t) * k + rank] = ej * (1.0f / denom);
      }
    }
    const uint64_t chose = __ballot(sel);
    if (e == 0) S.chose[t] = chose;
    S.slot_of[t][e] = static_cast<int8_t>(sel ? rank : -1);
  }
  const bool tables = store && p.counts != nullptr;  // uniform
  if (!tables && !to_lds) return;
  __syncthreads();
  if (t == 0) {
    // dispatch on wave 0, lane e owning expert e: its rows are the tokens
    // that chose it, in token order; first rows and touched indices are
    // popcounts of the choice masks below the lane
    uint64_t M[kTinyT];
#pragma unroll
    for (int u = 0; u < kTinyT; ++u) M[u] = S.chose[u];
    const uint64_t lt = lanemask_lt();
    int cnt = 0, off = 0, total = 0;
    uint64_t any = 0;
#pragma unroll
    for (int u = 0; u < kTinyT; ++u) {
      cnt += static_cast<int>((M[u] >> e) & 1u);
      off += __popcll(M[u] & lt);
      total += __popcll(M[u]);
      any |= M[u];
    }
    const int tidx = __popcll(any & lt);
    const int ntouched = __popcll(any);
    // M tiles per expert: one per touched expert when a tile holds every
    // row a tiny batch can give an expert
    int toff = tidx, ntl = ntouched;
    const int tl = (cnt + p.tile_m - 1) / p.tile_m;
    if (p.tile_m < kTinyT) toff = wave_excl_scan(tl, ntl);
    if (valid) {
      if (tables) {
        p.counts[e] = cnt;
        p.offsets[e] = off;
        p.exp_tile0[e] = toff;
        if (cnt > 0 && p.touched != nullptr)
          *reinterpret_cast<int4*>(p.touched + 4 * tidx) = make_int4(e, off, cnt, 0);
        if (p.tile_e != nullptr)
          for (int j = 0; j < tl; ++j)
            if (toff + j < p.max_tiles) p.tile_e[toff + j] = e;
      }
      if (to_lds && cnt > 0) S.touched[tidx] = make_int4(e, off, cnt, 0);
      int r = off;
#pragma unroll
      for (int u = 0; u < kTinyT; ++u) {
        if ((M[u] >> e) & 1u) {
          const int pair = u * k + S.slot_of[u][e];
          if (tables) {
            p.perm[r] = pair;
            p.inv[pair] = r;
          }
          if (to_lds) S.row_token[r] = static_cast<int8_t>(u);
          ++r;
        }
      }
    }
    if (e == 0) {
      if (tables) {
        p.offsets[E] = total;
        p.exp_tile0[E] = ntl;
        p.meta[0] = min(ntl, p.max_tiles);
        p.meta[1] = ntouched;
      }
      if (to_lds) S.ntouched = ntouched;
    }
  }
  if (to_lds) __syncthreads();
}

}  // namespace moe
