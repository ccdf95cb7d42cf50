// Host side of libmoe.so: argument validation, workspace planning and the
// launch sequence of every entry point declared in include/moe.h.
//
// Every check below is plain host arithmetic that runs before the first HIP
// call, so a rejected call enqueues nothing and the checks run on machines
// without a GPU.

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>

#include "moe_internal.h"

namespace moe {

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

size_t elem_bytes(const moe_config& c) { return c.dtype == MOE_BF16 ? 2 : 4; }

moe_status check_cfg(const moe_config* c) {
  if (c == nullptr) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->d <= 0 || c->E <= 0 || c->h <= 0) return MOE_ERR_INVALID_ARG;
  if (c->top_k < 1 || c->top_k > c->E) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->mode != MOE_SOFTMAX_ALL && c->mode != MOE_SOFTMAX_SELECTED && c->mode != MOE_SIGMOID)
    return MOE_ERR_INVALID_ARG;
  if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (c->has_router_bias != 0 && c->has_router_bias != 1) return MOE_ERR_INVALID_ARG;
  if (c->shared_gate != 0 && c->shared_gate != 1) return MOE_ERR_INVALID_ARG;
  if (c->shared_h < 0) return MOE_ERR_INVALID_ARG;
  if (c->shared_gate && c->shared_h == 0) return MOE_ERR_INVALID_ARG;
  if (c->expert_quant != MOE_QUANT_NONE && c->expert_quant != MOE_QUANT_Q4_G64)
    return MOE_ERR_INVALID_ARG;
  if (c->E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if (c->d % 8 != 0 || c->h % 8 != 0 || c->shared_h % 8 != 0) return MOE_ERR_UNSUPPORTED;
  // int32 row/element indices inside the kernels, and byte offsets of the
  // bf16 outputs below 2^31 (buffer stores mask lanes with offset 2^31)
  const long long P = static_cast<long long>(c->T) * c->top_k;
  const long long big = 1LL << 30;
  if (P * c->d >= big || P * c->h >= big || static_cast<long long>(c->T) * c->d >= big ||
      static_cast<long long>(c->T) * (c->shared_h > 0 ? c->shared_h : 1) >= big)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Required tensor pointer: non-null and 16-byte aligned.
moe_status need(const void* p) {
  if (p == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(p)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Optional tensor pointer: null, or 16-byte aligned.
moe_status maybe(const void* p) {
  if (p != nullptr && !aligned16(p)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

#define MOE_TRY(expr)                   \
  do {                                  \
    const moe_status st_ = (expr);      \
    if (st_ != MOE_OK) return st_;      \
  } while (0)

#define MOE_HIP(expr)                         \
  do {                                        \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

moe_status check_ws(const moe_config& c, int entry, const void* ws, size_t ws_bytes) {
  const size_t need_bytes = moe_workspace_size_entry(&c, entry);
  if (ws_bytes < need_bytes) return MOE_ERR_WORKSPACE;
  if (need_bytes > 0 && (ws == nullptr || !aligned256(ws))) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<unsigned char*>(ws) + off);
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

WsLayout ws_layout(const moe_config& c) {
  const size_t T = static_cast<size_t>(c.T), E = static_cast<size_t>(c.E);
  const size_t P = T * static_cast<size_t>(c.top_k);
  const size_t NB = static_cast<size_t>(ceil_div(c.T, route_tokens(c.T)));
  const size_t MT = static_cast<size_t>(max_m_tiles(static_cast<int>(P), c.E));
  const size_t eb = elem_bytes(c);
  const size_t hs = static_cast<size_t>(c.shared_h);
  WsLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at_ = o;
    o += align256(bytes);
    return at_;
  };
  L.blk_hist = take(NB * E * 4);
  L.lrank = take(P * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm = take(P * 4);
  L.inv = take(P * 4);
  L.tile_e = take(MT * 4);
  L.exp_tile0 = take((E + 1) * 4);
  L.meta = take(16);
  L.touched = take(E * 16);
  // split-router logits (one route block)
  const bool sg = c.shared_h > 0 && c.shared_gate;
  const int ncp = route_part_cols(c.E, sg);
  L.part = take(c.T <= kRouteTokensMax ? T * static_cast<size_t>(ncp) * 4 : 0);
  L.ids = take(P * 4);
  L.gates = take(P * 4);
  L.sgate = take(T * 4);
  L.end_tables = o;
  L.act = take(P * static_cast<size_t>(c.h) * eb);
  L.act_s = take(T * hs * eb);
  L.end_act = o;
  L.y = take(P * static_cast<size_t>(c.d) * eb);
  L.ys = take(hs > 0 ? T * static_cast<size_t>(c.d) * eb : 0);
  L.end = o;
  return L;
}

// Backward workspace: the forward's routing tables (with 128-row tiles),
// then the logits and the backward's own buffers.
struct BwdLayout {
  WsLayout tables;
  size_t logits, rtok, dh, gact, dz, part, dxr, dh_s, gact_s, dz_s, part_s, dx_s, dlb, dpre, sg_part,
      rpart;
  size_t tile_e256, exp_tile0_256, meta256;  // 256-row tile table (the z product's tiles)
  size_t end;
};

BwdLayout bwd_layout(const moe_config& c) {
  BwdLayout B{};
  B.tables = ws_layout(c);
  size_t o = B.tables.end_tables;
  auto take = [&](size_t bytes) {
    const size_t at_ = o;
    o += align256(bytes);
    return at_;
  };
  const size_t T = static_cast<size_t>(c.T), P = T * static_cast<size_t>(c.top_k);
  const size_t d = static_cast<size_t>(c.d), h = static_cast<size_t>(c.h);
  const size_t hs = static_cast<size_t>(c.shared_h);
  const size_t epad = static_cast<size_t>(ceil_div(c.E, 8) * 8);
  // dG partial sums: one per 32 hidden units (a wave's share of a z tile)
  const size_t np = 2 * static_cast<size_t>(ceil_div(c.h, 64));
  const size_t nps = hs > 0 ? 2 * static_cast<size_t>(ceil_div(c.shared_h, 64)) : 0;
  B.logits = take(T * static_cast<size_t>(c.E) * 4);
  B.rtok = take(P * 4);
  B.dh = take(P * h * 2);
  B.gact = take(P * h * 2);
  B.dz = take(P * 2 * h * 2);
  B.part = take(P * np * 4);
  B.dxr = take(P * d * 2);
  B.dh_s = take(T * hs * 2);
  B.gact_s = take(T * hs * 2);
  B.dz_s = take(T * 2 * hs * 2);
  B.part_s = take(T * nps * 4);
  B.dx_s = take(hs > 0 ? T * d * 4 : 0);
  B.dlb = take(T * epad * 2);
  B.dpre = take(T * 4);
  B.sg_part = take(static_cast<size_t>(ceil_div(c.T, kSgateTokens)) * d * 4);
  B.rpart = take(static_cast<size_t>(ceil_div(c.T, kBwdRouterChunk)) * static_cast<size_t>(c.E) * d * 4);
  B.tile_e256 = take(static_cast<size_t>(max_m_tiles(c.T * c.top_k, c.E, kTileMLarge)) * 4);
  B.exp_tile0_256 = take((static_cast<size_t>(c.E) + 1) * 4);
  B.meta256 = take(16);
  B.end = o;
  return B;
}

}  // namespace moe

using namespace moe;

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: a required pointer is NULL or a size/option is out of range";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape, alignment or expert count outside what the kernels support";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing, too small or not 256-byte aligned";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    case MOE_ERR_SCRATCH_LIMIT: return "MOE_ERR_SCRATCH_LIMIT: the call needs a larger workspace than the no-alloc entry point's static array (MOE_NOALLOC_SCRATCH_BYTES)";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status moe_validate_config(const moe_config* cfg) { return check_cfg(cfg); }

size_t moe_workspace_size_entry(const moe_config* cfg, int32_t entry) {
  if (check_cfg(cfg) != MOE_OK) return 0;
  const WsLayout L = ws_layout(*cfg);
  switch (entry) {
    case MOE_ENTRY_LAYER_FORWARD: return L.end;
    case MOE_ENTRY_DISPATCH:
    case MOE_ENTRY_GATE_UP:
    case MOE_ENTRY_DOWN: return L.end_tables;
    case MOE_ENTRY_EXPERT_FFN: return L.act_s;
    case MOE_ENTRY_SHARED_EXPERT: return L.end_act;
    case MOE_ENTRY_ROUTING_STATS:
      return cfg->T > 0 ? align256(static_cast<size_t>(stats_blocks(cfg->T)) * (cfg->E + 1) * 4) : 0;
    case MOE_ENTRY_LAYER_BACKWARD: return bwd_layout(*cfg).end;
    default: return 0;
  }
}

size_t moe_workspace_size(const moe_config* cfg) {
  return moe_workspace_size_entry(cfg, MOE_ENTRY_LAYER_FORWARD);
}

size_t moe_workspace_table_offset(const moe_config* cfg, int32_t table) {
  if (check_cfg(cfg) != MOE_OK) return SIZE_MAX;
  const WsLayout L = ws_layout(*cfg);
  switch (table) {
    case MOE_TABLE_OFFSETS: return L.offsets;
    case MOE_TABLE_PERM: return L.perm;
    case MOE_TABLE_INV: return L.inv;
    default: return SIZE_MAX;
  }
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* b_router, int32_t* ids, float* gates, float* logits,
                     void* stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.T == 0) return MOE_OK;
  MOE_TRY(need(x));
  MOE_TRY(need(w_router));
  MOE_TRY(need(ids));
  MOE_TRY(need(gates));
  MOE_TRY(maybe(logits));
  if (c.has_router_bias) MOE_TRY(need(b_router));
  RouteParams p{};
  p.x = x;
  p.w_router = w_router;
  p.bias = c.has_router_bias ? b_router : nullptr;
  p.T = c.T; p.d = c.d; p.E = c.E; p.k = c.top_k; p.mode = c.mode; p.renorm = c.renormalize;
  p.rt = route_tokens(c.T);
  p.ids = ids;
  p.gates = gates;
  p.logits = logits;
  MOE_HIP(launch_route(p, c.dtype, as_stream(stream)));
  return MOE_OK;
}

moe_status moe_dispatch(const moe_config* cfg, const int32_t* ids, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                        size_t ws_bytes, void* stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.T == 0) return MOE_OK;
  MOE_TRY(need(ids));
  MOE_TRY(need(counts));
  MOE_TRY(need(offsets));
  MOE_TRY(need(perm));
  MOE_TRY(need(inv));
  MOE_TRY(check_ws(c, MOE_ENTRY_DISPATCH, ws, ws_bytes));
  const WsLayout L = ws_layout(c);
  hipStream_t s = as_stream(stream);
  const int rt = route_tokens(c.T);
  RankParams rp{ids, c.T, c.E, c.top_k, rt, at<int32_t>(ws, L.blk_hist), at<int32_t>(ws, L.lrank)};
  MOE_HIP(launch_rank(rp, s));
  const int tm = choose_tile_m(c.T * c.top_k, c.E);
  ScanParams sp{at<int32_t>(ws, L.blk_hist), ceil_div(c.T, rt), c.E, counts};
  ScatterParams xp{ids, at<int32_t>(ws, L.blk_hist), at<int32_t>(ws, L.lrank), c.T, c.E,
                   c.top_k, rt, perm, inv, counts, offsets, max_m_tiles(c.T * c.top_k, c.E, tm), tm,
                   at<int32_t>(ws, L.tile_e), at<int32_t>(ws, L.exp_tile0), at<int32_t>(ws, L.meta),
                   at<int32_t>(ws, L.touched)};
  if (dispatch_fused(sp.NB, c.E)) {
    MOE_HIP(launch_dispatch(sp, xp, s));
  } else {
    MOE_HIP(launch_scan(sp, s));
    MOE_HIP(launch_scatter(xp, s));
  }
  return MOE_OK;
}

namespace {

GemmParams gemm_base(const moe_config& c, void* ws, const int32_t* offsets, int kind) {
  const WsLayout L = ws_layout(c);
  GemmParams g{};
  g.kind = kind;
  g.dtype = c.dtype;
  g.k = c.top_k;
  g.offsets = offsets;
  g.tile_e = at<int32_t>(ws, L.tile_e);
  g.exp_tile0 = at<int32_t>(ws, L.exp_tile0);
  g.meta = at<int32_t>(ws, L.meta);
  g.touched = at<int32_t>(ws, L.touched);
  g.E = c.E;
  g.P = c.T * c.top_k;
  g.tile_m = choose_tile_m(g.P, c.E);
  g.max_mtiles = max_m_tiles(g.P, c.E, g.tile_m);
  g.a_rows = c.T;
  return g;
}

moe_status run_tiles(const moe_config& c, void* ws, const int32_t* offsets, hipStream_t s) {
  const WsLayout L = ws_layout(c);
  const int tm = choose_tile_m(c.T * c.top_k, c.E);
  TilesParams tp{offsets, c.E, c.T * c.top_k, max_m_tiles(c.T * c.top_k, c.E, tm), tm,
                 at<int32_t>(ws, L.tile_e), at<int32_t>(ws, L.exp_tile0),
                 at<int32_t>(ws, L.meta), at<int32_t>(ws, L.touched)};
  MOE_HIP(launch_tiles(tp, s));
  return MOE_OK;
}

moe_status run_gate_up(const moe_config& c, void* ws, const void* x, const int32_t* perm,
                       const int32_t* offsets, const void* wg, const void* wu, void* act,
                       hipStream_t s) {
  GemmParams g = gemm_base(c, ws, offsets, 0);
  g.a = x; g.perm = perm; g.K = c.d;
  g.b0 = wg; g.b1 = wu; g.N = c.h; g.out = act;
  MOE_HIP(use_small_gemm(c) ? launch_gemm_small(g, s) : launch_gemm(g, s));
  return MOE_OK;
}

moe_status run_down(const moe_config& c, void* ws, const void* act, const int32_t* offsets,
                    const void* wd, void* y, hipStream_t s) {
  GemmParams g = gemm_base(c, ws, offsets, 1);
  g.a = act; g.K = c.h;
  g.b0 = wd; g.N = c.d; g.out = y;
  MOE_HIP(use_small_gemm(c) ? launch_gemm_small(g, s) : launch_gemm(g, s));
  return MOE_OK;
}

}  // namespace

moe_status moe_gate_up(const moe_config* cfg, const void* x, const int32_t* perm,
                       const int32_t* offsets, const void* w_gate, const void* w_up,
                       void* act, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.expert_quant != MOE_QUANT_NONE) return MOE_ERR_UNSUPPORTED;
  if (c.T == 0) return MOE_OK;
  MOE_TRY(need(x)); MOE_TRY(need(perm)); MOE_TRY(need(offsets));
  MOE_TRY(need(w_gate)); MOE_TRY(need(w_up)); MOE_TRY(need(act));
  MOE_TRY(check_ws(c, MOE_ENTRY_GATE_UP, ws, ws_bytes));
  hipStream_t s = as_stream(stream);
  MOE_TRY(run_tiles(c, ws, offsets, s));
  return run_gate_up(c, ws, x, perm, offsets, w_gate, w_up, act, s);
}

moe_status moe_down(const moe_config* cfg, const void* act, const int32_t* offsets,
                    const void* w_down, void* y, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.expert_quant != MOE_QUANT_NONE) return MOE_ERR_UNSUPPORTED;
  if (c.T == 0) return MOE_OK;
  MOE_TRY(need(act)); MOE_TRY(need(offsets)); MOE_TRY(need(w_down)); MOE_TRY(need(y));
  MOE_TRY(check_ws(c, MOE_ENTRY_DOWN, ws, ws_bytes));
  hipStream_t s = as_stream(stream);
  MOE_TRY(run_tiles(c, ws, offsets, s));
  return run_down(c, ws, act, offsets, w_down, y, s);
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* x, const int32_t* perm,
                          const int32_t* offsets, const void* w_gate, const void* w_up,
                          const void* w_down, void* y, void* ws, size_t ws_bytes,
                          void* stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.expert_quant != MOE_QUANT_NONE) return MOE_ERR_UNSUPPORTED;
  if (c.T == 0) return MOE_OK;
  MOE_TRY(need(x)); MOE_TRY(need(perm)); MOE_TRY(need(offsets));
  MOE_TRY(need(w_gate)); MOE_TRY(need(w_up)); MOE_TRY(need(w_down)); MOE_TRY(need(y));
  MOE_TRY(check_ws(c, MOE_ENTRY_EXPERT_FFN, ws, ws_bytes));
  const WsLayout L = ws_layout(c);
  hipStream_t s = as_stream(stream);
  MOE_TRY(run_tiles(c, ws, offsets, s));
  void* act = at<void>(ws, L.act);
  MOE_TRY(run_gate_up(c, ws, x, perm, offsets, w_gate, w_up, act, s));
  return run_down(c, ws, act, offsets, w_down, y, s);
}

moe_status moe_shared_expert(const moe_config* cfg, const void* x, const void* ws_gate,
                             const void* ws_up, const void* ws_down,
                             const void* w_shared_gate, void* s_out, void* ws,
                             size_t ws_bytes, void* stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (c.shared_h <= 0) return MOE_ERR_INVALID_ARG;
  MOE_TRY(need(x)); MOE_TRY(need(ws_gate)); MOE_TRY(need(ws_up)); MOE_TRY(need(ws_down));
  MOE_TRY(maybe(w_shared_gate)); MOE_TRY(need(s_out));
  MOE_TRY(check_ws(c, MOE_ENTRY_SHARED_EXPERT, ws, ws_bytes));
  const WsLayout L = ws_layout(c);
  hipStream_t s = as_stream(stream);
  float* sg = nullptr;
  if (w_shared_gate != nullptr) {
    sg = at<float>(ws, L.sgate);
    RowDotSigmoidParams rp{x, w_shared_gate, c.T, c.d, c.dtype, sg};
    MOE_HIP(launch_rowdot_sigmoid(rp, s));
  }
  void* act_s = at<void>(ws, L.act_s);
  GemmParams g{};
  g.kind = 0; g.dtype = c.dtype; g.k = c.top_k; g.E = c.E;
  g.P = 0; g.max_mtiles = 0; g.a_rows = c.T;  // no routed rows: the shared group only
  g.tile_m = choose_tile_m(c.T, 1);
  g.shared_T = c.T; g.sa = x; g.sK = c.d; g.sb0 = ws_gate; g.sb1 = ws_up; g.sN = c.shared_h;
  g.sout = act_s;
  MOE_HIP(launch_gemm(g, s));
  GemmParams g2 = g;
  g2.kind = 1; g2.sa = act_s; g2.sK = c.shared_h; g2.sb0 = ws_down; g2.sb1 = nullptr;
  g2.sN = c.d; g2.sout = s_out;
  MOE_HIP(launch_gemm(g2, s));
  if (sg != nullptr) {
    ScaleRowsParams sp{s_out, sg, c.T, c.d, c.dtype};
    MOE_HIP(launch_scale_rows(sp, s));
  }
  return MOE_OK;
}

moe_status moe_combine(const moe_config* cfg, const void* y, const int32_t* inv,
                       const float* gates, const void* shared, void* out, void* stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.T == 0) return MOE_OK;
  MOE_TRY(need(y)); MOE_TRY(need(inv)); MOE_TRY(need(gates)); MOE_TRY(maybe(shared));
  MOE_TRY(need(out));
  CombineParams p{y, inv, gates, shared, nullptr, out, c.T, c.d, c.top_k, c.dtype, c.T * c.top_k};
  MOE_HIP(launch_combine(p, as_stream(stream)));
  return MOE_OK;
}

moe_status moe_routing_stats(const moe_config* cfg, const float* logits, const int32_t* counts,
                             float alpha, float* share, float* mean_prob, float* scalars,
                             void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.T == 0) return MOE_OK;
  MOE_TRY(need(logits)); MOE_TRY(need(counts)); MOE_TRY(need(share)); MOE_TRY(need(mean_prob));
  MOE_TRY(need(scalars));
  if (!(alpha >= 0.0f) || alpha == INFINITY) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(c, MOE_ENTRY_ROUTING_STATS, ws, ws_bytes));
  StatsParams p{logits, counts, c.T, c.E, c.top_k, c.mode, alpha, static_cast<float*>(ws),
                stats_blocks(c.T), stats_tokens_per_block(c.T), share, mean_prob, scalars};
  MOE_HIP(launch_stats(p, as_stream(stream)));
  return MOE_OK;
}

moe_status moe_layer_forward_traced(const moe_config* cfg, const moe_weights* w,
                                    const void* x, void* out, int32_t* ids, float* gates,
                                    int32_t* counts, void* ws, size_t ws_bytes,
                                    void* const* stage_events, void* stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (w == nullptr) return MOE_ERR_INVALID_ARG;
  MOE_TRY(need(x)); MOE_TRY(need(out));
  MOE_TRY(need(w->w_router)); MOE_TRY(need(w->w_gate)); MOE_TRY(need(w->w_up));
  MOE_TRY(need(w->w_down));
  if (c.has_router_bias) MOE_TRY(need(w->b_router));
  if (c.shared_h > 0) {
    MOE_TRY(need(w->ws_gate)); MOE_TRY(need(w->ws_up)); MOE_TRY(need(w->ws_down));
    if (c.shared_gate) MOE_TRY(need(w->w_shared_gate));
  }
  const bool q4 = c.expert_quant == MOE_QUANT_Q4_G64;
  if (q4) {
    if (!q4_supported(c)) return MOE_ERR_UNSUPPORTED;
    MOE_TRY(need(w->w_gate_sb)); MOE_TRY(need(w->w_up_sb)); MOE_TRY(need(w->w_down_sb));
  }
  MOE_TRY(maybe(ids)); MOE_TRY(maybe(gates)); MOE_TRY(maybe(counts));
  MOE_TRY(check_ws(c, MOE_ENTRY_LAYER_FORWARD, ws, ws_bytes));
  if (c.T == 0) return MOE_OK;

  const WsLayout L = ws_layout(c);
  hipStream_t s = as_stream(stream);
  auto mark = [&](int i) -> hipError_t {
    if (stage_events == nullptr || stage_events[i] == nullptr) return hipSuccess;
    return hipEventRecord(reinterpret_cast<hipEvent_t>(stage_events[i]), s);
  };
  const int rt = route_tokens(c.T);
  const int NB = ceil_div(c.T, rt);
  const int tm = choose_tile_m(c.T * c.top_k, c.E);
  int32_t* ids_p = ids != nullptr ? ids : at<int32_t>(ws, L.ids);
  float* gates_p = gates != nullptr ? gates : at<float>(ws, L.gates);
  int32_t* counts_p = counts != nullptr ? counts : at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* perm = at<int32_t>(ws, L.perm);
  int32_t* inv = at<int32_t>(ws, L.inv);
  const bool gated = c.shared_h > 0 && c.shared_gate;
  float* sg = gated ? at<float>(ws, L.sgate) : nullptr;

  const bool fused_route = NB == 1 && route_in_gate_up(c);
  MOE_HIP(mark(0));
  RouteParams rp{};
  rp.x = x;
  rp.w_router = w->w_router;
  rp.bias = c.has_router_bias ? w->b_router : nullptr;
  rp.w_sgate = gated ? w->w_shared_gate : nullptr;
  rp.T = c.T; rp.d = c.d; rp.E = c.E; rp.k = c.top_k; rp.mode = c.mode; rp.renorm = c.renormalize;
  rp.rt = rt;
  rp.ids = ids_p;
  rp.gates = gates_p;
  rp.logits = nullptr;
  rp.sgate = sg;
  rp.blk_hist = at<int32_t>(ws, L.blk_hist);
  rp.lrank = at<int32_t>(ws, L.lrank);
  if (NB == 1) {
    rp.counts = counts_p; rp.offsets = offsets; rp.perm = perm; rp.inv = inv;
    rp.tile_e = at<int32_t>(ws, L.tile_e); rp.exp_tile0 = at<int32_t>(ws, L.exp_tile0);
    rp.meta = at<int32_t>(ws, L.meta);
    rp.touched = at<int32_t>(ws, L.touched);
    rp.tile_m = tm;
    rp.max_tiles = max_m_tiles(c.T * c.top_k, c.E, tm);
    // the small-batch GEMMs need no tile table
    if (use_small_gemm(c)) rp.tile_e = nullptr;
    rp.part = at<float>(ws, L.part);
    rp.ncp = route_part_cols(c.E, gated);
    // the smallest batches (route_in_gate_up): the selection and the
    // dispatch tables are made inside the gate/up launch from these logits
    if (fused_route) MOE_HIP(launch_route_part(rp, c.dtype, s));
    else MOE_HIP(launch_route_split(rp, c.dtype, s));
  } else {
    MOE_HIP(launch_route(rp, c.dtype, s));
  }
  MOE_HIP(mark(1));
  if (NB > 1) {
    ScanParams sp{at<int32_t>(ws, L.blk_hist), NB, c.E, counts_p};
    ScatterParams xp{ids_p, at<int32_t>(ws, L.blk_hist), at<int32_t>(ws, L.lrank), c.T, c.E,
                     c.top_k, rt, perm, inv, counts_p, offsets, max_m_tiles(c.T * c.top_k, c.E, tm), tm,
                     at<int32_t>(ws, L.tile_e), at<int32_t>(ws, L.exp_tile0), at<int32_t>(ws, L.meta),
                     at<int32_t>(ws, L.touched)};
    if (dispatch_fused(sp.NB, c.E)) {
      MOE_HIP(launch_dispatch(sp, xp, s));
    } else {
      MOE_HIP(launch_scan(sp, s));
      MOE_HIP(launch_scatter(xp, s));
    }
  }
  MOE_HIP(mark(2));

  void* act = at<void>(ws, L.act);
  void* act_s = at<void>(ws, L.act_s);
  void* y = at<void>(ws, L.y);
  void* ys = at<void>(ws, L.ys);
  const bool small = use_small_gemm(c);
  // the shared expert alone on the tiled kernel (the small-batch kernels run
  // the routed experts only)
  auto shared_only = [&](int kind) {
    GemmParams g{};
    g.kind = kind; g.dtype = c.dtype; g.k = c.top_k; g.E = c.E;
    g.P = 0; g.max_mtiles = 0; g.a_rows = c.T;
    g.tile_m = choose_tile_m(c.T, 1);
    g.shared_T = c.T;
    if (kind == 0) {
      g.sa = x; g.sK = c.d; g.sb0 = w->ws_gate; g.sb1 = w->ws_up; g.sN = c.shared_h; g.sout = act_s;
    } else {
      g.sa = act_s; g.sK = c.shared_h; g.sb0 = w->ws_down; g.sN = c.d; g.sout = ys;
    }
    return g;
  };
  GemmParams g = gemm_base(c, ws, offsets, 0);
  g.a = x; g.perm = perm; g.K = c.d; g.b0 = w->w_gate; g.b1 = w->w_up; g.N = c.h; g.out = act;
  if (q4) { g.quant = MOE_QUANT_Q4_G64; g.b0_sb = w->w_gate_sb; g.b1_sb = w->w_up_sb; }
  if (small) {
    MOE_HIP(launch_gemm_small(g, s, fused_route ? &rp : nullptr));
    if (c.shared_h > 0) MOE_HIP(launch_gemm(shared_only(0), s));
  } else {
    if (c.shared_h > 0) {
      g.shared_T = c.T; g.sa = x; g.sK = c.d; g.sb0 = w->ws_gate; g.sb1 = w->ws_up;
      g.sN = c.shared_h; g.sout = act_s;
    }
    MOE_HIP(launch_gemm(g, s));
  }
  MOE_HIP(mark(3));
  GemmParams g2 = gemm_base(c, ws, offsets, 1);
  g2.a = act; g2.K = c.h; g2.b0 = w->w_down; g2.N = c.d; g2.out = y;
  if (q4) { g2.quant = MOE_QUANT_Q4_G64; g2.b0_sb = w->w_down_sb; }
  CombineParams cp{y, inv, gates_p, c.shared_h > 0 ? ys : nullptr, sg, out, c.T, c.d, c.top_k,
                    c.dtype, c.T * c.top_k};
  const bool fused_combine = down_combine_fused(c);
  if (fused_combine) {
    // the shared rows first: the down launch adds them
    if (c.shared_h > 0) MOE_HIP(launch_gemm(shared_only(1), s));
    MOE_HIP(launch_down_combine(g2, cp, s));
  } else if (small) {
    MOE_HIP(launch_gemm_small(g2, s));
    if (c.shared_h > 0) MOE_HIP(launch_gemm(shared_only(1), s));
  } else {
    if (c.shared_h > 0) {
      g2.shared_T = c.T; g2.sa = act_s; g2.sK = c.shared_h; g2.sb0 = w->ws_down;
      g2.sN = c.d; g2.sout = ys;
    }
    MOE_HIP(launch_gemm(g2, s));
  }
  MOE_HIP(mark(4));
  if (!fused_combine) MOE_HIP(launch_combine(cp, s));
  MOE_HIP(mark(5));
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_config* cfg, const moe_weights* w, const void* x,
                             void* out, int32_t* ids, float* gates, int32_t* counts, void* ws,
                             size_t ws_bytes, void* stream) {
  return moe_layer_forward_traced(cfg, w, x, out, ids, gates, counts, ws, ws_bytes, nullptr,
                                  stream);
}

moe_status moe_layer_backward(const moe_config* cfg, const moe_weights* w, const void* x,
                              const void* dout, const moe_grads* gr, void* ws, size_t ws_bytes,
                              void* stream) {
  return moe_layer_backward_traced(cfg, w, x, dout, gr, ws, ws_bytes, nullptr, stream);
}

moe_status moe_layer_backward_traced(const moe_config* cfg, const moe_weights* w, const void* x,
                                     const void* dout, const moe_grads* gr, void* ws,
                                     size_t ws_bytes, void* const* stage_events, void* stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.dtype != MOE_BF16 || c.expert_quant != MOE_QUANT_NONE) return MOE_ERR_UNSUPPORTED;
  if (w == nullptr || gr == nullptr) return MOE_ERR_INVALID_ARG;
  MOE_TRY(need(w->w_router)); MOE_TRY(need(w->w_gate)); MOE_TRY(need(w->w_up));
  MOE_TRY(need(w->w_down));
  if (c.has_router_bias) MOE_TRY(need(w->b_router));
  MOE_TRY(need(gr->dw_router)); MOE_TRY(need(gr->dw_gate)); MOE_TRY(need(gr->dw_up));
  MOE_TRY(need(gr->dw_down));
  const bool has_sh = c.shared_h > 0;
  const bool gated = has_sh && c.shared_gate;
  if (has_sh) {
    MOE_TRY(need(w->ws_gate)); MOE_TRY(need(w->ws_up)); MOE_TRY(need(w->ws_down));
    MOE_TRY(need(gr->dws_gate)); MOE_TRY(need(gr->dws_up)); MOE_TRY(need(gr->dws_down));
    if (gated) { MOE_TRY(need(w->w_shared_gate)); MOE_TRY(need(gr->dw_shared_gate)); }
  }
  if (c.T > 0) { MOE_TRY(need(x)); MOE_TRY(need(dout)); MOE_TRY(need(gr->dx)); }
  MOE_TRY(maybe(gr->dgates)); MOE_TRY(maybe(gr->dlogits));
  MOE_TRY(check_ws(c, MOE_ENTRY_LAYER_BACKWARD, ws, ws_bytes));

  hipStream_t s = as_stream(stream);
  auto mark = [&](int i) -> hipError_t {
    if (stage_events == nullptr || stage_events[i] == nullptr) return hipSuccess;
    return hipEventRecord(reinterpret_cast<hipEvent_t>(stage_events[i]), s);
  };
  const BwdLayout B = bwd_layout(c);
  const WsLayout& L = B.tables;
  if (c.T == 0) {
    // no token: every weight gradient is zero
    const size_t E = static_cast<size_t>(c.E), d = static_cast<size_t>(c.d);
    const size_t h = static_cast<size_t>(c.h), hs = static_cast<size_t>(c.shared_h);
    MOE_HIP(launch_fill_zero(gr->dw_router, E * d, s));
    MOE_HIP(launch_fill_zero(gr->dw_gate, E * h * d, s));
    MOE_HIP(launch_fill_zero(gr->dw_up, E * h * d, s));
    MOE_HIP(launch_fill_zero(gr->dw_down, E * d * h, s));
    if (has_sh) {
      MOE_HIP(launch_fill_zero(gr->dws_gate, hs * d, s));
      MOE_HIP(launch_fill_zero(gr->dws_up, hs * d, s));
      MOE_HIP(launch_fill_zero(gr->dws_down, d * hs, s));
      if (gated) MOE_HIP(launch_fill_zero(gr->dw_shared_gate, d, s));
    }
    return MOE_OK;
  }
  const int rt = route_tokens(c.T);
  const int NB = ceil_div(c.T, rt);
  const int tm = kTileM;
  const int P = c.T * c.top_k;
  int32_t* ids = at<int32_t>(ws, L.ids);
  float* gates = at<float>(ws, L.gates);
  int32_t* counts = at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* perm = at<int32_t>(ws, L.perm);
  int32_t* inv = at<int32_t>(ws, L.inv);
  float* sg = gated ? at<float>(ws, L.sgate) : nullptr;
  float* logits = at<float>(ws, B.logits);

  MOE_HIP(mark(0));
  RouteParams rp{};
  rp.x = x;
  rp.w_router = w->w_router;
  rp.bias = c.has_router_bias ? w->b_router : nullptr;
  rp.w_sgate = gated ? w->w_shared_gate : nullptr;
  rp.T = c.T; rp.d = c.d; rp.E = c.E; rp.k = c.top_k; rp.mode = c.mode; rp.renorm = c.renormalize;
  rp.rt = rt;
  rp.ids = ids;
  rp.gates = gates;
  rp.logits = logits;
  rp.sgate = sg;
  rp.blk_hist = at<int32_t>(ws, L.blk_hist);
  rp.lrank = at<int32_t>(ws, L.lrank);
  if (NB == 1) {
    rp.counts = counts; rp.offsets = offsets; rp.perm = perm; rp.inv = inv;
    rp.tile_e = at<int32_t>(ws, L.tile_e); rp.exp_tile0 = at<int32_t>(ws, L.exp_tile0);
    rp.meta = at<int32_t>(ws, L.meta);
    rp.touched = at<int32_t>(ws, L.touched);
    rp.tile_m = tm;
    rp.max_tiles = max_m_tiles(P, c.E, tm);
    rp.part = at<float>(ws, L.part);
    rp.ncp = route_part_cols(c.E, gated);
    MOE_HIP(launch_route_split(rp, c.dtype, s));
  } else {
    MOE_HIP(launch_route(rp, c.dtype, s));
    ScanParams sp{at<int32_t>(ws, L.blk_hist), NB, c.E, counts};
    ScatterParams xp{ids, at<int32_t>(ws, L.blk_hist), at<int32_t>(ws, L.lrank), c.T, c.E,
                     c.top_k, rt, perm, inv, counts, offsets, max_m_tiles(P, c.E, tm), tm,
                     at<int32_t>(ws, L.tile_e), at<int32_t>(ws, L.exp_tile0), at<int32_t>(ws, L.meta),
                     at<int32_t>(ws, L.touched)};
    if (dispatch_fused(sp.NB, c.E)) {
      MOE_HIP(launch_dispatch(sp, xp, s));
    } else {
      MOE_HIP(launch_scan(sp, s));
      MOE_HIP(launch_scatter(xp, s));
    }
  }

  BwdParams bp{};
  bp.T = c.T; bp.d = c.d; bp.E = c.E; bp.Epad = ceil_div(c.E, 8) * 8; bp.h = c.h;
  bp.hs = c.shared_h; bp.k = c.top_k; bp.mode = c.mode; bp.renorm = c.renormalize;
  bp.max_mtiles = max_m_tiles(P, c.E, tm);
  bp.meta = at<int32_t>(ws, L.meta); bp.tile_e = at<int32_t>(ws, L.tile_e);
  bp.exp_tile0 = at<int32_t>(ws, L.exp_tile0); bp.offsets = offsets; bp.perm = perm;
  bp.inv = inv; bp.ids = ids; bp.gates = gates; bp.logits = logits; bp.sgate = sg;
  bp.x = static_cast<const uint16_t*>(x);
  bp.dout = static_cast<const uint16_t*>(dout);
  bp.w_router = static_cast<const uint16_t*>(w->w_router);
  bp.w_gate = static_cast<const uint16_t*>(w->w_gate);
  bp.w_up = static_cast<const uint16_t*>(w->w_up);
  bp.w_down = static_cast<const uint16_t*>(w->w_down);
  if (has_sh) {
    bp.ws_gate = static_cast<const uint16_t*>(w->ws_gate);
    bp.ws_up = static_cast<const uint16_t*>(w->ws_up);
    bp.ws_down = static_cast<const uint16_t*>(w->ws_down);
    bp.dh_s = at<uint16_t>(ws, B.dh_s); bp.gact_s = at<uint16_t>(ws, B.gact_s);
    bp.dz_s = at<uint16_t>(ws, B.dz_s); bp.part_s = at<float>(ws, B.part_s);
    bp.dx_s = at<float>(ws, B.dx_s);
    bp.dws_gate = gr->dws_gate; bp.dws_up = gr->dws_up; bp.dws_down = gr->dws_down;
    if (gated) {
      bp.w_shared_gate = static_cast<const uint16_t*>(w->w_shared_gate);
      bp.dpre = at<float>(ws, B.dpre);
      bp.sg_part = at<float>(ws, B.sg_part);
      bp.dw_shared_gate = gr->dw_shared_gate;
    }
  }
  bp.rtok = at<int>(ws, B.rtok);
  bp.dh = at<uint16_t>(ws, B.dh); bp.gact = at<uint16_t>(ws, B.gact); bp.dz = at<uint16_t>(ws, B.dz);
  bp.part = at<float>(ws, B.part); bp.dxr = at<uint16_t>(ws, B.dxr);
  bp.dlb = at<uint16_t>(ws, B.dlb);
  bp.rpart = at<float>(ws, B.rpart);
  bp.dx = gr->dx; bp.dw_router = gr->dw_router; bp.dw_gate = gr->dw_gate; bp.dw_up = gr->dw_up;
  bp.dw_down = gr->dw_down; bp.dgates = gr->dgates; bp.dlogits = gr->dlogits;
  // at least 256 rows per expert on average: the gate/up product (z) and
  // the dx rows run on the forward's 256-row tiles, from a 256-row tile
  // table of the same dispatch, routed and shared rows in one launch each
  GemmParams zg{}, xg{}, wgu{}, wdn{};
  if (choose_tile_m(P, c.E) == kTileMLarge) {
    TilesParams tp{offsets, c.E, P, max_m_tiles(P, c.E, kTileMLarge), kTileMLarge,
                   at<int32_t>(ws, B.tile_e256), at<int32_t>(ws, B.exp_tile0_256),
                   at<int32_t>(ws, B.meta256), nullptr};
    MOE_HIP(launch_tiles(tp, s));
    zg.kind = 2; zg.dtype = c.dtype;
    zg.a = x; zg.perm = perm; zg.k = c.top_k; zg.K = c.d;
    zg.b0 = w->w_gate; zg.b1 = w->w_up; zg.N = c.h;
    zg.offsets = offsets; zg.tile_e = at<int32_t>(ws, B.tile_e256);
    zg.exp_tile0 = at<int32_t>(ws, B.exp_tile0_256); zg.meta = at<int32_t>(ws, B.meta256);
    zg.E = c.E; zg.P = P; zg.max_mtiles = max_m_tiles(P, c.E, kTileMLarge);
    zg.tile_m = kTileMLarge; zg.a_rows = c.T;
    if (has_sh) {
      zg.shared_T = c.T; zg.sa = x; zg.sK = c.d; zg.sb0 = w->ws_gate; zg.sb1 = w->ws_up;
      zg.sN = c.shared_h;
    }
    zg.zdh = bp.dh; zg.zdh_s = bp.dh_s; zg.zgates = gates; zg.zsgate = sg;
    zg.zga = bp.gact; zg.zga_s = bp.gact_s; zg.zdz = bp.dz; zg.zdz_s = bp.dz_s;
    zg.zpart = bp.part; zg.zpart_s = bp.part_s;
    zg.znpart = 2 * ceil_div(c.h, 64);
    zg.znpart_s = has_sh ? 2 * ceil_div(c.shared_h, 64) : 0;
    bp.zg = &zg;
    // dx rows = dz [W_g; W_u] (K = 2h), float32 in pair order
    xg.kind = 3; xg.dtype = c.dtype;
    xg.a = bp.dz; xg.perm = perm; xg.k = c.top_k; xg.K = 2 * c.h;
    xg.b0 = w->w_gate; xg.b1 = w->w_up; xg.N = c.d; xg.out = bp.dxr;
    xg.offsets = offsets; xg.tile_e = zg.tile_e; xg.exp_tile0 = zg.exp_tile0; xg.meta = zg.meta;
    xg.E = c.E; xg.P = P; xg.max_mtiles = zg.max_mtiles;
    xg.tile_m = kTileMLarge; xg.a_rows = c.T;
    if (has_sh) {
      xg.shared_T = c.T; xg.sa = bp.dz_s; xg.sK = 2 * c.shared_h; xg.sb0 = w->ws_gate;
      xg.sb1 = w->ws_up; xg.sN = c.d; xg.sout = bp.dx_s;
    }
    bp.xg = &xg;
    // the weight gradients on 256 x 256 tiles: dW_g|u = dz^T x, dW_d = dO^T (g a)
    wgu.kind = 4; wgu.dtype = c.dtype; wgu.perm = perm; wgu.k = c.top_k; wgu.offsets = offsets;
    wgu.E = c.E; wgu.P = P; wgu.a_rows = c.T; wgu.tile_m = kTileMLarge; wgu.rtok = bp.rtok;
    wdn = wgu;
    wdn.kind = 5;
    wgu.a = bp.dz; wgu.b0 = x; wgu.M = 2 * c.h; wgu.N = c.d;
    wgu.out = gr->dw_gate; wgu.out2 = gr->dw_up;
    wdn.a = dout; wdn.b0 = bp.gact; wdn.M = c.d; wdn.N = c.h; wdn.out = gr->dw_down;
    if (has_sh) {
      wgu.shared_T = c.T; wgu.sa = bp.dz_s; wgu.sb0 = x; wgu.sM = 2 * c.shared_h; wgu.sN = c.d;
      wgu.sout = gr->dws_gate; wgu.sout2 = gr->dws_up;
      wdn.shared_T = c.T; wdn.sa = dout; wdn.sb0 = bp.gact_s; wdn.sM = c.d; wdn.sN = c.shared_h;
      wdn.sout = gr->dws_down;
    }
    // measured: faster at 512-546 rows per expert on average (shared_routed
    // dW_gate|up 1288 -> 1096 us, small_moe_sigmoid 184 -> 134), slower at the
    // skewed prefill shape's 1024 (1175 -> 1317: the 128 x 128 tiles, four
    // workgroups per CU, balance its uneven experts better)
    if (static_cast<long long>(P) < 768LL * c.E) {
      bp.wgu = &wgu;
      bp.wdn = &wdn;
    }
  }
  MOE_HIP(mark(1));
  MOE_HIP(launch_backward(bp, s, stage_events != nullptr ? stage_events + 1 : nullptr));
  return MOE_OK;
}

}  // extern "C"
