// C-ABI host layer: argument checks, capacity, workspace layout and the
// launch sequence of every entry point declared in include/moe.h.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "moe.h"
#include "moe_internal.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int esize(const moe_config* c) { return c->dtype == MOE_BF16 ? 2 : 4; }

moe_status check_config(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->num_tokens < 0 || c->num_tokens >= (int64_t(1) << 30)) return MOE_ERR_INVALID_ARG;
  if (c->hidden_size <= 0) return MOE_ERR_INVALID_ARG;
  if (c->num_experts < 1 || c->num_experts > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
  if (c->k != 1 && c->k != 2) return MOE_ERR_INVALID_ARG;
  if (c->k > c->num_experts) return MOE_ERR_INVALID_ARG;
  if (c->drop_tokens != 0 && c->drop_tokens != 1) return MOE_ERR_INVALID_ARG;
  if (c->drop_tokens && !(c->capacity_factor > 0.0 && isfinite(c->capacity_factor))) return MOE_ERR_INVALID_ARG;
  if (c->min_capacity < 0) return MOE_ERR_INVALID_ARG;
  if (c->ffn_hidden < 0) return MOE_ERR_INVALID_ARG;
  if (c->activation < MOE_ACT_NONE || c->activation > MOE_ACT_GELU) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->normalize_topk != 0 && c->normalize_topk != 1) return MOE_ERR_INVALID_ARG;
  if (c->loss_kind != MOE_LOSS_BALANCE && c->loss_kind != MOE_LOSS_USAGE_STD) return MOE_ERR_INVALID_ARG;
  if (c->save_preact != 0 && c->save_preact != 1) return MOE_ERR_INVALID_ARG;
  // kernels move rows as 16-byte vectors
  const int vec = c->dtype == MOE_BF16 ? 8 : 4;
  if (c->hidden_size % vec) return MOE_ERR_UNSUPPORTED;
  if (c->ffn_hidden % vec) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int64_t capacity_of(const moe_config* c) {
  if (!c->drop_tokens) return -1;
  // max(min_capacity, ceil((k*T/E) * capacity_factor)) in IEEE double, this order
  const double per_expert = (double)((int64_t)c->k * c->num_tokens) / (double)c->num_experts;
  const double cap = ceil(per_expert * c->capacity_factor);
  int64_t C = cap >= 4.0e18 ? (int64_t)4000000000000000000LL : (int64_t)cap;
  if (C < c->min_capacity) C = c->min_capacity;
  return C;
}

int64_t max_rows_of(const moe_config* c) {
  const int64_t kt = (int64_t)c->k * c->num_tokens;
  const int64_t C = capacity_of(c);
  if (C < 0 || C >= kt) return kt;
  const int64_t ec = C * c->num_experts;
  return ec < kt ? ec : kt;
}

struct Layout {
  int64_t T, C, rows;
  int tiles, tile_tokens;
  size_t tile_cnt, me_tile, me_sum, demand, idx, slot, weight, offset;
  size_t x_disp, a_save, h_disp, y_disp, d_act;
  size_t total;
};

Layout layout_of(const moe_config* c) {
  Layout L;
  L.T = c->num_tokens;
  L.C = capacity_of(c);
  L.rows = max_rows_of(c);
  const int E = c->num_experts, k = c->k, d = c->hidden_size, h = c->ffn_hidden;
  const int tt = gate_tile_tokens(E);
  L.tile_tokens = tt;
  L.tiles = (int)((L.T + tt - 1) / tt);
  const size_t s = (size_t)esize(c);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  L.tile_cnt = take((size_t)L.tiles * k * E * 4);
  L.me_tile = take((size_t)L.tiles * E * 4);
  L.me_sum = take((size_t)E * 8);
  L.demand = take((size_t)2 * E * 4);
  L.idx = take((size_t)L.T * k * 4);
  L.slot = take((size_t)L.T * k * 4);
  L.weight = take((size_t)L.T * k * 4);
  L.offset = take((size_t)(E + 1) * 4);
  L.x_disp = take((size_t)L.rows * d * s);
  L.a_save = take((c->save_preact && h > 0) ? (size_t)L.rows * h * s : 0);
  L.h_disp = take(h > 0 ? (size_t)L.rows * h * s : 0);
  L.y_disp = take((size_t)L.rows * d * s);
  L.d_act = take(h > 0 ? (size_t)L.rows * h * s : 0);
  L.total = off;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<unsigned char*>(ws) + off);
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY_HIP(expr)                        \
  do {                                           \
    hipError_t _e = (expr);                      \
    if (_e != hipSuccess) return MOE_ERR_HIP;    \
  } while (0)

moe_status run_gate(const moe_config* c, const Layout& L, const void* x, const void* w_router,
                    const float* b_router, const float* logits_in, float* logits_out, int32_t* expert_idx,
                    int32_t* slot, float* weight, int32_t* expert_count, int32_t* expert_offset,
                    float* gate_loss, void* ws, hipStream_t s) {
  if (L.T == 0) return hip_status(launch_gate_empty(expert_count, expert_offset, gate_loss, c->num_experts, s));
  GateArgs a;
  a.x = x;
  a.w_router = w_router;
  a.b_router = b_router;
  a.logits_in = logits_in;
  a.logits_out = logits_out;
  a.expert_idx = expert_idx;
  a.slot = slot;
  a.weight = weight;
  a.expert_count = expert_count;
  a.expert_offset = expert_offset;
  a.gate_loss = gate_loss;
  a.tile_cnt = at<int32_t>(ws, L.tile_cnt);
  a.me_tile = at<float>(ws, L.me_tile);
  a.me_sum = at<double>(ws, L.me_sum);
  a.demand = at<int32_t>(ws, L.demand);
  a.T = L.T;
  a.C = L.C;
  a.d = c->hidden_size;
  a.E = c->num_experts;
  a.k = c->k;
  a.normalize = c->normalize_topk;
  a.loss_kind = c->loss_kind;
  a.num_tiles = L.tiles;
  MOE_TRY_HIP(launch_gate(a, c->dtype, s));
  MOE_TRY_HIP(launch_slot_finalize(a, L.tile_tokens, s));
  return MOE_OK;
}

moe_status run_ffn(const moe_config* c, const Layout& L, const void* x_disp, const int32_t* offset,
                   const void* w1, const void* b1, const void* w2, const void* b2, void* a_save,
                   void* h_disp, void* y_disp, hipStream_t s) {
  const int d = c->hidden_size, h = c->ffn_hidden;
  GemmArgs g;
  g.offset = offset;
  g.max_rows = L.rows;
  g.E = c->num_experts;
  if (h > 0) {
    g.X = x_disp;
    g.W = w1;
    g.bias = b1;
    g.Y = h_disp;
    g.Apre = a_save;
    g.N = h;
    g.K = d;
    g.act = c->activation;
    MOE_TRY_HIP(launch_grouped_gemm(g, c->dtype, s));
    g.X = h_disp;
    g.W = w2;
    g.bias = b2;
    g.Y = y_disp;
    g.Apre = nullptr;
    g.N = d;
    g.K = h;
    g.act = ACT_NONE;
    MOE_TRY_HIP(launch_grouped_gemm(g, c->dtype, s));
  } else {
    g.X = x_disp;
    g.W = w1;
    g.bias = b1;
    g.Y = y_disp;
    g.Apre = nullptr;
    g.N = d;
    g.K = d;
    g.act = c->activation;
    MOE_TRY_HIP(launch_grouped_gemm(g, c->dtype, s));
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: configuration not supported by the kernels";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime or launch error";
  }
  return "unknown moe_status";
}

moe_status moe_capacity(const moe_config* cfg, int64_t* C) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!C) return MOE_ERR_INVALID_ARG;
  *C = capacity_of(cfg);
  return MOE_OK;
}

moe_status moe_max_rows(const moe_config* cfg, int64_t* rows) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!rows) return MOE_ERR_INVALID_ARG;
  *rows = max_rows_of(cfg);
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = layout_of(cfg).total;
  return MOE_OK;
}

moe_status moe_workspace_views(const moe_config* cfg, void* ws, void** x_disp, void** a_save, void** h_disp,
                               void** y_disp, int32_t** expert_offset) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!ws) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg);
  if (x_disp) *x_disp = at<void>(ws, L.x_disp);
  if (a_save) *a_save = (cfg->save_preact && cfg->ffn_hidden > 0) ? at<void>(ws, L.a_save) : nullptr;
  if (h_disp) *h_disp = cfg->ffn_hidden > 0 ? at<void>(ws, L.h_disp) : nullptr;
  if (y_disp) *y_disp = at<void>(ws, L.y_disp);
  if (expert_offset) *expert_offset = at<int32_t>(ws, L.offset);
  return MOE_OK;
}

moe_status moe_gate(const moe_config* cfg, const void* x, const void* w_router, const float* b_router,
                    const float* logits_in, float* logits_out, int32_t* expert_idx, int32_t* slot,
                    float* weight, int32_t* expert_count, int32_t* expert_offset, float* gate_loss, void* ws,
                    size_t ws_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  // per-token arrays may be NULL only when there are no tokens
  const bool tok = cfg->num_tokens > 0;
  if (tok && !logits_in && (!x || !w_router)) return MOE_ERR_INVALID_ARG;
  if (tok && (!expert_idx || !slot || !weight)) return MOE_ERR_INVALID_ARG;
  if (!expert_count || !expert_offset || !gate_loss || !ws) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return run_gate(cfg, L, x, w_router, b_router, logits_in, logits_out, expert_idx, slot, weight, expert_count,
                  expert_offset, gate_loss, ws, static_cast<hipStream_t>(stream));
}

moe_status moe_dispatch(const moe_config* cfg, const void* x, const int32_t* expert_idx, const int32_t* slot,
                        const int32_t* expert_offset, void* x_disp, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!x || !expert_idx || !slot || !expert_offset || !x_disp) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_dispatch(x, expert_idx, slot, expert_offset, x_disp, cfg->num_tokens, cfg->k,
                                    cfg->hidden_size * esize(cfg), static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* x_disp, const int32_t* expert_offset, const void* w1,
                          const void* b1, const void* w2, const void* b2, void* a_save, void* h_disp,
                          void* y_disp, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!x_disp || !expert_offset || !w1 || !y_disp) return MOE_ERR_INVALID_ARG;
  if (cfg->ffn_hidden > 0 && (!w2 || !h_disp)) return MOE_ERR_INVALID_ARG;
  if (cfg->ffn_hidden == 0 && w2) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg);
  return run_ffn(cfg, L, x_disp, expert_offset, w1, b1, w2, b2, cfg->ffn_hidden > 0 ? a_save : nullptr, h_disp,
                 y_disp, static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn_backward(const moe_config* cfg, const void* x_disp, const int32_t* expert_offset,
                                   const void* w1, const void* w2, const void* a_save, const void* h_disp,
                                   const void* dy_disp, void* dx_disp, void* dw1, float* db1, void* dw2,
                                   float* db2, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->ffn_hidden <= 0) return MOE_ERR_INVALID_ARG;
  if (!x_disp || !expert_offset || !w1 || !w2 || !a_save || !h_disp || !dy_disp || !dx_disp || !dw1 || !dw2 ||
      !ws)
    return MOE_ERR_INVALID_ARG;
  // the backward kernels are bf16 only and write 16-element row segments
  if (cfg->dtype != MOE_BF16 || cfg->hidden_size % 16 || cfg->ffn_hidden % 16) return MOE_ERR_UNSUPPORTED;
  const Layout L = layout_of(cfg);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  GemmBwdArgs b;
  b.X = x_disp;
  b.W1 = w1;
  b.W2 = w2;
  b.A = a_save;
  b.H = h_disp;
  b.dY = dy_disp;
  b.dA = at<void>(ws, L.d_act);
  b.dX = dx_disp;
  b.dW1 = dw1;
  b.dW2 = dw2;
  b.db1 = db1;
  b.db2 = db2;
  b.offset = expert_offset;
  b.max_rows = L.rows;
  b.E = cfg->num_experts;
  b.d = cfg->hidden_size;
  b.h = cfg->ffn_hidden;
  b.act = cfg->activation;
  return hip_status(launch_ffn_backward(b, cfg->dtype, static_cast<hipStream_t>(stream)));
}

moe_status moe_combine(const moe_config* cfg, const void* y_disp, const int32_t* expert_idx, const int32_t* slot,
                       const float* weight, const int32_t* expert_offset, void* out, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!y_disp || !expert_idx || !slot || !weight || !expert_offset || !out) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(y_disp, expert_idx, slot, weight, expert_offset, out, cfg->num_tokens, cfg->k,
                                   cfg->hidden_size, cfg->dtype, static_cast<hipStream_t>(stream)));
}

moe_status moe_layer_forward(const moe_config* cfg, const void* x, const void* w_router, const float* b_router,
                             const float* logits_in, const void* w1, const void* b1, const void* w2, const void* b2,
                             void* out, float* gate_loss, int32_t* expert_count, float* logits_out,
                             int32_t* expert_idx, int32_t* slot, float* weight, void* ws, size_t ws_bytes,
                             void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const bool tok = cfg->num_tokens > 0;
  if (tok && (!x || !out || (!logits_in && !w_router))) return MOE_ERR_INVALID_ARG;
  if (!w1 || !gate_loss || !expert_count || !ws) return MOE_ERR_INVALID_ARG;
  if (cfg->ffn_hidden > 0 && !w2) return MOE_ERR_INVALID_ARG;
  if (cfg->ffn_hidden == 0 && w2) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* idx = expert_idx ? expert_idx : at<int32_t>(ws, L.idx);
  int32_t* sl = slot ? slot : at<int32_t>(ws, L.slot);
  float* wt = weight ? weight : at<float>(ws, L.weight);
  int32_t* off = at<int32_t>(ws, L.offset);
  st = run_gate(cfg, L, x, w_router, b_router, logits_in, logits_out, idx, sl, wt, expert_count, off, gate_loss, ws,
                s);
  if (st != MOE_OK || L.T == 0) return st;
  void* xd = at<void>(ws, L.x_disp);
  void* hd = cfg->ffn_hidden > 0 ? at<void>(ws, L.h_disp) : nullptr;
  void* as = (cfg->save_preact && cfg->ffn_hidden > 0) ? at<void>(ws, L.a_save) : nullptr;
  void* yd = at<void>(ws, L.y_disp);
  MOE_TRY_HIP(launch_dispatch(x, idx, sl, off, xd, L.T, cfg->k, cfg->hidden_size * esize(cfg), s));
  st = run_ffn(cfg, L, xd, off, w1, b1, w2, b2, as, hd, yd, s);
  if (st != MOE_OK) return st;
  MOE_TRY_HIP(launch_combine(yd, idx, sl, wt, off, out, L.T, cfg->k, cfg->hidden_size, cfg->dtype, s));
  return MOE_OK;
}

}  // extern "C"
