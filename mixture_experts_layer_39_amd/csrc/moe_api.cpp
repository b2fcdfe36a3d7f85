// C-ABI host layer: argument checks, capacity, workspace layout and the
// launch sequence of every entry point declared in include/moe.h.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int esize(const moe_config* c) { return c->dtype == MOE_BF16 ? 2 : 4; }

static_assert(kDecodeMaxTokens == MOE_SMALL_BATCH_MAX, "small-batch token limit");

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
  if (c->small_batch < -1 || c->small_batch > 1) return MOE_ERR_INVALID_ARG;
  // the random gate options: RSample and RTS are k = 1 options, second-expert
  // sampling a k = 2 one (as in the gate the options come from)
  if (c->noisy_gate_policy < MOE_NOISE_NONE || c->noisy_gate_policy > MOE_NOISE_RSAMPLE) return MOE_ERR_INVALID_ARG;
  if (c->use_rts != 0 && c->use_rts != 1) return MOE_ERR_INVALID_ARG;
  if (c->second_expert_sampling != 0 && c->second_expert_sampling != 1) return MOE_ERR_INVALID_ARG;
  if (c->noisy_gate_policy == MOE_NOISE_RSAMPLE && c->k != 1) return MOE_ERR_INVALID_ARG;
  if (c->use_rts && c->k != 1) return MOE_ERR_INVALID_ARG;
  if (c->second_expert_sampling && c->k != 2) return MOE_ERR_INVALID_ARG;
  if (c->noisy_gate_policy == MOE_NOISE_JITTER && c->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (c->use_residual != 0 && c->use_residual != 1) return MOE_ERR_INVALID_ARG;
  if (c->use_residual && c->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (c->packed_weights != 0 && c->packed_weights != 1) return MOE_ERR_INVALID_ARG;
  if (c->packed_weights) {
    // only the large-tile GEMM (and the one-launch small-batch kernel) read
    // the packed layout: bf16, both expert Linears on that path
    const int d = c->hidden_size, h = c->ffn_hidden;
    const bool big = h > 0 ? grouped_gemm_is_big(d, h, c->dtype) && grouped_gemm_is_big(h, d, c->dtype)
                           : grouped_gemm_is_big(d, d, c->dtype);
    if (c->dtype != MOE_BF16 || !big) return MOE_ERR_UNSUPPORTED;
  }
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
  size_t tile_cnt, me_tile, me_sum, demand, gate_sync, gate_end, idx, slot, weight, offset;
  size_t x_disp, a_save, h_disp, y_disp, d_act;
  size_t row_tok;   // inference forward: token of each packed row (the first Linear gathers x through it)
  int64_t h_ld;   // row pitch (elements) of h_disp in the layer forward
  size_t dec_logits, dec_prob, dec_part, dec_bar;   // small-batch forward: logits, probabilities, partial logits, barrier
  // backward regions (save_preact == 1 only)
  int Ep;
  RouterChunks rc;
  size_t logits, dwg, dlg, dl_hl, wfrag, top1, coef, dbpart, choff, wpart, xj;
  size_t r_off, r_a, r_h, r_y, r_coef, r_dact, r_dx, r_dlc, r_cwpart, r_cbpart;   // residual MoE
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
  L.gate_sync = take(4);
  L.gate_end = off;   // the gate's own scratch ends here (moe_gate_noalloc)
  L.idx = take((size_t)L.T * k * 4);
  L.slot = take((size_t)L.T * k * 4);
  L.weight = take((size_t)L.T * k * 4);
  L.offset = take((size_t)(E + 1) * 4);
  L.x_disp = take((size_t)L.rows * d * s);
  L.row_tok = take((size_t)L.rows * 4);
  L.a_save = take((c->save_preact && h > 0) ? (size_t)L.rows * h * s : 0);
  // Without save_preact nothing outside the forward reads h_disp, and the
  // second Linear reads it faster with an odd number of 128-byte lines per
  // row: with an even number the rows of a K step crowd into fewer memory
  // channels (measured at h = 5120: 7.6% off that GEMM).
  L.h_ld = h;
  if (!c->save_preact && h > 0 && grouped_gemm_is_big(d, h, c->dtype) && grouped_gemm_is_big(h, d, c->dtype) &&
      ((int64_t)h * 2 / 128) % 2 == 0)
    L.h_ld = h + 64;
  L.h_disp = take(h > 0 ? (size_t)L.rows * L.h_ld * s : 0);
  L.y_disp = take((size_t)L.rows * d * s);
  L.d_act = take(h > 0 ? (size_t)L.rows * h * s : 0);
  L.dec_logits = take(L.T <= kDecodeMaxTokens ? (size_t)L.T * E * 4 : 0);
  L.dec_prob = take(L.T <= kDecodeMaxTokens ? (size_t)L.T * E * 4 : 0);
  L.dec_part = take(L.T <= kDecodeMaxTokens ? (size_t)kDecodeMaxSlices * L.T * E * 4 : 0);
  L.dec_bar = take(L.T <= kDecodeMaxTokens ? 4096 : 0);
  const bool train = c->save_preact != 0;
  L.Ep = router_ep(E);
  L.rc = train ? router_chunks(L.T, d, E) : RouterChunks{0, 0};
  const size_t nbt = (size_t)((L.T + kGateBwdTokens - 1) / kGateBwdTokens);
  L.logits = take(train ? (size_t)L.T * E * 4 : 0);
  L.dwg = take(train ? (size_t)L.T * k * 4 : 0);
  L.dlg = take(train ? (size_t)L.T * E * 4 : 0);
  L.dl_hl = take(train ? (size_t)L.T * 2 * L.Ep * 2 : 0);
  L.wfrag = take(train ? (size_t)d * L.Ep * 2 : 0);
  L.top1 = take(train ? (size_t)kTop1Parts * E * 4 : 0);
  L.coef = take(train ? (size_t)E * 4 : 0);
  L.dbpart = take(train ? nbt * E * 4 : 0);
  L.choff = take(train ? (size_t)(kRouterMaxChunks + 1) * 4 : 0);
  L.wpart = take(train ? (size_t)L.rc.S * 2 * L.Ep * d * 4 : 0);
  // the router's jittered input, rebuilt for its weight gradient
  L.xj = take(train && c->noisy_gate_policy == MOE_NOISE_JITTER ? (size_t)L.T * d * 2 : 0);
  // the residual MoE's dense branch (one "expert" of all T rows), its
  // coefficients, and for training its backward buffers
  const bool res = c->use_residual != 0;
  const int64_t nch = residual_coef_chunks(L.T);
  L.r_off = take(res ? 8 : 0);
  L.r_a = take(res && train && h > 0 ? (size_t)L.T * h * s : 0);
  L.r_h = take(res && h > 0 ? (size_t)L.T * h * s : 0);
  L.r_y = take(res ? (size_t)L.T * d * s : 0);
  L.r_coef = take(res ? (size_t)L.T * 2 * 4 : 0);
  L.r_dact = take(res && train && h > 0 ? (size_t)L.T * h * s : 0);
  L.r_dx = take(res && train ? (size_t)L.T * d * s : 0);
  L.r_dlc = take(res && train ? (size_t)L.T * 2 * 4 : 0);
  L.r_cwpart = take(res && train ? (size_t)nch * 2 * d * 4 : 0);
  L.r_cbpart = take(res && train ? (size_t)nch * 2 * 4 : 0);
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

// The gate.  With defer (set only when no Random Token Selection follows),
// the slot fix-up is left to the caller's dispatch (launch_dispatch_finalize
// with *args): slot then holds the in-tile ranks until that dispatch runs.
moe_status run_gate(const moe_config* c, const Layout& L, const void* x, const void* w_router,
                    const float* b_router, const float* logits_in, float* logits_out, int32_t* expert_idx,
                    int32_t* slot, float* weight, int32_t* expert_count, int32_t* expert_offset,
                    float* gate_loss, void* ws, hipStream_t s, GateArgs* defer = nullptr) {
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
  a.sync = at<uint32_t>(ws, L.gate_sync);
  a.T = L.T;
  a.C = L.C;
  a.d = c->hidden_size;
  a.E = c->num_experts;
  a.k = c->k;
  a.normalize = c->normalize_topk;
  a.loss_kind = c->loss_kind;
  const bool rnd = c->noisy_gate_policy != MOE_NOISE_NONE || c->second_expert_sampling;
  a.tile_tokens = gate_tile_tokens_for(c->num_experts, c->hidden_size, c->dtype, logits_in != nullptr, rnd);
  a.num_tiles = (int32_t)((L.T + a.tile_tokens - 1) / a.tile_tokens);   // <= L.tiles (64-token tiles)
  a.jitter = c->noisy_gate_policy == MOE_NOISE_JITTER;
  a.rsample = c->noisy_gate_policy == MOE_NOISE_RSAMPLE;
  a.second = c->second_expert_sampling;
  a.seed_lo = (uint32_t)(c->seed & 0xffffffffu);
  a.seed_hi = (uint32_t)(c->seed >> 32);
  // jitter acts on the router's input: there is none when the logits are given
  if (a.jitter && logits_in) return MOE_ERR_INVALID_ARG;
  MOE_TRY_HIP(launch_gate(a, c->dtype, s));
  const bool rts = c->use_rts && L.C >= 0;
  if (defer && !rts) {
    *defer = a;
    return MOE_OK;
  }
  if (defer) defer->T = -1;   // slots are final: a plain dispatch follows
  MOE_TRY_HIP(launch_slot_finalize(a, s));
  if (rts) MOE_TRY_HIP(launch_rts_select(a, s));
  return MOE_OK;
}

// Row tile height for the forward Linears of a layer.  Every row tile
// streams its expert's whole weight tile, so an expert with a few rows more
// than a multiple of 256 pays for a nearly empty tile.  320-row tiles (a
// fifth 32-row block per token-side wave, the row offsets of the loads in
// scalar registers to make room for its accumulators) put up to 640 rows in
// two tiles; they cost more per tile, and they pay off where the largest
// expert (the capacity when tokens are dropped, else the mean) needs fewer
// row tiles with them and at most three: with more tiles per expert the
// weights come back from the L2 in groups of row tiles anyway.
int forward_tile_rows(const moe_config* c, const Layout& L) {
  const int64_t E = c->num_experts, kt = L.T * c->k;
  const int64_t m = L.C >= 0 ? std::min(L.C, kt) : (kt + E - 1) / E;
  const int64_t t5 = (m + 319) / 320, t4 = (m + 255) / 256;
  return (m > 0 && t5 < t4 && t5 <= 3) ? 320 : 256;
}

// h_ld: row pitch of h_disp (and a_save) in elements.  row_tok non-null:
// x_disp is the token matrix [T, d] itself and the first Linear reads packed
// row r from its row row_tok[r].
moe_status run_ffn(const moe_config* c, const Layout& L, const void* x_disp, const int32_t* offset,
                   const void* w1, const void* b1, const void* w2, const void* b2, void* a_save,
                   void* h_disp, void* y_disp, int64_t h_ld, hipStream_t s, const int32_t* row_tok = nullptr) {
  const int d = c->hidden_size, h = c->ffn_hidden;
  GemmArgs g;
  g.offset = offset;
  g.max_rows = L.rows;
  g.E = c->num_experts;
  g.w_packed = c->packed_weights;
  g.x_map = row_tok;
  g.x_rows = L.T;
  g.tile_rows = forward_tile_rows(c, L);
  if (h > 0) {
    g.X = x_disp;
    g.W = w1;
    g.bias = b1;
    g.Y = h_disp;
    g.Apre = a_save;
    g.N = h;
    g.K = d;
    g.act = c->activation;
    g.y_ld = h_ld;
    MOE_TRY_HIP(launch_grouped_gemm(g, c->dtype, s));
    g.x_map = nullptr;
    g.X = h_disp;
    g.W = w2;
    g.bias = b2;
    g.Y = y_disp;
    g.Apre = nullptr;
    g.N = d;
    g.K = h;
    g.act = ACT_NONE;
    g.x_ld = h_ld;
    g.y_ld = 0;
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

// Gate, dispatch and the expert FFNs of the multi-kernel forward (y_disp in
// ws); the caller combines.
moe_status forward_experts(const moe_config* cfg, const Layout& L, const void* x, const void* w_router,
                           const float* b_router, const float* logits_in, const void* w1, const void* b1,
                           const void* w2, const void* b2, float* gate_loss, int32_t* expert_count,
                           float* logits_out, int32_t* idx, int32_t* sl, float* wt, int32_t* off, void* ws,
                           hipStream_t s) {
  // training: the backward needs the logits, so keep them when the caller does not
  float* lg = (logits_out || !cfg->save_preact) ? logits_out : at<float>(ws, L.logits);
  GateArgs ga;
  moe_status st =
      run_gate(cfg, L, x, w_router, b_router, logits_in, lg, idx, sl, wt, expert_count, off, gate_loss, ws, s, &ga);
  if (st != MOE_OK || L.T == 0) return st;
  void* xd = at<void>(ws, L.x_disp);
  void* hd = cfg->ffn_hidden > 0 ? at<void>(ws, L.h_disp) : nullptr;
  void* as = (cfg->save_preact && cfg->ffn_hidden > 0) ? at<void>(ws, L.a_save) : nullptr;
  void* yd = at<void>(ws, L.y_disp);
  // Inference on the large-tile GEMM: no dispatched copy of x; a row map
  // (4 bytes per packed row) tells the first Linear which token row each
  // packed row is, and it loads that row of x directly.  The gathering form
  // runs 256-row tiles; where the layer's Linears take 320-row tiles the
  // copy stays (the taller tiles gain more than the copy costs).  Training
  // keeps the copy, which the backward reads.
  const int d = cfg->hidden_size, n1 = cfg->ffn_hidden > 0 ? cfg->ffn_hidden : d;
  if (!cfg->save_preact && grouped_gemm_is_big(d, n1, cfg->dtype) && L.T * d * 2 < (int64_t(1) << 31) &&
      forward_tile_rows(cfg, L) == 256) {
    int32_t* rt = at<int32_t>(ws, L.row_tok);
    if (ga.T >= 0)
      MOE_TRY_HIP(launch_row_map_finalize(ga, rt, s));
    else
      MOE_TRY_HIP(launch_row_map(idx, sl, off, rt, L.T, cfg->k, s));
    return run_ffn(cfg, L, x, off, w1, b1, w2, b2, as, hd, yd, L.h_ld, s, rt);
  }
  if (ga.T >= 0)
    MOE_TRY_HIP(launch_dispatch_finalize(x, ga, xd, d * esize(cfg), s));
  else
    MOE_TRY_HIP(launch_dispatch(x, idx, sl, off, xd, L.T, cfg->k, d * esize(cfg), s));
  return run_ffn(cfg, L, xd, off, w1, b1, w2, b2, as, hd, yd, L.h_ld, s);
}

moe_status check_gate_args(const moe_config* cfg, const void* x, const void* w_router, const float* logits_in,
                           const int32_t* expert_idx, const int32_t* slot, const float* weight,
                           const int32_t* expert_count, const int32_t* expert_offset, const float* gate_loss) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  // per-token arrays may be NULL only when there are no tokens
  const bool tok = cfg->num_tokens > 0;
  if (tok && !logits_in && (!x || !w_router)) return MOE_ERR_INVALID_ARG;
  if (tok && (!expert_idx || !slot || !weight)) return MOE_ERR_INVALID_ARG;
  if (!expert_count || !expert_offset || !gate_loss) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// ---------------------------------------------------------------- library-owned gate scratch
// moe_gate_noalloc keeps the gate's per-tile counts, per-tile probability
// sums, their totals and the demand (the first regions of the workspace
// layout, which every gate kernel writes before it reads them, so nothing
// needs clearing) in this array instead of a caller workspace.  Each device
// holds its own copy for the life of the process.  In host code the name is
// a host-side stand-in, never a device address: the kernels get the address
// that hipGetSymbolAddress returns for the current device.
constexpr size_t kGateScratchBytes = (size_t)MOE_GATE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kGateScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up on the
// first call made with that device current and kept for later calls.
hipError_t gate_scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
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

moe_status moe_packed_weight_bytes(int32_t num_experts, int64_t n, int64_t k, int32_t dtype, size_t* bytes) {
  if (!bytes || num_experts < 1 || num_experts > MOE_MAX_EXPERTS || n <= 0 || k <= 0) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ERR_INVALID_ARG;
  if (n >= (int64_t(1) << 31) || k >= (int64_t(1) << 31)) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 || !grouped_gemm_is_big(k, n, dtype)) return MOE_ERR_UNSUPPORTED;
  *bytes = (size_t)num_experts * (size_t)((n + 255) / 256 * 256) * (size_t)k * 2;
  return MOE_OK;
}

moe_status moe_pack_expert_weight(int32_t num_experts, int64_t n, int64_t k, int32_t dtype, const void* w,
                                  void* w_packed, void* stream) {
  size_t bytes = 0;
  const moe_status st = moe_packed_weight_bytes(num_experts, n, k, dtype, &bytes);
  if (st != MOE_OK) return st;
  if (!w || !w_packed) return MOE_ERR_INVALID_ARG;
  // the kernel reads and writes 16-byte chunks
  if (reinterpret_cast<uintptr_t>(w) % 16 || reinterpret_cast<uintptr_t>(w_packed) % 16) return MOE_ERR_INVALID_ARG;
  const char* a = static_cast<const char*>(w);
  const char* b = static_cast<const char*>(w_packed);
  const size_t in_bytes = (size_t)num_experts * (size_t)n * (size_t)k * 2;
  if (a < b + bytes && b < a + in_bytes) return MOE_ERR_INVALID_ARG;   // overlap
  MOE_TRY_HIP(launch_pack_expert_weight(w, w_packed, num_experts, n, k, static_cast<hipStream_t>(stream)));
  return MOE_OK;
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

moe_status moe_workspace_h_ld(const moe_config* cfg, int64_t* h_ld) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!h_ld) return MOE_ERR_INVALID_ARG;
  *h_ld = cfg->ffn_hidden > 0 ? layout_of(cfg).h_ld : 0;
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

moe_status moe_workspace_status(const moe_config* cfg, void* ws, uint32_t** status) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!ws || !status) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg);
  *status = cfg->num_tokens <= kDecodeMaxTokens ? at<uint32_t>(ws, L.dec_bar) + kDecodeStatusWord : nullptr;
  return MOE_OK;
}

moe_status moe_gate(const moe_config* cfg, const void* x, const void* w_router, const float* b_router,
                    const float* logits_in, float* logits_out, int32_t* expert_idx, int32_t* slot,
                    float* weight, int32_t* expert_count, int32_t* expert_offset, float* gate_loss, void* ws,
                    size_t ws_bytes, void* stream) {
  moe_status st = check_gate_args(cfg, x, w_router, logits_in, expert_idx, slot, weight, expert_count,
                                  expert_offset, gate_loss);
  if (st != MOE_OK) return st;
  if (!ws) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return run_gate(cfg, L, x, w_router, b_router, logits_in, logits_out, expert_idx, slot, weight, expert_count,
                  expert_offset, gate_loss, ws, static_cast<hipStream_t>(stream));
}

moe_status moe_gate_noalloc(const moe_config* cfg, const void* x, const void* w_router, const float* b_router,
                            const float* logits_in, float* logits_out, int32_t* expert_idx, int32_t* slot,
                            float* weight, int32_t* expert_count, int32_t* expert_offset, float* gate_loss,
                            void* stream) {
  moe_status st = check_gate_args(cfg, x, w_router, logits_in, expert_idx, slot, weight, expert_count,
                                  expert_offset, gate_loss);
  if (st != MOE_OK) return st;
  const Layout L = layout_of(cfg);
  if (L.gate_end > kGateScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (gate_scratch_of_current_device(&ws) != hipSuccess) return MOE_ERR_HIP;
  // run_gate reads and writes only the gate's regions, [0, L.gate_end)
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
                          const void* b1, const void* w2, const void* b2, void* a_save, void* h_disp, int64_t h_ld,
                          void* y_disp, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!x_disp || !expert_offset || !w1 || !y_disp) return MOE_ERR_INVALID_ARG;
  if (cfg->ffn_hidden > 0 && (!w2 || !h_disp)) return MOE_ERR_INVALID_ARG;
  if (cfg->ffn_hidden == 0 && w2) return MOE_ERR_INVALID_ARG;
  const int64_t h = cfg->ffn_hidden, d = cfg->hidden_size;
  if (h_ld == 0) h_ld = h;
  if (h_ld != h && !(h > 0 && h_ld == h + 64)) return MOE_ERR_INVALID_ARG;
  if (h_ld != h && !(grouped_gemm_is_big(d, h, cfg->dtype) && grouped_gemm_is_big(h, d, cfg->dtype)))
    return MOE_ERR_UNSUPPORTED;
  const Layout L = layout_of(cfg);
  return run_ffn(cfg, L, x_disp, expert_offset, w1, b1, w2, b2, h > 0 ? a_save : nullptr, h_disp, y_disp, h_ld,
                 static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn_backward(const moe_config* cfg, const void* x_disp, const int32_t* expert_offset,
                                   const void* w1, const void* w2, const void* a_save, const void* h_disp,
                                   const void* dy_disp, void* dx_disp, void* dw1, float* db1, void* dw2,
                                   float* db2, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->ffn_hidden <= 0 || cfg->packed_weights) return MOE_ERR_INVALID_ARG;   // the backward reads nn.Linear weights
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
  if (cfg->use_residual) return MOE_ERR_INVALID_ARG;   // moe_residual_layer_forward takes the dense branch
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
  // a few tokens, inference: the whole forward in one persistent launch
  const bool small = cfg->small_batch > 0 || (cfg->small_batch == 0 && L.T <= MOE_SMALL_BATCH_AUTO);
  const bool random_gate = cfg->noisy_gate_policy != MOE_NOISE_NONE || cfg->use_rts || cfg->second_expert_sampling;
  if (small && !cfg->save_preact && !random_gate &&
      decode_fits(L.T, cfg->hidden_size, cfg->ffn_hidden, cfg->num_experts, cfg->k, cfg->dtype)) {
    DecodeArgs da{};
    da.x = static_cast<const bf16*>(x);
    da.w_router = static_cast<const bf16*>(w_router);
    da.b_router = b_router;
    da.logits_in = logits_in;
    da.logits = logits_out ? logits_out : at<float>(ws, L.dec_logits);
    da.w1 = static_cast<const bf16*>(w1);
    da.b1 = static_cast<const bf16*>(b1);
    da.w2 = static_cast<const bf16*>(w2);
    da.w_packed = cfg->packed_weights;
    da.b2 = static_cast<const bf16*>(b2);
    da.out = static_cast<bf16*>(out);
    da.gate_loss = gate_loss;
    da.expert_count = expert_count;
    da.expert_offset = off;
    da.expert_idx = idx;
    da.slot = sl;
    da.weight = wt;
    da.x_disp = at<bf16>(ws, L.x_disp);
    da.h_disp = cfg->ffn_hidden > 0 ? at<bf16>(ws, L.h_disp) : nullptr;
    da.y_disp = at<bf16>(ws, L.y_disp);
    da.prob = at<float>(ws, L.dec_prob);
    da.part = at<float>(ws, L.dec_part);
    da.bar = at<unsigned>(ws, L.dec_bar);
    da.C = L.C;
    da.T = (int32_t)L.T;
    da.d = cfg->hidden_size;
    da.h = cfg->ffn_hidden;
    da.E = cfg->num_experts;
    da.k = cfg->k;
    da.normalize = cfg->normalize_topk;
    da.loss_kind = cfg->loss_kind;
    da.act = cfg->activation;
    const hipError_t e = launch_decode(da, s);
    if (e == hipSuccess) return MOE_OK;
    // a device where the grid would not be resident takes the multi-kernel path
    if (e != hipErrorNotSupported) return MOE_ERR_HIP;
    (void)hipGetLastError();
  }
  st = forward_experts(cfg, L, x, w_router, b_router, logits_in, w1, b1, w2, b2, gate_loss, expert_count,
                       logits_out, idx, sl, wt, off, ws, s);
  if (st != MOE_OK || L.T == 0) return st;
  MOE_TRY_HIP(launch_combine(at<void>(ws, L.y_disp), idx, sl, wt, off, out, L.T, cfg->k, cfg->hidden_size,
                             cfg->dtype, s));
  return MOE_OK;
}

moe_status moe_combine_backward(const moe_config* cfg, const void* dout, const void* y_disp,
                                const int32_t* expert_idx, const int32_t* slot, const float* weight,
                                const int32_t* expert_offset, void* dy_disp, float* dweight, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!dout || !y_disp || !expert_idx || !slot || !weight || !expert_offset || !dy_disp || !dweight)
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine_backward(dout, y_disp, expert_idx, slot, weight, expert_offset, dy_disp, dweight,
                                            cfg->num_tokens, cfg->k, cfg->hidden_size, cfg->dtype,
                                            static_cast<hipStream_t>(stream)));
}

namespace {

// The logit gradient from the gate-weight gradient (and dloss for BALANCE);
// optionally also its hi/lo split and column partial sums in the workspace.
moe_status run_gate_backward(const moe_config* c, const Layout& L, const float* logits, const int32_t* idx,
                             const float* dw, const float* dloss, float* dlogits, bool split, void* ws,
                             hipStream_t s) {
  GateBwdArgs g{};
  g.logits = logits;
  g.idx = idx;
  g.dw = dw;
  g.coef = nullptr;
  if (c->loss_kind == MOE_LOSS_BALANCE && dloss) {
    MOE_TRY_HIP(launch_top1_coef(idx, c->k, L.T, c->num_experts, dloss, at<int32_t>(ws, L.top1),
                                 at<float>(ws, L.coef), s));
    g.coef = at<float>(ws, L.coef);
  }
  g.dlogits = dlogits;
  g.dl_hl = split ? at<uint16_t>(ws, L.dl_hl) : nullptr;
  g.dbpart = split ? at<float>(ws, L.dbpart) : nullptr;
  g.T = L.T;
  g.E = c->num_experts;
  g.k = c->k;
  g.Ep = L.Ep;
  g.normalize = c->normalize_topk;
  MOE_TRY_HIP(launch_gate_backward(g, s));
  return MOE_OK;
}

// The hi/lo split and column partial sums of a given logit gradient.
moe_status run_split(const moe_config* c, const Layout& L, const float* dlogits, void* ws, hipStream_t s) {
  GateBwdArgs g{};
  g.dlogits = const_cast<float*>(dlogits);   // read only without logits
  g.dl_hl = at<uint16_t>(ws, L.dl_hl);
  g.dbpart = at<float>(ws, L.dbpart);
  g.T = L.T;
  g.E = c->num_experts;
  g.k = c->k;
  g.Ep = L.Ep;
  MOE_TRY_HIP(launch_gate_backward(g, s));
  return MOE_OK;
}

moe_status run_input_grad(const moe_config* c, const Layout& L, const void* dx_disp, const int32_t* idx,
                          const int32_t* slot, const int32_t* offset, const void* w_router, void* dx, void* ws,
                          hipStream_t s, const void* dx_add = nullptr, const float* dlc = nullptr,
                          const void* coef_w = nullptr) {
  InputGradArgs g{};
  g.dx_add = static_cast<const bf16*>(dx_add);
  g.dlc = dlc;
  g.coef_w = static_cast<const bf16*>(coef_w);
  g.dx_disp = static_cast<const bf16*>(dx_disp);
  g.idx = idx;
  g.slot = slot;
  g.offset = offset;
  g.dl_hl = w_router ? at<uint16_t>(ws, L.dl_hl) : nullptr;
  g.wfrag = at<uint16_t>(ws, L.wfrag);
  g.dx = static_cast<bf16*>(dx);
  g.T = L.T;
  g.d = c->hidden_size;
  g.k = c->k;
  g.Ep = L.Ep;
  g.jitter = c->noisy_gate_policy == MOE_NOISE_JITTER;
  g.seed_lo = (uint32_t)(c->seed & 0xffffffffu);
  g.seed_hi = (uint32_t)(c->seed >> 32);
  if (w_router)
    MOE_TRY_HIP(launch_router_pack(w_router, at<uint16_t>(ws, L.wfrag), c->num_experts, c->hidden_size, L.Ep, s));
  MOE_TRY_HIP(launch_input_grad(g, s));
  return MOE_OK;
}

moe_status run_router_wgrad(const moe_config* c, const Layout& L, const void* x, float* dw_router, float* db_router,
                            void* ws, hipStream_t s) {
  RouterWgradArgs r{};
  r.x = x;
  if (c->noisy_gate_policy == MOE_NOISE_JITTER) {
    // dW_r = dlogits^T x_j: the input the router read
    bf16* xj = at<bf16>(ws, L.xj);
    MOE_TRY_HIP(launch_jitter_input(static_cast<const bf16*>(x), xj, L.T, c->hidden_size,
                                    (uint32_t)(c->seed & 0xffffffffu), (uint32_t)(c->seed >> 32), s));
    r.x = xj;
  }
  r.dl_hl = at<uint16_t>(ws, L.dl_hl);
  r.dbpart = at<float>(ws, L.dbpart);
  r.choff = at<int32_t>(ws, L.choff);
  r.part = at<float>(ws, L.wpart);
  r.dw_router = dw_router;
  r.db_router = db_router;
  r.T = L.T;
  r.d = c->hidden_size;
  r.E = c->num_experts;
  r.Ep = L.Ep;
  const hipError_t e = launch_router_wgrad(r, s);
  if (e == hipErrorNotSupported) return MOE_ERR_UNSUPPORTED;
  return hip_status(e);
}

// Shapes the router and dispatch backward kernels take: bf16, d a multiple
// of 32 (64 for the router weight gradient), the backward workspace regions.
moe_status check_backward(const moe_config* c, bool router_weights) {
  if (!c->save_preact || c->packed_weights) return MOE_ERR_INVALID_ARG;   // nn.Linear weights only
  if (c->dtype != MOE_BF16 || c->hidden_size % 32) return MOE_ERR_UNSUPPORTED;
  if (router_weights && c->hidden_size % 64) return MOE_ERR_UNSUPPORTED;
  const Layout L = layout_of(c);
  if (router_weights && L.rc.S > kRouterMaxChunks) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The layer backward after the combine's backward (dY_disp in ws's y_disp,
// gate-weight gradient in ws): expert FFNs, gate, dispatch with the router
// input term (plus the residual layer's extra terms), router weights.
moe_status backward_experts(const moe_config* cfg, const Layout& L, const void* x, const void* w_router,
                            const void* w1, const void* w2, const float* lg, const int32_t* idx, const int32_t* sl,
                            const float* wt, const int32_t* off, const float* dloss, void* dx, float* dl,
                            float* dw_router, float* db_router, void* dw1, float* db1, void* dw2, float* db2,
                            void* ws, hipStream_t s, const void* dx_add = nullptr, const float* dlc = nullptr,
                            const void* coef_w = nullptr) {
  (void)wt;
  const bool tok = L.T > 0;
  void* yd = at<void>(ws, L.y_disp);
  moe_status st;
  // expert FFNs: dX_disp over dY_disp
  GemmBwdArgs b;
  b.X = at<void>(ws, L.x_disp);
  b.W1 = w1;
  b.W2 = w2;
  b.A = at<void>(ws, L.a_save);
  b.H = at<void>(ws, L.h_disp);
  b.dY = yd;
  b.dA = at<void>(ws, L.d_act);
  b.dX = yd;
  b.dW1 = dw1;
  b.dW2 = dw2;
  b.db1 = db1;
  b.db2 = db2;
  b.offset = off;
  b.max_rows = L.T > 0 ? L.rows : 0;
  b.E = cfg->num_experts;
  b.d = cfg->hidden_size;
  b.h = cfg->ffn_hidden;
  b.act = cfg->activation;
  MOE_TRY_HIP(launch_ffn_backward(b, cfg->dtype, s));
  if (!tok) return run_router_wgrad(cfg, L, x, dw_router, db_router, ws, s);
  // gate: logit gradient (and its split for the router products)
  st = run_gate_backward(cfg, L, lg, idx, at<float>(ws, L.dwg), dloss, dl, w_router != nullptr, ws, s);
  if (st != MOE_OK) return st;
  // dispatch backward plus the router input gradient
  st = run_input_grad(cfg, L, yd, idx, sl, off, w_router, dx, ws, s, dx_add, dlc, coef_w);
  if (st != MOE_OK) return st;
  if (dw_router || db_router) return run_router_wgrad(cfg, L, x, dw_router, db_router, ws, s);
  return MOE_OK;
}

}  // namespace

moe_status moe_gate_backward(const moe_config* cfg, const float* logits, const int32_t* expert_idx,
                             const float* dweight, const float* dloss, float* dlogits, void* ws, size_t ws_bytes,
                             void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!cfg->save_preact || !ws) return MOE_ERR_INVALID_ARG;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!logits || !expert_idx || !dweight || !dlogits) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return run_gate_backward(cfg, L, logits, expert_idx, dweight, dloss, dlogits, false, ws,
                           static_cast<hipStream_t>(stream));
}

moe_status moe_dispatch_backward(const moe_config* cfg, const void* dx_disp, const int32_t* expert_idx,
                                 const int32_t* slot, const int32_t* expert_offset, const void* w_router,
                                 const float* dlogits, void* dx, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!ws) return MOE_ERR_INVALID_ARG;
  if ((st = check_backward(cfg, false)) != MOE_OK) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!dx_disp || !expert_idx || !slot || !expert_offset || !dx || (w_router && !dlogits)) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w_router && (st = run_split(cfg, L, dlogits, ws, s)) != MOE_OK) return st;
  return run_input_grad(cfg, L, dx_disp, expert_idx, slot, expert_offset, w_router, dx, ws, s);
}

moe_status moe_router_backward(const moe_config* cfg, const void* x, const float* dlogits, float* dw_router,
                               float* db_router, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!ws || (!dw_router && !db_router)) return MOE_ERR_INVALID_ARG;
  if ((st = check_backward(cfg, dw_router != nullptr)) != MOE_OK) return st;
  const bool tok = cfg->num_tokens > 0;
  if (tok && (!dlogits || (dw_router && !x))) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (tok && (st = run_split(cfg, L, dlogits, ws, s)) != MOE_OK) return st;
  return run_router_wgrad(cfg, L, x, dw_router, db_router, ws, s);
}

moe_status moe_layer_backward(const moe_config* cfg, const void* x, const void* w_router, const void* w1,
                              const void* w2, const float* logits, const int32_t* expert_idx, const int32_t* slot,
                              const float* weight, const void* dout, const float* dloss, void* dx, float* dlogits,
                              float* dw_router, float* db_router, void* dw1, float* db1, void* dw2, float* db2,
                              void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->use_residual) return MOE_ERR_INVALID_ARG;   // moe_residual_layer_backward
  if (cfg->ffn_hidden <= 0 || !ws || !w1 || !w2 || !dw1 || !dw2) return MOE_ERR_INVALID_ARG;
  if (!w_router && (dw_router || db_router)) return MOE_ERR_INVALID_ARG;
  const bool router_w = w_router && dw_router;
  if ((st = check_backward(cfg, router_w)) != MOE_OK) return st;
  if (cfg->ffn_hidden % 16) return MOE_ERR_UNSUPPORTED;
  const bool tok = cfg->num_tokens > 0;
  if (tok && (!dout || !dx || (!w_router && !dlogits) || (router_w && !x))) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t* idx = expert_idx ? expert_idx : at<int32_t>(ws, L.idx);
  const int32_t* sl = slot ? slot : at<int32_t>(ws, L.slot);
  const float* wt = weight ? weight : at<float>(ws, L.weight);
  const float* lg = logits ? logits : at<float>(ws, L.logits);
  float* dl = dlogits ? dlogits : at<float>(ws, L.dlg);
  const int32_t* off = at<int32_t>(ws, L.offset);
  void* yd = at<void>(ws, L.y_disp);   // y_disp, then dY_disp, then dX_disp

  // combine backward: dY_disp over y_disp, gate-weight gradient
  MOE_TRY_HIP(launch_combine_backward(dout, yd, idx, sl, wt, off, yd, at<float>(ws, L.dwg), L.T, cfg->k,
                                      cfg->hidden_size, cfg->dtype, s));
  return backward_experts(cfg, L, x, w_router, w1, w2, lg, idx, sl, wt, off, dloss, dx, dl, dw_router, db_router,
                          dw1, db1, dw2, db2, ws, s);
}


moe_status moe_residual_layer_forward(const moe_config* cfg, const void* x, const void* w_router,
                                      const float* b_router, const float* logits_in, const void* w1,
                                      const void* b1, const void* w2, const void* b2, const void* mlp_w1,
                                      const void* mlp_b1, const void* mlp_w2, const void* mlp_b2,
                                      const void* coef_w, const float* coef_b, void* out, float* gate_loss,
                                      int32_t* expert_count, float* coef_out, float* logits_out,
                                      int32_t* expert_idx, int32_t* slot, float* weight, void* ws,
                                      size_t ws_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!cfg->use_residual) return MOE_ERR_INVALID_ARG;
  const int d = cfg->hidden_size, h = cfg->ffn_hidden;
  const bool tok = cfg->num_tokens > 0;
  if (tok && (!x || !out || (!logits_in && !w_router))) return MOE_ERR_INVALID_ARG;
  if (!w1 || !mlp_w1 || !gate_loss || !expert_count || !ws) return MOE_ERR_INVALID_ARG;
  if ((h > 0) != (w2 != nullptr) || (h > 0) != (mlp_w2 != nullptr)) return MOE_ERR_INVALID_ARG;
  if (coef_b && !coef_w) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* idx = expert_idx ? expert_idx : at<int32_t>(ws, L.idx);
  int32_t* sl = slot ? slot : at<int32_t>(ws, L.slot);
  float* wt = weight ? weight : at<float>(ws, L.weight);
  int32_t* off = at<int32_t>(ws, L.offset);
  // the MoE branch: gate, dispatch, experts (the combine is fused below)
  st = forward_experts(cfg, L, x, w_router, b_router, logits_in, w1, b1, w2, b2, gate_loss, expert_count,
                       logits_out, idx, sl, wt, off, ws, s);
  if (st != MOE_OK || L.T == 0) return st;
  // the dense branch: the grouped GEMM with one "expert" holding all T rows
  int32_t* roff = at<int32_t>(ws, L.r_off);
  MOE_TRY_HIP(launch_residual_offsets(roff, L.T, s));
  GemmArgs g;
  g.offset = roff;
  g.max_rows = L.T;
  g.E = 1;
  g.X = x;
  g.W = mlp_w1;
  g.bias = mlp_b1;
  if (h > 0) {
    g.Y = at<void>(ws, L.r_h);
    g.Apre = cfg->save_preact ? at<void>(ws, L.r_a) : nullptr;
    g.N = h;
    g.K = d;
    g.act = cfg->activation;
    MOE_TRY_HIP(launch_grouped_gemm(g, cfg->dtype, s));
    g.X = at<void>(ws, L.r_h);
    g.W = mlp_w2;
    g.bias = mlp_b2;
    g.Y = at<void>(ws, L.r_y);
    g.Apre = nullptr;
    g.N = d;
    g.K = h;
    g.act = ACT_NONE;
  } else {
    g.Y = at<void>(ws, L.r_y);
    g.Apre = nullptr;
    g.N = d;
    g.K = d;
    g.act = cfg->activation;
  }
  MOE_TRY_HIP(launch_grouped_gemm(g, cfg->dtype, s));
  // the coefficients and the mix, with the combine of the MoE branch
  ResidualArgs r{};
  r.x = static_cast<const bf16*>(x);
  r.coef_w = static_cast<const bf16*>(coef_w);
  r.coef_b = coef_b;
  r.y_disp = at<bf16>(ws, L.y_disp);
  r.mlp_y = at<bf16>(ws, L.r_y);
  r.expert_idx = idx;
  r.slot = sl;
  r.weight = wt;
  r.offset = off;
  r.out = static_cast<bf16*>(out);
  r.coef = at<float>(ws, L.r_coef);
  r.T = L.T;
  r.d = d;
  r.k = cfg->k;
  r.coef_out = coef_out;
  MOE_TRY_HIP(launch_residual_combine(r, s));
  return MOE_OK;
}

moe_status moe_residual_layer_backward(const moe_config* cfg, const void* x, const void* w_router,
                                       const void* w1, const void* w2, const void* mlp_w1,
                                       const void* mlp_w2, const void* coef_w, const float* logits,
                                       const int32_t* expert_idx, const int32_t* slot, const float* weight,
                                       const void* dout, const float* dloss, void* dx, float* dlogits,
                                       float* dw_router, float* db_router, void* dw1, float* db1, void* dw2,
                                       float* db2, void* mlp_dw1, float* mlp_db1, void* mlp_dw2,
                                       float* mlp_db2, float* dcoef_w, float* dcoef_b, void* ws,
                                       size_t ws_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!cfg->use_residual) return MOE_ERR_INVALID_ARG;
  if (cfg->ffn_hidden <= 0 || !ws || !w1 || !w2 || !dw1 || !dw2) return MOE_ERR_INVALID_ARG;
  if (!mlp_w1 || !mlp_w2 || !mlp_dw1 || !mlp_dw2) return MOE_ERR_INVALID_ARG;
  if (!w_router && (dw_router || db_router)) return MOE_ERR_INVALID_ARG;
  if (!coef_w && (dcoef_w || dcoef_b)) return MOE_ERR_INVALID_ARG;
  const bool router_w = w_router && dw_router;
  if ((st = check_backward(cfg, router_w)) != MOE_OK) return st;
  if (cfg->ffn_hidden % 16) return MOE_ERR_UNSUPPORTED;
  const bool tok = cfg->num_tokens > 0;
  if (tok && (!x || !dout || !dx || (!w_router && !dlogits))) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t* idx = expert_idx ? expert_idx : at<int32_t>(ws, L.idx);
  const int32_t* sl = slot ? slot : at<int32_t>(ws, L.slot);
  const float* wt = weight ? weight : at<float>(ws, L.weight);
  const float* lg = logits ? logits : at<float>(ws, L.logits);
  float* dl = dlogits ? dlogits : at<float>(ws, L.dlg);
  const int32_t* off = at<int32_t>(ws, L.offset);
  // the mix's backward: dY_disp over y_disp, the MLP's upstream over its
  // output, the gate-weight and coefficient-logit gradients
  ResidualArgs r{};
  r.x = static_cast<const bf16*>(x);
  r.coef_w = static_cast<const bf16*>(coef_w);
  r.y_disp = at<bf16>(ws, L.y_disp);
  r.mlp_y = at<bf16>(ws, L.r_y);
  r.expert_idx = idx;
  r.slot = sl;
  r.weight = wt;
  r.offset = off;
  r.coef = at<float>(ws, L.r_coef);
  r.dout = static_cast<const bf16*>(dout);
  r.dw = at<float>(ws, L.dwg);
  r.dlc = coef_w ? at<float>(ws, L.r_dlc) : nullptr;
  r.cw_part = at<float>(ws, L.r_cwpart);
  r.cb_part = at<float>(ws, L.r_cbpart);
  r.dcoef_w = dcoef_w;
  r.dcoef_b = dcoef_b;
  r.T = L.T;
  r.d = cfg->hidden_size;
  r.k = cfg->k;
  MOE_TRY_HIP(launch_residual_combine_backward(r, s));
  // the dense branch's backward (one expert of all T rows); its input
  // gradient is added to dx below
  GemmBwdArgs b;
  b.X = x;
  b.W1 = mlp_w1;
  b.W2 = mlp_w2;
  b.A = at<void>(ws, L.r_a);
  b.H = at<void>(ws, L.r_h);
  b.dY = at<void>(ws, L.r_y);
  b.dA = at<void>(ws, L.r_dact);
  b.dX = at<void>(ws, L.r_dx);
  b.dW1 = mlp_dw1;
  b.dW2 = mlp_dw2;
  b.db1 = mlp_db1;
  b.db2 = mlp_db2;
  b.offset = at<int32_t>(ws, L.r_off);
  b.max_rows = L.T;
  b.E = 1;
  b.d = cfg->hidden_size;
  b.h = cfg->ffn_hidden;
  b.act = cfg->activation;
  MOE_TRY_HIP(launch_ffn_backward(b, cfg->dtype, s));   // no tokens: zero weight gradients
  // the MoE branch and dx with the dense branch's and the coefficients' terms
  st = backward_experts(cfg, L, x, w_router, w1, w2, lg, idx, sl, wt, off, dloss, dx, dl, dw_router, db_router, dw1,
                        db1, dw2, db2, ws, s, at<void>(ws, L.r_dx), r.dlc, coef_w);
  if (st != MOE_OK) return st;
  if (coef_w && (dcoef_w || dcoef_b)) MOE_TRY_HIP(launch_coef_wgrad(r, s));
  return MOE_OK;
}
}  // extern "C"
