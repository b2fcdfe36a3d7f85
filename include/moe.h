/*
 * moe.h - C ABI of a top-k gated Mixture-of-Experts layer for one MI355X
 * (gfx950) GPU: gate, dispatch, expert FFNs, combine, the fused layer
 * forward, and the backward of every step and of the whole layer.
 *
 * What the calls compute follows these pages (cited by title and section):
 *   [ds.moe]     "deepspeed.moe 模块" overview (adg.csdn.net): §2.1 the MoE
 *                class (hidden_size, num_experts, k, capacity_factor,
 *                min_capacity, drop_tokens) returning (output, gate_loss,
 *                expert_count); §3.1 the forward steps (gate, dispatch, expert
 *                compute, weighted merge, load-balance loss).
 *   [MoE-sched]  "MoE混合专家架构：大模型高效推理的智能调度原理" (lpnh.cn):
 *                §3.1 MoELayer, Steps 1-5 (router Linear, top-k, flatten and
 *                scatter into per-expert buffers, expert FFN Linear-GELU-Linear,
 *                gather and weighted sum) and the capacity / drop-tokens items.
 *   [DS-MoE-traps] DeepSeek-MoE fine-tuning article (lnwmold.com), ch.1:
 *                softmax over the router logits, top-2 on it, weighted sum;
 *                the capacity formula and the usage-std balance loss;
 *                ch.2 §2.1 the gradient mask (experts without tokens get no
 *                gradient) and ch.3 §3.1 the TopKRouter backward (the top-k
 *                selection passes gradient only to the chosen positions).
 *
 * Conventions for every call
 *  - Pointers named as device pointers must point to GPU memory of the
 *    current HIP device; the caller allocates and owns all of it, including
 *    the workspace sized by moe_workspace_size().  The library never
 *    allocates, frees or synchronises, and keeps no state between calls.
 *  - Tensors are dense row-major.  x is [T, d] (a [B, S, d] batch flattened
 *    with token t = b*S + s).  Expert weights use the nn.Linear layout
 *    [out, in]: w1 [E, h, d], w2 [E, d, h], b1 [E, h], b2 [E, d].  With
 *    ffn_hidden == 0 the expert is one Linear: w1 [E, d, d], b1 [E, d].
 *  - dtype MOE_BF16: x, weights, biases b1/b2, dispatched buffers and out are
 *    bf16 with fp32 accumulation; MOE_F32: all of those are fp32.  Router
 *    logits, router bias, gate weights and gate_loss are always fp32; indices,
 *    slots, counts and offsets int32.
 *  - stream is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    on it in order; the call returns before it finishes.
 *  - Errors: argument checks happen before anything is enqueued and return
 *    MOE_ERR_INVALID_ARG (bad value or missing pointer) or MOE_ERR_UNSUPPORTED
 *    (valid but outside what the kernels take, e.g. a row not a multiple of
 *    16 bytes); MOE_ERR_WORKSPACE if ws_bytes is too small; MOE_ERR_HIP if a
 *    launch fails.  Nothing is written on an error.
 *  - Routing is deterministic: identical inputs give bit-identical outputs.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Activation after the first Linear (or after the only Linear when
 * ffn_hidden == 0).  GELU is the exact erf form 0.5*x*(1+erf(x/sqrt(2))),
 * nn.GELU()'s default, as in [MoE-sched] §3.1 item 2 (Linear-GELU-Linear),
 * evaluated in fp32 to within 2.5e-6*|x| (the large-tile GEMM and the
 * small-batch kernel: a fitted 2^P form of the normal CDF's tail; the
 * other kernels: erff), far below the bf16 rounding of the stored
 * result. */
typedef enum { MOE_ACT_NONE = 0, MOE_ACT_RELU = 1, MOE_ACT_GELU = 2 } moe_act;

/* gate_loss kind, returned without the caller's loss weight.
 * BALANCE:   E * sum_e mean_t(p[t,e]) * (#tokens whose top-1 is e)/T, p the
 *            softmax over all experts, top-1 counted before capacity
 *            ([ds.moe] §3.1 step 5 names a load-balancing loss).
 * USAGE_STD: population std over experts of (#choices of e)/(k*T), all k
 *            choices before capacity, plus 1e-6 ([DS-MoE-traps] ch.1, the
 *            balance-loss table: lambda * (std(usage_prob) + 1e-6)). */
typedef enum { MOE_LOSS_BALANCE = 0, MOE_LOSS_USAGE_STD = 1 } moe_loss_kind;

/* Gate noise policy ([ds.moe] §2.1 noisy_gate_policy: "jitter" or "rsample"). */
typedef enum { MOE_NOISE_NONE = 0, MOE_NOISE_JITTER = 1, MOE_NOISE_RSAMPLE = 2 } moe_noise;

#define MOE_MAX_EXPERTS 256
/* Token counts of the fused small-batch forward (moe_config.small_batch). */
#define MOE_SMALL_BATCH_MAX 256
#define MOE_SMALL_BATCH_AUTO 64

/* Layer configuration ([ds.moe] §2.1 MoE arguments). */
typedef struct moe_config {
  int64_t num_tokens;      /* T >= 0, T < 2^30                                  */
  double capacity_factor;  /* > 0 when drop_tokens                              */
  int32_t hidden_size;     /* d > 0                                             */
  int32_t num_experts;     /* E, 1..MOE_MAX_EXPERTS                             */
  int32_t k;               /* 1 or 2, k <= E                                    */
  int32_t min_capacity;    /* >= 0                                              */
  int32_t drop_tokens;     /* 1: claims past the capacity are dropped;
                              0: no capacity, buffers sized by the counts      */
  int32_t ffn_hidden;      /* h >= 0; 0 = the expert is one Linear(d -> d)      */
  int32_t activation;      /* moe_act                                           */
  int32_t dtype;           /* moe_dtype                                         */
  int32_t normalize_topk;  /* 0: weight = softmax prob of the chosen expert;
                              1: the k chosen probs rescaled to sum to 1, i.e.
                              softmax over the top-k logits ([MoE-sched] §3.1
                              Step 2).  Computed before any drop.              */
  int32_t loss_kind;       /* moe_loss_kind                                     */
  int32_t save_preact;     /* 1 (training): moe_layer_forward keeps in the
                              workspace what the backward needs (the first
                              Linear's pre-activation, and the logits when
                              logits_out is NULL), and the workspace has the
                              regions the *_backward calls below use          */
  int32_t small_batch;     /* inference forward of a few tokens in one launch
                              (the fused small-batch kernel, up to
                              MOE_SMALL_BATCH_MAX tokens, bf16, d and h
                              multiples of 128, save_preact == 0):
                              0: when T <= MOE_SMALL_BATCH_AUTO;
                              1: whenever it applies; -1: never               */
  /* Seeded random gate options ([ds.moe] §2.1 noisy_gate_policy, use_rts,
   * top2_2nd_expert_sampling; the formulas, which the pages do not give,
   * follow the published DeepSpeed gate).  Every draw comes from
   * Philox4x32-10 keyed by seed: draw n of stream s is word n % 4 of the
   * block at counter (n / 4 low, n / 4 high, s, 0), key (seed low, seed
   * high); a word w gives u = ((w >> 9) + 0.5) * 2^-23 in (0, 1).  Streams:
   * 0 jitter (n = t*d + i), 1 RSample (n = t*E + e), 2 second expert
   * (n = t*E + e), 3 RTS (n = t).  All 0: the deterministic gate.  These
   * are training options: the caller sets them only when training; the
   * one-launch small-batch forward does not take them.                     */
  int32_t noisy_gate_policy;      /* moe_noise.  JITTER: the router reads
                              bf16(x * ((1 - 0.01) + 0.02 * u)) (fp32 product
                              and sum, each rounded once); the experts read
                              x; needs the router (not logits_in) and bf16.
                              RSample (k == 1): the expert is the argmax of
                              fp32(logit + g), g = -log(-log u); the weight
                              stays the clean softmax probability.          */
  int32_t use_rts;                /* k == 1: an expert whose demand exceeds C
                              keeps the C claims with the largest stream-3
                              words (ties to the lower token), in token
                              order; counts, offsets and loss unchanged     */
  int32_t second_expert_sampling; /* k == 2: the second expert is the argmax
                              over the other experts of fp32(logit + g)     */
  int32_t use_residual;           /* 1: the residual MoE of PR-MoE ([ds.moe]
                              §2.1 use_residual, §2.3, §3.3): the layer runs
                              through moe_residual_layer_forward / _backward
                              (moe_layer_forward and moe_layer_backward
                              refuse it) and the workspace holds the dense
                              branch's buffers                               */
  uint64_t seed;                  /* Philox key                             */
  int32_t packed_weights;         /* 1: the expert weights w1 and w2 given to
                              the forward calls (moe_expert_ffn,
                              moe_layer_forward, moe_residual_layer_forward)
                              are in the packed layout that
                              moe_pack_expert_weight writes; needs bf16 and
                              both Linears on the large-tile path (K a
                              multiple of 64, N of 16, see
                              moe_pack_expert_weight).  The backward calls
                              refuse it (MOE_ERR_INVALID_ARG): they read the
                              nn.Linear layout.  The dense branch of the
                              residual MoE is never packed.  0: nn.Linear
                              layout [E, out, in].                           */
} moe_config;

/* Static text for a status code. */
const char* moe_status_string(moe_status s);

/* Expert capacity C = max(min_capacity, ceil((k*T/E) * capacity_factor)),
 * evaluated in IEEE double exactly in that order ([DS-MoE-traps] ch.1
 * capacity row; [MoE-sched] §3.1 item 3).  *C = -1 when drop_tokens == 0.
 * Host only; C is a host pointer. */
moe_status moe_capacity(const moe_config* cfg, int64_t* C);

/* Upper bound on the packed rows N = sum_e expert_count[e]:
 * min(k*T, E*C) with a capacity, k*T without.  Host only. */
moe_status moe_max_rows(const moe_config* cfg, int64_t* rows);

/* Bytes of device workspace that every call below needs for cfg (the fused
 * forward's intermediate buffers included).  Host only. */
moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* Gate ([MoE-sched] §3.1 Steps 1-2; [ds.moe] §3.1 step 1 and step 5).
 * logits[t,e] = x[t]·w_router[e] (+ b_router[e]) accumulated in fp32, or
 * logits_in when it is non-NULL (then x / w_router are not read).
 * p = softmax over the E logits; the k chosen experts are the k largest
 * logits, ties to the lower expert index (-0.0 equals +0.0).  Non-finite
 * logits are outside the contract, but the chosen experts are always valid
 * indices: a NaN ranks as -inf, so a token whose logits are all -inf or NaN
 * takes the lowest indices.
 * Capacity slots: every top-1 claim in token order, then every top-2 claim in
 * token order, takes the next free slot of its expert; a slot >= C is dropped
 * (slot = -1).  expert_count[e] = kept claims of e, expert_offset the
 * exclusive prefix of expert_count (E+1 entries).
 *   x          device, [T, d] dtype            (ignored if logits_in)
 *   w_router   device, [E, d] dtype            (ignored if logits_in)
 *   b_router   device, [E] fp32, nullable  (ignored if logits_in)
 *   logits_in  device, [T, E] fp32, nullable
 *   logits_out device, [T, E] fp32, nullable: the logits used
 *   expert_idx device, [T, k] int32 out;  slot device, [T, k] int32 out
 *   weight     device, [T, k] fp32 out (gate weight of each choice)
 *   expert_count device [E] int32 out; expert_offset device [E+1] int32 out
 *   gate_loss  device, [1] fp32 out
 *   ws, ws_bytes  device workspace of moe_workspace_size() bytes */
moe_status moe_gate(const moe_config* cfg, const void* x, const void* w_router,
                    const float* b_router, const float* logits_in, float* logits_out,
                    int32_t* expert_idx, int32_t* slot, float* weight,
                    int32_t* expert_count, int32_t* expert_offset, float* gate_loss,
                    void* ws, size_t ws_bytes, void* stream);

/* The gate of moe_gate without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, kernels and
 * results as moe_gate; the gate's scratch (per-tile counts and probability
 * sums, about T/64 * E * (4k + 4) bytes) lives in a library-owned device
 * array of MOE_GATE_NOALLOC_SCRATCH_BYTES per GPU, held until the process
 * ends.  MOE_ERR_WORKSPACE when cfg needs more than that (with E = 256,
 * k = 2: beyond about T = 174000 tokens).  Nothing is allocated or freed.  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (concurrent streams, or host threads) race and must be serialised by
 * the caller (one stream, or events). */
#define MOE_GATE_NOALLOC_SCRATCH_BYTES (8u << 20)
moe_status moe_gate_noalloc(const moe_config* cfg, const void* x, const void* w_router,
                            const float* b_router, const float* logits_in, float* logits_out,
                            int32_t* expert_idx, int32_t* slot, float* weight,
                            int32_t* expert_count, int32_t* expert_offset, float* gate_loss,
                            void* stream);

/* Packed expert weights (the layout of the expert weights in device
 * memory, not a step of the layer: [MoE-sched] §3.1 Step 4 multiplies each
 * expert's token rows by its weight whatever the layout).  An expert weight
 * in the nn.Linear layout w[E, N, K] (N outputs, K inputs; w1: N = h,
 * K = d; w2: N = d, K = h; ffn_hidden == 0: N = K = d) is rewritten as
 * blocks of 256 output rows x 64 inputs, each block contiguous (32 KB in
 * bf16):
 *   packed[((e * ceil(N/256) + n / 256) * (K/64) + k / 64) * 16384
 *          + (n % 256) * 64 + k % 64] = w[e, n, k]
 * with zeros in the rows n >= N of the last block.  A 64-wide K step of a
 * 256-feature tile of the grouped GEMM is then one contiguous 32 KB read
 * instead of 256 rows of 128 bytes K elements apart, which spread over few
 * memory channels; a caller that keeps its inference weights packed (once,
 * after loading or after each update) runs the forward's GEMMs faster.
 * Needs dtype bf16, K a positive multiple of 64, N a positive multiple of
 * 16 (MOE_ERR_UNSUPPORTED otherwise, MOE_ERR_INVALID_ARG for non-positive
 * sizes or E outside 1..MOE_MAX_EXPERTS).
 *   moe_packed_weight_bytes: the packed size, E * ceil(N/256) * 256 * K * 2.
 *   moe_pack_expert_weight: w device [E, N, K]; w_packed device, that many
 *   bytes, must not overlap w; enqueued on stream. */
moe_status moe_packed_weight_bytes(int32_t num_experts, int64_t n, int64_t k, int32_t dtype,
                                   size_t* bytes);
moe_status moe_pack_expert_weight(int32_t num_experts, int64_t n, int64_t k, int32_t dtype,
                                  const void* w, void* w_packed, void* stream);

/* Dispatch ([MoE-sched] §3.1 Step 3; [ds.moe] §3.1 step 2 on one GPU):
 * for every kept claim (t, j): x_disp[expert_offset[e] + slot[t,j]] = x[t],
 * e = expert_idx[t,j].  x_disp is the packed expert-major buffer, device,
 * [>= moe_max_rows, d] dtype; rows past expert_offset[E] are not written. */
moe_status moe_dispatch(const moe_config* cfg, const void* x, const int32_t* expert_idx,
                        const int32_t* slot, const int32_t* expert_offset, void* x_disp,
                        void* stream);

/* Expert FFNs on the packed buffer ([MoE-sched] §3.1 Step 4; [ds.moe] §3.1
 * step 3): for the rows of expert e,
 *   a = x_disp·w1[e]^T + b1[e];  h = act(a);  y = h·w2[e]^T + b2[e]
 * (ffn_hidden == 0: y = act(x_disp·w1[e]^T + b1[e]); w2/b2/h_disp/a_save are
 * not used and may be NULL).  fp32 accumulation; bias and activation in fp32;
 * a, h and y are stored as dtype.  b1/b2 nullable (no bias).
 *   x_disp device [rows, d]; h_disp device [rows, h]; y_disp device [rows, d]
 *   a_save device [rows, h], nullable: the pre-activation for the backward
 * where rows >= expert_offset[E] (moe_max_rows suffices).  h_ld is the row
 * pitch of h_disp and a_save in elements: 0 or h for contiguous rows, or
 * h + 64 (only for bf16 with d and h multiples of 64, else
 * MOE_ERR_UNSUPPORTED; MOE_ERR_INVALID_ARG for any other value).  An odd
 * number of 128-byte lines per row lets the second Linear read h_disp
 * faster; moe_workspace_h_ld gives the pitch moe_layer_forward uses. */
moe_status moe_expert_ffn(const moe_config* cfg, const void* x_disp, const int32_t* expert_offset,
                          const void* w1, const void* b1, const void* w2, const void* b2,
                          void* a_save, void* h_disp, int64_t h_ld, void* y_disp,
                          void* ws, size_t ws_bytes, void* stream);

/* Backward of the expert FFNs for an upstream gradient dy_disp [rows, d]
 * (dx_disp may be the same buffer as dy_disp: dY's last read precedes the
 * first write of dX)
 * (chain rule of Linear-act-Linear, per expert e on its packed rows):
 *   dh = dy·w2[e];  da = dh ⊙ act'(a_save)  (stored as dtype);
 *   dx = da·w1[e];  dw2[e] = dy^T·h;  dw1[e] = da^T·x;
 *   db2[e] = sum_rows dy;  db1[e] = sum_rows da   (fp32, nullable)
 * Needs ffn_hidden > 0; MOE_ERR_UNSUPPORTED unless dtype is MOE_BF16 and d
 * and h are multiples of 16.  dx_disp device [rows, d] bf16; dw1 [E, h, d]
 * and dw2 [E, d, h] bf16 (fp32 accumulation; experts with no rows get
 * zeros); db1 [E, h], db2 [E, d] fp32.  ws as above (it also holds dA).
 * a_save and h_disp are read with contiguous rows (pitch h), as the forward
 * writes them with h_ld = 0 or with cfg->save_preact. */
moe_status moe_expert_ffn_backward(const moe_config* cfg, const void* x_disp,
                                   const int32_t* expert_offset, const void* w1, const void* w2,
                                   const void* a_save, const void* h_disp, const void* dy_disp,
                                   void* dx_disp, void* dw1, float* db1, void* dw2, float* db2,
                                   void* ws, size_t ws_bytes, void* stream);

/* Combine ([MoE-sched] §3.1 Step 5; [ds.moe] §3.1 step 4):
 * out[t] = sum over j = 0..k-1 with slot[t,j] >= 0 of
 *          weight[t,j] * y_disp[expert_offset[expert_idx[t,j]] + slot[t,j]],
 * summed in fp32 in j order and stored as dtype; a token whose claims were
 * all dropped gets a zero row.  out device [T, d]. */
moe_status moe_combine(const moe_config* cfg, const void* y_disp, const int32_t* expert_idx,
                       const int32_t* slot, const float* weight, const int32_t* expert_offset,
                       void* out, void* stream);

/* The whole layer forward on one stream with no host synchronisation:
 * gate -> dispatch -> expert FFNs -> combine.  Returns ([ds.moe] §2.1) the
 * output out [T, d] dtype, gate_loss [1] fp32 and expert_count [E] int32
 * (all device).  logits_out, expert_idx, slot, weight are optional outputs
 * (nullable, shapes as in moe_gate); when NULL the workspace holds them.
 * x/w_router/b_router/logits_in as in moe_gate; w1/b1/w2/b2 as in
 * moe_expert_ffn.  Intermediates stay in the workspace; see
 * moe_workspace_views.
 * Small batches at inference (cfg->small_batch, save_preact == 0) run as
 * one persistent launch of one workgroup per CU ([ds.moe] §4 inference
 * notes: gating and token assignment fused to save launches) with the same
 * results: routing, slots, counts, offsets and packed rows identical, the
 * floating-point outputs within rounding of the multi-kernel path (the
 * router's K is split into slices added in order).  Its grid barriers wait
 * a bounded time; on a device where some other kernel keeps CUs busy for
 * seconds, a wait that runs out stops the kernel and sets *gate_loss to
 * NaN (the other outputs are then undefined). */
moe_status moe_layer_forward(const moe_config* cfg, const void* x, const void* w_router,
                             const float* b_router, const float* logits_in,
                             const void* w1, const void* b1, const void* w2, const void* b2,
                             void* out, float* gate_loss, int32_t* expert_count,
                             float* logits_out, int32_t* expert_idx, int32_t* slot,
                             float* weight, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Backward of the layer.  Gradients follow the chain rule through the
 * forward above; the top-k choice and the capacity slots are piecewise
 * constant and pass no gradient ([DS-MoE-traps] ch.3 §3.1 TopKRouter
 * backward, ch.2 §2.1 gradient mask); the chosen probabilities reach every
 * logit through the softmax.  bf16 only for the calls that run GEMMs.
 * Those that take ws need a config with save_preact = 1 (else
 * MOE_ERR_INVALID_ARG) and ws of moe_workspace_size() bytes.
 * ------------------------------------------------------------------------ */

/* Backward of moe_combine: for every kept claim (t, j) at packed row
 * r = expert_offset[e] + slot[t,j]:
 *   dy_disp[r]    = weight[t,j] * dout[t]   (fp32 product, stored as dtype)
 *   dweight[t,j]  = <dout[t], y_disp[r]>    (fp32 accumulation)
 * and dweight = 0 for dropped claims.  dout device [T, d] dtype; y_disp and
 * dy_disp device [rows, d] dtype and MAY BE THE SAME BUFFER (each row is
 * read, then overwritten, by the one wavefront that owns its claim);
 * dweight device [T, k] fp32. */
moe_status moe_combine_backward(const moe_config* cfg, const void* dout, const void* y_disp,
                                const int32_t* expert_idx, const int32_t* slot, const float* weight,
                                const int32_t* expert_offset, void* dy_disp, float* dweight, void* stream);

/* Logit gradient of the gate ([MoE-sched] §3.1 Step 2; [ds.moe] §3.1 step 5):
 * p = softmax(logits[t]);  dp[e_j] += dweight[t,j] (when normalize_topk,
 * w_j = p_j / S with S the sum of the k chosen p, so dp[e_i] +=
 * (dweight_i - sum_j dweight_j w_j) / S);  BALANCE loss: dp[e] +=
 * dloss * E * ce_e / T, ce_e the share of tokens whose top-1 is e
 * (USAGE_STD depends on counts only and adds nothing);
 * dlogits[t] = p * (dp - <p, dp>), all fp32.
 *   logits   device [T, E] fp32: the logits the forward used
 *   dweight  device [T, k] fp32 (from moe_combine_backward)
 *   dloss    device [1] fp32, the upstream gradient of gate_loss; NULL = 0
 *   dlogits  device [T, E] fp32 out */
moe_status moe_gate_backward(const moe_config* cfg, const float* logits, const int32_t* expert_idx,
                             const float* dweight, const float* dloss, float* dlogits, void* ws,
                             size_t ws_bytes, void* stream);

/* Backward of moe_dispatch plus, when w_router is non-NULL, the router
 * Linear's input gradient ([MoE-sched] §3.1 Steps 1 and 3):
 *   dx[t] = sum over kept j (choice order) of dx_disp[row(t,j)]
 *           + dlogits[t] · w_router            (fp32, one rounding to bf16)
 * The router product runs on bf16 matrix cores with dlogits split into two
 * bf16 terms (|error| <= 2^-16 |dlogits| per element before the fp32 sum).
 * A token with every claim dropped gets the router term only.
 *   dx_disp device [rows, d] bf16;  w_router device [E, d] bf16, nullable;
 *   dlogits device [T, E] fp32 (needed with w_router);  dx device [T, d] bf16.
 * MOE_ERR_UNSUPPORTED unless bf16 and d % 32 == 0. */
moe_status moe_dispatch_backward(const moe_config* cfg, const void* dx_disp, const int32_t* expert_idx,
                                 const int32_t* slot, const int32_t* expert_offset, const void* w_router,
                                 const float* dlogits, void* dx, void* ws, size_t ws_bytes, void* stream);

/* Router weight gradients ([MoE-sched] §3.1 Step 1, the router Linear):
 *   dw_router[e, :] = sum_t dlogits[t, e] * x[t, :]   fp32 [E, d], nullable
 *   db_router[e]    = sum_t dlogits[t, e]              fp32 [E], nullable
 * (at least one non-NULL).  x device [T, d] bf16.  Token chunks are summed
 * in a fixed order, so results are bit-identical run to run.
 * MOE_ERR_UNSUPPORTED unless bf16 and d % 64 == 0 (for dw_router). */
moe_status moe_router_backward(const moe_config* cfg, const void* x, const float* dlogits,
                               float* dw_router, float* db_router, void* ws, size_t ws_bytes,
                               void* stream);

/* The whole layer backward on one stream, after moe_layer_forward with the
 * same cfg (save_preact = 1, ffn_hidden > 0, bf16) and the same ws, whose
 * intermediates it consumes (afterwards ws's y_disp region holds dX_disp):
 *   moe_combine_backward -> moe_expert_ffn_backward -> moe_gate_backward ->
 *   moe_dispatch_backward (with the router input term) -> moe_router_backward.
 * Gradients of <dout, out> + dloss * gate_loss with respect to:
 *   dx [T, d] bf16;  dlogits [T, E] fp32 (nullable when w_router is given;
 *   required when the forward took logits_in, i.e. w_router == NULL);
 *   dw_router [E, d] fp32, db_router [E] fp32 (nullable; need w_router);
 *   dw1 [E, h, d], dw2 [E, d, h] bf16; db1 [E, h], db2 [E, d] fp32 (nullable).
 * logits, expert_idx, slot, weight: what the forward wrote, or NULL if the
 * forward kept them in ws (logits_out / expert_idx / slot / weight NULL).
 * x, w_router, w1, w2 as in moe_layer_forward; dout device [T, d] bf16;
 * dloss device [1] fp32 or NULL (= 0).  MOE_ERR_UNSUPPORTED unless d is a
 * multiple of 32 (64 with dw_router) and h of 16. */
moe_status moe_layer_backward(const moe_config* cfg, const void* x, const void* w_router, const void* w1,
                              const void* w2, const float* logits, const int32_t* expert_idx,
                              const int32_t* slot, const float* weight, const void* dout,
                              const float* dloss, void* dx, float* dlogits, float* dw_router,
                              float* db_router, void* dw1, float* db1, void* dw2, float* db2, void* ws,
                              size_t ws_bytes, void* stream);

/* Residual MoE forward (PR-MoE: [ds.moe] §2.1 use_residual, §2.3, §3.3;
 * the mix is not on the pages, the published layer's is taken):
 *   out[t] = c0[t] * moe[t] + c1[t] * mlp(x[t])
 * moe: this layer's MoE output before rounding (gate, dispatch, experts,
 * combine exactly as moe_layer_forward);  mlp: the expert's architecture
 * with its own weights on every token, mlp_w1 [h, d] (or [d, d] when
 * ffn_hidden == 0), mlp_b1 [h] (nullable), mlp_w2 [d, h] (NULL when
 * ffn_hidden == 0), mlp_b2 [d] (nullable), dtype; its activation output
 * and output are stored as dtype like an expert's;
 * c[t] = softmax(x[t] · coef_w^T + coef_b) over two entries, coef_w [2, d]
 * dtype, coef_b [2] fp32 (nullable); with coef_w NULL, c = (1, 1), the plain
 * residual sum.  The sum and the mix are fp32 with one rounding of out.
 * coef_out [T, 2] fp32 (nullable; the backward reads the workspace copy).
 * Other arguments as in moe_layer_forward.  Requires cfg->use_residual == 1
 * and bf16; the one-launch small-batch path is not used.  With
 * save_preact the workspace keeps the dense branch's pre-activation for
 * moe_residual_layer_backward. */
moe_status moe_residual_layer_forward(const moe_config* cfg, const void* x, const void* w_router,
                                      const float* b_router, const float* logits_in, const void* w1,
                                      const void* b1, const void* w2, const void* b2, const void* mlp_w1,
                                      const void* mlp_b1, const void* mlp_w2, const void* mlp_b2,
                                      const void* coef_w, const float* coef_b, void* out, float* gate_loss,
                                      int32_t* expert_count, float* coef_out, float* logits_out,
                                      int32_t* expert_idx, int32_t* slot, float* weight, void* ws,
                                      size_t ws_bytes, void* stream);

/* Residual MoE backward, after moe_residual_layer_forward with the same cfg
 * (save_preact = 1, use_residual = 1, ffn_hidden > 0, bf16) and ws.
 * Gradients of <dout, out> + dloss * gate_loss: the MoE branch as
 * moe_layer_backward with dout scaled by c0; the dense branch as an expert
 * backward with dout scaled by c1 (mlp_dw1 [h, d], mlp_dw2 [d, h] bf16,
 * mlp_db1 [h], mlp_db2 [d] fp32 nullable); the coefficients' logit gradient
 * c * (dc - <c, dc>) with dc = (<dout, moe>, <dout, mlp>), giving
 * dcoef_w [2, d] and dcoef_b [2] fp32 (nullable; need coef_w) and its term
 * in dx.  dx [T, d] bf16 sums the three input gradients with one rounding.
 * Other arguments as in moe_layer_backward. */
moe_status moe_residual_layer_backward(const moe_config* cfg, const void* x, const void* w_router,
                                       const void* w1, const void* w2, const void* mlp_w1,
                                       const void* mlp_w2, const void* coef_w, const float* logits,
                                       const int32_t* expert_idx, const int32_t* slot, const float* weight,
                                       const void* dout, const float* dloss, void* dx, float* dlogits,
                                       float* dw_router, float* db_router, void* dw1, float* db1, void* dw2,
                                       float* db2, void* mlp_dw1, float* mlp_db1, void* mlp_dw2,
                                       float* mlp_db2, float* dcoef_w, float* dcoef_b, void* ws,
                                       size_t ws_bytes, void* stream);

/* Device addresses, inside a workspace ws, of the intermediates that
 * moe_layer_forward leaves there (valid until the next call that uses ws):
 * packed x_disp [rows, d] (with cfg->save_preact always; without it the
 * multi-kernel forward may skip the copy, its first Linear then loading each
 * packed row from x through a row map kept in the workspace, and x_disp is
 * not written), a_save [rows, h] (only with cfg->save_preact),
 * h_disp [rows, h], y_disp [rows, d] and expert_offset [E+1] int32.  The
 * rows of h_disp are contiguous with cfg->save_preact; without it the
 * forward may keep them at a pitch of h + 64 elements, in a region sized
 * for that pitch.  Any
 * output pointer may be NULL.  Host only; computes addresses, reads nothing. */
moe_status moe_workspace_views(const moe_config* cfg, void* ws, void** x_disp, void** a_save,
                               void** h_disp, void** y_disp, int32_t** expert_offset);

/* The row pitch (elements) at which moe_layer_forward keeps h_disp in the
 * workspace for this cfg (h, or h + 64 without save_preact as described at
 * moe_workspace_views; 0 when ffn_hidden == 0).  Host only;
 * MOE_ERR_INVALID_ARG for an invalid cfg or a NULL h_ld. */
moe_status moe_workspace_h_ld(const moe_config* cfg, int64_t* h_ld);

/* Device address, inside a workspace ws, of the status word of the
 * one-launch small-batch forward (see moe_layer_forward): a uint32 that the
 * launch zeroes first and sets to 1 if one of its grid barriers stopped
 * waiting (its other outputs are then undefined, and *gate_loss is NaN).
 * It holds the last small-batch launch's status until the next one on ws;
 * the caller reads it after synchronising the stream.  *status = NULL when
 * cfg->num_tokens exceeds MOE_SMALL_BATCH_MAX (no such launch for cfg).
 * Host only; computes an address, reads nothing. */
moe_status moe_workspace_status(const moe_config* cfg, void* ws, uint32_t** status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
