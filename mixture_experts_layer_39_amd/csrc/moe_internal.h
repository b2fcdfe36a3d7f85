// Internal declarations shared by the HIP kernels and the C-ABI host layer.
// Not installed; the public interface is include/moe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define MOE_MAX_EXPERTS_DEV 256

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Two floats to two bf16 (round to nearest even) in one 32-bit word, lo in
// the low half: a single v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v r = __builtin_convertvector((f32x2){lo, hi}, bf16x2v);
  return __builtin_bit_cast(uint32_t, r);
}

enum { DT_F32 = 0, DT_BF16 = 1 };
enum { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2 };
enum { LOSS_BALANCE = 0, LOSS_USAGE_STD = 1 };

// GELU(x) = x Phi(x) = max(x, 0) - |x| Phi(-|x|).  For t in [0, 5.5],
// Phi(-t) = 2^P(t) with P the degree-7 polynomial below: a Chebyshev
// least-squares fit of log2 Phi(-t) on that interval, coefficients rounded
// to fp32; evaluated in fp32, 2^P(t) is within 4.3e-6 (relative) of
// Phi(-t).  Past 5.5, Phi(-t) < 1.9e-8 is below fp32 rounding of x Phi(x)
// for x > 0 and gives |x| Phi(x) < 1.9e-8 |x| for x < 0, so the term is
// dropped.  |GELU error| <= 2.2e-6 |x|, far below bf16 rounding.  One exp2
// and eleven VALU operations, no branch; NaN propagates, GELU(+-inf) is
// +inf and 0.
__device__ __forceinline__ float gelu_fast(float x) {
  const float ax = fabsf(x);
  const float s = ax > 5.5f ? 0.f : ax;   // NaN stays NaN
  float p = fmaf(-0x1.01da94p-19f, s, 0x1.0971d8p-14f);
  p = fmaf(p, s, -0x1.ee9e1p-11f);
  p = fmaf(p, s, 0x1.185ecp-7f);
  p = fmaf(p, s, -0x1.bacb96p-5f);
  p = fmaf(p, s, -0x1.d56212p-2f);
  p = fmaf(p, s, -0x1.26ba2cp+0f);
  p = fmaf(p, s, -0x1.ffff32p-1f);
  // max(x, 0) as one v_max: fmaxf adds a second instruction to quiet a
  // signalling NaN in x, which is not needed here (a NaN x already makes s,
  // and so the result, NaN)
  float xp;
  asm("v_max_f32 %0, 0, %1" : "=v"(xp) : "v"(x));
  return fmaf(-s, __builtin_amdgcn_exp2f(p), xp);
}

template <int ACT>
__device__ __forceinline__ float act_fixed(float v) {
  if constexpr (ACT == ACT_RELU) return fmaxf(v, 0.f);
  else if constexpr (ACT == ACT_GELU) return gelu_fast(v);
  else return v;
}


// ---------------------------------------------------------------- gate
// Tokens per gate tile: at most 64 (four groups of 16, one per wavefront),
// which sizes the per-tile workspace; gate_tile_tokens_for gives the tile a
// launch uses (256 for the deterministic 65..128-expert bf16 router).
inline int gate_tile_tokens(int) { return 64; }
int gate_tile_tokens_for(int E, int d, int dtype, bool logits_in, bool random_options);

struct GateArgs {
  const void* x;            // [T, d] dtype (router GEMM modes)
  const void* w_router;     // [E, d] dtype
  const float* b_router;    // [E] or null
  const float* logits_in;   // [T, E] or null
  float* logits_out;        // [T, E] or null
  int32_t* expert_idx;      // [T, k]
  int32_t* slot;            // [T, k]: raw per-(choice, expert) rank on exit
  float* weight;            // [T, k]
  int32_t* expert_count;    // [E]
  int32_t* expert_offset;   // [E+1]
  float* gate_loss;         // [1]
  int32_t* tile_cnt;        // [k*E, tiles]: claims per (choice, expert) column and
                            // tile; the scan turns it into the exclusive prefix
  float* me_tile;           // [tiles, E] per-tile sums of the softmax probabilities
  double* me_sum;           // [E] their totals
  int32_t* demand;          // [k, E] total claims per (choice, expert)
  uint32_t* sync;           // arrival counter of the scan kernel (zeroed by the gate kernel)
  int64_t T;
  int64_t C;                // capacity, < 0 = none
  int32_t d, E, k;
  int32_t normalize, loss_kind;
  int32_t num_tiles;
  int32_t tile_tokens;      // tokens per tile (64, or 256 for the 65..128-expert router)
  int32_t jitter, rsample, second;   // random gate options (router input jitter,
                                     // Gumbel top-1, Gumbel second expert)
  uint32_t seed_lo, seed_hi;         // Philox4x32-10 key
};

hipError_t launch_gate(const GateArgs& a, int dtype, hipStream_t s);
// Random Token Selection (k = 1, with a capacity): after the slot fix-up,
// every expert whose demand exceeds C keeps its C claims of largest priority.
hipError_t launch_rts_select(const GateArgs& a, hipStream_t s);
hipError_t launch_slot_finalize(const GateArgs& a, hipStream_t s);
hipError_t launch_gate_empty(int32_t* expert_count, int32_t* expert_offset, float* gate_loss,
                             int E, hipStream_t s);

// ---------------------------------------------------------------- dispatch / combine
hipError_t launch_dispatch(const void* x, const int32_t* expert_idx, const int32_t* slot,
                           const int32_t* expert_offset, void* x_disp, int64_t T, int k,
                           int row_bytes, hipStream_t s);
// Dispatch with the gate's slot fix-up fused in (g as the gate ran it, its
// slots still the in-tile ranks): writes the final slots and the packed rows.
hipError_t launch_dispatch_finalize(const void* x, const GateArgs& g, void* x_disp, int row_bytes, hipStream_t s);
// The dispatch as a row map (packed row -> token) for a first Linear that
// gathers its rows from x: from final slots, or with the slot fix-up fused in.
hipError_t launch_row_map(const int32_t* expert_idx, const int32_t* slot, const int32_t* expert_offset,
                          int32_t* row_tok, int64_t T, int k, hipStream_t s);
hipError_t launch_row_map_finalize(const GateArgs& g, int32_t* row_tok, hipStream_t s);
hipError_t launch_combine(const void* y_disp, const int32_t* expert_idx, const int32_t* slot,
                          const float* weight, const int32_t* expert_offset, void* out,
                          int64_t T, int k, int d, int dtype, hipStream_t s);

// ---------------------------------------------------------------- expert GEMMs
// Y[rows of e] = act(X[rows of e] · W[e]^T + bias[e]) on the packed layout.
struct GemmArgs {
  const void* X;             // [rows, K]
  const void* W;             // [E, N, K]
  const void* bias;          // [E, N] or null
  void* Y;                   // [rows, N]
  void* Apre;                // [rows, N] pre-activation, or null
  const int32_t* offset;     // [E+1]
  int64_t max_rows;          // upper bound on offset[E] (sizes the grid)
  int32_t E, N, K, act;
  int64_t x_ld = 0, y_ld = 0;  // row pitches of X and Y (and Apre) in elements; 0: K and N.
                               // Other pitches only where grouped_gemm_is_big holds.
  int32_t w_packed = 0;        // W in the packed layout (moe_pack_expert_weight); big path only
  const int32_t* x_map = nullptr;  // non-null: X is the token matrix [x_rows, K] and packed row r
                                   // reads X row x_map[r] (the dispatch folded into the loads;
                                   // big path, bf16, contiguous X only)
  int64_t x_rows = 0;
  int32_t tile_rows = 256;         // row tile height of the large-tile GEMM: 256, or 320 (K-contiguous X,
                                   // no x_map): an expert of up to 640 rows in two row tiles, not three
};
hipError_t launch_grouped_gemm(const GemmArgs& a, int dtype, hipStream_t s);
// Compute units of the current device (cached per device).
int device_cus();
// Whether launch_grouped_gemm runs this shape on the large-tile kernel.
bool grouped_gemm_is_big(int64_t K, int64_t N, int dtype);
// Expert weight [E, N, K] (bf16) into the packed layout: blocks of 256 rows
// x 64 K values, each contiguous, rows past N zero.
hipError_t launch_pack_expert_weight(const void* w, void* wp, int E, int64_t N, int64_t K, hipStream_t s);

// Backward pieces (see gemm_bwd.hip).
struct GemmBwdArgs {
  const void* X;         // [rows, d]   x_disp
  const void* W1;        // [E, h, d]
  const void* W2;        // [E, d, h]
  const void* A;         // [rows, h]   saved pre-activation
  const void* H;         // [rows, h]
  const void* dY;        // [rows, d]
  void* dA;              // [rows, h]   workspace
  void* dX;              // [rows, d]
  void* dW1;             // [E, h, d]
  void* dW2;             // [E, d, h]
  float* db1;            // [E, h] or null
  float* db2;            // [E, d] or null
  const int32_t* offset; // [E+1]
  int64_t max_rows;
  int32_t E, d, h, act;
};
hipError_t launch_ffn_backward(const GemmBwdArgs& a, int dtype, hipStream_t s);
// The four backward GEMMs on the large-tile kernel, or hipErrorNotSupported.
hipError_t launch_backward_big(const GemmBwdArgs& a, hipStream_t s);

// ---------------------------------------------------------------- layer backward
// Router-gradient layout: the logit gradient is carried as two bf16 arrays
// (hi = bf16(g), lo = bf16(g - hi), |g - hi - lo| <= 2^-16 |g|) side by
// side in rows of 2*Ep, Ep = E rounded up to 32 (zero padded), so that the
// router products run on bf16 MFMA at nearly fp32 accuracy.
inline int router_ep(int E) { return (E + 31) / 32 * 32; }

// Token chunks of the router weight gradient dW_r = dlogits^T x: the token
// range is cut into S chunks (a multiple of 64 tokens each, at least 1024
// unless T is smaller) so that S x (feature tiles) fills the chip; each chunk
// yields an fp32 partial [2*Ep, d] that a second kernel sums in chunk order.
struct RouterChunks {
  int S, chunk;
};
inline RouterChunks router_chunks(int64_t T, int d, int E) {
  RouterChunks r{0, 0};
  if (T <= 0) return r;
  const int64_t ep2 = 2 * (int64_t)router_ep(E);
  const int64_t tiles = ((ep2 + 255) / 256) * ((d + 255) / 256);
  int64_t S = (256 + tiles - 1) / tiles;
  const int64_t smax = (T + 1023) / 1024;
  if (S > smax) S = smax;
  // a chunk's operand bytes must stay below 2^31 (32-bit buffer offsets)
  const int64_t wmax = (d > ep2 ? d : ep2) * 2;
  const int64_t smin = (T * wmax + (int64_t(1) << 30) - 1) >> 30;
  if (S < smin) S = smin;
  if (S < 1) S = 1;
  int64_t chunk = ((T + S - 1) / S + 63) / 64 * 64;
  r.chunk = (int)chunk;
  r.S = (int)((T + chunk - 1) / chunk);
  return r;
}
constexpr int kRouterMaxChunks = 256;
constexpr int kTop1Parts = 64;          // workgroups of the top-1 histogram
constexpr int kGateBwdTokens = 32;      // tokens per gate-backward workgroup

hipError_t launch_combine_backward(const void* dout, const void* y_disp, const int32_t* expert_idx,
                                   const int32_t* slot, const float* weight, const int32_t* expert_offset,
                                   void* dy_disp, float* dweight, int64_t T, int k, int d, int dtype,
                                   hipStream_t s);

struct GateBwdArgs {
  const float* logits;      // [T, E] (the logits of the forward); null = dlogits is an input
  const int32_t* idx;       // [T, k]
  const float* dw;          // [T, k] gradient of the gate weights
  const float* coef;        // [E] dloss*E*ce_e/T (BALANCE), or null
  float* dlogits;           // [T, E]: output (from logits) or input
  uint16_t* dl_hl;          // [T, 2*Ep] bf16 hi/lo split, or null
  float* dbpart;            // [E, ceil(T/kGateBwdTokens)] column partial sums, or null
  int64_t T;
  int32_t E, k, Ep, normalize;
};
hipError_t launch_top1_coef(const int32_t* idx, int k, int64_t T, int E, const float* dloss, int32_t* part,
                            float* coef, hipStream_t s);
hipError_t launch_gate_backward(const GateBwdArgs& a, hipStream_t s);

struct InputGradArgs {
  const bf16* dx_disp;      // [rows, d]
  const int32_t* idx;       // [T, k]
  const int32_t* slot;      // [T, k]
  const int32_t* offset;    // [E+1]
  const uint16_t* dl_hl;    // [T, 2*Ep] or null (no router term)
  const uint16_t* wfrag;    // [d * Ep] router weight in MFMA fragment order, zero padded
  bf16* dx;                 // [T, d]
  int64_t T;
  int32_t d, k, Ep;
  int32_t jitter;           // the router read x * factor: its term is scaled by the factor
  uint32_t seed_lo, seed_hi;
  const bf16* dx_add;       // [T, d] added to dx, or null (the residual MLP's input gradient)
  const float* dlc;         // [T, 2] coefficient logit gradient, or null
  const bf16* coef_w;       // [2, d]: with dlc, dx += dlc[t] · coef_w
};
hipError_t launch_router_pack(const void* w_router, uint16_t* wfrag, int E, int d, int Ep, hipStream_t s);
hipError_t launch_input_grad(const InputGradArgs& a, hipStream_t s);
// The router's jittered input bf16(x * factor) [T, d] (the forward gate's
// arithmetic), for the router weight gradient.
hipError_t launch_jitter_input(const bf16* x, bf16* xj, int64_t T, int d, uint32_t seed_lo, uint32_t seed_hi,
                               hipStream_t s);

// dW_r (fp32 [E, d], nullable) and db_r (fp32 [E], nullable) from the split
// logit gradient and x; part: [S, 2*Ep, d] fp32, choff: [S+1] int32.
struct RouterWgradArgs {
  const void* x;            // [T, d] bf16
  const uint16_t* dl_hl;    // [T, 2*Ep]
  const float* dbpart;      // [E, ceil(T/kGateBwdTokens)]
  int32_t* choff;
  float* part;
  float* dw_router;
  float* db_router;
  int64_t T;
  int32_t d, E, Ep;
};
hipError_t launch_router_wgrad(const RouterWgradArgs& a, hipStream_t s);
// The chunked product on the large-tile GEMM: part[c] = dl_hl[chunk c]^T x[chunk c].
hipError_t launch_router_partials(const uint16_t* dl_hl, const void* x, const int32_t* choff, float* part,
                                  int64_t T, int S, int d, int Ep, hipStream_t s);

// ---------------------------------------------------------------- residual MoE
// Per-token parts of the residual (PR-MoE) layer, see residual.hip.
struct ResidualArgs {
  const bf16* x;             // [T, d]
  const bf16* coef_w;        // [2, d] or null: then the coefficients are (1, 1)
  const float* coef_b;       // [2] or null
  bf16* y_disp;              // [rows, d]; the backward writes dY_disp over it
  bf16* mlp_y;               // [T, d]; the backward writes the MLP's upstream over it
  const int32_t* expert_idx; // [T, k]
  const int32_t* slot;       // [T, k]
  const float* weight;       // [T, k]
  const int32_t* offset;     // [E+1]
  bf16* out;                 // [T, d] forward output
  float* coef;               // [T, 2] coefficients (forward out, backward in)
  float* coef_out;           // [T, 2] the caller's copy (forward), or null
  const bf16* dout;          // [T, d] backward upstream
  float* dw;                 // [T, k] gate-weight gradient
  float* dlc;                // [T, 2] coefficient logit gradient, or null (no coef_w)
  float* cw_part;            // [chunks, 2, d] partial dW_c
  float* cb_part;            // [chunks, 2] partial db_c
  float* dcoef_w;            // [2, d] or null
  float* dcoef_b;            // [2] or null
  int64_t T;
  int32_t d, k;
};
int residual_coef_chunks(int64_t T);
hipError_t launch_residual_offsets(int32_t* off, int64_t T, hipStream_t s);
hipError_t launch_residual_combine(const ResidualArgs& a, hipStream_t s);
hipError_t launch_residual_combine_backward(const ResidualArgs& a, hipStream_t s);
hipError_t launch_coef_wgrad(const ResidualArgs& a, hipStream_t s);

// ---------------------------------------------------------------- small-batch forward
// The whole forward in one persistent kernel for up to kDecodeMaxTokens
// tokens (bf16, d and h multiples of 128, inference: no pre-activation kept).
constexpr int kDecodeMaxTokens = 256;
constexpr int kDecodeMaxSlices = 16;
// Index (32-bit words) of the status word in the small-batch kernel's barrier
// region: 0 after a launch whose grid barriers all completed, 1 if a wait ran
// out.
constexpr int kDecodeStatusWord = 16 * 32 + 32;
struct DecodeArgs {
  const bf16* x;            // [T, d]
  const bf16* w_router;     // [E, d] (unused with logits_in)
  const float* b_router;    // [E] or null
  const float* logits_in;   // [T, E] or null
  float* logits;            // [T, E]: the logits used (caller's or workspace)
  const bf16* w1;           // [E, n1, d], n1 = h (or d for a single Linear)
  const bf16* b1;           // [E, n1] or null
  const bf16* w2;           // [E, d, h] or null
  int32_t w_packed;         // w1 and w2 in the packed layout
  const bf16* b2;           // [E, d] or null
  bf16* out;                // [T, d]
  float* gate_loss;
  int32_t* expert_count;    // [E]
  int32_t* expert_offset;   // [E+1]
  int32_t* expert_idx;      // [T, k]
  int32_t* slot;            // [T, k]
  float* weight;            // [T, k]
  bf16* x_disp;             // [rows, d]
  bf16* h_disp;             // [rows, h]
  bf16* y_disp;             // [rows, d]
  float* prob;              // [T, E] softmax probabilities (BALANCE loss)
  float* part;              // [kDecodeMaxSlices, T, E] partial router products
  unsigned* bar;            // [1024] grid-barrier counters and status (zeroed per call)
  int64_t C;                // capacity, < 0 = none
  int32_t T, d, h, E, k, normalize, loss_kind, act;
  int32_t ks;               // K slices of the router product (set by launch_decode)
};
bool decode_fits(int64_t T, int d, int h, int E, int k, int dtype);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

// Zero fill of n bytes (a kernel, so that it can sit in a captured graph).
hipError_t launch_zero_bytes(void* p, size_t n, hipStream_t s);

}  // namespace moe
