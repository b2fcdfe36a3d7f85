// Gate of the MoE layer: router GEMM, softmax, top-k, capacity slots,
// expert counts and gate_loss, as three kernels: the gate proper, a scan over
// tiles, and a slot fix-up.
//
// What is computed ("MoE混合专家架构：大模型高效推理的智能调度原理" §3.1,
// MoELayer Steps 1-3; "deepspeed.moe 模块" overview §3.1 steps 1 and 5;
// the DeepSeek-MoE fine-tuning article ch.1 pseudocode and capacity row):
//   logits = x · W_r^T (+ b_r);  p = softmax over the experts;
//   top-k experts by (logit desc, index asc);  weight = p of the choice
//   (optionally renormalised over the k);
//   slot of claim (t, j) = rank of t among the choice-j claims of expert e,
//   plus (for j = 1) the total choice-0 demand of e; dropped if >= C.
//
// Design (gfx950):
//  * Gate kernel: one workgroup (4 waves) per tile of 64 tokens (32 when
//    E > 128); tiles never wait for one another.
//  * Router GEMM on MFMA v_mfma_f32_16x16x32_bf16 with experts on the MFMA
//    row side and tokens on the column side: a lane ends up holding 4
//    consecutive experts of one token, and a token's E logits sit in the 4
//    lanes {n, n+16, n+32, n+48}.  The hidden dimension is split over the 4
//    waves in 128-wide steps (each lane streams 64 contiguous bytes of its x
//    row per step; the four lane quarters cover 256 contiguous bytes) and the
//    partial logits are summed through LDS in a fixed order.
//  * Softmax and top-k are per-lane scans plus two xor-shuffles; ties go to
//    the lower index because every comparison is (value, index).
//  * Ranks inside the tile come from an LDS scan; each tile writes its
//    per-(choice, expert) counts and softmax column sums.
//  * Scan kernel: one workgroup per (choice, expert) column turns the
//    column's tile counts into exclusive prefixes (tile order) and its total
//    demand, and sums the column's probability mass in a fixed order, so the
//    results are bit-identical run to run.  (A single-pass decoupled
//    look-back chained one cross-XCD load per tile and took ~4x longer.)
//  * Fix-up kernel: slot = tile prefix + rank (+ choice-0 demand for
//    choice 1), dropped at or past the capacity; its last workgroup forms
//    the expert counts, offsets and the loss.  Kernel boundaries order all of
//    this, so no kernel waits on another workgroup.
//  * Random gate options (seeded, Philox4x32-10; reading R15): jitter
//    multiplies the x fragments by their factors just before the router's
//    MFMAs; RSample and second-expert sampling add Gumbel draws to the
//    selection keys only; Random Token Selection re-picks the kept claims of
//    an over-capacity expert in a kernel of its own after the fix-up.
#include <math.h>

#include "moe_internal.h"
#include "philox.h"

namespace moe {
namespace {

enum { MODE_LOGITS_IN = 0, MODE_BF16 = 1, MODE_F32 = 2, MODE_BF16_DMA = 3 };


__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Keep the better of (v, i) and the lane `mask` away: larger value, then
// lower index.
__device__ __forceinline__ void merge_best(float& v, int& i, int mask) {
  const float ov = __shfl_xor(v, mask);
  const int oi = __shfl_xor(i, mask);
  const bool take = (ov > v) | ((ov == v) & (oi < i));
  v = take ? ov : v;
  i = take ? oi : i;
}

// Router GEMM K chunk staged in LDS per step: 256 for up to 64 experts, 128
// for 128, 64 for 256, so that the double-buffered weight chunk stays at
// 64 KB at most; a long chunk keeps more bytes in flight per barrier.
template <int EP>
constexpr int gate_kc() { return EP <= 64 ? 256 : EP <= 128 ? 128 : 64; }

// s_waitcnt vmcnt(N): wait until at most N vector-memory loads of this wave
// are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt 6:4
// and lgkmcnt 11:8 at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Inclusive sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15) in a
// fixed order; lane 16r+15 ends with the row's total.
__device__ __forceinline__ float row_sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));  // row_shr:1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));  // row_shr:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));  // row_shr:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));  // row_shr:8
  return v;
}

// Router product staged by LDS-DMA (bf16, d a multiple of KC): per 64-token
// tile, the K dimension in steps of KC; each step's operands (64 token rows,
// then EP weight rows, KCB bytes of each) go from global memory straight
// into one of NS LDS stages, NS - 1 steps ahead of their use, so that a
// workgroup keeps (NS - 1) * STAGE bytes in flight without holding them in
// registers.  Chunk c of stage row r sits in slot c ^ swz(r), so the 16 rows
// that one fragment read touches fall in distinct bank groups.
template <int EP>
struct GateDma {
  static constexpr int KCB = EP <= 64 ? 256 : 128;   // bytes of a row per step
  static constexpr int KC = KCB / 2;                  // K elements per step
  static constexpr int CPR = KCB / 16;                // 16-byte chunks per row
  static constexpr int ROWS = 64 + EP;
  static constexpr int STAGE = ROWS * KCB;
  static constexpr int NS = (144 * 1024) / STAGE < 8 ? (144 * 1024) / STAGE : 8;   // stages in the ring
  static constexpr int RPI = 1024 / KCB;              // rows per 1 KB load
  static constexpr int LPW = ROWS * KCB / 1024 / 4;   // loads per wave and step
  static_assert(ROWS * KCB % 4096 == 0 && 64 % RPI == 0, "loads must split evenly over the waves");
  static_assert(NS >= 3 && LPW * (NS - 2) < 64, "ring depth");
  __device__ static __forceinline__ int swz(int r) { return CPR == 16 ? (r & 15) : ((r >> 1) & 7); }
};

// Wait until at most `later` steps' loads (LPW each) issued after the one
// needed next are still outstanding.
template <int LPW, int MAXL>
__device__ __forceinline__ void wait_steps(int later) {
  if constexpr (MAXL <= 0) {
    wait_vm<0>();
  } else {
    if (later >= MAXL) wait_vm<LPW * MAXL>();
    else wait_steps<LPW, MAXL - 1>(later);
  }
}

template <int EP>
constexpr bool gate_dma_fits(int d) { return d > 0 && (d * 2) % GateDma<EP>::KCB == 0; }

// The router reads x * ((1 - eps) + 2 eps u), eps = 0.01, each product and
// sum rounded once in fp32, then stored as bf16 (jitter option): the 8 values
// at K positions kk .. kk+7 of token tx.
__device__ __forceinline__ void jitter8(const GateArgs& a, bf16x8& xv, int64_t tx, int kk) {
  if (tx < a.T && kk < a.d) {
    const uint64_t n0 = (uint64_t)tx * a.d + kk;   // a multiple of 8
    const uint4 w0 = philox_block(a.seed_lo, a.seed_hi, kStreamJitter, n0 >> 2);
    const uint4 w1 = philox_block(a.seed_lo, a.seed_hi, kStreamJitter, (n0 >> 2) + 1);
    const uint32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float f = __fadd_rn(0.99f, __fmul_rn(0.02f, philox_uniform(wv[j])));
      xv[j] = static_cast<bf16>(__fmul_rn(static_cast<float>(xv[j]), f));
    }
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gate_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One LDS-DMA load (16 bytes per lane, lane i's bytes at dst + 16 i).  A plain
// function: the host compilation pass cannot instantiate a template that
// names the target builtin.
__device__ __forceinline__ void gate_dma_load1(__amdgpu_buffer_rsrc_t r, unsigned char* dst, uint32_t voff,
                                               uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

// This wave's loads of one K step into one stage: load j of wave w covers
// stage rows (w * LPW + j) * RPI .. + RPI - 1, token rows (from rx) below 64,
// weight rows (from rw) above; voff holds each load's per-lane source offset
// and the step adds step * KCB through the scalar offset.
template <int EP>
__device__ __forceinline__ void gate_dma_issue(unsigned char* smem, __amdgpu_buffer_rsrc_t rx,
                                               __amdgpu_buffer_rsrc_t rw, const uint32_t* voff, int wv, int step,
                                               int stage) {
  using DM = GateDma<EP>;
#pragma unroll
  for (int j = 0; j < DM::LPW; ++j) {
    const int g = wv * DM::LPW + j;
    unsigned char* dst = smem + stage * DM::STAGE + g * 1024;
    gate_dma_load1(g * DM::RPI < 64 ? rx : rw, dst, voff[j], (uint32_t)(step * DM::KCB));
  }
}

// Fragments of one K step of the router product: for lane quarter q, the
// token row's and the NET weight rows' chunks q*NSUB + i (i < NSUB), the same
// order on both operands.
template <int EP>
struct GateFrags {
  bf16x8 x[GateDma<EP>::CPR / 4];
  bf16x8 w[GateDma<EP>::CPR / 4][EP / 16];
};

template <int EP>
__device__ __forceinline__ void gate_read_frags(const unsigned char* sb, int xr, int n, int q, GateFrags<EP>& f) {
  using DM = GateDma<EP>;
  constexpr int NSUB = DM::CPR / 4;
#pragma unroll
  for (int i = 0; i < NSUB; ++i) {
    const int c = q * NSUB + i;
    f.x[i] = *reinterpret_cast<const bf16x8*>(sb + xr * DM::KCB + ((c ^ DM::swz(xr)) * 16));
#pragma unroll
    for (int et = 0; et < EP / 16; ++et) {
      const int wr = 64 + et * 16 + n;
      f.w[i][et] = *reinterpret_cast<const bf16x8*>(sb + wr * DM::KCB + ((c ^ DM::swz(wr)) * 16));
    }
  }
}

template <int EP, bool JIT>
__device__ __forceinline__ void gate_mfma_step(const GateArgs& a, GateFrags<EP>& f, int64_t tx, int ks, int q,
                                               f32x4 (&acc)[EP / 16]) {
  using DM = GateDma<EP>;
  constexpr int NSUB = DM::CPR / 4;
#pragma unroll
  for (int i = 0; i < NSUB; ++i) {
    if constexpr (JIT) jitter8(a, f.x[i], tx, ks * DM::KC + (q * NSUB + i) * 8);
#pragma unroll
    for (int et = 0; et < EP / 16; ++et)
      acc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.w[i][et], f.x[i], acc[et], 0, 0, 0);
  }
}

// The router product of one 64-token tile on the LDS-DMA stages: this
// wave's 16 tokens (lane n) against all EP experts, acc[et] holding experts
// et*16 + q*4 .. +3 for lane quarter q.  The fragments of step ks+1 are read
// while the MFMAs of step ks run (two register sets, the loop unrolled by
// two), so step ks+1's stage must have landed by the barrier of step ks.
template <int EP, bool JIT>
__device__ __forceinline__ void gate_dma_product(const GateArgs& a, unsigned char* smem, int64_t t0,
                                                 f32x4 (&acc)[EP / 16]) {
  using DM = GateDma<EP>;
  constexpr int NET = EP / 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, q = lane >> 4;
  const int d = a.d;
  const int64_t T = a.T;
  const int nsteps = d / DM::KC;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int64_t rows_valid = T - t0 < 64 ? T - t0 : 64;
  const int64_t tx = t0 + wave * 16 + n;
  const __amdgpu_buffer_rsrc_t rx = gate_rsrc(static_cast<const bf16*>(a.x) + t0 * d, (uint32_t)(rows_valid * d * 2));
  const __amdgpu_buffer_rsrc_t rw = gate_rsrc(a.w_router, (uint32_t)((int64_t)a.E * d * 2));
  // per-lane source offset of each of this wave's loads
  uint32_t voff[DM::LPW];
#pragma unroll
  for (int j = 0; j < DM::LPW; ++j) {
    const int g = wv * DM::LPW + j;
    const int row = g * DM::RPI + lane / DM::CPR;
    const int c = (lane % DM::CPR) ^ DM::swz(row);
    const int src_row = row < 64 ? row : row - 64;
    voff[j] = (uint32_t)src_row * (uint32_t)(d * 2) + (uint32_t)c * 16u;
  }
#pragma unroll
  for (int et = 0; et < NET; ++et) acc[et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < DM::NS - 1; ++st)
    if (st < nsteps) gate_dma_issue<EP>(smem, rx, rw, voff, wv, st, st);
  const int xr = wave * 16 + n;
  GateFrags<EP> fa, fb;
  // step 0's stage, then its fragments
  wait_steps<DM::LPW, DM::NS - 2>(nsteps - 1);
  __syncthreads();
  gate_read_frags<EP>(smem, xr, n, q, fa);
  // One step: make step ks+1's stage visible (own loads landed, then the
  // barrier, which also frees the stage read during step ks-1 for the loads
  // of step ks+NS-1), read its fragments into `nx`, then step ks's MFMAs on `cu`.
  auto step = [&](int ks, GateFrags<EP>& cu, GateFrags<EP>& nx) {
    if (ks + 1 < nsteps) {
      wait_steps<DM::LPW, DM::NS - 3>(nsteps - 2 - ks);
      __syncthreads();
      if (ks + DM::NS - 1 < nsteps)
        gate_dma_issue<EP>(smem, rx, rw, voff, wv, ks + DM::NS - 1, (ks + DM::NS - 1) % DM::NS);
      gate_read_frags<EP>(smem + ((ks + 1) % DM::NS) * DM::STAGE, xr, n, q, nx);
    }
    gate_mfma_step<EP, JIT>(a, cu, tx, ks, q, acc);
  };
  int ks = 0;
  for (; ks + 1 < nsteps; ks += 2) {
    step(ks, fa, fb);
    step(ks + 1, fb, fa);
  }
  if (ks < nsteps) step(ks, fa, fb);
}

// ---------------------------------------------------------------------------
// Gate for 65..128 experts (bf16 router, d a multiple of 64): 256-token tiles
// on v_mfma_f32_32x32x16_bf16.  At these expert counts the router product
// is no longer small next to the token stream (2E flops per token element),
// and the 16x16 layout above reads every weight fragment once per 16 tokens
// from LDS; here each wave owns 64 tokens (two 32-token blocks) against all
// 128 experts (four 32-expert blocks), which halves the LDS bytes per flop,
// and one tile per workgroup streams the router weight from L2 once per 256
// tokens.  Stage: 256 token rows then 128 weight rows of 128 bytes (one
// 64-wide K step), three stages.  MFMA layouts: A = 32 experts x 16 K
// (lane l: expert row l % 32, K half l / 32), B = 32 tokens x 16 K; the
// 16 results of lane l are experts 8 (r / 4) + 4 (l / 32) + r % 4 of the
// block for token l % 32, so a token's 128 logits sit in lanes l and l ^ 32.
namespace gbig {
constexpr int EP = 128, TT = 256, KCB = 128, KC = 64;
constexpr int ROWS = TT + EP;
constexpr int STAGE = ROWS * KCB;        // 48 KB
constexpr int NS = 3;
constexpr int RPI = 1024 / KCB;          // rows per 1 KB load
constexpr int LPW = ROWS * KCB / 1024 / 4;
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
}  // namespace gbig

// The stage loads of one K step for this wave (rows below TT from rx, the
// weight rows from rw).
__device__ __forceinline__ void gate_big_issue(unsigned char* smem, __amdgpu_buffer_rsrc_t rx,
                                               __amdgpu_buffer_rsrc_t rw, const uint32_t* voff, int wv, int step,
                                               int stage) {
  using namespace gbig;
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int g = wv * LPW + j;
    gate_dma_load1(g * RPI < TT ? rx : rw, smem + stage * STAGE + g * 1024, voff[j], (uint32_t)(step * KCB));
  }
}

__device__ __forceinline__ void gate_big_product(const GateArgs& a, unsigned char* smem, int64_t t0,
                                                 f32x16 (&acc)[2][4]) {
  using namespace gbig;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int d = a.d;
  const int64_t T = a.T;
  const int nsteps = d / KC;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int64_t rows_valid = T - t0 < TT ? T - t0 : TT;
  const __amdgpu_buffer_rsrc_t rx = gate_rsrc(static_cast<const bf16*>(a.x) + t0 * d, (uint32_t)(rows_valid * d * 2));
  const __amdgpu_buffer_rsrc_t rw = gate_rsrc(a.w_router, (uint32_t)((int64_t)a.E * d * 2));
  uint32_t voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int g = wv * LPW + j;
    const int row = g * RPI + lane / 8;
    const int c = (lane % 8) ^ swz(row);
    const int src_row = row < TT ? row : row - TT;
    voff[j] = (uint32_t)src_row * (uint32_t)(d * 2) + (uint32_t)c * 16u;
  }
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tb][eb][r] = 0.f;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nsteps) gate_big_issue(smem, rx, rw, voff, wv, st, st);
  for (int ks = 0; ks < nsteps; ++ks) {
    wait_steps<LPW, NS - 2>(nsteps - 1 - ks);
    __syncthreads();   // every wave's loads of this stage have landed; the stage read last step is free
    if (ks + NS - 1 < nsteps) gate_big_issue(smem, rx, rw, voff, wv, ks + NS - 1, (ks + NS - 1) % NS);
    const unsigned char* sb = smem + (ks % NS) * STAGE;
    // sub-step i covers, for lane half h, chunk h*4 + i of each row (the same
    // order on both operands)
    bf16x8 xf[4][2], wf[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = h * 4 + i;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int xr = wave * 64 + tb * 32 + l32;
        xf[i][tb] = *reinterpret_cast<const bf16x8*>(sb + xr * KCB + ((c ^ swz(xr)) * 16));
      }
#pragma unroll
      for (int eb = 0; eb < 4; ++eb) {
        const int wr = TT + eb * 32 + l32;
        wf[i][eb] = *reinterpret_cast<const bf16x8*>(sb + wr * KCB + ((c ^ swz(wr)) * 16));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int eb = 0; eb < 4; ++eb)
          acc[tb][eb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i][eb], xf[i][tb], acc[tb][eb], 0, 0, 0);
    }
  }
}

// The gate kernel of this layout (the deterministic gate; the random
// options take the 16x16 kernel).
__global__ __launch_bounds__(256) void gate_big_kernel(GateArgs a) {
  using namespace gbig;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* s_wc = reinterpret_cast<int*>(smem + NS * STAGE);        // [4 waves][2 choices][EP]
  float* s_me = reinterpret_cast<float*>(s_wc + 4 * 2 * EP);    // [4 waves][2 lane rows][EP]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int E = a.E, K = a.k, KE = a.k * a.E;
  const int64_t T = a.T;
  const int tile = blockIdx.x;
  const int64_t t0 = (int64_t)tile * TT;
  for (int i = tid; i < 4 * 2 * EP; i += 256) s_wc[i] = 0;

  // expert of result r in block eb for this lane
  auto expert = [&](int eb, int r) { return eb * 32 + 8 * (r >> 2) + 4 * h + (r & 3); };
  f32x16 acc[2][4];
  if (a.logits_in) {
    // given logits, in the product's layout (so that both paths share the
    // selection below bit for bit)
    __syncthreads();
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int64_t t = t0 + wave * 64 + tb * 32 + l32;
#pragma unroll
      for (int eb = 0; eb < 4; ++eb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = expert(eb, r);
          acc[tb][eb][r] = (t < T && e < E) ? a.logits_in[t * E + e] : 0.f;
        }
    }
  } else {
    gate_big_product(a, smem, t0, acc);
  }
  const float* br = a.logits_in ? nullptr : a.b_router;
  constexpr float kLog2e = 1.4426950408889634f;
  int sel0[2], sel1[2];
  float pr0[2], pr1[2], mxs[2], inv[2];
  bool tv[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int64_t t = t0 + wave * 64 + tb * 32 + l32;
    tv[tb] = t < T;
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = expert(eb, r);
        float v = acc[tb][eb][r];
        if (br) v += br[e < E ? e : E - 1];
        acc[tb][eb][r] = e < E ? v : -INFINITY;
      }
    if (a.logits_out && tv[tb]) {
#pragma unroll
      for (int eb = 0; eb < 4; ++eb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = expert(eb, r);
          if (e < E) a.logits_out[t * E + e] = acc[tb][eb][r];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[tb][eb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float sum = 0.f;
    // top-1 / top-2 by (value desc, index asc); padding experts have key
    // -inf and an index past the running one's start (E), so never win
    float v0 = -INFINITY, v1 = -INFINITY;
    int i0 = E, i1 = E;
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = expert(eb, r);
        const float l = acc[tb][eb][r];
        sum += e < E ? __builtin_amdgcn_exp2f((l - mx) * kLog2e) : 0.f;
        const float key = l != l ? -INFINITY : l;
        const bool better = (key > v0) | ((key == v0) & (e < i0));
        v0 = better ? key : v0;
        i0 = better ? e : i0;
      }
    sum += __shfl_xor(sum, 32);
    merge_best(v0, i0, 32);
    if (K == 2) {
#pragma unroll
      for (int eb = 0; eb < 4; ++eb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = expert(eb, r);
          const float l = acc[tb][eb][r];
          const float key = l != l ? -INFINITY : l;
          const bool better = (e != i0) & ((key > v1) | ((key == v1) & (e < i1)));
          v1 = better ? key : v1;
          i1 = better ? e : i1;
        }
      merge_best(v1, i1, 32);
    }
    mxs[tb] = mx;
    inv[tb] = 1.f / sum;
    float p0 = __builtin_amdgcn_exp2f((v0 - mx) * kLog2e) * inv[tb];
    float p1 = (K == 2) ? __builtin_amdgcn_exp2f((v1 - mx) * kLog2e) * inv[tb] : 0.f;
    if (a.normalize) {
      const float s2 = p0 + p1;
      p0 = p0 / s2;
      p1 = p1 / s2;
    }
    pr0[tb] = p0;
    pr1[tb] = p1;
    sel0[tb] = tv[tb] ? i0 : -1;
    sel1[tb] = (tv[tb] && K == 2) ? i1 : -1;
  }
  // Ranks inside the tile, part 1: among this wave's 64 tokens (block 0's
  // 32, then block 1's), the earlier ones with the same expert, by readlane;
  // and this wave's claims per (choice, expert) in LDS.
  int r0[2] = {0, 0}, r1[2] = {0, 0};
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const int a0 = __builtin_amdgcn_readlane(sel0[0], m), b0 = __builtin_amdgcn_readlane(sel0[1], m);
    const int a1 = __builtin_amdgcn_readlane(sel1[0], m), b1 = __builtin_amdgcn_readlane(sel1[1], m);
    r0[0] += (m < l32) & (a0 == sel0[0]);
    r0[1] += (a0 == sel0[1]) + ((m < l32) & (b0 == sel0[1]));
    r1[0] += (m < l32) & (a1 == sel1[0]);
    r1[1] += (a1 == sel1[1]) + ((m < l32) & (b1 == sel1[1]));
  }
  if (h == 0) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      if (!tv[tb]) continue;
      const int64_t t = t0 + wave * 64 + tb * 32 + l32;
      atomicAdd(&s_wc[(wave * 2) * EP + sel0[tb]], 1);
      a.expert_idx[t * K] = sel0[tb];
      a.weight[t * K] = pr0[tb];
      if (K == 2) {
        atomicAdd(&s_wc[(wave * 2 + 1) * EP + sel1[tb]], 1);
        a.expert_idx[t * K + 1] = sel1[tb];
        a.weight[t * K + 1] = pr1[tb];
      }
    }
  }
  // per-tile column sums of p for the balance loss: a lane's two tokens,
  // then each 16-lane DPP row in a fixed order; rows, lane halves and waves
  // are added below
#pragma unroll
  for (int eb = 0; eb < 4; ++eb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = expert(eb, r);
      const float q0 = (tv[0] && e < E) ? __builtin_amdgcn_exp2f((acc[0][eb][r] - mxs[0]) * kLog2e) * inv[0] : 0.f;
      const float q1 = (tv[1] && e < E) ? __builtin_amdgcn_exp2f((acc[1][eb][r] - mxs[1]) * kLog2e) * inv[1] : 0.f;
      const float v = row_sum16(q0 + q1);
      if ((lane & 15) == 15) s_me[(wave * 2 + ((lane >> 4) & 1)) * EP + e] = v;
    }
  __syncthreads();
  // part 2: plus the same claims of the earlier waves
  if (h == 0) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      if (!tv[tb]) continue;
      const int64_t t = t0 + wave * 64 + tb * 32 + l32;
      int q0 = r0[tb], q1 = r1[tb];
      for (int w = 0; w < wave; ++w) {
        q0 += s_wc[(w * 2) * EP + sel0[tb]];
        if (K == 2) q1 += s_wc[(w * 2 + 1) * EP + sel1[tb]];
      }
      a.slot[t * K] = q0;
      if (K == 2) a.slot[t * K + 1] = q1;
    }
  }
  for (int e = tid; e < E; e += 256) {
    float v = 0.f;
    for (int g = 0; g < 8; ++g) v += s_me[g * EP + e];
    a.me_tile[(int64_t)tile * E + e] = v;
  }
  for (int c = tid; c < KE; c += 256) {
    const int j = c / E, e = c - j * E;
    int cnt = 0;
    for (int w = 0; w < 4; ++w) cnt += s_wc[(w * 2 + j) * EP + e];
    a.tile_cnt[(int64_t)c * a.num_tiles + tile] = cnt;
  }
  // the scan kernel's arrival counter starts at zero (stored after this
  // wave's LDS-DMA loads, which vmcnt counts in order)
  if (tile == 0 && tid == 0) *a.sync = 0u;
}

// RND: the seeded random gate options may be on (jitter, RSample, sampled
// second expert); without it their code is compiled out, which keeps the
// kernel small enough for the instruction cache.
template <int EP, int TG, int MODE, bool RND>
__global__ __launch_bounds__(256) void gate_kernel(GateArgs a) {
  constexpr int NET = EP / 16;   // 16-expert MFMA row tiles
  constexpr int TT = TG * 16;    // tokens per tile
  constexpr int KC = gate_kc<EP>();
  constexpr int CPR = KC / 8;    // 16-byte chunks per weight row of a K chunk
  using DM = GateDma<EP>;
  constexpr size_t W_BYTES = (MODE == MODE_BF16) ? size_t(2) * EP * KC * 2
                             : (MODE == MODE_BF16_DMA) ? size_t(DM::NS) * DM::STAGE : 0;
  static_assert(TG == 4, "four waves of 16 tokens: one token per lane in the rank pass");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* s_wc = reinterpret_cast<int*>(smem + W_BYTES);                 // [TG][2][EP] claims per wave
  float* s_me = reinterpret_cast<float*>(s_wc + TG * 2 * EP);         // [TG][EP]
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, n = lane & 15, q = lane >> 4;
  const int E = a.E, K = a.k, KE = a.k * a.E;
  const int64_t T = a.T;

  const int tile = blockIdx.x;
  const int64_t t0 = (int64_t)tile * TT;
  for (int i = tid; i < TG * 2 * EP; i += 256) s_wc[i] = 0;
  __syncthreads();

  // ------------------------------------------------------------ logits
  // lg[et][r] = logit of expert et*16 + q*4 + r for token t0 + wave*16 + n
  float lg[NET][4];
  const int64_t tx = t0 + wave * 16 + n;
  if constexpr (MODE == MODE_BF16_DMA) {
    // Each wave computes its own 16 tokens over the whole hidden dimension
    // (no cross-wave reduction); all four share the weight rows of a stage.
    f32x4 acc[NET];
    if (RND && a.jitter) gate_dma_product<EP, RND>(a, smem, t0, acc);
    else gate_dma_product<EP, false>(a, smem, t0, acc);
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) lg[et][r] = acc[et][r];
  } else if constexpr (MODE == MODE_BF16) {
    // Any d (a multiple of 8): the router weight streams through LDS in K
    // chunks of KC (double-buffered, register-staged), the x fragments come
    // straight from global memory one K step ahead.
    const bf16* x = static_cast<const bf16*>(a.x);
    const bf16* w = static_cast<const bf16*>(a.w_router);
    const int d = a.d;
    const int nsteps = (d + KC - 1) / KC;
    constexpr int WL = EP * CPR / 256;   // weight chunk loads per thread and step
    const bf16x8 zero8 = {};
    auto load_w = [&](int ks, bf16x8 (&wr)[WL]) {
#pragma unroll
      for (int j = 0; j < WL; ++j) {
        const int c = tid + 256 * j;
        const int row = c / CPR, col = c % CPR;
        const int kk = ks * KC + col * 8;
        wr[j] = (row < E && kk < d) ? ld_bf16x8(w + (int64_t)row * d + kk) : zero8;
      }
    };
    auto store_w = [&](int buf, const bf16x8 (&wr)[WL]) {
      unsigned char* base = smem + (size_t)buf * EP * KC * 2;
#pragma unroll
      for (int j = 0; j < WL; ++j) {
        const int c = tid + 256 * j;
        const int row = c / CPR, col = c % CPR;
        *reinterpret_cast<bf16x8*>(base + (size_t)row * KC * 2 + ((col ^ (row & 15)) % CPR) * 16) = wr[j];
      }
    };
    auto load_x = [&](int ks, bf16x8 (&xb)[KC / 32]) {
#pragma unroll
      for (int i = 0; i < KC / 32; ++i) {
        const int kk = ks * KC + q * (KC / 4) + i * 8;
        xb[i] = (tx < T && kk < d) ? ld_bf16x8(x + tx * d + kk) : zero8;
      }
    };
    f32x4 acc[NET];
#pragma unroll
    for (int et = 0; et < NET; ++et) acc[et] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 wr[WL], xb[KC / 32], xn[KC / 32];
    load_w(0, wr);
    load_x(0, xb);
    store_w(0, wr);
    __syncthreads();
    for (int ks = 0; ks < nsteps; ++ks) {
      const bool more = ks + 1 < nsteps;
      if (more) {
        load_w(ks + 1, wr);
        load_x(ks + 1, xn);
      }
      if (RND && a.jitter) {
#pragma unroll
        for (int i = 0; i < KC / 32; ++i) jitter8(a, xb[i], tx, ks * KC + q * (KC / 4) + i * 8);
      }
      const unsigned char* wb = smem + (size_t)(ks & 1) * EP * KC * 2;
      // fragment i covers K values q*(KC/4) + 8i .. +7 of the chunk for lane
      // quarter q (the same order on both operands)
#pragma unroll
      for (int et = 0; et < NET; ++et) {
        const int row = et * 16 + n;
#pragma unroll
        for (int i = 0; i < KC / 32; ++i) {
          const int col = q * (KC / 32) + i;
          const bf16x8 wa = *reinterpret_cast<const bf16x8*>(wb + (size_t)row * KC * 2 + ((col ^ (row & 15)) % CPR) * 16);
          acc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xb[i], acc[et], 0, 0, 0);
        }
      }
      if (more) {
        store_w((ks + 1) & 1, wr);
#pragma unroll
        for (int i = 0; i < KC / 32; ++i) xb[i] = xn[i];
      }
      __syncthreads();
    }
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) lg[et][r] = acc[et][r];
  } else if constexpr (MODE == MODE_F32) {
    const float* x = static_cast<const float*>(a.x);
    const float* w = static_cast<const float*>(a.w_router);
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = et * 16 + q * 4 + r;
        float s = 0.f;
        if (tx < T && e < E)
          for (int kk = 0; kk < a.d; ++kk) s = fmaf(x[tx * a.d + kk], w[(int64_t)e * a.d + kk], s);
        lg[et][r] = s;
      }
  } else {
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = et * 16 + q * 4 + r;
        lg[et][r] = (tx < T && e < E) ? a.logits_in[tx * E + e] : 0.f;
      }
  }

  // ------------------------------------------------------------ softmax, top-k
  const int64_t t = tx;
  const bool tv = t < T;
  const float* br = MODE != MODE_LOGITS_IN ? a.b_router : nullptr;
  if (br) {
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = et * 16 + q * 4 + r;
        lg[et][r] += br[e < E ? e : E - 1];
      }
  }
#pragma unroll
  for (int et = 0; et < NET; ++et)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (et * 16 + q * 4 + r >= E) lg[et][r] = -INFINITY;
  if (a.logits_out && tv) {
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = et * 16 + q * 4 + r;
        if (e < E) a.logits_out[t * E + e] = lg[et][r];
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int et = 0; et < NET; ++et)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, lg[et][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // exp(l - mx) once per logit, as 2^((l - mx) log2 e); padding experts give 0
  constexpr float kLog2e = 1.4426950408889634f;
  float ex[NET][4];
  float sum = 0.f;
#pragma unroll
  for (int et = 0; et < NET; ++et)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ex[et][r] = (et * 16 + q * 4 + r < E) ? __builtin_amdgcn_exp2f((lg[et][r] - mx) * kLog2e) : 0.f;
      sum += ex[et][r];
    }
  sum += __shfl_xor(sum, 16);
  sum += __shfl_xor(sum, 32);
  const float inv = 1.f / sum;

  // top-1, by (value desc, index asc).  The selection key of a NaN logit
  // is -inf and the running index starts past every expert, so that even a
  // token whose logits are all -inf or NaN (outside the contract) gets a
  // valid expert (the lowest index) and no later step indexes out of range.
  // With RSample (k = 1) the top-1 key is fp32(logit + g), g a Gumbel draw
  // of stream 1 at t*E + e; with second-expert sampling (k = 2) the top-2
  // key is the same with stream 2.  The weights use the clean logits.
  const bool noisy0 = RND && a.rsample != 0, noisy1 = RND && a.second != 0 && K == 2;
  auto gumbel = [&](uint32_t stream, int e) {
    const uint32_t w = philox_draw(a.seed_lo, a.seed_hi, stream, (uint64_t)t * E + e);
    return -logf(-logf(philox_uniform(w)));
  };
  // Padding experts (e >= E) have key -inf and an index past the running
  // one's start (E), so they never win; the comparisons are selects, not
  // branches.
  float v0 = -INFINITY;
  int i0 = E;
#pragma unroll
  for (int et = 0; et < NET; ++et)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = et * 16 + q * 4 + r;
      float key = lg[et][r] != lg[et][r] ? -INFINITY : lg[et][r];
      if (noisy0 && e < E) key = __fadd_rn(key, gumbel(kStreamRSample, e));
      const bool better = (key > v0) | ((key == v0) & (e < i0));
      v0 = better ? key : v0;
      i0 = better ? e : i0;
    }
  merge_best(v0, i0, 16);
  merge_best(v0, i0, 32);
  // top-2 (best other than the top-1)
  float v1 = -INFINITY;
  int i1 = E;
  if (K == 2) {
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = et * 16 + q * 4 + r;
        float key = lg[et][r] != lg[et][r] ? -INFINITY : lg[et][r];
        if (noisy1 && e < E) key = __fadd_rn(key, gumbel(kStreamSecond, e));
        const bool better = (e != i0) & ((key > v1) | ((key == v1) & (e < i1)));
        v1 = better ? key : v1;
        i1 = better ? e : i1;
      }
    merge_best(v1, i1, 16);
    merge_best(v1, i1, 32);
  }
  if (noisy0 || noisy1) {
    // a noisy key is not the logit: fetch the chosen experts' clean logits
    // from the lanes that hold them
    float o0 = -INFINITY, o1 = -INFINITY;
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = et * 16 + q * 4 + r;
        if (e == i0) o0 = lg[et][r];
        if (e == i1) o1 = lg[et][r];
      }
    o0 = fmaxf(o0, __shfl_xor(o0, 16));
    o0 = fmaxf(o0, __shfl_xor(o0, 32));
    o1 = fmaxf(o1, __shfl_xor(o1, 16));
    o1 = fmaxf(o1, __shfl_xor(o1, 32));
    if (noisy0) v0 = o0;
    if (noisy1) v1 = o1;
  }
  // the chosen probabilities, from the same exponential as the lane that
  // holds the expert
  float p0 = __builtin_amdgcn_exp2f((v0 - mx) * kLog2e) * inv;
  float p1 = (K == 2) ? __builtin_amdgcn_exp2f((v1 - mx) * kLog2e) * inv : 0.f;
  if (a.normalize) {
    const float s2 = p0 + p1;
    p0 = p0 / s2;
    p1 = p1 / s2;
  }
  // Ranks inside the tile, part 1: among this wave's 16 tokens, the earlier
  // ones with the same expert (each lane reads the other tokens' choices
  // with readlane), and this wave's claims per (choice, expert) in LDS.
  const int sel0 = tv ? i0 : -1, sel1 = (tv && K == 2) ? i1 : -1;
  int r0 = 0, r1 = 0;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int o0 = __builtin_amdgcn_readlane(sel0, m), o1 = __builtin_amdgcn_readlane(sel1, m);
    r0 += (m < n) & (o0 == sel0);
    r1 += (m < n) & (o1 == sel1);
  }
  if (q == 0 && tv) {
    atomicAdd(&s_wc[(wave * 2) * EP + i0], 1);
    if (K == 2) atomicAdd(&s_wc[(wave * 2 + 1) * EP + i1], 1);
    a.expert_idx[t * K] = i0;
    a.weight[t * K] = p0;
    if (K == 2) {
      a.expert_idx[t * K + 1] = i1;
      a.weight[t * K + 1] = p1;
    }
  }
  // per-tile column sums of p for the balance loss: the wave's 16 tokens by
  // a DPP row sum (fixed order), then the TG waves in order below
#pragma unroll
  for (int et = 0; et < NET; ++et)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = et * 16 + q * 4 + r;
      const float pe = row_sum16(tv ? ex[et][r] * inv : 0.f);
      if (n == 15 && e < EP) s_me[wave * EP + e] = pe;
    }
  __syncthreads();

  // ------------------------------------------------------------ ranks in the tile
  // part 2: plus the same claims of the earlier waves (tokens in tile order);
  // raw slot = rank inside the tile, the fix-up adds the tile prefix
  if (q == 0 && tv) {
    for (int w = 0; w < wave; ++w) {
      r0 += s_wc[(w * 2) * EP + i0];
      if (K == 2) r1 += s_wc[(w * 2 + 1) * EP + i1];
    }
    a.slot[t * K] = r0;
    if (K == 2) a.slot[t * K + 1] = r1;
  }
  for (int e = tid; e < E; e += 256) {
    float v = 0.f;
    for (int g = 0; g < TG; ++g) v += s_me[g * EP + e];
    a.me_tile[(int64_t)tile * E + e] = v;
  }
  for (int c = tid; c < KE; c += 256) {
    const int j = c / E, e = c - j * E;
    int cnt = 0;
    for (int w = 0; w < TG; ++w) cnt += s_wc[(w * 2 + j) * EP + e];
    a.tile_cnt[(int64_t)c * a.num_tiles + tile] = cnt;
  }
  // the scan kernel's arrival counter starts at zero (it runs after this
  // one; stored after this wave's LDS-DMA loads, which vmcnt counts in order)
  if (tile == 0 && tid == 0) *a.sync = 0u;
}

// Inclusive scan over a wavefront (fixed order).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Sum over a wavefront by a butterfly (fixed order; every lane gets it).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Inclusive scan over the workgroup's 256 threads in thread order.
__device__ __forceinline__ int block_incl_scan(int v, int* s_w) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_incl_scan(v);
  if (lane == 63) s_w[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += s_w[w];
  __syncthreads();
  return v + add;
}

// Sum over the workgroup's 256 threads: waves by butterflies, then the four
// wave sums in order (every thread gets it).
__device__ __forceinline__ double block_sum(double v, double* s_w) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) s_w[wave] = v;
  __syncthreads();
  const double r = ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];
  __syncthreads();
  return r;
}

// Expert counts (capacity applied per choice in order), offsets and the loss
// from the scan's demands and probability mass, by one workgroup; every sum
// runs in a fixed order.
__device__ void gate_counts_and_loss(const GateArgs& a) {
  __shared__ int s_wi[4];
  __shared__ double s_wd[4];
  const int tid = threadIdx.x;   // blockDim.x == 256 == MOE_MAX_EXPERTS_DEV
  const int E = a.E, K = a.k;
  const int64_t T = a.T;
  const int64_t C = a.C;
  const int d0 = tid < E ? a.demand[tid] : 0;
  const int d1 = (tid < E && K == 2) ? a.demand[E + tid] : 0;
  // loaded with the demand, not after the offsets' scan
  const double msum = (tid < E && a.loss_kind == LOSS_BALANCE && T > 0) ? a.me_sum[tid] : 0.0;
  int kept = 0;
  if (tid < E) {
    int64_t kp;
    if (C < 0) {
      kp = (int64_t)d0 + d1;
    } else {
      kp = d0 < C ? d0 : C;
      if (K == 2) {
        const int64_t room = C - d0;
        kp += room <= 0 ? 0 : (d1 < room ? d1 : room);
      }
    }
    kept = (int)kp;
    a.expert_count[tid] = kept;
  }
  const int incl = block_incl_scan(kept, s_wi);
  if (tid < E) a.expert_offset[tid] = incl - kept;
  if (tid == E - 1) a.expert_offset[E] = incl;
  double loss = 0.0;
  if (T > 0) {
    if (a.loss_kind == LOSS_BALANCE) {
      const double term = tid < E ? (msum / (double)T) * ((double)d0 / (double)T) : 0.0;
      loss = (double)E * block_sum(term, s_wd);
    } else {
      const double denom = (double)K * (double)T;
      const double u = tid < E ? (double)(d0 + d1) / denom : 0.0;
      const double mean = block_sum(u, s_wd) / (double)E;
      const double dv = tid < E ? (u - mean) * (u - mean) : 0.0;
      loss = sqrt(block_sum(dv, s_wd) / (double)E) + 1e-6;
    }
  }
  if (tid == 0) *a.gate_loss = (float)loss;
}

// Exclusive prefix over tiles of one (choice, expert) column, its total
// demand and (choice-0 columns) the expert's probability mass.  The last
// workgroup to finish forms the expert counts, offsets and the loss.
__global__ __launch_bounds__(256) void gate_scan_kernel(GateArgs a) {
  __shared__ int s_wi[4];
  __shared__ double s_wd[4];
  __shared__ int s_last;
  const int tid = threadIdx.x, c = blockIdx.x;
  const int E = a.E;
  const int nt = a.num_tiles;
  int32_t* col = a.tile_cnt + (int64_t)c * nt;
  // each thread owns a contiguous run of tiles
  const int per = (nt + 255) / 256;
  const int lo = min(nt, tid * per), hi = min(nt, lo + per);
  // the column's counts and (choice-0 columns) the expert's per-tile
  // probability sums are loaded together, before the scan's barriers
  // (the run's first count stays in a register for the prefix pass: up to
  // 256 tiles that is the whole run)
  const int first = lo < hi ? col[lo] : 0;
  int sum = first;
  for (int i = lo + 1; i < hi; ++i) sum += col[i];
  double m = 0.0;   // probability mass of expert c: runs in tile order, then a fixed tree
  if (c < E)
    for (int i = lo; i < hi; ++i) m += (double)a.me_tile[(int64_t)i * E + c];
  const int incl = block_incl_scan(sum, s_wi);
  int run = incl - sum;
  if (lo < hi) {
    col[lo] = run;
    run += first;
  }
  for (int i = lo + 1; i < hi; ++i) {
    const int v = col[i];
    col[i] = run;
    run += v;
  }
  if (tid == 255) a.demand[c] = incl;
  if (c < E) {
    m = block_sum(m, s_wd);
    if (tid == 0) a.me_sum[c] = m;
  }
  // arrival: every wave waits until its own stores have reached the L2 (a
  // workgroup barrier does not wait for another wave's stores), then one
  // thread's agent-scope release writes the L2 back and adds to the counter,
  // which the gate kernel zeroed
  wait_vm<0>();
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned old = __hip_atomic_fetch_add(a.sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  gate_counts_and_loss(a);
}

// Final slots: the rank inside the tile plus the column's prefix over earlier
// tiles; choice 1 also adds the expert's total choice-0 demand; a slot at or
// past the capacity is dropped.
__device__ __forceinline__ int32_t final_slot(const GateArgs& a, int64_t i) {
  const int tile_tokens = a.tile_tokens;
  const int k = a.k, E = a.E;
  const int j = (int)(i % k);
  const int64_t t = i / k;
  const int e = a.expert_idx[i];
  const int c = j * E + e;
  int64_t s = (int64_t)a.slot[i] + a.tile_cnt[(int64_t)c * a.num_tiles + t / tile_tokens];
  if (j == 1) s += a.demand[e];
  return (a.C >= 0 && s >= a.C) ? -1 : (int32_t)s;
}

__global__ __launch_bounds__(256) void slot_finalize_kernel(GateArgs a) {
  const int64_t n = a.T * a.k;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  a.slot[i] = final_slot(a, i);
}

// Exclusive rank of the calling thread's flag among the workgroup's 256
// flags (thread order), and their total; ballots within a wavefront, wave
// totals through LDS.
__device__ __forceinline__ int block_rank(bool flag, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t b = __ballot(flag);
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  if (lane == 0) wave_tot[wave] = __popcll(b);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) before += wave_tot[w];
    total += wave_tot[w];
  }
  __syncthreads();
  return before + __popcll(b & lt);
}

// Random Token Selection (k = 1 with a capacity; DeepSpeed's use_rts as
// reading R15 takes it): an expert whose demand D exceeds C keeps the C
// claimants of largest priority (the stream-3 word of the token; equal words
// to the lower token) and numbers them 0.. in token order; the rest are
// dropped.  Counts, offsets and the loss do not change.  One workgroup per
// expert: the C-th largest priority by a radix select over four 8-bit
// digits (LDS histograms over the expert's claimants), then one pass in
// token order that ranks the kept claims with workgroup scans.
__global__ __launch_bounds__(256) void rts_select_kernel(GateArgs a) {
  __shared__ int hist[256];
  __shared__ int wave_tot[4];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  const int e = blockIdx.x, tid = threadIdx.x;
  const int64_t T = a.T, C = a.C;
  if (C < 0 || (int64_t)a.demand[e] <= C) return;
  uint32_t prefix = 0, mask = 0;
  int need = (int)C;   // claimants still to take among those matching prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int64_t t = tid; t < T; t += 256) {
      if (a.expert_idx[t] != e) continue;
      const uint32_t p = philox_draw(a.seed_lo, a.seed_hi, kStreamRts, (uint64_t)t);
      if ((p & mask) == prefix) atomicAdd(&hist[(p >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid == 0) {
      // the digit where the count from the top reaches `need`
      int above = 0, b = 255;
      for (; b > 0; --b) {
        if (above + hist[b] >= need) break;
        above += hist[b];
      }
      s_prefix = prefix | ((uint32_t)b << shift);
      s_need = need - above;
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    mask |= 0xffu << shift;
  }
  // prefix is now the C-th largest priority; every claimant above it is kept,
  // and the first `need` (in token order) of those equal to it
  int run_eq = 0, run_kept = 0;
  for (int64_t base = 0; base < T; base += 256) {
    const int64_t t = base + tid;
    const bool claim = t < T && a.expert_idx[t] == e;
    const uint32_t p = claim ? philox_draw(a.seed_lo, a.seed_hi, kStreamRts, (uint64_t)t) : 0u;
    const bool eq = claim && p == prefix;
    int n_eq, n_kept;
    const int eq_rank = run_eq + block_rank(eq, wave_tot, n_eq);
    const bool keep = claim && (p > prefix || (eq && eq_rank < need));
    const int kept_rank = run_kept + block_rank(keep, wave_tot, n_kept);
    if (claim) a.slot[t] = keep ? kept_rank : -1;
    run_eq += n_eq;
    run_kept += n_kept;
  }
}

__global__ void gate_empty_kernel(int32_t* count, int32_t* offset, float* loss, int E) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    if (e < E) count[e] = 0;
    offset[e] = 0;
  }
  if (threadIdx.x == 0) *loss = 0.f;
}

template <int EP, int TG, int MODE>
size_t gate_lds_bytes() {
  constexpr int TT = TG * 16;
  const size_t wbytes = (MODE == MODE_BF16) ? size_t(2) * EP * gate_kc<EP>() * 2
                        : (MODE == MODE_BF16_DMA) ? size_t(GateDma<EP>::NS) * GateDma<EP>::STAGE : 0;
  return wbytes + 4 * (TG * 2 * EP + TG * EP);
}

template <int EP, int TG, int MODE, bool RND>
hipError_t launch_gate_rnd(const GateArgs& a, hipStream_t s) {
  const size_t lds = gate_lds_bytes<EP, TG, MODE>();
  auto kern = gate_kernel<EP, TG, MODE, RND>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(a.num_tiles), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int EP, int TG, int MODE>
hipError_t launch_gate_t(const GateArgs& a, hipStream_t s) {
  if (a.jitter || a.rsample || a.second) return launch_gate_rnd<EP, TG, MODE, true>(a, s);
  return launch_gate_rnd<EP, TG, MODE, false>(a, s);
}

hipError_t launch_gate_big(const GateArgs& a, hipStream_t s) {
  const size_t lds = (size_t)gbig::NS * gbig::STAGE + 4 * (4 * 2 * gbig::EP + 8 * gbig::EP);
  auto kern = gate_big_kernel;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.num_tiles), dim3(256), lds, s, a);
  return hipGetLastError();
}

// The bf16 router takes the LDS-DMA kernel when d fills whole K steps.
template <int EP>
hipError_t launch_gate_bf16(const GateArgs& a, hipStream_t s) {
  if (gate_dma_fits<EP>(a.d)) return launch_gate_t<EP, 4, MODE_BF16_DMA>(a, s);
  return launch_gate_t<EP, 4, MODE_BF16>(a, s);
}

template <int MODE>
hipError_t launch_gate_mode(const GateArgs& a, hipStream_t s) {
  const int E = a.E;
  if constexpr (MODE == MODE_BF16) {
    if (E <= 16) return launch_gate_bf16<16>(a, s);
    if (E <= 32) return launch_gate_bf16<32>(a, s);
    if (E <= 64) return launch_gate_bf16<64>(a, s);
    if (E <= 128) return launch_gate_bf16<128>(a, s);
    return launch_gate_bf16<256>(a, s);
  } else {
    if (E <= 16) return launch_gate_t<16, 4, MODE>(a, s);
    if (E <= 32) return launch_gate_t<32, 4, MODE>(a, s);
    if (E <= 64) return launch_gate_t<64, 4, MODE>(a, s);
    if (E <= 128) return launch_gate_t<128, 4, MODE>(a, s);
    return launch_gate_t<256, 4, MODE>(a, s);
  }
}

}  // namespace

int gate_tile_tokens_for(int E, int d, int dtype, bool logits_in, bool random_options) {
  if (!random_options && E > 64 && E <= gbig::EP && (logits_in || (dtype == DT_BF16 && d > 0 && d % gbig::KC == 0)))
    return gbig::TT;
  return 64;
}

hipError_t launch_gate(const GateArgs& a, int dtype, hipStream_t s) {
  hipError_t e;
  if (a.tile_tokens == gbig::TT) e = launch_gate_big(a, s);
  else if (a.logits_in) e = launch_gate_mode<MODE_LOGITS_IN>(a, s);
  else if (dtype == DT_BF16) e = launch_gate_mode<MODE_BF16>(a, s);
  else e = launch_gate_mode<MODE_F32>(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gate_scan_kernel, dim3((unsigned)(a.k * a.E)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_slot_finalize(const GateArgs& a, hipStream_t s) {
  const int64_t n = a.T * a.k;
  hipLaunchKernelGGL(slot_finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rts_select(const GateArgs& a, hipStream_t s) {
  if (a.k != 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rts_select_kernel, dim3((unsigned)a.E), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gate_empty(int32_t* expert_count, int32_t* expert_offset, float* gate_loss, int E,
                             hipStream_t s) {
  hipLaunchKernelGGL(gate_empty_kernel, dim3(1), dim3(256), 0, s, expert_count, expert_offset, gate_loss, E);
  return hipGetLastError();
}

}  // namespace moe
