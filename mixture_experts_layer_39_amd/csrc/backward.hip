// Backward of the layer around the expert FFNs: combine, the gate (softmax,
// top-k weights and gate_loss), dispatch and the router Linear.
//
// What is computed: the chain rule through the forward of
// "MoE混合专家架构：大模型高效推理的智能调度原理" §3.1 (MoELayer Steps 1-5) and
// "deepspeed.moe 模块" overview §3.1.  The top-k choice and the capacity slots
// are piecewise constant and pass no gradient: the top-k operation hands its
// gradient only to the chosen positions (DeepSeek-MoE fine-tuning article,
// ch.3 §3.1, the TopKRouter backward) and an expert without tokens gets none
// (ch.2 §2.1, the gradient mask).
//   combine:   dY_disp[row(t,j)] = w[t,j] * dOut[t];  dw[t,j] = <dOut[t], y_disp[row(t,j)]>
//   gate:      dp[t, e_j] += dw[t,j]   (renormalised weights w_j = p_j / S:
//              dp[t, e_i] += (dw_i - sum_j dw_j w_j) / S);
//              BALANCE loss: dp[t, e] += dloss * E * ce_e / T;
//              dlogits[t] = p[t] * (dp[t] - <p[t], dp[t]>)
//   dispatch and router input: dX[t] = sum_j dX_disp[row(t,j)] + dlogits[t] · W_r
//   router weights: dW_r = dlogits^T · x;  db_r = column sums of dlogits
//
// Design (gfx950):
//  * Combine backward is the combine kernel's traversal (one wavefront per
//    token, 16-byte vectors): the token's dOut row is read once, each kept
//    row of y_disp once, and dY_disp is written over y_disp in place (each
//    packed row belongs to exactly one claim, so one wavefront owns it).
//  * Gate backward: a group of 32 or 64 lanes per token, each lane holding
//    one to four consecutive experts; the softmax's max and sum are
//    xor-shuffles inside the group, the chosen probabilities one shuffle
//    each.  It also writes the logit gradient as a bf16 hi/lo pair
//    (hi = bf16(g), lo = bf16(g - hi)) and per-workgroup column sums.
//  * The router's input gradient dlogits · W_r has K = E (at most 256): it
//    runs on v_mfma_f32_32x32x16_bf16 twice (hi and lo), which keeps ~16
//    bits of the fp32 gradient.  W_r is packed once per call into MFMA
//    fragment order (1 MB at most, L2-resident), so each fragment is one
//    contiguous 1 KB load.  The result goes through LDS to token rows, where
//    the dispatch-backward gather (the dX_disp rows of the token's kept
//    claims) and the bf16 store are whole contiguous row segments; the sum is
//    rounded once.
//  * dW_r = dlogits^T x has K = T: the token range is cut into chunks, each
//    chunk's product runs on the large-tile GEMM (both operands transposed,
//    fp32 partial output), and one kernel adds the chunks and the hi/lo
//    halves in a fixed order, so results are bit-identical run to run.
#include "moe_internal.h"
#include "philox.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float lo16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

unsigned row_grid(int64_t T) {
  int64_t blocks = (T + kWaves - 1) / kWaves;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

// ---------------------------------------------------------------- combine backward
// y and dy may be the same buffer: each lane reads its vectors of a row before
// it writes the same vectors, and no other wavefront touches that row (so the
// two pointers are deliberately not restrict-qualified).  Each lane loads
// U vectors of dOut and of both rows before any store, so that U x 3 loads
// are in flight (a store may alias a later load, which keeps the compiler
// from hoisting loads across stores by itself).
template <int DT>
__device__ __forceinline__ void cb_unpack(const u32x4 v, float (&f)[8]) {
  if constexpr (DT == DT_BF16) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = lo16(u[i]);
      f[2 * i + 1] = hi16(u[i]);
    }
  } else {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
}

template <int DT>
__device__ __forceinline__ u32x4 cb_scale(float w, const float (&f)[8]) {
  if constexpr (DT == DT_BF16)
    return u32x4{pack_bf16x2(w * f[0], w * f[1]), pack_bf16x2(w * f[2], w * f[3]), pack_bf16x2(w * f[4], w * f[5]),
                 pack_bf16x2(w * f[6], w * f[7])};
  else
    return u32x4{__float_as_uint(w * f[0]), __float_as_uint(w * f[1]), __float_as_uint(w * f[2]),
                 __float_as_uint(w * f[3])};
}

template <int DT>
__global__ __launch_bounds__(256) void combine_backward_kernel(const u32x4* __restrict__ dout, const u32x4* y,
                                                               const int32_t* __restrict__ expert_idx,
                                                               const int32_t* __restrict__ slot,
                                                               const float* __restrict__ weight,
                                                               const int32_t* __restrict__ offset, u32x4* dy,
                                                               float* __restrict__ dw, int64_t T, int k, int nvec) {
  constexpr int U = 4;
  constexpr int NE = DT == DT_BF16 ? 8 : 4;   // elements per vector
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  for (int64_t t = wave_id; t < T; t += nwaves) {
    // every index load of the token before the first wait: slot, expert and
    // weight of each choice, then the kept claims' offsets
    const int s0 = slot[t * k], e0 = expert_idx[t * k];
    const int s1 = k == 2 ? slot[t * k + 1] : -1, e1 = k == 2 ? expert_idx[t * k + 1] : 0;
    const float wt0 = weight[t * k], wt1 = k == 2 ? weight[t * k + 1] : 0.f;
    const int64_t r0 = s0 >= 0 ? (int64_t)offset[e0] + s0 : -1;
    const int64_t r1 = s1 >= 0 ? (int64_t)offset[e1] + s1 : -1;
    const float w0 = r0 >= 0 ? wt0 : 0.f, w1 = r1 >= 0 ? wt1 : 0.f;
    float dot0 = 0.f, dot1 = 0.f;
    if (r0 >= 0 || r1 >= 0) {
      const u32x4* src = dout + t * nvec;
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int v0 = lane; v0 < nvec; v0 += 64 * U) {
        u32x4 o[U], ya[U], yb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int v = v0 + 64 * u;
          const bool in = v < nvec;
          o[u] = in ? __builtin_nontemporal_load(src + v) : z;
          ya[u] = (in && r0 >= 0) ? y[r0 * nvec + v] : z;
          yb[u] = (in && r1 >= 0) ? y[r1 * nvec + v] : z;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int v = v0 + 64 * u;
          if (v >= nvec) break;
          float of[8], fa[8], fb[8];
          cb_unpack<DT>(o[u], of);
          cb_unpack<DT>(ya[u], fa);
          cb_unpack<DT>(yb[u], fb);
#pragma unroll
          for (int i = 0; i < NE; ++i) {
            dot0 = fmaf(of[i], fa[i], dot0);
            dot1 = fmaf(of[i], fb[i], dot1);
          }
          if (r0 >= 0) dy[r0 * nvec + v] = cb_scale<DT>(w0, of);
          if (r1 >= 0) dy[r1 * nvec + v] = cb_scale<DT>(w1, of);
        }
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      dot0 += __shfl_xor(dot0, m);
      dot1 += __shfl_xor(dot1, m);
    }
    if (lane == 0) {
      dw[t * k] = r0 >= 0 ? dot0 : 0.f;
      if (k == 2) dw[t * k + 1] = r1 >= 0 ? dot1 : 0.f;
    }
  }
}

// ---------------------------------------------------------------- top-1 counts
// Workgroup b counts the top-1 choices of its token range into part[b][E].
__global__ __launch_bounds__(256) void top1_count_kernel(const int32_t* __restrict__ idx, int k, int64_t T, int E,
                                                         int32_t* __restrict__ part) {
  __shared__ int h[MOE_MAX_EXPERTS_DEV];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t per = (T + gridDim.x - 1) / gridDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * per;
  const int64_t t1 = t0 + per < T ? t0 + per : T;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += 256) {
    const int e = idx[t * k];
    if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) part[(int64_t)blockIdx.x * E + e] = h[e];
}

// coef[e] = dloss * E * ce_e / T, ce_e = (top-1 choices of e) / T.
__global__ __launch_bounds__(256) void top1_coef_kernel(const int32_t* __restrict__ part, int nparts, int E,
                                                        int64_t T, const float* __restrict__ dloss,
                                                        float* __restrict__ coef) {
  const int e = threadIdx.x;
  if (e >= E) return;
  int c = 0;
  for (int p = 0; p < nparts; ++p) c += part[p * E + e];
  const float g = dloss ? dloss[0] : 0.f;
  const float ce = (float)c / (float)T;
  coef[e] = g * (float)E * ce / (float)T;
}

// ---------------------------------------------------------------- gate backward
// Group of G lanes per token (G = 32 or 64), lane gl holding the EPL
// consecutive experts gl*EPL .. +EPL-1.  The softmax needs one max and one
// sum over the group (xor-shuffles with offsets below G, so they stay inside
// the group); the chosen experts' probabilities are read from the lanes
// that hold them; <p, dp> needs no further reduction, because dp is the
// BALANCE coefficient (summed with the exponentials) plus the two chosen
// terms.
template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
template <int G>
__device__ __forceinline__ void group_sum2(float& a, float& b) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) {
    a += __shfl_xor(a, m);
    b += __shfl_xor(b, m);
  }
}

// bf16 bits of v (round to nearest even)
__device__ __forceinline__ uint32_t bf16_bits(float v) { return pack_bf16x2(v, 0.f) & 0xffffu; }

template <int EPL>
__device__ __forceinline__ float pick(const float (&v)[EPL], int i) {
  float r = v[0];
#pragma unroll
  for (int j = 1; j < EPL; ++j)
    if (i == j) r = v[j];
  return r;
}

template <int G, int EPL, bool FROM_LOGITS>
__global__ __launch_bounds__(256) void gate_backward_kernel(GateBwdArgs a) {
  constexpr int GPW = 64 / G;   // tokens per wave and pass
  __shared__ float s_db[kWaves * GPW][G * EPL + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / G, gl = lane % G, gbase = lane - gl;
  const int E = a.E, k = a.k, Ep = a.Ep;
  const int eb = gl * EPL;      // this lane's first expert
  const int64_t T = a.T;
  const int64_t tb0 = (int64_t)blockIdx.x * kGateBwdTokens;
  float dbacc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) dbacc[i] = 0.f;

  for (int it0 = 0; it0 < kGateBwdTokens; it0 += kWaves * GPW) {
    const int64_t t = tb0 + it0 + wave * GPW + grp;
    const bool valid = t < T;
    float dl[EPL];
    if constexpr (FROM_LOGITS) {
      float p[EPL], cf[EPL];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = eb + i;
        p[i] = (valid && e < E) ? a.logits[t * E + e] : -INFINITY;
        cf[i] = (a.coef && e < E) ? a.coef[e] : 0.f;
        mx = fmaxf(mx, p[i]);
      }
      mx = group_max<G>(mx);
      if (!valid) mx = 0.f;
      float sum = 0.f, sc = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = eb + i;
        p[i] = (valid && e < E) ? expf(p[i] - mx) : 0.f;
        sum += p[i];
        sc = fmaf(p[i], cf[i], sc);
      }
      group_sum2<G>(sum, sc);
      if (!valid) sum = 1.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) p[i] = p[i] / sum;
      // the chosen experts and the probabilities their owner lanes hold
      int e0 = valid ? a.idx[t * k] : 0;
      int e1 = (valid && k == 2) ? a.idx[t * k + 1] : 0;
      e0 = min(max(e0, 0), E - 1);
      e1 = min(max(e1, 0), E - 1);
      const float g0 = valid ? a.dw[t * k] : 0.f;
      const float g1 = (valid && k == 2) ? a.dw[t * k + 1] : 0.f;
      const float pe0 = __shfl(pick<EPL>(p, e0 % EPL), gbase + e0 / EPL);
      const float pe1 = k == 2 ? __shfl(pick<EPL>(p, e1 % EPL), gbase + e1 / EPL) : 0.f;
      if (k != 2) e1 = -1;
      float c0 = g0, c1 = g1;
      if (a.normalize) {
        const float S = pe0 + pe1;
        const float corr = g0 * (pe0 / S) + g1 * (pe1 / S);
        c0 = (g0 - corr) / S;
        c1 = (g1 - corr) / S;
      }
      // <p, dp> = sum_e p_e coef_e + p_e0 c0 + p_e1 c1
      const float pdp = sc / sum + pe0 * c0 + pe1 * c1;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = eb + i;
        float dp = cf[i];
        if (e == e0) dp += c0;
        if (e == e1) dp += c1;
        dl[i] = p[i] * (dp - pdp);
      }
    } else {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = eb + i;
        dl[i] = (valid && e < E) ? a.dlogits[t * E + e] : 0.f;
      }
    }
    if (valid) {
      uint32_t hb[EPL], lb[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = eb + i;
        if (FROM_LOGITS && e < E) a.dlogits[t * E + e] = dl[i];
        hb[i] = bf16_bits(dl[i]);
        lb[i] = bf16_bits(dl[i] - __uint_as_float(hb[i] << 16));
        dbacc[i] += dl[i];
      }
      // (with EPL even and Ep a multiple of 32, eb < Ep covers the whole pair)
      if (a.dl_hl && eb < Ep) {
        uint16_t* hrow = a.dl_hl + t * 2 * Ep + eb;
        if constexpr (EPL % 2 == 0) {
#pragma unroll
          for (int i = 0; i < EPL; i += 2) {
            reinterpret_cast<uint32_t*>(hrow)[i / 2] = hb[i] | (hb[i + 1] << 16);
            reinterpret_cast<uint32_t*>(hrow + Ep)[i / 2] = lb[i] | (lb[i + 1] << 16);
          }
        } else {
#pragma unroll
          for (int i = 0; i < EPL; ++i) {
            if (eb + i < Ep) {
              hrow[i] = (uint16_t)hb[i];
              hrow[Ep + i] = (uint16_t)lb[i];
            }
          }
        }
      }
    }
  }
  if (!a.dbpart) return;
  // column partial sums of this workgroup's tokens, in a fixed order, stored
  // expert-major: dbpart[e][workgroup]
#pragma unroll
  for (int i = 0; i < EPL; ++i) s_db[wave * GPW + grp][eb + i] = dbacc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    float s = 0.f;
    for (int r = 0; r < kWaves * GPW; ++r) s += s_db[r][e];
    a.dbpart[(int64_t)e * gridDim.x + blockIdx.x] = s;
  }
}

// ---------------------------------------------------------------- router input gradient
// The router weight in MFMA A-fragment order: for feature block fb (32
// features), K step ks (16 experts) and lane l = 32*hh + n, the 8 values
// W_r[ks*16 + 8*hh + j][fb*32 + fmap(n)], j = 0..7, with fmap(n) =
// ((n>>2)&1)*16 + (n>>3)*4 + (n&3) (zero past E).  A wavefront then loads
// one fragment as one contiguous kilobyte.
__global__ __launch_bounds__(256) void router_pack_kernel(const uint16_t* __restrict__ wr,
                                                          uint16_t* __restrict__ wfrag, int E, int d, int Ep) {
  const int64_t total = (int64_t)d * Ep;
  const int epk = Ep / 16;
  for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < total; o += (int64_t)gridDim.x * 256) {
    const int j = (int)(o & 7);
    const int l = (int)((o >> 3) & 63);
    const int64_t q = o >> 9;
    const int ks = (int)(q % epk), fb = (int)(q / epk);
    const int hh = l >> 5, n = l & 31;
    const int e = ks * 16 + 8 * hh + j;
    const int f = fb * 32 + ((n >> 2) & 1) * 16 + (n >> 3) * 4 + (n & 3);
    wfrag[o] = e < E ? wr[(int64_t)e * d + f] : (uint16_t)0;
  }
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Workgroup: 32 * TB tokens, all d features in chunks of 256.  Per chunk,
// phase 1: wave w computes the router term for the tokens (TB blocks of 32
// MFMA columns) and features 64w .. +63 of the chunk (two 32-row MFMA
// blocks; row l&31 is feature fmap(l&31), so accumulator register r of lane
// l is feature 16*(l>>5) + r of its block) and writes it to LDS as
// [token][feature] fp32.  Each chunk streams the packed router weight's
// 64 KB for the chunk from L2, so TB = 2 halves that stream per token (it
// was the larger part of the kernel's operand traffic at 32 tokens).
// Phase 2: wave w takes tokens 8*TB*w .. +8*TB-1, two per instruction (half
// a wavefront covers a token's 256 features as 16-byte vectors), adds the
// token's gathered dX_disp rows and the router term and stores the row
// segment.  One workgroup walks each token's rows from start to end, and its
// B fragments (the tokens' logit gradient) are loaded once for all chunks.
// The gathered rows of a chunk are issued after its operand loads (loads
// complete in order, so the K loop never waits on them).  EPK = Ep / 16 K
// steps (0: no router term).
constexpr int kIgFeat = 256, kIgPitch = kIgFeat + 4;

template <int EPK, int TB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TB == 1 ? 4 : 2, 8)))
void input_grad_kernel(InputGradArgs a) {
  constexpr int kIgTok = 32 * TB;     // tokens per workgroup
  constexpr int NP = 4 * TB;          // phase 2: token pairs per wave
  __shared__ __attribute__((aligned(16))) float tile[EPK > 0 ? kIgTok : 1][kIgPitch];
  constexpr int Ep = EPK * 16;
  const int d = a.d, k = a.k;
  const int64_t t0 = (int64_t)blockIdx.x * kIgTok;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, hh = lane >> 5;

  // phase 2: this lane's token pair rows (token 8*TB*w + 2i + hh), -1 if none
  int64_t rw0[NP], rw1[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int64_t t = t0 + 8 * TB * wave + 2 * i + hh;
    rw0[i] = rw1[i] = -1;
    if (t < a.T) {
      const int s0 = a.slot[t * k];
      if (s0 >= 0) rw0[i] = (int64_t)a.offset[a.idx[t * k]] + s0;
      if (k == 2) {
        const int s1 = a.slot[t * k + 1];
        if (s1 >= 0) rw1[i] = (int64_t)a.offset[a.idx[t * k + 1]] + s1;
      }
    }
  }

  // phase 1 operands: the B fragments (the tokens' logit gradient, hi and
  // lo) are reloaded per chunk from L1 rather than kept in registers
  const bf16x8 zero = {};
  const uint16_t* brow[TB];
  bool tv[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    const int64_t tb = t0 + 32 * b + n;
    tv[b] = tb < a.T;
    brow[b] = EPK > 0 ? a.dl_hl + (tv[b] ? tb : 0) * 2 * Ep + 8 * hh : nullptr;
  }

  for (int f0 = 0; f0 < d; f0 += kIgFeat) {
    const int fl = f0 + 8 * n;            // phase 2: this lane's 8 features
    const bool fin = fl < d;
    uint4 g0[NP], g1[NP];
    auto gather = [&]() {
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        g0[i] = g1[i] = make_uint4(0u, 0u, 0u, 0u);
        if (fin && rw0[i] >= 0) g0[i] = *reinterpret_cast<const uint4*>(a.dx_disp + rw0[i] * d + fl);
        if (fin && rw1[i] >= 0) g1[i] = *reinterpret_cast<const uint4*>(a.dx_disp + rw1[i] * d + fl);
      }
    };
    if constexpr (EPK > 0) {
      const int fw = f0 + 64 * wave;
      const int nb = min(2, (d - fw) / 32);     // valid feature blocks (wave-uniform, may be <= 0)
      f32x16 acc[2][TB];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int c = 0; c < TB; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[b][c][r] = 0.f;
      // with 64 tokens (TB = 2, 256 registers) the operands of step ks + 1
      // are loaded while step ks's MFMAs run; 32-token workgroups keep the
      // register budget of four waves per SIMD and load each step's own
      constexpr bool PIPE = TB == 2;
      bf16x8 hn[TB], ln[TB], avn[2];
      auto load_ops = [&](int ks) {
#pragma unroll
        for (int c = 0; c < TB; ++c) {
          hn[c] = tv[c] ? ld8(brow[c] + ks * 16) : zero;
          ln[c] = tv[c] ? ld8(brow[c] + Ep + ks * 16) : zero;
        }
#pragma unroll
        for (int b = 0; b < 2; ++b)
          avn[b] = b < nb ? ld8(a.wfrag + (((int64_t)(fw / 32 + b) * EPK + ks) * 64 + lane) * 8) : zero;
      };
      if constexpr (PIPE) load_ops(0);
#pragma unroll
      for (int ks = 0; ks < EPK; ++ks) {
        if constexpr (!PIPE) load_ops(ks);
        bf16x8 h[TB], l[TB], av[2];
#pragma unroll
        for (int c = 0; c < TB; ++c) {
          h[c] = hn[c];
          l[c] = ln[c];
        }
        av[0] = avn[0];
        av[1] = avn[1];
        if constexpr (PIPE) {
          if (ks + 1 < EPK) load_ops(ks + 1);
        }
        if (ks == EPK - 1) {
          __builtin_amdgcn_sched_barrier(0);
          gather();
          __builtin_amdgcn_sched_barrier(0);
        }
        // hi products of every block, then lo: never two MFMAs back to back on one accumulator
#pragma unroll
        for (int c = 0; c < TB; ++c)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            if (b < nb) acc[b][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[b], h[c], acc[b][c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < TB; ++c)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            if (b < nb) acc[b][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[b], l[c], acc[b][c], 0, 0, 0);
      }
      __syncthreads();   // the previous chunk's phase 2 has read the tile
#pragma unroll
      for (int c = 0; c < TB; ++c)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float4* dst = reinterpret_cast<float4*>(&tile[32 * c + n][64 * wave + 32 * b + 16 * hh]);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dst[q] = make_float4(acc[b][c][4 * q], acc[b][c][4 * q + 1], acc[b][c][4 * q + 2], acc[b][c][4 * q + 3]);
        }
      __syncthreads();
    } else {
      gather();
    }

#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int tl = 8 * TB * wave + 2 * i + hh;
      const int64_t t = t0 + tl;
      if (t >= a.T || !fin) continue;
      const uint32_t u0[4] = {g0[i].x, g0[i].y, g0[i].z, g0[i].w};
      const uint32_t u1[4] = {g1[i].x, g1[i].y, g1[i].z, g1[i].w};
      float v[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = lo16(u0[q]) + lo16(u1[q]);
        v[2 * q + 1] = hi16(u0[q]) + hi16(u1[q]);
      }
      if constexpr (EPK > 0) {
        const float4 r0 = *reinterpret_cast<const float4*>(&tile[tl][8 * n]);
        const float4 r1 = *reinterpret_cast<const float4*>(&tile[tl][8 * n + 4]);
        float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
        if (a.jitter) {
          // the router read x * factor, so its input gradient carries the
          // factor (the bf16 rounding of the product taken as identity)
          const uint64_t n0 = (uint64_t)t * d + fl;   // a multiple of 8
          const uint4 w0 = philox_block(a.seed_lo, a.seed_hi, kStreamJitter, n0 >> 2);
          const uint4 w1 = philox_block(a.seed_lo, a.seed_hi, kStreamJitter, (n0 >> 2) + 1);
          const uint32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) rv[j] *= __fadd_rn(0.99f, __fmul_rn(0.02f, philox_uniform(wv[j])));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] += rv[j];
      }
      if (a.dx_add) {
        // the residual MLP's input gradient
        float xa[8];
        const uint4 u = *reinterpret_cast<const uint4*>(a.dx_add + t * d + fl);
        const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xa[2 * q] = lo16(uu[q]);
          xa[2 * q + 1] = hi16(uu[q]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] += xa[j];
      }
      if (a.dlc) {
        // the mixing coefficients' logit gradient through their Linear
        const float g0 = a.dlc[2 * t], g1 = a.dlc[2 * t + 1];
        const uint4 c0 = *reinterpret_cast<const uint4*>(a.coef_w + fl);
        const uint4 c1 = *reinterpret_cast<const uint4*>(a.coef_w + d + fl);
        const uint32_t u0[4] = {c0.x, c0.y, c0.z, c0.w}, u1[4] = {c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] += g0 * lo16(u0[q]) + g1 * lo16(u1[q]);
          v[2 * q + 1] += g0 * hi16(u0[q]) + g1 * hi16(u1[q]);
        }
      }
      *reinterpret_cast<uint4*>(a.dx + t * d + fl) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                                pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
  }
}

// ---------------------------------------------------------------- router weight gradient
__global__ __launch_bounds__(256) void chunk_offsets_kernel(int32_t* __restrict__ off, int S, int chunk, int64_t T) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i > S) return;
  const int64_t v = (int64_t)i * chunk;
  off[i] = (int32_t)(v < T ? v : T);
}

// dw[e][f] = sum over chunks c (in order) of part[c][e][f] + part[c][Ep+e][f].
__global__ __launch_bounds__(256) void router_reduce_kernel(const float4* __restrict__ part, int S, int E, int Ep,
                                                            int d, float4* __restrict__ dw) {
  const int d4 = d / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)E * d4) return;
  const int e = (int)(i / d4), f4 = (int)(i % d4);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c = 0; c < S; ++c) {
    const float4 h = part[((int64_t)c * 2 * Ep + e) * d4 + f4];
    const float4 l = part[((int64_t)c * 2 * Ep + Ep + e) * d4 + f4];
    s.x += h.x + l.x;
    s.y += h.y + l.y;
    s.z += h.z + l.z;
    s.w += h.w + l.w;
  }
  dw[i] = s;
}

// db[e] = sum of the gate-backward workgroups' partial sums dbpart[e][0..nb):
// one workgroup per expert, thread i adding partials i, i+256, ... in order,
// then a fixed-order tree over the threads.
__global__ __launch_bounds__(256) void db_reduce_kernel(const float* __restrict__ dbpart, int nb,
                                                        float* __restrict__ db) {
  __shared__ float s[256];
  const int e = blockIdx.x;
  float acc = 0.f;
  for (int b = threadIdx.x; b < nb; b += 256) acc += dbpart[(int64_t)e * nb + b];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) s[threadIdx.x] += s[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) db[e] = s[0];
}

__global__ __launch_bounds__(256) void zero_bytes_kernel(uint4* __restrict__ p16, size_t n16,
                                                         unsigned char* __restrict__ tail, size_t ntail) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p16[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_combine_backward(const void* dout, const void* y_disp, const int32_t* expert_idx,
                                   const int32_t* slot, const float* weight, const int32_t* expert_offset,
                                   void* dy_disp, float* dweight, int64_t T, int k, int d, int dtype,
                                   hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nvec = d * (dtype == DT_BF16 ? 2 : 4) / 16;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(combine_backward_kernel<DT_BF16>, dim3(row_grid(T)), dim3(256), 0, s,
                       static_cast<const u32x4*>(dout), static_cast<const u32x4*>(y_disp), expert_idx, slot, weight,
                       expert_offset, static_cast<u32x4*>(dy_disp), dweight, T, k, nvec);
  else
    hipLaunchKernelGGL(combine_backward_kernel<DT_F32>, dim3(row_grid(T)), dim3(256), 0, s,
                       static_cast<const u32x4*>(dout), static_cast<const u32x4*>(y_disp), expert_idx, slot, weight,
                       expert_offset, static_cast<u32x4*>(dy_disp), dweight, T, k, nvec);
  return hipGetLastError();
}

hipError_t launch_top1_coef(const int32_t* idx, int k, int64_t T, int E, const float* dloss, int32_t* part,
                            float* coef, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int nparts = (int)((T + 4095) / 4096);
  if (nparts > kTop1Parts) nparts = kTop1Parts;
  hipLaunchKernelGGL(top1_count_kernel, dim3(nparts), dim3(256), 0, s, idx, k, T, E, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(top1_coef_kernel, dim3(1), dim3(256), 0, s, part, nparts, E, T, dloss, coef);
  return hipGetLastError();
}

hipError_t launch_gate_backward(const GateBwdArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.T + kGateBwdTokens - 1) / kGateBwdTokens));
  const bool fl = a.logits != nullptr;
#define MOE_GB(G, EPL)                                                                 \
  do {                                                                                 \
    if (fl) hipLaunchKernelGGL((gate_backward_kernel<G, EPL, true>), grid, dim3(256), 0, s, a);  \
    else hipLaunchKernelGGL((gate_backward_kernel<G, EPL, false>), grid, dim3(256), 0, s, a);    \
  } while (0)
  if (a.Ep <= 32) MOE_GB(32, 1);
  else if (a.Ep <= 64) MOE_GB(64, 1);
  else if (a.Ep <= 128) MOE_GB(64, 2);
  else if (a.Ep <= 192) MOE_GB(64, 3);
  else MOE_GB(64, 4);
#undef MOE_GB
  return hipGetLastError();
}

hipError_t launch_router_pack(const void* w_router, uint16_t* wfrag, int E, int d, int Ep, hipStream_t s) {
  const int64_t n = (int64_t)d * Ep;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(router_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const uint16_t*>(w_router), wfrag, E, d, Ep);
  return hipGetLastError();
}

template <int TB>
hipError_t launch_input_grad_tb(const InputGradArgs& a, hipStream_t s) {
  const int64_t tiles = (a.T + 32 * TB - 1) / (32 * TB);
  const dim3 grid((unsigned)tiles);
  switch (a.dl_hl ? a.Ep / 16 : 0) {
    case 0: hipLaunchKernelGGL((input_grad_kernel<0, TB>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((input_grad_kernel<2, TB>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((input_grad_kernel<4, TB>), grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL((input_grad_kernel<6, TB>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((input_grad_kernel<8, TB>), grid, dim3(256), 0, s, a); break;
    case 10: hipLaunchKernelGGL((input_grad_kernel<10, TB>), grid, dim3(256), 0, s, a); break;
    case 12: hipLaunchKernelGGL((input_grad_kernel<12, TB>), grid, dim3(256), 0, s, a); break;
    case 14: hipLaunchKernelGGL((input_grad_kernel<14, TB>), grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((input_grad_kernel<16, TB>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_input_grad(const InputGradArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  // 64 tokens per workgroup once that still gives every CU two workgroups
  // (the router term's weight stream per token halves); 32 below that
  if (a.dl_hl && a.T >= (int64_t)64 * 2 * device_cus()) return launch_input_grad_tb<2>(a, s);
  return launch_input_grad_tb<1>(a, s);
}

hipError_t launch_router_wgrad(const RouterWgradArgs& a, hipStream_t s) {
  hipError_t e;
  if (a.T == 0) {
    if (a.dw_router && (e = launch_zero_bytes(a.dw_router, (size_t)a.E * a.d * 4, s)) != hipSuccess) return e;
    if (a.db_router && (e = launch_zero_bytes(a.db_router, (size_t)a.E * 4, s)) != hipSuccess) return e;
    return hipSuccess;
  }
  if (a.dw_router) {
    const RouterChunks rc = router_chunks(a.T, a.d, a.E);
    hipLaunchKernelGGL(chunk_offsets_kernel, dim3((rc.S + 256) / 256), dim3(256), 0, s, a.choff, rc.S, rc.chunk,
                       a.T);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_router_partials(a.dl_hl, a.x, a.choff, a.part, a.T, rc.S, a.d, a.Ep, s)) != hipSuccess) return e;
    const int64_t n4 = (int64_t)a.E * a.d / 4;
    hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(a.part), rc.S, a.E, a.Ep, a.d,
                       reinterpret_cast<float4*>(a.dw_router));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.db_router) {
    const int nb = (int)((a.T + kGateBwdTokens - 1) / kGateBwdTokens);
    hipLaunchKernelGGL(db_reduce_kernel, dim3(a.E), dim3(256), 0, s, a.dbpart, nb, a.db_router);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_zero_bytes(void* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t n16 = n / 16, ntail = n % 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_bytes_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint4*>(p), n16,
                     static_cast<unsigned char*>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

namespace {
// x_j = bf16(x * ((1 - 0.01) + 0.02 u)), u the stream-0 uniform of element
// t*d + i, the product and the sum each rounded once in fp32: what the gate
// kernel's router read under jitter.
__global__ __launch_bounds__(256) void jitter_input_kernel(const bf16* __restrict__ x, bf16* __restrict__ xj,
                                                           int64_t nvec, uint32_t seed_lo, uint32_t seed_hi) {
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < nvec; v += (int64_t)gridDim.x * 256) {
    bf16x8 xv = *reinterpret_cast<const bf16x8*>(x + v * 8);
    const uint4 w0 = philox_block(seed_lo, seed_hi, kStreamJitter, (uint64_t)v * 2);
    const uint4 w1 = philox_block(seed_lo, seed_hi, kStreamJitter, (uint64_t)v * 2 + 1);
    const uint32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float f = __fadd_rn(0.99f, __fmul_rn(0.02f, philox_uniform(wv[j])));
      xv[j] = static_cast<bf16>(__fmul_rn(static_cast<float>(xv[j]), f));
    }
    *reinterpret_cast<bf16x8*>(xj + v * 8) = xv;
  }
}
}  // namespace

hipError_t launch_jitter_input(const bf16* x, bf16* xj, int64_t T, int d, uint32_t seed_lo, uint32_t seed_hi,
                               hipStream_t s) {
  const int64_t nvec = T * d / 8;
  if (nvec == 0) return hipSuccess;
  const int64_t blocks = (nvec + 255) / 256;
  hipLaunchKernelGGL(jitter_input_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, x, xj,
                     nvec, seed_lo, seed_hi);
  return hipGetLastError();
}

}  // namespace moe
