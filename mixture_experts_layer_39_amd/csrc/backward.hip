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
//    one to four experts; softmax and the two reductions are xor-shuffles
//    inside the group.  It also writes the logit gradient as a bf16 hi/lo
//    pair (hi = bf16(g), lo = bf16(g - hi)) and per-workgroup column sums.
//  * The router's input gradient dlogits · W_r has K = E (at most 256): it
//    runs on v_mfma_f32_32x32x16_bf16 twice (hi and lo), which keeps ~16
//    bits of the fp32 gradient, with fragments loaded straight from global
//    memory (W_r^T is 1 MB at most and stays in L2).  Features are the MFMA
//    rows, in the permuted order that gives each lane 16 consecutive output
//    features of one token, so the dispatch-backward gather (dX_disp rows of
//    the token's kept claims) and the bf16 store are 32-byte vectors in the
//    same kernel; the sum is rounded once.
//  * dW_r = dlogits^T x has K = T: the token range is cut into chunks, each
//    chunk's product runs on the large-tile GEMM (both operands transposed,
//    fp32 partial output), and one kernel adds the chunks and the hi/lo
//    halves in a fixed order, so results are bit-identical run to run.
#include "moe_internal.h"

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
// y and dy may be the same buffer: each lane reads its vector of a row before
// it writes the same vector, and no other wavefront touches that row (so the
// two pointers are deliberately not restrict-qualified).
template <int DT>
__global__ __launch_bounds__(256) void combine_backward_kernel(const u32x4* __restrict__ dout, const u32x4* y,
                                                               const int32_t* __restrict__ expert_idx,
                                                               const int32_t* __restrict__ slot,
                                                               const float* __restrict__ weight,
                                                               const int32_t* __restrict__ offset, u32x4* dy,
                                                               float* __restrict__ dw, int64_t T, int k, int nvec) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  for (int64_t t = wave_id; t < T; t += nwaves) {
    int64_t r0 = -1, r1 = -1;
    float w0 = 0.f, w1 = 0.f;
    {
      const int s0 = slot[t * k];
      if (s0 >= 0) {
        r0 = (int64_t)offset[expert_idx[t * k]] + s0;
        w0 = weight[t * k];
      }
      if (k == 2) {
        const int s1 = slot[t * k + 1];
        if (s1 >= 0) {
          r1 = (int64_t)offset[expert_idx[t * k + 1]] + s1;
          w1 = weight[t * k + 1];
        }
      }
    }
    float dot0 = 0.f, dot1 = 0.f;
    if (r0 >= 0 || r1 >= 0) {
      const u32x4* src = dout + t * nvec;
      for (int v = lane; v < nvec; v += 64) {
        const u32x4 o = __builtin_nontemporal_load(src + v);
        if constexpr (DT == DT_BF16) {
          const uint32_t ou[4] = {o.x, o.y, o.z, o.w};
          float of[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            of[2 * i] = lo16(ou[i]);
            of[2 * i + 1] = hi16(ou[i]);
          }
          if (r0 >= 0) {
            const u32x4 a = y[r0 * nvec + v];
            const uint32_t au[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              dot0 = fmaf(of[2 * i], lo16(au[i]), dot0);
              dot0 = fmaf(of[2 * i + 1], hi16(au[i]), dot0);
            }
            dy[r0 * nvec + v] = u32x4{pack_bf16x2(w0 * of[0], w0 * of[1]), pack_bf16x2(w0 * of[2], w0 * of[3]),
                                      pack_bf16x2(w0 * of[4], w0 * of[5]), pack_bf16x2(w0 * of[6], w0 * of[7])};
          }
          if (r1 >= 0) {
            const u32x4 b = y[r1 * nvec + v];
            const uint32_t bu[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              dot1 = fmaf(of[2 * i], lo16(bu[i]), dot1);
              dot1 = fmaf(of[2 * i + 1], hi16(bu[i]), dot1);
            }
            dy[r1 * nvec + v] = u32x4{pack_bf16x2(w1 * of[0], w1 * of[1]), pack_bf16x2(w1 * of[2], w1 * of[3]),
                                      pack_bf16x2(w1 * of[4], w1 * of[5]), pack_bf16x2(w1 * of[6], w1 * of[7])};
          }
        } else {
          const float of[4] = {__uint_as_float(o.x), __uint_as_float(o.y), __uint_as_float(o.z),
                               __uint_as_float(o.w)};
          if (r0 >= 0) {
            const u32x4 a = y[r0 * nvec + v];
            dot0 = fmaf(of[0], __uint_as_float(a.x), dot0);
            dot0 = fmaf(of[1], __uint_as_float(a.y), dot0);
            dot0 = fmaf(of[2], __uint_as_float(a.z), dot0);
            dot0 = fmaf(of[3], __uint_as_float(a.w), dot0);
            dy[r0 * nvec + v] = u32x4{__float_as_uint(w0 * of[0]), __float_as_uint(w0 * of[1]),
                                      __float_as_uint(w0 * of[2]), __float_as_uint(w0 * of[3])};
          }
          if (r1 >= 0) {
            const u32x4 b = y[r1 * nvec + v];
            dot1 = fmaf(of[0], __uint_as_float(b.x), dot1);
            dot1 = fmaf(of[1], __uint_as_float(b.y), dot1);
            dot1 = fmaf(of[2], __uint_as_float(b.z), dot1);
            dot1 = fmaf(of[3], __uint_as_float(b.w), dot1);
            dy[r1 * nvec + v] = u32x4{__float_as_uint(w1 * of[0]), __float_as_uint(w1 * of[1]),
                                      __float_as_uint(w1 * of[2]), __float_as_uint(w1 * of[3])};
          }
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
// Group of G lanes per token (G = 32 or 64), lane gl holding experts
// gl + G*i, i < EPL.  Reductions are xor-shuffles with offsets below G, so
// they stay inside the group.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// bf16 bits of v (round to nearest even)
__device__ __forceinline__ uint32_t bf16_bits(float v) { return pack_bf16x2(v, 0.f) & 0xffffu; }

template <int G, int EPL, bool FROM_LOGITS>
__global__ __launch_bounds__(256) void gate_backward_kernel(GateBwdArgs a) {
  constexpr int GPW = 64 / G;   // tokens per wave and pass
  __shared__ float s_db[kWaves * GPW][G * EPL];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / G, gl = lane % G;
  const int E = a.E, k = a.k, Ep = a.Ep;
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
      float p[EPL];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = gl + G * i;
        p[i] = (valid && e < E) ? a.logits[t * E + e] : -INFINITY;
        mx = fmaxf(mx, p[i]);
      }
      mx = group_max<G>(mx);
      if (!valid) mx = 0.f;
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = gl + G * i;
        p[i] = (valid && e < E) ? expf(p[i] - mx) : 0.f;
        sum += p[i];
      }
      sum = group_sum<G>(sum);
      if (!valid) sum = 1.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) p[i] = p[i] / sum;
      // the chosen experts, their gate-weight gradients and probabilities
      // (each probability is held by one lane: the group sum is exact)
      const int e0 = valid ? a.idx[t * k] : -1;
      const int e1 = (valid && k == 2) ? a.idx[t * k + 1] : -1;
      const float g0 = valid ? a.dw[t * k] : 0.f;
      const float g1 = (valid && k == 2) ? a.dw[t * k + 1] : 0.f;
      float pe0 = 0.f, pe1 = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = gl + G * i;
        if (e == e0) pe0 = p[i];
        if (e == e1) pe1 = p[i];
      }
      pe0 = group_sum<G>(pe0);
      pe1 = group_sum<G>(pe1);
      float c0 = g0, c1 = g1;
      if (a.normalize) {
        const float S = pe0 + pe1;
        const float corr = g0 * (pe0 / S) + g1 * (pe1 / S);
        c0 = (g0 - corr) / S;
        c1 = (g1 - corr) / S;
      }
      float dp[EPL];
      float pdp = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = gl + G * i;
        dp[i] = (a.coef && e < E) ? a.coef[e] : 0.f;
        if (e == e0) dp[i] += c0;
        if (e == e1) dp[i] += c1;
        pdp = fmaf(p[i], dp[i], pdp);
      }
      pdp = group_sum<G>(pdp);
#pragma unroll
      for (int i = 0; i < EPL; ++i) dl[i] = p[i] * (dp[i] - pdp);
    } else {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = gl + G * i;
        dl[i] = (valid && e < E) ? a.dlogits[t * E + e] : 0.f;
      }
    }
    if (valid) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = gl + G * i;
        if (FROM_LOGITS && e < E) a.dlogits[t * E + e] = dl[i];
        if (a.dl_hl && e < Ep) {
          const uint32_t hb = bf16_bits(dl[i]);
          const uint32_t lb = bf16_bits(dl[i] - __uint_as_float(hb << 16));
          a.dl_hl[t * 2 * Ep + e] = (uint16_t)hb;
          a.dl_hl[t * 2 * Ep + Ep + e] = (uint16_t)lb;
        }
        dbacc[i] += dl[i];
      }
    }
  }
  if (!a.dbpart) return;
  // column partial sums of this workgroup's tokens, in a fixed order
#pragma unroll
  for (int i = 0; i < EPL; ++i) s_db[wave * GPW + grp][gl + G * i] = dbacc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    float s = 0.f;
    for (int r = 0; r < kWaves * GPW; ++r) s += s_db[r][e];
    a.dbpart[(int64_t)blockIdx.x * E + e] = s;
  }
}

// ---------------------------------------------------------------- router input gradient
// wrT[f][e] = W_r[e][f] for e < E, zero for E <= e < Ep.
__global__ __launch_bounds__(256) void router_transpose_kernel(const uint16_t* __restrict__ wr,
                                                               uint16_t* __restrict__ wrT, int E, int d, int Ep) {
  const int64_t n = (int64_t)d * Ep;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int f = (int)(i / Ep), e = (int)(i % Ep);
    wrT[i] = e < E ? wr[(int64_t)e * d + f] : (uint16_t)0;
  }
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ void add16(float (&v)[16], const bf16* row) {
  const uint4* p = reinterpret_cast<const uint4*>(row);
  const uint4 a = p[0], b = p[1];
  const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    v[2 * q] += lo16(u[q]);
    v[2 * q + 1] += hi16(u[q]);
  }
}

// Workgroup tile: 64 tokens x 256 features; wave w takes tokens
// 32*(w&1) .. +31 (MFMA columns) and features 128*(w>>1) .. +127 (four
// 32-row MFMA blocks).  Lane l's MFMA row l&31 reads feature fmap(l&31), so
// that accumulator register r of lane l is feature 16*(l>>5) + r of its block.
template <bool ROUTER>
__global__ __launch_bounds__(256) void input_grad_kernel(InputGradArgs a) {
  const int d = a.d, k = a.k, Ep = a.Ep;
  const int nft = (d + 255) / 256;
  const int64_t tile = blockIdx.x;
  const int ft = (int)(tile % nft);
  const int64_t tt = tile / nft;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int64_t tb = tt * 64 + (wave & 1) * 32 + n;
  const int fw = ft * 256 + (wave >> 1) * 128;
  const bool tv = tb < a.T;
  f32x16 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;
  if constexpr (ROUTER) {
    const int fm = ((n >> 2) & 1) * 16 + (n >> 3) * 4 + (n & 3);
    const uint16_t* brow = a.dl_hl + (tv ? tb : 0) * 2 * Ep + 8 * hh;
    const bf16x8 zero = {};
    for (int kk = 0; kk < Ep; kk += 16) {
      const bf16x8 bh = tv ? ld8(brow + kk) : zero;
      const bf16x8 bl = tv ? ld8(brow + Ep + kk) : zero;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int fb = fw + 32 * b;
        if (fb < d) {
          const bf16x8 av = ld8(a.wrT + (int64_t)(fb + fm) * Ep + kk + 8 * hh);
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bh, acc[b], 0, 0, 0);
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bl, acc[b], 0, 0, 0);
        }
      }
    }
  }
  if (!tv) return;
  int64_t r0 = -1, r1 = -1;
  {
    const int s0 = a.slot[tb * k];
    if (s0 >= 0) r0 = (int64_t)a.offset[a.idx[tb * k]] + s0;
    if (k == 2) {
      const int s1 = a.slot[tb * k + 1];
      if (s1 >= 0) r1 = (int64_t)a.offset[a.idx[tb * k + 1]] + s1;
    }
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int f0 = fw + 32 * b + 16 * hh;
    if (fw + 32 * b >= d) break;
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = 0.f;
    if (r0 >= 0) add16(v, a.dx_disp + r0 * d + f0);
    if (r1 >= 0) add16(v, a.dx_disp + r1 * d + f0);
    if constexpr (ROUTER) {
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] += acc[b][r];
    }
    uint4* p = reinterpret_cast<uint4*>(a.dx + tb * d + f0);
    p[0] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7]));
    p[1] = make_uint4(pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]),
                      pack_bf16x2(v[14], v[15]));
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

// db[e] = sum of the gate-backward workgroups' partial sums: 64 experts per
// workgroup, the four waves take contiguous quarters of the partial rows and
// are added in wave order.
__global__ __launch_bounds__(256) void db_reduce_kernel(const float* __restrict__ dbpart, int nb, int E,
                                                        float* __restrict__ db) {
  __shared__ float s[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int per = (nb + 3) / 4;
  const int b0 = wave * per, b1 = min(nb, b0 + per);
  float acc = 0.f;
  if (e < E)
    for (int b = b0; b < b1; ++b) acc += dbpart[(int64_t)b * E + e];
  s[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && e < E) db[e] = ((s[0][lane] + s[1][lane]) + s[2][lane]) + s[3][lane];
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

hipError_t launch_router_transpose(const void* w_router, uint16_t* wrT, int E, int d, int Ep, hipStream_t s) {
  const int64_t n = (int64_t)d * Ep;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(router_transpose_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const uint16_t*>(w_router), wrT, E, d, Ep);
  return hipGetLastError();
}

hipError_t launch_input_grad(const InputGradArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t tiles = ((a.T + 63) / 64) * ((a.d + 255) / 256);
  if (a.dl_hl)
    hipLaunchKernelGGL(input_grad_kernel<true>, dim3((unsigned)tiles), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(input_grad_kernel<false>, dim3((unsigned)tiles), dim3(256), 0, s, a);
  return hipGetLastError();
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
    hipLaunchKernelGGL(db_reduce_kernel, dim3((a.E + 63) / 64), dim3(256), 0, s, a.dbpart, nb, a.E, a.db_router);
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

}  // namespace moe
