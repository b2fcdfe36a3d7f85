// Residual MoE (PR-MoE's use_residual): the mix of the MoE output with a
// dense MLP of the expert's architecture, and its backward.
//
// What is computed ("deepspeed.moe 模块" overview §2.1 use_residual, §2.3 and
// §3.3 PR-MoE: a fixed MLP combined with the dynamic experts through a
// residual connection; the mix is not on the pages, reading R16 takes the
// published layer's):
//   c[t]   = softmax(x[t] · W_c^T + b_c) over two entries, or (1, 1) without W_c
//   out[t] = c0 · sum over kept choices j of w[t,j] · y_disp[row(t,j)]
//          + c1 · mlp_y[t]
// The dense MLP runs on the grouped GEMM as one expert whose rows are all T
// tokens (offsets {0, T}); what is here is the per-token part.
//
// Design (gfx950): one wavefront per token, 16-byte lanes along the row,
// the two coefficient dot products reduced by xor-shuffles in a fixed order
// (so results are bit-identical run to run); fp32 sums, one rounding of the
// output.  The backward's per-token part reads dOut, the kept y rows and the
// MLP output once, writes dY_disp over y_disp and the MLP's upstream gradient
// over mlp_y (each row owned by one token), and returns the gate-weight and
// coefficient-logit gradients; W_c's gradient is a fixed-order sum over
// token chunks.
#include "moe_internal.h"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWaves = 4;   // wavefronts per workgroup, one token each in turn

__device__ __forceinline__ void unpack8(const u32x4 v, float (&f)[8]) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ void claims(const int32_t* expert_idx, const int32_t* slot, const float* weight,
                                       const int32_t* offset, int64_t t, int k, int64_t& r0, int64_t& r1, float& w0,
                                       float& w1) {
  r0 = r1 = -1;
  w0 = w1 = 0.f;
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

__global__ void residual_offsets_kernel(int32_t* off, int64_t T) {
  if (threadIdx.x == 0) {
    off[0] = 0;
    off[1] = (int32_t)T;
  }
}

__global__ __launch_bounds__(256) void residual_combine_kernel(ResidualArgs a) {
  const int lane = threadIdx.x & 63;
  const int nvec = a.d / 8;
  const u32x4* x = reinterpret_cast<const u32x4*>(a.x);
  const u32x4* y = reinterpret_cast<const u32x4*>(a.y_disp);
  const u32x4* my = reinterpret_cast<const u32x4*>(a.mlp_y);
  const u32x4* cw = reinterpret_cast<const u32x4*>(a.coef_w);
  u32x4* out = reinterpret_cast<u32x4*>(a.out);
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); t < a.T; t += nw) {
    float c0 = 1.f, c1 = 1.f;
    if (cw) {
      float l0 = 0.f, l1 = 0.f;
      for (int v = lane; v < nvec; v += 64) {
        float xf[8], w0f[8], w1f[8];
        unpack8(x[t * nvec + v], xf);
        unpack8(cw[v], w0f);
        unpack8(cw[nvec + v], w1f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          l0 = fmaf(xf[i], w0f[i], l0);
          l1 = fmaf(xf[i], w1f[i], l1);
        }
      }
      l0 = wave_sum(l0) + (a.coef_b ? a.coef_b[0] : 0.f);
      l1 = wave_sum(l1) + (a.coef_b ? a.coef_b[1] : 0.f);
      const float m = fmaxf(l0, l1);
      const float e0 = expf(l0 - m), e1 = expf(l1 - m);
      c0 = e0 / (e0 + e1);
      c1 = e1 / (e0 + e1);
    }
    if (lane == 0) {
      a.coef[2 * t] = c0;
      a.coef[2 * t + 1] = c1;
      if (a.coef_out) {
        a.coef_out[2 * t] = c0;
        a.coef_out[2 * t + 1] = c1;
      }
    }
    int64_t r0, r1;
    float w0, w1;
    claims(a.expert_idx, a.slot, a.weight, a.offset, t, a.k, r0, r1, w0, w1);
    for (int v = lane; v < nvec; v += 64) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, f[8];
      if (r0 >= 0) {
        unpack8(y[r0 * nvec + v], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = w0 * f[i];
      }
      if (r1 >= 0) {
        unpack8(y[r1 * nvec + v], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(w1, f[i], acc[i]);
      }
      unpack8(my[t * nvec + v], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = c0 * acc[i] + c1 * f[i];
      out[t * nvec + v] = pack8(acc);
    }
  }
}

// Per token: dY_disp rows = w_j c0 dOut (over y_disp), the gate-weight
// gradient c0 <dOut, y_j>, the MLP's upstream c1 dOut (over mlp_y), and with
// coefficient weights the logit gradient dl = c (dc - <c, dc>) of
// dc = (<dOut, sum_j w_j y_j>, <dOut, mlp_y>).
__global__ __launch_bounds__(256) void residual_combine_backward_kernel(ResidualArgs a) {
  constexpr int U = 4;
  const int lane = threadIdx.x & 63;
  const int nvec = a.d / 8;
  const u32x4* dout = reinterpret_cast<const u32x4*>(a.dout);
  u32x4* y = reinterpret_cast<u32x4*>(a.y_disp);   // y rows in, dY rows out
  u32x4* my = reinterpret_cast<u32x4*>(a.mlp_y);   // MLP output in, its upstream gradient out
  const u32x4 z = {0u, 0u, 0u, 0u};
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); t < a.T; t += nw) {
    const float c0 = a.coef[2 * t], c1 = a.coef[2 * t + 1];
    int64_t r0, r1;
    float w0, w1;
    claims(a.expert_idx, a.slot, a.weight, a.offset, t, a.k, r0, r1, w0, w1);
    float dot0 = 0.f, dot1 = 0.f, dotm = 0.f;
    for (int v0 = lane; v0 < nvec; v0 += 64 * U) {
      u32x4 o[U], ya[U], yb[U], ym[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + 64 * u;
        const bool in = v < nvec;
        o[u] = in ? dout[t * nvec + v] : z;
        ya[u] = (in && r0 >= 0) ? y[r0 * nvec + v] : z;
        yb[u] = (in && r1 >= 0) ? y[r1 * nvec + v] : z;
        ym[u] = in ? my[t * nvec + v] : z;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + 64 * u;
        if (v >= nvec) break;
        float of[8], fa[8], fb[8], fm[8], g[8];
        unpack8(o[u], of);
        unpack8(ya[u], fa);
        unpack8(yb[u], fb);
        unpack8(ym[u], fm);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dot0 = fmaf(of[i], fa[i], dot0);
          dot1 = fmaf(of[i], fb[i], dot1);
          dotm = fmaf(of[i], fm[i], dotm);
        }
        if (r0 >= 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) g[i] = w0 * (c0 * of[i]);
          y[r0 * nvec + v] = pack8(g);
        }
        if (r1 >= 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) g[i] = w1 * (c0 * of[i]);
          y[r1 * nvec + v] = pack8(g);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = c1 * of[i];
        my[t * nvec + v] = pack8(g);
      }
    }
    dot0 = wave_sum(dot0);
    dot1 = wave_sum(dot1);
    dotm = wave_sum(dotm);
    if (lane == 0) {
      a.dw[t * a.k] = r0 >= 0 ? c0 * dot0 : 0.f;
      if (a.k == 2) a.dw[t * a.k + 1] = r1 >= 0 ? c0 * dot1 : 0.f;
      if (a.dlc) {
        const float dc0 = (r0 >= 0 ? w0 * dot0 : 0.f) + (r1 >= 0 ? w1 * dot1 : 0.f);
        const float dc1 = dotm;
        const float mean = c0 * dc0 + c1 * dc1;
        a.dlc[2 * t] = c0 * (dc0 - mean);
        a.dlc[2 * t + 1] = c1 * (dc1 - mean);
      }
    }
  }
}

// dW_c partials: workgroup b sums tokens [b*kCoefChunk, (b+1)*kCoefChunk) of
// dl^T x for 8 columns per thread (16-byte loads along the row), and the
// chunk's column sums of dl for db_c; the reduce adds the chunks in order.
constexpr int kCoefChunk = 64;

__global__ __launch_bounds__(256) void coef_wgrad_partial_kernel(ResidualArgs a) {
  const int nvec = a.d / 8;
  const u32x4* x = reinterpret_cast<const u32x4*>(a.x);
  const int64_t t0 = (int64_t)blockIdx.x * kCoefChunk;
  const int64_t t1 = t0 + kCoefChunk < a.T ? t0 + kCoefChunk : a.T;
  for (int v = threadIdx.x; v < nvec; v += 256) {
    float s0[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, s1[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int64_t t = t0; t < t1; ++t) {
      float xf[8];
      unpack8(x[t * nvec + v], xf);
      const float g0 = a.dlc[2 * t], g1 = a.dlc[2 * t + 1];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s0[i] = fmaf(g0, xf[i], s0[i]);
        s1[i] = fmaf(g1, xf[i], s1[i]);
      }
    }
    float* p = a.cw_part + (int64_t)blockIdx.x * 2 * a.d;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[8 * v + i] = s0[i];
      p[a.d + 8 * v + i] = s1[i];
    }
  }
  if (threadIdx.x < 2) {
    float s = 0.f;
    for (int64_t t = t0; t < t1; ++t) s += a.dlc[2 * t + threadIdx.x];
    a.cb_part[2 * blockIdx.x + threadIdx.x] = s;
  }
}

__global__ __launch_bounds__(256) void coef_wgrad_reduce_kernel(ResidualArgs a, int nchunk) {
  const int64_t n = 2 * (int64_t)a.d;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float s = 0.f;
    for (int c = 0; c < nchunk; ++c) s += a.cw_part[(int64_t)c * n + i];
    if (a.dcoef_w) a.dcoef_w[i] = s;
  }
  if (blockIdx.x == 0 && threadIdx.x < 2 && a.dcoef_b) {
    float s = 0.f;
    for (int c = 0; c < nchunk; ++c) s += a.cb_part[2 * c + threadIdx.x];
    a.dcoef_b[threadIdx.x] = s;
  }
}

unsigned grid_for(int64_t T) {
  const int64_t g = (T + kWaves - 1) / kWaves;
  return (unsigned)(g < 8192 ? (g > 0 ? g : 1) : 8192);
}

}  // namespace

int residual_coef_chunks(int64_t T) { return (int)((T + kCoefChunk - 1) / kCoefChunk); }

hipError_t launch_residual_offsets(int32_t* off, int64_t T, hipStream_t s) {
  hipLaunchKernelGGL(residual_offsets_kernel, dim3(1), dim3(64), 0, s, off, T);
  return hipGetLastError();
}

hipError_t launch_residual_combine(const ResidualArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(residual_combine_kernel, dim3(grid_for(a.T)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_residual_combine_backward(const ResidualArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(residual_combine_backward_kernel, dim3(grid_for(a.T)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_coef_wgrad(const ResidualArgs& a, hipStream_t s) {
  const int nchunk = residual_coef_chunks(a.T);
  if (nchunk > 0) {
    hipLaunchKernelGGL(coef_wgrad_partial_kernel, dim3((unsigned)nchunk), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n = 2 * (int64_t)a.d;
  const unsigned g = (unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(coef_wgrad_reduce_kernel, dim3(g), dim3(256), 0, s, a, nchunk);
  return hipGetLastError();
}

}  // namespace moe
