// Dispatch (token rows -> packed expert-major rows) and gate-weighted
// combine (packed rows -> token order).
//
// What is computed ("MoE混合专家架构：大模型高效推理的智能调度原理" §3.1,
// MoELayer Step 3 flatten-and-scatter into one [tokens_of_expert, hidden]
// tensor per expert, and Step 5 gather with the top-k weights back to the
// input's shape; "deepspeed.moe 模块" overview §3.1 steps 2 and 4):
//   dispatch: x_disp[offset[e] + slot[t,j]] = x[t] for every kept (t, j)
//   combine:  out[t] = sum_{kept j, in order} w[t,j] * y_disp[row(t,j)]
//
// Design (gfx950): one wavefront per token.  Every row here is at least a
// few hundred contiguous bytes, so each lane moves 16-byte vectors and a
// wavefront covers 1 KiB of a row per instruction: loads and stores are fully
// coalesced without an LDS staging step.  Dispatch reads each token row once
// and writes it to each of its kept destinations (scatter form, so x is read
// T times, not k*T).  Combine is the gather form: each output row is written
// exactly once, the fp32 sum runs in choice order with no atomics, and a
// token whose claims were all dropped gets zeros.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }


__global__ __launch_bounds__(256) void dispatch_kernel(const u32x4* __restrict__ x,
                                                       const int32_t* __restrict__ expert_idx,
                                                       const int32_t* __restrict__ slot,
                                                       const int32_t* __restrict__ offset,
                                                       u32x4* __restrict__ x_disp, int64_t T, int k,
                                                       int nvec) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t t = wave_id; t < T; t += nwaves) {
    int64_t r0 = -1, r1 = -1;
    {
      const int s0 = slot[t * k];
      if (s0 >= 0) r0 = (int64_t)offset[expert_idx[t * k]] + s0;
      if (k == 2) {
        const int s1 = slot[t * k + 1];
        if (s1 >= 0) r1 = (int64_t)offset[expert_idx[t * k + 1]] + s1;
      }
    }
    if (r0 < 0 && r1 < 0) continue;
    const u32x4* src = x + t * nvec;
    for (int v = lane; v < nvec; v += 64) {
      const u32x4 val = __builtin_nontemporal_load(src + v);
      if (r0 >= 0) x_disp[r0 * nvec + v] = val;
      if (r1 >= 0) x_disp[r1 * nvec + v] = val;
    }
  }
}

template <int DT>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4* __restrict__ y,
                                                      const int32_t* __restrict__ expert_idx,
                                                      const int32_t* __restrict__ slot,
                                                      const float* __restrict__ weight,
                                                      const int32_t* __restrict__ offset,
                                                      u32x4* __restrict__ out, int64_t T, int k,
                                                      int nvec) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
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
    u32x4* dst = out + t * nvec;
    for (int v = lane; v < nvec; v += 64) {
      if constexpr (DT == DT_BF16) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (r0 >= 0) {
          const u32x4 a = __builtin_nontemporal_load(y + r0 * nvec + v);
          const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] = w0 * bf16_lo(u[i]);
            acc[2 * i + 1] = w0 * bf16_hi(u[i]);
          }
        }
        if (r1 >= 0) {
          const u32x4 b = __builtin_nontemporal_load(y + r1 * nvec + v);
          const uint32_t u[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(w1, bf16_lo(u[i]), acc[2 * i]);
            acc[2 * i + 1] = fmaf(w1, bf16_hi(u[i]), acc[2 * i + 1]);
          }
        }
        u32x4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        dst[v] = o;
      } else {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        if (r0 >= 0) {
          const u32x4 a = y[r0 * nvec + v];
          acc[0] = w0 * __uint_as_float(a.x);
          acc[1] = w0 * __uint_as_float(a.y);
          acc[2] = w0 * __uint_as_float(a.z);
          acc[3] = w0 * __uint_as_float(a.w);
        }
        if (r1 >= 0) {
          const u32x4 b = y[r1 * nvec + v];
          acc[0] = fmaf(w1, __uint_as_float(b.x), acc[0]);
          acc[1] = fmaf(w1, __uint_as_float(b.y), acc[1]);
          acc[2] = fmaf(w1, __uint_as_float(b.z), acc[2]);
          acc[3] = fmaf(w1, __uint_as_float(b.w), acc[3]);
        }
        dst[v] = u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                       __float_as_uint(acc[3])};
      }
    }
  }
}

unsigned row_grid(int64_t T) {
  // enough waves to keep every CU streaming, capped so each wave loops a few times
  int64_t blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

}  // namespace

hipError_t launch_dispatch(const void* x, const int32_t* expert_idx, const int32_t* slot,
                           const int32_t* expert_offset, void* x_disp, int64_t T, int k, int row_bytes,
                           hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(dispatch_kernel, dim3(row_grid(T)), dim3(256), 0, s, static_cast<const u32x4*>(x),
                     expert_idx, slot, expert_offset, static_cast<u32x4*>(x_disp), T, k, row_bytes / 16);
  return hipGetLastError();
}

hipError_t launch_combine(const void* y_disp, const int32_t* expert_idx, const int32_t* slot,
                          const float* weight, const int32_t* expert_offset, void* out, int64_t T, int k,
                          int d, int dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int esize = dtype == DT_BF16 ? 2 : 4;
  const int nvec = d * esize / 16;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(combine_kernel<DT_BF16>, dim3(row_grid(T)), dim3(256), 0, s,
                       static_cast<const u32x4*>(y_disp), expert_idx, slot, weight, expert_offset,
                       static_cast<u32x4*>(out), T, k, nvec);
  else
    hipLaunchKernelGGL(combine_kernel<DT_F32>, dim3(row_grid(T)), dim3(256), 0, s,
                       static_cast<const u32x4*>(y_disp), expert_idx, slot, weight, expert_offset,
                       static_cast<u32x4*>(out), T, k, nvec);
  return hipGetLastError();
}

}  // namespace moe
