// Gate of the MoE layer: router GEMM, softmax, top-k, capacity slots,
// expert counts and gate_loss, as one single-pass kernel plus a small slot
// fix-up kernel.
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
//  * One workgroup (4 waves) per tile of 64 tokens (32 when E > 128).  Tiles
//    are numbered by an atomic ticket, so every lower tile is already
//    resident when a tile looks back at it.
//  * Router GEMM on MFMA v_mfma_f32_16x16x32_bf16 with experts on the MFMA
//    row side and tokens on the column side: a lane ends up holding 4
//    consecutive experts of one token, and a token's E logits sit in the 4
//    lanes {n, n+16, n+32, n+48}.  The hidden dimension is split over the 4
//    waves in 128-wide steps (each lane streams 64 contiguous bytes of its x
//    row per step; the four lane quarters cover 256 contiguous bytes) and the
//    partial logits are summed through LDS in a fixed order.
//  * Softmax and top-k are per-lane scans plus two xor-shuffles; ties go to
//    the lower index because every comparison is (value, index).
//  * Ranks inside the tile come from an LDS scan; ranks across tiles from a
//    decoupled look-back over per-(choice, expert) status words, one thread
//    per column, so the whole prefix sum is one pass over the tokens.
//  * Softmax column sums for the loss are reduced tile -> group of 32 tiles
//    -> all, each level by the last arriving workgroup, always summing in
//    index order, so the loss is bit-identical run to run.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr uint32_t ST_AGG = 1u << 30;   // word holds this tile's own count
constexpr uint32_t ST_INC = 2u << 30;   // word holds the inclusive prefix
constexpr uint32_t ST_VAL = (1u << 30) - 1u;

enum { MODE_LOGITS_IN = 0, MODE_BF16 = 1, MODE_F32 = 2 };

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Keep the better of (v, i) and the lane `mask` away: larger value, then
// lower index.
__device__ __forceinline__ void merge_best(float& v, int& i, int mask) {
  const float ov = __shfl_xor(v, mask);
  const int oi = __shfl_xor(i, mask);
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

template <int EP, int TG, int MODE>
__global__ __launch_bounds__(256) void gate_kernel(GateArgs a) {
  constexpr int NET = EP / 16;   // 16-expert MFMA row tiles
  constexpr int TT = TG * 16;    // tokens per tile
  constexpr size_t RED_BYTES = (MODE == MODE_BF16) ? size_t(4) * TG * NET * 64 * 16 : 0;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  f32x4* red = reinterpret_cast<f32x4*>(smem);                       // [4][TG][NET][64]
  int* s_sel = reinterpret_cast<int*>(smem + RED_BYTES);              // [2][TT]
  int* s_rnk = s_sel + 2 * TT;                                        // [2][TT]
  int* s_cnt = s_rnk + 2 * TT;                                        // [2*EP]
  int* s_base = s_cnt + 2 * EP;                                       // [2*EP]
  float* s_me = reinterpret_cast<float*>(s_base + 2 * EP);            // [TG][EP]
  double* s_dme = reinterpret_cast<double*>(s_me + TG * EP);          // [EP]
  __shared__ int s_tile;
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, n = lane & 15, q = lane >> 4;
  const int E = a.E, K = a.k, KE = a.k * a.E;
  const int64_t T = a.T;

  if (tid == 0) s_tile = (int)atomicAdd(&a.counters[0], 1u);
  __syncthreads();
  const int tile = s_tile;
  const int64_t t0 = (int64_t)tile * TT;

  // ------------------------------------------------------------ logits
  // lg[et][r] = logit of expert et*16 + q*4 + r for token t0 + wave*16 + n
  float lg[NET][4];
  if constexpr (MODE == MODE_BF16) {
    const bf16* x = static_cast<const bf16*>(a.x);
    const bf16* w = static_cast<const bf16*>(a.w_router);
    const int d = a.d;
    f32x4 acc[NET][TG];
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int g = 0; g < TG; ++g) acc[et][g] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 zero8 = {};
    const int nsteps = (d + 127) / 128;
    for (int ms = wave; ms < nsteps; ms += 4) {
      const int kb = ms * 128 + q * 32;
      bf16x8 xb[TG][4];
#pragma unroll
      for (int g = 0; g < TG; ++g) {
        const int64_t t = t0 + g * 16 + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = kb + i * 8;
          xb[g][i] = (t < T && kk < d) ? ld_bf16x8(x + t * d + kk) : zero8;
        }
      }
#pragma unroll
      for (int et = 0; et < NET; ++et) {
        const int e = et * 16 + n;
        bf16x8 wa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = kb + i * 8;
          wa[i] = (e < E && kk < d) ? ld_bf16x8(w + (int64_t)e * d + kk) : zero8;
        }
#pragma unroll
        for (int g = 0; g < TG; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[et][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[i], xb[g][i], acc[et][g], 0, 0, 0);
      }
    }
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int g = 0; g < TG; ++g) red[((wave * TG + g) * NET + et) * 64 + lane] = acc[et][g];
    __syncthreads();
    if (wave < TG) {
#pragma unroll
      for (int et = 0; et < NET; ++et) {
        f32x4 s = red[((0 * TG + wave) * NET + et) * 64 + lane];
#pragma unroll
        for (int ws = 1; ws < 4; ++ws) {
          const f32x4 o = red[((ws * TG + wave) * NET + et) * 64 + lane];
          s[0] += o[0];
          s[1] += o[1];
          s[2] += o[2];
          s[3] += o[3];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) lg[et][r] = s[r];
      }
    }
  } else if constexpr (MODE == MODE_F32) {
    if (wave < TG) {
      const float* x = static_cast<const float*>(a.x);
      const float* w = static_cast<const float*>(a.w_router);
      const int64_t t = t0 + wave * 16 + n;
#pragma unroll
      for (int et = 0; et < NET; ++et)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = et * 16 + q * 4 + r;
          float s = 0.f;
          if (t < T && e < E)
            for (int kk = 0; kk < a.d; ++kk) s = fmaf(x[t * a.d + kk], w[(int64_t)e * a.d + kk], s);
          lg[et][r] = s;
        }
    }
  } else {
    if (wave < TG) {
      const int64_t t = t0 + wave * 16 + n;
#pragma unroll
      for (int et = 0; et < NET; ++et)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = et * 16 + q * 4 + r;
          lg[et][r] = (t < T && e < E) ? a.logits_in[t * E + e] : 0.f;
        }
    }
  }

  // ------------------------------------------------------------ softmax, top-k
  if (wave < TG) {
    const int64_t t = t0 + wave * 16 + n;
    const bool tv = t < T;
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = et * 16 + q * 4 + r;
        if (e < E) {
          if (MODE != MODE_LOGITS_IN && a.b_router) lg[et][r] += a.b_router[e];
        } else {
          lg[et][r] = -INFINITY;
        }
      }
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
    float sum = 0.f;
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (et * 16 + q * 4 + r < E) sum += expf(lg[et][r] - mx);
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);

    // top-1
    float v0 = -INFINITY;
    int i0 = 0x7fffffff;
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = et * 16 + q * 4 + r;
        if (e < E && lg[et][r] > v0) {
          v0 = lg[et][r];
          i0 = e;
        }
      }
    merge_best(v0, i0, 16);
    merge_best(v0, i0, 32);
    // top-2 (best other than the top-1)
    float v1 = -INFINITY;
    int i1 = 0x7fffffff;
    if (K == 2) {
#pragma unroll
      for (int et = 0; et < NET; ++et)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = et * 16 + q * 4 + r;
          if (e < E && e != i0 && lg[et][r] > v1) {
            v1 = lg[et][r];
            i1 = e;
          }
        }
      merge_best(v1, i1, 16);
      merge_best(v1, i1, 32);
    }
    float p0 = expf(v0 - mx) / sum;
    float p1 = (K == 2) ? expf(v1 - mx) / sum : 0.f;
    if (a.normalize) {
      const float s = p0 + p1;
      p0 = p0 / s;
      p1 = p1 / s;
    }
    if (q == 0) {
      const int slot_in_tile = wave * 16 + n;
      s_sel[slot_in_tile] = tv ? i0 : -1;
      s_sel[TT + slot_in_tile] = (tv && K == 2) ? i1 : -1;
      if (tv) {
        a.expert_idx[t * K] = i0;
        a.weight[t * K] = p0;
        if (K == 2) {
          a.expert_idx[t * K + 1] = i1;
          a.weight[t * K + 1] = p1;
        }
      }
    }
    // per-tile column sums of p for the balance loss (16 tokens of this
    // wave by butterfly, then the TG waves in order below)
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = et * 16 + q * 4 + r;
        float pe = (tv && e < E) ? expf(lg[et][r] - mx) / sum : 0.f;
        pe += __shfl_xor(pe, 1);
        pe += __shfl_xor(pe, 2);
        pe += __shfl_xor(pe, 4);
        pe += __shfl_xor(pe, 8);
        if (n == 0 && e < EP) s_me[wave * EP + e] = pe;
      }
  }
  __syncthreads();

  // ------------------------------------------------------------ ranks in the tile
  for (int i = tid; i < K * TT; i += 256) {
    const int j = i / TT, nn = i - j * TT;
    const int e = s_sel[i];
    int r = 0;
    if (e >= 0)
      for (int m = 0; m < nn; ++m) r += (s_sel[j * TT + m] == e);
    s_rnk[i] = r;
  }
  for (int c = tid; c < KE; c += 256) {
    const int j = c / E, e = c - j * E;
    int cnt = 0;
    for (int m = 0; m < TT; ++m) cnt += (s_sel[j * TT + m] == e);
    s_cnt[c] = cnt;
  }
  for (int e = tid; e < E; e += 256) {
    float v = 0.f;
    for (int g = 0; g < TG; ++g) v += s_me[g * EP + e];
    a.me_tile[(int64_t)tile * E + e] = v;
  }
  __syncthreads();

  // ------------------------------------------------------------ decoupled look-back
  uint32_t* my = a.status + (int64_t)tile * KE;
  for (int c = tid; c < KE; c += 256) st_agent(&my[c], (tile == 0 ? ST_INC : ST_AGG) | (uint32_t)s_cnt[c]);
  for (int c = tid; c < KE; c += 256) {
    uint32_t prefix = 0;
    if (tile > 0) {
      int p = tile - 1;
      for (;;) {
        const uint32_t v = ld_agent(&a.status[(int64_t)p * KE + c]);
        if ((v & ~ST_VAL) == 0) {
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        prefix += v & ST_VAL;
        if (v & ST_INC) break;
        --p;
      }
      st_agent(&my[c], ST_INC | (prefix + (uint32_t)s_cnt[c]));
    }
    s_base[c] = (int)prefix;
  }
  __syncthreads();
  for (int i = tid; i < K * TT; i += 256) {
    const int j = i / TT, nn = i - j * TT;
    const int e = s_sel[i];
    if (e >= 0) a.slot[(t0 + nn) * K + j] = s_base[j * E + e] + s_rnk[i];
  }

  // ------------------------------------------------------------ loss sums: tile -> group
  __threadfence();
  __syncthreads();
  const int grp = tile / kGateGroupTiles;
  const int g_first = grp * kGateGroupTiles;
  const int g_last = min(g_first + kGateGroupTiles, a.num_tiles);
  if (tid == 0) s_last = (atomicAdd(&a.counters[2 + grp], 1u) == (uint32_t)(g_last - g_first - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int e = tid; e < E; e += 256) {
    float v = 0.f;
    for (int p = g_first; p < g_last; ++p) v += a.me_tile[(int64_t)p * E + e];
    a.me_group[(int64_t)grp * E + e] = v;
  }
  // ------------------------------------------------------------ group -> all; finalize
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&a.counters[1], 1u) == (uint32_t)(a.num_groups - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  const uint32_t* last = a.status + (int64_t)(a.num_tiles - 1) * KE;
  for (int c = tid; c < KE; c += 256) {
    const int v = (int)(ld_agent(&last[c]) & ST_VAL);
    s_cnt[c] = v;
    a.demand[c] = v;
  }
  __syncthreads();
  const int64_t C = a.C;
  for (int e = tid; e < E; e += 256) {
    const int64_t d0 = s_cnt[e];
    const int64_t d1 = (K == 2) ? s_cnt[E + e] : 0;
    int64_t kept;
    if (C < 0) {
      kept = d0 + d1;
    } else {
      kept = d0 < C ? d0 : C;
      if (K == 2) {
        const int64_t room = C - d0;
        kept += room <= 0 ? 0 : (d1 < room ? d1 : room);
      }
    }
    a.expert_count[e] = (int32_t)kept;
    s_base[e] = (int)kept;
    double me = 0.0;
    for (int g = 0; g < a.num_groups; ++g) me += (double)a.me_group[(int64_t)g * E + e];
    s_dme[e] = me;
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      a.expert_offset[e] = acc;
      acc += s_base[e];
    }
    a.expert_offset[E] = acc;
    double loss = 0.0;
    if (T > 0) {
      if (a.loss_kind == LOSS_BALANCE) {
        for (int e = 0; e < E; ++e) loss += (s_dme[e] / (double)T) * ((double)s_cnt[e] / (double)T);
        loss *= (double)E;
      } else {
        const double denom = (double)K * (double)T;
        double mean = 0.0;
        for (int e = 0; e < E; ++e) mean += (double)(s_cnt[e] + (K == 2 ? s_cnt[E + e] : 0)) / denom;
        mean /= (double)E;
        double var = 0.0;
        for (int e = 0; e < E; ++e) {
          const double u = (double)(s_cnt[e] + (K == 2 ? s_cnt[E + e] : 0)) / denom - mean;
          var += u * u;
        }
        loss = sqrt(var / (double)E) + 1e-6;
      }
    }
    *a.gate_loss = (float)loss;
  }
}

__global__ void zero_u32_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Final slots: choice 0 keeps its rank; choice 1 adds the expert's total
// choice-0 demand; a slot at or past the capacity is dropped.
__global__ void slot_finalize_kernel(const int32_t* __restrict__ expert_idx, int32_t* __restrict__ slot,
                                     const int32_t* __restrict__ demand, int64_t n, int k, int64_t C) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int j = (int)(i % k);
  const int e = expert_idx[i];
  int64_t s = slot[i];
  if (j == 1) s += demand[e];
  slot[i] = (C >= 0 && s >= C) ? -1 : (int32_t)s;
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
  constexpr int NET = EP / 16, TT = TG * 16;
  size_t red = (MODE == MODE_BF16) ? size_t(4) * TG * NET * 64 * 16 : 0;
  return red + 4 * (2 * TT + 2 * TT + 2 * EP + 2 * EP + TG * EP) + 8 * EP;
}

template <int EP, int TG, int MODE>
hipError_t launch_gate_t(const GateArgs& a, hipStream_t s) {
  const size_t lds = gate_lds_bytes<EP, TG, MODE>();
  auto kern = gate_kernel<EP, TG, MODE>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(a.num_tiles), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_gate_mode(const GateArgs& a, hipStream_t s) {
  const int E = a.E;
  if (E <= 16) return launch_gate_t<16, 4, MODE>(a, s);
  if (E <= 32) return launch_gate_t<32, 4, MODE>(a, s);
  if (E <= 64) return launch_gate_t<64, 4, MODE>(a, s);
  if (E <= 128) return launch_gate_t<128, 4, MODE>(a, s);
  return launch_gate_t<256, 2, MODE>(a, s);
}

}  // namespace

size_t gate_sync_words(int64_t T, int E, int k) {
  const int tt = gate_tile_tokens(E);
  const int64_t tiles = (T + tt - 1) / tt;
  const int64_t groups = (tiles + kGateGroupTiles - 1) / kGateGroupTiles;
  return (size_t)(2 + groups) + (size_t)tiles * k * E;
}

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_gate(const GateArgs& a, int dtype, hipStream_t s) {
  if (a.logits_in) return launch_gate_mode<MODE_LOGITS_IN>(a, s);
  if (dtype == DT_BF16) return launch_gate_mode<MODE_BF16>(a, s);
  return launch_gate_mode<MODE_F32>(a, s);
}

hipError_t launch_slot_finalize(const int32_t* expert_idx, int32_t* slot, const int32_t* demand,
                                int64_t T, int k, int E, int64_t C, hipStream_t s) {
  (void)E;
  const int64_t n = T * k;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     expert_idx, slot, demand, n, k, C);
  return hipGetLastError();
}

hipError_t launch_gate_empty(int32_t* expert_count, int32_t* expert_offset, float* gate_loss, int E,
                             hipStream_t s) {
  hipLaunchKernelGGL(gate_empty_kernel, dim3(1), dim3(256), 0, s, expert_count, expert_offset, gate_loss, E);
  return hipGetLastError();
}

}  // namespace moe
