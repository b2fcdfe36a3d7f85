// Grouped GEMM of the expert FFNs on the packed expert-major buffer.
//
// What is computed ("MoE混合专家架构：大模型高效推理的智能调度原理" §3.1,
// MoELayer item 2 and Step 4: every expert is Linear -> GELU -> Linear and
// runs on the tokens routed to it; "deepspeed.moe 模块" overview §2.1, whose
// example expert is one nn.Linear):
//   for each expert e and its rows R_e = [offset[e], offset[e+1]):
//     Y[R_e] = act(X[R_e] · W[e]^T + bias[e])      W[e] is [N, K] (nn.Linear)
// with fp32 accumulation, bias and activation in fp32, one rounding to the
// storage type.  Run twice per FFN (Linear1 + activation, then Linear2).
//
// Design (gfx950, bf16):
//  * Workgroup tile BT tokens x BF features, 4 waves in a WT x WF grid, the
//    K dimension in 64-wide steps staged through double-buffered LDS
//    (global -> registers -> LDS, one barrier per step).  LDS rows are padded
//    to 144 bytes so the 16-byte fragment reads of 8 consecutive lanes fall
//    in distinct bank groups.
//  * v_mfma_f32_32x32x16_bf16 with weights on the MFMA row side and tokens on
//    the column side.  Weight rows are stored into LDS in a permuted order so
//    that each lane's 16 accumulators are 16 consecutive output features of
//    one token: the epilogue writes two 16-byte vectors per lane.
//  * Within one 64-wide K step a lane reads 32 contiguous k values of its row
//    for 4 MFMAs (k is permuted identically on both operands, which leaves
//    the dot product unchanged).
//  * Ragged rows need no host synchronisation: the grid is sized for the
//    worst case, each workgroup recomputes the per-expert tile prefix from
//    expert_offset (a wavefront scan) and exits if it has no tile.  Tiles are
//    ordered expert -> group of 8 row tiles -> feature tile -> row tile, so
//    workgroups running together share one weight tile, and the blockIdx ->
//    tile map gives every XCD one contiguous run of tiles (XCDs take
//    workgroups round-robin), keeping each expert's working set in one L2.
// The fp32 path (small problems only) is a plain FMA kernel.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBK = 64;              // K elements per step
constexpr int kRowBytes = kBK * 2 + 16;  // padded LDS row
constexpr int kGroupM = 8;           // row tiles per scheduling group
constexpr int kXcds = 8;

__device__ __forceinline__ int lds_row_of_feature(int f) {
  // feature f (0..31) of a 32-row block is stored at this LDS row so that the
  // MFMA row m = lane&31 reads feature ((m>>2)&1)*16 + (m>>3)*4 + (m&3)
  return ((f >> 2) & 3) * 8 + (f >> 4) * 4 + (f & 3);
}

__device__ __forceinline__ float act_apply(float v, int act) {
  if (act == ACT_RELU) return fmaxf(v, 0.f);
  if (act == ACT_GELU) return 0.5f * v * (1.f + erff(v * 0.7071067811865476f));
  return v;
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16 l = static_cast<bf16>(lo);
  const bf16 h = static_cast<bf16>(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

// Tile scheduler shared by the kernels: per-expert row-tile prefix (exclusive)
// in s_pref[0..E], computed by wavefront 0.  E <= 256.
template <int BT>
__device__ __forceinline__ void tile_prefix(const int32_t* __restrict__ offset, int E, int* s_pref) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) == 0) {
    int c[4];
    int s = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane * 4 + r;
      c[r] = e < E ? (offset[e + 1] - offset[e] + BT - 1) / BT : 0;
      s += c[r];
    }
    int incl = s;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int v = __shfl_up(incl, m);
      if (lane >= m) incl += v;
    }
    int excl = incl - s;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane * 4 + r;
      if (e <= E) s_pref[e] = excl;
      excl += c[r];
    }
    if (lane == 63 && E == MOE_MAX_EXPERTS_DEV) s_pref[E] = incl;
  }
}

struct TileCoord {
  int e, mt, nf;
};

// Map a linear tile id to (expert, row tile, feature tile).
__device__ __forceinline__ TileCoord tile_coord(int tile, const int* s_pref, int E, int ntf) {
  int lo = 0, hi = E;  // find e with s_pref[e]*ntf <= tile < s_pref[e+1]*ntf
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] * ntf <= tile) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int mte = s_pref[e + 1] - s_pref[e];
  const int local = tile - s_pref[e] * ntf;
  const int mg = local / (kGroupM * ntf);
  const int rem = local - mg * kGroupM * ntf;
  const int gs = min(kGroupM, mte - mg * kGroupM);
  TileCoord c;
  c.e = e;
  c.nf = rem / gs;
  c.mt = mg * kGroupM + (rem - c.nf * gs);
  return c;
}

template <int BT, int BF, int WT, int WF>
__global__ __launch_bounds__(WT * WF * 64) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int NTH = WT * WF * 64;
  constexpr int TW = BT / WT, FW = BF / WF;
  constexpr int NTT = TW / 32, NFF = FW / 32;
  constexpr int STAGE = (BT + BF) * kRowBytes;
  constexpr int CH = (BT + BF) * 8 / NTH;  // 16-byte chunks per thread per step
  static_assert((BT + BF) * 8 % NTH == 0, "chunks must divide evenly");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_pref[MOE_MAX_EXPERTS_DEV + 1];

  const int E = a.E, N = a.N, K = a.K;
  const int ntf = (N + BF - 1) / BF;
  tile_prefix<BT>(a.offset, E, s_pref);
  __syncthreads();
  const int total = s_pref[E] * ntf;
  const int share = (total + kXcds - 1) / kXcds;
  const int loc = blockIdx.x / kXcds;
  const int tile = (blockIdx.x % kXcds) * share + loc;
  if (loc >= share || tile >= total) return;
  const TileCoord tc = tile_coord(tile, s_pref, E, ntf);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wt = wave / WF, wf = wave % WF;
  const int row0 = a.offset[tc.e];
  const int mrows = a.offset[tc.e + 1] - row0;
  const int mbase = tc.mt * BT;              // first row of the tile within the expert
  const int mvalid = min(BT, mrows - mbase);
  const int n0 = tc.nf * BF;

  const bf16* X = static_cast<const bf16*>(a.X) + (int64_t)(row0 + mbase) * K;
  const bf16* W = static_cast<const bf16*>(a.W) + ((int64_t)tc.e * N + n0) * K;

  // per-thread chunk descriptors (fixed across K steps)
  const bf16* gsrc[CH];
  int ldst[CH];
  bool gval[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + i * NTH;
    const int row = c >> 3, col = c & 7;
    if (row < BT) {
      gval[i] = row < mvalid;
      gsrc[i] = X + (int64_t)row * K + col * 8;
      ldst[i] = row * kRowBytes + col * 16;
    } else {
      const int f = row - BT;
      gval[i] = n0 + f < N;
      gsrc[i] = W + (int64_t)f * K + col * 8;
      ldst[i] = (BT + (f & ~31) + lds_row_of_feature(f & 31)) * kRowBytes + col * 16;
    }
  }

  f32x16 acc[NFF][NTT];
#pragma unroll
  for (int i = 0; i < NFF; ++i)
#pragma unroll
    for (int j = 0; j < NTT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 stage[CH];
  const int nk = (K + kBK - 1) / kBK;
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int kcol = k0 + ((tid + i * NTH) & 7) * 8;
      stage[i] = (gval[i] && kcol < K) ? *reinterpret_cast<const uint4*>(gsrc[i] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) *reinterpret_cast<uint4*>(smem + buf * STAGE + ldst[i]) = stage[i];
  };

  gload(0);
  lstore(0);
  __syncthreads();
  const int hsel = lane >> 5, r32 = lane & 31;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
    const unsigned char* Xs = smem + cur * STAGE;
    const unsigned char* Ws = Xs + BT * kRowBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kb = (hsel * 32 + i * 8) * 2;
      bf16x8 af[NFF], bx[NTT];
#pragma unroll
      for (int ff = 0; ff < NFF; ++ff)
        af[ff] = *reinterpret_cast<const bf16x8*>(Ws + (wf * FW + ff * 32 + r32) * kRowBytes + kb);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
        bx[tt] = *reinterpret_cast<const bf16x8*>(Xs + (wt * TW + tt * 32 + r32) * kRowBytes + kb);
#pragma unroll
      for (int ff = 0; ff < NFF; ++ff)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
          acc[ff][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ff], bx[tt], acc[ff][tt], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds 16 consecutive features of one token per (ff, tt)
  const bf16* bias = static_cast<const bf16*>(a.bias);
  bf16* Y = static_cast<bf16*>(a.Y);
  bf16* Apre = static_cast<bf16*>(a.Apre);
#pragma unroll
  for (int ff = 0; ff < NFF; ++ff) {
    const int f0 = n0 + wf * FW + ff * 32 + hsel * 16;
    float bv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) bv[r] = 0.f;
    if (bias) {
      const bf16* bp = bias + (int64_t)tc.e * N + f0;
#pragma unroll
      for (int r = 0; r < 16; ++r) bv[r] = (f0 + r < N) ? static_cast<float>(bp[r]) : 0.f;
    }
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const int rloc = wt * TW + tt * 32 + r32;
      if (rloc >= mvalid) continue;
      const int64_t grow = (int64_t)row0 + mbase + rloc;
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = acc[ff][tt][r] + bv[r];
      if (f0 + 16 <= N) {
        if (Apre) {
          uint4* p = reinterpret_cast<uint4*>(Apre + grow * N + f0);
          p[0] = make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
          p[1] = make_uint4(pack2(v[8], v[9]), pack2(v[10], v[11]), pack2(v[12], v[13]), pack2(v[14], v[15]));
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = act_apply(v[r], a.act);
        uint4* p = reinterpret_cast<uint4*>(Y + grow * N + f0);
        p[0] = make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
        p[1] = make_uint4(pack2(v[8], v[9]), pack2(v[10], v[11]), pack2(v[12], v[13]), pack2(v[14], v[15]));
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (f0 + r < N) {
            if (Apre) Apre[grow * N + f0 + r] = static_cast<bf16>(v[r]);
            Y[grow * N + f0 + r] = static_cast<bf16>(act_apply(v[r], a.act));
          }
        }
      }
    }
  }
}

// fp32: one thread per output element (used for the small fp32 layers).
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  const int n = blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t row = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
  const int E = a.E;
  if (n >= a.N || row >= a.offset[E]) return;
  int lo = 0, hi = E;  // offset[lo] <= row < offset[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.offset[mid] <= row) lo = mid; else hi = mid;
  }
  const float* x = static_cast<const float*>(a.X) + row * a.K;
  const float* w = static_cast<const float*>(a.W) + ((int64_t)lo * a.N + n) * a.K;
  float s = 0.f;
  for (int k = 0; k < a.K; ++k) s = fmaf(x[k], w[k], s);
  if (a.bias) s += static_cast<const float*>(a.bias)[(int64_t)lo * a.N + n];
  if (a.Apre) static_cast<float*>(a.Apre)[row * a.N + n] = s;
  static_cast<float*>(a.Y)[row * a.N + n] = act_apply(s, a.act);
}

template <int BT, int BF, int WT, int WF>
hipError_t launch_bf16(const GemmArgs& a, hipStream_t s) {
  constexpr int STAGE = (BT + BF) * kRowBytes;
  constexpr size_t lds = 2 * (size_t)STAGE;
  auto kern = gemm_bf16_kernel<BT, BF, WT, WF>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t max_mtiles = (a.max_rows + BT - 1) / BT + a.E;
  const int64_t ntf = (a.N + BF - 1) / BF;
  int64_t grid = max_mtiles * ntf;
  grid = (grid + kXcds - 1) / kXcds * kXcds;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WT * WF * 64), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmArgs& a, int dtype, hipStream_t s) {
  if (a.max_rows <= 0) return hipSuccess;
  if (dtype == DT_BF16) return launch_bf16<128, 128, 2, 2>(a, s);
  dim3 grid((a.N + 63) / 64, (unsigned)((a.max_rows + 3) / 4));
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
