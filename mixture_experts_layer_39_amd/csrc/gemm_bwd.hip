// Backward of the expert FFNs on the packed expert-major buffer.
//
// For the rows R_e of expert e, with X = x_disp, A = saved pre-activation,
// H = act(A), dY the upstream gradient (chain rule of Linear-act-Linear, the
// expert of "MoE混合专家架构：大模型高效推理的智能调度原理" §3.1 item 2):
//   dH  = dY · W2[e]              (W2[e] is [d, h]: contraction over d)
//   dA  = dH ⊙ act'(A)            (stored as bf16)
//   dX  = dA · W1[e]              (W1[e] is [h, d]: contraction over h)
//   dW2[e] = dY^T · H             (contraction over the rows of the expert)
//   dW1[e] = dA^T · X
//   db2[e] = colsum dY,  db1[e] = colsum dA   (fp32, optional)
//
// Design (gfx950): one register-staged MFMA kernel (128 x 128 tile, 4 waves
// of 64 x 64, v_mfma_f32_32x32x16_bf16, K in 64-wide steps through
// double-buffered LDS).  Its two operand loaders read either a K-contiguous
// source (16-byte chunks straight to LDS rows) or a row-contiguous source:
// then a thread fetches an 8 (k) x 8 (row) block as eight 16-byte loads,
// transposes it in registers with v_perm and writes eight K-contiguous
// 16-byte LDS rows, so the MFMA operands always see K-contiguous rows and no
// weight or activation tensor is ever transposed in HBM.
//   dgrad (dH, dX): tokens of the expert on the MFMA column side (ragged, tile
//     list from expert_offset), weights row-contiguous on the row side;
//   wgrad (dW1, dW2): both operands row-contiguous, K = the expert's rows
//     (ragged, zero-padded); one tile list per expert, experts with no rows
//     write zeros.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBK = 64;
constexpr int kRowB = kBK * 2 + 16;  // padded LDS row: 144 bytes
constexpr int kT = 128;              // tile edge (tokens and features)
constexpr int kXcds = 8;

enum { L_KC = 0, L_RC = 1 };                    // operand layouts
enum { EPI_STORE = 0, EPI_DACT = 1 };           // epilogues
enum { M_ROWS = 0, M_WGRAD = 1 };               // scheduling modes

struct BwdGemm {
  const bf16* A;      // row side ("features")
  const bf16* B;      // column side ("tokens" for dgrad, a feature dim for wgrad)
  bf16* Y;            // output, Y[col * ldy + row]
  const bf16* S;      // saved pre-activation for EPI_DACT, indexed like Y
  const int32_t* offset;
  int64_t a_estride;  // per-expert stride of A (weights); 0 for activations
  int32_t lda, ldb, ldy;
  int32_t nrows;      // row-side extent (features)
  int32_t ncols;      // column-side extent for M_WGRAD
  int32_t kdim;       // K for M_ROWS
  int32_t E, act;
  int64_t max_rows;
};

__device__ __forceinline__ int lds_row_of_feature(int f) {
  return ((f >> 2) & 3) * 8 + (f >> 4) * 4 + (f & 3);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }

// erf by Abramowitz & Stegun 7.1.26 (|error| <= 1.5e-7), odd extension.
__device__ __forceinline__ float erf_as(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, az, 1.f));
  float p = fmaf(1.061405429f, t, -1.453152027f);
  p = fmaf(p, t, 1.421413741f);
  p = fmaf(p, t, -0.284496736f);
  p = fmaf(p, t, 0.254829592f);
  p *= t;
  const float e = __builtin_amdgcn_exp2f(-az * az * 1.4426950408889634f);
  return __builtin_copysignf(fmaf(-p, e, 1.f), z);
}

// d/da act(a)
__device__ __forceinline__ float act_grad(float a, int act) {
  if (act == ACT_RELU) return a > 0.f ? 1.f : 0.f;
  if (act == ACT_GELU) {
    const float cdf = 0.5f * (1.f + erf_as(a * 0.7071067811865476f));
    const float pdf = 0.3989422804014327f * __builtin_amdgcn_exp2f(-0.5f * a * a * 1.4426950408889634f);
    return fmaf(a, pdf, cdf);
  }
  return 1.f;
}

// Transpose an 8x8 block of bf16: in[r] holds elements (r, 0..7); out[j]
// holds elements (0..7, j).
__device__ __forceinline__ void transpose8(const uint4 (&in)[8], uint4 (&out)[8]) {
  uint32_t w[8][4];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    w[r][0] = in[r].x;
    w[r][1] = in[r].y;
    w[r][2] = in[r].z;
    w[r][3] = in[r].w;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = __builtin_amdgcn_perm(w[2 * q + 1][j >> 1], w[2 * q][j >> 1], sel);
    out[j] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

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

// Loads of one operand tile (kT rows x 64 k) into registers and from there
// into LDS (row r at byte r*kRowB + k*2; for the row side, rows are stored at
// the permuted position that gives each lane 16 consecutive output rows).
template <int LAYOUT, bool ROWSIDE>
struct Loader {
  // K-contiguous: 1024 16-byte chunks, 4 per thread.
  // Row-contiguous: 128 blocks of 8x8, one per thread for threads < 128.
  static constexpr int NREG = LAYOUT == L_KC ? 4 : 8;
  uint4 reg[NREG];
  const bf16* base;  // element (row 0, k 0) of this tile
  int ld, rows_valid;

  __device__ __forceinline__ void load(int k0, int kvalid) {
    const int tid = threadIdx.x;
    if constexpr (LAYOUT == L_KC) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + i * 256;
        const int row = c >> 3, col = c & 7;
        const int kk = k0 + col * 8;
        reg[i] = (row < rows_valid && kk < kvalid) ? *reinterpret_cast<const uint4*>(base + (int64_t)row * ld + kk)
                                                   : make_uint4(0, 0, 0, 0);
      }
    } else {
      const int blk = tid & 127;
      const int kb = blk >> 4, rb = blk & 15;  // k block (0..7), row block (0..15)
      const bool rv = tid < 128 && rb * 8 + 8 <= rows_valid;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int kk = k0 + kb * 8 + r;
        reg[r] = (rv && kk < kvalid) ? *reinterpret_cast<const uint4*>(base + (int64_t)kk * ld + rb * 8)
                                     : make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ int lds_row(int row) const {
    return ROWSIDE ? ((row & ~31) + lds_row_of_feature(row & 31)) : row;
  }
  __device__ __forceinline__ void store(unsigned char* tile) const {
    const int tid = threadIdx.x;
    if constexpr (LAYOUT == L_KC) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + i * 256;
        const int row = c >> 3, col = c & 7;
        *reinterpret_cast<uint4*>(tile + lds_row(row) * kRowB + col * 16) = reg[i];
      }
    } else {
      if (tid < 128) {
        const int kb = tid >> 4, rb = tid & 15;
        uint4 t[8];
        transpose8(reg, t);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint4*>(tile + lds_row(rb * 8 + j) * kRowB + kb * 16) = t[j];
      }
    }
  }
};

template <int LA, int LB, int MODE, int EPI>
__global__ __launch_bounds__(256) void bwd_gemm_kernel(BwdGemm g) {
  constexpr int STAGE = 2 * kT * kRowB;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_pref[MOE_MAX_EXPERTS_DEV + 1];

  const int E = g.E;
  const int ntr = (g.nrows + kT - 1) / kT;  // row-side tiles
  int e, ct, rt, row0 = 0, mrows = 0;
  if constexpr (MODE == M_ROWS) {
    tile_prefix<kT>(g.offset, E, s_pref);
    __syncthreads();
    const int total = s_pref[E] * ntr;
    const int share = (total + kXcds - 1) / kXcds;
    const int loc = blockIdx.x / kXcds;
    const int tile = (blockIdx.x % kXcds) * share + loc;
    if (loc >= share || tile >= total) return;
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] * ntr <= tile) lo = mid; else hi = mid;
    }
    e = lo;
    const int mte = s_pref[e + 1] - s_pref[e];
    const int local = tile - s_pref[e] * ntr;
    rt = local / mte;
    ct = local - rt * mte;  // consecutive workgroups share a weight tile
    row0 = g.offset[e];
    mrows = g.offset[e + 1] - row0;
  } else {
    const int ntc = (g.ncols + kT - 1) / kT;
    const int per_e = ntc * ntr;
    e = blockIdx.x / per_e;
    const int local = blockIdx.x - e * per_e;
    ct = local / ntr;
    rt = local - ct * ntr;
    row0 = g.offset[e];
    mrows = g.offset[e + 1] - row0;
  }

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wt = wave >> 1, wf = wave & 1;
  const int r0 = rt * kT, c0 = ct * kT;
  const int rows_valid = min(kT, g.nrows - r0);
  int cols_valid, kdim;
  Loader<LA, true> la;
  Loader<LB, false> lb;
  if constexpr (MODE == M_ROWS) {
    // A: weights of expert e, row-side elements r0.. ; B: the expert's tokens
    cols_valid = min(kT, mrows - c0);
    kdim = g.kdim;
    la.base = g.A + (int64_t)e * g.a_estride + (LA == L_KC ? (int64_t)r0 * g.lda : (int64_t)r0);
    lb.base = g.B + (int64_t)(row0 + c0) * g.ldb;
  } else {
    // both operands are activations of the expert's rows, K = rows
    cols_valid = min(kT, g.ncols - c0);
    kdim = mrows;
    la.base = g.A + (int64_t)row0 * g.lda + r0;
    lb.base = g.B + (int64_t)row0 * g.ldb + c0;
  }
  la.ld = g.lda;
  la.rows_valid = rows_valid;
  lb.ld = g.ldb;
  lb.rows_valid = cols_valid;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (kdim + kBK - 1) / kBK;
  if (nk > 0) {
    la.load(0, kdim);
    lb.load(0, kdim);
    la.store(smem + kT * kRowB);  // row side after the column side in each stage
    lb.store(smem);
    __syncthreads();
  }
  const int hsel = lane >> 5, r32 = lane & 31;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load((kt + 1) * kBK, kdim);
      lb.load((kt + 1) * kBK, kdim);
    }
    const unsigned char* Bs = smem + cur * STAGE;
    const unsigned char* As = Bs + kT * kRowB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kb = (hsel * 32 + i * 8) * 2;
      bf16x8 af[2], bx[2];
#pragma unroll
      for (int ff = 0; ff < 2; ++ff)
        af[ff] = *reinterpret_cast<const bf16x8*>(As + (wf * 64 + ff * 32 + r32) * kRowB + kb);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        bx[tt] = *reinterpret_cast<const bf16x8*>(Bs + (wt * 64 + tt * 32 + r32) * kRowB + kb);
#pragma unroll
      for (int ff = 0; ff < 2; ++ff)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          acc[ff][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ff], bx[tt], acc[ff][tt], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      la.store(smem + (cur ^ 1) * STAGE + kT * kRowB);
      lb.store(smem + (cur ^ 1) * STAGE);
    }
    __syncthreads();
  }

  // epilogue: lane holds 16 consecutive row-side elements of one column
#pragma unroll
  for (int ff = 0; ff < 2; ++ff) {
    const int rl = wf * 64 + ff * 32 + hsel * 16;
    if (rl >= rows_valid) continue;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int cl = wt * 64 + tt * 32 + r32;
      if (cl >= cols_valid) continue;
      int64_t yoff;
      if constexpr (MODE == M_ROWS) yoff = (int64_t)(row0 + c0 + cl) * g.ldy + r0 + rl;
      else yoff = ((int64_t)e * g.ncols + c0 + cl) * g.ldy + r0 + rl;
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = acc[ff][tt][r];
      if constexpr (EPI == EPI_DACT) {
        const uint4* sp = reinterpret_cast<const uint4*>(g.S + yoff);
        const uint4 s0 = sp[0], s1 = sp[1];
        const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[2 * i] *= act_grad(__uint_as_float(sw[i] << 16), g.act);
          v[2 * i + 1] *= act_grad(__uint_as_float(sw[i] & 0xffff0000u), g.act);
        }
      }
      uint4* p = reinterpret_cast<uint4*>(g.Y + yoff);
      p[0] = make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
      p[1] = make_uint4(pack2(v[8], v[9]), pack2(v[10], v[11]), pack2(v[12], v[13]), pack2(v[14], v[15]));
    }
  }
}

// Column sums over each expert's packed rows, out[e][c] = sum of M[r][c] for
// the rows r of e (fp32, in a fixed order).  Workgroup: 256 columns of one
// expert; thread = (group of 8 columns, row lane 0..7): the 32 column groups
// of a row lane read one row's 512 contiguous bytes, four rows in flight per
// thread; the eight row lanes are added in order through LDS.
__global__ __launch_bounds__(256) void colsum_kernel(const bf16* __restrict__ M, const int32_t* __restrict__ offset,
                                                     float* __restrict__ out, int ncols) {
  __shared__ float red[8][257];
  const int e = blockIdx.y;
  const int cg = threadIdx.x & 31, rl = threadIdx.x >> 5;
  const int c0 = blockIdx.x * 256 + cg * 8;
  const int r0 = offset[e], r1 = offset[e + 1];
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const uint4 v) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s[2 * q] += __uint_as_float(u[q] << 16);
      s[2 * q + 1] += __uint_as_float(u[q] & 0xffff0000u);
    }
  };
  if (c0 < ncols) {
    const bf16* base = M + c0;
    int r = r0 + rl;
    for (; r + 24 < r1; r += 32) {
      const uint4 a = *reinterpret_cast<const uint4*>(base + (int64_t)r * ncols);
      const uint4 b = *reinterpret_cast<const uint4*>(base + (int64_t)(r + 8) * ncols);
      const uint4 c = *reinterpret_cast<const uint4*>(base + (int64_t)(r + 16) * ncols);
      const uint4 d = *reinterpret_cast<const uint4*>(base + (int64_t)(r + 24) * ncols);
      add(a);
      add(b);
      add(c);
      add(d);
    }
    for (; r < r1; r += 8) add(*reinterpret_cast<const uint4*>(base + (int64_t)r * ncols));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rl][cg * 8 + i] = s[i];
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < ncols) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t += red[i][threadIdx.x];
    out[(int64_t)e * ncols + c] = t;
  }
}

template <int LA, int LB, int MODE, int EPI>
hipError_t launch(const BwdGemm& g, hipStream_t s) {
  constexpr size_t lds = 2 * (size_t)2 * kT * kRowB;
  auto kern = bwd_gemm_kernel<LA, LB, MODE, EPI>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  int64_t grid;
  const int64_t ntr = (g.nrows + kT - 1) / kT;
  if (MODE == M_ROWS) {
    grid = ((g.max_rows + kT - 1) / kT + g.E) * ntr;
    grid = (grid + kXcds - 1) / kXcds * kXcds;
  } else {
    grid = (int64_t)g.E * ((g.ncols + kT - 1) / kT) * ntr;
  }
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_backward(const GemmBwdArgs& a, int dtype, hipStream_t s) {
  if (dtype != DT_BF16) return hipErrorNotSupported;
  const bf16* X = static_cast<const bf16*>(a.X);
  const bf16* W1 = static_cast<const bf16*>(a.W1);
  const bf16* W2 = static_cast<const bf16*>(a.W2);
  const bf16* A = static_cast<const bf16*>(a.A);
  const bf16* H = static_cast<const bf16*>(a.H);
  const bf16* dY = static_cast<const bf16*>(a.dY);
  bf16* dA = static_cast<bf16*>(a.dA);
  const int d = a.d, h = a.h;
  hipError_t err;
  if (a.max_rows <= 0) {
    // no rows at all: every gradient is zero
    if ((err = launch_zero_bytes(a.dW1, (size_t)a.E * h * d * 2, s)) != hipSuccess) return err;
    if ((err = launch_zero_bytes(a.dW2, (size_t)a.E * d * h * 2, s)) != hipSuccess) return err;
    if (a.db1 && (err = launch_zero_bytes(a.db1, (size_t)a.E * h * 4, s)) != hipSuccess) return err;
    if (a.db2 && (err = launch_zero_bytes(a.db2, (size_t)a.E * d * 4, s)) != hipSuccess) return err;
    return hipSuccess;
  }
  // Order: db2 and dW2 are the last reads of dY, before dX is written, so
  // that dX may take dY's memory.
  if (a.db2) {
    hipLaunchKernelGGL(colsum_kernel, dim3((d + 255) / 256, a.E), dim3(256), 0, s, dY, a.offset, a.db2, d);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  BwdGemm g{};
  g.offset = a.offset;
  g.E = a.E;
  g.act = a.act;
  g.max_rows = a.max_rows;

  // the large-tile kernel when the shapes fit it, else the 128 x 128 kernels below
  err = launch_backward_big(a, s);
  if (err != hipSuccess && err != hipErrorNotSupported) return err;
  if (err == hipErrorNotSupported) {
  // dA = (dY · W2[e]) ⊙ act'(A): rows = h (W2[e] row-contiguous along h), K = d
  g.A = W2; g.a_estride = (int64_t)d * h; g.lda = h;
  g.B = dY; g.ldb = d;
  g.Y = dA; g.S = A; g.ldy = h;
  g.nrows = h; g.kdim = d;
  if ((err = launch<L_RC, L_KC, M_ROWS, EPI_DACT>(g, s)) != hipSuccess) return err;

  // dW2[e][d][h] = dY^T · H: rows = h (from H), columns = d (from dY), K = rows of e
  g.A = H; g.a_estride = 0; g.lda = h;
  g.B = dY; g.ldb = d;
  g.Y = static_cast<bf16*>(a.dW2); g.S = nullptr; g.ldy = h;
  g.nrows = h; g.ncols = d;
  if ((err = launch<L_RC, L_RC, M_WGRAD, EPI_STORE>(g, s)) != hipSuccess) return err;

  // dX = dA · W1[e]: rows = d (W1[e] row-contiguous along d), K = h
  g.A = W1; g.a_estride = (int64_t)h * d; g.lda = d;
  g.B = dA; g.ldb = h;
  g.Y = static_cast<bf16*>(a.dX); g.ldy = d;
  g.nrows = d; g.kdim = h;
  if ((err = launch<L_RC, L_KC, M_ROWS, EPI_STORE>(g, s)) != hipSuccess) return err;

  // dW1[e][h][d] = dA^T · X: rows = d (from X), columns = h (from dA)
  g.A = X; g.a_estride = 0; g.lda = d;
  g.B = dA; g.ldb = h;
  g.Y = static_cast<bf16*>(a.dW1); g.ldy = d;
  g.nrows = d; g.ncols = h;
  if ((err = launch<L_RC, L_RC, M_WGRAD, EPI_STORE>(g, s)) != hipSuccess) return err;
  }

  if (a.db1) {
    hipLaunchKernelGGL(colsum_kernel, dim3((h + 255) / 256, a.E), dim3(256), 0, s, (const bf16*)dA, a.offset, a.db1, h);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
