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

enum { MODE_LOGITS_IN = 0, MODE_BF16 = 1, MODE_F32 = 2 };


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

// Router GEMM K chunk staged in LDS per step: 256 for up to 64 experts, 128
// for 128, 64 for 256, so that the double-buffered weight chunk stays at
// 64 KB at most; a long chunk keeps more bytes in flight per barrier.
template <int EP>
constexpr int gate_kc() { return EP <= 64 ? 256 : EP <= 128 ? 128 : 64; }

template <int EP, int TG, int MODE>
__global__ __launch_bounds__(256) void gate_kernel(GateArgs a) {
  constexpr int NET = EP / 16;   // 16-expert MFMA row tiles
  constexpr int TT = TG * 16;    // tokens per tile
  constexpr int KC = gate_kc<EP>();
  constexpr int CPR = KC / 8;    // 16-byte chunks per weight row of a K chunk
  constexpr size_t W_BYTES = (MODE == MODE_BF16) ? size_t(2) * EP * KC * 2 : 0;
  static_assert(MODE != MODE_BF16 || TG == 4, "the router GEMM gives each wave its own 16 tokens");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* s_sel = reinterpret_cast<int*>(smem + W_BYTES);                // [2][TT]
  int* s_rnk = s_sel + 2 * TT;                                        // [2][TT]
  float* s_me = reinterpret_cast<float*>(s_rnk + 2 * TT);             // [TG][EP]
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, n = lane & 15, q = lane >> 4;
  const int E = a.E, K = a.k, KE = a.k * a.E;
  const int64_t T = a.T;

  const int tile = blockIdx.x;
  const int64_t t0 = (int64_t)tile * TT;

  // ------------------------------------------------------------ logits
  // lg[et][r] = logit of expert et*16 + q*4 + r for token t0 + wave*16 + n
  float lg[NET][4];
  if constexpr (MODE == MODE_BF16) {
    // Each wave computes its own 16 tokens over the whole hidden dimension,
    // so no cross-wave reduction is needed.  The router weight streams
    // through LDS in K chunks of KC (double-buffered, loaded once per
    // workgroup and read by all four waves); chunk c of weight row r sits in
    // slot c ^ (r & 15), so the 16 rows one fragment read touches fall in 16
    // different banks.  The x fragments come straight from global memory,
    // one K step ahead.
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
    const int64_t tx = t0 + wave * 16 + n;
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
      if (a.jitter) {
        // the router reads x * ((1 - eps) + 2 eps u), eps = 0.01, each
        // product and sum rounded once in fp32, then stored as bf16
#pragma unroll
        for (int i = 0; i < KC / 32; ++i) {
          const int kk = ks * KC + q * (KC / 4) + i * 8;
          if (tx < T && kk < d) {
            const uint64_t n0 = (uint64_t)tx * d + kk;   // a multiple of 8
            const uint4 w0 = philox_block(a.seed_lo, a.seed_hi, kStreamJitter, n0 >> 2);
            const uint4 w1 = philox_block(a.seed_lo, a.seed_hi, kStreamJitter, (n0 >> 2) + 1);
            const uint32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float f = __fadd_rn(0.99f, __fmul_rn(0.02f, philox_uniform(wv[j])));
              xb[i][j] = static_cast<bf16>(__fmul_rn(static_cast<float>(xb[i][j]), f));
            }
          }
        }
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

    // top-1, by (value desc, index asc).  The selection key of a NaN logit
    // is -inf and the running index starts past every expert, so that even a
    // token whose logits are all -inf or NaN (outside the contract) gets a
    // valid expert (the lowest index) and no later step indexes out of range.
    // With RSample (k = 1) the top-1 key is fp32(logit + g), g a Gumbel draw
    // of stream 1 at t*E + e; with second-expert sampling (k = 2) the top-2
    // key is the same with stream 2.  The weights use the clean logits.
    const bool noisy0 = a.rsample != 0, noisy1 = a.second != 0 && K == 2;
    auto gumbel = [&](uint32_t stream, int e) {
      const uint32_t w = philox_draw(a.seed_lo, a.seed_hi, stream, (uint64_t)t * E + e);
      return -logf(-logf(philox_uniform(w)));
    };
    float v0 = -INFINITY;
    int i0 = E;
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = et * 16 + q * 4 + r;
        float key = lg[et][r] != lg[et][r] ? -INFINITY : lg[et][r];
        if (noisy0 && e < E) key = __fadd_rn(key, gumbel(kStreamRSample, e));
        if (e < E && (key > v0 || (key == v0 && e < i0))) {
          v0 = key;
          i0 = e;
        }
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
          if (e < E && e != i0 && (key > v1 || (key == v1 && e < i1))) {
            v1 = key;
            i1 = e;
          }
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
    a.tile_cnt[(int64_t)c * a.num_tiles + tile] = cnt;
  }
  for (int e = tid; e < E; e += 256) {
    float v = 0.f;
    for (int g = 0; g < TG; ++g) v += s_me[g * EP + e];
    a.me_tile[(int64_t)tile * E + e] = v;
  }
  __syncthreads();
  // raw slot = rank inside the tile; the fix-up kernel adds the tile prefix
  for (int i = tid; i < K * TT; i += 256) {
    const int j = i / TT, nn = i - j * TT;
    if (s_sel[i] >= 0) a.slot[(t0 + nn) * K + j] = s_rnk[i];
  }
}

// Exclusive prefix over tiles of one (choice, expert) column, its total
// demand and (choice-0 columns) the expert's probability mass.
__global__ __launch_bounds__(256) void gate_scan_kernel(GateArgs a) {
  __shared__ int s_part[256];
  __shared__ double s_dred[256];
  const int tid = threadIdx.x, c = blockIdx.x;
  const int E = a.E;
  const int nt = a.num_tiles;
  int32_t* col = a.tile_cnt + (int64_t)c * nt;
  // each thread owns a contiguous run of tiles
  const int per = (nt + 255) / 256;
  const int lo = min(nt, tid * per), hi = min(nt, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += col[i];
  s_part[tid] = sum;
  __syncthreads();
  // inclusive scan of the 256 partial sums (Hillis-Steele in LDS)
  for (int off = 1; off < 256; off <<= 1) {
    const int v = tid >= off ? s_part[tid - off] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int run = s_part[tid] - sum;
  for (int i = lo; i < hi; ++i) {
    const int v = col[i];
    col[i] = run;
    run += v;
  }
  if (tid == 255) a.demand[c] = s_part[255];
  if (c < E) {
    // probability mass of expert c: runs in tile order, then a fixed tree
    double m = 0.0;
    for (int i = lo; i < hi; ++i) m += (double)a.me_tile[(int64_t)i * E + c];
    s_dred[tid] = m;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if (tid < off) s_dred[tid] += s_dred[tid + off];
      __syncthreads();
    }
    if (tid == 0) a.me_sum[c] = s_dred[0];
  }
}

// Expert counts (capacity applied per choice in order), offsets and the loss
// from the scan's demands and probability mass, by one workgroup.
__device__ void gate_counts_and_loss(const GateArgs& a) {
  __shared__ int s_cnt[2 * MOE_MAX_EXPERTS_DEV];
  __shared__ int s_base[MOE_MAX_EXPERTS_DEV];
  __shared__ double s_dme[MOE_MAX_EXPERTS_DEV];
  const int tid = threadIdx.x;
  const int E = a.E, K = a.k, KE = a.k * a.E;
  const int64_t T = a.T;
  for (int cc = tid; cc < KE; cc += blockDim.x) s_cnt[cc] = a.demand[cc];
  __syncthreads();
  const int64_t C = a.C;
  for (int e = tid; e < E; e += blockDim.x) {
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
    s_dme[e] = a.me_sum[e];
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

// Final slots: the rank inside the tile plus the column's prefix over earlier
// tiles; choice 1 also adds the expert's total choice-0 demand; a slot at or
// past the capacity is dropped.  The grid's last workgroup instead forms the
// expert counts, offsets and the loss.
__global__ __launch_bounds__(256) void slot_finalize_kernel(GateArgs a, int tile_tokens) {
  if (blockIdx.x == gridDim.x - 1) {
    gate_counts_and_loss(a);
    return;
  }
  const int64_t n = a.T * a.k;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int k = a.k, E = a.E;
  const int j = (int)(i % k);
  const int64_t t = i / k;
  const int e = a.expert_idx[i];
  const int c = j * E + e;
  int64_t s = (int64_t)a.slot[i] + a.tile_cnt[(int64_t)c * a.num_tiles + t / tile_tokens];
  if (j == 1) s += a.demand[e];
  a.slot[i] = (a.C >= 0 && s >= a.C) ? -1 : (int32_t)s;
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
  const size_t wbytes = (MODE == MODE_BF16) ? size_t(2) * EP * gate_kc<EP>() * 2 : 0;
  return wbytes + 4 * (2 * TT + 2 * TT + TG * EP);
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
  return launch_gate_t<256, 4, MODE>(a, s);
}

}  // namespace

hipError_t launch_gate(const GateArgs& a, int dtype, hipStream_t s) {
  hipError_t e;
  if (a.logits_in) e = launch_gate_mode<MODE_LOGITS_IN>(a, s);
  else if (dtype == DT_BF16) e = launch_gate_mode<MODE_BF16>(a, s);
  else e = launch_gate_mode<MODE_F32>(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gate_scan_kernel, dim3((unsigned)(a.k * a.E)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_slot_finalize(const GateArgs& a, int tile_tokens, hipStream_t s) {
  const int64_t n = a.T * a.k;
  hipLaunchKernelGGL(slot_finalize_kernel, dim3((unsigned)((n + 255) / 256 + 1)), dim3(256), 0, s, a, tile_tokens);
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
