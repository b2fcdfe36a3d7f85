// Small-batch (decode / evaluation) forward of the whole layer in one
// persistent kernel: router GEMM, softmax, top-k, capacity slots, counts,
// offsets, gate_loss, dispatch, both expert Linears and the combine.
//
// What is computed is the forward of "MoE混合专家架构：大模型高效推理的智能调度原理"
// §3.1 (MoELayer Steps 1-5) and "deepspeed.moe 模块" overview §3.1, exactly as
// the multi-kernel path computes it (same routing rules, same capacity rule,
// same loss).  The pages' inference notes ask for the gating and the token
// assignment fused into one launch to cut kernel-launch overhead; with a few
// tokens the layer is one pass over the chosen experts' weights, and seven
// launches of a few microseconds each would cost more than that pass.
//
// Design (gfx950): a plain launch of one workgroup per CU (so the whole grid
// is resident), phases separated by grid barriers of our own: two levels of
// arrival counters on separate cache lines, polled with a sleep (the
// runtime's cooperative grid sync took 30-60 us per barrier here, and its
// launch about 20 us more than a plain one):
//  1. Router products: items of 16 experts x 16 tokens x one of ks slices of
//     K (ks grows while there are at most 16 items, so a few tokens still spread
//     the router weight over many CUs), the four wavefronts splitting the
//     slice (v_mfma_f32_16x16x32_bf16), fp32 partials.
//  2. Routing: a wavefront per token adds the slices in order (+ bias), then
//     softmax max and sum, top-1 / top-2 by (value desc, index asc) with
//     xor-shuffles; then, after a barrier, every workgroup forms the capacity
//     slots in claim order (all top-1 claims in token order, then all top-2)
//     from 64-token chunks, where a lane's rank among equal experts comes
//     from nine ballots over the bits of the expert id + 1, the offsets by a
//     wavefront scan, and the packed row -> token map.  The last two
//     workgroups write slots, counts, offsets and the loss.
//  3. Expert Linear 1 (+ bias, activation): items of 16 output features of
//     one expert; the four wavefronts split K, each streaming its weight
//     quarter through a ring of loads that runs on across items, and add
//     their partial products through LDS in a fixed order; the token rows
//     are gathered straight from x (dispatch fused in).
//  4. Expert Linear 2 (+ bias) on the packed hidden rows, the same way.
//  5. Combine: out[t] = sum over kept choices, in order, of w * y_disp row.
// The weights of the chosen experts are read once; every work loop has a
// fixed trip count that every workgroup reaches, so every barrier completes.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kFB = 16;   // output features per work item (MFMA rows)
constexpr int kRing = 16; // K-steps in flight per wavefront in the expert Linears

__device__ __forceinline__ bf16x8 ldv(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ void best_merge(float& v, int& i, int mask) {
  const float ov = __shfl_xor(v, mask);
  const int oi = __shfl_xor(i, mask);
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

template <int G>
__device__ __forceinline__ float gmax(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
template <int G>
__device__ __forceinline__ float gsum(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

struct DecShared {
  int slot[2][kDecodeMaxTokens];
  int idx[2][kDecodeMaxTokens];
  float w[2][kDecodeMaxTokens];
  int run[2][MOE_MAX_EXPERTS_DEV];       // claims per (choice, expert)
  int cnt[MOE_MAX_EXPERTS_DEV];
  int off[MOE_MAX_EXPERTS_DEV + 1];
  int ipre[MOE_MAX_EXPERTS_DEV + 1];     // work-item prefix over experts with rows
  int rowtok[2 * kDecodeMaxTokens];
  float red[4][64][4];                   // split-K partial products
  double dred[256];
};

// The calling wave's quarter of K of one 16-output x (up to) 16-row block:
// A = weight rows (K-contiguous), B = token rows.  Fragments are loaded in
// batches of 16 K steps ahead of their products, so that a wavefront keeps
// 16 KB of the weight stream in flight.
__device__ __forceinline__ f32x4 lin_quarter(const bf16* wrow, const bf16* brow, bool bvalid, int k0, int k1) {
  constexpr int NB = 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const bf16x8 zero = {};
  int kk = k0;
  for (; kk + 32 * NB <= k1; kk += 32 * NB) {
    bf16x8 av[NB], bv[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      av[i] = ldv(wrow + kk + 32 * i);
      bv[i] = bvalid ? ldv(brow + kk + 32 * i) : zero;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[i], acc, 0, 0, 0);
  }
  for (; kk < k1; kk += 32) {
    const bf16x8 av = ldv(wrow + kk);
    const bf16x8 bv = bvalid ? ldv(brow + kk) : zero;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ float act_rt(float v, int act) {
  if (act == ACT_GELU) return act_fixed<ACT_GELU>(v);
  if (act == ACT_RELU) return act_fixed<ACT_RELU>(v);
  return v;
}

// Grid barrier in two levels, each counter on its own 128-byte line: a
// workgroup arrives at the counter of its group (workgroup index mod 16);
// the last arrival of a group in this phase arrives at the top counter,
// which every workgroup polls with a sleep between reads.  Counters grow by
// one per phase (zeroed by the init kernel that precedes the launch), so
// phase p is complete when the top counter reaches p times the number of
// groups.  The grid is one workgroup per CU and the kernel's resources allow
// several per CU, so on a device not held by a kernel that never ends every
// workgroup is resident and every wait ends.  The spin is bounded all the
// same: a wait that gives up records it in the status word and returns
// false, and the workgroup then stops (its reads would see data that was
// never written) after setting gate_loss to NaN and the status word (which
// the host can read through moe_workspace_status) to 1.
//
// Publishing: every wavefront first waits until its own stores have been
// acknowledged by the L2 (s_waitcnt vmcnt(0)), then the workgroup barrier,
// then thread 0's agent-scope release writes this XCD's L2 back before it
// arrives.  A workgroup barrier orders the waves' execution but does not
// wait for their outstanding global stores (on gfx950 __syncthreads compiles
// to a bare s_barrier), and a release fence waits only for the issuing
// wave's own memory operations before the write-back (buffer_wbl2).  Without
// the per-wave wait, a store of another wave still on its way to the L2 when
// the write-back runs stays in this XCD's L2, and a workgroup on another XCD
// (own L2) can read the old value.  Stores by several waves that other
// workgroups read after a barrier happen here in the routing phase (a wave
// per token) and in the row copy.  (A full release in every wave does the
// same but repeats the L2 write-back four times per workgroup: about 7 us
// more per barrier, measured.)
constexpr int kBarGroups = 16, kBarLine = 32;   // 32 words = 128 bytes
constexpr int kBarTop = kBarGroups * kBarLine, kBarStatus = kBarTop + kBarLine;
constexpr int kBarWords = kBarStatus + 1;
static_assert(kBarStatus == kDecodeStatusWord, "status word index");

__device__ __forceinline__ bool grid_barrier(unsigned* bar, unsigned phase, int* ok) {
  // each wave: its stores have reached the L2 (vmcnt(0); expcnt, lgkmcnt not waited on)
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned nwg = gridDim.x;
    const unsigned g = blockIdx.x % kBarGroups;
    const unsigned groups = nwg < (unsigned)kBarGroups ? nwg : (unsigned)kBarGroups;
    const unsigned gsize = (nwg - g + kBarGroups - 1) / kBarGroups;   // workgroups in group g
    // one release (with every wave's stores in the L2, its write-back
    // publishes all of the workgroup's), relaxed arrivals and polls (an acquire per poll would invalidate the
    // XCD's L2 on every read), then one acquire
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned old = __hip_atomic_fetch_add(&bar[g * kBarLine], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == phase * gsize)
      __hip_atomic_fetch_add(&bar[kBarTop], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned spins = 0;
    int done = 1;
    while (__hip_atomic_load(&bar[kBarTop], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < phase * groups) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > (1u << 22)) {
        __hip_atomic_store(&bar[kBarStatus], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        done = 0;
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *ok = done;
  }
  __syncthreads();
  return *ok != 0;
}

// Sum over the workgroup's 256 threads in a fixed tree order (every thread
// gets the total).
__device__ double block_sum(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
#pragma unroll
  for (int m = 128; m >= 1; m >>= 1) {
    if (tid < m) red[tid] += red[tid + m];
    __syncthreads();
  }
  const double total = red[0];
  __syncthreads();
  return total;
}

// One token's softmax, top-1 / top-2 (value desc, index asc; a NaN ranks as
// -inf and the running index starts past every expert) and gate weights, by
// one wavefront with lane l holding experts l, l+64, ...  The probabilities
// go to prob[t] when asked (the BALANCE loss sums them per expert).
template <int EPL>
__device__ void route_token(const DecodeArgs& a, int t, float* prob) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, k = a.k, T = a.T;
  float l[EPL];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      if (a.logits_in) {
        l[i] = a.logits_in[(int64_t)t * E + e];
      } else {
        // the K slices' partial products (all loads issued before the
        // first add), added in slice order, then the bias
        float pv[kDecodeMaxSlices];
#pragma unroll
        for (int sl = 0; sl < kDecodeMaxSlices; ++sl)
          pv[sl] = sl < a.ks ? a.part[((int64_t)sl * T + t) * E + e] : 0.f;
        float v = pv[0];
#pragma unroll
        for (int sl = 1; sl < kDecodeMaxSlices; ++sl)
          if (sl < a.ks) v += pv[sl];
        l[i] = v + (a.b_router ? a.b_router[e] : 0.f);
      }
      if (a.logits) a.logits[(int64_t)t * E + e] = l[i];
    } else {
      l[i] = -INFINITY;
    }
    mx = fmaxf(mx, l[i]);
  }
  mx = gmax<64>(mx);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + 64 * i < E) sum += expf(l[i] - mx);
  sum = gsum<64>(sum);
  float v0 = -INFINITY, v1 = -INFINITY;
  int i0 = E, i1 = E;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    const float key = l[i] != l[i] ? -INFINITY : l[i];
    if (e < E && (key > v0 || (key == v0 && e < i0))) {
      v0 = key;
      i0 = e;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) best_merge(v0, i0, m);
  if (k == 2) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      const float key = l[i] != l[i] ? -INFINITY : l[i];
      if (e < E && e != i0 && (key > v1 || (key == v1 && e < i1))) {
        v1 = key;
        i1 = e;
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) best_merge(v1, i1, m);
  }
  float p0 = expf(v0 - mx) / sum;
  float p1 = (k == 2) ? expf(v1 - mx) / sum : 0.f;
  if (a.normalize) {
    const float s = p0 + p1;
    p0 = p0 / s;
    p1 = p1 / s;
  }
  if (prob) {
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + 64 * i < E) prob[(int64_t)t * E + lane + 64 * i] = expf(l[i] - mx) / sum;
  }
  if (lane == 0) {
    a.expert_idx[t * k] = i0;
    a.weight[t * k] = p0;
    if (k == 2) {
      a.expert_idx[t * k + 1] = i1;
      a.weight[t * k + 1] = p1;
    }
  }
}

// Capacity slots, counts, offsets, the work-item prefix and the row -> token
// map from the routed experts (every workgroup, from global memory).
__device__ void assign_slots(const DecodeArgs& a, DecShared& S) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, E = a.E, k = a.k;
  for (int i = tid; i < k * T; i += 256) {
    const int t = i / k, j = i - t * k;
    S.idx[j][t] = a.expert_idx[i];
    S.w[j][t] = a.weight[i];
  }
  for (int e = tid; e < E; e += 256) S.run[0][e] = S.run[1][e] = 0;
  __syncthreads();
  // claim order: every top-1 claim in token order, then every top-2 claim;
  // a lane's rank among the lanes of its 64-token chunk with the same expert
  // comes from nine ballots over the bits of (expert + 1)
  if (wave == 0) {
    for (int j = 0; j < k; ++j) {
      for (int c0 = 0; c0 < T; c0 += 64) {
        const int t = c0 + lane;
        const int e = t < T ? S.idx[j][t] : -1;
        const unsigned key = (unsigned)(e + 1);
        uint64_t same = ~0ull;
#pragma unroll
        for (int b = 0; b < 9; ++b) {
          const uint64_t bal = __ballot((key >> b) & 1u);
          same &= ((key >> b) & 1u) ? bal : ~bal;
        }
        const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
        const int rank = __popcll(same & lt);
        const int base = e >= 0 ? S.run[j][e] : 0;
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): every base is read before any update
        __builtin_amdgcn_wave_barrier();
        if (e >= 0) {
          int sl = base + rank;
          if (j == 1) sl += S.run[0][e];
          S.slot[j][t] = (a.C >= 0 && sl >= a.C) ? -1 : sl;
          if (rank == 0) S.run[j][e] = base + __popcll(same);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    const int64_t d0 = S.run[0][e];
    const int64_t d1 = k == 2 ? S.run[1][e] : 0;
    int64_t kept;
    if (a.C < 0) {
      kept = d0 + d1;
    } else {
      kept = d0 < a.C ? d0 : a.C;
      if (k == 2) {
        const int64_t room = a.C - d0;
        kept += room <= 0 ? 0 : (d1 < room ? d1 : room);
      }
    }
    S.cnt[e] = (int)kept;
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive prefixes over experts: lane l holds experts 4l .. 4l+3
    const int nfb1 = ((a.h > 0 ? a.h : a.d) + kFB - 1) / kFB;
    int c[4], n = 0, it = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      c[i] = e < E ? S.cnt[e] : 0;
      n += c[i];
      it += c[i] > 0 ? nfb1 : 0;
    }
    int sn = n, sit = it;   // inclusive scans over lanes
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int un = __shfl_up(sn, m), uit = __shfl_up(sit, m);
      if (lane >= m) {
        sn += un;
        sit += uit;
      }
    }
    int acc = sn - n, iacc = sit - it;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) {
        S.off[e] = acc;
        S.ipre[e] = iacc;
      }
      acc += c[i];
      iacc += c[i] > 0 ? nfb1 : 0;
    }
    if (lane == 63) {
      S.off[E] = sn;
      S.ipre[E] = sit;
    }
  }
  __syncthreads();
  for (int i = tid; i < k * T; i += 256) {
    const int j = i / T, t = i - j * T;
    const int sl = S.slot[j][t];
    if (sl >= 0) S.rowtok[S.off[S.idx[j][t]] + sl] = t;
  }
  __syncthreads();
}

// gate_loss, by workgroup 0: BALANCE = E * sum_e mean_t p[t,e] * (top-1
// share of e), USAGE_STD = population std of the usage + 1e-6 (double).
__device__ float compute_loss(const DecodeArgs& a, const float* prob, DecShared& S) {
  const int tid = threadIdx.x;
  const int T = a.T, E = a.E, k = a.k;
  if (a.loss_kind == LOSS_BALANCE) {
    // E * sum_e me_e * ce_e with me_e the mean probability, ce_e the top-1 share
    double part = 0.0;
    if (tid < E) {
      double me = 0.0;
      for (int t = 0; t < T; ++t) me += (double)prob[(int64_t)t * E + tid];
      part = (me / (double)T) * ((double)S.run[0][tid] / (double)T);
    }
    return (float)(block_sum(part, S.dred) * (double)E);
  }
  // population standard deviation of the experts' shares of all k*T choices
  const double denom = (double)k * (double)T;
  const double u = tid < E ? (double)(S.run[0][tid] + (k == 2 ? S.run[1][tid] : 0)) / denom : 0.0;
  const double mean = block_sum(u, S.dred) / (double)E;
  const double dv = tid < E ? (u - mean) * (u - mean) : 0.0;
  const double var = block_sum(dv, S.dred) / (double)E;
  return (float)(sqrt(var) + 1e-6);
}

// One 16-output x 16-row block of a Linear, the four wavefronts splitting K
// and adding through LDS in wave order; returns on wavefront 0 the sums for
// rows (lane & 15) and outputs 4*(lane>>4) .. +3.
__device__ __forceinline__ f32x4 block_product(const bf16* wrow, const bf16* brow, bool bvalid, int K, DecShared& S) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kq = K / 4;
  const f32x4 acc = lin_quarter(wrow, brow, bvalid, wave * kq, (wave + 1) * kq);
  *reinterpret_cast<f32x4*>(S.red[wave][lane]) = acc;
  __syncthreads();
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = ((S.red[0][lane][i] + S.red[1][lane][i]) + S.red[2][lane][i]) + S.red[3][lane][i];
  }
  __syncthreads();
  return s;
}

// Per-lane view of one work unit of an expert Linear: 16 output features of
// one expert times one block of (up to) 16 of its rows.
struct LinUnit {
  const bf16* w;   // start of the lane's weight row (feature f0 + lane % 16)
  const bf16* b;   // lane's input row at the same K offset (a valid row when past the block's end)
  int e, f0, rb;   // expert, first output feature, first row of the block
};

// One expert Linear (phase 1: x rows -> hidden with bias and activation,
// phase 2: hidden rows -> y_disp with bias) over this workgroup's items
// (blockIdx.x, + gridDim.x, ...; an item is 16 output features of one expert
// with rows, split into 16-row blocks).  The four wavefronts split K into
// quarters and add their partial products through LDS in wave order.  Each
// wavefront keeps a ring of NB K-steps of (weight, input) fragments in
// flight and refills a slot as soon as its product is issued, from the
// current unit or, past its end, from the next one, so the weight stream
// does not pause at unit boundaries.  A quarter whose step count is not a
// multiple of NB is padded with steps that load a valid address and whose
// products are skipped.
template <int NB>
__device__ void decode_linear(const DecodeArgs& a, DecShared& S, int phase) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n16 = lane & 15, q = lane >> 4;
  const int E = a.E, d = a.d, h = a.h;
  const int n1 = h > 0 ? h : d;
  const int nfb1 = n1 / kFB;
  const int K = phase == 1 ? d : h, nout = phase == 1 ? n1 : d;
  const int nfb = nout / kFB;
  const int items = phase == 1 ? S.ipre[E] : S.ipre[E] / nfb1 * nfb;
  const int nst = K / 128;                       // K steps of 32 per wavefront
  const int npad = (nst + NB - 1) / NB * NB;
  const int kw = wave * nst * 32 + q * 8;        // lane's K offset
  const bf16* W = phase == 1 ? a.w1 : a.w2;
  const bf16* X = phase == 1 ? a.x : a.h_disp;
  const bf16* bias = phase == 1 ? a.b1 : a.b2;
  bf16* Y = (phase == 1 && h > 0) ? a.h_disp : a.y_disp;
  const bool act = phase == 1;
  const int nwg = gridDim.x;
  // Weight element k of a row sits at (k / 64) * kb + k % 64 from the row's
  // start: kb = 64 in the row-major layout [E, nout, K]; with packed weights
  // row n of expert e starts block (e * ntf + n / 256) * (K / 64) at
  // (n % 256) * 64 and its K step k / 64 is the block kb = 16384 elements on.
  const bool packed = a.w_packed != 0;
  const int ntf = (nout + 255) / 256;
  const int kb = packed ? 16384 : 64;
  auto wrow = [&](int e, int n) -> const bf16* {
    return packed ? W + (((int64_t)e * ntf + n / 256) * (K / 64)) * 16384 + (n % 256) * 64
                  : W + ((int64_t)e * nout + n) * K;
  };
  auto wat = [&](const bf16* row, int k) -> const bf16* { return row + (k >> 6) * kb + (k & 63); };

  auto unit = [&](int it, int rb) {
    const int key = phase == 1 ? it : (it / nfb) * nfb1;   // the expert's first phase-1 item
    int lo = 0, hi = E;                                     // expert e with ipre[e] <= key < ipre[e+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (S.ipre[mid] <= key) lo = mid; else hi = mid;
    }
    LinUnit u;
    u.e = lo;
    u.f0 = (phase == 1 ? it - S.ipre[lo] : it % nfb) * kFB;
    u.rb = rb;
    u.w = wrow(lo, u.f0 + n16);
    const int rr = rb + n16;
    const int r = S.off[lo] + (rr < S.cnt[lo] ? rr : 0);
    u.b = X + (int64_t)(phase == 1 ? S.rowtok[r] : r) * K + kw;
    return u;
  };

  int it = blockIdx.x;
  if (it >= items) return;                       // uniform over the workgroup
  LinUnit cur = unit(it, 0);
  bf16x8 av[NB], bv[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int s = j < nst ? j : nst - 1;
    av[j] = ldv(wat(cur.w, kw + 32 * s));
    bv[j] = ldv(cur.b + 32 * s);
  }
  for (;;) {
    int nit = it, nrb = cur.rb + kFB;
    if (nrb >= S.cnt[cur.e]) {
      nit = it + nwg;
      nrb = 0;
    }
    const bool more = nit < items;
    const LinUnit nxt = more ? unit(nit, nrb) : cur;
    // the unit's 16 biases come through scalar loads (a uniform address),
    // whose counter is not the vector-memory one: waiting for them in the
    // epilogue does not drain the ring of weight loads
    uint32_t bw[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (bias) {
      const int eu = __builtin_amdgcn_readfirstlane(cur.e), fu = __builtin_amdgcn_readfirstlane(cur.f0);
      typedef const __attribute__((address_space(4))) uint32_t* const_u32p;
      const const_u32p bp = (const_u32p)(bias + (int64_t)eu * nout + fu);
#pragma unroll
      for (int i = 0; i < 8; ++i) bw[i] = bp[i];
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < npad; j0 += NB) {
#pragma unroll
      for (int jj = 0; jj < NB; ++jj) {
        const int s = j0 + jj;
        if (s < nst) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[jj], bv[jj], acc, 0, 0, 0);
        const int s2 = s + NB;
        const bool here = s2 < npad;
        int ss = here ? s2 : s2 - npad;
        ss = ss < nst ? ss : nst - 1;
        av[jj] = ldv(wat(here ? cur.w : nxt.w, kw + 32 * ss));
        bv[jj] = ldv((here ? cur.b : nxt.b) + 32 * ss);
      }
    }
    *reinterpret_cast<f32x4*>(S.red[wave][lane]) = acc;
    __syncthreads();
    const int rr = cur.rb + n16;
    if (wave == 0 && rr < S.cnt[cur.e]) {
      // lane holds row rr, outputs f0 + 4q .. +3
      // this lane's outputs f0 + 4q .. +3 are the bf16 pairs 2q and 2q + 1
      const uint32_t b0 = q == 0 ? bw[0] : q == 1 ? bw[2] : q == 2 ? bw[4] : bw[6];
      const uint32_t b1 = q == 0 ? bw[1] : q == 1 ? bw[3] : q == 2 ? bw[5] : bw[7];
      const float bv4[4] = {__uint_as_float(b0 << 16), __uint_as_float(b0 & 0xffff0000u),
                            __uint_as_float(b1 << 16), __uint_as_float(b1 & 0xffff0000u)};
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = (((S.red[0][lane][i] + S.red[1][lane][i]) + S.red[2][lane][i]) + S.red[3][lane][i]) + bv4[i];
        if (act) v[i] = act_rt(v[i], a.act);
      }
      bf16* dst = Y + (int64_t)(S.off[cur.e] + rr) * nout + cur.f0 + 4 * q;
      *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
    __syncthreads();
    if (!more) break;
    cur = nxt;
    it = nit;
  }
}

__global__ void decode_init_kernel(unsigned* bar) {
  for (int i = threadIdx.x; i < kBarWords; i += blockDim.x) bar[i] = 0u;
}

__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  __shared__ DecShared S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, E = a.E, k = a.k, d = a.d, h = a.h;
  const unsigned nwg = gridDim.x;
  const int n16 = lane & 15, q = lane >> 4;

  __shared__ int bar_ok;
  unsigned phase = 0;   // barriers passed (the counters' targets follow it)
  // a barrier that gave up: the data it guards may be missing, so stop
#define DECODE_BARRIER()                                  \
  if (!grid_barrier(a.bar, ++phase, &bar_ok)) {           \
    if (tid == 0) *a.gate_loss = __builtin_nanf("");      \
    return;                                               \
  }

  // ---------------------------------------------------------------- 1. logits
  // partial router products over a.ks slices of K: items of 16 experts x 16
  // tokens x one slice, the four wavefronts splitting the slice (so that a
  // few tokens still spread the router weight's read over many CUs); the
  // routing phase adds the slices in order
  if (!a.logits_in) {
    const int ne = (E + 15) / 16, nt = (T + 15) / 16, ks = a.ks, kc = d / a.ks;
    for (int it = blockIdx.x; it < ne * nt * ks; it += nwg) {
      const int sl = it % ks, r = it / ks;
      const int e0 = (r % ne) * 16, t0 = (r / ne) * 16;
      const int er = e0 + n16, tr = t0 + n16;
      // rows of the weight past E read expert 0's (their results are dropped)
      const bf16* wrow = a.w_router + (int64_t)(er < E ? er : 0) * d + sl * kc + q * 8;
      const bf16* xrow = a.x + (int64_t)(tr < T ? tr : 0) * d + sl * kc + q * 8;
      const f32x4 acc = block_product(wrow, xrow, tr < T, kc, S);
      if (wave == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = e0 + 4 * q + i;
          if (tr < T && e < E) a.part[((int64_t)sl * T + tr) * E + e] = acc[i];
        }
      }
    }
    DECODE_BARRIER();
  }

  // ---------------------------------------------------------------- 2. routing
  float* prob = a.loss_kind == LOSS_BALANCE ? a.prob : nullptr;
  for (int t = blockIdx.x * 4 + wave; t < T; t += nwg * 4) {
    if (E <= 64) route_token<1>(a, t, prob);
    else if (E <= 128) route_token<2>(a, t, prob);
    else if (E <= 192) route_token<3>(a, t, prob);
    else route_token<4>(a, t, prob);
  }
  DECODE_BARRIER();
  assign_slots(a, S);
  // the caller's outputs of the routing go from the last workgroups, which
  // have the fewest Linear items when the items do not divide evenly
  if (blockIdx.x == nwg - 1) {
    for (int i = tid; i < k * T; i += 256) {
      const int t = i / k, j = i - t * k;
      a.slot[i] = S.slot[j][t];
    }
    for (int e = tid; e <= E; e += 256) {
      if (e < E) a.expert_count[e] = S.cnt[e];
      a.expert_offset[e] = S.off[e];
    }
  }
  if (blockIdx.x == (nwg >= 2 ? nwg - 2 : 0)) {
    const float loss = compute_loss(a, prob, S);
    if (tid == 0) *a.gate_loss = loss;
  }
  // the packed copy of the token rows (x_disp), a row per workgroup in turn
  const int nrows = S.off[E];
  for (int r = blockIdx.x; r < nrows; r += nwg) {
    const uint4* src = reinterpret_cast<const uint4*>(a.x + (int64_t)S.rowtok[r] * d);
    uint4* dst = reinterpret_cast<uint4*>(a.x_disp + (int64_t)r * d);
    for (int v = tid; v < d / 8; v += 256) dst[v] = src[v];
  }

  // ---------------------------------------------------------------- 3./4. Linears
  decode_linear<kRing>(a, S, 1);
  DECODE_BARRIER();
  if (h > 0) {
    decode_linear<kRing>(a, S, 2);
    DECODE_BARRIER();
  }
#undef DECODE_BARRIER

  // ---------------------------------------------------------------- 5. combine
  const int nv = d / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < (int64_t)T * nv; i += (int64_t)nwg * 256) {
    const int t = (int)(i / nv), v = (int)(i % nv);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int sl = S.slot[j][t];
      if (sl < 0) continue;
      const float w = S.w[j][t];
      const uint4 y = reinterpret_cast<const uint4*>(a.y_disp + (int64_t)(S.off[S.idx[j][t]] + sl) * d)[v];
      const uint32_t u[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        acc[2 * qq] = fmaf(w, __uint_as_float(u[qq] << 16), acc[2 * qq]);
        acc[2 * qq + 1] = fmaf(w, __uint_as_float(u[qq] & 0xffff0000u), acc[2 * qq + 1]);
      }
    }
    reinterpret_cast<uint4*>(a.out + (int64_t)t * d)[v] =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                   pack_bf16x2(acc[6], acc[7]));
  }
}

}  // namespace

bool decode_fits(int64_t T, int d, int h, int E, int k, int dtype) {
  if (dtype != DT_BF16 || T < 1 || T > kDecodeMaxTokens || k < 1 || k > 2 || E < k) return false;
  if (d % 128 != 0 || (h > 0 && h % 128 != 0)) return false;
  return true;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (!decode_fits(a.T, a.d, a.h, a.E, a.k, DT_BF16)) return hipErrorNotSupported;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel, 256, 0)) != hipSuccess) return e;
  // one workgroup per CU: the whole grid is resident at once
  if (per_cu < 1 || cus < 1) return hipErrorNotSupported;
  const int grid = cus;
  DecodeArgs args = a;
  // K slices of the router product: the largest divisor of d / 128 (at most
  // kDecodeMaxSlices) that keeps the items at 16 or fewer (more slices spread
  // the router weight wider but give the routing phase more partial sums to
  // gather; 16 items measured best at 1 and 16 tokens)
  const int ntile = ((a.E + 15) / 16) * ((a.T + 15) / 16);
  args.ks = 1;
  for (int c = 2; c <= kDecodeMaxSlices; ++c)
    if ((a.d / 128) % c == 0 && ntile * c <= 16) args.ks = c;
  hipLaunchKernelGGL(decode_init_kernel, dim3(1), dim3(256), 0, s, a.bar);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // a plain launch: the cooperative launch API waits for the device to drain
  // on both sides of the kernel (about 20 us here), and the grid is resident
  // without it (see above)
  hipLaunchKernelGGL(decode_kernel, dim3(grid), dim3(256), 0, s, args);
  return hipGetLastError();
}

}  // namespace moe
