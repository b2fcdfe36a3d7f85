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

#include <algorithm>
#include <utility>

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

__device__ __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }

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

// ---------------------------------------------------------------------------
// Large-tile bf16 kernel: 256 x 256 output tiles, 4 waves each owning 128 x
// 128 of it (16 MFMA 32x32x16 tiles, 256 accumulators per lane), one
// persistent workgroup per CU.  It serves the forward Linears and the four
// GEMMs of the expert backward; the output's rows are the "token side" of
// the tile and its (memory-contiguous) columns the "feature side".
//  * Operands go from global memory straight into LDS (buffer_load ... lds),
//    no register staging.  An operand is either K-contiguous (its rows are
//    tile rows or features, K along the row: the forward's X and W) or
//    transposed (its rows are K, the tile's 256 rows/features along the row:
//    the backward's W as [K, N] and the packed activations as [rows, ·] when
//    the contraction runs over the rows).
//    K-contiguous: each load instruction moves 8 rows x 128 bytes of one
//    64-wide K step; the 16-byte chunk c of row r lands in slot
//    c ^ ((r >> 1) & 7), so the fragment reads of 16 consecutive rows hit
//    16 different bank groups.
//    Transposed: each load instruction moves 2 K rows x 512 bytes; chunk c of
//    K row r lands in slot c ^ ((r & 3) * 4); fragments are read with
//    ds_read_b64_tr_b16 (in each group of 16 lanes, lane i receives element
//    i % 4 of the 8-byte read of lane 4j + i / 4 as its element j), which
//    gives every lane 4 consecutive K values of one column.
//    Rows (or, transposed, K rows) past the valid range lie outside the
//    buffer descriptor's range and read as zero.
//  * Double-buffered 64-wide K steps: the loads of step s+2 are issued during
//    the last sub-step of step s, one per MFMA, and land while step s+1's
//    MFMAs run.
//  * Persistent: the grid is one workgroup per CU; each workgroup walks a
//    strided run of tiles inside its XCD's contiguous share, so the tiles
//    running together on one XCD share operands in its L2.  The first K step
//    of the next tile is loaded while the current tile finishes its last step
//    and its epilogue, and the tile prefix is computed once per workgroup.
//  * Token-row tiles (forward, backward data gradients): an expert's rows are
//    split into ceil(M/256) tiles of equal size rounded up to 32; the two
//    token-side waves take alternate 32-row blocks and skip blocks past the
//    tile's rows, so a short tile costs proportionally less.
//    Weight-gradient tiles: the output is [M, N] per expert and K is the
//    expert's ragged row count (experts without rows are zero-filled apart).
namespace big {
constexpr int BT = 256, BF = 256, BKB = 128;  // BKB: bytes of one row's K step
constexpr int TILE_BYTES = 256 * BKB;          // one 256-row operand tile (both layouts)
constexpr int TRB = 512;                       // bytes of one K row of a transposed tile
// RB: 32-row token blocks per token-side wave: 4 (256-row token tiles), or
// 5 (320 rows) for the forward Linears on K-contiguous operands where the
// caller asks for it (GemmArgs::tile_rows).
constexpr int rows_of(int rb) { return 64 * rb; }
constexpr int stage_of(int rb) { return rows_of(rb) * BKB + TILE_BYTES; }   // token tile + feature tile
constexpr int lds_of(int rb) { return 2 * stage_of(rb); }                    // double buffered
}  // namespace big


// operand layout; OP_GATHER: K-contiguous token rows gathered through a
// packed-row -> token map (the inference forward's first Linear reads x
// itself instead of a dispatched copy)
enum { OP_KC = 0, OP_TR = 1, OP_GATHER = 2 };
enum { BM_ROWS = 0, BM_WGRAD = 1 };     // token-row tiles / weight-gradient tiles
enum { BE_ACT = 0, BE_DACT = 1, BE_STORE = 2, BE_F32 = 3 };   // epilogue

struct BigArgs {
  const bf16* tok;          // token-side operand
  const bf16* feat;         // feature-side operand
  const bf16* bias;         // BE_ACT: [E, N] or null
  const bf16* S;            // BE_DACT: pre-activation [rows, N]
  bf16* Y;                  // output
  float* Yf;                // BE_F32: fp32 output
  bf16* Apre;               // BE_ACT: pre-activation output [rows, N] or null
  const int32_t* offset;    // [E+1]
  int64_t max_rows;         // upper bound on offset[E]
  int64_t tok_ld;           // elements between the token operand's memory rows
  int64_t feat_ld;          // elements between the feature operand's memory rows
  int64_t feat_estride;     // elements between experts' feature operands (0: packed rows)
  int64_t y_ld, y_estride;  // output row pitch; per-expert output stride (weight gradients)
  int32_t E, N, K, M, act;  // K: contraction (token-row tiles); M: output rows (weight gradients)
  int32_t feat_packed;      // K-contiguous feature operand in packed blocks of 256 rows x 64 K
  const int32_t* tok_map;   // OP_GATHER: token row of each packed row
  int64_t tok_rows;         // OP_GATHER: rows of the token operand
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Per-expert tile counts (exclusive prefix in s_pref[0..E]), by wavefront 0:
// token-row tiles ceil(rows/256), or mtw weight-gradient row tiles for every
// expert that has rows.
template <int MODE, int BTR>
__device__ __forceinline__ void big_prefix(const int32_t* __restrict__ offset, int E, int mtw, int* s_pref) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) == 0) {
    int c[4];
    int s = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane * 4 + r;
      const int rows = e < E ? offset[e + 1] - offset[e] : 0;
      c[r] = MODE == BM_WGRAD ? (rows > 0 ? mtw : 0) : (rows + BTR - 1) / BTR;
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

// One output tile as this wave sees it.
struct BigTile {
  int e, row0;            // expert, its first packed row
  int mbase, mvalid;      // first tile row (expert-relative, or output row) and row count
  int n0, nk;             // first feature, 64-wide K steps
  int nbw;                // this wave's valid 32-row token blocks (0..RB)
  const int32_t* map;     // OP_GATHER: the token row of each tile row (tok_map from the tile's first row)
  __amdgpu_buffer_rsrc_t lr;   // the operand this wave loads (token or feature side)
};

// Per-workgroup constants of the big kernel.
struct BigCtx {
  unsigned char* smem;
  int wt, wf, h, r32, wave, lds_op;
  bool tr;                      // this wave's operand is transposed
  uint32_t vbase_e, vbase_o;    // per-lane load offsets for even / odd instructions
  uint32_t sbase, ld_bytes;     // per-wave row base; bytes between operand rows
  uint32_t kstride;             // K-contiguous: bytes between consecutive 64-wide K steps
  uint32_t ch_e, ch_o;          // K-contiguous: this lane's chunk byte offset for even / odd instructions
  uint32_t stage_bytes;         // one stage: token tile + feature tile
  uint32_t tok_half;            // bytes of a token-side wave's half of the token tile
  int rb;                       // 32-row token blocks per token-side wave
};

// slice >= 0: features 64*slice .. +63 of the tile only (K-contiguous
// feature operand, token-row tiles).
template <int TOK, int FEAT, int MODE>
__device__ __forceinline__ BigTile big_tile_desc(const BigArgs& a, const BigCtx& c, int tile, const int* s_pref,
                                                 int ntf, int slice = -1) {
  using namespace big;
  const TileCoord tc = tile_coord(tile, s_pref, a.E, ntf);
  BigTile t;
  t.map = nullptr;
  t.e = tc.e;
  t.row0 = a.offset[tc.e];
  const int rows = a.offset[tc.e + 1] - t.row0;
  t.n0 = tc.nf * BF + (slice > 0 ? slice * 64 : 0);
  if constexpr (MODE == BM_WGRAD) {
    t.mbase = tc.mt * BT;
    t.mvalid = min(BT, a.M - t.mbase);
    t.nk = (rows + 63) / 64;
  } else {
    const int nmt = s_pref[tc.e + 1] - s_pref[tc.e];
    const int per = (((rows + nmt - 1) / nmt) + 31) & ~31;   // rows per tile, balanced
    t.mbase = tc.mt * per;
    t.mvalid = min(per, rows - t.mbase);
    t.nk = a.K / 64;
  }
  const int nvb = (t.mvalid + 31) >> 5;                        // valid 32-row blocks
  // this wave's token blocks are wt, wt+2, wt+4, wt+6; the valid ones are a
  // prefix of that list
  t.nbw = nvb > c.wt ? min(c.rb, (nvb - c.wt + 1) >> 1) : 0;
  if (c.wave >= 2) {
    const int ncols = min(slice >= 0 ? 64 : BF, a.N - t.n0);
    if constexpr (FEAT == OP_KC) {
      // packed: the tile's K steps are consecutive 32 KB blocks whose rows
      // past N are zero, so the descriptor covers all of them (from the
      // slice's first row on)
      const int64_t off = a.feat_packed ? (int64_t)(t.n0 - tc.nf * BF) * 64 + (int64_t)tc.nf * BF * a.feat_ld
                                        : (int64_t)t.n0 * a.feat_ld;
      const bf16* p = a.feat + (int64_t)tc.e * a.feat_estride + off;
      t.lr = make_rsrc(p, a.feat_packed ? (uint32_t)(a.K / 64) * (256u * 128u) - (uint32_t)(t.n0 - tc.nf * BF) * 128u
                                        : (uint32_t)ncols * c.ld_bytes);
    } else {
      const int krows = MODE == BM_WGRAD ? rows : a.K;
      const bf16* p = a.feat + (int64_t)tc.e * a.feat_estride + (MODE == BM_WGRAD ? (int64_t)t.row0 * a.feat_ld : 0) +
                      t.n0;
      t.lr = make_rsrc(p, krows > 0 ? (uint32_t)(((int64_t)(krows - 1) * a.feat_ld + ncols) * 2) : 0u);
    }
  } else {
    if constexpr (TOK == OP_GATHER) {
      // the whole token matrix; each load's source row comes from the map
      // (big_map_load / big_map_offsets)
      t.lr = make_rsrc(a.tok, (uint32_t)(a.tok_rows * c.ld_bytes));
      t.map = a.tok_map + t.row0 + t.mbase;
    } else if constexpr (TOK == OP_KC) {
      const bf16* p = a.tok + (int64_t)(t.row0 + t.mbase) * a.tok_ld;
      t.lr = make_rsrc(p, (uint32_t)t.mvalid * c.ld_bytes);
    } else {
      const bf16* p = a.tok + (int64_t)t.row0 * a.tok_ld + t.mbase;
      t.lr = make_rsrc(p, rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * a.tok_ld + t.mvalid) * 2) : 0u);
    }
  }
  return t;
}

// Load number i (0..15) of this wave's share of one 64-wide K step (kstep)
// into a stage.  K-contiguous: 8 rows x 128 bytes; waves 0-1 fill the token
// tile, waves 2-3 the feature tile (feature rows permuted so the MFMA row
// m = lane&31 reads feature ((m>>2)&1)*16 + (m>>3)*4 + (m&3)); the row goes
// in the per-lane offset, which the buffer range check always covers, and
// only the position along K (inside a valid row, or, for packed weights,
// the K step's 32 KB block of the tile) in the scalar offset.
// Transposed: K rows 2i, 2i+1 of this wave's 32, 512 bytes each; the K row
// goes in the per-lane offset (K rows past the end read as zero).
// nfw: 32-feature blocks per feature-side wave (4, or 1 in a 64-feature
// slice, whose waves load 4 instructions each).
// GATHER: the token waves take their per-lane byte offset from gv (load i's
// gathered row and chunk, from big_map_offsets) instead of the tile row.
template <bool GATHER, bool SOFF>
__device__ __forceinline__ void big_issue_one(const BigCtx& c, __amdgpu_buffer_rsrc_t lr, int stage, int kstep, int i,
                                              int nfw = 4, uint32_t gv = 0) {
  using namespace big;
  // both layouts put load i of this wave at the same LDS offset: 16 KB per
  // wave (4 KB per wave in a slice), 1 KB per instruction (8 rows x 128 B,
  // or 2 K rows x 512 B)
  const bool fw = c.wave >= 2;
  unsigned char* dst = c.smem + stage * c.stage_bytes + c.lds_op + (c.wave & 1) * (fw ? 4096u * nfw : c.tok_half) +
                       i * 1024;
  // wave-uniform row offset and K offset, chosen without a branch
  const uint32_t g = fw ? (uint32_t)((i >> 2) * 32 + (i & 3) * 4) : (uint32_t)(i * 8);
  const uint32_t kc_row = (fw ? (uint32_t)(c.wave & 1) * 32u * (uint32_t)nfw * c.ld_bytes : c.sbase) + g * c.ld_bytes;
  const uint32_t tr_row = (uint32_t)(kstep * 64 + (c.wave & 1) * 32 + 2 * i) * c.ld_bytes;
  const uint32_t vrow = c.tr ? tr_row : kc_row;
  uint32_t soff, voff;
  if constexpr (SOFF) {
    // the row in the scalar offset (both offsets count towards the range
    // check): no per-load VGPR, which the 320-row tile needs for its fifth
    // accumulator block; with the VGPR to spare the per-lane form is faster
    soff = vrow + (uint32_t)kstep * c.kstride;
    voff = (i & 1) ? c.vbase_o : c.vbase_e;
  } else {
    soff = c.tr ? 0u : (uint32_t)kstep * c.kstride;
    voff = ((i & 1) ? c.vbase_o : c.vbase_e) + vrow;
  }
  if constexpr (GATHER) {
    if (!fw) {
      voff = gv;
      soff = (uint32_t)kstep * c.kstride;
    }
  }
  __builtin_amdgcn_raw_ptr_buffer_load_lds(lr, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

template <int NF, bool GATHER, int RB>
__device__ __forceinline__ void big_issue(const BigCtx& c, __amdgpu_buffer_rsrc_t lr, int stage, int kstep,
                                          const uint32_t (&gv)[16]) {
#pragma unroll
  for (int i = 0; i < 4 * RB; ++i)
    if (c.wave < 2 || i < 4 * NF) big_issue_one<GATHER, RB == 5>(c, lr, stage, kstep, i, NF, gv[GATHER ? i : 0]);   // gathering: RB == 4, 16 loads
  static_assert(!GATHER || RB == 4, "gathered token rows use 256-row tiles");
}

// Gathered token rows, token waves: raw[i] = the token row that load i of
// this lane reads (tile row (wave&1)*128 + 8i + lane/8), or -1 past the
// tile's nvalid rows; then the loads' byte offsets (row and this lane's
// chunk; a row of -1 becomes an offset past every descriptor's end, which
// reads zeros).  The two are separate so that the map loads can be issued
// long before their values are needed.
__device__ __forceinline__ void big_map_load(const BigCtx& c, const int32_t* map, int nvalid, int32_t (&raw)[16]) {
  const int lrow = (threadIdx.x & 63) >> 3;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = (c.wave & 1) * 128 + 8 * i + lrow;
    raw[i] = (c.wave < 2 && r < nvalid) ? map[r] : -1;
  }
}

__device__ __forceinline__ void big_map_offsets(const BigCtx& c, const int32_t (&raw)[16], uint32_t (&gv)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    gv[i] = raw[i] < 0 ? 0xF0000000u : (uint32_t)raw[i] * c.ld_bytes + ((i & 1) ? c.ch_o : c.ch_e);
}

// This tile's bias (zero without one) into LDS for the epilogue.
__device__ __forceinline__ void big_bias(const BigArgs& a, const BigTile& t, float* s_bias) {
  const int f = t.n0 + threadIdx.x;
  s_bias[threadIdx.x] = (a.bias && f < a.N) ? static_cast<float>(a.bias[(int64_t)t.e * a.N + f]) : 0.f;
}

// Read one accumulator element out of its AGPR at the point of use.  Without
// this the compiler copies all 256 accumulators into VGPRs when the K loop
// ends and spills part of them to scratch.
__device__ __forceinline__ float agpr_read(float v) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(v));
  return r;
}

// One MFMA whose accumulator the register allocator must keep in VGPRs: a
// 320-row tile needs 320 accumulators per lane, 64 more than the AGPR file
// holds, and with the compiler choosing the register class of every MFMA it
// copied accumulators between the two files on every K step.  The 32x32x16
// MFMA is 8 passes; the only later readers of these registers are the
// following MFMAs on the same block (a sub-step later, with the
// back-to-back accumulation the hardware supports) and the epilogue, which
// waits out the write-to-VALU-read interval first (big_tile).
__device__ __forceinline__ void mfma_vacc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// The accumulator block blk = ff*4 + tt, read out of its AGPRs (constant
// indices inside each case; blocks with tt >= NB or ff >= NF do not exist).
template <int NB, int NF, int RB>
__device__ __forceinline__ void acc_block(const f32x16 (&acc)[NF][RB], int blk, float (&v)[16]) {
  switch (blk) {
#define MOE_AB(FF, TT)                                              \
  case FF * RB + TT:                                                \
    if constexpr (TT < NB && FF < NF && TT < RB) {                  \
      _Pragma("unroll") for (int r = 0; r < 16; ++r) v[r] = agpr_read(acc[FF][TT][r]); \
    }                                                               \
    break;
    MOE_AB(0, 0) MOE_AB(0, 1) MOE_AB(0, 2) MOE_AB(0, 3)
    MOE_AB(1, 0) MOE_AB(1, 1) MOE_AB(1, 2) MOE_AB(1, 3)
    MOE_AB(2, 0) MOE_AB(2, 1) MOE_AB(2, 2) MOE_AB(2, 3)
    MOE_AB(3, 0) MOE_AB(3, 1) MOE_AB(3, 2) MOE_AB(3, 3)
#undef MOE_AB
#define MOE_AB5(FF)                                                 \
  case RB == 5 ? FF * RB + 4 : 100 + FF:                            \
    if constexpr (RB == 5 && 4 < NB && FF < NF) {                   \
      _Pragma("unroll") for (int r = 0; r < 16; ++r) v[r] = acc[FF][RB - 1][r]; \
    }                                                               \
    break;
    MOE_AB5(0) MOE_AB5(1) MOE_AB5(2) MOE_AB5(3)
#undef MOE_AB5
    default: break;
  }
}

// d/dx of the activation, from the same erf as gelu_fast: for GELU
// Phi(x) + x phi(x), with phi(x) = exp(-x^2/2) / sqrt(2 pi).
template <int ACT>
__device__ __forceinline__ float act_grad_fixed(float x) {
  if constexpr (ACT == ACT_RELU) {
    return x > 0.f ? 1.f : 0.f;
  } else if constexpr (ACT == ACT_GELU) {
    const float z = fabsf(x) * 0.7071067811865476f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.f));
    float poly = fmaf(1.061405429f, t, -1.453152027f);
    poly = fmaf(poly, t, 1.421413741f);
    poly = fmaf(poly, t, -0.284496736f);
    poly = fmaf(poly, t, 0.254829592f);
    poly *= t;
    const float e = __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);   // exp(-x^2/2)
    const float erf_v = __builtin_copysignf(fmaf(-poly, e, 1.f), x);
    return 0.5f * (1.f + erf_v) + x * e * 0.3989422804014327f;
  } else {
    return 1.f;
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Epilogue of one 32x32 accumulator: this lane's 16 consecutive output
// columns f0.. of tile row rloc, as two 16-byte vectors.
//  BE_ACT:   + bias (from LDS), optional pre-activation store, activation.
//  BE_DACT:  times act'(S) at the same position.
//  BE_STORE: as is.
//  BE_F32:   as is, in fp32 (four 16-byte vectors).
template <int EPI, int ACT, int MODE>
__device__ __forceinline__ void big_store(const BigArgs& a, float (&v)[16], const BigTile& t, int rloc, int fl,
                                          const float* s_bias) {
  const int f0 = t.n0 + fl;
  int64_t off;
  if constexpr (MODE == BM_WGRAD)
    off = (int64_t)t.e * a.y_estride + (int64_t)(t.mbase + rloc) * a.y_ld + f0;
  else
    off = ((int64_t)t.row0 + t.mbase + rloc) * a.y_ld + f0;
  if constexpr (EPI == BE_ACT) {
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] += s_bias[fl + r];
    if (a.Apre) {
      uint4* p = reinterpret_cast<uint4*>(a.Apre + off);
      p[0] = make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
      p[1] = make_uint4(pack2(v[8], v[9]), pack2(v[10], v[11]), pack2(v[12], v[13]), pack2(v[14], v[15]));
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = act_fixed<ACT>(v[r]);
  } else if constexpr (EPI == BE_DACT) {
    if constexpr (ACT != ACT_NONE) {
      const uint4* sp = reinterpret_cast<const uint4*>(a.S + off);
      const uint4 s0 = sp[0], s1 = sp[1];
      const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        v[2 * q] *= act_grad_fixed<ACT>(bf16_lo(sw[q]));
        v[2 * q + 1] *= act_grad_fixed<ACT>(bf16_hi(sw[q]));
      }
    }
  }
  if constexpr (EPI == BE_F32) {
    float4* q = reinterpret_cast<float4*>(a.Yf + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    return;
  }
  uint4* p = reinterpret_cast<uint4*>(a.Y + off);
  p[0] = make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
  p[1] = make_uint4(pack2(v[8], v[9]), pack2(v[10], v[11]), pack2(v[12], v[13]), pack2(v[14], v[15]));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// One ds_read_b64_tr_b16.  The restrict-qualified pointer gives the read
// alias-scope information; without it the compiler assumes the read may
// alias any LDS-DMA load in flight and puts a full vmcnt(0) wait before it,
// which serialises the load pipeline.  The kernel's own waitcnt + barrier at
// every K step already keeps reads off a stage whose loads are in flight.
__device__ __forceinline__ v4i16 ds_read_tr16(const __attribute__((address_space(3))) v4i16* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
}

// One fragment of 8 K values (sub-step i) of a transposed operand: two
// ds_read_b64_tr_b16 of 4 K rows each.  col is this lane's source column for
// the read (its group of 16 lanes covers 16 columns of one 32-wide block).
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char* tile, int i, int h, int lane16, int col) {
  using namespace big;
  const int k0 = 8 * (h * 4 + i) + (lane16 >> 2);            // K row of this lane's first read
  const int sw = ((col >> 3) ^ ((lane16 >> 2) * 4)) * 16 + (col & 7) * 2;
  const v4i16 lo = ds_read_tr16((const __attribute__((address_space(3))) v4i16*)(tile + k0 * TRB + sw));
  const v4i16 hi = ds_read_tr16((const __attribute__((address_space(3))) v4i16*)(tile + (k0 + 4) * TRB + sw));
  const v8i16 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, r);
}

// One wave's share of a tile with NB valid 32-row token blocks (NB in 0..4)
// and NF 32-feature blocks (4; 1 in a 64-feature slice): every wave runs the
// same K steps and barriers; MFMAs of absent blocks are not issued at all,
// and each 32x32 block sees the same MFMA sequence whatever NB and NF.
// Accumulators live only inside this function.  K step s of this tile sits
// in stage (s + sb) & 1; its step 0 was issued before the call unless
// `cold`.  If there is a next tile (always a whole one), its step 0 is
// issued into the stage this tile's step nk-2 used (the other stage when
// nk == 1), which is stage 0 of the next tile's numbering with
// sb' = (sb + nk) & 1.
template <int NB, int NF, int EPI, int ACT, int TOK, int FEAT, int MODE, int RB>
__device__ __forceinline__ void big_tile(const BigArgs& a, const BigCtx& c, const BigTile& t, int sb, bool has_next,
                                         __amdgpu_buffer_rsrc_t next_lr, const int32_t* next_map, int next_valid,
                                         uint32_t (&gv)[16], const float* s_bias, bool cold) {
  constexpr bool GATHER = TOK == OP_GATHER;
  static_assert(RB == 4 || (RB == 5 && TOK == OP_KC && FEAT == OP_KC && MODE == BM_ROWS), "320-row tiles: forward only");
  constexpr int LPH = 2 * RB;      // loads per half of a K step's loads (token side: 4 * RB in all)
  using namespace big;
  unsigned char* smem = c.smem;
  const int nk = t.nk, wt = c.wt, wf = c.wf, h = c.h, r32 = c.r32;
  const int N = a.N;
  const int lane = threadIdx.x & 63, lane16 = lane & 15, mh = (lane >> 4) & 1, q4 = lane & 3;
  f32x16 acc[NF][RB];
#pragma unroll
  for (int i = 0; i < NF; ++i)
#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // Fragment registers: four sets, so that sub-step i+2's fragments are read
  // while sub-step i's MFMAs run (sub-step i uses set i), two sub-steps
  // (about 1000 cycles) ahead of their use.  Sub-step i of a 64-wide K step
  // covers, for lane half h, the 8 K values of chunk h*4+i (the same order
  // on both operands, which leaves the dot product alone).
  bf16x8 fa[4][NF], fb[4][NB > 0 ? NB : 1];
  constexpr int NM = NF * NB;      // MFMAs per sub-step
  constexpr int NR = NF + NB;      // fragment reads per sub-step
  // transposed-read source columns of this lane within a 32-wide block: the
  // token side reads columns in order, the feature side in the permuted order
  // that gives each lane 16 consecutive output features
  const int tok_col = mh * 16 + 4 * q4;
  const int feat_col = (q4 & 1) * 16 + mh * 8 + (q4 >> 1) * 4;
  // fragment read r of sub-step i from a stage into a set, in the order the
  // MFMAs consume them: token block 0, the four feature blocks, then the
  // other token blocks
  auto read1 = [&](int stage, int i, int set, int r) {
    const unsigned char* Xs = smem + stage * stage_of(RB);
    const unsigned char* Ws = Xs + rows_of(RB) * BKB;
    const int sw = (((h * 4 + i) ^ ((r32 >> 1) & 7)) * 16);
    const bool tokr = NB > 0 && (r == 0 || r >= NF + 1);
    const int tt = r == 0 ? 0 : r - NF;
    const int ff = NB > 0 ? r - 1 : r;
    if (tokr) {
      if constexpr (TOK != OP_TR)
        fb[set][tt] = *reinterpret_cast<const bf16x8*>(Xs + ((wt + 2 * tt) * 32 + r32) * BKB + sw);
      else
        fb[set][tt] = tr_frag(Xs, i, h, lane16, (wt + 2 * tt) * 32 + tok_col);
    } else {
      if constexpr (FEAT == OP_KC)
        fa[set][ff] = *reinterpret_cast<const bf16x8*>(Ws + (wf * 32 * NF + ff * 32 + r32) * BKB + sw);
      else
        fa[set][ff] = tr_frag(Ws, i, h, lane16, wf * 32 * NF + ff * 32 + feat_col);
    }
  };
  // MFMA j of a sub-step: token block j / NF with feature block j % NF
  auto mfma1 = [&](int set, int j) {
    const int tt = j / NF, ff = j % NF;
    if constexpr (NB == 5) {
      if (tt == 4) {   // the fifth token block: accumulators in VGPRs
        mfma_vacc(acc[ff][4], fa[set][ff], fb[set][4]);
        return;
      }
    }
    acc[ff][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][ff], fb[set][tt], acc[ff][tt], 0, 0, 0);
  };
  // One sub-step in a fixed issue order: each MFMA is followed by its share
  // of the fragment reads of the sub-step two ahead (one after each of the
  // first NR MFMAs) and, when loading, of half (lhalf) of the 4 * RB
  // global->LDS loads, so that the memory instructions issue in the shadow
  // of the MFMAs instead of in a bubble.
  auto substep = [&](auto loads, int mset, int rstage, int ri, int rset, __amdgpu_buffer_rsrc_t llr, int lstage,
                     int lkstep, int lhalf) {
    constexpr bool LOADS = decltype(loads)::value;
    constexpr int NJ = NM > NR ? NM : NR;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j < NM) mfma1(mset, j);
      if constexpr (LOADS) {
        if constexpr (NM > 0) {
#pragma unroll
          for (int q = j * LPH / NM; q < (j + 1) * LPH / NM && j < NM; ++q)
            if (c.wave < 2 || lhalf * LPH + q < 4 * NF)
              big_issue_one<GATHER, RB == 5>(c, llr, lstage, lkstep, lhalf * LPH + q, NF,
                                    gv[GATHER ? lhalf * LPH + q : 0]);
        } else {
          if (j == 0) {
#pragma unroll
            for (int q = 0; q < LPH; ++q)
              if (c.wave < 2 || lhalf * LPH + q < 4 * NF)
                big_issue_one<GATHER, RB == 5>(c, llr, lstage, lkstep, lhalf * LPH + q, NF,
                                      gv[GATHER ? lhalf * LPH + q : 0]);
          }
        }
      }
      if (j < NR && ri >= 0) read1(rstage, ri, rset, j);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using NoLoads = std::integral_constant<bool, false>;
  using Loads = std::integral_constant<bool, true>;
  const __amdgpu_buffer_rsrc_t no_lr = make_rsrc(a.tok, 0);
  // Stage s holds K step s (mod 2, offset by sb).  The one barrier per step
  // sits before sub-step 2: by then every wave has read all of the current
  // stage (sub-steps 2 and 3 were read during 0 and 1, so the loads two
  // steps ahead may overwrite it) and the next stage has landed (so its
  // first two sub-steps can be read while sub-steps 2 and 3 compute).  The
  // last step is peeled off so that in the loop the operands read after the
  // barrier are known to have arrived at its wait.  What sub-steps 2 and 3
  // of step kt load into the stage they have just finished: step kt+2 of
  // this tile, else step 0 of the next tile, else nothing (a descriptor with
  // no records: the loads return zeros and touch no memory).
  const __amdgpu_buffer_rsrc_t tail_lr = has_next ? next_lr : no_lr;
  // GATHER: gv holds this tile's load offsets until the loads turn to the
  // next tile's first K step; the next tile's map is read during the first
  // K step, a step before the barrier that waits for it
  int32_t nraw[16];
  if (cold) big_issue<NF, GATHER, RB>(c, t.lr, sb & 1, 0, gv);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  if (nk > 1) {
    big_issue<NF, GATHER, RB>(c, t.lr, (sb + 1) & 1, 1, gv);
  } else {
    if constexpr (GATHER) {
      big_map_load(c, next_map, has_next ? next_valid : 0, nraw);
      big_map_offsets(c, nraw, gv);
    }
    big_issue<NF, GATHER, RB>(c, tail_lr, (sb + 1) & 1, 0, gv);
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) read1(sb, 0, 0, r);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < NR; ++r) read1(sb, 1, 1, r);
  __builtin_amdgcn_sched_barrier(0);
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const int cur = (kt + sb) & 1;
    substep(NoLoads{}, 0, cur, 2, 2, no_lr, 0, 0, 0);
    substep(NoLoads{}, 1, cur, 3, 3, no_lr, 0, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);  // own loads of the next stage and own reads of this one
    __builtin_amdgcn_s_barrier();
    const bool more = kt + 2 < nk;
    const __amdgpu_buffer_rsrc_t llr = more ? t.lr : tail_lr;
    if constexpr (GATHER) {
      if (kt == 0) big_map_load(c, next_map, has_next ? next_valid : 0, nraw);
      if (!more) big_map_offsets(c, nraw, gv);
    }
    substep(Loads{}, 2, cur ^ 1, 0, 0, llr, cur, more ? kt + 2 : 0, 0);
    substep(Loads{}, 3, cur ^ 1, 1, 1, llr, cur, more ? kt + 2 : 0, 1);
  }
  {
    const int cur = (nk - 1 + sb) & 1;
    substep(NoLoads{}, 0, cur, 2, 2, no_lr, 0, 0, 0);
    substep(NoLoads{}, 1, cur, 3, 3, no_lr, 0, 0, 0);
    substep(NoLoads{}, 2, cur, -1, 0, no_lr, 0, 0, 0);
    substep(NoLoads{}, 3, cur, -1, 0, no_lr, 0, 0, 0);
  }

  // the fifth block's accumulators come from MFMAs the compiler cannot see
  // into: wait out the MFMA-write to VALU-read interval before any read
  if constexpr (NB == 5) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  // one compact loop over the accumulator blocks keeps the epilogue small
  // enough to stay in the instruction cache
#pragma nounroll
  for (int blk = 0; blk < RB * NF; ++blk) {
    const int ff = blk / RB, tt = blk - ff * RB;
    const int rloc = (wt + 2 * tt) * 32 + r32;
    const int fl = wf * 32 * NF + ff * 32 + h * 16;   // column offset within the tile
    if (tt >= NB || t.n0 + fl >= N) continue;
    float v[16];
    acc_block<NB, NF, RB>(acc, blk, v);
    if (rloc < t.mvalid) big_store<EPI, ACT, MODE>(a, v, t, rloc, fl, s_bias);
  }
}

template <int EPI, int ACT, int TOK, int FEAT, int MODE, int RB>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_big_kernel(BigArgs a) {
  using namespace big;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_pref[MOE_MAX_EXPERTS_DEV + 1];
  __shared__ float s_bias[2][BF];   // alternate tiles use alternate halves

  const int E = a.E, N = a.N;
  const int ntf = (N + BF - 1) / BF;
  const int mtw = MODE == BM_WGRAD ? (a.M + BT - 1) / BT : 0;
  big_prefix<MODE, rows_of(RB)>(a.offset, E, mtw, s_pref);
  __syncthreads();
  const int total = s_pref[E] * ntf;
  // Tail split (forward token-row tiles): when the tiles leave a last round
  // that at most a quarter of the workgroups would run (R = total mod G of
  // them; or all tiles, when there are at most G / 4), every workgroup runs
  // exactly floor(total / G) whole tiles and the R leftover tiles run as
  // four 64-feature slices each, on four workgroups of the leftover tile's
  // XCD, after their whole tiles.  A slice gives the same bits as the whole
  // tile (each 32x32 block, the same MFMA sequence).
  const int G = gridDim.x;
  int R = 0;
  if constexpr (MODE == BM_ROWS && FEAT == OP_KC) {
    // the slice map below needs 4 * ceil(R / 8) workgroups per XCD
    const int r = total % G;
    if ((total > G || total * 4 <= G) && r * 4 <= G && ((r + kXcds - 1) / kXcds) * 4 <= G / kXcds) R = r;
  }
  const int F = total - R;   // whole tiles
  // this XCD's contiguous share of the whole tiles, walked with stride L by
  // its L workgroups (XCDs take workgroups round-robin)
  const int per_xcd = G / kXcds;
  const int share = (F + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds;
  const int loc = (int)blockIdx.x / kXcds;
  const int t_end = min(F, (xcd + 1) * share);
  int tile = xcd * share + loc;
  // this workgroup's slice: leftover tile (loc / 4) * 8 + xcd, slice loc % 4
  const int slice_tile = (loc / 4) * kXcds + xcd;
  const bool has_slice = slice_tile < R;
  if (tile >= t_end && !has_slice) return;

  // the wave index is uniform across the wave; say so, so that descriptor
  // and LDS-base choices below stay in scalar registers
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  BigCtx c;
  c.smem = smem;
  c.wt = wave >> 1;
  c.wf = wave & 1;
  c.h = lane >> 5;
  c.r32 = lane & 31;
  c.wave = wave;
  c.rb = RB;
  c.stage_bytes = stage_of(RB);
  c.tok_half = 32 * RB * BKB;
  c.lds_op = wave >= 2 ? rows_of(RB) * BKB : 0;
  c.tr = wave >= 2 ? FEAT == OP_TR : TOK == OP_TR;
  c.ld_bytes = (uint32_t)((wave >= 2 ? a.feat_ld : a.tok_ld) * 2);
  c.kstride = 128;
  if (wave >= 2 && FEAT == OP_KC && a.feat_packed) {
    // packed weights: a K step of the tile is one block of 256 rows x 128 B
    c.ld_bytes = 128;
    c.kstride = 256 * 128;
  }
  if (!c.tr) {
    // K-contiguous: this lane's source row / chunk for each of its 16 load
    // instructions.  Chunk c of tile row r sits in slot c ^ ((r >> 1) & 7).
    // For load i the rows are 8i + lrow (+ a multiple of 16 per wave), so
    // (r >> 1) & 7 = 4 * (i & 1) + (lrow >> 1): two lane patterns, even and
    // odd i.  Load i of this wave covers tile rows (wave&1)*128 + i*8 .. +7.
    // For the token side the source row is that row; for the feature side it
    // is the permuted feature, which works out to a per-lane part
    // ((lrow>>2)&1)*16 + (lrow&3) plus a wave-uniform part (i>>2)*32 +
    // (i&3)*4, so each load needs one VGPR offset and one SGPR offset.
    const int lrow = lane >> 3;
    const int chunk_e = (lane & 7) ^ (lrow >> 1);
    const int chunk_o = (lane & 7) ^ (4 + (lrow >> 1));
    const uint32_t vrow = (uint32_t)(wave >= 2 ? (((lrow >> 2) & 1) * 16 + (lrow & 3)) : lrow) * c.ld_bytes;
    c.vbase_e = vrow + chunk_e * 16;
    c.vbase_o = vrow + chunk_o * 16;
    c.ch_e = chunk_e * 16;
    c.ch_o = chunk_o * 16;
    c.sbase = (uint32_t)(wave & 1) * 32 * RB * c.ld_bytes;
  } else {
    // Transposed: load i moves K rows r, r+1 (r = (wave&1)*32 + 2i), lane j
    // filling slot j % 32 of row r + j / 32; slot p of K row r holds chunk
    // p ^ ((r & 3) * 4), and (r & 3) = 2 * (i & 1) + j / 32.
    const int half = lane >> 5, p = lane & 31;
    c.vbase_e = (uint32_t)half * c.ld_bytes + (uint32_t)((p ^ (half * 4)) * 16);
    c.vbase_o = (uint32_t)half * c.ld_bytes + (uint32_t)((p ^ ((2 + half) * 4)) * 16);
    c.sbase = 0;
  }

  int sb = 0, par = 0;
  // OP_GATHER: the token waves' load offsets of the tile in hand (see big_tile)
  uint32_t gv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) gv[i] = 0u;
  if (tile < t_end) {
    BigTile cur = big_tile_desc<TOK, FEAT, MODE>(a, c, tile, s_pref, ntf);
    if constexpr (TOK == OP_GATHER) {
      int32_t raw[16];
      big_map_load(c, cur.map, cur.mvalid, raw);
      big_map_offsets(c, raw, gv);
    }
    big_issue<4, TOK == OP_GATHER, RB>(c, cur.lr, 0, 0, gv);
    if constexpr (EPI == BE_ACT) big_bias(a, cur, s_bias[0]);
    for (;;) {
      const int next = tile + per_xcd;
      const bool has_next = next < t_end;
      BigTile nt = cur;
      if (has_next) nt = big_tile_desc<TOK, FEAT, MODE>(a, c, next, s_pref, ntf);
      switch (cur.nbw) {
        case 5:
          if constexpr (RB == 5)
            big_tile<5, 4, EPI, ACT, TOK, FEAT, MODE, RB>(a, c, cur, sb, has_next, nt.lr, nt.map, nt.mvalid, gv, s_bias[par], false);
          break;
        case 4: big_tile<4, 4, EPI, ACT, TOK, FEAT, MODE, RB>(a, c, cur, sb, has_next, nt.lr, nt.map, nt.mvalid, gv, s_bias[par], false); break;
        case 3: big_tile<3, 4, EPI, ACT, TOK, FEAT, MODE, RB>(a, c, cur, sb, has_next, nt.lr, nt.map, nt.mvalid, gv, s_bias[par], false); break;
        case 2: big_tile<2, 4, EPI, ACT, TOK, FEAT, MODE, RB>(a, c, cur, sb, has_next, nt.lr, nt.map, nt.mvalid, gv, s_bias[par], false); break;
        case 1: big_tile<1, 4, EPI, ACT, TOK, FEAT, MODE, RB>(a, c, cur, sb, has_next, nt.lr, nt.map, nt.mvalid, gv, s_bias[par], false); break;
        default: big_tile<0, 4, EPI, ACT, TOK, FEAT, MODE, RB>(a, c, cur, sb, has_next, nt.lr, nt.map, nt.mvalid, gv, s_bias[par], false); break;
      }
      // the next tile's numbering starts at the stage this tile's step nk-2
      // used, whose last reads came before this tile's last barrier
      sb = (sb + cur.nk) & 1;
      par ^= 1;
      if (!has_next) break;
      if constexpr (EPI == BE_ACT) big_bias(a, nt, s_bias[par]);   // visible after the next tile's first barrier
      cur = nt;
      tile = next;
    }
  }
  if constexpr (MODE == BM_ROWS && FEAT == OP_KC) {
    if (has_slice) {
      const BigTile st = big_tile_desc<TOK, FEAT, MODE>(a, c, F + slice_tile, s_pref, ntf, loc % 4);
      if (st.n0 < a.N) {   // uniform: the slice's first feature
        if constexpr (EPI == BE_ACT) big_bias(a, st, s_bias[par]);   // visible after the slice's first barrier
        if constexpr (TOK == OP_GATHER) {
          int32_t raw[16];
          big_map_load(c, st.map, st.mvalid, raw);
          big_map_offsets(c, raw, gv);
        }
        const __amdgpu_buffer_rsrc_t none = make_rsrc(a.tok, 0);
        switch (st.nbw) {
          case 5:
            if constexpr (RB == 5)
              big_tile<5, 1, EPI, ACT, TOK, FEAT, MODE, RB>(a, c, st, sb, false, none, nullptr, 0, gv, s_bias[par], true);
            break;
          case 4: big_tile<4, 1, EPI, ACT, TOK, FEAT, MODE, RB>(a, c, st, sb, false, none, nullptr, 0, gv, s_bias[par], true); break;
          case 3: big_tile<3, 1, EPI, ACT, TOK, FEAT, MODE, RB>(a, c, st, sb, false, none, nullptr, 0, gv, s_bias[par], true); break;
          case 2: big_tile<2, 1, EPI, ACT, TOK, FEAT, MODE, RB>(a, c, st, sb, false, none, nullptr, 0, gv, s_bias[par], true); break;
          case 1: big_tile<1, 1, EPI, ACT, TOK, FEAT, MODE, RB>(a, c, st, sb, false, none, nullptr, 0, gv, s_bias[par], true); break;
          default: big_tile<0, 1, EPI, ACT, TOK, FEAT, MODE, RB>(a, c, st, sb, false, none, nullptr, 0, gv, s_bias[par], true); break;
        }
      }
    }
  }
}

// Zero the weight gradient of every expert without rows (their tiles are not
// in the weight-gradient schedule).
__global__ __launch_bounds__(256) void zero_empty_experts_kernel(bf16* Y, const int32_t* offset, int64_t per_expert) {
  const int e = blockIdx.y;
  if (offset[e + 1] != offset[e]) return;
  uint4* p = reinterpret_cast<uint4*>(Y + (int64_t)e * per_expert);
  const int64_t n = per_expert / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
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

template <int EPI, int ACT, int TOK, int FEAT, int MODE, int RB = 4>
hipError_t launch_big(const BigArgs& a, hipStream_t s) {
  auto kern = gemm_bf16_big_kernel<EPI, ACT, TOK, FEAT, MODE, RB>;
  constexpr int lds = big::lds_of(RB);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  // at most one workgroup per CU (LDS use allows no more), never more than
  // the worst-case tile count (four slices per tile on the forward path,
  // which splits a short round of tiles), a whole number per XCD
  const int64_t ntf = (a.N + big::BF - 1) / big::BF;
  const int64_t mtiles = MODE == BM_WGRAD ? (int64_t)a.E * ((a.M + big::BT - 1) / big::BT)
                                          : (a.max_rows + big::rows_of(RB) - 1) / big::rows_of(RB) + a.E;
  const int64_t units = (MODE == BM_ROWS && FEAT == OP_KC ? 4 : 1) * mtiles * ntf;
  int64_t grid = std::min<int64_t>(units, device_cus());
  grid = std::max<int64_t>(kXcds, grid / kXcds * kXcds);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int EPI, int TOK, int FEAT, int MODE, int RB = 4>
hipError_t launch_big_act(const BigArgs& a, hipStream_t s) {
  if (a.act == ACT_GELU) return launch_big<EPI, ACT_GELU, TOK, FEAT, MODE, RB>(a, s);
  if (a.act == ACT_RELU) return launch_big<EPI, ACT_RELU, TOK, FEAT, MODE, RB>(a, s);
  return launch_big<EPI, ACT_NONE, TOK, FEAT, MODE, RB>(a, s);
}

hipError_t launch_bf16_big(const GemmArgs& g, hipStream_t s) {
  BigArgs a{};
  a.tok = static_cast<const bf16*>(g.X);
  a.feat = static_cast<const bf16*>(g.W);
  a.bias = static_cast<const bf16*>(g.bias);
  a.S = nullptr;
  a.Y = static_cast<bf16*>(g.Y);
  a.Apre = static_cast<bf16*>(g.Apre);
  a.offset = g.offset;
  a.max_rows = g.max_rows;
  a.tok_ld = g.x_ld ? g.x_ld : g.K;
  a.feat_ld = g.K;
  // packed: an expert's blocks cover ceil(N/256) * 256 rows; tile nf still
  // starts nf * 256 * K elements into them
  a.feat_estride = (int64_t)(g.w_packed ? (g.N + big::BF - 1) / big::BF * big::BF : g.N) * g.K;
  a.feat_packed = g.w_packed;
  a.y_ld = g.y_ld ? g.y_ld : g.N;
  a.y_estride = 0;
  a.E = g.E;
  a.N = g.N;
  a.K = g.K;
  a.M = 0;
  a.act = g.act;
  if (g.x_map) {
    // rows gathered from the token matrix: one 32-bit descriptor covers it
    if (g.x_ld && g.x_ld != g.K) return hipErrorInvalidValue;
    if (g.x_rows * g.K * 2 >= (int64_t(1) << 31)) return hipErrorNotSupported;
    a.tok_ld = g.K;
    a.tok_map = g.x_map;
    a.tok_rows = g.x_rows;
    return launch_big_act<BE_ACT, OP_GATHER, OP_KC, BM_ROWS>(a, s);
  }
  if (g.tile_rows == 320) return launch_big_act<BE_ACT, OP_KC, OP_KC, BM_ROWS, 5>(a, s);
  return launch_big_act<BE_ACT, OP_KC, OP_KC, BM_ROWS>(a, s);
}

}  // namespace

// Number of compute units of the current device (the persistent grid).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// The four GEMMs of the expert backward on the large-tile kernel (transposed
// operands read with ds_read_b64_tr_b16), or hipErrorNotSupported when the
// shapes do not fit it: both dims multiples of 64, every per-launch byte
// offset below 2^31.
hipError_t launch_backward_big(const GemmBwdArgs& g, hipStream_t s) {
  const int64_t d = g.d, h = g.h;
  if (d % 64 != 0 || h % 64 != 0) return hipErrorNotSupported;
  const int64_t lim = int64_t(1) << 31;
  if (d * h * 2 >= lim || (g.max_rows + 64) * std::max(d, h) * 2 >= lim || 256 * std::max(d, h) * 2 >= lim)
    return hipErrorNotSupported;
  if (g.max_rows <= 0) return hipSuccess;
  hipError_t e;
  const bf16* X = static_cast<const bf16*>(g.X);
  const bf16* dY = static_cast<const bf16*>(g.dY);
  bf16* dA = static_cast<bf16*>(g.dA);
  BigArgs a{};
  a.offset = g.offset;
  a.max_rows = g.max_rows;
  a.E = g.E;
  a.bias = nullptr;
  a.Apre = nullptr;

  // dA = (dY · W2[e]) ⊙ act'(A): token rows, K = d; W2[e] is [d, h] = [K, N]
  a.tok = dY; a.tok_ld = d;
  a.feat = static_cast<const bf16*>(g.W2); a.feat_ld = h; a.feat_estride = d * h;
  a.S = static_cast<const bf16*>(g.A);
  a.Y = dA; a.y_ld = h; a.y_estride = 0;
  a.N = (int)h; a.K = (int)d; a.M = 0; a.act = g.act;
  if ((e = launch_big_act<BE_DACT, OP_KC, OP_TR, BM_ROWS>(a, s)) != hipSuccess) return e;

  // dW2[e] = dY^T · H, [d, h]: K = the expert's rows (the last use of dY)
  a.tok = dY; a.tok_ld = d;
  a.feat = static_cast<const bf16*>(g.H); a.feat_ld = h; a.feat_estride = 0;
  a.S = nullptr;
  a.Y = static_cast<bf16*>(g.dW2); a.y_ld = h; a.y_estride = d * h;
  a.N = (int)h; a.M = (int)d; a.K = 0; a.act = ACT_NONE;
  if ((e = launch_big<BE_STORE, ACT_NONE, OP_TR, OP_TR, BM_WGRAD>(a, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(zero_empty_experts_kernel, dim3(64, g.E), dim3(256), 0, s, a.Y, g.offset, d * h);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // dX = dA · W1[e]: token rows, K = h; W1[e] is [h, d] = [K, N] (dX may overwrite dY)
  a.tok = dA; a.tok_ld = h;
  a.feat = static_cast<const bf16*>(g.W1); a.feat_ld = d; a.feat_estride = h * d;
  a.Y = static_cast<bf16*>(g.dX); a.y_ld = d; a.y_estride = 0;
  a.N = (int)d; a.K = (int)h; a.M = 0;
  if ((e = launch_big<BE_STORE, ACT_NONE, OP_KC, OP_TR, BM_ROWS>(a, s)) != hipSuccess) return e;

  // dW1[e] = dA^T · X, [h, d]
  a.tok = dA; a.tok_ld = h;
  a.feat = X; a.feat_ld = d; a.feat_estride = 0;
  a.Y = static_cast<bf16*>(g.dW1); a.y_ld = d; a.y_estride = h * d;
  a.N = (int)d; a.M = (int)h; a.K = 0;
  if ((e = launch_big<BE_STORE, ACT_NONE, OP_TR, OP_TR, BM_WGRAD>(a, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(zero_empty_experts_kernel, dim3(64, g.E), dim3(256), 0, s, a.Y, g.offset, h * d);
  return hipGetLastError();
}

// Chunked router weight gradient: part[c] = dl_hl[rows of chunk c]^T x[rows
// of chunk c], [2*Ep, d] fp32 per chunk, on the weight-gradient tiles with
// the chunks in the role of experts (choff holds their row offsets).
hipError_t launch_router_partials(const uint16_t* dl_hl, const void* x, const int32_t* choff, float* part,
                                  int64_t T, int S, int d, int Ep, hipStream_t s) {
  if (d % 64 != 0 || S < 1 || S > MOE_MAX_EXPERTS_DEV) return hipErrorNotSupported;
  BigArgs a{};
  a.tok = reinterpret_cast<const bf16*>(dl_hl);
  a.tok_ld = 2 * Ep;
  a.feat = static_cast<const bf16*>(x);
  a.feat_ld = d;
  a.feat_estride = 0;
  a.Yf = part;
  a.y_ld = d;
  a.y_estride = (int64_t)2 * Ep * d;
  a.offset = choff;
  a.max_rows = T;
  a.E = S;
  a.N = d;
  a.M = 2 * Ep;
  a.K = 0;
  a.act = ACT_NONE;
  return launch_big<BE_F32, ACT_NONE, OP_TR, OP_TR, BM_WGRAD>(a, s);
}

// The large-tile kernel needs whole 64-wide K steps, whole 16-feature output
// groups, and byte offsets of one operand tile below 2^31 (buffer offsets are
// 32-bit).
bool grouped_gemm_is_big(int64_t K, int64_t N, int dtype) {
  return dtype == DT_BF16 && K > 0 && K % 64 == 0 && N % 16 == 0 && (int64_t)256 * (K + 64) * 2 < (int64_t(1) << 31);
}

// Packed expert weight: one thread per 16-byte chunk of the packed tensor,
// [E][ceil(N/256)][K/64][256][64], reading row n = nf*256 + r of expert e
// (zeros past N).
__global__ __launch_bounds__(256) void pack_expert_weight_kernel(const uint4* __restrict__ w, uint4* __restrict__ wp,
                                                                 int64_t N, int64_t K, int64_t ntf, int64_t chunks) {
  const int64_t nk = K / 64;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < chunks; i += (int64_t)gridDim.x * 256) {
    const int64_t c8 = i & 7;             // 16-byte chunk within the 128-byte row of the block
    const int64_t r = (i >> 3) & 255;     // row within the block
    int64_t b = i >> 11;                  // block: ((e * ntf + nf) * nk + ks)
    const int64_t ks = b % nk;
    b /= nk;
    const int64_t nf = b % ntf;
    const int64_t e = b / ntf;
    const int64_t n = nf * 256 + r;
    wp[i] = n < N ? w[((e * N + n) * K + ks * 64) / 8 + c8] : make_uint4(0u, 0u, 0u, 0u);
  }
}

hipError_t launch_pack_expert_weight(const void* w, void* wp, int E, int64_t N, int64_t K, hipStream_t s) {
  const int64_t ntf = (N + 255) / 256;
  const int64_t chunks = (int64_t)E * ntf * 256 * K / 8;
  if (chunks <= 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>((chunks + 255) / 256, 8192);
  hipLaunchKernelGGL(pack_expert_weight_kernel, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const uint4*>(w),
                     static_cast<uint4*>(wp), N, K, ntf, chunks);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmArgs& a, int dtype, hipStream_t s) {
  if (a.max_rows <= 0) return hipSuccess;
  if ((a.w_packed || a.x_map) && !grouped_gemm_is_big(a.K, a.N, dtype)) return hipErrorNotSupported;
  const bool pitched = (a.x_ld && a.x_ld != a.K) || (a.y_ld && a.y_ld != a.N);
  if (pitched && (a.x_ld && a.x_ld < a.K || a.y_ld && a.y_ld < a.N || a.x_ld > a.K + 64)) return hipErrorInvalidValue;
  if (grouped_gemm_is_big(a.K, a.N, dtype)) return launch_bf16_big(a, s);
  if (pitched) return hipErrorNotSupported;
  if (dtype == DT_BF16) return launch_bf16<128, 128, 2, 2>(a, s);
  dim3 grid((a.N + 63) / 64, (unsigned)((a.max_rows + 3) / 4));
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
