// Host-side check of the C ABI's host layer, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_abi_sanitized.py):
// the host-only calls over a grid of configurations, with the invariants of
// the workspace layout they report, and the argument checks of the device
// calls on inputs they must reject before anything is enqueued.  A sanitizer
// finding aborts the program; an invariant failure prints it and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "moe.h"

static int failures = 0;

#define CHECK(cond, ...)                    \
  do {                                      \
    if (!(cond)) {                          \
      fprintf(stderr, "FAIL %s: ", #cond);  \
      fprintf(stderr, __VA_ARGS__);         \
      fprintf(stderr, "\n");                \
      ++failures;                           \
    }                                       \
  } while (0)

static moe_config make(int64_t T, int d, int E, int k, double cf, int minc, int drop, int h, int act, int dt) {
  moe_config c = {};
  c.num_tokens = T;
  c.capacity_factor = cf;
  c.hidden_size = d;
  c.num_experts = E;
  c.k = k;
  c.min_capacity = minc;
  c.drop_tokens = drop;
  c.ffn_hidden = h;
  c.activation = act;
  c.dtype = dt;
  return c;
}

// Every region the views report lies inside [base, base + size) and the
// packed buffers do not overlap.
static void check_layout(const moe_config& c) {
  size_t ws = 0;
  if (moe_workspace_size(&c, &ws) != MOE_OK) return;
  int64_t rows = -1, C = -2, hld = -1;
  CHECK(moe_max_rows(&c, &rows) == MOE_OK, "max_rows");
  CHECK(moe_capacity(&c, &C) == MOE_OK, "capacity");
  CHECK(moe_workspace_h_ld(&c, &hld) == MOE_OK, "h_ld");
  CHECK(rows >= 0 && rows <= (int64_t)c.k * c.num_tokens, "rows %lld", (long long)rows);
  if (c.drop_tokens) {
    CHECK(C >= c.min_capacity, "C %lld", (long long)C);
    CHECK(rows <= C * c.num_experts || rows == (int64_t)c.k * c.num_tokens, "rows vs capacity");
  } else {
    CHECK(C == -1, "no capacity gives -1");
  }
  const size_t s = c.dtype == MOE_BF16 ? 2 : 4;
  const uintptr_t base = (uintptr_t)1 << 40;
  void* ptrs[4] = {nullptr, nullptr, nullptr, nullptr};
  int32_t* off = nullptr;
  CHECK(moe_workspace_views(&c, (void*)base, &ptrs[0], &ptrs[1], &ptrs[2], &ptrs[3], &off) == MOE_OK, "views");
  const size_t h = (size_t)c.ffn_hidden;
  const size_t sizes[4] = {(size_t)rows * c.hidden_size * s, c.save_preact && h ? (size_t)rows * h * s : 0,
                           h ? (size_t)rows * (size_t)hld * s : 0, (size_t)rows * c.hidden_size * s};
  for (int i = 0; i < 4; ++i) {
    if (!ptrs[i]) continue;
    const uintptr_t p = (uintptr_t)ptrs[i];
    CHECK(p >= base && p + sizes[i] <= base + ws, "region %d outside the workspace", i);
    CHECK(p % 256 == 0, "region %d alignment", i);
    for (int j = 0; j < i; ++j) {
      if (!ptrs[j]) continue;
      const uintptr_t q = (uintptr_t)ptrs[j];
      CHECK(p + sizes[i] <= q || q + sizes[j] <= p, "regions %d and %d overlap", i, j);
    }
  }
  CHECK((uintptr_t)off >= base && (uintptr_t)off + 4 * (c.num_experts + 1) <= base + ws, "offsets");
  uint32_t* st = nullptr;
  CHECK(moe_workspace_status(&c, (void*)base, &st) == MOE_OK, "status");
  if (c.num_tokens <= MOE_SMALL_BATCH_MAX)
    CHECK(st && (uintptr_t)st >= base && (uintptr_t)st + 4 <= base + ws, "status word");
  else
    CHECK(st == nullptr, "no status word past the small-batch limit");
}

int main() {
  const int64_t Ts[] = {0, 1, 63, 64, 65, 256, 257, 1000, 16384, 65536};
  const int ds[] = {8, 96, 512, 2048};
  const int Es[] = {1, 3, 8, 64, 65, 128, 256};
  const int hs[] = {0, 176, 1536};
  const double cfs[] = {0.5, 1.0, 1.1, 2.0};
  long n = 0;
  for (int64_t T : Ts)
    for (int d : ds)
      for (int E : Es)
        for (int k = 1; k <= 2 && k <= E; ++k)
          for (int h : hs)
            for (double cf : cfs)
              for (int drop = 0; drop < 2; ++drop)
                for (int dt = 0; dt < 2; ++dt)
                  for (int sp = 0; sp < 2; ++sp) {
                    moe_config c = make(T, d, E, k, cf, 4, drop, h, h ? MOE_ACT_GELU : MOE_ACT_NONE, dt);
                    c.save_preact = sp;
                    c.use_residual = (T % 2 == 1) && dt == MOE_BF16;
                    check_layout(c);
                    ++n;
                  }
  // configurations the checks must reject
  moe_config bad[] = {
      make(-1, 64, 8, 2, 1.0, 4, 1, 0, 0, 1),        // negative T
      make(64, 0, 8, 2, 1.0, 4, 1, 0, 0, 1),         // d = 0
      make(64, 64, 0, 1, 1.0, 4, 1, 0, 0, 1),        // no experts
      make(64, 64, 257, 2, 1.0, 4, 1, 0, 0, 1),      // too many experts
      make(64, 64, 8, 3, 1.0, 4, 1, 0, 0, 1),        // k = 3
      make(64, 64, 1, 2, 1.0, 4, 1, 0, 0, 1),        // k > E
      make(64, 64, 8, 2, 0.0, 4, 1, 0, 0, 1),        // capacity factor 0 with drops
      make(64, 64, 8, 2, 1.0, -1, 1, 0, 0, 1),       // negative min_capacity
      make(64, 64, 8, 2, 1.0, 4, 2, 0, 0, 1),        // drop_tokens = 2
      make(64, 64, 8, 2, 1.0, 4, 1, -8, 0, 1),       // negative h
      make(64, 64, 8, 2, 1.0, 4, 1, 0, 7, 1),        // unknown activation
      make(64, 64, 8, 2, 1.0, 4, 1, 0, 0, 5),        // unknown dtype
  };
  for (const moe_config& c : bad) {
    int64_t v;
    size_t b;
    CHECK(moe_capacity(&c, &v) == MOE_ERR_INVALID_ARG, "capacity of a bad config");
    CHECK(moe_workspace_size(&c, &b) == MOE_ERR_INVALID_ARG, "workspace size of a bad config");
  }
  CHECK(moe_capacity(nullptr, nullptr) == MOE_ERR_INVALID_ARG, "null config");
  // device calls whose arguments are rejected before any launch
  moe_config c = make(1000, 512, 8, 2, 1.0, 4, 1, 1024, MOE_ACT_GELU, MOE_BF16);
  void* fake = (void*)((uintptr_t)1 << 40);
  CHECK(moe_gate(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                 nullptr, 0, nullptr) == MOE_ERR_INVALID_ARG, "gate without inputs");
  CHECK(moe_layer_forward(&c, fake, fake, nullptr, nullptr, fake, nullptr, fake, nullptr, fake, (float*)fake,
                          (int32_t*)fake, nullptr, nullptr, nullptr, nullptr, fake, 16, nullptr) == MOE_ERR_WORKSPACE,
        "layer forward with a small workspace");
  CHECK(moe_gate_noalloc(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         nullptr, nullptr, nullptr) == MOE_ERR_INVALID_ARG, "no-allocation gate without inputs");
  moe_config big = make(1 << 20, 512, 256, 2, 1.0, 4, 1, 0, 0, MOE_BF16);
  CHECK(moe_gate_noalloc(&big, fake, fake, nullptr, nullptr, nullptr, (int32_t*)fake, (int32_t*)fake, (float*)fake,
                         (int32_t*)fake, (int32_t*)fake, (float*)fake, nullptr) == MOE_ERR_WORKSPACE,
        "no-allocation gate past its scratch");
  for (int st = 0; st < 6; ++st) CHECK(moe_status_string((moe_status)st) != nullptr, "status string");
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("OK %ld configurations\n", n);
  return 0;
}
