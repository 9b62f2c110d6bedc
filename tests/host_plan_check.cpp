// CPU checks of the launch planner (csrc/cf_plan.h), built by
// tests/test_host_planner.py with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer. A fake device is a (workgroups per CU, CUs)
// pair; no HIP header or call is involved.
//
// Checked for every problem and device of a sweep:
//  * the grid never exceeds the resident capacity (per_cu * cus), and a strip
//    wider than that capacity is refused when its row op needs an exchange;
//  * the persistent loop (rounds of `grid` tiles from tile 0, each workgroup
//    taking round_tile(...) and stopping at the first tile past the end)
//    visits every tile exactly once;
//  * with an exchange, every round is a whole number of strips, so all tiles
//    of a strip are processed in the same round (co-resident workgroups);
//  * in a full round with XCD rectangles, the tiles of the workgroups on one
//    XCD (workgroup w on XCD w % 8) form one xcd_a x xcd_b rectangle of
//    (strip, column) tiles;
//  * the workspace covers every slot the kernel addresses;
// and check_gemm / check_epilogue on descriptors with random fields run
// without undefined behaviour and refuse what they must.
#define CF_HD
#include "cf_plan.h"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <set>
#include <vector>

static int g_fail = 0;
#define CHECK(c, ...)                                   \
  do {                                                  \
    if (!(c)) {                                         \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                \
      std::fprintf(stderr, "\n");                       \
      if (++g_fail > 20) std::exit(1);                  \
    }                                                   \
  } while (0)

// Stores a raw int in an enum field, as a C caller may (any value, not only
// an enumerator).
template <class E>
static void setv(E& f, int64_t v) {
  const int x = (int)v;
  std::memcpy(&f, &x, sizeof x);
}

static cf_epilogue make_epi(cf_row_op op) {
  cf_epilogue e;
  std::memset(&e, 0, sizeof(e));
  e.struct_size = sizeof(cf_epilogue);
  e.alpha = 1.0f;
  e.residual_dtype = CF_BF16;
  e.vec_dtype = CF_BF16;
  e.row_op = op;
  return e;
}

static void check_plan(int64_t M, int64_t N, cf_row_op op, int64_t per_cu, int64_t cus, bool col = false) {
  cf_epilogue e = make_epi(op);
  setv(e.axis, col ? CF_AXIS_COLUMN : CF_AXIS_ROW);
  const cf::GemmPlan g = cf::plan_gemm(M, N, &e);
  CHECK(g.group == (col ? g.strips : g.tiles_n), "group width");
  cf::GridPlan gp;
  const cf_status st = cf::plan_grid(g, per_cu, cus, &gp);
  const int64_t cap = per_cu * cus;
  if (g.exchange && g.group > cap) {
    CHECK(st == CF_ERR_UNSUPPORTED, "M=%lld N=%lld cap=%lld: strip wider than capacity not refused",
          (long long)M, (long long)N, (long long)cap);
    return;
  }
  CHECK(st == CF_OK, "plan_grid refused M=%lld N=%lld", (long long)M, (long long)N);
  if (st != CF_OK) return;
  CHECK(gp.grid >= 1 && gp.grid <= cap && gp.grid <= g.tiles, "grid %lld outside [1, min(cap %lld, tiles %lld)]",
        (long long)gp.grid, (long long)cap, (long long)g.tiles);
  if (g.exchange) CHECK(gp.grid % g.group == 0, "grid %lld not whole groups of %lld", (long long)gp.grid, (long long)g.group);
  // the persistent loop
  std::vector<int> seen((size_t)g.tiles, 0);
  const int grid = (int)gp.grid, tiles = (int)g.tiles, tn = (int)g.group;
  for (int base = 0; base < tiles; base += grid) {
    std::vector<std::set<int64_t>> xs(8), ys(8);
    std::vector<int> xcount(8, 0);
    for (int bid = 0; bid < grid; ++bid) {
      const int t = cf::round_tile(base, bid, grid, tiles, tn, gp.xcd_a, gp.xcd_b);
      if (t >= tiles) continue;
      CHECK(t >= 0, "negative tile");
      if (t < 0) continue;
      ++seen[(size_t)t];
      CHECK(t >= base && t < base + grid, "tile %d outside its round [%d, %d)", t, base, base + grid);
      if (g.exchange) {
        // the exchange group of t (a row strip, or a tile column) lies
        // entirely inside this round
        const int s0 = (t / tn) * tn;
        CHECK(s0 >= base && s0 + tn <= base + grid, "group of tile %d split across rounds", t);
      }
      xs[bid & 7].insert(t / tn);
      ys[bid & 7].insert(t % tn);
      ++xcount[bid & 7];
    }
    if (gp.xcd_a > 0 && base + grid <= tiles) {
      for (int x = 0; x < 8; ++x) {
        CHECK((int64_t)xs[x].size() == gp.xcd_a && (int64_t)ys[x].size() == gp.xcd_b &&
                  xcount[x] == gp.xcd_a * gp.xcd_b,
              "XCD %d of round %d: %zu strips x %zu columns for %d tiles, want %d x %d", x, base, xs[x].size(),
              ys[x].size(), xcount[x], gp.xcd_a, gp.xcd_b);
        // contiguous rectangle
        if (!xs[x].empty())
          CHECK(*xs[x].rbegin() - *xs[x].begin() + 1 == (int64_t)xs[x].size() &&
                    *ys[x].rbegin() - *ys[x].begin() + 1 == (int64_t)ys[x].size(),
                "XCD %d: tiles not a contiguous rectangle", x);
      }
    }
  }
  for (int t = 0; t < tiles; ++t) CHECK(seen[(size_t)t] == 1, "tile %d visited %d times", t, seen[(size_t)t]);
  // workspace: the kernel's slot addressing (512 words per tile and stage,
  // 16 * 256 for top-k) stays inside the planned bytes
  if (g.exchange) {
    const size_t words = op == CF_ROW_TOPK ? 16 * 256 : 512;
    const size_t need = cf::kWsHeaderBytes + (size_t)g.tiles * words * 8;
    CHECK(g.ws_bytes >= need, "workspace %zu < %zu", g.ws_bytes, need);
    CHECK(g.ws_bytes % 256 == 0 || (g.ws_bytes - cf::kWsHeaderBytes) % 256 == 0, "slot area not 256-aligned");
  }
}

static void fuzz_checks(unsigned seed, int n) {
  std::mt19937_64 rng(seed);
  auto pick = [&](std::initializer_list<int64_t> v) { return *(v.begin() + rng() % v.size()); };
  const uintptr_t base = 0x7f0000000000ull;
  for (int i = 0; i < n; ++i) {
    cf_epilogue e = make_epi(CF_ROW_NONE);
    setv(e.row_op, pick({0, 1, 2, 3, 4, 5, 6, -1}));
    e.struct_size = (uint32_t)pick({(int64_t)sizeof(cf_epilogue), 8, 0});
    e.alpha = (float)pick({1, 0, -3}) * ((rng() % 17) ? 1.0f : NAN);
    e.eps = (rng() % 13) ? 1e-5f : -1.0f;
    setv(e.act, pick({0, 1, 7}));
    e.bias = (rng() & 1) ? (const void*)(base + pick({0, 1, 2, 16})) : nullptr;
    e.residual = (rng() % 3 == 0) ? (const void*)(base + pick({0, 2, 16})) : nullptr;
    e.ld_residual = pick({0, 64, 4096, 1 << 20});
    setv(e.residual_dtype, pick({0, 1, 5}));
    setv(e.vec_dtype, pick({0, 1, 9}));
    e.gamma = (rng() & 1) ? (const void*)(base + 32) : nullptr;
    e.beta = (rng() % 3 == 0) ? (const void*)(base + 64) : nullptr;
    e.x_out = (rng() % 5 == 0) ? (void*)(base + pick({0, 2, 16})) : nullptr;
    e.ld_x_out = pick({0, 64, 4096});
    setv(e.x_out_dtype, pick({0, 1, 3}));
    setv(e.mask, pick({0, 0, 1, 4}));
    e.row_stats = (rng() % 4 == 0) ? (float*)(base + pick({0, 2})) : nullptr;
    e.row_index = (rng() % 3 == 0) ? (int32_t*)(base + pick({0, 2})) : nullptr;
    setv(e.row_op2, pick({0, 0, 1, 2, 3, 4, 9}));
    setv(e.axis, pick({0, 0, 1, 5}));
    e.eps2 = (rng() & 1) ? 0.0f : 1e-6f;
    e.topk = (int32_t)pick({0, 1, 4, 8, 9});
    const int64_t M = pick({0, 1, 255, 256, 8192, -1, 1ll << 31});
    const int64_t N = pick({0, 8, 250, 4096, 70000});
    const int64_t K = pick({0, 32, 100, 4096, 11008});
    const int64_t lda = K + pick({0, 8, -1});
    const int64_t ldb = (rng() & 1 ? N : K) + pick({0, 8});
    const int64_t ldc = N + pick({0, 8, -1});
    const void* A = (rng() % 11) ? (const void*)(base + pick({0, 16, 2})) : nullptr;
    const void* B = (const void*)(base + (1 << 20));
    void* C = (rng() % 7) ? (void*)(base + (2 << 20)) : nullptr;
    const void* ws = (rng() & 1) ? (const void*)(base + (3 << 20) + pick({0, 16})) : nullptr;
    cf::GemmChecked out;
    const cf_status st = cf::check_gemm(M, N, K, A, lda, B, ldb, (int)pick({0, 1, 2}), (int)pick({0, 1, 2}),
                                        C, ldc, (int)pick({0, 1}), (rng() % 9) ? &e : nullptr, ws,
                                        (size_t)pick({0, 4096, 1 << 24, 1ll << 30}), (rng() & 1) != 0, &out);
    CHECK(st >= CF_OK && st <= CF_ERR_DEVICE_TIMEOUT, "status %d out of range", (int)st);
    if (st == CF_OK && !out.empty) {
      CHECK(M > 0 && N > 0, "accepted an empty or negative shape");
      if (out.plan.col) CHECK(out.vec && out.row_op >= CF_ROW_SOFTMAX && out.row_op <= CF_ROW_RMSNORM,
                              "column reduction accepted outside its fast-path row ops");
      CHECK(out.plan.tiles == ((M + 255) / 256) * ((N + 255) / 256), "tile count");
    }
  }
}

int main() {
  const int64_t Ms[] = {1, 255, 256, 300, 2048, 8192, 16384, 65536};
  const int64_t Ns[] = {8, 256, 257, 768, 1000, 4096, 8192, 16384, 65536};
  const int64_t devs[][2] = {{1, 256}, {2, 256}, {1, 304}, {1, 80}, {1, 8}, {1, 1}, {2, 7}};
  const cf_row_op ops[] = {CF_ROW_NONE, CF_ROW_LAYERNORM, CF_ROW_TOPK};
  int n = 0;
  for (int64_t M : Ms)
    for (int64_t N : Ns)
      for (const auto& d : devs) {
        for (cf_row_op op : ops) {
          check_plan(M, N, op, d[0], d[1]);
          ++n;
        }
        check_plan(M, N, CF_ROW_SOFTMAX, d[0], d[1], true);   // column reduction: tile-column groups
        ++n;
      }
  fuzz_checks(1234, 200000);
  if (g_fail) {
    std::fprintf(stderr, "%d failures\n", g_fail);
    return 1;
  }
  std::printf("planner ok: %d problems x devices, 200000 fuzzed argument sets\n", n);
  return 0;
}
