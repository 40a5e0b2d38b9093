// Host-only checks of the launch planning and argument validation shared with the kernels.
// Built with g++ and sanitizers by tests/test_abi.py; prints "OK" and exits 0 when every check holds.
#include <cstdio>
#include <set>
#include <vector>

#include "validate.hpp"

using namespace attn;

static int failures = 0;
#define EXPECT(cond, ...)                       \
  do {                                          \
    if (!(cond)) {                              \
      if (failures < 20) {                      \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
        std::printf(__VA_ARGS__);               \
        std::printf("\n");                      \
      }                                         \
      ++failures;                               \
    }                                           \
  } while (0)

// Keys a query may see, by enumerating the window offsets (independent of na_axis_ok).
static std::set<int> window_keys(const NaGeom& g, int q) {
  const int y = q / g.grid_w, x = q % g.grid_w;
  std::vector<int> rows, cols;
  if (g.wrap_h) {
    for (int d = -g.rad_h; d <= g.rad_h; ++d) rows.push_back(((y + d) % g.grid_h + g.grid_h) % g.grid_h);
  } else {
    int s = y - g.rad_h;
    s = s < 0 ? 0 : (s > g.grid_h - g.kernel_h ? g.grid_h - g.kernel_h : s);
    for (int i = 0; i < g.kernel_h; ++i) rows.push_back(s + i);
  }
  if (g.wrap_w) {
    for (int d = -g.rad_w; d <= g.rad_w; ++d) cols.push_back(((x + d) % g.grid_w + g.grid_w) % g.grid_w);
  } else {
    int s = x - g.rad_w;
    s = s < 0 ? 0 : (s > g.grid_w - g.kernel_w ? g.grid_w - g.kernel_w : s);
    for (int i = 0; i < g.kernel_w; ++i) cols.push_back(s + i);
  }
  std::set<int> keys;
  for (int r : rows)
    for (int c : cols) keys.insert(r * g.grid_w + c);
  return keys;
}

static void check_na(int gh, int gw, int kh, int kw, int wh, int ww, int BM, int BN) {
  const NaGeom g{gh, gw, kh, kw, kh / 2, kw / 2, wh, ww};
  const int N = gh * gw;
  const int n_tiles = (int)cdiv(N, BN);
  for (int q0 = 0; q0 < N; q0 += BM) {
    const KvRun run = kv_run(MASK_NA2D, N, BM, BN, q0, g);
    EXPECT(run.first >= 0 && run.first < n_tiles && run.count >= 1 && run.count <= n_tiles,
           "run out of range grid %dx%d k%dx%d wrap%d%d q0 %d", gh, gw, kh, kw, wh, ww, q0);
    std::set<int> visited;
    for (int i = 0; i < run.count; ++i) {
      const int t = kv_tile_at(run, i, n_tiles);
      EXPECT(t >= 0 && t < n_tiles, "tile index %d out of range", t);
      EXPECT(visited.insert(t).second, "tile %d visited twice (grid %dx%d k%dx%d q0 %d)", t, gh, gw, kh, kw, q0);
    }
    for (int q = q0; q < N && q < q0 + BM; ++q) {
      const std::set<int> want = window_keys(g, q);
      EXPECT((int)want.size() == kh * kw, "window size");
      const int yq = q / gw, xq = q % gw;
      for (int key = 0; key < N; ++key) {
        const bool ok = na_axis_ok(yq, key / gw, gh, kh, g.rad_h, wh) && na_axis_ok(xq, key % gw, gw, kw, g.rad_w, ww);
        EXPECT(ok == (want.count(key) == 1), "predicate vs window, grid %dx%d k%dx%d wrap%d%d q %d key %d", gh, gw,
               kh, kw, wh, ww, q, key);
        if (ok) EXPECT(visited.count(key / BN) == 1, "allowed key %d of query %d in a skipped tile", key, q);
      }
    }
  }
}

static void check_causal(int N, int BM, int BN) {
  const int n_tiles = (int)cdiv(N, BN);
  for (int q0 = 0; q0 < N; q0 += BM) {
    const KvRun run = kv_run(MASK_CAUSAL, N, BM, BN, q0, NaGeom{});
    const int q_last = (q0 + BM < N ? q0 + BM : N) - 1;
    EXPECT(run.first == 0 && run.count == q_last / BN + 1 && run.count <= n_tiles, "causal run N %d q0 %d", N, q0);
    for (int i = 0; i < run.count; ++i) {
      const int t = kv_tile_at(run, i, n_tiles);
      // a tile needs no element mask only if every key is <= every query of the tile and < N
      if (!tile_needs_mask(MASK_CAUSAL, N, BN, q0, t)) EXPECT((t + 1) * BN - 1 <= q0 && (t + 1) * BN <= N, "mask flag");
    }
  }
}

static void check_work_items(int mask, int BH, int n_qtiles) {
  const int n_wg = BH * n_qtiles;
  std::vector<int> seen(n_wg, 0);
  for (int wg = 0; wg < n_wg; ++wg) {
    const WorkItem w = work_item(mask, wg, n_wg, n_qtiles, BH);
    EXPECT(w.bh >= 0 && w.bh < BH && w.qtile >= 0 && w.qtile < n_qtiles, "work item out of range");
    if (w.bh >= 0 && w.bh < BH && w.qtile >= 0 && w.qtile < n_qtiles) seen[w.bh * n_qtiles + w.qtile]++;
  }
  for (int i = 0; i < n_wg; ++i) EXPECT(seen[i] == 1, "work item %d covered %d times", i, seen[i]);
}

// The remainder split: whole tiles and parts cover every (tile, key tile) once;
// parts of one tile are contiguous, non-empty key ranges in order; slots are
// distinct; every CU gets about the same amount of work.
static void check_split(int64_t n_tiles, int32_t n_kv, int32_t cus) {
  const SplitPlan p = split_plan(MASK_NONE, n_tiles, n_kv, cus);
  EXPECT(split_plan(MASK_CAUSAL, n_tiles, n_kv, cus).rem == 0, "causal never splits");
  EXPECT(split_plan(MASK_NA2D, n_tiles, n_kv, cus).rem == 0, "2D neighbourhood never splits");
  if (p.rem == 0) return;
  EXPECT(n_tiles < 2 * (int64_t)cus, "split only below two tiles per CU");
  EXPECT(p.full == 0 || p.full == cus, "whole tiles fill one round of CUs");
  EXPECT(p.full + p.rem == n_tiles, "every tile is whole or split");
  EXPECT(p.parts >= 2 && p.parts <= kMaxParts && p.parts * kMinPartTiles <= n_kv, "parts %d of %d key tiles",
         p.parts, n_kv);
  EXPECT((int64_t)p.rem * p.parts <= cus, "parts fit one round of CUs");
  std::vector<int> seen((size_t)n_tiles * n_kv, 0);
  for (int32_t g = 0; g < p.groups(); ++g) {
    if (g < p.full) {
      const int32_t tile = xcd_contiguous(g, p.full);
      EXPECT(tile >= 0 && tile < p.full, "whole tile %d out of range", tile);
      for (int32_t t = 0; t < n_kv; ++t) seen[(size_t)tile * n_kv + t]++;
    } else {
      const int32_t slot = g - p.full;
      const int32_t tile = p.full + slot / p.parts;
      const KvRun r = part_run(n_kv, p.parts, slot % p.parts);
      EXPECT(slot < p.slots(), "slot out of range");
      EXPECT(tile < n_tiles && r.count >= kMinPartTiles - 1 && r.count >= 1 && r.first + r.count <= n_kv,
             "part out of its tile");
      if (slot % p.parts > 0) {
        const KvRun prev = part_run(n_kv, p.parts, slot % p.parts - 1);
        EXPECT(prev.first + prev.count == r.first, "parts not contiguous");
      }
      for (int32_t t = r.first; t < r.first + r.count; ++t) seen[(size_t)tile * n_kv + t]++;
    }
  }
  for (int v : seen) EXPECT(v == 1, "unit done %d times", v);
}

// The column bits of the block-masked neighbourhood kernel agree with the element predicate.
static void check_col_bits() {
  for (int W : {32, 64, 96, 128})
    for (int kw = 1; kw <= W; kw += 2)
      for (int wrap = 0; wrap < 2; ++wrap)
        for (int cq = 0; cq < W; ++cq)
          for (int half = 0; half < 2; ++half) {
            uint32_t bits[2] = {7u, 7u};
            na_col_bits(cq, half, W, kw, kw / 2, wrap, W / 32, bits);
            for (int ph = 0; ph < 4; ++ph)
              for (int r = 0; r < 16; ++r) {
                const int xk = ph * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                const bool want = ph < W / 32 && na_axis_ok(cq, xk, W, kw, kw / 2, wrap);
                const bool got = (bits[ph >> 1] >> ((ph & 1) * 16 + r)) & 1u;
                EXPECT(got == want, "col bits W %d kw %d wrap %d cq %d half %d ph %d r %d", W, kw, wrap, cq, half, ph, r);
              }
          }
}

static void check_limit_bits() {
  for (int lim = -40; lim <= 40; ++lim) {
    uint32_t want = 0;
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) <= lim) want |= 1u << r;
    EXPECT(limit_bits(lim) == want, "limit_bits(%d) = %x, want %x", lim, limit_bits(lim), want);
  }
}

static void check_validation() {
  attn_na2d_params_t p{64, 64, 7, 7, 1, 1, 1, 1};
  EXPECT(check_problem(2, 5, 4096, 64, 0.125f, ATTN_MASK_NONE, nullptr) == ATTN_OK, "valid none");
  EXPECT(check_problem(2, 4, 4096, 32, 0.17f, ATTN_MASK_NA2D, &p) == ATTN_OK, "valid na2d");
  EXPECT(check_problem(0, 5, 4096, 64, 0.125f, 0, nullptr) == ATTN_ERR_INVALID_ARG, "B=0");
  EXPECT(check_problem(2, -1, 4096, 64, 0.125f, 0, nullptr) == ATTN_ERR_INVALID_ARG, "H<0");
  EXPECT(check_problem(2, 5, 0, 64, 0.125f, 0, nullptr) == ATTN_ERR_INVALID_ARG, "N=0");
  EXPECT(check_problem(2, 5, 64, 128, 0.125f, 0, nullptr) == ATTN_ERR_UNSUPPORTED, "d=128");
  EXPECT(check_problem(2, 5, 64, 64, 1.0f / 0.0f, 0, nullptr) == ATTN_ERR_INVALID_ARG, "inf scale");
  EXPECT(check_problem(2, 5, 64, 64, 0.1f, 3, nullptr) == ATTN_ERR_INVALID_ARG, "mode 3");
  EXPECT(check_problem(2, 5, 64, 64, 0.1f, ATTN_MASK_CAUSAL, &p) == ATTN_ERR_INVALID_ARG, "params with causal");
  EXPECT(check_problem(2, 5, 64, 64, 0.1f, ATTN_MASK_NA2D, nullptr) == ATTN_ERR_INVALID_ARG, "na2d no params");
  EXPECT(check_problem(1, 1, (int64_t)1 << 31, 64, 0.1f, 0, nullptr) == ATTN_ERR_UNSUPPORTED, "N too large");
  EXPECT(check_problem((int64_t)1 << 20, (int64_t)1 << 20, 4096, 64, 0.1f, 0, nullptr) == ATTN_ERR_UNSUPPORTED,
         "too many work-groups");
  attn_na2d_params_t bad = p;
  bad.grid_h = 63;
  EXPECT(check_problem(1, 1, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_ERR_PARAMS, "grid mismatch");
  bad = p; bad.kernel_h = 6;
  EXPECT(check_problem(1, 1, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_ERR_PARAMS, "even kernel");
  bad = p; bad.kernel_w = 65;
  EXPECT(check_problem(1, 1, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_ERR_PARAMS, "kernel > grid");
  bad = p; bad.wrap_w = 2;
  EXPECT(check_problem(1, 1, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_ERR_PARAMS, "wrap 2");
  bad = p; bad.dil_h = 2;
  EXPECT(check_problem(1, 1, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_ERR_PARAMS, "dilation");
  char buf[256];
  const void* a = buf + 16;
  EXPECT(check_pointers(a, buf + 32, buf + 48, buf + 64, 1, 1, 1, 8) == ATTN_OK, "disjoint aligned");
  EXPECT(check_pointers(a, buf + 32, buf + 48, buf + 72, 1, 1, 1, 8) == ATTN_ERR_ALIGNMENT, "misaligned o");
  EXPECT(check_pointers(a, buf + 32, buf + 48, buf + 48, 1, 1, 1, 8) == ATTN_ERR_INVALID_ARG, "o aliases v");
  EXPECT(check_pointers(nullptr, buf + 32, buf + 48, buf + 64, 1, 1, 1, 8) == ATTN_ERR_INVALID_ARG, "null q");
}

int main() {
  check_validation();
  check_col_bits();
  check_limit_bits();
  for (int BN : {64, 128}) {
    for (int N : {1, 2, 63, 64, 65, 127, 128, 129, 200, 255, 256, 257, 600}) check_causal(N, kBlockM, BN);
    const int dims[] = {1, 2, 3, 5, 7, 9, 12, 17};
    for (int gh : dims)
      for (int gw : dims)
        for (int kh = 1; kh <= gh; kh += 2)
          for (int kw = 1; kw <= gw; kw += 4)
            for (int wh = 0; wh < 2; ++wh)
              for (int ww = 0; ww < 2; ++ww) check_na(gh, gw, kh, kw, wh, ww, kBlockM, BN);
    check_na(64, 64, 7, 7, 1, 1, kBlockM, BN);
    check_na(64, 64, 7, 7, 0, 0, kBlockM, BN);
    check_na(33, 17, 9, 3, 1, 1, kBlockM, BN);
    check_na(3, 200, 3, 11, 1, 1, kBlockM, BN);
    check_na(96, 40, 5, 5, 1, 0, kBlockM, BN);
  }
  for (int mask : {MASK_NONE, MASK_CAUSAL})
    for (int BH : {1, 3, 8, 10, 64})
      for (int nq : {1, 2, 7, 32, 72}) check_work_items(mask, BH, nq);
  // split plans: the sizes of the unmasked workloads and small or odd shapes
  EXPECT(split_plan(MASK_NONE, 320, 32, 256).rem == 64 && split_plan(MASK_NONE, 320, 32, 256).parts == 4,
         "B2 H5 N4096: 256 whole tiles, 64 tiles in 4 parts");
  EXPECT(split_plan(MASK_NONE, 720, 72, 256).rem == 0, "B2 H5 N9216 is over two rounds deep: no split");
  EXPECT(split_plan(MASK_NONE, 512, 32, 256).rem == 0, "two full rounds need no split");
  EXPECT(split_plan(MASK_NONE, 256, 32, 256).rem == 0, "one full round needs no split");
  EXPECT(split_plan(MASK_NONE, 2, 2, 256).rem == 0, "tiny problems do not split");
  for (int32_t cus : {1, 2, 7, 64, 80, 256, 304})
    for (int64_t n_tiles : {1, 2, 3, 5, 16, 21, 33, 40, 48, 72, 80, 100, 255, 256, 257, 320, 400, 511, 512, 513})
      for (int32_t n_kv : {1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 32, 33, 72}) check_split(n_tiles, n_kv, cus);
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("OK\n");
  return 0;
}
