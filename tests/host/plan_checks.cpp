// Host-only checks of the launch planning and argument validation shared with the kernels.
// Built with g++ and sanitizers by tests/test_abi.py; prints "OK" and exits 0 when every check holds.
#include <algorithm>
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

// Window cells of coordinate c along one axis, enumerated (independent of
// na_axis_ok and na_dil_ok): wrapped, c + dil * t mod len for |t| <= r; clamped,
// the list of cells congruent to c mod dil with a kernel-long window slid inside it.
static std::vector<int> axis_cells(int c, int len, int kernel, int wrap, int dil) {
  std::vector<int> out;
  const int r = kernel / 2;
  if (wrap) {
    for (int t = -r; t <= r; ++t) out.push_back(((c + dil * t) % len + len) % len);
    return out;
  }
  std::vector<int> sub;
  for (int x = c % dil; x < len; x += dil) sub.push_back(x);
  int i = 0;
  while (sub[i] != c) ++i;
  int s = i - r;
  s = s < 0 ? 0 : (s > (int)sub.size() - kernel ? (int)sub.size() - kernel : s);
  for (int t = 0; t < kernel; ++t) out.push_back(sub[s + t]);
  return out;
}

static NaGeom geom(int gd, int gh, int gw, int kd, int kh, int kw, int wd, int wh, int ww, int dd, int dh, int dw) {
  return NaGeom{gh, gw, kh, kw, kh / 2, kw / 2, wh, ww, dh, dw, gd, kd, kd / 2, wd, dd};
}

// Keys a query may see, by enumerating the window cells of each axis.
static std::set<int> window_keys(const NaGeom& g, int q) {
  const int plane = g.grid_h * g.grid_w;
  const int z = q / plane, y = q % plane / g.grid_w, x = q % g.grid_w;
  std::set<int> keys;
  for (int zc : axis_cells(z, g.grid_d, g.kernel_d, g.wrap_d, g.dil_d))
    for (int yc : axis_cells(y, g.grid_h, g.kernel_h, g.wrap_h, g.dil_h))
      for (int xc : axis_cells(x, g.grid_w, g.kernel_w, g.wrap_w, g.dil_w)) keys.insert((zc * g.grid_h + yc) * g.grid_w + xc);
  return keys;
}

// The kernel's element predicate for (query, key): the undilated form when every
// dilation is 1, else the anchor form.
static bool kernel_predicate(const NaGeom& g, int q, int key) {
  const int plane = g.grid_h * g.grid_w;
  const int zq = q / plane, yq = q % plane / g.grid_w, xq = q % g.grid_w;
  const int zk = key / plane, yk = key % plane / g.grid_w, xk = key % g.grid_w;
  if ((g.dil_d | g.dil_h | g.dil_w) == 1)
    return na_axis_ok(zq, zk, g.grid_d, g.kernel_d, g.rad_d, g.wrap_d) &&
           na_axis_ok(yq, yk, g.grid_h, g.kernel_h, g.rad_h, g.wrap_h) &&
           na_axis_ok(xq, xk, g.grid_w, g.kernel_w, g.rad_w, g.wrap_w);
  const int az = na_dil_anchor(zq, g.grid_d, g.kernel_d, g.rad_d, g.wrap_d, g.dil_d);
  const int ay = na_dil_anchor(yq, g.grid_h, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h);
  const int ax = na_dil_anchor(xq, g.grid_w, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w);
  return na_dil_ok(az, zk, g.grid_d, g.kernel_d, g.rad_d, g.wrap_d, g.dil_d) &&
         na_dil_ok(ay, yk, g.grid_h, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h) &&
         na_dil_ok(ax, xk, g.grid_w, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w);
}

static bool geom_valid(const NaGeom& g) {
  return na_axis_valid(g.grid_d, g.kernel_d, g.wrap_d, g.dil_d) && na_axis_valid(g.grid_h, g.kernel_h, g.wrap_h, g.dil_h) &&
         na_axis_valid(g.grid_w, g.kernel_w, g.wrap_w, g.dil_w);
}

// The run of key tiles of every query tile visits each tile once and holds every
// key the window allows; the kernel's predicate equals the enumerated window.
static void check_na_geom(const NaGeom& g, int BM, int BN) {
  if (!geom_valid(g)) return;
  const int N = g.grid_d * g.grid_h * g.grid_w;
  const int n_tiles = (int)cdiv(N, BN);
  const int window = g.kernel_d * g.kernel_h * g.kernel_w;
  for (int q0 = 0; q0 < N; q0 += BM) {
    const KvRun run = kv_run(MASK_NA, N, N, BM, BN, q0, g);
    EXPECT(run.first >= 0 && run.first < n_tiles && run.count >= 1 && run.count <= n_tiles,
           "run out of range grid %dx%dx%d q0 %d", g.grid_d, g.grid_h, g.grid_w, q0);
    std::set<int> visited;
    for (int i = 0; i < run.count; ++i) {
      const int t = kv_tile_at(run, i, n_tiles);
      EXPECT(t >= 0 && t < n_tiles, "tile index %d out of range", t);
      EXPECT(visited.insert(t).second, "tile %d visited twice (grid %dx%dx%d q0 %d)", t, g.grid_d, g.grid_h, g.grid_w, q0);
    }
    for (int q = q0; q < N && q < q0 + BM; ++q) {
      const std::set<int> want = window_keys(g, q);
      EXPECT((int)want.size() == window, "window size %d, want %d (grid %dx%dx%d k %d,%d,%d dil %d,%d,%d)",
             (int)want.size(), window, g.grid_d, g.grid_h, g.grid_w, g.kernel_d, g.kernel_h, g.kernel_w, g.dil_d,
             g.dil_h, g.dil_w);
      for (int key = 0; key < N; ++key) {
        const bool ok = kernel_predicate(g, q, key);
        EXPECT(ok == (want.count(key) == 1), "predicate vs window, grid %dx%dx%d k %d,%d,%d wrap %d%d%d dil %d,%d,%d q %d key %d",
               g.grid_d, g.grid_h, g.grid_w, g.kernel_d, g.kernel_h, g.kernel_w, g.wrap_d, g.wrap_h, g.wrap_w,
               g.dil_d, g.dil_h, g.dil_w, q, key);
        if (ok) EXPECT(visited.count(key / BN) == 1, "allowed key %d of query %d in a skipped tile", key, q);
      }
    }
  }
}

// The grid-window bit masks (a tile window from the per-axis masks, then each
// lane's 16 keys per block) agree with the enumerated window for every query and
// key tile.
template <int WORDS>
static void check_grid_bits_bn(const NaGeom& g) {
  const int BN = 32 * WORDS;
  const int W = g.grid_w, plane = g.grid_h * W, N = g.grid_d * plane;
  const int n_tiles = (int)cdiv(N, BN);
  for (int q = 0; q < N; ++q) {
    const GridMasks m = na_grid_masks(q / plane, q % plane / W, q % W, g);
    const std::set<int> want = window_keys(g, q);
    for (int t = 0; t < n_tiles; ++t) {
      const int k0 = t * BN, row0 = k0 / W;
      uint32_t w[WORDS];
      na_tile_window(m, row0, k0 - row0 * W, g, w);
      for (int half = 0; half < 2; ++half)
        for (int sb = 0; sb < WORDS; ++sb) {
          const uint32_t bits = lane_block_bits(w[sb], half);
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + sb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool x = key < N && want.count(key) == 1;
            EXPECT((((bits >> r) & 1u) == 1u) == x, "grid bits %dx%dx%d k %d,%d,%d wrap %d%d%d dil %d,%d,%d BN %d q %d key %d",
                   g.grid_d, g.grid_h, g.grid_w, g.kernel_d, g.kernel_h, g.kernel_w, g.wrap_d, g.wrap_h, g.wrap_w,
                   g.dil_d, g.dil_h, g.dil_w, BN, q, key);
          }
        }
    }
  }
}

// The backward's reverse masks: for every key and query tile, bit r of each block says
// whether that query's window holds the key.
static void check_reverse_bits(const NaGeom& g) {
  if (!geom_valid(g) || !na_grid_eligible(g)) return;
  const int W = g.grid_w, plane = g.grid_h * W, N = g.grid_d * plane, BN = 128;
  std::vector<std::set<int>> sees(N);
  for (int q = 0; q < N; ++q)
    for (int k : window_keys(g, q)) sees[k].insert(q);
  for (int key = 0; key < N; ++key) {
    const GridMasks m = na_grid_reverse_masks(key / plane, key % plane / W, key % W, g);
    for (int t = 0; t < (int)cdiv(N, BN); ++t) {
      const int q0 = t * BN, row0 = q0 / W;
      uint32_t w[4];
      na_tile_window(m, row0, q0 - row0 * W, g, w);
      for (int half = 0; half < 2; ++half)
        for (int sb = 0; sb < 4; ++sb) {
          const uint32_t bits = lane_block_bits(w[sb], half);
          for (int r = 0; r < 16; ++r) {
            const int q = q0 + sb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool x = q < N && sees[key].count(q) == 1;
            EXPECT((((bits >> r) & 1u) == 1u) == x, "reverse bits %dx%dx%d k %d,%d,%d wrap %d%d%d dil %d,%d,%d key %d query %d",
                   g.grid_d, g.grid_h, g.grid_w, g.kernel_d, g.kernel_h, g.kernel_w, g.wrap_d, g.wrap_h, g.wrap_w,
                   g.dil_d, g.dil_h, g.dil_w, key, q);
          }
        }
    }
  }
}

static void check_grid_bits(const NaGeom& g, int BN) {
  if (!geom_valid(g) || !na_grid_eligible(g)) return;
  if (BN == 64) check_grid_bits_bn<2>(g);
  else check_grid_bits_bn<4>(g);
}

// The backward's run of query tiles for a key tile: each tile once, and every query
// whose window holds a key of the tile is in a visited tile.
static void check_query_run(const NaGeom& g, int BN) {
  if (!geom_valid(g)) return;
  const int N = g.grid_d * g.grid_h * g.grid_w;
  const int n_tiles = (int)cdiv(N, BN);
  std::vector<std::set<int>> sees(N);  // queries that see key k
  for (int q = 0; q < N; ++q)
    for (int k : window_keys(g, q)) sees[k].insert(q);
  for (int k0 = 0; k0 < N; k0 += BN) {
    const KvRun run = na_query_run(g, N, BN, k0);
    EXPECT(run.count >= 1 && run.count <= n_tiles, "query run count %d", run.count);
    std::set<int> visited;
    for (int i = 0; i < run.count; ++i) {
      const int t = kv_tile_at(run, i, n_tiles);
      EXPECT(t >= 0 && t < n_tiles && visited.insert(t).second, "query tile %d out of range or twice", t);
    }
    for (int k = k0; k < N && k < k0 + BN; ++k)
      for (int q : sees[k])
        EXPECT(visited.count(q / BN) == 1, "query %d sees key %d but its tile is skipped (grid %dx%dx%d k %d,%d,%d wrap %d%d%d dil %d,%d,%d)",
               q, k, g.grid_d, g.grid_h, g.grid_w, g.kernel_d, g.kernel_h, g.kernel_w, g.wrap_d, g.wrap_h, g.wrap_w,
               g.dil_d, g.dil_h, g.dil_w);
  }
}

static void check_na(int gh, int gw, int kh, int kw, int wh, int ww, int BM, int BN) {
  check_na_geom(geom(1, gh, gw, 1, kh, kw, 0, wh, ww, 1, 1, 1), BM, BN);
}

// The patch groups of a plane: every token held by exactly one lane position of one
// patch (sub-grid cells (u0 + i, v0 + j), i < kPatchRows, j < kPatchCols, inside the
// sub-grids, at patch_token), and the sub-grid geometry keeps the window.
static void check_patch_rows(const NaGeom& g) {
  std::vector<int> held(g.grid_h * g.grid_w, 0);
  for (int py = 0; py < na_patch_row_groups(g); ++py)
    for (int px = 0; px < na_patch_col_groups(g, na_patch_cols_strided(g)); ++px) {
      const PatchGroup pr = na_patch_group(g, py, px, na_patch_cols_strided(g));
      EXPECT(pr.geom.kernel_h == g.kernel_h && pr.geom.kernel_w == g.kernel_w && pr.pitch == g.grid_w,
             "sub-grid geometry keeps the window and the pitch");
      for (int i = 0; i < kPatchRows; ++i)
        for (int j = 0; j < kPatchCols; ++j)
          if (pr.u0 + i < pr.geom.grid_h && pr.v0 + j < pr.geom.grid_w) {
            const int y = pr.rho + pr.stride * (pr.u0 + i), x = pr.rho_x + pr.stride_x * (pr.v0 + j);
            EXPECT(y >= 0 && y < g.grid_h && x >= 0 && x < g.grid_w, "patch (%d,%d) cell (%d,%d) is (%d,%d)", py, px,
                   i, j, y, x);
            if (y >= 0 && y < g.grid_h && x >= 0 && x < g.grid_w) {
              EXPECT(patch_token(pr, pr.u0 + i, pr.v0 + j) == y * g.grid_w + x, "patch_token");
              ++held[y * g.grid_w + x];
            }
          }
    }
  for (int t = 0; t < g.grid_h * g.grid_w; ++t)
    EXPECT(held[t] == 1, "token %d held by %d patch cells (%dx%d dil %d,%d wrap %d%d)", t, held[t], g.grid_h, g.grid_w,
           g.dil_h, g.dil_w, g.wrap_h, g.wrap_w);
}

// The patch kernel (MASK_NA_PATCH) as it walks its LDS rectangle: for every patch,
// wavefront and lane, the cells it marks visible are exactly the query's window
// (enumerated independently), each once; the rectangle fits the kernel's LDS rows;
// every step's four blocks lie inside them; and the first step holds a visible key
// of every query (it sets the reference maximum).
static int check_patch(const NaGeom& g0, int lds_rows) {
  if (!na_patch_eligible(g0, lds_rows)) return 0;
  check_patch_rows(g0);
  for (int py = 0; py < na_patch_row_groups(g0); ++py)
    for (int px = 0; px < na_patch_col_groups(g0, na_patch_cols_strided(g0)); ++px) {
      // rows and columns in the coordinates of the patch's sub-grids, as the kernel takes them
      const PatchGroup pr = na_patch_group(g0, py, px, na_patch_cols_strided(g0));
      const NaGeom& g = pr.geom;
      const int H = g.grid_h, W = g.grid_w, y0 = pr.u0, x0 = pr.v0;
      const PatchBands pb = na_patch_bands(y0, x0, g);
      EXPECT(pb.cols.count >= 1 && pb.cols.count <= kPatchKeyCols && pb.rows.count >= 1 && pb.rows.count + 3 <= lds_rows,
             "patch bands %d x %d (grid %dx%d k %d,%d wrap %d%d)", pb.rows.count, pb.cols.count, H, W, g.kernel_h,
             g.kernel_w, g.wrap_h, g.wrap_w);
      for (int w = 0; w < 4; ++w) {
        const int wy0 = y0 + 2 * w;
        if (wy0 >= H) continue;
        const Band wb = na_band(wy0, imin(wy0 + 1, H - 1), H, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h);
        int off = wb.start - pb.rows.start;
        off += off < 0 ? H : 0;
        const int n_steps = (wb.count + 3) / 4;
        EXPECT(off >= 0 && off + wb.count <= pb.rows.count && off + 4 * n_steps <= pb.rows.count + 3,
               "wave band off %d count %d of %d rows", off, wb.count, pb.rows.count);
        for (int col = 0; col < 32; ++col) {
          const int qy = wy0 + col / 16, qx = x0 + col % 16;
          if (qy >= H || qx >= W) continue;
          // the kernel's window bits: kernel cells dil apart from lo_x and lo_y in band cells
          auto win_first = [](int c, int len, int kernel, int rad, int wrap, int dil) {
            return wrap ? c - rad * dil : na_dil_anchor(c, len, kernel, rad, wrap, dil);
          };
          int lo_x = win_first(qx, W, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w) - pb.cols.start;
          lo_x += lo_x < 0 ? W : 0;
          EXPECT(lo_x >= 0 && lo_x + g.dil_w * (g.kernel_w - 1) < 64, "column window offset %d", lo_x);
          uint64_t cm64 = 0;
          for (int t = 0; t < g.kernel_w; ++t) cm64 |= 1ull << (lo_x + g.dil_w * t);
          cm64 |= cm64 >> pb.cols.count;
          const uint32_t cm = (uint32_t)cm64 & (uint32_t)((1ull << pb.cols.count) - 1ull);
          int lo_y = win_first(qy, H, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h) - pb.rows.start;
          lo_y += lo_y < 0 ? H : 0;
          EXPECT(lo_y >= 0 && lo_y + g.dil_h * (g.kernel_h - 1) < pb.rows.count, "row window offset %d", lo_y);
          uint32_t rows_w = 0;
          for (int t = 0; t < g.kernel_h; ++t) rows_w |= 1u << (lo_y + g.dil_h * t);
          std::vector<int> seen;
          bool first_step = false;
          for (int st = 0; st < n_steps; ++st)
            for (int sb = 0; sb < 4; ++sb) {
              const int r = off + 4 * st + sb;
              int ky = pb.rows.start + r;
              ky -= ky >= H ? H : 0;
              const bool rok = ((rows_w >> r) & 1u) != 0u;
              for (int x = 0; x < kPatchKeyCols; ++x) {
                int kx = pb.cols.start + x;
                kx -= kx >= W ? W : 0;
                if (rok && ((cm >> x) & 1u)) {
                  EXPECT(r < pb.rows.count && x < pb.cols.count && ky >= 0 && ky < H && kx >= 0 && kx < W,
                         "visible cell outside the rectangle");
                  seen.push_back(patch_token(pr, ky, kx));
                  first_step = first_step || st == 0;
                }
              }
            }
          std::set<int> want;  // the window on the grid itself
          for (int yc : axis_cells(pr.rho + pr.stride * qy, g0.grid_h, g0.kernel_h, g0.wrap_h, g0.dil_h))
            for (int xc : axis_cells(pr.rho_x + pr.stride_x * qx, g0.grid_w, g0.kernel_w, g0.wrap_w, g0.dil_w))
              want.insert(yc * g0.grid_w + xc);
          const std::set<int> got(seen.begin(), seen.end());
          EXPECT(got.size() == seen.size() && got == want,
                 "patch window of query (%d,%d): %zu cells (%zu distinct), want %zu (grid %dx%d k %d,%d wrap %d%d)", qy, qx,
                 seen.size(), got.size(), want.size(), H, W, g.kernel_h, g.kernel_w, g.wrap_h, g.wrap_w);
          // the first step sets the reference maximum; dilated clamped windows may leave it to the guard
          if (g.dil_h == 1) EXPECT(first_step, "query (%d,%d) sees no key in its first step", qy, qx);
        }
      }
    }
  return 1;
}

// The row groups of a plane: every grid row held by exactly one wavefront of one group,
// and a group's band rows distinct grid rows.
static void check_row_groups(const NaGeom& g) {
  std::vector<int> held(g.grid_h, 0);
  for (int gi = 0; gi < na_row_groups(g); ++gi)
    for (bool rev : {false, true}) {
      const RowGroup rg = na_row_group(g, gi, rev);
      if (!rev)
        for (int w = 0; w < kRowsGroup; ++w)
          if (rg.u0 + w < rg.len) {
            const int y = rg.rho + rg.stride * (rg.u0 + w);
            EXPECT(y >= 0 && y < g.grid_h, "group %d wavefront %d holds row %d", gi, w, y);
            if (y >= 0 && y < g.grid_h) ++held[y];
          }
      std::set<int> rows;
      for (int r = 0; r < rg.band.count; ++r) rows.insert(row_group_row(rg, r));
      EXPECT((int)rows.size() == rg.band.count, "group %d: %zu distinct band rows of %d", gi, rows.size(),
             rg.band.count);
    }
  for (int y = 0; y < g.grid_h; ++y)
    EXPECT(held[y] == 1, "grid row %d held %d times (H %d dil %d wrap %d)", y, held[y], g.grid_h, g.dil_h, g.wrap_h);
}

// The row kernel (MASK_NA_ROWS) as it walks its stages: for every plane, group of
// rows, wavefront and lane, the cells it marks visible (visible planes of the plane
// band, visible rows of the group's row band, the lane's column bits) are exactly the
// query's window, each once; every group's row band fits the stage.
static int check_rows(const NaGeom& g, int lds_rows) {
  if (!na_rows_eligible(g, lds_rows)) return 0;
  const int H = g.grid_h, W = g.grid_w, D = g.grid_d;
  check_row_groups(g);
  for (int z = 0; z < D; ++z)
    for (int gi = 0; gi < na_row_groups(g); ++gi) {
      const Band bz = na_band(z, z, D, g.kernel_d, g.rad_d, g.wrap_d, g.dil_d);
      const RowGroup rg = na_row_group(g, gi, false);
      const Band by = rg.band;
      EXPECT(by.count >= 1 && by.count <= lds_rows && by.count <= rg.len && bz.count >= 1 && bz.count <= D,
             "rows bands %d, %d", by.count, bz.count);
      for (int w = 0; w < kRowsGroup; ++w) {
        if (rg.u0 + w >= rg.len) continue;
        const int y = rg.rho + rg.stride * (rg.u0 + w);
        for (int x = 0; x < W; ++x) {
          const GridMasks gm = na_grid_masks(z, y, x, g);
          std::vector<int> seen;
          for (int i = 0; i < bz.count; ++i) {
            const int zk = (bz.start + i) % D;
            if (!bit128(gm.z0, gm.z1, zk)) continue;
            for (int r = 0; r < by.count; ++r) {
              const int yk = row_group_row(rg, r);
              EXPECT(yk >= 0 && yk < H, "band row %d of the group maps to grid row %d", r, yk);
              if (!bit128(gm.y0, gm.y1, yk)) continue;
              for (int xk = 0; xk < 32; ++xk)
                if ((((uint32_t)gm.x0 >> xk) & 1u) != 0) {
                  EXPECT(xk < W, "column bit past the grid width");
                  seen.push_back((zk * H + yk) * W + xk);
                }
            }
          }
          const int q = (z * H + y) * W + x;
          const std::set<int> want = window_keys(g, q), got(seen.begin(), seen.end());
          EXPECT(got.size() == seen.size() && got == want,
                 "rows window of query %d: %zu cells (%zu distinct), want %zu (grid %dx%dx%d k %d,%d,%d wrap %d%d%d "
                 "dil %d,%d,%d)", q, seen.size(), got.size(), want.size(), D, H, W, g.kernel_d, g.kernel_h,
                 g.kernel_w, g.wrap_d, g.wrap_h, g.wrap_w, g.dil_d, g.dil_h, g.dil_w);
        }
      }
    }
  return 1;
}

// The dK/dV row kernel as it walks its stages: for every key plane, group of key
// rows, wavefront and lane, the query cells it marks (visible planes of the reverse
// plane band, visible rows of the group's reverse row band, the lane's query-column
// bits, all from the key's reverse masks) are exactly the queries whose window holds
// the key, each once; every group's reverse row band fits the stage.
static int check_rows_reverse(const NaGeom& g, int lds_rows) {
  if (!na_rows_reverse_eligible(g, lds_rows)) return 0;
  const int H = g.grid_h, W = g.grid_w, D = g.grid_d, N = D * H * W;
  std::vector<std::set<int>> seers(N);
  for (int q = 0; q < N; ++q)
    for (int k : window_keys(g, q)) seers[k].insert(q);
  check_row_groups(g);
  for (int z = 0; z < D; ++z)
    for (int gi = 0; gi < na_row_groups(g); ++gi) {
      const Band bz = na_band_reverse(z, z, D, g.kernel_d, g.rad_d, g.wrap_d, g.dil_d);
      const RowGroup rg = na_row_group(g, gi, true);
      const Band by = rg.band;
      EXPECT(by.count >= 1 && by.count <= lds_rows && by.count <= rg.len && bz.count >= 1 && bz.count <= D,
             "reverse bands %d, %d", by.count, bz.count);
      int own = z - bz.start;
      own += own < 0 ? D : 0;
      EXPECT(own >= 0 && own < bz.count, "the key plane %d lies in its reverse band", z);
      for (int w = 0; w < kRowsGroup; ++w) {
        if (rg.u0 + w >= rg.len) continue;
        const int y = rg.rho + rg.stride * (rg.u0 + w);
        for (int x = 0; x < W; ++x) {
          const GridMasks rm = na_grid_reverse_masks(z, y, x, g);
          std::vector<int> seen;
          for (int i = 0; i < bz.count; ++i) {
            const int zq = (bz.start + i) % D;
            if (!bit128(rm.z0, rm.z1, zq)) continue;
            for (int r = 0; r < by.count; ++r) {
              const int yq = row_group_row(rg, r);
              EXPECT(yq >= 0 && yq < H, "band row %d of the group maps to grid row %d", r, yq);
              if (!bit128(rm.y0, rm.y1, yq)) continue;
              for (int xq = 0; xq < 32; ++xq)
                if ((((uint32_t)rm.x0 >> xq) & 1u) != 0) {
                  EXPECT(xq < W, "query column bit past the grid width");
                  seen.push_back((zq * H + yq) * W + xq);
                }
            }
          }
          const int k = (z * H + y) * W + x;
          const std::set<int> got(seen.begin(), seen.end());
          EXPECT(got.size() == seen.size() && got == seers[k],
                 "reverse rows of key %d: %zu cells (%zu distinct), want %zu (grid %dx%dx%d k %d,%d,%d wrap %d%d%d "
                 "dil %d,%d,%d)", k, seen.size(), got.size(), seers[k].size(), D, H, W, g.kernel_d, g.kernel_h,
                 g.kernel_w, g.wrap_d, g.wrap_h, g.wrap_w, g.dil_d, g.dil_h, g.dil_w);
        }
      }
    }
  return 1;
}

// The backward patch kernels as they walk their rectangles: for every patch, wavefront
// and lane (a query of the dQ kernel, reverse = false; a key of the dK/dV kernel), the
// cells it marks (its wavefront's band rows of the rectangle whose row bit is set, its
// column bits) are exactly its window (the queries that see its key), each once, and
// every rectangle fits `lds_rows` rows of 32 tokens.
static int check_patch_bwd(const NaGeom& g0, int lds_rows, bool reverse) {
  if (!na_patch_bwd_eligible(g0, lds_rows, reverse)) return 0;
  const int N = g0.grid_h * g0.grid_w;
  std::vector<std::vector<int>> want(N);  // sorted, distinct
  for (int q = 0; q < N; ++q)
    for (int k : window_keys(g0, q)) {
      if (reverse) want[k].push_back(q);  // q ascending: sorted
      else want[q].push_back(k);          // from a set: sorted
    }
  check_patch_rows(g0);
  for (int py = 0; py < na_patch_row_groups(g0); ++py)
    for (int px = 0; px < na_patch_col_groups(g0, na_patch_cols_strided(g0)); ++px) {
      // rows and columns in the coordinates of the patch's sub-grids, as the kernels take them
      const PatchGroup pr = na_patch_group(g0, py, px, na_patch_cols_strided(g0));
      const NaGeom& g = pr.geom;
      const int H = g.grid_h, W = g.grid_w, y0 = pr.u0, x0 = pr.v0;
      const PatchBands pb = reverse ? na_patch_reverse_bands(y0, x0, g) : na_patch_bands(y0, x0, g);
      EXPECT(pb.rows.count >= 1 && pb.rows.count <= lds_rows && pb.cols.count >= 1 && pb.cols.count <= kPatchKeyCols,
             "patch rectangle %d x %d", pb.rows.count, pb.cols.count);
      for (int w = 0; w < 4; ++w) {
        if (y0 + 2 * w >= H) continue;
        const int wy0 = y0 + 2 * w;
        const Band wb = reverse ? na_band_reverse(wy0, imin(wy0 + 1, H - 1), H, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h)
                                : na_band(wy0, imin(wy0 + 1, H - 1), H, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h);
        int off = wb.start - pb.rows.start;
        off += off < 0 ? H : 0;
        EXPECT(off >= 0 && off + wb.count <= pb.rows.count, "wavefront band [%d, +%d) inside the rectangle's %d rows",
               off, wb.count, pb.rows.count);
        for (int c = 0; c < 32; ++c) {
          const int cy = wy0 + (c >> 4), cx = x0 + (c & 15);
          if (cy >= H || cx >= W) continue;
          const uint32_t cm = band_window_bits(cx, pb.cols, W, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w, reverse);
          const uint32_t rows_w = band_window_bits(cy, pb.rows, H, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h, reverse);
          std::vector<int> seen;
          for (int r = off; r < off + wb.count; ++r) {
            if (!((rows_w >> r) & 1u)) continue;
            const int ty = (pb.rows.start + r) % H;
            for (int x = 0; x < pb.cols.count; ++x)
              if ((cm >> x) & 1u) seen.push_back(patch_token(pr, ty, (pb.cols.start + x) % W));
          }
          const int me = patch_token(pr, cy, cx);
          std::sort(seen.begin(), seen.end());
          EXPECT(seen == want[me],  // equal sorted lists: the same cells, each once
                 "%s patch cells of token %d: %zu, want %zu (grid %dx%d k %d,%d wrap %d%d dil %d,%d)",
                 reverse ? "dK/dV" : "dQ", me, seen.size(), want[me].size(), H, W, g.kernel_h, g.kernel_w, g.wrap_h,
                 g.wrap_w, g.dil_h, g.dil_w);
        }
      }
    }
  return 1;
}

static void check_causal(int Nq, int Nkv, int BM, int BN) {
  const int n_tiles = (int)cdiv(Nkv, BN);
  for (int q0 = 0; q0 < Nq; q0 += BM) {
    const KvRun run = kv_run(MASK_CAUSAL, Nq, Nkv, BM, BN, q0, NaGeom{});
    const int q_last = (q0 + BM < Nq ? q0 + BM : Nq) - 1;
    const int want = q_last / BN + 1 < n_tiles ? q_last / BN + 1 : n_tiles;
    EXPECT(run.first == 0 && run.count == want, "causal run Nq %d Nkv %d q0 %d", Nq, Nkv, q0);
    for (int i = 0; i < run.count; ++i) {
      const int t = kv_tile_at(run, i, n_tiles);
      // a tile needs no element mask only if every key is <= every query of the tile and < Nkv
      if (!tile_needs_mask(MASK_CAUSAL, Nkv, BN, q0, t))
        EXPECT((t + 1) * BN - 1 <= q0 && (t + 1) * BN <= Nkv, "mask flag");
    }
    // every key j <= q_last, j < Nkv lies in a visited tile
    for (int j = 0; j <= q_last && j < Nkv; ++j) EXPECT(j / BN < run.count, "causal key %d skipped", j);
  }
}

static void check_work_items(int mask, int BH, int n_qtiles, int group) {
  const int n_wg = BH * n_qtiles;
  std::vector<int> seen(n_wg, 0), xcd_of_head(BH, -1);
  for (int wg = 0; wg < n_wg; ++wg) {
    const WorkItem w = work_item(mask, wg, n_wg, n_qtiles, BH, group);
    EXPECT(w.bh >= 0 && w.bh < BH && w.qtile >= 0 && w.qtile < n_qtiles, "work item out of range");
    if (w.bh >= 0 && w.bh < BH && w.qtile >= 0 && w.qtile < n_qtiles) seen[w.bh * n_qtiles + w.qtile]++;
    if (mask == MASK_CAUSAL) {
      // superblocks of 8 * group heads: inside one, longest (highest query tile) first; and a
      // superblock with a multiple of 8 heads keeps each head on one XCD (wg % 8)
      const int span = 8 * group, blk = wg / (span * n_qtiles);
      const int heads = std::min(span, BH - blk * span);
      EXPECT(w.bh / span == blk, "causal item %d leaves its superblock", wg);
      if (wg > 0 && (wg - 1) / (span * n_qtiles) == blk) {
        const WorkItem prev = work_item(mask, wg - 1, n_wg, n_qtiles, BH, group);
        EXPECT(prev.qtile >= w.qtile, "causal items not longest first at %d", wg);
      }
      if (heads % 8 == 0 && w.bh >= 0 && w.bh < BH) {
        if (xcd_of_head[w.bh] < 0) xcd_of_head[w.bh] = wg % 8;
        EXPECT(xcd_of_head[w.bh] == wg % 8, "head %d spread over XCDs", w.bh);
      }
    }
  }
  for (int i = 0; i < n_wg; ++i) EXPECT(seen[i] == 1, "work item %d covered %d times", i, seen[i]);
}

// The remainder split: whole tiles and parts cover every (tile, key tile) once;
// parts of one tile are contiguous, non-empty key ranges in order; slots are
// distinct; every CU gets about the same amount of work.
static void check_split(int64_t n_tiles, int32_t n_kv, int32_t cus) {
  const SplitPlan p = split_plan(MASK_NONE, n_tiles, n_kv, cus);
  EXPECT(split_plan(MASK_CAUSAL, n_tiles, n_kv, cus).rem == 0, "causal never splits");
  EXPECT(split_plan(ATTN_MASK_NA2D, n_tiles, n_kv, cus).rem == 0, "2D neighbourhood never splits");
  EXPECT(split_plan(ATTN_MASK_NA3D, n_tiles, n_kv, cus).rem == 0, "3D neighbourhood never splits");
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
  EXPECT(check_problem(2, 5, 4096, 4096, 64, 0.125f, ATTN_MASK_NONE, nullptr) == ATTN_OK, "valid none");
  EXPECT(check_problem(2, 5, 4096, 77, 64, 0.125f, ATTN_MASK_NONE, nullptr) == ATTN_OK, "valid cross");
  EXPECT(check_problem(2, 5, 100, 300, 64, 0.125f, ATTN_MASK_CAUSAL, nullptr) == ATTN_OK, "valid causal cross");
  EXPECT(check_problem(2, 4, 4096, 4096, 32, 0.17f, ATTN_MASK_NA2D, &p) == ATTN_OK, "valid na2d");
  EXPECT(check_problem(2, 5, 64, 64, 128, 0.1f, 0, nullptr) == ATTN_OK, "d=128");
  EXPECT(check_problem(0, 5, 4096, 4096, 64, 0.125f, 0, nullptr) == ATTN_ERR_INVALID_ARG, "B=0");
  EXPECT(check_problem(2, -1, 4096, 4096, 64, 0.125f, 0, nullptr) == ATTN_ERR_INVALID_ARG, "H<0");
  EXPECT(check_problem(2, 5, 0, 4096, 64, 0.125f, 0, nullptr) == ATTN_ERR_INVALID_ARG, "Nq=0");
  EXPECT(check_problem(2, 5, 4096, 0, 64, 0.125f, 0, nullptr) == ATTN_ERR_INVALID_ARG, "Nkv=0");
  EXPECT(check_problem(2, 5, 64, 64, 96, 0.125f, 0, nullptr) == ATTN_ERR_UNSUPPORTED, "d=96");
  // one head's Q and dO rows pass a 32-bit buffer record count in the backward only
  EXPECT(check_problem(1, 1, 33554432, 64, 64, 0.125f, 0, nullptr) == ATTN_OK, "forward: Nq * d * 2 = 2^32");
  EXPECT(check_bwd_problem(1, 1, 33554432, 64, 64, 0.125f, 0, nullptr) == ATTN_ERR_UNSUPPORTED,
         "backward: Nq * d * 2 = 2^32");
  EXPECT(check_bwd_problem(1, 1, 16777215, 64, 64, 0.125f, 0, nullptr) == ATTN_OK, "backward: Nq * d * 2 < 2^31");
  EXPECT(check_problem(2, 5, 64, 64, 64, 1.0f / 0.0f, 0, nullptr) == ATTN_ERR_INVALID_ARG, "inf scale");
  EXPECT(check_problem(2, 5, 64, 64, 64, 0.1f, 4, nullptr) == ATTN_ERR_INVALID_ARG, "mode 4");
  EXPECT(check_problem(2, 5, 64, 64, 64, 0.1f, ATTN_MASK_CAUSAL, &p) == ATTN_ERR_INVALID_ARG, "params with causal");
  EXPECT(check_problem(2, 5, 64, 64, 64, 0.1f, ATTN_MASK_NA2D, nullptr) == ATTN_ERR_INVALID_ARG, "na2d no params");
  EXPECT(check_problem(2, 5, 64, 64, 64, 0.1f, ATTN_MASK_NA3D, nullptr) == ATTN_ERR_INVALID_ARG, "na3d no params");
  EXPECT(check_problem(1, 1, (int64_t)1 << 31, 1 << 20, 64, 0.1f, 0, nullptr) == ATTN_ERR_UNSUPPORTED, "Nq too large");
  EXPECT(check_problem(1, 1, 1 << 20, (int64_t)1 << 31, 64, 0.1f, 0, nullptr) == ATTN_ERR_UNSUPPORTED, "Nkv too large");
  EXPECT(check_problem((int64_t)1 << 20, (int64_t)1 << 20, 4096, 4096, 64, 0.1f, 0, nullptr) == ATTN_ERR_UNSUPPORTED,
         "too many work-groups");
  attn_na2d_params_t bad = p;
  bad.grid_h = 63;
  EXPECT(check_problem(1, 1, 4096, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_ERR_PARAMS, "grid mismatch");
  EXPECT(check_problem(1, 1, 4096, 4000, 32, 0.1f, ATTN_MASK_NA2D, &p) == ATTN_ERR_PARAMS, "Nq != Nkv");
  bad = p; bad.kernel_h = 6;
  EXPECT(check_problem(1, 1, 4096, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_ERR_PARAMS, "even kernel");
  bad = p; bad.kernel_w = 65;
  EXPECT(check_problem(1, 1, 4096, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_ERR_PARAMS, "kernel > grid");
  bad = p; bad.wrap_w = 2;
  EXPECT(check_problem(1, 1, 4096, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_ERR_PARAMS, "wrap 2");
  bad = p; bad.dil_h = 0;
  EXPECT(check_problem(1, 1, 4096, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_ERR_PARAMS, "dilation 0");
  bad = p; bad.dil_h = 10;  // wrapped: (7 - 1) * 10 < 64
  EXPECT(check_problem(1, 1, 4096, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_OK, "wrapped dilation 10");
  bad.dil_h = 11;           // (7 - 1) * 11 >= 64
  EXPECT(check_problem(1, 1, 4096, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_ERR_PARAMS, "wrapped dilation 11");
  bad = p; bad.wrap_w = 0; bad.dil_w = 9;  // clamped: 7 * 9 <= 64
  EXPECT(check_problem(1, 1, 4096, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_OK, "clamped dilation 9");
  bad.dil_w = 10;                          // 7 * 10 > 64
  EXPECT(check_problem(1, 1, 4096, 4096, 32, 0.1f, ATTN_MASK_NA2D, &bad) == ATTN_ERR_PARAMS, "clamped dilation 10");
  attn_na3d_params_t v3{20, 20, 20, 5, 5, 5, 1, 1, 0, 1, 1, 1};
  EXPECT(check_problem(2, 4, 8000, 8000, 32, 0.1f, ATTN_MASK_NA3D, &v3) == ATTN_OK, "valid na3d");
  attn_na3d_params_t b3 = v3;
  b3.grid_d = 19;
  EXPECT(check_problem(2, 4, 8000, 8000, 32, 0.1f, ATTN_MASK_NA3D, &b3) == ATTN_ERR_PARAMS, "3D grid mismatch");
  b3 = v3; b3.kernel_d = 4;
  EXPECT(check_problem(2, 4, 8000, 8000, 32, 0.1f, ATTN_MASK_NA3D, &b3) == ATTN_ERR_PARAMS, "even depth kernel");
  b3 = v3; b3.wrap_d = 3;
  EXPECT(check_problem(2, 4, 8000, 8000, 32, 0.1f, ATTN_MASK_NA3D, &b3) == ATTN_ERR_PARAMS, "depth wrap 3");
  b3 = v3; b3.dil_w = 5;  // clamped: 5 * 5 > 20
  EXPECT(check_problem(2, 4, 8000, 8000, 32, 0.1f, ATTN_MASK_NA3D, &b3) == ATTN_ERR_PARAMS, "3D clamped dilation");
  alignas(256) char buf[512];
  auto prob = [&](const void* q, const void* k, const void* v, void* o, float* lse) {
    return Problem{q, k, v, o, lse, 1, 1, 1, 1, 8, 0.5f, ATTN_MASK_NONE, nullptr};
  };
  EXPECT(check_pointers(prob(buf + 16, buf + 32, buf + 48, buf + 64, nullptr)) == ATTN_OK, "disjoint aligned");
  EXPECT(check_pointers(prob(buf + 16, buf + 32, buf + 48, buf + 72, nullptr)) == ATTN_ERR_ALIGNMENT, "misaligned o");
  EXPECT(check_pointers(prob(buf + 16, buf + 32, buf + 48, buf + 48, nullptr)) == ATTN_ERR_INVALID_ARG, "o aliases v");
  EXPECT(check_pointers(prob(nullptr, buf + 32, buf + 48, buf + 64, nullptr)) == ATTN_ERR_INVALID_ARG, "null q");
  EXPECT(check_pointers(prob(buf + 16, buf + 32, buf + 48, buf + 64, (float*)(buf + 80))) == ATTN_OK, "lse");
  EXPECT(check_pointers(prob(buf + 16, buf + 32, buf + 48, buf + 64, (float*)(buf + 82))) == ATTN_ERR_ALIGNMENT,
         "misaligned lse");
  EXPECT(check_pointers(prob(buf + 16, buf + 32, buf + 48, buf + 64, (float*)(buf + 64))) == ATTN_ERR_INVALID_ARG,
         "lse aliases o");
  EXPECT(check_pointers(prob(buf + 16, buf + 32, buf + 48, buf + 64, (float*)(buf + 36))) == ATTN_ERR_INVALID_ARG,
         "lse inside k");
  // Nq != Nkv: k and v are [1, 1, 3, 8] (48 bytes), q and o [1, 1, 1, 8]
  Problem x{buf + 16, buf + 32, buf + 80, buf + 128, nullptr, 1, 1, 1, 3, 8, 0.5f, ATTN_MASK_NONE, nullptr};
  EXPECT(check_pointers(x) == ATTN_OK, "cross disjoint");
  x.o = buf + 112;  // inside v's 48 bytes
  EXPECT(check_pointers(x) == ATTN_ERR_INVALID_ARG, "o inside the longer v");
  x.o = buf + 128;
  EXPECT(check_workspace(buf + 256, 64, 64, x) == ATTN_OK, "workspace disjoint");
  EXPECT(check_workspace(buf + 256, 32, 64, x) == ATTN_ERR_WORKSPACE, "workspace small");
  x.lse = (float*)(buf + 260);
  EXPECT(check_workspace(buf + 256, 64, 64, x) == ATTN_ERR_WORKSPACE, "workspace overlaps lse");
}

int main() {
  check_validation();
  check_col_bits();
  check_limit_bits();
  for (int BN : {64, 128}) {
    for (int N : {1, 2, 63, 64, 65, 127, 128, 129, 200, 255, 256, 257, 600}) {
      check_causal(N, N, kBlockM, BN);
      for (int Nkv : {1, 77, 128, 300}) check_causal(N, Nkv, kBlockM, BN);
    }
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
    // dilation in 2D
    for (int gh : {5, 7, 12, 17})
      for (int gw : {6, 9, 20})
        for (int dh : {1, 2, 3})
          for (int dw : {1, 2, 4})
            for (int k : {1, 3, 5})
              for (int wh = 0; wh < 2; ++wh)
                for (int ww = 0; ww < 2; ++ww) check_na_geom(geom(1, gh, gw, 1, k, 3, 0, wh, ww, 1, dh, dw), kBlockM, BN);
    // 3D, with and without dilation
    const int d3[][3] = {{2, 3, 4}, {3, 5, 4}, {4, 4, 8}, {5, 3, 7}, {6, 6, 6}, {9, 2, 5}};
    for (const auto& gd : d3)
      for (int kd : {1, 3, 5})
        for (int kh : {1, 3})
          for (int wd = 0; wd < 2; ++wd)
            for (int wh = 0; wh < 2; ++wh)
              for (int ww = 0; ww < 2; ++ww)
                for (int dd : {1, 2})
                  check_na_geom(geom(gd[0], gd[1], gd[2], kd, kh, 3, wd, wh, ww, dd, 1, gd[2] >= 7 ? 2 : 1), kBlockM, BN);
    check_na_geom(geom(20, 20, 20, 5, 5, 5, 1, 1, 0, 1, 1, 1), kBlockM, BN);
    check_na_geom(geom(16, 16, 16, 3, 3, 3, 1, 0, 1, 2, 2, 2), kBlockM, BN);
  }
  // the backward's reverse window masks
  check_reverse_bits(geom(1, 7, 13, 1, 3, 5, 0, 0, 0, 1, 1, 1));
  check_reverse_bits(geom(1, 10, 6, 1, 5, 3, 0, 1, 0, 1, 1, 1));
  check_reverse_bits(geom(1, 17, 9, 1, 5, 3, 0, 0, 0, 1, 3, 2));
  check_reverse_bits(geom(1, 16, 20, 1, 3, 5, 0, 1, 1, 1, 2, 3));
  check_reverse_bits(geom(3, 5, 4, 3, 3, 3, 1, 1, 1, 1, 1, 1));
  check_reverse_bits(geom(6, 6, 6, 3, 3, 3, 1, 0, 1, 2, 2, 2));
  check_reverse_bits(geom(10, 9, 8, 3, 3, 3, 0, 0, 0, 3, 3, 2));
  // the backward's query runs
  for (int gh : {1, 3, 5, 9, 17})
    for (int gw : {2, 5, 8, 13, 40})
      for (int kh = 1; kh <= 5; kh += 2)
        for (int wh = 0; wh < 2; ++wh)
          for (int ww = 0; ww < 2; ++ww)
            for (int dil : {1, 2}) check_query_run(geom(1, gh, gw, 1, kh, 3, 0, wh, ww, 1, dil, 1), 128);
  check_query_run(geom(4, 5, 6, 3, 3, 3, 1, 0, 1, 1, 1, 1), 128);
  check_query_run(geom(6, 6, 6, 3, 3, 3, 1, 0, 1, 2, 2, 2), 128);
  check_query_run(geom(10, 9, 8, 3, 3, 3, 0, 0, 0, 3, 3, 2), 128);
  check_query_run(geom(1, 64, 64, 1, 7, 7, 0, 1, 1, 1, 1, 1), 128);
  check_query_run(geom(1, 64, 64, 1, 7, 7, 0, 0, 0, 1, 1, 1), 128);
  check_query_run(geom(1, 33, 17, 1, 9, 3, 0, 1, 1, 1, 1, 1), 128);
  // grid-window bit masks: widths 4..124 (incl. 61..65 around the 64-bit word boundary), 3D, dilation
  for (int BN : {64, 128}) {
    for (int W : {4, 5, 7, 20, 31, 33, 40, 61, 62, 63, 64, 65, 100, 124})
      for (int kw : {1, 3, 5})
        for (int ww = 0; ww < 2; ++ww)
          check_grid_bits(geom(1, 3, W, 1, 3, kw, 0, 1, ww, 1, 1, W >= 20 ? 2 : 1), BN);
    check_grid_bits(geom(4, 5, 6, 3, 3, 3, 1, 0, 1, 1, 1, 1), BN);
    check_grid_bits(geom(6, 6, 6, 3, 3, 3, 1, 0, 1, 2, 2, 2), BN);
    check_grid_bits(geom(10, 9, 8, 3, 3, 3, 0, 0, 0, 3, 3, 2), BN);
    check_grid_bits(geom(3, 4, 20, 3, 3, 5, 1, 1, 0, 1, 1, 3), BN);
    check_grid_bits(geom(2, 66, 4, 1, 5, 3, 0, 1, 1, 1, 9, 1), BN);   // 66 rows: row bits in the upper word
    check_grid_bits(geom(70, 2, 4, 5, 1, 1, 1, 0, 0, 3, 1, 1), BN);   // 70 planes
  }
  {
    // patch kernel: grids, windows and wrap flags around the limits of na_patch_eligible
    int eligible = 0, tried = 0, bwd_dq = 0, bwd_dkv = 0;
    for (int H : {7, 11, 17, 33, 64})
      for (int W : {9, 17, 32, 33, 64})
        for (int k : {1, 3, 7, 9, 13, 17, 19})
          for (int wh = 0; wh < 2; ++wh)
            for (int ww = 0; ww < 2; ++ww)
              for (int lds_rows : {17, 24}) {
                const int dil = (k + wh + ww) % 3 == 0 ? 2 : 1;  // a third of the shapes dilated
                const NaGeom g = geom(1, H, W, 1, k, k == 1 ? 3 : k - 2, 0, wh, ww, 1, dil, dil);
                if (!geom_valid(g)) continue;
                ++tried;
                eligible += check_patch(g, lds_rows);
                // each shape once, at one of the two rectangle sizes (d = 32: 24 rows, d = 64: 17)
                if ((H + W + k + lds_rows) % 2 == 0) {
                  bwd_dq += check_patch_bwd(g, lds_rows, false);
                  bwd_dkv += check_patch_bwd(g, lds_rows, true);
                }
              }
    EXPECT(eligible > 100 && eligible < tried, "patch eligibility covers %d of %d shapes", eligible, tried);
    EXPECT(bwd_dq > 40 && bwd_dkv > 30 && bwd_dkv <= tried, "backward patch eligibility: dQ %d, dK/dV %d of %d",
           bwd_dq, bwd_dkv, tried);
    EXPECT(na_patch_bwd_eligible(geom(1, 64, 64, 1, 7, 7, 0, 1, 1, 1, 1, 1), 24, false) &&
               na_patch_bwd_eligible(geom(1, 64, 64, 1, 7, 7, 0, 1, 1, 1, 1, 1), 24, true),
           "64x64 grid, 7x7 wrapped window: both backward patch kernels");
    const NaGeom c4 = geom(1, 64, 64, 1, 7, 7, 0, 1, 1, 1, 1, 1);
    EXPECT(na_patch_eligible(c4, 24) && na_patch_eligible(c4, 17), "64x64 grid, 7x7 wrapped window takes the patch kernel");
    EXPECT(na_patch_eligible(geom(1, 64, 64, 1, 7, 7, 0, 1, 1, 1, 2, 2), 17) &&
               na_patch_bwd_eligible(geom(1, 64, 64, 1, 7, 7, 0, 1, 1, 1, 2, 2), 17, false) &&
               na_patch_bwd_eligible(geom(1, 64, 64, 1, 7, 7, 0, 1, 1, 1, 2, 2), 17, true),
           "and with dilation 2: patches of rows of one parity, 14-row bands, also in 17 rows (d = 64)");
    EXPECT(!na_patch_eligible(geom(1, 63, 64, 1, 7, 7, 0, 1, 1, 1, 2, 2), 17) &&
               na_patch_eligible(geom(1, 63, 64, 1, 7, 7, 0, 1, 1, 1, 2, 2), 24),
           "63 wrapped rows at dilation 2: consecutive rows, 20-row bands, not in 17 rows");
    EXPECT(!na_patch_eligible(geom(4, 20, 20, 3, 5, 5, 1, 1, 1, 1, 1, 1), 24), "3D windows do not");
    EXPECT(!na_patch_eligible(geom(1, 64, 64, 1, 7, 19, 0, 1, 1, 1, 1, 1), 24), "19 columns wide: the band passes 32");
    // columns of one residue mod the dilation: 16 + 2 rad sub-grid columns per band
    EXPECT(check_patch(geom(1, 64, 64, 1, 7, 7, 0, 1, 1, 1, 4, 4), 17) == 1 &&
               check_patch_bwd(geom(1, 64, 64, 1, 7, 7, 0, 1, 1, 1, 4, 4), 17, false) == 1 &&
               check_patch_bwd(geom(1, 64, 64, 1, 7, 7, 0, 1, 1, 1, 4, 4), 17, true) == 1,
           "64x64 grid, 7x7 window of dilation 4: patches of one residue per axis, 14 x 22 rectangles");
    EXPECT(check_patch(geom(1, 40, 48, 1, 5, 9, 0, 0, 0, 1, 3, 3), 24) == 1 &&
               check_patch_bwd(geom(1, 40, 48, 1, 5, 9, 0, 0, 0, 1, 3, 3), 24, false) == 1 &&
               check_patch_bwd(geom(1, 40, 48, 1, 5, 9, 0, 0, 0, 1, 3, 3), 24, true) == 1,
           "clamped 5x9 window of dilation 3 on 40x48: residue sub-grids of unequal lengths");
    EXPECT(check_patch(geom(1, 33, 50, 1, 5, 5, 0, 1, 0, 1, 2, 3), 24) == 1 &&
               check_patch_bwd(geom(1, 33, 50, 1, 5, 5, 0, 1, 0, 1, 2, 3), 24, true) == 1,
           "33 wrapped rows (consecutive) and 50 clamped columns of dilation 3 (one residue)");
    EXPECT(!na_patch_eligible(geom(1, 64, 66, 1, 7, 7, 0, 1, 1, 1, 4, 4), 24),
           "66 wrapped columns at dilation 4: consecutive columns, a 40-column band");
    EXPECT(!na_patch_cols_strided(geom(1, 64, 64, 1, 7, 7, 0, 1, 1, 1, 2, 2)) &&
               na_patch_cols_strided(geom(1, 64, 64, 1, 7, 7, 0, 1, 1, 1, 4, 4)),
           "columns by residue only where consecutive ones pass 32 (dilation 2: 28 columns fit)");
  }
  {
    // row kernel: narrow 2D and 3D grids, wrap and clamp per axis, dilation
    int eligible = 0, eligible_rev = 0, tried = 0, wide = 0, wide_rev = 0;
    for (int D : {1, 5})
      for (int H : {4, 9, 20})
        for (int W : {7, 20, 32})
          for (int k : {1, 3, 5})
            for (int dil : {1, 2})
              for (int wrap = 0; wrap < 8; ++wrap) {
                const NaGeom g = geom(D, H, W, D == 1 ? 1 : k, k, k == 1 ? 3 : k, (wrap >> 2) & 1, (wrap >> 1) & 1,
                                      wrap & 1, D == 1 ? 1 : dil, dil, 1);
                if (!geom_valid(g)) continue;
                ++tried;
                eligible += check_rows(g, 10);
                if (W % 2 == 1) check_rows(g, 8);  // the backward dQ row kernel's stages at d = 64
                eligible_rev += check_rows_reverse(g, 8);
                // the wide 12-row stages, where the narrow ones do not fit
                if (!na_rows_eligible(g, 10)) wide += check_rows(g, 12);
                if (!na_rows_reverse_eligible(g, 8)) wide_rev += check_rows_reverse(g, 12);
              }
    EXPECT(wide_rev > 10, "wide row stages take %d (forward) and %d (reverse) more shapes", wide, wide_rev);
    // the wide forward stages: wrapped rows that the dilation does not divide keep consecutive groups
    EXPECT(check_rows(geom(5, 15, 9, 3, 5, 3, 1, 1, 0, 2, 2, 1), 12) == 1 &&
               check_rows(geom(2, 13, 20, 1, 5, 5, 0, 1, 0, 1, 2, 3), 12) == 1 &&
               check_rows_reverse(geom(5, 15, 9, 3, 5, 3, 1, 1, 0, 2, 2, 1), 12) == 1,
           "wide stages of consecutive dilated rows");
    EXPECT(na_rows_eligible(geom(20, 20, 20, 5, 5, 5, 1, 1, 0, 2, 2, 2), 8) &&
               na_rows_reverse_eligible(geom(20, 20, 20, 5, 5, 5, 1, 1, 0, 2, 2, 2), 8),
           "20x20x20, 5x5x5 window of dilation 2: groups of one residue, 8-row bands");
    EXPECT(!na_rows_strided(geom(5, 15, 9, 3, 5, 3, 1, 1, 0, 2, 2, 1)) &&
               !na_rows_eligible(geom(5, 15, 9, 3, 5, 3, 1, 1, 0, 2, 2, 1), 10) &&
               na_rows_eligible(geom(5, 15, 9, 3, 5, 3, 1, 1, 0, 2, 2, 1), 12),
           "15 wrapped rows at dilation 2: consecutive rows, 12-row bands, the wide stages");
    EXPECT(na_rows_reverse_eligible(geom(20, 20, 20, 5, 5, 5, 0, 0, 0, 1, 1, 1), 12),
           "clamped 5x5x5 windows: the 10-row reverse bands near the borders fit the wide stages");
    EXPECT(eligible > 100 && eligible <= tried, "row-kernel eligibility covers %d of %d shapes", eligible, tried);
    EXPECT(eligible_rev > 80 && eligible_rev < eligible, "dK/dV row-kernel eligibility covers %d of %d shapes",
           eligible_rev, tried);
    EXPECT(na_rows_reverse_eligible(geom(20, 20, 20, 5, 5, 5, 1, 1, 0, 1, 1, 1), 8),
           "20x20x20, 5x5x5 window: dK/dV by key rows");
    EXPECT(!na_rows_reverse_eligible(geom(1, 20, 20, 1, 5, 5, 1, 0, 0, 1, 1, 1), 8),
           "clamped 5-row windows near a border: 10 query rows reach the key rows 4..7");
    // the reverse band of one clamped axis against brute force, every coordinate range
    for (int len : {1, 2, 5, 9, 20, 23})
      for (int kernel : {1, 3, 5, 7})
        for (int dil : {1, 2, 3, 4})
          for (int wrap : {0, 1}) {
            const NaGeom ax = geom(1, 1, len, 1, 1, kernel, 0, 0, wrap, 1, 1, dil);
            if (!geom_valid(ax)) continue;
            for (int c0 = 0; c0 < len; ++c0)
              for (int c1 = c0; c1 < len && c1 < c0 + 4; ++c1) {
                const Band b = na_band_reverse(c0, c1, len, kernel, ax.rad_w, wrap, dil);
                EXPECT(b.count >= 1 && b.count <= len && b.start >= 0 && b.start < len, "reverse band in range");
                for (int q = 0; q < len; ++q)
                  for (int k = c0; k <= c1; ++k) {
                    const bool sees = na_dil_ok(na_dil_anchor(q, len, kernel, ax.rad_w, wrap, dil), k, len, kernel,
                                                ax.rad_w, wrap, dil);
                    const int off = ((q - b.start) % len + len) % len;
                    EXPECT(!sees || off < b.count, "query %d sees key %d outside the reverse band (len %d k %d dil %d "
                           "wrap %d)", q, k, len, kernel, dil, wrap);
                  }
                if (!wrap && dil == 1) {  // exact: its ends are seers
                  bool first = false, last = false;
                  for (int k = c0; k <= c1; ++k) {
                    first |= na_axis_ok(b.start, k, len, kernel, ax.rad_w, 0);
                    last |= na_axis_ok(b.start + b.count - 1, k, len, kernel, ax.rad_w, 0);
                  }
                  EXPECT(first && last, "clamped reverse band [%d, +%d) is tight", b.start, b.count);
                }
                if (!wrap && dil > 1) {  // within dil - 1 cells of a seer at each end
                  bool first = false, last = false;
                  for (int q = 0; q < len; ++q)
                    for (int k = c0; k <= c1; ++k)
                      if (na_dil_ok(na_dil_anchor(q, len, kernel, ax.rad_w, 0, dil), k, len, kernel, ax.rad_w, 0, dil)) {
                        first |= q - b.start < dil;
                        last |= b.start + b.count - 1 - q < dil;
                      }
                  EXPECT(first && last, "dilated clamped reverse band [%d, +%d) within dil of its queries (len %d k %d "
                         "dil %d)", b.start, b.count, len, kernel, dil);
                }
              }
            if (!wrap)  // the exact reverse run of a clamped axis: the queries whose enumerated window holds x
              for (int x = 0; x < len; ++x) {
                std::vector<int> want, got;
                for (int q = 0; q < len; ++q)
                  for (int c : axis_cells(q, len, kernel, 0, dil))
                    if (c == x) want.push_back(q);
                const Band r = na_clamped_reverse_run(x, len, kernel, ax.rad_w, dil);
                for (int u = 0; u < r.count; ++u) got.push_back(r.start + dil * u);
                EXPECT(got == want, "clamped reverse run of %d: %zu queries, want %zu (len %d k %d dil %d)", x,
                       got.size(), want.size(), len, kernel, dil);
              }
          }
    EXPECT(na_rows_eligible(geom(20, 20, 20, 5, 5, 5, 1, 1, 0, 1, 1, 1), 10), "20x20x20, 5x5x5 window takes the row kernel");
    EXPECT(!na_rows_eligible(geom(1, 64, 64, 1, 7, 7, 0, 1, 1, 1, 1, 1), 10), "64 wide does not");
  }
  for (int mask : {MASK_NONE, MASK_CAUSAL})
    for (int BH : {1, 3, 8, 10, 64, 80})
      for (int nq : {1, 2, 7, 16, 32, 72})
        for (int group : {1, 2, 4, 64}) check_work_items(mask, BH, nq, group);
  EXPECT(causal_group(16, 256, 2) == 4, "N 2048 at d 64: 4 heads x 16 tiles fill an XCD's 64 slots");
  EXPECT(causal_group(16, 256, 1) == 2 && causal_group(64, 256, 2) == 1 && causal_group(1, 256, 2) == 64,
         "causal groups at d 128, long sequences and one tile");
  EXPECT(causal_group(40, 256, 2) == 1 && causal_group(0, 256, 2) == 1, "causal group at least 1");
  // split plans: the sizes of the unmasked workloads and small or odd shapes
  EXPECT(split_plan(MASK_NONE, 320, 32, 256).rem == 64 && split_plan(MASK_NONE, 320, 32, 256).parts == 4,
         "B2 H5 N4096: 256 whole tiles, 64 tiles in 4 parts");
  EXPECT(split_plan(MASK_NONE, 720, 72, 256).rem == 0, "B2 H5 N9216 is over two rounds deep: no split");
  EXPECT(split_plan(MASK_NONE, 512, 32, 256).rem == 0, "two full rounds need no split");
  EXPECT(split_plan(MASK_NONE, 256, 32, 256).rem == 0, "one full round needs no split");
  EXPECT(split_plan(MASK_NONE, 2, 2, 256).rem == 0, "tiny problems do not split");
  for (int32_t cus : {1, 2, 7, 64, 80, 256, 304})
    for (int64_t n_tiles : {1, 2, 3, 5, 16, 21, 33, 40, 48, 72, 80, 100, 255, 256, 257, 320, 400, 511, 512, 513})
      for (int32_t n_kv : {1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 32, 33, 64, 72, 144}) check_split(n_tiles, n_kv, cus);
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("OK\n");
  return 0;
}
