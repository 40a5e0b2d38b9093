// Which key/value tiles a query tile visits, and which of them need an element mask.
//
// Plain constexpr C++: clang compiles constexpr functions for both host and
// device, so the kernel and a host-only test build share this logic.
//
// A query tile covers queries [q0, q0 + BM) (clipped to Nq). Key tiles are
// BN consecutive tokens; tile t covers keys [t*BN, t*BN + BN) (clipped to
// Nkv). The tiles to visit form one circular run: tiles (first + i) mod
// n_tiles for i = 0 .. count-1, each visited once.
//
//  * no mask: every tile (all keys are visible; PhotoRoom's xformers post,
//    the running-softmax paragraph: keys are read tile by tile);
//  * causal: tiles up to the one holding the tile's last query (keys after a
//    query are masked, "Profiling in PyTorch", the naive causal module), so
//    fully masked tiles are never visited;
//  * neighbourhood (2D, or 3D as for the MR volumes of NATTEN issue 142):
//    the band of grid planes, or of rows of one plane, that any query of the
//    tile can see (the same issue: skipping key tiles that are fully masked is
//    predictable per query tile). With a wrapped axis the band is taken modulo
//    its length and the run of tiles wraps modulo the tile count; no input is
//    padded.
#pragma once

#include <stdint.h>

namespace attn {

// Kernel mask kinds. MASK_NA covers every 2D and 3D neighbourhood window with any
// dilation (an element predicate). The bit-mask kinds cover the common grids:
// MASK_NA_BLOCKS the 2D, undilated window on grids whose width is a multiple of
// 32 (at most 128); MASK_NA_GRID any window on grids of width 4..124 whose
// height and depth are at most 128 (na_grid_eligible). Two kernels of their own
// take most windows instead of query tiles: MASK_NA_PATCH 2D undilated windows in
// query patches (na_patch_eligible), MASK_NA_ROWS any window on grids at most 32
// wide in grid rows (na_rows_eligible).
enum : int {
  MASK_NONE = 0, MASK_CAUSAL = 1, MASK_NA = 2, MASK_NA_BLOCKS = 3, MASK_NA_GRID = 4, MASK_NA_PATCH = 5, MASK_NA_ROWS = 6
};
constexpr bool is_na(int mask) {
  return mask == MASK_NA || mask == MASK_NA_BLOCKS || mask == MASK_NA_GRID || mask == MASK_NA_PATCH ||
         mask == MASK_NA_ROWS;
}

// Neighbourhood geometry in the form the kernel uses. Token n sits at depth
// z = n / (grid_h * grid_w), row y and column x of its plane (row-major); a 2D
// grid has one plane (grid_d = kernel_d = dil_d = 1, rad_d = wrap_d = 0).
struct NaGeom {
  int32_t grid_h, grid_w;
  int32_t kernel_h, kernel_w;
  int32_t rad_h, rad_w;    // kernel / 2
  int32_t wrap_h, wrap_w;  // 1 = circular, 0 = clamped
  int32_t dil_h, dil_w;    // dilation (1 = contiguous window)
  int32_t grid_d, kernel_d, rad_d, wrap_d, dil_d;  // depth axis
};

struct KvRun {
  int32_t first;  // first tile index
  int32_t count;  // number of tiles to visit
};

constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int32_t imin(int32_t a, int32_t b) { return a < b ? a : b; }
constexpr int32_t imax(int32_t a, int32_t b) { return a > b ? a : b; }
constexpr int32_t iclamp(int32_t x, int32_t lo, int32_t hi) { return imin(imax(x, lo), hi); }
constexpr int32_t imod(int32_t a, int32_t m) { return ((a % m) + m) % m; }

// Coordinates [start, start + count) (mod len when wrapped) holding every
// window cell of every query coordinate in [c0, c1] along one axis.
struct Band {
  int32_t start, count;
};

constexpr Band na_band(int32_t c0, int32_t c1, int32_t len, int32_t kernel, int32_t rad, int32_t wrap, int32_t dil) {
  if (wrap) {  // cells (c + dil * t) mod len, |t| <= rad
    const int32_t count = (c1 - c0 + 1) + 2 * rad * dil;
    if (count >= len) return Band{0, len};
    return Band{imod(c0 - rad * dil, len), count};
  }
  // Clamped: the window of c is c - rad dil ... c + rad dil, pushed inwards near the
  // ends (na_dil_anchor). A window pushed back from the far end still starts at or
  // after len - kernel dil (its last cell is its sub-grid's, within dil of the end),
  // one pushed from the near end ends at or before kernel dil - 1 (its first cell is
  // its sub-grid's, below dil). Exact at dil = 1, where the window starts at
  // clamp(c - rad, 0, len - kernel), a non-decreasing function of c.
  const int32_t s = imax(0, imin(c0 - rad * dil, len - kernel * dil));
  const int32_t e = imin(len - 1, imax(c1 + rad * dil, kernel * dil - 1));
  return Band{s, e - s + 1};
}

// Along one axis, the query coordinates whose window holds some key coordinate in
// [c0, c1]: a wrapped window is symmetric (query c sees key c' iff key c sees
// query c'), so it is na_band itself. On a clamped axis the queries of key x share
// its residue mod dil and, on that sub-grid, run from x's sub-coordinate less rad
// to it plus rad, except that the first kernel cells of the sub-grid are seen from
// its first cell on (by the windows pushed inwards) and its last kernel cells up to
// its last: so the queries of keys at or past kernel dil start within rad dil
// before them, and those of keys before len - kernel dil end within rad dil after
// them. Exact at dil = 1 (the window start clamp(c - rad, 0, len - kernel) is
// non-decreasing in c); a superset by less than dil cells at each end otherwise.
constexpr Band na_band_reverse(int32_t c0, int32_t c1, int32_t len, int32_t kernel, int32_t rad, int32_t wrap,
                               int32_t dil) {
  if (wrap) return na_band(c0, c1, len, kernel, rad, wrap, dil);
  const int32_t first = c0 >= kernel * dil ? c0 - rad * dil : 0;
  const int32_t last = c1 < len - kernel * dil ? c1 + rad * dil : len - 1;
  return Band{first, last - first + 1};
}

constexpr KvRun kv_run(int mask, int32_t Nq, int32_t Nkv, int32_t BM, int32_t BN, int32_t q0, const NaGeom& g,
                       bool reverse = false) {
  const int32_t n_tiles = (int32_t)cdiv(Nkv, BN);
  const int32_t q_last = imin(q0 + BM, Nq) - 1;
  if (mask == MASK_CAUSAL) return KvRun{0, imin(q_last / BN + 1, n_tiles)};
  if (!is_na(mask)) return KvRun{0, n_tiles};
  const int32_t N = Nkv;  // = Nq for the neighbourhood masks
  const int32_t plane = g.grid_h * g.grid_w;
  const int32_t z0 = q0 / plane, z1 = q_last / plane;
  auto band = [reverse](int32_t c0, int32_t c1, int32_t len, int32_t kernel, int32_t rad, int32_t wrap, int32_t dil) {
    return reverse ? na_band_reverse(c0, c1, len, kernel, rad, wrap, dil)
                   : na_band(c0, c1, len, kernel, rad, wrap, dil);
  };
  const Band bz = band(z0, z1, g.grid_d, g.kernel_d, g.rad_d, g.wrap_d, g.dil_d);
  int32_t tok_start = bz.start * plane, tok_len = bz.count * plane;
  if (bz.count == 1) {  // one plane (then z0 = z1): narrow it to the band of rows
    const Band by = band((q0 - z0 * plane) / g.grid_w, (q_last - z1 * plane) / g.grid_w, g.grid_h, g.kernel_h,
                         g.rad_h, g.wrap_h, g.dil_h);
    // a row band that wraps inside one plane of several is not one run of tokens
    if (g.grid_d == 1 || by.start + by.count <= g.grid_h) {
      tok_start += by.start * g.grid_w;
      tok_len = by.count * g.grid_w;
    }
  }
  if (tok_len >= N) return KvRun{0, n_tiles};
  const int32_t tok_end = tok_start + tok_len;  // exclusive, may pass N when the band wraps
  if (tok_end <= N) {
    const int32_t a = tok_start / BN, b = (tok_end - 1) / BN;
    return KvRun{a, b - a + 1};
  }
  // wrapped band: tokens [tok_start, N) then [0, tok_end - N)
  const int32_t a = tok_start / BN;             // first tile of the upper part
  const int32_t b = (tok_end - N - 1) / BN;     // last tile of the lower part
  if (b >= a - 1) return KvRun{0, n_tiles};     // the two parts meet: every tile
  return KvRun{a, (n_tiles - a) + b + 1};
}

constexpr int32_t kv_tile_at(const KvRun& run, int32_t i, int32_t n_tiles) {
  int32_t t = run.first + i;
  return t >= n_tiles ? t - n_tiles : t;
}

// Backward of a neighbourhood window: the run of query tiles (BN queries each)
// holding every query whose window reaches a key of the tile [k0, k0 + BN), from
// the reverse bands (na_band_reverse) of the tile's keys; the element test decides
// within it.
constexpr KvRun na_query_run(const NaGeom& g, int32_t N, int32_t BN, int32_t k0) {
  return kv_run(MASK_NA, N, N, BN, BN, k0, g, true);
}

// Does key tile t need the element mask for the query tile starting at q0?
constexpr bool tile_needs_mask(int mask, int32_t Nkv, int32_t BN, int32_t q0, int32_t t) {
  const int32_t k_end = t * BN + BN;  // exclusive
  if (k_end > Nkv) return true;       // ragged last tile: keys past Nkv
  if (mask == MASK_CAUSAL) return k_end - 1 > q0;  // some key lies after some query
  return is_na(mask);
}

// Element predicate of the undilated neighbourhood window along one axis, for
// query coordinate cq and key coordinate ck. Branch-free in the coordinates (the
// wrap flag is uniform), so callers can combine axes with a plain select.
constexpr bool na_axis_ok(int32_t cq, int32_t ck, int32_t len, int32_t kernel, int32_t rad, int32_t wrap) {
  if (wrap) {
    int32_t dlt = cq - ck;
    dlt = dlt < 0 ? -dlt : dlt;
    dlt = imin(dlt, len - dlt);
    return dlt <= rad;
  }
  const int32_t start = iclamp(cq - rad, 0, len - kernel);
  return (uint32_t)(ck - start) < (uint32_t)kernel;
}

// The query-side part of the dilated window test along one axis, computed once
// per query: wrapped, the query coordinate itself; clamped, the first cell of
// its window, g + dil * clamp(c / dil - r, 0, L_g - kernel), where g = c mod dil
// and L_g is the length of the sub-grid of cells congruent to g.
constexpr int32_t na_dil_anchor(int32_t cq, int32_t len, int32_t kernel, int32_t rad, int32_t wrap, int32_t dil) {
  if (wrap) return cq;
  if (dil == 1) return iclamp(cq - rad, 0, len - kernel);  // the same, without the divisions
  const int32_t g = cq % dil;
  const int32_t sub_len = (len - 1 - g) / dil + 1;
  return g + dil * iclamp(cq / dil - rad, 0, sub_len - kernel);
}

// Dilated window test for key coordinate ck against a query's anchor. Wrapped:
// ck = (c + dil * t) mod len for some |t| <= rad. Clamped: ck is one of the
// kernel cells anchor, anchor + dil, ..., anchor + (kernel - 1) * dil.
constexpr bool na_dil_ok(int32_t anchor, int32_t ck, int32_t len, int32_t kernel, int32_t rad, int32_t wrap,
                         int32_t dil) {
  if (wrap) {
    int32_t f = ck - anchor;
    f += f < 0 ? len : 0;          // forward distance in [0, len)
    const int32_t b = len - f;     // backward distance in (0, len]
    const int32_t reach = rad * dil;
    if (dil == 1) return f <= reach || b <= reach;  // every distance is a multiple of 1
    return (f <= reach && f % dil == 0) || (b <= reach && b % dil == 0);
  }
  const int32_t off = ck - anchor;
  if (dil == 1) return (uint32_t)off <= (uint32_t)(kernel - 1);
  return (uint32_t)off <= (uint32_t)((kernel - 1) * dil) && off % dil == 0;
}

// ---------------------------------------------------------------------------
// Grid-window bit masks (MASK_NA_GRID).
//
// A query's window is the product of one window per axis, so each lane keeps one
// bit mask per axis: bit c of an axis mask says whether coordinate c lies in the
// query's window along that axis (the dilated cells of na_dil_ok). For a key
// tile, one pass over the grid rows it touches ORs the column mask, shifted to
// where each row starts in the tile, into a tile mask wherever the row's plane and
// row bits are set; the shifts are the same for every lane. Each lane then takes
// the 16 bits of its own keys in each 32-key block.
constexpr bool na_grid_eligible(const NaGeom& g) {
  return g.grid_w >= 4 && g.grid_w <= 124 && g.grid_h <= 128 && g.grid_d <= 128;
}

// Per-axis window masks of one query, as pairs of 64-bit words (bit c of the pair
// is coordinate c). Named words, not arrays: an array indexed by a lane-dependent
// value would be placed in scratch memory.
struct GridMasks {
  uint64_t x0, x1;  // columns
  uint64_t y0, y1;  // rows of a plane
  uint64_t z0, z1;  // planes
};

// Window cells of coordinate c along one axis (len <= 128) as a 128-bit mask (lo, hi).
constexpr void na_axis_mask(int32_t c, int32_t len, int32_t kernel, int32_t rad, int32_t wrap, int32_t dil,
                            uint64_t& lo, uint64_t& hi) {
  lo = hi = 0;
  const int32_t anchor = na_dil_anchor(c, len, kernel, rad, wrap, dil);
  for (int32_t t = 0; t < kernel; ++t) {
    // wrapped: c + dil (t - rad) lies in (-len, 2 len) since (kernel - 1) dil < len
    int32_t cell = wrap ? c + dil * (t - rad) : anchor + dil * t;
    cell += cell < 0 ? len : 0;
    cell -= cell >= len ? len : 0;
    const uint64_t bit = 1ull << (cell & 63);
    lo |= cell < 64 ? bit : 0ull;
    hi |= cell < 64 ? 0ull : bit;
  }
}

constexpr GridMasks na_grid_masks(int32_t zq, int32_t yq, int32_t xq, const NaGeom& g) {
  GridMasks m{};
  na_axis_mask(xq, g.grid_w, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w, m.x0, m.x1);
  na_axis_mask(yq, g.grid_h, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h, m.y0, m.y1);
  na_axis_mask(zq, g.grid_d, g.kernel_d, g.rad_d, g.wrap_d, g.dil_d, m.z0, m.z1);
  return m;
}

// On a clamped axis the queries whose window holds key coordinate x share x's
// residue mod dil (na_dil_anchor takes the window inside that sub-grid of congruent
// cells) and, on the sub-grid, form the undilated reverse run of x's sub-grid
// coordinate: queries start, start + dil, ..., count of them.
constexpr Band na_clamped_reverse_run(int32_t x, int32_t len, int32_t kernel, int32_t rad, int32_t dil) {
  if (dil == 1) return na_band_reverse(x, x, len, kernel, rad, 0, 1);
  const int32_t g = x % dil, sub_len = (len - 1 - g) / dil + 1;
  const Band r = na_band_reverse(x / dil, x / dil, sub_len, kernel, rad, 0, 1);
  return Band{g + dil * r.start, r.count};
}

// The reverse relation, for the backward: bit c of an axis mask says whether the
// window of query coordinate c holds key coordinate x. Wrapped windows are
// symmetric (c + dil * t = x mod L with |t| <= r), so it is the window of x itself;
// a clamped one is na_clamped_reverse_run.
constexpr void na_axis_reverse_mask(int32_t x, int32_t len, int32_t kernel, int32_t rad, int32_t wrap, int32_t dil,
                                    uint64_t& lo, uint64_t& hi) {
  if (wrap) {
    na_axis_mask(x, len, kernel, rad, wrap, dil, lo, hi);
    return;
  }
  lo = hi = 0;
  const Band run = na_clamped_reverse_run(x, len, kernel, rad, dil);
  for (int32_t u = 0; u < run.count; ++u) {
    const int32_t c = run.start + dil * u;
    const uint64_t bit = 1ull << (c & 63);
    lo |= c < 64 ? bit : 0ull;
    hi |= c < 64 ? 0ull : bit;
  }
}

constexpr GridMasks na_grid_reverse_masks(int32_t zk, int32_t yk, int32_t xk, const NaGeom& g) {
  GridMasks m{};
  na_axis_reverse_mask(xk, g.grid_w, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w, m.x0, m.x1);
  na_axis_reverse_mask(yk, g.grid_h, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h, m.y0, m.y1);
  na_axis_reverse_mask(zk, g.grid_d, g.kernel_d, g.rad_d, g.wrap_d, g.dil_d, m.z0, m.z1);
  return m;
}

// Bit c of a 128-bit mask (lo, hi), c < 128.
constexpr uint64_t bit128(uint64_t lo, uint64_t hi, int32_t c) { return ((c < 64 ? lo : hi) >> (c & 63)) & 1ull; }

// Bits o .. o + 31 of a 128-bit mask (lo, hi); bits below 0 or past 127 read as 0.
constexpr uint32_t mask_bits32(uint64_t lo, uint64_t hi, int32_t o) {
  if (o <= -32 || o >= 128) return 0u;
  if (o < 0) return (uint32_t)(lo << (-o));
  if (o < 64) return (uint32_t)((lo >> o) | (o > 32 ? hi << (64 - o) : 0ull));
  return (uint32_t)(hi >> (o - 64));
}

// Window of one query over a key tile of 32 * WORDS keys starting at grid row row0,
// column x0 (rows counted over all planes): bit i of w[i / 32] says whether key
// k0 + i lies in the window; keys past the last row read as 0. Every branch and
// shift depends on the tile only, not on the lane.
template <int WORDS>
constexpr void na_tile_window(const GridMasks& m, int32_t row0, int32_t x0, const NaGeom& g, uint32_t (&w)[WORDS]) {
  for (int i = 0; i < WORDS; ++i) w[i] = 0u;
  int32_t z = row0 / g.grid_h, y = row0 - z * g.grid_h;
  for (int32_t sh = -x0; sh < 32 * WORDS && z < g.grid_d; sh += g.grid_w) {  // sh: tile offset of the row's column 0
    const bool ok = (bit128(m.z0, m.z1, z) & bit128(m.y0, m.y1, y)) != 0;
    for (int i = 0; i < WORDS; ++i) {
      const int32_t o = 32 * i - sh;  // column at bit 0 of word i
      if (o > -32 && o < g.grid_w) w[i] |= ok ? mask_bits32(m.x0, m.x1, o) : 0u;
    }
    if (++y == g.grid_h) {
      y = 0;
      ++z;
    }
  }
}

// The 16 keys a lane holds in a 32-key MFMA block are block offsets 8g + 4*half +
// (0..3), g = 0..3; element r = 4g + j of the block. Gathers their bits from the
// block's word of a tile mask.
constexpr uint32_t lane_block_bits(uint32_t w, int32_t half) {
  const uint32_t v = w >> (4 * half);
  return (v & 0xFu) | ((v >> 4) & 0xF0u) | ((v >> 8) & 0xF00u) | ((v >> 12) & 0xF000u);
}

// Bits [a, b) of a 128-bit column mask, in its 64-bit half h (bit i = column 64h + i).
constexpr uint64_t col_range_bits(int32_t a, int32_t b, int32_t h) {
  const int32_t lo = imax(a - 64 * h, 0), hi = imin(b - 64 * h, 64);
  if (hi <= lo) return 0;
  const uint64_t m = hi - lo == 64 ? ~0ull : ((1ull << (hi - lo)) - 1);
  return m << lo;
}

// Column window of a query in column cq of a grid of width W <= 128, as a
// 128-bit mask (two halves): bit x set iff na_axis_ok(cq, x, W, kernel, rad, wrap).
constexpr void na_col_window(int32_t cq, int32_t W, int32_t kernel, int32_t rad, int32_t wrap, uint64_t (&m)[2]) {
  int32_t s = 0, e = 0, s2 = 0, e2 = 0;  // [s, e) and, for a wrapped window, [s2, e2)
  if (wrap) {
    s = imod(cq - rad, W);
    e = s + kernel;
    if (e > W) {
      s2 = 0;
      e2 = e - W;
      e = W;
    }
  } else {
    s = iclamp(cq - rad, 0, W - kernel);
    e = s + kernel;
  }
  for (int32_t h = 0; h < 2; ++h) m[h] = col_range_bits(s, e, h) | col_range_bits(s2, e2, h);
}

// Per-lane column bits of the block-masked neighbourhood kernel (grid width a
// multiple of 32, at most 128): bit 16 * (phase & 1) + r of bits[phase >> 1] says
// whether accumulator element r of a 32-key block starting at column 32 * phase
// lies in the window. Element r of half-wave `half` holds column
// 32 * phase + 8 * (r / 4) + 4 * half + r % 4, so each group of 4 elements is one
// aligned nibble of the window mask.
constexpr void na_col_bits(int32_t cq, int32_t half, int32_t W, int32_t kernel, int32_t rad, int32_t wrap,
                           int32_t phases, uint32_t (&bits)[2]) {
  uint64_t m[2] = {0, 0};
  na_col_window(cq, W, kernel, rad, wrap, m);
  bits[0] = bits[1] = 0;
  for (int32_t ph = 0; ph < 4; ++ph) {
    if (ph >= phases) break;
    for (int32_t g = 0; g < 4; ++g) {
      const int32_t pos = 32 * ph + 8 * g + 4 * half;  // multiple of 4: the nibble stays in one half
      const uint32_t nib = (uint32_t)(m[pos >> 6] >> (pos & 63)) & 0xFu;
      bits[ph >> 1] |= nib << ((ph & 1) * 16 + 4 * g);
    }
  }
}

// Cells of one residue mod the dilation. On a dilated axis (that, when wrapped, the
// dilation divides; with windows wider than one cell) the cells congruent to rho mod dil form a sub-grid on which every
// window is an undilated window: clamped, na_dil_anchor takes it inside that
// sub-grid; wrapped, it steps dil cells at a time around a cycle of len / dil of
// them. The row and patch kernels then take the rows (and the patch kernels, where
// needed, the columns) of a work-group from one sub-grid, whose bands count 2 rad
// cells of margin rather than 2 rad dil.
constexpr bool na_axis_strided(int32_t len, int32_t kernel, int32_t dil, int32_t wrap) {
  return kernel > 1 && dil > 1 && (!wrap || len % dil == 0);  // a one-cell window gains nothing
}

constexpr bool na_rows_strided(const NaGeom& g) { return na_axis_strided(g.grid_h, g.kernel_h, g.dil_h, g.wrap_h); }

// ---------------------------------------------------------------------------
// Query patches of 2D neighbourhood windows (MASK_NA_PATCH), dilated or not.
//
// A query tile of consecutive tokens spans whole grid rows, so its wavefronts
// score every key of the rows their windows reach, most of them outside every
// window (a 32-query run of one row against 64-column rows: 38 of 64 columns
// hold some window cell, and the tile's band of rows is the union over its two
// query rows). A patch of 8 rows x 16 columns instead reaches a band of rows
// (na_band over its rows) times a band of at most 32 columns (na_band over its
// columns). The work-group copies that rectangle into LDS once, each key row of
// it as one 32-key block (its column band, padded to 32 with keys read as zero
// and masked); wavefront w, holding patch rows 2w and 2w + 1, then scores only
// the key rows of its own rows' band, four blocks per step.
constexpr int32_t kPatchRows = 8, kPatchCols = 16, kPatchKeyCols = 32;

struct PatchBands {
  Band rows, cols;
};

constexpr PatchBands na_patch_bands(int32_t y0, int32_t x0, const NaGeom& g) {
  return PatchBands{
      na_band(y0, imin(y0 + kPatchRows, g.grid_h) - 1, g.grid_h, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h),
      na_band(x0, imin(x0 + kPatchCols, g.grid_w) - 1, g.grid_w, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w)};
}

// Groups of `per` cells along one axis of `len` cells: consecutive cells of one
// residue sub-grid when the axis is strided (na_axis_strided), else of the axis
// itself. Sub-grid cell u is axis cell rho + stride u, u < len.
struct AxisGroup {
  int32_t rho, stride, len, u0;
};

constexpr int32_t na_axis_groups(int32_t len, int32_t kernel, int32_t dil, int32_t wrap, int32_t per) {
  if (!na_axis_strided(len, kernel, dil, wrap)) return (int32_t)cdiv(len, per);
  int32_t n = 0;
  for (int32_t rho = 0; rho < dil; ++rho) n += (int32_t)cdiv((len - 1 - rho) / dil + 1, per);
  return n;
}

constexpr AxisGroup na_axis_group(int32_t len, int32_t kernel, int32_t dil, int32_t wrap, int32_t i, int32_t per) {
  if (!na_axis_strided(len, kernel, dil, wrap)) return AxisGroup{0, 1, len, i * per};
  for (int32_t rho = 0; rho < dil; ++rho) {
    const int32_t sub = (len - 1 - rho) / dil + 1, n = (int32_t)cdiv(sub, per);
    if (i < n || rho == dil - 1) return AxisGroup{rho, dil, sub, i * per};
    i -= n;
  }
  return AxisGroup{0, 1, len, 0};  // not reached (dil >= 1)
}

// Patch (py, px) of a plane: its rows and columns (AxisGroup per axis, patches of
// kPatchRows x kPatchCols sub-grid cells from (u0, v0)) and `geom`, the window
// geometry in the sub-grids' coordinates (a strided axis has its sub-grid's length
// and dilation 1). The patch kernels work in those coordinates throughout and map
// to the grid only to address tokens (patch_token, with the grid's row pitch).
struct PatchGroup {
  int32_t rho, stride, u0;      // rows
  int32_t rho_x, stride_x, v0;  // columns
  int32_t pitch;                // tokens per grid row
  NaGeom geom;
};

// Rows are always taken by residue where the axis allows (a row is a run of tokens
// either way). Columns only where consecutive ones would not fit, a forward or reverse
// column band past one 32-key block: columns dil apart cost coalescing (a 7x7 window
// of dilation 2, whose 28-column bands fit, ran 0.95x forward and 0.88x backward with
// them).
constexpr bool na_patch_cols_strided(const NaGeom& g) {
  if (!na_axis_strided(g.grid_w, g.kernel_w, g.dil_w, g.wrap_w)) return false;
  for (int32_t x0 = 0; x0 < g.grid_w; x0 += kPatchCols) {
    const int32_t x1 = imin(x0 + kPatchCols, g.grid_w) - 1;
    if (na_band(x0, x1, g.grid_w, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w).count > kPatchKeyCols ||
        na_band_reverse(x0, x1, g.grid_w, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w).count > kPatchKeyCols)
      return true;
  }
  return false;
}

constexpr int32_t na_patch_row_groups(const NaGeom& g) {
  return na_axis_groups(g.grid_h, g.kernel_h, g.dil_h, g.wrap_h, kPatchRows);
}
constexpr int32_t na_patch_col_groups(const NaGeom& g, bool cols_strided) {
  return cols_strided ? na_axis_groups(g.grid_w, g.kernel_w, g.dil_w, g.wrap_w, kPatchCols)
                      : (int32_t)cdiv(g.grid_w, kPatchCols);
}

// cols_strided: na_patch_cols_strided(g), decided once per problem.
constexpr PatchGroup na_patch_group(const NaGeom& g, int32_t py, int32_t px, bool cols_strided) {
  const AxisGroup r = na_axis_group(g.grid_h, g.kernel_h, g.dil_h, g.wrap_h, py, kPatchRows);
  const AxisGroup c = cols_strided ? na_axis_group(g.grid_w, g.kernel_w, g.dil_w, g.wrap_w, px, kPatchCols)
                                   : AxisGroup{0, 1, g.grid_w, px * kPatchCols};
  PatchGroup p{r.rho, r.stride, r.u0, c.rho, c.stride, c.u0, g.grid_w, g};
  p.geom.grid_h = r.len;
  p.geom.dil_h = r.stride > 1 ? 1 : g.dil_h;
  p.geom.grid_w = c.len;
  p.geom.dil_w = c.stride > 1 ? 1 : g.dil_w;
  return p;
}

// Token of sub-grid cell (row y, column x) of a patch's plane.
constexpr int32_t patch_token(const PatchGroup& p, int32_t y, int32_t x) {
  return (p.rho + p.stride * y) * p.pitch + p.rho_x + p.stride_x * x;
}

// One plane; every column band within one 32-key block; a wrapped row band shorter
// than the axis (so the band of a wavefront's two rows is one run of its
// work-group's band); and every row band, plus the 3 rows a wavefront's last step
// of four may read past it, within the kernel's `lds_rows`.
constexpr bool na_patch_eligible(const NaGeom& g, int32_t lds_rows) {
  if (g.grid_d != 1) return false;
  const bool cs = na_patch_cols_strided(g);
  for (int32_t px = 0, n = na_patch_col_groups(g, cs); px < n; ++px) {
    const PatchGroup pg = na_patch_group(g, 0, px, cs);
    if (na_patch_bands(0, pg.v0, pg.geom).cols.count > kPatchKeyCols) return false;
  }
  for (int32_t py = 0, n = na_patch_row_groups(g); py < n; ++py) {
    const PatchGroup pr = na_patch_group(g, py, 0, cs);
    const Band rows = na_patch_bands(pr.u0, 0, pr.geom).rows;
    if (rows.count + 3 > lds_rows || (pr.geom.wrap_h && rows.count >= pr.geom.grid_h)) return false;
  }
  return true;
}

// Backward of the patch kernel: dK and dV of an 8 x 16 patch of keys over the
// rectangle of queries whose windows reach them (na_band_reverse per axis).
constexpr PatchBands na_patch_reverse_bands(int32_t y0, int32_t x0, const NaGeom& g) {
  return PatchBands{
      na_band_reverse(y0, imin(y0 + kPatchRows, g.grid_h) - 1, g.grid_h, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h),
      na_band_reverse(x0, imin(x0 + kPatchCols, g.grid_w) - 1, g.grid_w, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w)};
}

// Bits over the cells of band b (start, mod len; count <= 32) of one axis for the
// coordinate c of a lane: bit i set iff the pair is in the window, with the lane as
// the query and cell i as the key (reverse = false) or the other way round.
constexpr uint32_t band_window_bits(int32_t c, Band b, int32_t len, int32_t kernel, int32_t rad, int32_t wrap,
                                    int32_t dil, bool reverse) {
  uint32_t m = 0;
  if (dil == 1) {  // the undilated predicate: compares only (the dilated one divides by dil)
    for (int32_t i = 0; i < b.count; ++i) {
      int32_t x = b.start + i;
      x -= x >= len ? len : 0;
      const bool ok = reverse ? na_axis_ok(x, c, len, kernel, rad, wrap) : na_axis_ok(c, x, len, kernel, rad, wrap);
      m |= (uint32_t)ok << i;
    }
    return m;
  }
  if (wrap || !reverse) {
    // the window's kernel cells, dil apart (a wrapped window is symmetric, so also its reverse),
    // placed at their offsets in the band; no cell repeats ((kernel - 1) * dil < len)
    const int32_t first = wrap ? c - rad * dil : na_dil_anchor(c, len, kernel, rad, wrap, dil);
    for (int32_t t = 0; t < kernel; ++t) {
      int32_t cell = first + dil * t;  // within (-len, 2 len)
      cell += cell < 0 ? len : 0;
      cell -= cell >= len ? len : 0;
      int32_t i = cell - b.start;
      i += i < 0 ? len : 0;
      m |= i < b.count ? uint32_t{1} << i : 0u;
    }
    return m;
  }
  const Band run = na_clamped_reverse_run(c, len, kernel, rad, dil);  // clamped and dilated: the queries that see c
  for (int32_t u = 0; u < run.count; ++u) {
    const int32_t i = run.start + dil * u - b.start;  // a clamped band does not wrap
    m |= (uint32_t)i < (uint32_t)b.count ? uint32_t{1} << i : 0u;
  }
  return m;
}

// The backward patch kernels' condition, for the key rectangles of the dQ kernel
// (reverse = false) or the query rectangles of the dK/dV kernel (reverse = true):
// one plane; every column band within one 32-token block; a wrapped row band
// shorter than the axis (so a wavefront's band is one run of its work-group's);
// every row band within `lds_rows`. Both kernels walk only their wavefront's band
// rows, so no rows past a band are read.
constexpr bool na_patch_bwd_eligible(const NaGeom& g, int32_t lds_rows, bool reverse) {
  if (g.grid_d != 1 || lds_rows <= 0) return false;
  const bool cs = na_patch_cols_strided(g);
  for (int32_t px = 0, n = na_patch_col_groups(g, cs); px < n; ++px) {
    const PatchGroup pg = na_patch_group(g, 0, px, cs);
    const PatchBands b = reverse ? na_patch_reverse_bands(0, pg.v0, pg.geom) : na_patch_bands(0, pg.v0, pg.geom);
    if (b.cols.count > kPatchKeyCols) return false;
  }
  for (int32_t py = 0, n = na_patch_row_groups(g); py < n; ++py) {
    const PatchGroup pr = na_patch_group(g, py, 0, cs);
    const Band rows = (reverse ? na_patch_reverse_bands(pr.u0, 0, pr.geom) : na_patch_bands(pr.u0, 0, pr.geom)).rows;
    if (rows.count > lds_rows || (pr.geom.wrap_h && rows.count >= pr.geom.grid_h)) return false;
  }
  return true;
}

// ---------------------------------------------------------------------------
// Grid rows of narrow grids (MASK_NA_ROWS).
//
// On a grid at most 32 wide, a wavefront holds one grid row of queries (lane column
// = grid column; lanes past the width idle) and a work-group 4 rows of one plane
// (consecutive, or of one residue mod the dilation: RowGroup). Every key row is then
// one 32-key block (its columns, padded with keys read as zero), so a query's window
// bits in any block are its own column bits, and whether a key row (plane, row) lies
// in the window is the same for every lane of a wavefront. The work-group streams the
// planes its windows reach (na_band of its plane) through two LDS stages, each the
// band of key rows of its 4 rows (na_row_group); each wavefront scores only its own
// visible rows of a stage.
constexpr int32_t kRowsGroup = 4;

// The rows of a group. With strided rows (na_rows_strided) a group takes 4
// consecutive rows of one residue sub-grid and its band is 4 + 2 rad sub-grid rows
// rather than 4 + 2 rad dil grid rows. Otherwise (dilation 1, or a wrapped axis the dilation does not divide) the
// sub-grid is the whole axis (rho 0, stride 1). Wavefront w holds grid row
// rho + stride (u0 + w) while u0 + w < len; band row r is the grid row of sub-grid
// cell (band.start + r) mod len.
struct RowGroup {
  int32_t rho, stride, len, u0;
  Band band;
};

// Groups per plane (both row kernels).
constexpr int32_t na_row_groups(const NaGeom& g) {
  return na_axis_groups(g.grid_h, g.kernel_h, g.dil_h, g.wrap_h, kRowsGroup);
}

// Group i of a plane with the band of rows its windows reach (reverse = false: the key
// rows of its query rows; true: the query rows whose windows reach its key rows).
constexpr RowGroup na_row_group(const NaGeom& g, int32_t i, bool reverse) {
  const AxisGroup a = na_axis_group(g.grid_h, g.kernel_h, g.dil_h, g.wrap_h, i, kRowsGroup);
  const int32_t dil = a.stride > 1 ? 1 : g.dil_h;  // a residue sub-grid holds undilated windows
  const int32_t u1 = imin(a.u0 + kRowsGroup, a.len) - 1;
  const Band band = reverse ? na_band_reverse(a.u0, u1, a.len, g.kernel_h, g.rad_h, g.wrap_h, dil)
                            : na_band(a.u0, u1, a.len, g.kernel_h, g.rad_h, g.wrap_h, dil);
  return RowGroup{a.rho, a.stride, a.len, a.u0, band};
}

// Grid row of band row r of a group.
constexpr int32_t row_group_row(const RowGroup& rg, int32_t r) {
  int32_t u = rg.band.start + r;
  u -= u >= rg.len ? rg.len : 0;
  return rg.rho + rg.stride * u;
}

// At most 32 columns (one block per key row), axes of at most 128 cells (the
// 128-bit window masks), and every group's band of rows within the kernel's
// `lds_rows` rows per stage.
constexpr bool na_rows_eligible(const NaGeom& g, int32_t lds_rows) {
  if (g.grid_w > 32 || g.grid_h > 128 || g.grid_d > 128) return false;
  for (int32_t i = 0, n = na_row_groups(g); i < n; ++i)
    if (na_row_group(g, i, false).band.count > lds_rows) return false;
  return true;
}

// The dK/dV row kernel's condition: na_rows_eligible's grid limits, and every
// group's band of query rows (dK and dV of 4 key rows of one plane per work-group,
// the query rows whose windows reach them streamed) within `lds_rows` rows per stage.
constexpr bool na_rows_reverse_eligible(const NaGeom& g, int32_t lds_rows) {
  if (g.grid_w > 32 || g.grid_h > 128 || g.grid_d > 128) return false;
  for (int32_t i = 0, n = na_row_groups(g); i < n; ++i)
    if (na_row_group(g, i, true).band.count > lds_rows) return false;
  return true;
}

// 16-bit mask of the accumulator elements of one 32-key block that a lane keeps
// when the keys it may see end at `lim` keys past the lane's first key of the
// block: element r holds key offset 8 * (r / 4) + r % 4, kept iff <= lim (so
// lim < 0 keeps none and lim >= 27 keeps all). Used for the causal diagonal
// (lim = query - first key) and the ragged last tile (lim = N - 1 - first key).
constexpr uint32_t limit_bits(int32_t lim) {
  uint32_t m = 0;
  for (int32_t g = 0; g < 4; ++g) m |= ((1u << iclamp(lim - 8 * g + 1, 0, 4)) - 1u) << (4 * g);
  return m;
}

// Map a work-group index to (head, query tile).
//
// Work-groups are dispatched round-robin over the 8 XCDs of the chip, each
// with its own L2. For equal-length work items the remap gives each XCD a
// contiguous block of logical items, so the query tiles of one head (which
// share its K and V) land on the same L2.
struct WorkItem {
  int32_t bh, qtile;
};

// Equal-length items: XCD x runs the contiguous block of logical items
// [x * n / 8, (x + 1) * n / 8); a tail that does not divide keeps dispatch order.
constexpr int32_t xcd_contiguous(int32_t wg, int32_t n) {
  const int32_t per_xcd = n / 8;
  return wg < per_xcd * 8 ? (wg % 8) * per_xcd + wg / 8 : wg;
}

// Causal items differ in length: query tile t of the forward (and of the dQ
// kernel) sees t + 1 key tiles, key tile t of the dK/dV kernel is seen by
// n - t query tiles. They are dispatched longest first (rank 0 = longest) in
// superblocks of 8 * group heads; within a superblock the order is rank major,
// head minor. Round-robin dispatch then keeps head h on XCD h % 8 (in every
// superblock whose head count is a multiple of 8) and spreads long and short
// items evenly over the XCDs. `group` heads per XCD are chosen so that their
// items fill the XCD's resident work-group slots (causal_group): the streamed
// tiles of only those heads share its L2 at a time, and the next superblock's
// longest items take the slots that the current one's shortest items free first.
struct RankedItem {
  int32_t bh, rank;
};

constexpr RankedItem causal_item(int32_t wg, int32_t n_tiles, int32_t BH, int32_t group) {
  const int32_t span = 8 * group;              // heads per superblock
  const int32_t per_block = span * n_tiles;    // items per superblock
  const int32_t blk = wg / per_block;
  const int32_t idx = wg - blk * per_block;
  const int32_t heads = BH - blk * span < span ? BH - blk * span : span;  // the last may hold fewer
  return RankedItem{blk * span + idx % heads, idx / heads};
}

// Heads per XCD whose n_tiles items fill its resident slots (cus / 8 CUs, wgs_per_cu
// work-groups each); at least 1.
constexpr int32_t causal_group(int32_t n_tiles, int32_t cus, int32_t wgs_per_cu) {
  const int32_t slots = cus / 8 * wgs_per_cu;
  return n_tiles > 0 && slots / n_tiles > 1 ? slots / n_tiles : 1;
}

constexpr WorkItem work_item(int mask, int32_t wg, int32_t n_wg, int32_t n_qtiles, int32_t BH, int32_t group) {
  if (mask == MASK_CAUSAL) {
    const RankedItem r = causal_item(wg, n_qtiles, BH, group);
    return WorkItem{r.bh, n_qtiles - 1 - r.rank};
  }
  const int32_t logical = xcd_contiguous(wg, n_wg);
  return WorkItem{logical / n_qtiles, logical % n_qtiles};
}

// ---------------------------------------------------------------------------
// Remainder split of the unmasked problem.
//
// One work-group per query tile leaves the chip unevenly loaded when the tile
// count is not a multiple of the CU count: 320 tiles on 256 CUs give 64 CUs
// two tiles while 192 CUs hold one. Here the first `full` tiles (whole rounds
// of one tile per CU) keep one work-group each, and each of the `rem` remaining
// tiles is cut along its key tiles into `parts` equal ranges, each run by a
// work-group of its own that sits beside a whole-tile work-group on some CU.
// With rem * parts close to the CU count every CU then does about the same
// work. A part ends in a partial result (the unnormalised output rows, the
// running maximum and the row sums over its keys) in a workspace slot; the
// work-group of the tile's last part to finish (an arrival counter per split
// tile) combines the parts exactly (the rescaling by 2^(m_i - m) of the
// running-softmax paragraph of PhotoRoom's xformers post, applied across
// parts) and writes the tile, while whole tiles are still running.
//
// Tiles are numbered head-major (tile = bh * n_qtiles + qtile). Work-group g <
// full takes a whole tile; the other work-groups take the rem * parts parts in
// part-major order, XCD-contiguously (an XCD holds one key range of consecutive
// tiles). Part p of tile full + r covers key tiles [p * n_kv / parts, (p + 1) *
// n_kv / parts) and writes workspace slot r * parts + p.
struct SplitPlan {
  int32_t full;   // whole tiles (work-groups 0 .. full - 1)
  int32_t rem;    // split tiles; 0 = no split
  int32_t parts;  // parts per split tile
  constexpr int32_t groups() const { return full + rem * parts; }
  constexpr int32_t slots() const { return rem * parts; }
};

// A part spans at least this many key tiles; no tile is cut into more parts.
constexpr int32_t kMinPartTiles = 2;
constexpr int32_t kMaxParts = 8;

constexpr KvRun part_run(int32_t n_kv, int32_t parts, int32_t p) {
  const int32_t a = (int32_t)((int64_t)p * n_kv / parts), b = (int32_t)((int64_t)(p + 1) * n_kv / parts);
  return KvRun{a, b - a};
}

// The split for n_tiles query tiles of n_kv key tiles on a device with `cus`
// CUs: rem = 0 (no split) unless the problem is unmasked, leaves a remainder
// after whole rounds of one tile per CU, and is at most one round deep (deeper
// problems are balanced by the dispatcher refilling CUs as tiles finish).
constexpr SplitPlan split_plan(int mask, int64_t n_tiles, int32_t n_kv, int32_t cus) {
  SplitPlan p{(int32_t)(n_tiles < INT32_MAX ? n_tiles : INT32_MAX), 0, 0};
  if (mask != MASK_NONE || cus < 1 || n_tiles < 1 || n_tiles >= 2 * (int64_t)cus) return p;
  const int32_t full = n_tiles >= cus ? cus : 0;
  const int32_t rem = (int32_t)(n_tiles - full);
  if (rem == 0) return p;
  int32_t parts = cus / rem;
  if (parts > n_kv / kMinPartTiles) parts = n_kv / kMinPartTiles;
  if (parts > kMaxParts) parts = kMaxParts;
  if (parts < 2) return p;
  return SplitPlan{full, rem, parts};
}

}  // namespace attn
