// Integer mask engine shared by the kernels, the debug exports and the host.
//
// Visibility of key j from query row i (all signed 32-bit integers):
//   i < L and j < L                               (sequence lengths, right padding:
//                                                  TE "JAX: Single-GPU Attention" sec. 1)
//   and (not causal or j <= i)                    (codelab "Speed up attention ...",
//                                                  section 7, lower-triangular mask)
//   and (wl < 0 or j >= i - wl)                   (window_size (left, right), TE page
//   and (wr < 0 or j <= i + wr)                    section 2; inclusive, -1 unbounded)
//
// Every visible row i < L sees at least key j = i, and the visible keys of a
// row form one interval whose two ends never decrease with i.  So the keys
// visible from any row of a block of consecutive rows form one interval,
// computed in closed form below, and likewise for the rows that see any key
// of a block of consecutive keys.  Tiles outside those intervals are skipped,
// tiles inside whose every pair is visible need no per-element predicate.
#pragma once

#ifdef __HIPCC__
#define ME_HD __host__ __device__ __forceinline__
#else
#define ME_HD inline
#endif

namespace sdpa {

enum TileClass : int { TILE_SKIP = 0, TILE_PARTIAL = 1, TILE_FULL = 2 };

struct MaskSpec {
  int L;       // valid length of this batch, in [0, S]
  int causal;  // 1 = j <= i
  int wl;      // left window, -1 = unbounded (normalised: -1 or < S)
  int wr;      // right window, -1 = unbounded (normalised: -1 or < S)
};

ME_HD int me_min(int a, int b) { return a < b ? a : b; }
ME_HD int me_max(int a, int b) { return a > b ? a : b; }

// A window of S or more is unbounded for a length-S sequence; normalising it
// to -1 keeps i +- w inside int range.
ME_HD int normalise_window(int w, int S) { return (w < 0 || w >= S) ? -1 : w; }

ME_HD MaskSpec make_mask(int L, int S, int causal, int wl, int wr) {
  MaskSpec m;
  m.L = me_min(me_max(L, 0), S);
  m.causal = causal ? 1 : 0;
  m.wl = normalise_window(wl, S);
  m.wr = normalise_window(wr, S);
  return m;
}

ME_HD bool visible(const MaskSpec& m, int i, int j) {
  return i < m.L && j < m.L && (!m.causal || j <= i) && (m.wl < 0 || j >= i - m.wl) &&
         (m.wr < 0 || j <= i + m.wr);
}

// Keys visible from any row in [i0, i1]: [lo, hi].  Returns false if none.
ME_HD bool key_range(const MaskSpec& m, int i0, int i1, int& lo, int& hi) {
  if (i0 >= m.L || i1 < i0) return false;
  i1 = me_min(i1, m.L - 1);
  lo = m.wl >= 0 ? me_max(0, i0 - m.wl) : 0;
  hi = m.L - 1;
  if (m.causal) hi = me_min(hi, i1);
  if (m.wr >= 0) hi = me_min(hi, i1 + m.wr);
  return lo <= hi;
}

// Rows that see any key in [j0, j1]: [lo, hi].  Returns false if none.
ME_HD bool query_range(const MaskSpec& m, int j0, int j1, int& lo, int& hi) {
  if (j0 >= m.L || j1 < j0) return false;
  j1 = me_min(j1, m.L - 1);
  lo = 0;
  if (m.causal) lo = me_max(lo, j0);
  if (m.wr >= 0) lo = me_max(lo, j0 - m.wr);
  hi = m.L - 1;
  if (m.wl >= 0) hi = me_min(hi, j1 + m.wl);
  return lo <= hi;
}

// Class of the tile rows [i0, i0+bm) x keys [j0, j0+bn).
ME_HD int tile_class(const MaskSpec& m, int i0, int bm, int j0, int bn) {
  int lo, hi;
  if (!key_range(m, i0, i0 + bm - 1, lo, hi)) return TILE_SKIP;
  const int i1 = i0 + bm - 1, j1 = j0 + bn - 1;
  if (j1 < lo || j0 > hi) return TILE_SKIP;
  const bool full = i1 < m.L && j1 < m.L && (!m.causal || j1 <= i0) &&
                    (m.wl < 0 || j0 >= i1 - m.wl) && (m.wr < 0 || j1 <= i0 + m.wr);
  return full ? TILE_FULL : TILE_PARTIAL;
}

// Key tiles f0 .. f1 (tile t holds keys t*bn .. t*bn+bn-1) that every row of
// [i0, i0+bm) sees in full, i.e. the tiles tile_class calls FULL for that row
// block; false when there are none.  Rows see keys from max(0, row-wl) to
// min(L-1, row [causal], row+wr); both bounds grow with the row, so the keys
// all rows see run from the last row's lower bound to the first row's upper.
ME_HD bool full_key_tiles(const MaskSpec& m, int i0, int bm, int bn, int& f0, int& f1) {
  const int i1 = i0 + bm - 1;
  if (i1 >= m.L) return false;
  int jlo = 0, jhi = m.L - 1;
  if (m.wl >= 0 && i1 - m.wl > jlo) jlo = i1 - m.wl;
  if (m.causal && i0 < jhi) jhi = i0;
  if (m.wr >= 0 && i0 + m.wr < jhi) jhi = i0 + m.wr;
  f0 = (jlo + bn - 1) / bn;
  f1 = (jhi + 1) / bn - 1;
  return f0 <= f1;
}

// 32-row blocks of the stored-dS workspace's slab for the 128-key tile kt
// (keys 128 kt .. 128 kt + 127): the rows that see any of its keys, from the
// first one rounded down to a multiple of 64 to the end of the last one's
// 64-row step; 0 when no row sees the tile.  Slabs are sized with the mask at
// the full length S (a shorter valid length only drops rows from the end, and
// leaves the first row in place), one slab per tile back to back.
ME_HD int ds_tile_blocks(const MaskSpec& m_full, int kt) {
  int lo, hi;
  if (!query_range(m_full, kt * 128, kt * 128 + 127, lo, hi)) return 0;
  return 2 * (hi / 64 - lo / 64 + 1);
}

}  // namespace sdpa
