// Tile orders of the grouped MFMA kernel, shared by the kernel and a host-side test hook.
//
// 1. XCD remap.  MI355X has 8 XCDs (32 CUs each), each with its own L2; the dispatcher
//    sends workgroup w to XCD (w mod 8).  xcd_remap() deals logical tiles to the XCDs in
//    chunks of kXcdChunk consecutive tiles, round robin: the tiles one XCD runs at once
//    are consecutive (they share operand panels in its L2), all XCDs work on the same
//    window of about 8 * kXcdChunk tiles (whose panels fit the shared last-level cache),
//    and tiles of different cost are spread over all XCDs.
// 2. Banded order inside one matrix.  Tile rows are grouped in bands of kBand rows and a
//    band is walked column by column, so consecutive tiles reuse the same kBand A panels
//    and step through B panels one at a time.  tri_band_decode() does this over the lower
//    triangle (ti >= tj), full_band_decode() over a full TM x TN grid.
#pragma once

#if defined(__HIP__)
#define MUON_HD __attribute__((host)) __attribute__((device)) inline
#else
#define MUON_HD inline
#endif

namespace muon {

constexpr int kXcds = 8;
constexpr int kXcdChunk = 32;
constexpr int kBand = 4;

// Logical tile index of workgroup w in a grid of `total` workgroups.  The workgroups past the
// last whole round of kXcds chunks (all of them in a launch of fewer than kXcds * kXcdChunk
// tiles) split the remaining tiles into one contiguous block per XCD, so they keep their L2
// locality too.
MUON_HD int xcd_remap(int w, int total) {
  const int round = kXcds * kXcdChunk;
  const int whole = total / round * round;
  if (w < whole) {
    const int x = w % kXcds, i = w / kXcds;
    return (i / kXcdChunk) * round + x * kXcdChunk + i % kXcdChunk;
  }
  // Tail: workgroups whole + j (j = 0 .. rest-1); XCD x gets q + (x < r) of them.
  const int j = w - whole, rest = total - whole;
  const int q = rest / kXcds, r = rest % kXcds;
  const int x = j % kXcds, i = j / kXcds;
  return whole + (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// t in [0, T(T+1)/2) -> (ti, tj), ti >= tj, for a T x T tile grid.
// Band s (rows 4s .. 4s+h-1, h = min(4, T-4s)) holds 4s*h tiles left of the diagonal block,
// walked column-major, then the h(h+1)/2 tiles of its diagonal block, column by column.
// Full bands before band s hold 8 s^2 + 2 s tiles.
MUON_HD void tri_band_decode(int t, int T, int& ti, int& tj) {
  int s = 0;
  while (8 * (s + 1) * (s + 1) + 2 * (s + 1) <= t && 4 * (s + 1) < T) ++s;
  int u = t - (8 * s * s + 2 * s);
  const int h = (T - 4 * s) < kBand ? (T - 4 * s) : kBand;
  if (u < 4 * s * h) {
    tj = u / h;
    ti = 4 * s + u % h;
  } else {
    int v = u - 4 * s * h;
    int c = 0;
    while (v >= h - c) {
      v -= h - c;
      ++c;
    }
    tj = 4 * s + c;
    ti = 4 * s + c + v;
  }
}

// ---- non-square tiles (TM rows x TN columns) ----------------------------------------
// A symmetric m x m output is computed on the tiles that hold an element on or below the
// diagonal (each such element lies in exactly one of them).

MUON_HD int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

// Column tiles of tile row ti that reach the diagonal (column tiles tj with TN tj <= the
// tile row's last row); it never decreases with ti.
MUON_HD int sym_row_tiles(int ti, int m, int TM, int TN) {
  const int last_row = (TM * ti + TM - 1 < m - 1) ? TM * ti + TM - 1 : m - 1;
  const int k = last_row / TN + 1;
  const int tn = ceil_div_i(m, TN);
  return k < tn ? k : tn;
}

// Number of tiles of a symmetric m x m output.
MUON_HD int sym_tiles(int m, int TM, int TN) {
  int n = 0;
  const int tm = ceil_div_i(m, TM);
  for (int ti = 0; ti < tm; ++ti) n += sym_row_tiles(ti, m, TM, TN);
  return n;
}

// t in [0, sym_tiles(m, TM, TN)) -> (ti, tj).  Bands of kBand tile rows; inside a band,
// column by column, the band rows whose tile row reaches that column (a suffix of the
// band).  With TM == TN this is tri_band_decode's order.
MUON_HD void sym_decode(int t, int m, int TM, int TN, int& ti, int& tj) {
  const int tm = ceil_div_i(m, TM);
  const int tn = ceil_div_i(m, TN);
  int r0 = 0;
  int h = tm < kBand ? tm : kBand;
  for (;;) {
    int cnt = 0;
    for (int r = 0; r < h; ++r) cnt += sym_row_tiles(r0 + r, m, TM, TN);
    if (t < cnt || r0 + h >= tm) break;
    t -= cnt;
    r0 += h;
    h = tm - r0 < kBand ? tm - r0 : kBand;
  }
  ti = r0;
  tj = 0;
  for (int c = 0; c < tn; ++c) {
    int k = 0;  // band rows whose tile row reaches column c
    for (int r = 0; r < h; ++r) k += sym_row_tiles(r0 + r, m, TM, TN) > c ? 1 : 0;
    if (t < k) {
      tj = c;
      ti = r0 + (h - k) + t;
      return;
    }
    t -= k;
  }
}

// t in [0, TM*TN) -> (ti, tj): bands of kBand tile rows, each walked column-major.
MUON_HD void full_band_decode(int t, int TM, int TN, int& ti, int& tj) {
  const int s = t / (kBand * TN);
  const int u = t - s * kBand * TN;
  const int h = (TM - kBand * s) < kBand ? (TM - kBand * s) : kBand;
  tj = u / h;
  ti = kBand * s + u % h;
}

}  // namespace muon
