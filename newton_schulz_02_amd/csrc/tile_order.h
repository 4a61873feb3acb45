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

// ---- tail split -----------------------------------------------------------------------
// A launch of T tiles on P compute units (one workgroup per unit at a time) runs F = T / P
// whole rounds; the R = T - F P tiles left over would hold R units for a whole tile time
// while the other P - R wait.  With the tail split the first F P workgroups run whole tiles
// as usual and the R tail tiles are cut along the contraction into pieces, one workgroup
// per piece:
//   kSplitEqual  (R <= P / 2): every tail tile is cut into c equal pieces (c R workgroups,
//                the c pieces of a tile and neighbouring tiles on one XCD); the tail takes
//                about 1/c of a tile time.
//   kSplitUneven (R > P / 2):  every tail tile is cut once, at s = K n / (n + 1) with
//                n = ceil(R / (P - R)).  Each XCD takes a run of tail tiles and gets the
//                workgroups of their first pieces [0, s) before those of their second pieces
//                [s, K): its units start on the long first pieces, and the rest run about n
//                second pieces each, so the tail takes about n / (n + 1) of a tile time.
// Pieces start and end on multiples of `unit` k-steps (the kernels' stage counts divide
// it), so each piece runs whole blocks of stages.  The last piece of a tile to finish adds
// the others' partial sums, in piece order, and stores the tile.
enum SplitMode : int32_t { kSplitNone = 0, kSplitEqual = 1, kSplitUneven = 2 };
constexpr int kMaxPieces = 8;

// The piece run by tail workgroup j (j in [0, wgs), in launch order; workgroup j runs on
// XCD j mod kXcds).  Returns false for a workgroup with no piece (padding of the uneven
// mode's deal); else tail tile t, piece `piece` of `pieces`.
MUON_HD bool split_item(int mode, int R, int wgs, int c, int j, int& t, int& piece, int& pieces) {
  t = 0;
  piece = 0;
  pieces = 1;
  if (mode == kSplitEqual) {
    const int u = xcd_remap(j, wgs);
    pieces = c;
    t = u / c;
    piece = u % c;
    return t < R;
  }
  if (mode != kSplitUneven) return false;
  // wgs is a multiple of 2 kXcds: XCD x runs wgs / kXcds workgroups, the first pieces of
  // tail tiles [x m, x m + m) and then their second pieces, m = wgs / (2 kXcds).
  const int m = wgs / (2 * kXcds);
  const int x = j % kXcds, i = j / kXcds;
  pieces = 2;
  piece = i < m ? 0 : 1;
  t = x * m + (i < m ? i : i - m);
  return t < R;
}

// K-step range [k0, k1) of piece `piece` of `pieces` of a tile of K k-steps.  Cuts fall on
// multiples of unit; the last piece ends at K (which need not be one).  n is the uneven
// mode's second pieces per unit.
MUON_HD void split_range(int mode, int n, int K, int unit, int piece, int pieces, int& k0, int& k1) {
  const int u = K / unit;
  if (mode == kSplitEqual) {
    k0 = unit * (piece * u / pieces);
    k1 = piece == pieces - 1 ? K : unit * ((piece + 1) * u / pieces);
    return;
  }
  if (mode == kSplitUneven) {
    int s = (u * n + (n + 1) / 2) / (n + 1);
    if (s > u - 1) s = u - 1;
    if (s < 1) s = 1;
    if (s > u) s = u;
    k0 = piece == 0 ? 0 : unit * s;
    k1 = piece == 0 ? unit * s : K;
    return;
  }
  k0 = 0;
  k1 = K;
}

// Split of a launch of T tiles over P units: mode, pieces per tail tile (equal mode) or
// second pieces per workgroup (uneven mode), the workgroups of the whole tiles and of the
// tail.  kmin is the smallest k-step count of the tail tiles; no piece is made shorter
// than two units.
struct SplitPlan {
  int mode = kSplitNone;
  int c = 1;          // equal mode: pieces per tail tile
  int n = 1;          // uneven mode: second pieces per unit (sets the cut)
  int dp_tiles = 0;   // whole tiles, run first
  int tail = 0;       // tail tiles R
  int tail_wgs = 0;   // workgroups of the tail pieces
  int slots = 0;      // partial-sum slots (one per piece of a tail tile)
};

MUON_HD SplitPlan plan_split(int T, int P, int kmin, int unit) {
  SplitPlan s;
  s.dp_tiles = T;
  if (T <= 0 || P <= 1) return s;
  const int R = T % P;
  const int units = kmin / unit;
  if (R == 0 || units < 4) return s;
  if (2 * R <= P) {
    int c = P / R;
    if (c > kMaxPieces) c = kMaxPieces;
    if (c > units / 2) c = units / 2;
    if (c < 2) return s;
    s.mode = kSplitEqual;
    s.c = c;
    s.tail_wgs = c * R;
    s.slots = c * R;
  } else {
    const int n = (R + (P - R) - 1) / (P - R);
    int k0, k1;
    split_range(kSplitUneven, n, kmin, unit, 0, 2, k0, k1);
    const int first = k1, second = n * (kmin - k1);
    // Worth it only if the longer side of the tail is clearly shorter than a whole tile.
    if (10 * (first > second ? first : second) > 9 * kmin) return s;
    s.mode = kSplitUneven;
    s.n = n;
    s.tail_wgs = (2 * R + 2 * kXcds - 1) / (2 * kXcds) * (2 * kXcds);
    s.slots = 2 * R;
  }
  s.dp_tiles = T - R;
  s.tail = R;
  return s;
}

}  // namespace muon
