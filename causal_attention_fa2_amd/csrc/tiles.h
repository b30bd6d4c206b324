// tiles.h -- integer mask logic shared by the host launchers and the kernels.
//
// Visibility follows the causal / sliding-window definition ("KYNETRA FOUNDRY" page, decoder-block
// paragraph for the strict left-to-right mask; "CUDA-LLM: A GitHub Repository for Development",
// section "The custom CUDA kernel", for the single window parameter and for fewer queries than
// keys). Everything here works on POSITIONS: with Sq query rows and S >= Sq keys the queries are
// the last Sq positions, so query row r stands at position i = r + (S - Sq), and
//   visible(i, j) = i < S && j < S && (!causal || j <= i) && (window == 0 || i - j < window).
// (i < S holds exactly when r < Sq.) The kernels add the offset S - Sq to their row indices.
// A rectangular block of rows [r0, r1] x keys [c0, c1] is EMPTY if no pair in it is visible (the
// kernels never touch it), FULL if every pair is visible and in range (no element mask needed),
// otherwise PARTIAL (element mask applied). Only integer arithmetic; no floating point decides
// anything here.
#ifndef ATTN_TILES_H_
#define ATTN_TILES_H_

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__ __forceinline__
#else
#define ATTN_HD inline
#endif

namespace fa {

ATTN_HD int imin_(int a, int b) { return a < b ? a : b; }
ATTN_HD int imax_(int a, int b) { return a > b ? a : b; }

ATTN_HD bool visible(int i, int j, int S, bool causal, int window) {
  return i < S && j < S && (!causal || j <= i) && (window == 0 || i - j < window);
}

// No visible pair in rows [r0, r1] x keys [c0, c1] (r0 <= r1, c0 <= c1, all >= 0).
ATTN_HD bool block_empty(int r0, int r1, int c0, int c1, int S, bool causal, int window) {
  if (r0 >= S || c0 >= S) return true;
  r1 = imin_(r1, S - 1);
  c1 = imin_(c1, S - 1);
  if (causal && c0 > r1) return true;                 // smallest key is after the last row
  if (window > 0 && r0 - c1 >= window) return true;   // largest key is out of the first row's window
  return false;
}

// Every pair in rows [r0, r1] x keys [c0, c1] is visible and inside [0, S).
ATTN_HD bool block_full(int r0, int r1, int c0, int c1, int S, bool causal, int window) {
  if (r1 >= S || c1 >= S) return false;
  if (causal && c1 > r0) return false;                // largest key must not pass the first row
  if (window > 0 && r1 - c0 >= window) return false;  // last row must still see the first key
  return true;
}

// Key tiles of width bc that hold any key visible to some position in [r0, r1] (r1 <= S - 1):
// tiles [*lo, *hi] (never empty: every position sees itself).
ATTN_HD void kv_tile_range(int r0, int r1, int S, int bc, bool causal, int window, int* lo, int* hi) {
  int jmax = causal ? r1 : S - 1;
  int jmin = window > 0 ? imax_(0, r0 - window + 1) : 0;
  *lo = jmin / bc;
  *hi = jmax / bc;
}

// Query tiles of height br (tile t = rows [t*br, t*br + br)) holding any query row that sees some
// key in [c0, c1] (c1 <= S - 1), the rows standing at positions row + off: tiles [*lo, *hi];
// *lo > *hi when no query sees these keys (they fall out of every window).
ATTN_HD void q_tile_range(int c0, int c1, int S, int off, int br, bool causal, int window, int* lo,
                          int* hi) {
  const int imin = imax_(causal ? c0 : 0, off) - off;
  const int imax = (window > 0 ? imin_(S - 1, c1 + window - 1) : S - 1) - off;
  if (imax < imin) {
    *lo = 1;
    *hi = 0;
    return;
  }
  *lo = imin / br;
  *hi = imax / br;
}

}  // namespace fa

#endif  // ATTN_TILES_H_
