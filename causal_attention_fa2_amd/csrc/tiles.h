// tiles.h -- integer mask logic shared by the host launchers and the kernels.
//
// Visibility follows the causal / sliding-window definition ("KYNETRA FOUNDRY" page, decoder-block
// paragraph for the strict left-to-right mask; "CUDA-LLM: A GitHub Repository for Development",
// section "The custom CUDA kernel", for the single window parameter and for fewer queries than
// keys; "KYNETRA FOUNDRY", Vaultecho paragraph, for the persistent sink tokens beside the window).
// Everything here works on POSITIONS: with Sq query rows and S >= Sq keys the queries are the last
// Sq positions, so query row r stands at position i = r + (S - Sq), and
//   visible(i, j) = i < S && j < S && (!causal || j <= i)
//                   && (window == 0 || i - j < window || j < sink).
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

// Key j against position i. Sink keys (j < sink) stay visible once the window has moved past them.
ATTN_HD bool visible(int i, int j, int S, bool causal, int window, int sink) {
  return i < S && j < S && (!causal || j <= i) && (window == 0 || i - j < window || j < sink);
}

// No visible pair in rows [r0, r1] x keys [c0, c1] (r0 <= r1, c0 <= c1, all >= 0).
ATTN_HD bool block_empty(int r0, int r1, int c0, int c1, int S, bool causal, int window, int sink) {
  if (r0 >= S || c0 >= S) return true;
  r1 = imin_(r1, S - 1);
  c1 = imin_(c1, S - 1);
  if (causal && c0 > r1) return true;  // smallest key is after the last row
  // largest key is out of the first row's window and no key is a sink
  if (window > 0 && r0 - c1 >= window && c0 >= sink) return true;
  return false;
}

// Every pair in rows [r0, r1] x keys [c0, c1] is visible and inside [0, S).
ATTN_HD bool block_full(int r0, int r1, int c0, int c1, int S, bool causal, int window, int sink) {
  if (r1 >= S || c1 >= S) return false;
  if (causal && c1 > r0) return false;  // largest key must not pass the first row
  // the last row must still see the first key that is not a sink
  if (window > 0 && c1 >= sink && r1 - imax_(c0, sink) >= window) return false;
  return true;
}

// Key tiles of width bc that hold any key visible to some position in [r0, r1] (r1 <= S - 1):
// the sink tiles [0, *ns) followed by the window tiles [*lo, *hi], with *ns < *lo (*ns = 0 when
// the two ranges touch: then [*lo, *hi] starts at 0 and covers both). Key tile of step s:
// s < *ns ? s : *lo + s - *ns; *ns + *hi - *lo + 1 steps. Never empty: every position sees itself.
ATTN_HD void kv_tile_range(int r0, int r1, int S, int bc, bool causal, int window, int sink, int* ns,
                           int* lo, int* hi) {
  const int jmax = causal ? r1 : S - 1;
  const int jmin = window > 0 ? imax_(0, r0 - window + 1) : 0;
  *lo = jmin / bc;
  *hi = jmax / bc;
  *ns = 0;
  if (window > 0 && sink > 0) {
    const int slast = imin_(sink, jmax + 1) - 1;  // last sink key some position sees
    const int n = slast / bc + 1;
    if (n >= *lo) *lo = 0;  // sink tiles reach the window tiles: one range
    else *ns = n;
  }
}

// Query tiles of height br (tile t = rows [t*br, t*br + br)) holding any query row that sees some
// key in [c0, c1] (c1 <= S - 1), the rows standing at positions row + off: tiles [*lo, *hi];
// *lo > *hi when no query sees these keys (they fall out of every window).
ATTN_HD void q_tile_range(int c0, int c1, int S, int off, int br, bool causal, int window, int sink,
                          int* lo, int* hi) {
  const int imin = imax_(causal ? c0 : 0, off) - off;
  // a sink key (c0 < sink) is seen by every later position
  const int imax = (window > 0 && c0 >= sink ? imin_(S - 1, c1 + window - 1) : S - 1) - off;
  if (imax < imin) {
    *lo = 1;
    *hi = 0;
    return;
  }
  *lo = imin / br;
  *hi = imax / br;
}

// Packed documents (page "Build a standalone, production grade system that trains a 4,...",
// curriculum section: documents concatenated into one buffer with boundary index arrays; attention
// resets at each boundary). cu[0..n] are the boundaries, 0 = cu[0] <= ... <= cu[n] = S; position t
// lies in document k = doc_index(cu, n, t), i.e. cu[k] <= t < cu[k + 1]. A key j is visible to a
// query i of the same batch row only if j >= cu[k(i)] (equivalently i < cu[k(j) + 1] under the
// causal mask), on top of the rules above. The search reads only cu[0..n] and ends after at most
// log2(n) + 1 steps whatever the array holds.
ATTN_HD int doc_index(const int* cu, int n, int pos) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= pos) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
ATTN_HD int doc_start(const int* cu, int n, int pos) { return cu[doc_index(cu, n, pos)]; }
ATTN_HD int doc_end(const int* cu, int n, int pos) { return cu[doc_index(cu, n, pos) + 1]; }

}  // namespace fa

#endif  // ATTN_TILES_H_
