// launch.h -- host-side interface between the C ABI (attn_api.cpp) and the kernel launchers.
#ifndef ATTN_LAUNCH_H_
#define ATTN_LAUNCH_H_

#include <stddef.h>
#include <stdint.h>

#include "tiles.h"

namespace fa {

enum { kF32 = 0, kBF16 = 1 };

// K / V in a paged cache: pools [num_blocks, Hkv, 2^shift, D]; logical block t of sequence b is
// pool block table[b * max_blocks + t]; sequence b has seqlen[b] keys (device arrays).
struct PagedKV {
  const int* table;
  const int* seqlen;
  int shift;
  int max_blocks;
  int num_blocks;
};

// Packed documents: cu [B, n + 1] int32 boundaries per batch row (device array); cu == nullptr:
// none. At most kMaxDocs documents per row (their boundaries are staged in LDS).
struct Docs {
  const int* cu;
  int n;
};
constexpr int kMaxDocs = 2047;

// Stored dS of the bf16 backward. The dK/dV pass forms every 32 x 32 block of
// dS = P o (dP - delta) of its visited tiles in registers (rounded to bf16, the operand of
// dK += dS^T Q); when the caller's workspace has room it also writes them out, and the dQ pass
// reads them back for dQ = dS K instead of recomputing S = Q K^T and dP = dO V^T (a third of its
// matrix products; the pages' backward recomputes the score tiles, which is what the pass does
// without the room). Masks without a window or sink keys only; which shapes: ds_bytes.
// Which blocks: query block i (rows 32i .. 32i+31) needs key blocks 0 .. n(i)-1 (its strip), n(i) =
// min(nkb, i + c) (c = nkb without the causal mask: every key). Layout, per (batch, KV head):
// one entry per 64-row query tile t and key block j < min(nkb, 2t + 1 + c) (the keys of the tile's
// second block), entries in order of t then j; an entry holds the G query heads of the group in
// order, each as its two 32-row blocks (2 KB each). A dQ workgroup of several heads at the same
// rows so reads one contiguous run per key block (runs of 2 KB per head and block were 22%
// slower to stream). A block is 2 KB: sixteen-byte chunk t*64 + h*32 + (k ^ 4*(2t + h)) holds key
// k's dS for queries 16t + 4h + {0, 1, 2, 3, 8, 9, 10, 11} (t, h in {0, 1}) -- the way a lane of
// the dK/dV pass holds them, so one block is written by two 1 KB stores per wave, with the key
// index swizzled so that the dQ pass's transposing LDS reads hit distinct banks.
struct DsMap {
  uint16_t* ds;         // null: the dQ pass recomputes
  int nqb, nkb;         // query / key blocks of 32
  int c;                // see above
  int G;                // query heads per KV head
  long long per_group;  // entries per (batch, KV head)
};
ATTN_HD int ds_strip_len(const DsMap& m, int i) { return imin_(m.nkb, i + m.c); }
// First entry of 64-row tile t: the tiles before it with fewer than nkb key blocks hold
// c + 1, c + 3, ..
ATTN_HD long long ds_tile_start(const DsMap& m, int t) {
  const int x = m.nkb - m.c - 1;
  const long long t1 = x <= 0 ? 0 : imin_((x + 1) / 2, t);
  return t1 * (t1 - 1) + (long long)(m.c + 1) * t1 + (long long)(t - t1) * m.nkb;
}
// Byte offset of block (query block i, key block j) of head hg of KV head bg (= b * Hkv + g).
ATTN_HD size_t ds_block_off(const DsMap& m, int bg, int hg, int i, int j) {
  return (((size_t)bg * m.per_group + ds_tile_start(m, i >> 1) + j) * m.G + hg) * 4096 + (size_t)(i & 1) * 2048;
}
inline DsMap ds_map(int Hq, int Hkv, int Sq, int Sk, int causal) {
  DsMap m;
  m.ds = nullptr;
  m.nqb = (Sq + 31) / 32;
  m.nkb = (Sk + 31) / 32;
  // causal: row 32i + 31 stands at position 32i + 31 + Sk - Sq and sees key blocks up to
  // i + (31 + Sk - Sq) / 32
  m.c = causal ? 1 + (31 + Sk - Sq) / 32 : m.nkb;
  m.G = Hq / Hkv;
  m.per_group = ds_tile_start(m, (m.nqb + 1) / 2);
  return m;
}
// Bytes of the stored dS (0: not used for these arguments). At most kDsMaxBytes (a 4096-token
// causal 64-head problem needs 1.1 GB; longer ones recompute). Only where it was measured to pay:
// D = 128 and at least kDsMinKeys keys. A stored block saves two 32 x 32 x D products of the dQ
// pass for 4 KB of HBM traffic and a pass of its own for the delta rows; against recomputing,
// whole fwd + bwd steps (64/8 heads unless noted) took 1-2% less at S = 4096, 22-31% less for 1
// or 100 queries against 4096 keys, the same at S = 2048, 12% more at S = 1024, and at D = 64
// 17% more at S = 8192 (16 heads) and 2% more at S = 1024 (4 x 16 heads).
constexpr size_t kDsMaxBytes = (size_t)4 << 30;
constexpr int kDsMinKeys = 2048;
inline size_t ds_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int window, int sink) {
  if (window != 0 || sink != 0 || D != 128 || Sk < kDsMinKeys) return 0;
  const DsMap m = ds_map(Hq, Hkv, Sq, Sk, causal);
  const size_t n = (size_t)B * Hq * (size_t)m.per_group * 4096;
  return n <= kDsMaxBytes ? n : 0;
}

struct Args {
  int dtype;
  const void* q;
  const void* k;
  const void* v;
  const void* o_in;   // backward: forward output
  void* o;            // forward: output
  float* lse;         // forward: output; backward: input
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;       // backward workspace: -rowsum(dO * O) (stored negated), [B, Hq, Sq]
  float* lse2;        // backward workspace: lse * log2(e), [B, Hq, Sq]
  float* xpart;       // backward workspace: sink-split chunk partials, or null (no split)
  float* part;        // backward workspace: fp32 dK / dV partial sums of the head-group parts
  int B, Hq, Hkv, Sq, Sk, D;  // Sq query rows, Sk >= Sq keys (queries: the last Sq positions)
  int causal, window, sink;  // sink: keys [0, sink) stay visible beside the window
  float scale;
  void* stream;
  bool paged;  // forward only: k, v are pools read through pg (Sk is then per sequence)
  PagedKV pg;
  Docs docs;   // packed documents (Sq = Sk, causal, no sinks)
  DsMap dsm;   // backward: stored dS (dsm.ds null: none)
};

// The argument checks every entry point shares: ATTN_OK (0) or the attn_status_t of the first
// failed check (sizes, head grouping, mask arguments, dtype, head dimension, scale).
int check_args(int dtype, int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int window,
               int sink, float scale);

// Tells the launch observer (attn_set_launch_hook) that `kernel` is about to be / has been
// enqueued on `stream`.
void notify_launch(const char* kernel, int after, void* stream);

// Each returns 0 on success, -1 if the HIP runtime reported a launch error.
int launch_fwd(const Args& a);
int launch_bwd(const Args& a);
int launch_dkdv(const Args& a);  // dK / dV pass (and its reduce), called by launch_bwd
// Key-split decode forward (bf16, (Hq / Hkv) * Sq <= 32): partials in `part`, then merged into
// a.o / a.lse. max_keys bounds every sequence's key count (sizes the chunk grid).
int launch_decode(const Args& a, float* part, int max_keys);
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int max_keys, int D);

// Forward workgroup shape for bf16: waves per workgroup (32 query rows each) and LDS ring depth
// (tiles in flight + 1).
#ifndef ATTN_FWD_WAVES
#define ATTN_FWD_WAVES 8
#endif
#ifndef ATTN_FWD_STAGES
#define ATTN_FWD_STAGES 2
#endif
constexpr int kFwdWaves = ATTN_FWD_WAVES, kFwdStages = ATTN_FWD_STAGES;
// Waves per workgroup of the bf16 forward pass when the visible key range of a row is short (and of
// the bf16 dQ pass always): a workgroup walks the union of its waves' key ranges, which for 32*NW rows
// exceeds one wave's by up to 32*(NW-1) keys. Measured against 8 waves: forward 6-15% and dQ 9-15%
// faster on the sliding-window (W = 1024) and packed-document (1.1-1.7k-token) workloads and on dense
// causal S = 1024; at dense causal S = 4096 the forward is 1.5% slower and dQ (with packed heads) 1%
// faster.
#ifndef ATTN_SHORT_WAVES
#define ATTN_SHORT_WAVES 4
#endif
#ifndef ATTN_SHORT_KEYS
#define ATTN_SHORT_KEYS 1024
#endif
constexpr int kShortWaves = ATTN_SHORT_WAVES, kShortKeys = ATTN_SHORT_KEYS;
// Short key ranges (the waves of a 32*kFwdWaves-row workgroup would idle much of the time): packed
// documents, or at most kShortKeys keys per query row on average over the whole sequence (a causal
// row at position p sees p + 1 keys, at most `window`). The test looks at Sk, causal and window
// only, never at Sq, so a query chunk (Sq < Sk) runs the same workgroups, and gives the same bits,
// as its rows do in the call over all Sk queries.
inline bool short_key_ranges(const Args& a) {
  if (a.docs.cu) return true;
  double mean = a.causal ? (a.Sk + 1) / 2.0 : (double)a.Sk;
  if (a.window > 0 && mean > a.window) mean = a.window;
  return mean <= kShortKeys;
}
// Medium key ranges (same mean, more than kShortKeys and at most kMidKeys keys per row): the
// 8-wave bf16 forward takes two softmax updates of 32*KB keys per workgroup barrier, from LDS stages
// of twice the keys (the same bits as one update per barrier). Measured against one update per
// barrier: 2% faster at dense causal S = 4096 (D = 128) and S = 8192 (D = 64), 5% with a 2048-key
// window at S = 8192, no different at dense causal S = 8192 (D = 128), 1-1.5% slower at S = 16384
// and S = 32768. dQ with the same stages was 1.5% slower at S = 4096 and keeps one block per barrier.
#ifndef ATTN_MID_KEYS
#define ATTN_MID_KEYS 4096
#endif
constexpr int kMidKeys = ATTN_MID_KEYS;
inline bool mid_key_ranges(const Args& a) {
  if (a.docs.cu) return false;
  double mean = a.causal ? (a.Sk + 1) / 2.0 : (double)a.Sk;
  if (a.window > 0 && mean > a.window) mean = a.window;
  return mean <= kMidKeys;
}

// Query heads of one KV group packed into a forward / dQ workgroup: the largest power of two that
// divides the group size G and the wave count NW, at most `cap`. Waves of different heads at the
// same query rows share the K / V tiles and have the same key range, so no wave idles on the
// causal diagonal while the others finish their longer rows (same bits as one head per workgroup).
// Measured against one head per workgroup: dQ with up to 8 heads 1-2.5% faster (S = 4096, and a
// 2048-key window at S = 8192); the forward with 2 heads 0.5-2.5% faster, with 4 or 8 heads no
// faster at S = 4096.
#ifndef ATTN_FWD_HEAD_PACK
#define ATTN_FWD_HEAD_PACK 2
#endif
#ifndef ATTN_DQ_HEAD_PACK
#define ATTN_DQ_HEAD_PACK 8
#endif
// Fewer heads while that leaves fewer than kPackMinGroups workgroups (a handful of query rows, e.g.
// one decode query per head: one head per workgroup spreads the heads over more compute units).
constexpr int kPackMinGroups = 256;
inline int heads_per_workgroup(int G, int NW, int cap, int B, int Hq, int Sq) {
  int gp = 1;
  while (gp * 2 <= cap && G % (gp * 2) == 0 && NW % (gp * 2) == 0) gp *= 2;
  auto groups = [&](int p) { return (long long)((Sq + 32 * NW / p - 1) / (32 * NW / p)) * B * (Hq / p); };
  while (gp > 1 && groups(gp) < kPackMinGroups) gp /= 2;
  return gp;
}

// dK/dV decomposition: a workgroup of kDkdvWaves waves owns 32*kDkdvWaves keys and processes key
// tile j and then key tile n_kt-1-j (equal work per workgroup under the causal mask). When that
// gives fewer than kDkdvMinGroups workgroups, the query-head group is split into `hs` parts (a
// power of two dividing Hq/Hkv) whose fp32 partial sums are reduced by a second kernel.
constexpr int kDkdvWaves = 4;
constexpr int kDkdvMinGroups = 256;
struct DkdvPlan {
  int n_kt, n_pairs, hs;
  int nc, c_lo, c_len;  // sink split: key tile 0's query tiles c_lo + [c*c_len, (c+1)*c_len), c < nc
};
inline DkdvPlan dkdv_plan(int B, int Hq, int Hkv, int Sk) {
  DkdvPlan p;
  p.n_kt = (Sk + 32 * kDkdvWaves - 1) / (32 * kDkdvWaves);
  p.n_pairs = (p.n_kt + 1) / 2;
  const long items = (long)B * Hkv * p.n_pairs;
  const int G = Hq / Hkv;
  p.hs = 1;
  while (items * p.hs < kDkdvMinGroups && G % (2 * p.hs) == 0) p.hs *= 2;
  p.nc = 1;
  p.c_lo = 0;
  p.c_len = 0;
  return p;
}

// Sink split of the bf16 dK/dV pass. With a window and sink keys (sink <= one key tile), key tile
// 0 is seen by every later query while any other tile only by about a window's worth, so the
// workgroup holding tile 0 would run several times longer than the rest. When that workgroup
// would outlast the average load of a compute unit, its query range (tiles of dkdv_query_rows(D)
// rows) is cut into nc chunks of about a quarter of an ordinary tile's range: chunk 0 stays with
// tile 0's workgroup, chunks 1.. become small extra workgroups that fill in behind the ordinary
// ones. Every chunk writes fp32 partial sums of tile 0's dK and dV (per head part) that a small
// reduce adds in a fixed order.
// Query rows per streamed tile of the bf16 dK/dV pass: 64 for both head sizes (with the lagged
// schedule's three stages and two P buffers, 128-row tiles at D = 64 would need 163 KB of LDS;
// 64-row tiles with the lag beat 128-row tiles with two barriers per step by 1-4%).
constexpr int dkdv_query_rows(int) { return 64; }
constexpr int kDkdvMaxChunks = 64;
constexpr int kComputeUnits = 256;  // MI355X
inline void dkdv_sink_split(DkdvPlan& p, int B, int Hq, int Hkv, int Sq, int Sk, int D, int window, int sink,
                            bool causal) {
  const int BR = dkdv_query_rows(D);
  const int BC = 32 * kDkdvWaves;
  if (window <= 0 || sink <= 0 || sink > BC) return;
  const int off = Sk - Sq;
  const int c1 = (BC < Sk ? BC : Sk) - 1;
  int lo0, hi0, lo1, hi1;
  q_tile_range(0, c1, Sk, off, BR, causal, window, sink, &lo0, &hi0);
  q_tile_range(0, c1, Sk, off, BR, causal, window, 0, &lo1, &hi1);
  const int nq0 = hi0 - lo0 + 1;
  const int nq1 = hi1 >= lo1 ? hi1 - lo1 + 1 : 1;
  if (nq0 <= nq1) return;
  // steps (query tiles x heads of a part) of tile 0's workgroup against a compute unit's share
  const long hpg = Hq / Hkv / p.hs;
  const long heavy = (long)(nq0 + nq1) * hpg;
  const long share = (long)B * Hkv * p.hs * p.n_pairs * 2 * nq1 * hpg / kComputeUnits;
  if (heavy * 10 <= share * 11) return;
  p.c_len = (nq1 + 3) / 4;
  int nc = (nq0 + p.c_len - 1) / p.c_len;
  if (nc > kDkdvMaxChunks) p.c_len = (nq0 + kDkdvMaxChunks - 1) / kDkdvMaxChunks;
  p.c_lo = lo0;
  p.nc = (nq0 + p.c_len - 1) / p.c_len;
}
inline size_t dkdv_chunk_bytes(const DkdvPlan& p, int B, int Hkv, int D) {
  return p.nc > 1 ? (size_t)p.nc * p.hs * B * Hkv * 2 * (32 * kDkdvWaves) * D * sizeof(float) : 0;
}

inline size_t delta_bytes(int B, int Hq, int Sq) {
  return ((size_t)B * Hq * Sq * sizeof(float) + 255) / 256 * 256;
}
// Workspace layout: -delta [B,Hq,Sq] f32 | lse * log2(e) [B,Hq,Sq] f32 | dK/dV partials (if the
// head group is split) | sink-split chunk partials or the stored dS (when the caller sized the
// workspace for them; a mask has at most one of the two).
inline size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D) {
  const DkdvPlan p = dkdv_plan(B, Hq, Hkv, Sk);
  size_t partials = p.hs > 1 ? (size_t)p.hs * 2 * B * Hkv * Sk * D * sizeof(float) : 0;
  return 2 * delta_bytes(B, Hq, Sq) + partials;
}
inline size_t bwd_workspace_bytes_for(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                                      int window, int sink) {
  DkdvPlan p = dkdv_plan(B, Hq, Hkv, Sk);
  dkdv_sink_split(p, B, Hq, Hkv, Sq, Sk, D, window, sink, causal != 0);
  return bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, D) + dkdv_chunk_bytes(p, B, Hkv, D) +
         ds_bytes(B, Hq, Hkv, Sq, Sk, D, causal, window, sink);
}

}  // namespace fa

#endif  // ATTN_LAUNCH_H_
