// attn_bwd.hip -- tiled causal / sliding-window GQA attention backward for gfx950.
//
// Method: "KYNETRA FOUNDRY" page, FlashAttention paragraph (the backward recomputes score tiles on
// the fly rather than storing them); "CUDA-LLM: A GitHub Repository for Development", section "The
// custom CUDA kernel" (probabilities are recomputed from the saved log-sum-exp); Grip paragraph of
// the first page (dK and dV of a shared K/V head sum over its query-head group).
//
// Launches on the caller's stream, no atomics anywhere:
//   1. dq_kernel: lanes own queries (as in the forward). Each wave first forms, for its own rows,
//      delta_i = sum_d dO_id * O_id in fp32 (O as the forward stored it) and the base-2
//      log-sum-exp lse_i * log2(e), and stores both for the dK / dV pass; then S^T = K Q^T and
//      dP^T = V dO^T from LDS key/value tiles, dS^T in registers is the B operand of
//      dQ^T += K^T dS^T with K^T read through the transposing LDS read.
//   2. dkdv_pair_kernel (bf16) / dkdv_kernel (fp32) (attn_dkdv.hip): the K and V rows of a wave's
//      32 keys stay in registers as B operands of S = Q K^T and dP = dO V^T, so a lane owns one
//      key and its accumulator holds query rows -- exactly the contraction side that
//      dV += P^T dO and dK += dS^T Q need. Query / dO / lse / delta tiles of the group's heads
//      stream through an LDS-DMA ring (bf16: three stages with one tile in flight, the dP wave one
//      tile behind the S wave; fp32: three stages, two in flight); dK and dV for the group accumulate in registers. A workgroup takes key tile j and then key tile T-1-j, so
//      under the causal mask every workgroup does the same amount of work. When that leaves too
//      few workgroups to fill the GPU, the head group is split into `hs` parts whose fp32 partial
//      sums go to the workspace and
//   3. dkdv_reduce_kernel (attn_dkdv.hip) adds them in a fixed order (deterministic) and rounds to the element type.
// With a stored dS (bf16, the shapes ds_bytes in launch.h admits, a workspace with room for it;
// layout at DsMap there) the order is bwd_prep_kernel (the delta and base-2 log-sum-exp rows), the
// dK / dV pass, which also writes each dS block it forms, and dq_ds_kernel, which reads those
// blocks for dQ = scale * dS K (no score or dP products in the dQ pass) and, in trailing
// workgroups, adds the dK / dV head-part partials.
// P and dS are rounded to the element type only as MFMA operands; all sums are fp32.
#include "device.h"
#include "launch.h"

namespace fa {

// This lane's half of sum_d dO_id * O_id for query row `o_row` (lanes l and l ^ 32 hold the two
// halves of the row: elements 16s + 8h .. +7, h = l / 32), from the dO fragments `df` of the same
// elements; pair_sum of it is delta_i. dq_kernel and bwd_prep_kernel both form delta through it.
template <class E, int D>
__device__ __forceinline__ float half_row_dot(const typename E::T* __restrict__ o_row, const Frag<E>* df,
                                              bool ok) {
  constexpr int DS = D / 16;
  const int half = lane_id() >> 5;
  float dl = 0.f;
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    const Frag<E> of = load_frag_global(o_row + 16 * s + 8 * half, ok);
    if constexpr (E::kBytes == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dl += bf16_to_f32(of.v[e] & 0xFFFFu) * bf16_to_f32(df[s].v[e] & 0xFFFFu);
        dl += bf16_to_f32(of.v[e] >> 16) * bf16_to_f32(df[s].v[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) dl += of.lo[e] * df[s].lo[e] + of.hi[e] * df[s].hi[e];
    }
  }
  return dl;
}

template <class E, int D, int NW, int KB, bool VL>
__global__ __launch_bounds__(NW * 64, E::kBytes == 2 && NW == 4 ? 2 : 1) void dq_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
    const typename E::T* __restrict__ O, const float* __restrict__ LSE, float* __restrict__ LSE2,
    float* __restrict__ delta, typename E::T* __restrict__ dQ,
    int B, int Hq, int Hkv, int Sq, int S, int causal, int window, int sink, float scale,
    float scale_log2, int n_qt, int gp, Docs docs) {
  constexpr int BC = 32 * KB;
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  typedef LdsTile<E, BC, D> KvTile;
  constexpr int kStage = 2 * KvTile::kBytes;
  constexpr int kOps = 2 * dma_tile_ops<E, BC, D, NW>();
  // K / V ring: bf16 two stages (one tile in flight; 1-2% faster than three), fp32 three
  constexpr int NST = E::kBytes == 2 ? 2 : 3;
  __shared__ __attribute__((aligned(1024))) char ring[NST * kStage];
  __shared__ int cu_s[VL ? kMaxDocs + 1 : 1];

  const int lane = lane_id();
  const int w = wave_id();
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // Same decomposition and order as the forward: gp query heads of one KV group per workgroup
  // (wave w: head w % gp of the chunk, rows q0 + 32 * (w / gp) ..), heaviest query tiles first, a
  // KV group's workgroups on one XCD.
  const int BR = 32 * NW / gp;
  const int G = Hq / Hkv;
  const int BG = B * Hkv;
  const int bg = blockIdx.x % BG;
  const int rest = blockIdx.x / BG;
  const int hc = rest % (G / gp);
  const int rank = rest / (G / gp);
  const int qt = causal ? n_qt - 1 - rank : rank;
  const int b = bg / Hkv;
  const int h = (bg - b * Hkv) * G + hc * gp + w % gp;
  const int off = S - Sq;  // query row r stands at key position r + off
  const size_t q_off = (size_t)(b * Hq + h) * Sq * D;
  const typename E::T* k_bg = K + (size_t)bg * S * D;
  const typename E::T* v_bg = V + (size_t)bg * S * D;

  const int q0 = qt * BR;
  const int qw = q0 + 32 * (w / gp);
  const int my_q = qw + l32;
  const bool q_ok = my_q < Sq;
  const int pw = qw + off;  // positions of this wave's rows
  const int my_p = my_q + off;

  // documents: ds_lane = start of this lane's query's document
  int ds_lane = 0;
  if constexpr (VL) {
    stage_docs(cu_s, docs.cu + (size_t)b * (docs.n + 1), docs.n, S);
    __syncthreads();
    ds_lane = doc_start(cu_s, docs.n, imin_(my_p, S - 1));
  }

  // key tiles: the sink tiles [0, jt_ns) then the window tiles [jt_lo, jt_hi]
  int jt_ns, jt_lo, jt_hi;
  kv_tile_range(q0 + off, imin_(q0 + BR - 1, Sq - 1) + off, S, BC, causal, window, sink, &jt_ns, &jt_lo,
                &jt_hi);
  if constexpr (VL) jt_lo = imax_(jt_lo, doc_start(cu_s, docs.n, q0 + off) / BC);  // no sinks here
  const int n_steps = jt_ns + jt_hi - jt_lo + 1;
  auto tile_of = [&](int s) __attribute__((always_inline)) { return s < jt_ns ? s : jt_lo + s - jt_ns; };
  constexpr bool kFast = dma_fast_ok<E, BC, D, NW>();
  const uint32_t dma_off = kFast ? dma_lane_off<KvTile, NW>() : 0;  // whole tiles: scalar base + offset
  auto issue = [&](int s, char* stg) __attribute__((always_inline)) {
    const int j0 = tile_of(s) * BC;
    if (kFast && j0 + BC <= S) {
      if constexpr (kFast) {
        dma_tile_fast<E, BC, D, NW>(stg, k_bg, j0, dma_off);
        dma_tile_fast<E, BC, D, NW>(stg + KvTile::kBytes, v_bg, j0, dma_off);
      }
    } else {
      dma_tile<E, BC, D, NW>(stg, k_bg, j0, S);
      dma_tile<E, BC, D, NW>(stg + KvTile::kBytes, v_bg, j0, S);
    }
  };
  issue(0, ring);
  if (NST == 3 && n_steps > 1) issue(1, ring + kStage);

  Frag<E> qf[DS], df[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    qf[s] = load_frag_global(Q + q_off + (size_t)my_q * D + 16 * s + 8 * half, q_ok);
    df[s] = load_frag_global(dO + q_off + (size_t)my_q * D + 16 * s + 8 * half, q_ok);
  }
  const size_t row_idx = (size_t)(b * Hq + h) * Sq + (q_ok ? my_q : 0);
  // delta_i = sum_d dO_id O_id: this lane holds half of row my_q's elements, its partner the rest
  const float dl = pair_sum(half_row_dot<E, D>(O + q_off + (size_t)my_q * D, df, q_ok));
  const float l2 = LSE[row_idx] * kLog2e;  // base-2 log-sum-exp used by both gradient kernels
  const float nlse2 = -l2;
  if (q_ok && half == 0) {
    delta[row_idx] = -dl;  // stored negated: the dK / dV pass starts its dP products from it
    LSE2[row_idx] = l2;
  }
  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};
  // -delta_i in every register: the accumulator the dP products start from, so they leave
  // dP - delta and dS = P o (dP - delta) takes one multiply per element
  f32x16_t ndl;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndl[r] = -dl;
  wait_vmcnt<0>();

  auto compute = [&](int s, const char* k_lds) __attribute__((always_inline)) {
    const char* v_lds = k_lds + KvTile::kBytes;
    const int j0 = tile_of(s) * BC;
    if (block_empty(pw, pw + 31, j0, j0 + BC - 1, S, causal, window, sink)) return;
    bool full = block_full(pw, pw + 31, j0, j0 + BC - 1, S, causal, window, sink);
    if constexpr (VL) {
      if (j0 + BC - 1 < __builtin_amdgcn_readlane(ds_lane, 0)) return;
      full = full && __builtin_amdgcn_readlane(ds_lane, 31) <= j0;
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16_t st = f32x16_t{}, dpt = ndl;
      // all K fragments of the key block are requested before its S products (one LDS latency),
      // the V fragments under those products
      Frag<E> kfr[DS];
#pragma unroll
      for (int s2 = 0; s2 < DS; ++s2) kfr[s2] = RowFrag<E, KvTile>::get(k_lds, 32 * kb + l32, s2);
      __builtin_amdgcn_sched_barrier(0);
      Frag<E> vfr[DS];
#pragma unroll
      for (int s2 = 0; s2 < DS; ++s2) {
        vfr[s2] = RowFrag<E, KvTile>::get(v_lds, 32 * kb + l32, s2);
        mma(st, kfr[s2], qf[s2]);
      }
#pragma unroll
      for (int s2 = 0; s2 < DS; ++s2) mma(dpt, vfr[s2], df[s2]);
      // P = exp2(S * scale * log2 e - lse * log2 e), masked to 0 in place on partial tiles (one
      // code path, so no register copies where masked and unmasked tiles rejoin), then
      // dS = P o (dP - delta).
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = __builtin_amdgcn_exp2f(fmaf(st[r], scale_log2, nlse2));
      if (!full) {
        const int mp = opaque(my_p);  // this lane's position, re-derived inside the masked path only
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * kb + acc_row(r);
          mask_zero(st, r, visible(mp, j, S, causal, window, sink) && !(VL && j < ds_lane));
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = st[r] * dpt[r];  // dpt holds dP - delta
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const Frag<E> sf = acc_frag<E>(st, t);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          mma(acc[db], TrFrag<E, KvTile>::get(k_lds, 32 * kb + 16 * t, 32 * db), sf);
      }
    }
  };
  ring_run<NST, kStage, kOps>(ring, n_steps, issue, compute);

  if (!q_ok) return;
  typename E::T* dq_row = dQ + q_off + (size_t)my_q * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * db + 8 * r4 + 4 * half;
      const float x0 = acc[db][4 * r4 + 0] * scale, x1 = acc[db][4 * r4 + 1] * scale;
      const float x2 = acc[db][4 * r4 + 2] * scale, x3 = acc[db][4 * r4 + 3] * scale;
      if constexpr (E::kBytes == 2) {
        *reinterpret_cast<u32x2_t*>(dq_row + d) = u32x2_t{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
      } else {
        *reinterpret_cast<f32x4_t*>(dq_row + d) = f32x4_t{x0, x1, x2, x3};
      }
    }
  }
}

// With a stored dS the rows' delta and base-2 log-sum-exp come first, from their own pass: one
// wave per 32 rows of the flattened [B * Hq * Sq] rows, the same arithmetic as dq_kernel's.
template <class E, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const typename E::T* __restrict__ O,
                                                       const typename E::T* __restrict__ dO,
                                                       const float* __restrict__ LSE, float* __restrict__ LSE2,
                                                       float* __restrict__ delta, long long rows) {
  constexpr int DS = D / 16;
  const int lane = lane_id();
  const int half = lane >> 5;
  const long long r = ((long long)blockIdx.x * 4 + wave_id()) * 32 + (lane & 31);
  const bool ok = r < rows;
  const size_t ro = (size_t)(ok ? r : 0);
  Frag<E> df[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) df[s] = load_frag_global(dO + ro * D + 16 * s + 8 * half, ok);
  const float dl = pair_sum(half_row_dot<E, D>(O + ro * D, df, ok));
  if (ok && half == 0) {
    delta[ro] = -dl;
    LSE2[ro] = LSE[ro] * kLog2e;
  }
}

// dQ from the stored dS (bf16; layout at DsMap): dQ^T += K^T dS^T over the key blocks of the
// wave's rows, with no S or dP products. Wave w owns 64 query rows (two 32-row blocks) of head
// w % gp of its KV group's chunk; per 32-key step the workgroup copies the K tile and each wave
// its own two dS blocks (2 KB each, as the dK/dV pass wrote them) into a three-stage LDS ring.
// Both operands come through transposing LDS reads: K^T as in dq_kernel, and dS^T (a lane per
// query, 8 keys) from the block, whose chunk holds one key's values for 8 queries: within each
// group of 16 lanes, lane s reads the four queries 16g + 4(s % 4) .. of key 4(s / 4) + .., i.e.
// chunk g*64 + (s & 1)*32 + (key ^ 4*(2g + (s & 1))), bytes 8 * ((s >> 1) & 1) .. Every block a
// query block needs (key blocks 0 .. ds_strip_len - 1) holds the exact dS of its pairs (zeros where
// the mask hides them), so no mask here.
// Workgroups n_dq.. of the same launch add the dK / dV head-part partials of a split head group
// (what dkdv_reduce_kernel does otherwise, the same sums in the same order): the short reduce
// fills in behind the dQ workgroups instead of taking a launch of its own (a prefill chunk's
// backward 2% faster, S = 4096 0.5%).
struct PartSum {
  const float* part;  // 2 * hs slices of n floats: dK part 0, dV part 0, dK part 1, ..
  uint16_t* dK;
  uint16_t* dV;
  size_t n;           // B * Hkv * S * D
  int hs;             // 1: nothing to add
  int n_dq;           // dQ workgroups before the reduce ones
};
constexpr int kPartChunks = 16;  // 1024-element chunks per reduce workgroup, loaded before any sum
template <int D>
__global__ __launch_bounds__(256, 2) void dq_ds_kernel(const uint16_t* __restrict__ K, uint16_t* __restrict__ dQ,
                                                        DsMap dsm, int B, int Hq, int Hkv, int Sq, int S,
                                                        int causal, float scale, int n_qt, int gp, PartSum ps) {
  if ((int)blockIdx.x >= ps.n_dq) {
    const size_t base = (size_t)(blockIdx.x - ps.n_dq) * kPartChunks * 1024 + threadIdx.x * 4;
    f32x4_t sk[kPartChunks], sv[kPartChunks];
#pragma unroll
    for (int c = 0; c < kPartChunks; ++c) {
      const size_t i = base + (size_t)c * 1024;
      if (i < ps.n) {
        sk[c] = *reinterpret_cast<const f32x4_t*>(ps.part + i);
        sv[c] = *reinterpret_cast<const f32x4_t*>(ps.part + ps.n + i);
      }
    }
    for (int p = 1; p < ps.hs; ++p) {
#pragma unroll
      for (int c = 0; c < kPartChunks; ++c) {
        const size_t i = base + (size_t)c * 1024;
        if (i < ps.n) {
          sk[c] += *reinterpret_cast<const f32x4_t*>(ps.part + (size_t)(2 * p) * ps.n + i);
          sv[c] += *reinterpret_cast<const f32x4_t*>(ps.part + (size_t)(2 * p + 1) * ps.n + i);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kPartChunks; ++c) {
      const size_t i = base + (size_t)c * 1024;
      if (i < ps.n) {
        const f32x4_t k4 = sk[c] * scale, v4 = sv[c];
        *reinterpret_cast<u32x2_t*>(ps.dK + i) = u32x2_t{pack_bf16x2(k4[0], k4[1]), pack_bf16x2(k4[2], k4[3])};
        *reinterpret_cast<u32x2_t*>(ps.dV + i) = u32x2_t{pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3])};
      }
    }
    return;
  }
  typedef BF16 E;
  constexpr int NW = 4;   // waves
  constexpr int RB = 2;   // 32-row query blocks per wave
  constexpr int DB = D / 32;
  typedef LdsTile<E, 32, D> KTile;
  constexpr int kStage = KTile::kBytes + NW * RB * 2048;
  constexpr int kOps = dma_tile_ops<E, 32, D, NW>() + 2 * RB;
  static_assert(dma_fast_ok<E, 32, D, NW>(), "whole K tiles copy with scalar bases");
  __shared__ __attribute__((aligned(1024))) char ring[3 * kStage];

  const int lane = lane_id();
  const int w = wave_id();
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // Decomposition and order as dq_kernel: gp heads of one KV group per workgroup, heaviest query
  // tiles first, a KV group's workgroups on one XCD.
  const int BR = 32 * RB * NW / gp;
  const int G = Hq / Hkv;
  const int BG = B * Hkv;
  const int bg = blockIdx.x % BG;
  const int rest = blockIdx.x / BG;
  const int hc = rest % (G / gp);
  const int rank = rest / (G / gp);
  const int qt = causal ? n_qt - 1 - rank : rank;
  const int b = bg / Hkv;
  const int h = (bg - b * Hkv) * G + hc * gp + w % gp;
  const int off = S - Sq;
  const uint16_t* k_bg = K + (size_t)bg * S * D;
  const int q0 = qt * BR;
  const int qw = q0 + 32 * RB * (w / gp);
  const int ib = qw / 32;  // this wave's first query block
  const int hg = hc * gp + w % gp;  // head within the KV group
  const char* ds_base = reinterpret_cast<const char*>(dsm.ds);

  // key blocks of the workgroup's rows (no window, no sinks)
  int jt_ns, jt_lo, jt_hi;
  kv_tile_range(q0 + off, imin_(q0 + BR - 1, Sq - 1) + off, S, 32, causal, 0, 0, &jt_ns, &jt_lo, &jt_hi);
  const int n_steps = jt_hi - jt_lo + 1;
  // block (query block i, key block j) lies in the strip of i: written by the dK/dV pass
  auto in_strip = [&](int i, int j) __attribute__((always_inline)) {
    return i < dsm.nqb && j < ds_strip_len(dsm, i);
  };
  const uint32_t k_off = dma_lane_off<KTile, NW>();
  auto issue = [&](int s, char* stg) __attribute__((always_inline)) {
    const int j = jt_lo + s;
    if ((j + 1) * 32 <= S) dma_tile_fast<E, 32, D, NW>(stg, k_bg, 32 * j, k_off);
    else dma_tile<E, 32, D, NW>(stg, k_bg, 32 * j, S);
    const uint32_t dl = lds_addr(stg + KTile::kBytes + w * RB * 2048);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // blocks outside the strip are not read back; their copy takes the region's first block.
      // Each block is read once: non-temporal loads (dQ 247 -> 213 us at S = 4096 against cached
      // loads; the K tiles, which every workgroup of the group reads, stay cached)
      const int i = ib + rb;
      const char* src = ds_base + (in_strip(i, j) ? ds_block_off(dsm, bg, hg, i, j) : 0);
      dma16_s<true>(lane * 16, src, dl + rb * 2048);
      dma16_s<true>(lane * 16, src + 1024, dl + rb * 2048 + 1024);
    }
  };
  issue(0, ring);
  if (n_steps > 1) issue(1, ring + kStage);

  f32x16_t acc[RB][DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[rb][db] = f32x16_t{};
  // transposing-read addresses of this lane inside a dS block, for keys 16t + 4h + (s >> 2) (+ 8)
  const int s16 = lane & 15;
  const int g = (lane >> 4) & 1;
  const int hw = s16 & 1;
  auto ds_off = [&](int key) __attribute__((always_inline)) {
    return ((g * 64 + hw * 32 + (key ^ (4 * (2 * g + hw)))) << 4) + 8 * ((s16 >> 1) & 1);
  };
  auto compute = [&](int s, const char* stg) __attribute__((always_inline)) {
    const int j = jt_lo + s;
    const char* ds_lds = stg + KTile::kBytes + w * RB * 2048;
    bool act[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) act[rb] = in_strip(ib + rb, j);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      Frag<E> kt[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) kt[db] = TrFrag<E, KTile>::get(stg, 16 * t, 32 * db);
      const int ka = 16 * t + 4 * half + (s16 >> 2);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (!act[rb]) continue;
        const char* blk = ds_lds + rb * 2048;
        s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)((__attribute__((address_space(3))) char*)(blk + ds_off(ka))));
        s16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)((__attribute__((address_space(3))) char*)(blk + ds_off(ka + 8))));
        Frag<E> f;
        const u32x2_t ux = __builtin_bit_cast(u32x2_t, x);
        const u32x2_t uy = __builtin_bit_cast(u32x2_t, y);
        f.v = u32x4_t{ux[0], ux[1], uy[0], uy[1]};
#pragma unroll
        for (int db = 0; db < DB; ++db) mma(acc[rb][db], kt[db], f);
      }
    }
  };
  ring_run<3, kStage, kOps>(ring, n_steps, issue, compute);

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int my_q = qw + 32 * rb + l32;
    if (my_q >= Sq) continue;
    uint16_t* dq_row = dQ + ((size_t)(b * Hq + h) * Sq + my_q) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * half;
        const float x0 = acc[rb][db][4 * r4 + 0] * scale, x1 = acc[rb][db][4 * r4 + 1] * scale;
        const float x2 = acc[rb][db][4 * r4 + 2] * scale, x3 = acc[rb][db][4 * r4 + 3] * scale;
        *reinterpret_cast<u32x2_t*>(dq_row + d) = u32x2_t{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
      }
    }
  }
}

template <int D>
static void launch_dq_ds(const Args& a) {
  constexpr int NW = 4, RB = 2;
  const int G = a.Hq / a.Hkv;
  // heads per workgroup: up to 4 (one per wave, all at the same 64 rows), fewer while that
  // leaves under kPackMinGroups workgroups
  int gp = 1;
  while (gp * 2 <= NW && G % (gp * 2) == 0) gp *= 2;
  auto groups = [&](int p) {
    const int br = 32 * RB * NW / p;
    return (long long)((a.Sq + br - 1) / br) * a.B * (a.Hq / p);
  };
  while (gp > 1 && groups(gp) < kPackMinGroups) gp /= 2;
  const int br = 32 * RB * NW / gp;
  const int n_qt = (a.Sq + br - 1) / br;
  // the dK / dV head-part partials of a split head group are added by trailing workgroups
  PartSum ps{a.part, (uint16_t*)a.dk, (uint16_t*)a.dv, (size_t)a.B * a.Hkv * a.Sk * D, 1, n_qt * a.B * a.Hq / gp};
  ps.hs = dkdv_plan(a.B, a.Hq, a.Hkv, a.Sk).hs;
  const int n_red = ps.hs > 1 ? (int)((ps.n + kPartChunks * 1024 - 1) / (kPartChunks * 1024)) : 0;
  hipLaunchKernelGGL((dq_ds_kernel<D>), dim3((unsigned)(ps.n_dq + n_red)), dim3(NW * 64), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.k, (uint16_t*)a.dq, a.dsm, a.B, a.Hq, a.Hkv,
                     a.Sq, a.Sk, a.causal, a.scale, n_qt, gp, ps);
}

// Key tiles: bf16 with 4 waves 64 keys (two workgroups share a compute unit; at D = 128 4% faster
// than 32 keys on packed documents, at D = 64 128 keys were 4-10% slower on the window workloads);
// bf16 with 8 waves (no longer launched) 64 keys, 128 for D = 64; fp32 32 keys.
template <class E, int D, int NW, bool VL>
static void launch_dq_nw(const Args& a) {
  typedef typename E::T T;
  constexpr int KB = E::kBytes == 2 ? (NW == 4 ? 2 : (D == 64 ? 4 : 2)) : 1;
  const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
  const int gp = heads_per_workgroup(a.Hq / a.Hkv, NW, ATTN_DQ_HEAD_PACK, a.B, a.Hq, a.Sq);
  const int br = 32 * NW / gp;  // query positions per workgroup
  const int n_qt = (a.Sq + br - 1) / br;
  hipLaunchKernelGGL((dq_kernel<E, D, NW, KB, VL>), dim3((unsigned)(n_qt * a.B * a.Hq / gp)), dim3(NW * 64), 0,
                     (hipStream_t)a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout,
                     (const T*)a.o_in, (const float*)a.lse, a.lse2, a.delta, (T*)a.dq, a.B, a.Hq, a.Hkv, a.Sq,
                     a.Sk, a.causal, a.window, a.sink, a.scale, scale_log2, n_qt, gp, a.docs);
}

// Waves per workgroup: 4, two workgroups per compute unit, for every shape. Against 8-wave
// workgroups (one per compute unit) on the dense and long-window shapes: 1% faster at S = 4096 and
// 8192, 3% on ragged 2777 x 3001, within 1% either way at S = 32768 and with a 2048-key window.
template <class E, int D>
static int launch_bwd_t(const Args& a) {
  if constexpr (E::kBytes == 2) {
    if (a.dsm.ds != nullptr) {  // delta rows, dK / dV with the stored dS, then dQ from it
      typedef typename E::T T;
      const long long rows = (long long)a.B * a.Hq * a.Sq;
      notify_launch("attn_bwd_prep", 0, a.stream);
      hipLaunchKernelGGL((bwd_prep_kernel<E, D>), dim3((unsigned)((rows + 127) / 128)), dim3(256), 0,
                         (hipStream_t)a.stream, (const T*)a.o_in, (const T*)a.dout, (const float*)a.lse,
                         a.lse2, a.delta, rows);
      notify_launch("attn_bwd_prep", 1, a.stream);
      if (launch_dkdv(a) != 0) return -1;
      notify_launch("attn_bwd_dq", 0, a.stream);
      launch_dq_ds<D>(a);
      notify_launch("attn_bwd_dq", 1, a.stream);
      return hipGetLastError() == hipSuccess ? 0 : -1;
    }
  }
  notify_launch("attn_bwd_dq", 0, a.stream);
  if constexpr (E::kBytes == 2) {
    if (a.docs.cu) launch_dq_nw<E, D, kShortWaves, true>(a);
    else launch_dq_nw<E, D, kShortWaves, false>(a);
  } else {
    if (a.docs.cu) launch_dq_nw<E, D, 4, true>(a);
    else launch_dq_nw<E, D, 4, false>(a);
  }
  notify_launch("attn_bwd_dq", 1, a.stream);
  // the dK / dV pass reads the delta and base-2 log-sum-exp rows that dq_kernel stored
  if (launch_dkdv(a) != 0) return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_bwd(const Args& a) {
  if (a.dtype == kBF16) return a.D == 64 ? launch_bwd_t<BF16, 64>(a) : launch_bwd_t<BF16, 128>(a);
  return a.D == 64 ? launch_bwd_t<F32, 64>(a) : launch_bwd_t<F32, 128>(a);
}

}  // namespace fa
