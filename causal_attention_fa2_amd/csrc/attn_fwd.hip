// attn_fwd.hip -- tiled causal / sliding-window GQA attention forward for gfx950.
//
// Method: "KYNETRA FOUNDRY" page, FlashAttention paragraph (query tiles stream key/value tiles
// through on-chip memory with a running max and running sum, rescaling the output accumulator, so
// the S x S matrix never reaches HBM); "CUDA-LLM: A GitHub Repository for Development", section
// "The custom CUDA kernel" (one window parameter for full-causal and sliding-window; the
// log-sum-exp is saved for the backward); Grip paragraph of the first page for the head groups.
//
// Work decomposition (one workgroup = NW waves of 32 query rows: gp query heads of one KV group x
// 32*NW/gp query positions, gp = heads_per_workgroup):
//   * each wave owns 32 query rows of one head; its Q rows stay in registers for the whole kernel as the
//     B operand of S^T = K Q^T (one accumulator column per query, so every lane owns one query:
//     the row max / row sum are in-lane plus one permlane32 swap with the partner lane);
//   * key / value tiles of 32*KB*NH rows stream through a ring of NST swizzled LDS tiles filled by
//     LDS-DMA (global_load_lds_dwordx4): the next NST-1 tiles are in flight while tile s is used,
//     with one workgroup barrier per tile and NH softmax updates of 32*KB keys per tile;
//   * P^T stays in registers and is the B operand of O^T = V^T P^T; V^T comes from LDS with the
//     gfx950 transposing read, so V is never transposed in memory;
//   * key tiles outside a wave's causal / window band are skipped, only boundary tiles are masked;
//   * softmax runs in base 2 (scale * log2 e folded into one FMA per score); the O accumulator
//     is rescaled only when a row max grows by more than 2^8; lse is exported as ln.
//   * grid order: heaviest query tiles first; within one tile index the head chunks of a KV group
//     are consecutive multiples of B*Hkv apart, so with round-robin XCD dispatch a KV group's
//     workgroups share one XCD (and its L2) when B*Hkv is a multiple of 8.
#include "device.h"
#include "launch.h"

namespace fa {

// PG: K and V are pools of a paged cache read through pg (page "KYNETRA FOUNDRY", paged-KV
// paragraph: a per-sequence block table maps token positions to pool blocks); S is then the
// sequence's own key count.
// VL: packed documents (docs); a query sees only keys from its own document's start on.
template <class E, int D, int NW, int KB, int NH, int NST, bool PG, bool VL>
__global__ __launch_bounds__(NW * 64, E::kBytes == 2 ? 2 : 1) void fwd_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, typename E::T* __restrict__ O, float* __restrict__ LSE,
    int B, int Hq, int Hkv, int Sq, int S, int causal, int window, int sink, float scale_log2,
    int n_qt, int gp, PagedKV pg, Docs docs) {
  constexpr int BC = 32 * KB;  // keys per softmax update
  constexpr int BT = BC * NH;  // keys per ring stage (NH updates per workgroup barrier)
  constexpr int DS = D / 16;  // 16-wide contraction steps over the head dimension
  constexpr int DB = D / 32;  // 32-wide output blocks over the head dimension
  typedef LdsTile<E, BT, D> KvTile;
  constexpr int kStage = 2 * KvTile::kBytes;
  // Waves 0 .. CW-1 issue the tile copies: all of them, except in the 8-wave bf16 workgroup with two
  // 64-key updates per stage at D = 128, where waves 0-3 (which the SIMDs serve first, so they wait
  // at the barrier for waves 4-7) issue them all: 2-3% faster there, 1% slower with D = 64 or one
  // update per stage.
  constexpr int CW = E::kBytes == 2 && !PG && NW == 8 && NH == 2 && D == 128 ? 4 : NW;
  constexpr int kOps = 2 * dma_tile_ops<E, BT, D, CW>();  // DMA instructions per copying wave per stage
  static_assert(NST == 2 || NST == 3, "ring depth");
  __shared__ __attribute__((aligned(1024))) char ring[NST * kStage];
  __shared__ int cu_s[VL ? kMaxDocs + 1 : 1];

  const int lane = lane_id();
  const int w = wave_id();
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // gp query heads of one KV group share a workgroup (and its K / V tiles): wave w takes head
  // w % gp of the workgroup's head chunk and query rows q0 + 32 * (w / gp) .. + 31, so the
  // workgroup covers BR = 32 * NW / gp query positions.
  const int BR = 32 * NW / gp;
  const int G = Hq / Hkv;
  const int BG = B * Hkv;
  const int bg = blockIdx.x % BG;
  const int rest = blockIdx.x / BG;
  const int hc = rest % (G / gp);
  const int rank = rest / (G / gp);
  const int qt = causal ? n_qt - 1 - rank : rank;
  const int b = bg / Hkv;
  const int g = bg - b * Hkv;
  const int h = g * G + hc * gp + w % gp;

  if constexpr (PG) S = imin_(imax_(pg.seqlen[b], Sq), pg.max_blocks << pg.shift);
  const int off = S - Sq;  // query row r stands at key position r + off
  const typename E::T* q_bh = Q + (size_t)(b * Hq + h) * Sq * D;
  const typename E::T* k_bg = K + (size_t)bg * S * D;
  const typename E::T* v_bg = V + (size_t)bg * S * D;

  const int q0 = qt * BR;
  const int qw = q0 + 32 * (w / gp);  // first row of this wave
  const int my_q = qw + l32;   // the query row this lane owns
  const bool q_ok = my_q < Sq;
  const int pw = qw + off;     // positions of this wave's rows: pw .. pw + 31
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
  kv_tile_range(q0 + off, imin_(q0 + BR - 1, Sq - 1) + off, S, BT, causal, window, sink, &jt_ns, &jt_lo,
                &jt_hi);
  if constexpr (VL) jt_lo = imax_(jt_lo, doc_start(cu_s, docs.n, q0 + off) / BT);  // no sinks here
  const int n_steps = jt_ns + jt_hi - jt_lo + 1;
  auto tile_of = [&](int s) __attribute__((always_inline)) { return s < jt_ns ? s : jt_lo + s - jt_ns; };

  const bool copier = w < CW;
  const uint32_t dma_off = dma_fast_ok<E, BT, D, CW>() && copier ? dma_lane_off<KvTile, CW>() : 0;  // whole tiles
  auto issue = [&](int s, char* stg) __attribute__((always_inline)) {
    const int j0 = tile_of(s) * BT;
    if constexpr (PG) {
      const int* tab = pg.table + (size_t)b * pg.max_blocks;
      dma_tile_paged<E, BT, D, NW>(stg, K, tab, g, Hkv, pg.shift, pg.num_blocks, j0, S);
      dma_tile_paged<E, BT, D, NW>(stg + KvTile::kBytes, V, tab, g, Hkv, pg.shift, pg.num_blocks, j0, S);
    } else if (!copier) {
    } else if (dma_fast_ok<E, BT, D, CW>() && j0 + BT <= S) {
      if constexpr (dma_fast_ok<E, BT, D, CW>()) {
        dma_tile_fast<E, BT, D, CW>(stg, k_bg, j0, dma_off);
        dma_tile_fast<E, BT, D, CW>(stg + KvTile::kBytes, v_bg, j0, dma_off);
      }
    } else {
      dma_tile<E, BT, D, CW>(stg, k_bg, j0, S);
      dma_tile<E, BT, D, CW>(stg + KvTile::kBytes, v_bg, j0, S);
    }
  };
  issue(0, ring);
  if (NST == 3 && n_steps > 1) issue(1, ring + kStage);

  Frag<E> qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) qf[s] = load_frag_global(q_bh + (size_t)my_q * D + 16 * s + 8 * half, q_ok);

  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};
  wait_vmcnt<0>();  // Q fragments (and the first tiles) have landed before the loop
  float m = kNegInf;  // running max of base-2 scores
  float l = 0.f;      // running sum of exp2(score - m) over this lane's keys

  // one softmax update over the BC keys j0 .. j0 + BC - 1, stored from row kr0 of the stage
  auto compute_general = [&](int j0, const char* k_lds, bool full, int kr0) __attribute__((always_inline)) {
    const char* v_lds = k_lds + KvTile::kBytes;

    // S^T = K Q^T for KB blocks of 32 keys: lane owns query my_q, registers hold keys. Each key
    // block's K fragments are all requested before its products (LDS latency paid once).
    f32x16_t st[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      Frag<E> kfr[DS];
#pragma unroll
      for (int s2 = 0; s2 < DS; ++s2) kfr[s2] = RowFrag<E, KvTile>::get(k_lds, kr0 + 32 * kb + l32, s2);
      __builtin_amdgcn_sched_barrier(0);
      st[kb] = f32x16_t{};
#pragma unroll
      for (int s2 = 0; s2 < DS; ++s2) mma(st[kb], kfr[s2], qf[s2]);
    }
    // The first key block's V^T fragments travel during the softmax.
    Frag<E> vt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) vt[db] = TrFrag<E, KvTile>::get(v_lds, kr0, 32 * db);
    __builtin_amdgcn_sched_barrier(0);

    // Row max of the raw scores (scale > 0 commutes with max); masked keys become -inf, in place
    // (the unmasked scores keep their registers, so the two paths need no copies to merge).
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * kb + acc_row(r);
          mask_neg_inf(st[kb], r, visible(my_p, j, S, causal, window, sink) && !(VL && j < ds_lane));
        }
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
    mx = pair_max(mx) * scale_log2;
    // Rescale a row only when its max grew by more than 2^8 (exponents stay <= 8, so P <= 256
    // and every sum stays far from overflow; O / l does not depend on the reference value). The
    // decision is per row, so a row's arithmetic never depends on other rows' keys; the multiply
    // instructions are skipped when no row of the wave needs them (alpha = 1 is exact otherwise).
    const bool grow = mx > m + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? (m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - mx)) : 1.f;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    m = grow ? mx : m;
    const float neg_m = m == kNegInf ? 0.f : -m;  // row with nothing visible yet: all P are 0

    // P^T = exp2(S^T * scale*log2e - m) as element-type fragments; the row sum adds the fp32
    // values (add_block4 order) before they are rounded for the product.
    Frag<E> pf[KB][2];
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[kb][r] = __builtin_amdgcn_exp2f(fmaf(st[kb][r], scale_log2, neg_m));
      add_block4(st[kb], ps);
#pragma unroll
      for (int t = 0; t < 2; ++t) pf[kb][t] = acc_frag<E>(st[kb], t);
    }
    l += sum4(ps);  // this lane's keys; the partner lane's half of the row is added at the end

    // O^T += V^T P^T, contraction over the tile's keys in the accumulator's row order; the next
    // 16 keys' V^T fragments are requested under the current products.
#pragma unroll
    for (int kt2 = 0; kt2 < 2 * KB; ++kt2) {
      Frag<E> nv[DB];
      if (kt2 + 1 < 2 * KB) {
#pragma unroll
        for (int db = 0; db < DB; ++db) nv[db] = TrFrag<E, KvTile>::get(v_lds, kr0 + 16 * (kt2 + 1), 32 * db);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) mma(acc[db], vt[db], pf[kt2 / 2][kt2 % 2]);
      if (kt2 + 1 < 2 * KB) {
#pragma unroll
        for (int db = 0; db < DB; ++db) vt[db] = nv[db];
      }
    }
  };

  auto compute = [&](int s, const char* k_lds) __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
      const int j0 = tile_of(s) * BT + hb * BC;
      if (block_empty(pw, pw + 31, j0, j0 + BC - 1, S, causal, window, sink)) continue;
      bool full = block_full(pw, pw + 31, j0, j0 + BC - 1, S, causal, window, sink);
      if constexpr (VL) {
        // every key before the first row's document start: empty; all after the last row's: full
        if (j0 + BC - 1 < __builtin_amdgcn_readlane(ds_lane, 0)) continue;
        full = full && __builtin_amdgcn_readlane(ds_lane, 31) <= j0;
      }
      compute_general(j0, k_lds, full, hb * BC);
    }
  };

  ring_run<NST, kStage, kOps>(ring, n_steps, issue, compute);

  l = pair_sum(l);
  if (!q_ok) return;
  const float inv_l = 1.f / l;
  typename E::T* o_row = O + ((size_t)(b * Hq + h) * Sq + my_q) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * db + 8 * r4 + 4 * half;  // registers 4*r4 .. 4*r4+3 hold d .. d+3
      const float x0 = acc[db][4 * r4 + 0] * inv_l, x1 = acc[db][4 * r4 + 1] * inv_l;
      const float x2 = acc[db][4 * r4 + 2] * inv_l, x3 = acc[db][4 * r4 + 3] * inv_l;
      if constexpr (E::kBytes == 2) {
        *reinterpret_cast<u32x2_t*>(o_row + d) = u32x2_t{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
      } else {
        *reinterpret_cast<f32x4_t*>(o_row + d) = f32x4_t{x0, x1, x2, x3};
      }
    }
  }
  if (half == 0) LSE[(size_t)(b * Hq + h) * Sq + my_q] = (m + __log2f(l)) * kLn2;
}

// Ring depth: bf16 two stages (one tile in flight; measured about 1% faster than three at
// S = 4096 and no different on the S_q = 1024 / 1 shapes), f32 three. Key tiles: 64 keys, 128 for
// bf16 with D = 64 (half the products per key block, so a longer tile per step: 12% faster there);
// the paged copy takes at most 64 rows per tile.
template <class E, int D, int NW, bool PG, bool VL, int NH = 1>
static void launch_fwd_nw(const Args& a) {
  constexpr int KB = E::kBytes == 2 ? (PG ? 2 : (D == 64 ? 4 : 2)) : 1;  // paged: tiles of at most 64 rows
  constexpr int NST = E::kBytes == 2 ? kFwdStages : 3;
  const int gp = PG ? 1 : heads_per_workgroup(a.Hq / a.Hkv, NW, ATTN_FWD_HEAD_PACK, a.B, a.Hq, a.Sq);
  const int br = 32 * NW / gp;  // query positions per workgroup
  const int n_qt = (a.Sq + br - 1) / br;
  const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
  hipLaunchKernelGGL((fwd_kernel<E, D, NW, KB, NH, NST, PG, VL>), dim3((unsigned)(n_qt * a.B * a.Hq / gp)),
                     dim3(NW * 64), 0, (hipStream_t)a.stream, (const typename E::T*)a.q, (const typename E::T*)a.k,
                     (const typename E::T*)a.v, (typename E::T*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.Sq, a.Sk,
                     a.causal, a.window, a.sink, scale_log2, n_qt, gp, a.pg, a.docs);
}

// Ring depth: bf16 two stages (one tile in flight; measured about 1% faster than three at
// S = 4096 and no different on the S_q = 1024 / 1 shapes), f32 three. Key tiles: 64 keys, 128 for
// bf16 with D = 64 (half the products per key block, so a longer tile per step: 12% faster there);
// the paged copy takes at most 64 rows per tile. Waves: kFwdWaves, or kShortWaves for short key
// ranges (short_key_ranges).
template <class E, int D>
static int launch_fwd_t(const Args& a) {
  notify_launch("attn_fwd", 0, a.stream);
  if constexpr (E::kBytes == 2) {
    if (a.paged) launch_fwd_nw<E, D, kFwdWaves, true, false>(a);
    else if (a.docs.cu) launch_fwd_nw<E, D, kShortWaves, false, true>(a);
    else if (short_key_ranges(a)) launch_fwd_nw<E, D, kShortWaves, false, false>(a);
    else if (mid_key_ranges(a)) launch_fwd_nw<E, D, kFwdWaves, false, false, 2>(a);
    else launch_fwd_nw<E, D, kFwdWaves, false, false>(a);
  } else {
    if (a.paged) launch_fwd_nw<E, D, 4, true, false>(a);
    else if (a.docs.cu) launch_fwd_nw<E, D, 4, false, true>(a);
    else launch_fwd_nw<E, D, 4, false, false>(a);
  }
  notify_launch("attn_fwd", 1, a.stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_fwd(const Args& a) {
  if (a.dtype == kBF16) return a.D == 64 ? launch_fwd_t<BF16, 64>(a) : launch_fwd_t<BF16, 128>(a);
  return a.D == 64 ? launch_fwd_t<F32, 64>(a) : launch_fwd_t<F32, 128>(a);
}

}  // namespace fa
