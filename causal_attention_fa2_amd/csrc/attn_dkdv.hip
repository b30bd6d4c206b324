// attn_dkdv.hip -- dK / dV pass of the tiled causal / sliding-window GQA attention backward.
//
// Method: "KYNETRA FOUNDRY" page, FlashAttention paragraph (score tiles are recomputed in the
// backward); "CUDA-LLM: A GitHub Repository for Development", section "The custom CUDA kernel"
// (probabilities recomputed from the saved log-sum-exp); Grip paragraph of the first page (dK and
// dV of a shared K/V head sum over its query-head group). The decomposition is described in
// attn_bwd.hip. This translation unit is compiled with the MFMA results kept in VGPRs: the S / dP
// products feed VALU work directly, and the dK / dV accumulators still fit beside them.
#include "device.h"
#include "launch.h"

namespace fa {

template <class E, int D, int NW, int QB, bool VL>
__global__ __launch_bounds__(NW * 64) void dkdv_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
    const float* __restrict__ LSE2, const float* __restrict__ delta, typename E::T* __restrict__ dK,
    typename E::T* __restrict__ dV, float* __restrict__ part, int B, int Hq, int Hkv, int Sq,
    int S, int causal, int window, int sink, float scale, float scale_log2, int n_kt, int n_pairs,
    int hs, Docs docs) {
  constexpr int BC = 32 * NW;  // keys per workgroup
  constexpr int BR = 32 * QB;  // query rows per streamed tile
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  static_assert(NW >= 2, "two waves copy lse and delta");
  typedef LdsTile<E, BR, D> QTile;
  constexpr int kTileOps = dma_tile_ops<E, BR, D, NW>();
  constexpr int kRowOff = 2 * QTile::kBytes;  // lse[64] then -delta[64] (fp32)
  constexpr int kStage = kRowOff + 512;
  __shared__ __attribute__((aligned(1024))) char st0[kStage];
  __shared__ __attribute__((aligned(1024))) char st1[kStage];
  __shared__ __attribute__((aligned(1024))) char st2[kStage];
  __shared__ int cu_s[VL ? kMaxDocs + 1 : 1];

  const int lane = lane_id();
  const int w = wave_id();
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // Work item: (batch x KV head, head part, key-tile pair). Items are dealt to XCDs in contiguous
  // chunks (dispatch is round-robin over the 8 XCDs) so the items of one KV head share an L2.
  const int T = B * Hkv * hs * n_pairs;
  const int wi = (T % 8 == 0) ? (int)(blockIdx.x % 8) * (T / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int pair = wi % n_pairs;
  const int t2 = wi / n_pairs;
  const int hp = t2 % hs;
  const int bg = t2 / hs;
  const int b = bg / Hkv;
  const int G = Hq / Hkv;
  const int hpg = G / hs;
  const int h0 = (bg - b * Hkv) * G + hp * hpg;
  const int ta = pair;
  const int tb = n_kt - 1 - pair;
  const bool two = tb > ta;
  const size_t kv_off = (size_t)bg * S * D;
  const int qoff = S - Sq;  // query row r stands at key position r + qoff
  if constexpr (VL) {
    stage_docs(cu_s, docs.cu + (size_t)b * (docs.n + 1), docs.n, S);
    __syncthreads();
  }
  int de_lane = 0;  // documents: end of this lane's key's document (rows at or past it cannot see it)

  // Segment = one key tile: the workgroup runs key tile ta, then key tile tb.
  int kt = ta, lo = 0, nq = 0, n_steps = 0;
  auto set_segment = [&](int t) __attribute__((always_inline)) {
    int hi;
    kt = t;
    q_tile_range(t * BC, imin_(t * BC + BC - 1, S - 1), S, qoff, BR, causal, window, sink, &lo, &hi);
    if constexpr (VL) hi = imin_(hi, (doc_end(cu_s, docs.n, imin_(t * BC + BC - 1, S - 1)) - 1 - qoff) / BR);
    nq = imax_(hi - lo + 1, 0);  // 0: no query sees these keys, so dK = dV = 0
    n_steps = hpg * nq;
  };
  // step -> (query head, first query row) of the current segment
  // Query tiles are visited from the last one down, so the workgroups of one KV head (which all
  // end at the last query tile) sweep the same Q / dO tiles at about the same time. Steps run
  // head by head; (hh, it) is a step's head offset and query-tile counter.
  constexpr bool kFast = dma_fast_ok<E, BR, D, NW>();
  const uint32_t dma_off = kFast ? dma_lane_off<QTile, NW>() : 0;  // whole tiles: scalar base + offset
  auto issue = [&](int hh, int it, char* stg) __attribute__((always_inline)) {
    const int i0 = (lo + nq - 1 - it) * BR;
    const size_t bh = (size_t)b * Hq + h0 + hh;
    if (kFast && i0 + BR <= Sq) {
      if constexpr (kFast) {
        dma_tile_fast<E, BR, D, NW>(stg, Q + bh * Sq * D, i0, dma_off);
        dma_tile_fast<E, BR, D, NW>(stg + QTile::kBytes, dO + bh * Sq * D, i0, dma_off);
      }
    } else {
      dma_tile<E, BR, D, NW>(stg, Q + bh * Sq * D, i0, Sq);
      dma_tile<E, BR, D, NW>(stg + QTile::kBytes, dO + bh * Sq * D, i0, Sq);
    }
    if (w == 0) dma_row_floats(stg + kRowOff, LSE2 + bh * Sq, i0, Sq);
    if (w == 1) dma_row_floats(stg + kRowOff + 256, delta + bh * Sq, i0, Sq);
  };
  auto advance = [&](int& hh, int& it) __attribute__((always_inline)) {
    if (++it == nq) {
      it = 0;
      ++hh;
    }
  };

  Frag<E> kf[DS], vf[DS];
  f32x16_t dk[DB], dv[DB];
  auto load_kv = [&]() __attribute__((always_inline)) {
    const int my_k = kt * BC + 32 * w + l32;
    const bool ok = my_k < S;
    if constexpr (VL) de_lane = doc_end(cu_s, docs.n, imin_(my_k, S - 1));
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      kf[s] = load_frag_global(K + kv_off + (size_t)my_k * D + 16 * s + 8 * half, ok);
      vf[s] = load_frag_global(V + kv_off + (size_t)my_k * D + 16 * s + 8 * half, ok);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dk[db] = f32x16_t{};
      dv[db] = f32x16_t{};
    }
  };
  // dk[db], dv[db]: register r holds key kw + acc_row(r), column 32*db + l32.
  auto flush = [&]() __attribute__((always_inline)) {
    const int kw = kt * BC + 32 * w;
    const size_t nkv = (size_t)B * Hkv * S * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kw + acc_row(r);
        if (key >= S) continue;
        const size_t off = kv_off + (size_t)key * D + 32 * db + l32;
        if (hs > 1) {
          part[(size_t)(2 * hp) * nkv + off] = dk[db][r];
          part[(size_t)(2 * hp + 1) * nkv + off] = dv[db][r];
        } else if constexpr (E::kBytes == 2) {
          dK[off] = (uint16_t)bf16_bits(dk[db][r] * scale);
          dV[off] = (uint16_t)bf16_bits(dv[db][r]);
        } else {
          dK[off] = dk[db][r] * scale;
          dV[off] = dv[db][r];
        }
      }
    }
  };

  auto compute = [&](int it, const char* q_lds) __attribute__((always_inline)) {
    const char* do_lds = q_lds + QTile::kBytes;
    const float* lse_lds = reinterpret_cast<const float*>(q_lds + kRowOff);
    const float* dl_lds = lse_lds + 64;
    const int i0 = (lo + nq - 1 - it) * BR;
    const int p0 = i0 + qoff;  // position of the tile's first row
    const int kw = kt * BC + 32 * w;
    const int my_k = kw + l32;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int r0 = p0 + 32 * qb;
      if (block_empty(r0, r0 + 31, kw, kw + 31, S, causal, window, sink)) continue;
      bool full = block_full(r0, r0 + 31, kw, kw + 31, S, causal, window, sink);
      if constexpr (VL) {
        // every row at or past the last key's document end: empty; all before the first key's: full
        if (r0 >= __builtin_amdgcn_readlane(de_lane, 31)) continue;
        full = full && r0 + 31 < __builtin_amdgcn_readlane(de_lane, 0);
      }
      // All Q / dO row fragments of this block in flight before the S / dP products, so the
      // LDS latency is paid once per block rather than once per MFMA.
      Frag<E> qa[DS], da[DS];
#pragma unroll
      for (int s2 = 0; s2 < DS; ++s2) {
        qa[s2] = RowFrag<E, QTile>::get(q_lds, 32 * qb + l32, s2);
        da[s2] = RowFrag<E, QTile>::get(do_lds, 32 * qb + l32, s2);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16_t sa = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
      for (int s2 = 0; s2 < DS; ++s2) {
        mma(sa, qa[s2], kf[s2]);
        mma(dp, da[s2], vf[s2]);
      }
      // The first half of the transposed dO / Q fragments travels during the softmax gradient.
      Frag<E> tdo[DB], tq[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        tdo[db] = TrFrag<E, QTile>::get(do_lds, 32 * qb, 32 * db);
        tq[db] = TrFrag<E, QTile>::get(q_lds, 32 * qb, 32 * db);
      }
      __builtin_amdgcn_sched_barrier(0);
      auto softmax_grad = [&](auto maskc) __attribute__((always_inline)) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int rb = 32 * qb + 8 * r4 + 4 * half;  // registers 4*r4 .. 4*r4+3: rows rb .. rb+3
          const f32x4_t lse4 = *reinterpret_cast<const f32x4_t*>(lse_lds + rb);
          const f32x4_t dl4 = *reinterpret_cast<const f32x4_t*>(dl_lds + rb);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int r = 4 * r4 + c;
            float p = __builtin_amdgcn_exp2f(fmaf(sa[r], scale_log2, -lse4[c]));
            if constexpr (decltype(maskc)::value) {
              const int i = p0 + rb + c;
              if (!visible(i, my_k, S, causal, window, sink) || (VL && i >= de_lane)) p = 0.f;
            }
            sa[r] = p;
            dp[r] = p * (dp[r] + dl4[c]);  // the rows hold -delta
          }
        }
      };
      if (full) softmax_grad(IC<0>{});
      else softmax_grad(IC<1>{});
      // dV += P^T dO, dK += dS^T Q (the second half's fragments are fetched under the first).
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const Frag<E> pf = acc_frag<E>(sa, t);
        const Frag<E> sf = acc_frag<E>(dp, t);
        Frag<E> ndo[DB], nq[DB];
        if (t == 0) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            ndo[db] = TrFrag<E, QTile>::get(do_lds, 32 * qb + 16, 32 * db);
            nq[db] = TrFrag<E, QTile>::get(q_lds, 32 * qb + 16, 32 * db);
          }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          mma(dv[db], pf, tdo[db]);
          mma(dk[db], sf, tq[db]);
        }
        if (t == 0) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            tdo[db] = ndo[db];
            tq[db] = nq[db];
          }
        }
      }
    }
  };

  // Step s: wait for this wave's part of tile s, barrier, start the copy of tile s+2 into the stage
  // everyone finished with at step s-1, use tile s. (ch, ct) are step s's counters, (ih, iq) step
  // s+2's.
  int ch, ct, ih, iq;
  auto step = [&](auto stc, int s) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
    char* cur = ST == 0 ? st0 : (ST == 1 ? st1 : st2);
    char* nn = ST == 0 ? st2 : (ST == 1 ? st0 : st1);
    if (s + 1 < n_steps) {
      if (w < 2) wait_vmcnt<2 * kTileOps + 1>();
      else wait_vmcnt<2 * kTileOps>();
    } else {
      wait_vmcnt<0>();
    }
    barrier_keep_vm();
    if (s + 2 < n_steps) {
      issue(ih, iq, nn);
      advance(ih, iq);
    }
    compute(ct, cur);
    advance(ch, ct);
  };
  const int n_seg = two ? 2 : 1;
  for (int seg = 0; seg < n_seg; ++seg) {
    if (seg) barrier_keep_vm();  // every wave is done with the previous segment's stages
    set_segment(seg ? tb : ta);
    load_kv();
    ch = 0, ct = 0, ih = 0, iq = 0;
    if (n_steps > 0) {
      issue(ih, iq, st0);
      advance(ih, iq);
    }
    if (n_steps > 1) {
      issue(ih, iq, st1);
      advance(ih, iq);
    }
    wait_vmcnt<0>();
    for (int s = 0; s < n_steps; s += 3) {
      step(IC<0>{}, s);
      if (s + 1 < n_steps) step(IC<1>{}, s + 1);
      if (s + 2 < n_steps) step(IC<2>{}, s + 2);
    }
    flush();
  }
}

// Split-role dK/dV kernel for bf16: the same decomposition as dkdv_kernel (a workgroup owns 128
// keys of one KV head and streams the head group's query tiles through an LDS-DMA ring, here of two
// stages), but with 8 waves, two per SIMD. Waves w and w + 4 run on the same SIMD and own the same 32 keys:
//   wave w     (S role):  S = Q K^T, P = exp2(S * scale * log2 e - lse * log2 e), dV += P^T dO
//   wave w + 4 (dP role): dP = dO V^T, dS = P o (dP - delta), dK += dS^T Q
// P passes from the S wave to its partner through LDS as bf16 in accumulator layout (2 KB per
// 32 x 32 block). The dP wave runs one query tile behind the S wave (three ring stages, two P
// buffers), so one workgroup barrier per tile orders both the ring and the P exchange, and within
// a tile the two waves of a SIMD share no data: the S wave's exponentials can run beside the dP
// wave's products and the other way round (1.5-5% faster than a schedule with a second barrier
// between the products S / dP and the P exchange). Per wave: its K or V fragments (B operand), its
// dV or dK accumulators and the two blocks' S / dP accumulators -- the two roles' state shares the
// same registers.
template <int D, int QB, bool VL>
__global__ __launch_bounds__(512, 1) void dkdv_pair_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, float* __restrict__ part, int B, int Hq,
    int Hkv, int Sq, int S, int causal, int window, int sink, float scale, float scale_log2,
    int n_kt, int n_pairs, int hs, Docs docs, float* __restrict__ xpart, int nc, int c_lo, int c_len,
    DsMap dsm) {
  typedef BF16 E;
  constexpr int NW = 8;        // waves
  constexpr int NP = 4;        // wave pairs, 32 keys each
  constexpr int BC = 32 * NP;  // keys per workgroup
  constexpr int BR = 32 * QB;  // query rows per streamed tile
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  typedef LdsTile<E, BR, D> QTile;
  static_assert(BR == dkdv_query_rows(D) && BC == 32 * kDkdvWaves, "the host plan assumes these tiles");
  static_assert(BR % 64 == 0 && 2 * (BR / 64) <= NW, "one row copy (64 floats) per wave");
  constexpr int kRowOff = 2 * QTile::kBytes;  // lse[BR] then -delta[BR] (fp32)
  constexpr int kRowWaves = 2 * (BR / 64);      // waves that copy 64 of those floats per tile
  constexpr int kStage = (kRowOff + 8 * BR + 1023) / 1024 * 1024;  // one ring stage, 1 KB aligned
  constexpr int kPBlock = 2048;  // one 32 x 32 bf16 P block, 32 bytes per lane
  constexpr int kPBuf = NP * QB * kPBlock;
  constexpr int kExtra = VL ? 4 * (kMaxDocs + 1) + 8 * kBalancedTiles : 0;
  // Lagged schedule: the dP-role wave works on the query tile before the S-role wave's, so one
  // barrier per step orders both the ring (three stages) and the P exchange (two buffers).
  static_assert(3 * kStage + 2 * kPBuf + kExtra <= 160 * 1024, "three stages and two P buffers fit in LDS");
  __shared__ __attribute__((aligned(1024))) char ring[3 * kStage];
  __shared__ __attribute__((aligned(1024))) char pbuf[2 * kPBuf];
  __shared__ int cu_s[VL ? kMaxDocs + 1 : 1];
  __shared__ int tile_cost[VL ? kBalancedTiles : 1];
  __shared__ int tile_order[VL ? kBalancedTiles : 1];

  const int lane = lane_id();
  const int w = wave_id();
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const bool srole = w < NP;  // S / P / dV wave (else dP / dS / dK)
  const int pw = w & (NP - 1);
  char* pslot = pbuf + pw * QB * kPBlock + lane * 16;

  // Work item: (batch x KV head, head part, key-tile pair), dealt to XCDs in contiguous chunks;
  // with a sink split, items T0.. are chunks 1..nc-1 of key tile 0 (batch x KV head, head part).
  // (the chunk items, which are smaller, follow in launch order and spread over all XCDs)
  const int BG = B * Hkv;
  const int T0 = BG * hs * n_pairs;
  const int bx = (int)blockIdx.x;
  const int wi = (bx < T0 && T0 % 8 == 0) ? (bx % 8) * (T0 / 8) + bx / 8 : bx;
  const bool extra = wi >= T0;
  const int e = wi - T0;
  const int pair = extra ? 0 : wi % n_pairs;
  const int t2 = extra ? e / (nc - 1) : wi / n_pairs;
  const int chunk = extra ? 1 + e % (nc - 1) : 0;
  const int hp = t2 % hs;
  const int bg = t2 / hs;
  const int b = bg / Hkv;
  const int G = Hq / Hkv;
  const int hpg = G / hs;
  const int h0 = (bg - b * Hkv) * G + hp * hpg;
  int ta = pair;
  int tb = n_kt - 1 - pair;
  const bool two = !extra && tb > ta;
  const size_t kv_off = (size_t)bg * S * D;
  const int qoff = S - Sq;  // query row r stands at key position r + qoff
  if constexpr (VL) {
    stage_docs(cu_s, docs.cu + (size_t)b * (docs.n + 1), docs.n, S);
    __syncthreads();
  }
  int de_lane = 0;  // documents: end of this lane's key's document (rows at or past it cannot see it)

  // Query tiles that key tile t's segment streams: [*lo, *lo + return value).
  auto tile_queries = [&](int t, int* lo) __attribute__((always_inline)) {
    int hi;
    q_tile_range(t * BC, imin_(t * BC + BC - 1, S - 1), S, qoff, BR, causal, window, sink, lo, &hi);
    if constexpr (VL) hi = imin_(hi, (doc_end(cu_s, docs.n, imin_(t * BC + BC - 1, S - 1)) - 1 - qoff) / BR);
    return imax_(hi - *lo + 1, 0);
  };
  if constexpr (VL) {
    // Packed documents: a key tile's work depends on where it lies in its document, so the
    // pairing of tile j with tile n_kt-1-j no longer balances. Every workgroup ranks the tiles by
    // their query-tile count (ties by index: the same order everywhere) and pair p takes the p-th
    // heaviest and the p-th lightest. Up to kBalancedTiles tiles; longer rows keep the plain pairing.
    if (n_kt <= kBalancedTiles) {
      for (int t = threadIdx.x; t < n_kt; t += blockDim.x) {
        int l0;
        tile_cost[t] = tile_queries(t, &l0);
      }
      __syncthreads();
      for (int t = threadIdx.x; t < n_kt; t += blockDim.x) {
        const int c = tile_cost[t];
        int rank = 0;
        for (int u = 0; u < n_kt; ++u) {
          const int cu = tile_cost[u];
          rank += (cu > c || (cu == c && u < t)) ? 1 : 0;
        }
        tile_order[rank] = t;
      }
      __syncthreads();
      if (!extra) {
        ta = tile_order[pair];
        tb = tile_order[n_kt - 1 - pair];
      }
    }
  }

  int kt = ta, lo = 0, nq = 0, n_steps = 0;
  auto set_segment = [&](int t) __attribute__((always_inline)) {
    kt = t;
    nq = tile_queries(t, &lo);  // 0: no query sees these keys, so dK = dV = 0
    if (nc > 1 && t == 0) {  // this item's chunk of key tile 0's query tiles
      const int hi = lo + nq - 1;
      lo = c_lo + chunk * c_len;
      nq = imax_(imin_(hi, lo + c_len - 1) - lo + 1, 0);
    }
    n_steps = hpg * nq;
  };
  // Query tiles run from the last one down, head by head; (hh, it) = head offset, tile counter.
  // The S-role waves 0 .. CW-1 issue the Q / dO tile copies right after each barrier (waves 0 and 1
  // also the lse / delta rows), so the dP-role waves, whose steps take longer, never wait for copy
  // instructions: 1.5-3.5% faster than copies shared by all eight waves at D = 128, no different at
  // D = 64; with all eight waves copying, copies spread between the products of a step had been 1%
  // faster, with the S-role waves copying they are 1-1.5% slower than copies right after the barrier.
  constexpr int CW = NP;
  constexpr bool kFast = dma_fast_ok<E, BR, D, CW>();
  const bool copier = w < CW;
  const uint32_t dma_off = kFast && copier ? dma_lane_off<QTile, CW>() : 0;  // whole tiles: scalar base + offset
  auto issue = [&](int hh, int it, char* stg) __attribute__((always_inline)) {
    const int i0 = (lo + nq - 1 - it) * BR;
    const size_t bh = (size_t)b * Hq + h0 + hh;
    if (!copier) {
    } else if (kFast && i0 + BR <= Sq) {
      if constexpr (kFast) {
        dma_tile_fast<E, BR, D, CW>(stg, Q + bh * Sq * D, i0, dma_off);
        dma_tile_fast<E, BR, D, CW>(stg + QTile::kBytes, dO + bh * Sq * D, i0, dma_off);
      }
    } else {
      dma_tile<E, BR, D, CW>(stg, Q + bh * Sq * D, i0, Sq);
      dma_tile<E, BR, D, CW>(stg + QTile::kBytes, dO + bh * Sq * D, i0, Sq);
    }
    if (w < kRowWaves) {  // wave 2c copies lse rows 64c.., wave 2c+1 the delta rows 64c..
      const int c = w >> 1;
      dma_row_floats(stg + kRowOff + (w & 1) * 4 * BR + 256 * c, ((w & 1) ? delta : LSE2) + bh * Sq, i0 + 64 * c, Sq);
    }
  };
  auto advance = [&](int& hh, int& it) __attribute__((always_inline)) {
    if (++it == nq) {
      it = 0;
      ++hh;
    }
  };

  // Everything below is specialised on the wave's role (fixed for the whole kernel), so the two
  // roles' values never meet in one register allocation: no copies where the paths rejoin.
  auto run = [&](auto role_c) __attribute__((always_inline)) {
    constexpr bool SR = decltype(role_c)::value != 0;
    Frag<E> kvf[DS];   // K (S role) or V (dP role) rows of this pair's keys: the B operand
    f32x16_t acc[DB];  // dV (S role) or dK (dP role); register r holds key kw + acc_row(r)
    auto load_kv = [&]() __attribute__((always_inline)) {
      const int my_k = kt * BC + 32 * pw + l32;
      const bool ok = my_k < S;
      if constexpr (VL) de_lane = doc_end(cu_s, docs.n, imin_(my_k, S - 1));
      const uint16_t* src = (SR ? K : V) + kv_off + (size_t)my_k * D + 8 * half;
#pragma unroll
      for (int s2 = 0; s2 < DS; ++s2) kvf[s2] = load_frag_global(src + 16 * s2, ok);
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};
    };
    auto flush = [&]() __attribute__((always_inline)) {
      const int kw = kt * BC + 32 * pw;
      const size_t nkv = (size_t)B * Hkv * S * D;
      const float mul = SR ? 1.f : scale;
      // sink split: key tile 0 goes to this chunk's slot [chunk][hp][bg][dK, dV][BC][D]
      const bool to_x = nc > 1 && kt == 0;
      float* xs_slot = to_x ? xpart + ((((size_t)chunk * hs + hp) * BG + bg) * 2 + (SR ? 1 : 0)) * BC * D : nullptr;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kw + acc_row(r);
          if (key >= S) continue;
          const size_t o = kv_off + (size_t)key * D + 32 * db + l32;
          if (to_x) {
            xs_slot[(size_t)key * D + 32 * db + l32] = acc[db][r];
          } else if (hs > 1) {
            part[(size_t)(2 * hp + (SR ? 1 : 0)) * nkv + o] = acc[db][r];
          } else {
            (SR ? dV : dK)[o] = (uint16_t)bf16_bits(acc[db][r] * mul);
          }
        }
      }
    };

    // One 64-row query tile. Blocks of 32 rows that see none of this pair's keys
    // (the causal diagonal, window edges) are computed like partial ones: every P is 0, so they
    // add exact zeros to dV and dK.
    auto compute = [&](int hh, int it, const char* q_lds, char* ps) __attribute__((always_inline)) {
      const char* do_lds = q_lds + QTile::kBytes;
      const float* lse_lds = reinterpret_cast<const float*>(q_lds + kRowOff);
      const float* dl_lds = lse_lds + BR;
      const int i0 = (lo + nq - 1 - it) * BR;
      const int p0 = i0 + qoff;  // position of the tile's first row
      const int kw = kt * BC + 32 * pw;
      const int my_k = kw + l32;
      f32x16_t xs[QB];  // S -> P (S role) or dP -> dS (dP role)
      Frag<E> pfr[QB][2];  // S role: P as the bf16 operand of dV += P^T dO
      // Phase 1: S = Q K^T and P (S role), dP = dO V^T (dP role).
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int r0 = p0 + 32 * qb;
        Frag<E> fr[DS];
#pragma unroll
        for (int s2 = 0; s2 < DS; ++s2) fr[s2] = RowFrag<E, QTile>::get(SR ? q_lds : do_lds, 32 * qb + l32, s2);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SR) {
          xs[qb] = f32x16_t{};
        } else {  // dP products start from -delta of each row, so they leave dP - delta
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4_t nd4 = *reinterpret_cast<const f32x4_t*>(dl_lds + 32 * qb + 8 * r4 + 4 * half);
#pragma unroll
            for (int c = 0; c < 4; ++c) xs[qb][4 * r4 + c] = nd4[c];
          }
        }
#pragma unroll
        for (int s2 = 0; s2 < DS; ++s2) mma(xs[qb], fr[s2], kvf[s2]);
        if constexpr (SR) {
          bool full = block_full(r0, r0 + 31, kw, kw + 31, S, causal, window, sink);
          if constexpr (VL) full = full && r0 + 31 < __builtin_amdgcn_readlane(de_lane, 0);
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int rb = 32 * qb + 8 * r4 + 4 * half;  // registers 4*r4 .. 4*r4+3: rows rb .. rb+3
            const f32x4_t lse4 = *reinterpret_cast<const f32x4_t*>(lse_lds + rb);
#pragma unroll
            for (int c = 0; c < 4; ++c)
              xs[qb][4 * r4 + c] = __builtin_amdgcn_exp2f(fmaf(xs[qb][4 * r4 + c], scale_log2, -lse4[c]));
          }
          if (!full) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int i = p0 + 32 * qb + acc_row(r);
              mask_zero(xs[qb], r, visible(i, my_k, S, causal, window, sink) && !(VL && i >= de_lane));
            }
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            pfr[qb][t] = acc_frag<E>(xs[qb], t);  // the dV operand too: converted once
            *reinterpret_cast<u32x4_t*>(ps + qb * kPBlock + t * 1024) = pfr[qb][t].v;
          }
        }
      }
      // Phase 2: dV += P^T dO (S role); dS = P o (dP - delta), dK += dS^T Q (dP role), and with
      // a stored dS its blocks that lie in their query block's strip (the rest are all zero: no
      // visible pair) go out as they enter the products.
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        char* ds_dst = nullptr;
        if constexpr (!SR) {
          const int i = i0 / 32 + qb, kb = kt * (BC / 32) + pw;
          if (dsm.ds != nullptr && i < dsm.nqb && kb < ds_strip_len(dsm, i))
            ds_dst = reinterpret_cast<char*>(dsm.ds) + ds_block_off(dsm, bg, hp * hpg + hh, i, kb);
        }
        if constexpr (!SR) {
          const u32x4_t pa = *reinterpret_cast<const u32x4_t*>(ps + qb * kPBlock);
          const u32x4_t pb = *reinterpret_cast<const u32x4_t*>(ps + qb * kPBlock + 1024);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t word = (r < 8 ? pa : pb)[(r & 7) >> 1];
            const float p = __uint_as_float((r & 1) ? (word & 0xFFFF0000u) : (word << 16));
            xs[qb][r] = p * xs[qb][r];  // xs already holds dP - delta
          }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          Frag<E> tr[DB];  // dO^T (S role) or Q^T (dP role), rows 32*qb + 16t ..
#pragma unroll
          for (int db = 0; db < DB; ++db) tr[db] = TrFrag<E, QTile>::get(SR ? do_lds : q_lds, 32 * qb + 16 * t, 32 * db);
          const Frag<E> af = SR ? pfr[qb][t] : acc_frag<E>(xs[qb], t);
          // chunk t*64 + half*32 + (key ^ 4*(2t + half)) of the block; streamed past the caches
          // (read back by the dQ pass only after this pass: 12% faster dQ than cached stores)
          if (!SR && ds_dst != nullptr)
            __builtin_nontemporal_store(
                af.v, reinterpret_cast<u32x4_t*>(ds_dst + t * 1024 + half * 512 + ((l32 ^ (8 * t + 4 * half)) << 4)));
#pragma unroll
          for (int db = 0; db < DB; ++db) mma(acc[db], af, tr[db]);
        }
      }
    };

    int ch, ct, ih, iq;
    // Lagged: interval k (after its one barrier) copies tile k + 1 into the stage tile k - 2 used,
    // while the S wave takes step k (tile k % 3, P buffer k % 2) and the dP wave step k - 1, whose P
    // the barrier has just published. Tile k - 2's last reader ran in interval k - 1, and so did the
    // last reader of P buffer k % 2.
    auto lagged = [&]() __attribute__((always_inline)) {
      int sc = 0;  // stage of tile k
      for (int k = 0; k <= n_steps; ++k) {
        const int sn = sc == 2 ? 0 : sc + 1;  // stage of tile k + 1
        const int sp = sc == 0 ? 2 : sc - 1;  // stage of tile k - 1
        // only the S-role waves copy; the dP-role waves' own memory operations are the stored dS
        // blocks, which nothing here waits for
        if constexpr (SR) wait_vmcnt<0>();
        barrier_keep_vm();
        if (k + 1 < n_steps) {
          issue(ih, iq, ring + sn * kStage);
          advance(ih, iq);
        }
        if constexpr (SR) {
          if (k < n_steps) {
            compute(ch, ct, ring + sc * kStage, pslot + (k & 1) * kPBuf);
            advance(ch, ct);
          }
        } else {
          if (k > 0) {
            compute(ch, ct, ring + sp * kStage, pslot + ((k - 1) & 1) * kPBuf);
            advance(ch, ct);
          }
        }
        sc = sn;
      }
    };
    const int n_seg = two ? 2 : 1;
    for (int seg = 0; seg < n_seg; ++seg) {
      if (seg) barrier_keep_vm();  // every wave is done with the previous segment's stages
      set_segment(seg ? tb : ta);
      load_kv();
      ch = 0, ct = 0, ih = 0, iq = 0;
      if (n_steps > 0) {
        issue(ih, iq, ring);
        advance(ih, iq);
      }
      if (n_steps > 0) lagged();
      flush();
    }
  };
  if (srole) run(IC<1>{});
  else run(IC<0>{});
}

// Adds the hs head-part partials. Rows below skip_rows of every (batch, KV head) are left to
// dkdv_chunk_reduce_kernel (their partials live in the sink-split slots instead).
template <class E>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(const float* __restrict__ part,
                                                          typename E::T* __restrict__ dK,
                                                          typename E::T* __restrict__ dV,
                                                          size_t n, int hs, float scale, int S, int D,
                                                          int skip_rows) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  if ((int)((i / D) % S) < skip_rows) return;
  f32x4_t sk = *reinterpret_cast<const f32x4_t*>(part + i);
  f32x4_t sv = *reinterpret_cast<const f32x4_t*>(part + n + i);
  for (int p = 1; p < hs; ++p) {
    sk += *reinterpret_cast<const f32x4_t*>(part + (size_t)(2 * p) * n + i);
    sv += *reinterpret_cast<const f32x4_t*>(part + (size_t)(2 * p + 1) * n + i);
  }
  sk *= scale;
  if constexpr (E::kBytes == 2) {
    *reinterpret_cast<u32x2_t*>(dK + i) = u32x2_t{pack_bf16x2(sk[0], sk[1]), pack_bf16x2(sk[2], sk[3])};
    *reinterpret_cast<u32x2_t*>(dV + i) = u32x2_t{pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3])};
  } else {
    *reinterpret_cast<f32x4_t*>(dK + i) = sk;
    *reinterpret_cast<f32x4_t*>(dV + i) = sv;
  }
}

// Sink split: dK / dV of key tile 0 (rows < min(BC, S) of every batch x KV head) = the sum over
// the nc * hs chunk slots, in a fixed order; dK takes the softmax scale here. One element per
// thread, slots read four at a time.
__global__ __launch_bounds__(256) void dkdv_chunk_reduce_kernel(const float* __restrict__ xpart,
                                                                uint16_t* __restrict__ dK,
                                                                uint16_t* __restrict__ dV, int BG,
                                                                int S, int D, int BC, int parts,
                                                                float scale) {
  const int rows = BC < S ? BC : S;
  const size_t per_bg = (size_t)BC * D;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // over BG x BC x D
  if (i >= (size_t)BG * per_bg) return;
  const int bg = (int)(i / per_bg);
  const size_t r = i - (size_t)bg * per_bg;  // key * D + d
  if ((int)(r / D) >= rows) return;
  const size_t stride = (size_t)BG * 2 * per_bg;  // from one slot to the next
  const float* pk = xpart + (size_t)bg * 2 * per_bg + r;
  float sk = 0.f, sv = 0.f;
  int p = 0;
  for (; p + 4 <= parts; p += 4) {
    float k4[4], v4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      k4[u] = pk[(size_t)(p + u) * stride];
      v4[u] = pk[(size_t)(p + u) * stride + per_bg];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sk += k4[u];
      sv += v4[u];
    }
  }
  for (; p < parts; ++p) {
    sk += pk[(size_t)p * stride];
    sv += pk[(size_t)p * stride + per_bg];
  }
  const size_t o = (size_t)bg * S * D + r;
  dK[o] = (uint16_t)bf16_bits(sk * scale);
  dV[o] = (uint16_t)bf16_bits(sv);
}

template <class E, int D>
static int launch_dkdv_t(const Args& a) {
  {
    hipStream_t st = (hipStream_t)a.stream;
    typedef typename E::T T;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    constexpr int NW = kDkdvWaves;
    constexpr int QB = E::kBytes == 2 ? dkdv_query_rows(D) / 32 : 1;
    DkdvPlan p = dkdv_plan(a.B, a.Hq, a.Hkv, a.Sk);
    if (E::kBytes == 2 && a.xpart != nullptr && !a.docs.cu)
      dkdv_sink_split(p, a.B, a.Hq, a.Hkv, a.Sq, a.Sk, D, a.window, a.sink, a.causal != 0);
    dim3 grid((unsigned)((p.n_pairs + p.nc - 1) * a.B * a.Hkv * p.hs));
    notify_launch("attn_bwd_dkdv", 0, a.stream);
    if constexpr (E::kBytes == 2) {
      auto kern = a.docs.cu ? dkdv_pair_kernel<D, QB, true> : dkdv_pair_kernel<D, QB, false>;
      hipLaunchKernelGGL(kern, grid, dim3(512), 0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                         (const T*)a.dout, (const float*)a.lse2, (const float*)a.delta, (T*)a.dk,
                         (T*)a.dv, a.part, a.B, a.Hq, a.Hkv, a.Sq, a.Sk, a.causal, a.window, a.sink,
                         a.scale, scale_log2, p.n_kt, p.n_pairs, p.hs, a.docs, a.xpart, p.nc, p.c_lo,
                         p.c_len, a.dsm);
    } else {
      auto kern = a.docs.cu ? dkdv_kernel<E, D, NW, QB, true> : dkdv_kernel<E, D, NW, QB, false>;
      hipLaunchKernelGGL(kern, grid, dim3(NW * 64), 0, st, (const T*)a.q, (const T*)a.k,
                         (const T*)a.v, (const T*)a.dout, (const float*)a.lse2, (const float*)a.delta,
                         (T*)a.dk, (T*)a.dv, a.part, a.B, a.Hq, a.Hkv, a.Sq, a.Sk, a.causal, a.window,
                         a.sink, a.scale, scale_log2, p.n_kt, p.n_pairs, p.hs, a.docs);
    }
    notify_launch("attn_bwd_dkdv", 1, a.stream);
    if (p.hs > 1 && a.dsm.ds == nullptr) {  // with a stored dS the dQ launch adds the parts
      const size_t n = (size_t)a.B * a.Hkv * a.Sk * D;
      dim3 rgrid((unsigned)((n / 4 + 255) / 256)), rblock(256);
      notify_launch("attn_bwd_dkdv_reduce", 0, a.stream);
      hipLaunchKernelGGL((dkdv_reduce_kernel<E>), rgrid, rblock, 0, st, (const float*)a.part,
                         (T*)a.dk, (T*)a.dv, n, p.hs, a.scale, a.Sk, D, p.nc > 1 ? 32 * kDkdvWaves : 0);
      notify_launch("attn_bwd_dkdv_reduce", 1, a.stream);
    }
    if constexpr (E::kBytes == 2) {
      if (p.nc > 1) {
        const int BC = 32 * kDkdvWaves;
        const size_t n = (size_t)a.B * a.Hkv * BC * D;
        dim3 cgrid((unsigned)((n + 255) / 256)), cblock(256);
        notify_launch("attn_bwd_dkdv_chunks", 0, a.stream);
        hipLaunchKernelGGL(dkdv_chunk_reduce_kernel, cgrid, cblock, 0, st, (const float*)a.xpart,
                           (uint16_t*)a.dk, (uint16_t*)a.dv, a.B * a.Hkv, a.Sk, D, BC, p.nc * p.hs,
                           a.scale);
        notify_launch("attn_bwd_dkdv_chunks", 1, a.stream);
      }
    }
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_dkdv(const Args& a) {
  if (a.dtype == kBF16) return a.D == 64 ? launch_dkdv_t<BF16, 64>(a) : launch_dkdv_t<BF16, 128>(a);
  return a.D == 64 ? launch_dkdv_t<F32, 64>(a) : launch_dkdv_t<F32, 128>(a);
}

}  // namespace fa
