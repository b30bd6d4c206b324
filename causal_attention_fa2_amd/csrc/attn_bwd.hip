// attn_bwd.hip -- tiled causal / sliding-window GQA attention backward for gfx950.
//
// Method: "KYNETRA FOUNDRY" page, FlashAttention paragraph (the backward recomputes score tiles on
// the fly rather than storing them); "CUDA-LLM: A GitHub Repository for Development", section "The
// custom CUDA kernel" (probabilities are recomputed from the saved log-sum-exp); Grip paragraph of
// the first page (dK and dV of a shared K/V head sum over its query-head group).
//
// Launches on the caller's stream, no atomics anywhere:
//   1. delta_kernel: delta_i = sum_d dO_id * O_id in fp32 (O as the forward stored it), and the
//      base-2 log-sum-exp lse_i * log2(e) that the gradient kernels exponentiate against.
//   2. dkdv_kernel: each wave owns 32 keys whose K and V rows stay in registers as B operands of
//      S = Q K^T and dP = dO V^T, so a lane owns one key and its accumulator holds query rows --
//      exactly the contraction side that dV += P^T dO and dK += dS^T Q need. Query / dO / lse /
//      delta tiles of the group's heads stream through a 3-stage LDS-DMA ring (two tiles in
//      flight ahead of the one in use); dK and dV for the
//      group accumulate in registers. A workgroup takes key tile j and then key tile T-1-j, so
//      under the causal mask every workgroup does the same amount of work. When that leaves too
//      few workgroups to fill the GPU, the head group is split into `hs` parts whose fp32 partial
//      sums go to the workspace and
//   3. dkdv_reduce_kernel adds them in a fixed order (deterministic) and rounds to the element type.
//   4. dq_kernel: lanes own queries (as in the forward): S^T = K Q^T and dP^T = V dO^T from LDS
//      key/value tiles, dS^T in registers is the B operand of dQ^T += K^T dS^T with K^T read
//      through the transposing LDS read.
// P and dS are rounded to the element type only as MFMA operands; all sums are fp32.
#include "device.h"
#include "launch.h"

namespace fa {

template <class E, int D>
__global__ __launch_bounds__(256) void delta_kernel(const typename E::T* __restrict__ O,
                                                    const typename E::T* __restrict__ dO,
                                                    const float* __restrict__ LSE,
                                                    float* __restrict__ delta,
                                                    float* __restrict__ lse2, int rows) {
  constexpr int TPR = D / 8;       // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;   // rows per block
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float s = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + part * 8;
    if constexpr (E::kBytes == 2) {
      const u32x4_t o = *reinterpret_cast<const u32x4_t*>(O + off);
      const u32x4_t d = *reinterpret_cast<const u32x4_t*>(dO + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s += bf16_to_f32(o[e] & 0xFFFFu) * bf16_to_f32(d[e] & 0xFFFFu);
        s += bf16_to_f32(o[e] >> 16) * bf16_to_f32(d[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) s += O[off + e] * dO[off + e];
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (part == 0 && row < rows) {
    delta[row] = s;
    lse2[row] = LSE[row] * kLog2e;  // base-2 log-sum-exp used by both gradient kernels
  }
}

template <class E, int D, int NW, int QB>
__global__ __launch_bounds__(NW * 64) void dkdv_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
    const float* __restrict__ LSE2, const float* __restrict__ delta, typename E::T* __restrict__ dK,
    typename E::T* __restrict__ dV, float* __restrict__ part, int B, int Hq, int Hkv, int S,
    int causal, int window, float scale, float scale_log2, int n_kt, int n_pairs, int hs) {
  constexpr int BC = 32 * NW;  // keys per workgroup
  constexpr int BR = 32 * QB;  // query rows per streamed tile
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  static_assert(NW >= 2, "two waves copy lse and delta");
  typedef LdsTile<E, BR, D> QTile;
  constexpr int kTileOps = dma_tile_ops<E, BR, D, NW>();
  constexpr int kRowOff = 2 * QTile::kBytes;  // lse[64] then delta[64] (fp32)
  constexpr int kStage = kRowOff + 512;
  __shared__ __attribute__((aligned(1024))) char st0[kStage];
  __shared__ __attribute__((aligned(1024))) char st1[kStage];
  __shared__ __attribute__((aligned(1024))) char st2[kStage];

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

  // Segment = one key tile: the workgroup runs key tile ta, then key tile tb.
  int kt = ta, lo = 0, nq = 0, n_steps = 0;
  auto set_segment = [&](int t) __attribute__((always_inline)) {
    int hi;
    kt = t;
    q_tile_range(t * BC, imin_(t * BC + BC - 1, S - 1), S, BR, causal, window, &lo, &hi);
    nq = hi - lo + 1;
    n_steps = hpg * nq;
  };
  // step -> (query head, first query row) of the current segment
  // Query tiles are visited from the last one down, so the workgroups of one KV head (which all
  // end at the last query tile) sweep the same Q / dO tiles at about the same time.
  auto issue = [&](int s, char* stg) __attribute__((always_inline)) {
    const int h = h0 + s / nq;
    const int i0 = (lo + nq - 1 - s % nq) * BR;
    const size_t bh = (size_t)b * Hq + h;
    dma_tile<E, BR, D, NW>(stg, Q + bh * S * D, i0, S);
    dma_tile<E, BR, D, NW>(stg + QTile::kBytes, dO + bh * S * D, i0, S);
    if (w == 0) dma_row_floats(stg + kRowOff, LSE2 + bh * S, i0, S);
    if (w == 1) dma_row_floats(stg + kRowOff + 256, delta + bh * S, i0, S);
  };

  Frag<E> kf[DS], vf[DS];
  f32x16_t dk[DB], dv[DB];
  auto load_kv = [&]() __attribute__((always_inline)) {
    const int my_k = kt * BC + 32 * w + l32;
    const bool ok = my_k < S;
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

  auto compute = [&](int s, const char* q_lds) __attribute__((always_inline)) {
    const char* do_lds = q_lds + QTile::kBytes;
    const float* lse_lds = reinterpret_cast<const float*>(q_lds + kRowOff);
    const float* dl_lds = lse_lds + 64;
    const int i0 = (lo + nq - 1 - s % nq) * BR;
    const int kw = kt * BC + 32 * w;
    const int my_k = kw + l32;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int r0 = i0 + 32 * qb;
      if (block_empty(r0, r0 + 31, kw, kw + 31, S, causal, window)) continue;
      const bool full = block_full(r0, r0 + 31, kw, kw + 31, S, causal, window);
      f32x16_t sa = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
      for (int s2 = 0; s2 < DS; ++s2) {
        mma(sa, RowFrag<E, QTile>::get(q_lds, 32 * qb + l32, s2), kf[s2]);
        mma(dp, RowFrag<E, QTile>::get(do_lds, 32 * qb + l32, s2), vf[s2]);
      }
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
              if (!visible(i0 + rb + c, my_k, S, causal, window)) p = 0.f;
            }
            sa[r] = p;
            dp[r] = p * (dp[r] - dl4[c]);
          }
        }
      };
      if (full) softmax_grad(IC<0>{});
      else softmax_grad(IC<1>{});
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const Frag<E> pf = acc_frag<E>(sa, t);
        const Frag<E> sf = acc_frag<E>(dp, t);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          mma(dv[db], pf, TrFrag<E, QTile>::get(do_lds, 32 * qb + 16 * t, 32 * db));
          mma(dk[db], sf, TrFrag<E, QTile>::get(q_lds, 32 * qb + 16 * t, 32 * db));
        }
      }
    }
  };

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
    if (s + 2 < n_steps) issue(s + 2, nn);
    compute(s, cur);
  };
  const int n_seg = two ? 2 : 1;
  for (int seg = 0; seg < n_seg; ++seg) {
    if (seg) barrier_keep_vm();  // every wave is done with the previous segment's stages
    set_segment(seg ? tb : ta);
    load_kv();
    issue(0, st0);
    if (n_steps > 1) issue(1, st1);
    wait_vmcnt<0>();
    for (int s = 0; s < n_steps; s += 3) {
      step(IC<0>{}, s);
      if (s + 1 < n_steps) step(IC<1>{}, s + 1);
      if (s + 2 < n_steps) step(IC<2>{}, s + 2);
    }
    flush();
  }
}

// dK = scale * sum_p part[p].dK, dV = sum_p part[p].dV over the hs head parts, in part order.
template <class E>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(const float* __restrict__ part,
                                                          typename E::T* __restrict__ dK,
                                                          typename E::T* __restrict__ dV,
                                                          size_t n, int hs, float scale) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
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

template <class E, int D, int NW, int KB>
__global__ __launch_bounds__(NW * 64) void dq_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
    const float* __restrict__ LSE2, const float* __restrict__ delta, typename E::T* __restrict__ dQ,
    int B, int Hq, int Hkv, int S, int causal, int window, float scale, float scale_log2, int n_qt) {
  constexpr int BR = 32 * NW;
  constexpr int BC = 32 * KB;
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  typedef LdsTile<E, BC, D> KvTile;
  constexpr int kStage = 2 * KvTile::kBytes;
  constexpr int kOps = 2 * dma_tile_ops<E, BC, D, NW>();
  __shared__ __attribute__((aligned(1024))) char st0[kStage];
  __shared__ __attribute__((aligned(1024))) char st1[kStage];
  __shared__ __attribute__((aligned(1024))) char st2[kStage];

  const int lane = lane_id();
  const int w = wave_id();
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // Same order as the forward: heaviest query tiles first, a KV group's heads on one XCD.
  const int G = Hq / Hkv;
  const int BG = B * Hkv;
  const int bg = blockIdx.x % BG;
  const int rest = blockIdx.x / BG;
  const int hh = rest % G;
  const int rank = rest / G;
  const int qt = causal ? n_qt - 1 - rank : rank;
  const int b = bg / Hkv;
  const int h = (bg - b * Hkv) * G + hh;
  const size_t q_off = (size_t)(b * Hq + h) * S * D;
  const typename E::T* k_bg = K + (size_t)bg * S * D;
  const typename E::T* v_bg = V + (size_t)bg * S * D;

  const int q0 = qt * BR;
  const int qw = q0 + 32 * w;
  const int my_q = qw + l32;
  const bool q_ok = my_q < S;

  int jt_lo, jt_hi;
  kv_tile_range(q0, imin_(q0 + BR - 1, S - 1), S, BC, causal, window, &jt_lo, &jt_hi);
  const int n_steps = jt_hi - jt_lo + 1;
  auto issue = [&](int s, char* stg) __attribute__((always_inline)) {
    const int j0 = (jt_lo + s) * BC;
    dma_tile<E, BC, D, NW>(stg, k_bg, j0, S);
    dma_tile<E, BC, D, NW>(stg + KvTile::kBytes, v_bg, j0, S);
  };
  issue(0, st0);
  if (n_steps > 1) issue(1, st1);

  Frag<E> qf[DS], df[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    qf[s] = load_frag_global(Q + q_off + (size_t)my_q * D + 16 * s + 8 * half, q_ok);
    df[s] = load_frag_global(dO + q_off + (size_t)my_q * D + 16 * s + 8 * half, q_ok);
  }
  const size_t row_idx = (size_t)(b * Hq + h) * S + (q_ok ? my_q : 0);
  const float nlse2 = -LSE2[row_idx];
  const float dl = delta[row_idx];
  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};
  wait_vmcnt<0>();

  auto compute = [&](int s, const char* k_lds) __attribute__((always_inline)) {
    const char* v_lds = k_lds + KvTile::kBytes;
    const int j0 = (jt_lo + s) * BC;
    if (block_empty(qw, qw + 31, j0, j0 + BC - 1, S, causal, window)) return;
    const bool full = block_full(qw, qw + 31, j0, j0 + BC - 1, S, causal, window);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16_t st = f32x16_t{}, dpt = f32x16_t{};
#pragma unroll
      for (int s2 = 0; s2 < DS; ++s2) {
        mma(st, RowFrag<E, KvTile>::get(k_lds, 32 * kb + l32, s2), qf[s2]);
        mma(dpt, RowFrag<E, KvTile>::get(v_lds, 32 * kb + l32, s2), df[s2]);
      }
      auto grad = [&](auto maskc) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(st[r], scale_log2, nlse2));
          if constexpr (decltype(maskc)::value) {
            if (!visible(my_q, j0 + 32 * kb + acc_row(r), S, causal, window)) p = 0.f;
          }
          st[r] = p * (dpt[r] - dl);
        }
      };
      if (full) grad(IC<0>{});
      else grad(IC<1>{});
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const Frag<E> sf = acc_frag<E>(st, t);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          mma(acc[db], TrFrag<E, KvTile>::get(k_lds, 32 * kb + 16 * t, 32 * db), sf);
      }
    }
  };
  auto step = [&](auto stc, int s) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
    char* cur = ST == 0 ? st0 : (ST == 1 ? st1 : st2);
    char* nn = ST == 0 ? st2 : (ST == 1 ? st0 : st1);
    if (s + 1 < n_steps) wait_vmcnt<kOps>();
    else wait_vmcnt<0>();
    barrier_keep_vm();
    if (s + 2 < n_steps) issue(s + 2, nn);
    compute(s, cur);
  };
  for (int s = 0; s < n_steps; s += 3) {
    step(IC<0>{}, s);
    if (s + 1 < n_steps) step(IC<1>{}, s + 1);
    if (s + 2 < n_steps) step(IC<2>{}, s + 2);
  }

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

template <class E, int D>
static int launch_bwd_t(const Args& a) {
  hipStream_t st = (hipStream_t)a.stream;
  typedef typename E::T T;
  const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
  {
    const int rows = a.B * a.Hq * a.S;
    constexpr int RPB = 256 / (D / 8);
    dim3 grid((unsigned)((rows + RPB - 1) / RPB)), block(256);
    notify_launch("attn_bwd_delta", 0, a.stream);
    hipLaunchKernelGGL((delta_kernel<E, D>), grid, block, 0, st, (const T*)a.o_in, (const T*)a.dout,
                       (const float*)a.lse, a.delta, a.lse2, rows);
    notify_launch("attn_bwd_delta", 1, a.stream);
  }
  {
    constexpr int NW = kDkdvWaves;
    constexpr int QB = E::kBytes == 2 ? 2 : 1;
    const DkdvPlan p = dkdv_plan(a.B, a.Hq, a.Hkv, a.S);
    dim3 grid((unsigned)(p.n_pairs * a.B * a.Hkv * p.hs)), block(NW * 64);
    notify_launch("attn_bwd_dkdv", 0, a.stream);
    hipLaunchKernelGGL((dkdv_kernel<E, D, NW, QB>), grid, block, 0, st, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, (const T*)a.dout, (const float*)a.lse2, (const float*)a.delta,
                       (T*)a.dk, (T*)a.dv, a.part, a.B, a.Hq, a.Hkv, a.S, a.causal, a.window, a.scale,
                       scale_log2, p.n_kt, p.n_pairs, p.hs);
    notify_launch("attn_bwd_dkdv", 1, a.stream);
    if (p.hs > 1) {
      const size_t n = (size_t)a.B * a.Hkv * a.S * D;
      dim3 rgrid((unsigned)((n / 4 + 255) / 256)), rblock(256);
      notify_launch("attn_bwd_dkdv_reduce", 0, a.stream);
      hipLaunchKernelGGL((dkdv_reduce_kernel<E>), rgrid, rblock, 0, st, (const float*)a.part,
                         (T*)a.dk, (T*)a.dv, n, p.hs, a.scale);
      notify_launch("attn_bwd_dkdv_reduce", 1, a.stream);
    }
  }
  {
    constexpr int NW = E::kBytes == 2 ? 8 : 4;
    constexpr int KB = E::kBytes == 2 ? 2 : 1;
    const int n_qt = (a.S + 32 * NW - 1) / (32 * NW);
    dim3 grid((unsigned)(n_qt * a.B * a.Hq)), block(NW * 64);
    notify_launch("attn_bwd_dq", 0, a.stream);
    hipLaunchKernelGGL((dq_kernel<E, D, NW, KB>), grid, block, 0, st, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, (const T*)a.dout, (const float*)a.lse2, (const float*)a.delta,
                       (T*)a.dq, a.B, a.Hq, a.Hkv, a.S, a.causal, a.window, a.scale, scale_log2, n_qt);
    notify_launch("attn_bwd_dq", 1, a.stream);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_bwd(const Args& a) {
  if (a.dtype == kBF16) return a.D == 64 ? launch_bwd_t<BF16, 64>(a) : launch_bwd_t<BF16, 128>(a);
  return a.D == 64 ? launch_bwd_t<F32, 64>(a) : launch_bwd_t<F32, 128>(a);
}

}  // namespace fa
