// attn_bwd.hip -- tiled causal / sliding-window GQA attention backward for gfx950.
//
// Method: "KYNETRA FOUNDRY" page, FlashAttention paragraph (the backward recomputes score tiles on
// the fly rather than storing them); "CUDA-LLM: A GitHub Repository for Development", section "The
// custom CUDA kernel" (probabilities are recomputed from the saved log-sum-exp); Grip paragraph of
// the first page (dK and dV of a shared K/V head sum over its query-head group).
//
// Three launches on the caller's stream, no atomics anywhere:
//   1. delta_kernel: delta_i = sum_d dO_id * O_id in fp32 (O as the forward stored it).
//   2. dkdv_kernel: one workgroup per (batch, KV head, 32*NW keys). Each wave owns 32 keys whose
//      K and V rows stay in registers as B operands of S = Q K^T and dP = dO V^T, so a lane owns
//      one key and its accumulator holds query rows -- exactly the contraction side that
//      dV += P^T dO and dK += dS^T Q need. Query / dO tiles of every head of the group stream
//      through LDS; dK and dV for the whole group accumulate in registers and are written once.
//   3. dq_kernel: one workgroup per (batch, query head, 32*NW rows), lanes own queries (as in the
//      forward): S^T = K Q^T and dP^T = V dO^T from LDS key/value tiles, dS^T in registers is the
//      B operand of dQ^T += K^T dS^T with K^T read through the transposing LDS read.
// P and dS are rounded to the element type only as MFMA operands; all sums are fp32.
#include "device.h"
#include "launch.h"

namespace fa {

template <class E, int D>
__global__ __launch_bounds__(256) void delta_kernel(const typename E::T* __restrict__ O,
                                                    const typename E::T* __restrict__ dO,
                                                    float* __restrict__ delta, int rows) {
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
  if (part == 0 && row < rows) delta[row] = s;
}

template <class E, int D, int NW, int QB>
__global__ __launch_bounds__(NW * 64) void dkdv_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ delta, typename E::T* __restrict__ dK,
    typename E::T* __restrict__ dV, int B, int Hq, int Hkv, int S, int causal, int window,
    float scale, float scale_log2, int n_kt) {
  constexpr int BC = 32 * NW;  // keys per workgroup
  constexpr int BR = 32 * QB;  // query rows per streamed tile
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  typedef LdsTile<E, BR, D> QTile;
  __shared__ __attribute__((aligned(16))) char smem[2 * QTile::kBytes + 2 * BR * 4];
  char* q_lds = smem;
  char* do_lds = smem + QTile::kBytes;
  float* lse_lds = reinterpret_cast<float*>(smem + 2 * QTile::kBytes);
  float* dl_lds = lse_lds + BR;

  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // Under the causal mask the first key tiles see the most query rows: launch those first.
  const int BG = B * Hkv;
  const int rank = blockIdx.x / BG;
  const int bg = blockIdx.x - rank * BG;
  const int kt = rank;
  const int b = bg / Hkv;
  const int g = bg - b * Hkv;
  const int G = Hq / Hkv;

  const int k0 = kt * BC;
  const int kw = k0 + 32 * w;
  const int my_k = kw + l32;
  const bool k_ok = my_k < S;
  const size_t kv_off = (size_t)(b * Hkv + g) * S * D;

  Frag<E> kf[DS], vf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    kf[s] = load_frag_global(K + kv_off + (size_t)my_k * D + 16 * s + 8 * half, k_ok);
    vf[s] = load_frag_global(V + kv_off + (size_t)my_k * D + 16 * s + 8 * half, k_ok);
  }
  f32x16_t dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16_t{};
    dv[db] = f32x16_t{};
  }

  int it_lo, it_hi;
  q_tile_range(k0, imin_(k0 + BC - 1, S - 1), S, BR, causal, window, &it_lo, &it_hi);

  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    const size_t bh = (size_t)(b * Hq + h);
    const typename E::T* q_bh = Q + bh * S * D;
    const typename E::T* do_bh = dO + bh * S * D;
    for (int it = it_lo; it <= it_hi; ++it) {
      const int i0 = it * BR;
      __syncthreads();
      load_tile<E, QTile, BR, D, NW * 64>(q_lds, q_bh, i0, S);
      load_tile<E, QTile, BR, D, NW * 64>(do_lds, do_bh, i0, S);
      for (int t = threadIdx.x; t < BR; t += NW * 64) {
        const bool ok = i0 + t < S;
        lse_lds[t] = ok ? LSE[bh * S + i0 + t] * kLog2e : 0.f;
        dl_lds[t] = ok ? delta[bh * S + i0 + t] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int r0 = i0 + 32 * qb;
        if (block_empty(r0, r0 + 31, kw, kw + 31, S, causal, window)) continue;
        const bool full = block_full(r0, r0 + 31, kw, kw + 31, S, causal, window);
        f32x16_t sa = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          mma(sa, RowFrag<E, QTile>::get(q_lds, 32 * qb + l32, s), kf[s]);
          mma(dp, RowFrag<E, QTile>::get(do_lds, 32 * qb + l32, s), vf[s]);
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int rb = 32 * qb + 8 * r4 + 4 * half;  // registers 4*r4 .. 4*r4+3: rows rb .. rb+3
          const f32x4_t lse4 = *reinterpret_cast<const f32x4_t*>(lse_lds + rb);
          const f32x4_t dl4 = *reinterpret_cast<const f32x4_t*>(dl_lds + rb);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int r = 4 * r4 + c;
            float p = __builtin_amdgcn_exp2f(sa[r] * scale_log2 - lse4[c]);
            if (!full && !visible(i0 + rb + c, my_k, S, causal, window)) p = 0.f;
            sa[r] = p;
            dp[r] = p * (dp[r] - dl4[c]);
          }
        }
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
    }
  }

  // dk[db], dv[db]: register r holds key kw + acc_row(r), column 32*db + l32.
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw + acc_row(r);
      if (key >= S) continue;
      const size_t off = kv_off + (size_t)key * D + 32 * db + l32;
      if constexpr (E::kBytes == 2) {
        dK[off] = (uint16_t)bf16_bits(dk[db][r] * scale);
        dV[off] = (uint16_t)bf16_bits(dv[db][r]);
      } else {
        dK[off] = dk[db][r] * scale;
        dV[off] = dv[db][r];
      }
    }
  }
}

template <class E, int D, int NW, int KB>
__global__ __launch_bounds__(NW * 64) void dq_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ delta, typename E::T* __restrict__ dQ,
    int B, int Hq, int Hkv, int S, int causal, int window, float scale, float scale_log2, int n_qt) {
  constexpr int BR = 32 * NW;
  constexpr int BC = 32 * KB;
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  typedef LdsTile<E, BC, D> KvTile;
  __shared__ __attribute__((aligned(16))) char smem[2 * KvTile::kBytes];
  char* k_lds = smem;
  char* v_lds = smem + KvTile::kBytes;

  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  const int BH = B * Hq;
  const int rank = blockIdx.x / BH;
  const int bh = blockIdx.x - rank * BH;
  const int qt = causal ? n_qt - 1 - rank : rank;
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int g = h / (Hq / Hkv);
  const size_t q_off = (size_t)(b * Hq + h) * S * D;
  const typename E::T* k_bg = K + (size_t)(b * Hkv + g) * S * D;
  const typename E::T* v_bg = V + (size_t)(b * Hkv + g) * S * D;

  const int q0 = qt * BR;
  const int qw = q0 + 32 * w;
  const int my_q = qw + l32;
  const bool q_ok = my_q < S;

  Frag<E> qf[DS], df[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    qf[s] = load_frag_global(Q + q_off + (size_t)my_q * D + 16 * s + 8 * half, q_ok);
    df[s] = load_frag_global(dO + q_off + (size_t)my_q * D + 16 * s + 8 * half, q_ok);
  }
  const size_t row_idx = (size_t)(b * Hq + h) * S + (q_ok ? my_q : 0);
  const float lse2 = LSE[row_idx] * kLog2e;
  const float dl = delta[row_idx];

  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};

  int jt_lo, jt_hi;
  kv_tile_range(q0, imin_(q0 + BR - 1, S - 1), S, BC, causal, window, &jt_lo, &jt_hi);
  for (int jt = jt_lo; jt <= jt_hi; ++jt) {
    const int j0 = jt * BC;
    __syncthreads();
    load_tile<E, KvTile, BC, D, NW * 64>(k_lds, k_bg, j0, S);
    load_tile<E, KvTile, BC, D, NW * 64>(v_lds, v_bg, j0, S);
    __syncthreads();
    if (block_empty(qw, qw + 31, j0, j0 + BC - 1, S, causal, window)) continue;
    const bool full = block_full(qw, qw + 31, j0, j0 + BC - 1, S, causal, window);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16_t st = f32x16_t{}, dpt = f32x16_t{};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        mma(st, RowFrag<E, KvTile>::get(k_lds, 32 * kb + l32, s), qf[s]);
        mma(dpt, RowFrag<E, KvTile>::get(v_lds, 32 * kb + l32, s), df[s]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(st[r] * scale_log2 - lse2);
        if (!full && !visible(my_q, j0 + 32 * kb + acc_row(r), S, causal, window)) p = 0.f;
        st[r] = p * (dpt[r] - dl);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const Frag<E> sf = acc_frag<E>(st, t);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          mma(acc[db], TrFrag<E, KvTile>::get(k_lds, 32 * kb + 16 * t, 32 * db), sf);
      }
    }
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
                       a.delta, rows);
    notify_launch("attn_bwd_delta", 1, a.stream);
  }
  {
    constexpr int NW = 4, QB = 1;
    const int n_kt = (a.S + 32 * NW - 1) / (32 * NW);
    dim3 grid((unsigned)(n_kt * a.B * a.Hkv)), block(NW * 64);
    notify_launch("attn_bwd_dkdv", 0, a.stream);
    hipLaunchKernelGGL((dkdv_kernel<E, D, NW, QB>), grid, block, 0, st, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, (const T*)a.dout, (const float*)a.lse, (const float*)a.delta,
                       (T*)a.dk, (T*)a.dv, a.B, a.Hq, a.Hkv, a.S, a.causal, a.window, a.scale,
                       scale_log2, n_kt);
    notify_launch("attn_bwd_dkdv", 1, a.stream);
  }
  {
    constexpr int NW = 4, KB = 2;
    const int n_qt = (a.S + 32 * NW - 1) / (32 * NW);
    dim3 grid((unsigned)(n_qt * a.B * a.Hq)), block(NW * 64);
    notify_launch("attn_bwd_dq", 0, a.stream);
    hipLaunchKernelGGL((dq_kernel<E, D, NW, KB>), grid, block, 0, st, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, (const T*)a.dout, (const float*)a.lse, (const float*)a.delta,
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
