// attn_decode.hip -- key-split forward for decode-shaped problems (few queries, many keys).
//
// What it computes is the forward of attn_fwd_qk / attn_fwd_paged (queries at the last Sq
// positions, "CUDA-LLM: A GitHub Repository for Development", section "The custom CUDA kernel";
// sink keys, "KYNETRA FOUNDRY" Vaultecho paragraph; paged K/V, same page, paged-KV paragraph).
// With one query per sequence the tiled forward gives each workgroup a single query row and walks
// every key serially; here the keys are split instead:
//   * work item = (batch, KV head, chunk of 128 keys); the G query heads x Sq queries that share
//     the KV head are packed into one 32-column block (G * Sq <= 32), so one product covers them;
//   * each of the 4 waves copies its own 32-key K and V tiles to LDS (LDS-DMA, waits on its own
//     copies only), forms S^T = K Q^T, exponentiates against its tile's row maximum and accumulates
//     O^T = V^T P^T; the 4 waves' (max, sum, O) merge through LDS into one partial per chunk;
//   * decode_combine_kernel merges the chunks' partials (max, rescaled sums) into O and the
//     natural-log LSE, in a fixed order (deterministic).
#include "device.h"
#include "launch.h"

namespace fa {

constexpr int kDecNW = 4;                // waves per workgroup
constexpr int kDecChunk = 32 * kDecNW;   // keys per work item

// Wave-private copy of a 32 x D tile (rows row0 .. row0 + 31, clamped to S - 1) into LDS: the wave
// issues every 1 KB block of the tile itself. rowptr(t) is the byte address of row t.
template <int D, class RowPtr>
__device__ __forceinline__ void dma_tile_wave(char* lds, RowPtr rowptr, int row0, int S) {
  typedef LdsTile<BF16, 32, D> Tile;
  constexpr int kBlocks = Tile::kBytes / 1024;
  const int lane = lane_id();
  const uint32_t base = lds_addr(lds);
#pragma unroll
  for (int blk = 0; blk < kBlocks; ++blk) {
    const int c = blk * 64 + lane;
    const int r = c / Tile::kChunks;
    const int pos = c % Tile::kChunks;
    const int gr = imin_(row0 + r, S - 1);
    dma16(rowptr(gr) + ((pos ^ Tile::swz(r)) << 4), base + blk * 1024);
  }
}

// Chunk c (keys [c * kDecChunk, c * kDecChunk + kDecChunk)) holds no key that a query of the
// sequence (positions off .. off + Sq - 1 of S keys) sees.
__device__ __forceinline__ bool decode_chunk_empty(int c, int off, int Sq, int S, int causal, int window,
                                                   int sink) {
  const int c0 = c * kDecChunk;
  return c0 >= S || block_empty(off, off + Sq - 1, c0, c0 + kDecChunk - 1, S, causal, window, sink);
}

// part layout per (chunk, b, g): R rows x D floats of unnormalised O, then R maxima (base 2), then
// R sums.
__device__ __forceinline__ size_t dec_part_index(int chunk, int bg, int BG, int R, int D) {
  return ((size_t)chunk * BG + bg) * (size_t)R * (D + 2);
}

template <int D, bool PG>
__global__ __launch_bounds__(kDecNW * 64) void decode_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    float* __restrict__ part, int B, int Hq, int Hkv, int Sq, int S, int causal, int window, int sink,
    float scale_log2, int n_chunk, PagedKV pg) {
  typedef BF16 E;
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  typedef LdsTile<E, 32, D> Tile;
  constexpr int kTile = Tile::kBytes;
  constexpr int kRow = D + 1;                            // padded row of the merge area (no bank conflicts)
  constexpr int kWave = 32 * kRow + 64;                   // per wave: O (32 rows) + 32 maxima + 32 sums
  constexpr int kMerge = kDecNW * kWave * 4;
  constexpr int kLds = 2 * kDecNW * kTile > kMerge ? 2 * kDecNW * kTile : kMerge;
  __shared__ __attribute__((aligned(1024))) char lds[kLds];

  const int lane = lane_id();
  const int w = wave_id();
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int G = Hq / Hkv;
  const int R = G * Sq;  // packed rows: n = hh * Sq + i
  const int BG = B * Hkv;
  const int chunk = blockIdx.x % n_chunk;
  const int bg = blockIdx.x / n_chunk;
  const int b = bg / Hkv;
  const int g = bg - b * Hkv;

  if constexpr (PG) S = imin_(imax_(pg.seqlen[b], Sq), pg.max_blocks << pg.shift);
  const int off = S - Sq;
  // A chunk past this sequence's keys or outside every query's window holds nothing: the whole
  // workgroup leaves at once and the combine skips the chunk by the same test.
  if (decode_chunk_empty(chunk, off, Sq, S, causal, window, sink)) return;

  // This lane's packed row: query head g*G + hh, query i at position off + i.
  const int n = l32;
  const bool row_ok = n < R;
  const int hh = row_ok ? n / Sq : 0;
  const int qi = row_ok ? n - hh * Sq : 0;
  const int my_p = row_ok ? off + qi : S;  // rows past R see nothing
  Frag<E> qf[DS];
  {
    const uint16_t* qrow = Q + ((size_t)(b * Hq + g * G + hh) * Sq + qi) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = load_frag_global(qrow + 16 * s, row_ok);
  }

  char* k_lds = lds + w * 2 * kTile;
  char* v_lds = k_lds + kTile;
  const int j0 = chunk * kDecChunk + 32 * w;
  const bool work = j0 < S && !block_empty(off, off + Sq - 1, j0, j0 + 31, S, causal, window, sink);
  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};
  float m = kNegInf, l = 0.f;
  if (work) {
    if constexpr (PG) {
      const int* tab = pg.table + (size_t)b * pg.max_blocks;
      const int lb_last = (S - 1) >> pg.shift;
      const int lb0 = j0 >> pg.shift;
      const int ph0 = imin_(imax_(tab[lb0], 0), pg.num_blocks - 1);
      const int ph1 = imin_(imax_(tab[imin_(lb0 + 1, lb_last)], 0), pg.num_blocks - 1);
      const int shift = pg.shift;
      auto rowptr = [&](const uint16_t* pool, int t) __attribute__((always_inline)) {
        const int phys = (t >> shift) == lb0 ? ph0 : ph1;
        const size_t row = (((size_t)phys * Hkv + g) << shift) | (size_t)(t & ((1 << shift) - 1));
        return reinterpret_cast<const char*>(pool + row * D);
      };
      dma_tile_wave<D>(k_lds, [&](int t) { return rowptr(K, t); }, j0, S);
      dma_tile_wave<D>(v_lds, [&](int t) { return rowptr(V, t); }, j0, S);
    } else {
      const uint16_t* kb = K + (size_t)bg * S * D;
      const uint16_t* vb = V + (size_t)bg * S * D;
      dma_tile_wave<D>(k_lds, [&](int t) { return reinterpret_cast<const char*>(kb + (size_t)t * D); }, j0, S);
      dma_tile_wave<D>(v_lds, [&](int t) { return reinterpret_cast<const char*>(vb + (size_t)t * D); }, j0, S);
    }
    wait_vmcnt<0>();  // this wave's own copies (and its Q fragments) have landed

    f32x16_t st = f32x16_t{};
#pragma unroll
    for (int s2 = 0; s2 < DS; ++s2) mma(st, RowFrag<E, Tile>::get(k_lds, l32, s2), qf[s2]);
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (!visible(my_p, j0 + acc_row(r), S, causal, window, sink)) st[r] = kNegInf;
      mx = fmaxf(mx, st[r]);
    }
    m = pair_max(mx) * scale_log2;  // -inf for a row that sees none of these keys
    const float neg_m = m == kNegInf ? 0.f : -m;
    Frag<E> pf[2];
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = __builtin_amdgcn_exp2f(fmaf(st[r], scale_log2, neg_m));
    add_block4(st, ps);
#pragma unroll
    for (int t = 0; t < 2; ++t) pf[t] = acc_frag<E>(st, t);
    l = pair_sum(sum4(ps));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int db = 0; db < DB; ++db) mma(acc[db], TrFrag<E, Tile>::get(v_lds, 16 * t, 32 * db), pf[t]);
    }
  }

  // Merge the 4 waves through LDS: wave w's O^T, maxima and sums, then one partial per chunk.
  __syncthreads();  // every wave is done reading its K / V tiles
  float* mo = reinterpret_cast<float*>(lds) + (size_t)w * kWave;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) mo[n * kRow + 32 * db + acc_row(r)] = acc[db][r];
  }
  if (half == 0) {
    mo[32 * kRow + n] = m;
    mo[32 * kRow + 32 + n] = l;
  }
  __syncthreads();
  float* out = part + dec_part_index(chunk, bg, BG, R, D);
  const float* mw = reinterpret_cast<const float*>(lds);
  for (int e = threadIdx.x; e < R * D; e += kDecNW * 64) {
    const int row = e / D;
    const int d = e - row * D;
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < kDecNW; ++v) M = fmaxf(M, mw[v * kWave + 32 * kRow + row]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < kDecNW; ++v) {
      const float* src = mw + v * kWave;
      const float mv = src[32 * kRow + row];
      const float f = mv == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mv - M);
      o += f * src[row * kRow + d];
      L += f * src[32 * kRow + 32 + row];
    }
    out[row * D + d] = o;
    if (d == 0) {
      out[R * D + row] = M;
      out[R * D + R + row] = L;
    }
  }
}

// One workgroup of D threads per (b, g, packed row): merge the non-empty chunks in chunk order, one
// pass over groups of kCombGroup chunks with a running maximum (all of a group's loads are issued
// before any is used). The chunk holding the row's own position is never empty, so L > 0. The
// loads stay unconditional: an empty chunk reads that chunk's partial instead and weighs 0.
constexpr int kCombGroup = 16;
template <int D, bool PG>
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ part,
                                                             uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                             int B, int Hq, int Hkv, int Sq, int S, int causal,
                                                             int window, int sink, int n_chunk, PagedKV pg) {
  const int G = Hq / Hkv;
  const int R = G * Sq;
  const int BG = B * Hkv;
  const int row = blockIdx.x % R;
  const int bg = blockIdx.x / R;
  const int b = bg / Hkv;
  const int g = bg - b * Hkv;
  const int d = threadIdx.x;
  if constexpr (PG) S = imin_(imax_(pg.seqlen[b], Sq), pg.max_blocks << pg.shift);
  const int off = S - Sq;
  const int nc = imin_(n_chunk, (S + kDecChunk - 1) / kDecChunk);  // later chunks lie past the keys
  const int c_self = (off + row % Sq) / kDecChunk;
  float M = kNegInf, o = 0.f, L = 0.f;
  for (int c0 = 0; c0 < nc; c0 += kCombGroup) {
    float mc[kCombGroup], oc[kCombGroup], lc[kCombGroup];
#pragma unroll
    for (int u = 0; u < kCombGroup; ++u) {
      const int c = c0 + u;
      const bool use = c < nc && !decode_chunk_empty(c, off, Sq, S, causal, window, sink);
      const float* p = part + dec_part_index(use ? c : c_self, bg, BG, R, D);
      mc[u] = p[R * D + row];
      oc[u] = p[row * D + d];
      lc[u] = p[R * D + R + row];
      if (!use) mc[u] = kNegInf;
    }
    float gm = M;
#pragma unroll
    for (int u = 0; u < kCombGroup; ++u) gm = fmaxf(gm, mc[u]);
    if (gm != kNegInf) {
      const float r = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - gm);
      o *= r;
      L *= r;
#pragma unroll
      for (int u = 0; u < kCombGroup; ++u) {
        const float f = mc[u] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mc[u] - gm);
        o += f * oc[u];
        L += f * lc[u];
      }
      M = gm;
    }
  }
  const int hh = row / Sq;
  const int qi = row - hh * Sq;
  const size_t orow = (size_t)(b * Hq + g * G + hh) * Sq + qi;
  O[orow * D + d] = (uint16_t)bf16_bits(o / L);
  if (d == 0) LSE[orow] = (M + __log2f(L)) * kLn2;
}

int decode_chunks(int max_keys) { return (max_keys + kDecChunk - 1) / kDecChunk; }

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int max_keys, int D) {
  const size_t R = (size_t)(Hq / Hkv) * Sq;
  return (size_t)decode_chunks(max_keys) * B * Hkv * R * (D + 2) * sizeof(float);
}

template <int D>
static int launch_decode_t(const Args& a, float* part, int max_keys) {
  hipStream_t st = (hipStream_t)a.stream;
  const int n_chunk = decode_chunks(max_keys);
  const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
  const int BG = a.B * a.Hkv;
  const int R = (a.Hq / a.Hkv) * a.Sq;
  notify_launch("attn_decode", 0, a.stream);
  auto kern = a.paged ? decode_kernel<D, true> : decode_kernel<D, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(n_chunk * BG)), dim3(kDecNW * 64), 0, st,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, part, a.B, a.Hq,
                     a.Hkv, a.Sq, a.Sk, a.causal, a.window, a.sink, scale_log2, n_chunk, a.pg);
  notify_launch("attn_decode", 1, a.stream);
  notify_launch("attn_decode_combine", 0, a.stream);
  auto comb = a.paged ? decode_combine_kernel<D, true> : decode_combine_kernel<D, false>;
  hipLaunchKernelGGL(comb, dim3((unsigned)(BG * R)), dim3(D), 0, st, (const float*)part, (uint16_t*)a.o,
                     a.lse, a.B, a.Hq, a.Hkv, a.Sq, a.Sk, a.causal, a.window, a.sink, n_chunk, a.pg);
  notify_launch("attn_decode_combine", 1, a.stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_decode(const Args& a, float* part, int max_keys) {
  return a.D == 64 ? launch_decode_t<64>(a, part, max_keys) : launch_decode_t<128>(a, part, max_keys);
}

}  // namespace fa
