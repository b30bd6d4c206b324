// device.h -- gfx950 building blocks for the attention kernels: element types, the 32x32 MFMA
// tile, the swizzled LDS tile layout and operand-fragment loads.
//
// MFMA 32x32 tile (v_mfma_f32_32x32x16_bf16; for f32, eight v_mfma_f32_32x32x2f32), lane l of the
// 64-lane wave, h = l / 32:
//   A operand: row m = l % 32, contraction elements k = 8h + e (e = 0..7, one 16-byte fragment)
//   B operand: column n = l % 32, contraction elements k = 8h + e
//   C/D accumulator register r (0..15): row 8*(r/4) + 4h + r%4, column l % 32
// So a lane's accumulator holds 16 rows of one column. Feeding those 16 values back as the
// contraction side of the next product needs no data movement: registers 8t..8t+7 cover rows
// 16t + 8*(e/4) + 4h + e%4, and the other operand is fetched with the same row permutation
// (tr_frag). The f32 variant feeds element e of every lane's fragment to the e-th 32x32x2 step,
// which contracts the same index set.
#ifndef ATTN_DEVICE_H_
#define ATTN_DEVICE_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tiles.h"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

struct BF16 {
  typedef uint16_t T;
  static constexpr int kBytes = 2;
};
struct F32 {
  typedef float T;
  static constexpr int kBytes = 4;
};

// Eight consecutive contraction elements of one operand row/column.
template <class E> struct Frag;
template <> struct Frag<BF16> { u32x4_t v; };
template <> struct Frag<F32> { f32x4_t lo, hi; };

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ void mma(f32x16_t& acc, const Frag<BF16>& a, const Frag<BF16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                __builtin_bit_cast(bf16x8_t, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16_t& acc, const Frag<F32>& a, const Frag<F32>& b) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[e], b.lo[e], acc, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[e], b.hi[e], acc, 0, 0, 0);
}

// ---------------------------------------------------------------- conversions
// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two floats -> packed bfloat16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Accumulator registers 8t..8t+7 as a contraction fragment (rows 16t + 8*(e/4) + 4h + e%4).
__device__ __forceinline__ Frag<BF16> acc_frag_bf16(const f32x16_t& a, int t) {
  Frag<BF16> f;
  f.v[0] = pack_bf16x2(a[8 * t + 0], a[8 * t + 1]);
  f.v[1] = pack_bf16x2(a[8 * t + 2], a[8 * t + 3]);
  f.v[2] = pack_bf16x2(a[8 * t + 4], a[8 * t + 5]);
  f.v[3] = pack_bf16x2(a[8 * t + 6], a[8 * t + 7]);
  return f;
}
template <class E> __device__ __forceinline__ Frag<E> acc_frag(const f32x16_t& a, int t);
template <> __device__ __forceinline__ Frag<BF16> acc_frag<BF16>(const f32x16_t& a, int t) {
  return acc_frag_bf16(a, t);
}
template <> __device__ __forceinline__ Frag<F32> acc_frag<F32>(const f32x16_t& a, int t) {
  Frag<F32> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.lo[e] = a[8 * t + e];
    f.hi[e] = a[8 * t + 4 + e];
  }
  return f;
}

// Adds the 16 exponentials of one 32-key block (one accumulator) into four running partial sums in
// register order: sum[r % 4] += p[r]. Summing the fp32 values before they are rounded for the P V
// product keeps the row sum on plain VALU adds (v_dot2c_f32_bf16 on the packed words runs about
// 2.5x slower while another wave of the SIMD issues matrix products). Every forward and decode
// kernel sums in this order, so rows computed by different kernels agree bit for bit.
__device__ __forceinline__ void add_block4(const f32x16_t& p, float (&sum)[4]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) sum[r & 3] += p[r];
}
__device__ __forceinline__ float sum4(const float (&sum)[4]) { return (sum[0] + sum[1]) + (sum[2] + sum[3]); }

// v[r] = keep ? v[r] : -inf, written back into the element's own register (no copy of the
// surviving values).
__device__ __forceinline__ void mask_neg_inf(f32x16_t& v, int r, bool keep) {
  const float ninf = kNegInf;
  float x = v[r];
  asm("v_cndmask_b32 %0, %1, %0, %2" : "+v"(x) : "v"(ninf), "s"(__builtin_amdgcn_ballot_w64(keep)));
  v[r] = x;
}

// v[r] = keep ? v[r] : 0, in place.
__device__ __forceinline__ void mask_zero(f32x16_t& v, int r, bool keep) {
  float x = v[r];
  asm("v_cndmask_b32 %0, 0, %0, %1" : "+v"(x) : "s"(__builtin_amdgcn_ballot_w64(keep)));
  v[r] = x;
}

// ---------------------------------------------------------------- global fragments
// 8 consecutive elements from global memory (16 B for bf16, 32 B for f32), or zeros.
__device__ __forceinline__ Frag<BF16> load_frag_global(const uint16_t* p, bool ok) {
  Frag<BF16> f;
  f.v = ok ? *reinterpret_cast<const u32x4_t*>(p) : u32x4_t{0, 0, 0, 0};
  return f;
}
__device__ __forceinline__ Frag<F32> load_frag_global(const float* p, bool ok) {
  Frag<F32> f;
  if (ok) {
    f.lo = *reinterpret_cast<const f32x4_t*>(p);
    f.hi = *reinterpret_cast<const f32x4_t*>(p + 4);
  } else {
    f.lo = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f.hi = f.lo;
  }
  return f;
}

// ---------------------------------------------------------------- LDS tiles
// A tile of ROWS rows x D elements, row-major, unpadded, stored as 16-byte chunks whose position
// inside the row is XOR-swizzled by the row index. The swizzle makes both access patterns used
// here free of bank conflicts: 16 lanes reading the same chunk of 16 consecutive rows (row_frag),
// and the transposing 8-byte reads of 4 consecutive rows x 64 bytes (tr_frag).
template <class E, int ROWS, int D>
struct LdsTile {
  static constexpr int kRowBytes = D * E::kBytes;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kBytes = ROWS * kRowBytes;
  static_assert(kChunks >= 8, "row must hold at least 8 chunks");

  __device__ static __forceinline__ int swz(int row) {
    if constexpr (kChunks >= 16) return 4 * (row & 3) + ((row >> 2) & 3);
    else return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
  }
  __device__ static __forceinline__ int chunk_off(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz(row)) << 4);
  }
};

template <class Tile>
__device__ __forceinline__ void lds_store_chunk(char* base, int row, int chunk, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(base + Tile::chunk_off(row, chunk)) = v;
}
template <class Tile>
__device__ __forceinline__ u32x4_t lds_load_chunk(const char* base, int row, int chunk) {
  return *reinterpret_cast<const u32x4_t*>(base + Tile::chunk_off(row, chunk));
}

// Fragment of row `row`, contraction elements 16s + 8h .. +7 (h = lane / 32).
template <class E, class Tile> struct RowFrag;
template <class Tile> struct RowFrag<BF16, Tile> {
  __device__ static __forceinline__ Frag<BF16> get(const char* base, int row, int s) {
    Frag<BF16> f;
    f.v = lds_load_chunk<Tile>(base, row, 2 * s + (lane_id() >> 5));
    return f;
  }
};
template <class Tile> struct RowFrag<F32, Tile> {
  __device__ static __forceinline__ Frag<F32> get(const char* base, int row, int s) {
    Frag<F32> f;
    int c = 4 * s + 2 * (lane_id() >> 5);
    f.lo = __builtin_bit_cast(f32x4_t, lds_load_chunk<Tile>(base, row, c));
    f.hi = __builtin_bit_cast(f32x4_t, lds_load_chunk<Tile>(base, row, c + 1));
    return f;
  }
};

// Transposed fragment: column n0 + lane % 32 of the tile, contraction over tile rows
// kbase + 8*(e/4) + 4h + e%4 (e = 0..7), i.e. the permutation that matches acc_frag(..., t)
// with kbase = 32*block + 16t. For bf16 this is two ds_read_b64_tr_b16: within each group of 16
// lanes, lane s reads 4 elements at (row k0 + s/4, column c0 + 4*(s%4)) and receives column
// c0 + s of rows k0 .. k0+3.
template <class E, class Tile> struct TrFrag;
template <class Tile> struct TrFrag<BF16, Tile> {
  __device__ static __forceinline__ Frag<BF16> get(const char* base, int kbase, int n0) {
    const int l = lane_id();
    const int s = l & 15;
    const int col = n0 + 16 * ((l >> 4) & 1) + 4 * (s & 3);
    const int row = kbase + 4 * (l >> 5) + (s >> 2);
    const int chunk = col >> 3;
    const int sub = (s & 1) * 8;
    const char* pa = base + Tile::chunk_off(row, chunk) + sub;
    const char* pb = base + Tile::chunk_off(row + 8, chunk) + sub;
    s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)((__attribute__((address_space(3))) char*)(pa)));
    s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)((__attribute__((address_space(3))) char*)(pb)));
    Frag<BF16> f;
    u32x2_t ua = __builtin_bit_cast(u32x2_t, a);
    u32x2_t ub = __builtin_bit_cast(u32x2_t, b);
    f.v = u32x4_t{ua[0], ua[1], ub[0], ub[1]};
    return f;
  }
};
template <class Tile> struct TrFrag<F32, Tile> {
  __device__ static __forceinline__ Frag<F32> get(const char* base, int kbase, int n0) {
    const int l = lane_id();
    const int col = n0 + (l & 31);
    const int rb = kbase + 4 * (l >> 5);
    Frag<F32> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f.lo[e] = *reinterpret_cast<const float*>(base + Tile::chunk_off(rb + e, col >> 2) + (col & 3) * 4);
      f.hi[e] = *reinterpret_cast<const float*>(base + Tile::chunk_off(rb + 8 + e, col >> 2) + (col & 3) * 4);
    }
    return f;
  }
};

// Cooperative copy of rows [row0, row0 + ROWS) of a [S, D] matrix into an LDS tile; rows at or
// beyond S are written as zeros (so masked keys contribute exact zeros, never NaN).
template <class E, class Tile, int ROWS, int D, int NTHREADS>
__device__ __forceinline__ void load_tile(char* lds, const typename E::T* __restrict__ src, int row0, int S) {
  constexpr int kChunksPerRow = Tile::kChunks;
  constexpr int kTotal = ROWS * kChunksPerRow;
  static_assert(kTotal % NTHREADS == 0, "tile chunks must divide evenly over the threads");
  constexpr int kPer = kTotal / NTHREADS;
  u32x4_t v[kPer];
#pragma unroll
  for (int n = 0; n < kPer; ++n) {
    const int c = threadIdx.x + n * NTHREADS;
    const int r = c / kChunksPerRow;
    const int ch = c % kChunksPerRow;
    const bool ok = row0 + r < S;
    const char* p = reinterpret_cast<const char*>(src + (size_t)(row0 + r) * D) + ch * 16;
    v[n] = ok ? *reinterpret_cast<const u32x4_t*>(p) : u32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int n = 0; n < kPer; ++n) {
    const int c = threadIdx.x + n * NTHREADS;
    lds_store_chunk<Tile>(lds, c / kChunksPerRow, c % kChunksPerRow, v[n]);
  }
}

// Max / sum of a value held by lanes l and l ^ 32 (the two halves of one accumulator column).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int N> struct IC { static constexpr int value = N; };  // compile-time stage index

// ---------------------------------------------------------------- asynchronous tile copies
// Wave index as a scalar (it is uniform across the wave; LDS-DMA needs the LDS address in M0).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Wait until at most N vector-memory operations of this wave are outstanding (gfx9 s_waitcnt
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that waits for this wave's own LDS instructions (lgkmcnt 0) but not for its
// outstanding vector-memory traffic, so LDS-DMA copies of later stages stay in flight. The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_keep_vm() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

// LDS-DMA: each lane copies 16 (resp. 4) bytes from its global address to LDS at
// lds_base + 16 * lane (resp. 4 * lane); lds_base must be wave-uniform (it goes to M0). Issued
// through inline asm so that the compiler does not add its own conservative wait for these copies
// before LDS reads: the kernels order them explicitly with wait_vmcnt<> + barrier_keep_vm().
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"((uint64_t)(uintptr_t)gptr), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"((uint64_t)(uintptr_t)gptr), "s"(lds_base) : "memory", "m0");
}

// Issue this wave's share of an asynchronous copy of rows [row0, row0 + ROWS) of a row-major
// [S, D] matrix into a swizzled LDS tile. One 16-byte LDS-DMA per lane moves 1 KB per wave:
// lane l writes the 16 bytes at (block base + 16 l), so lane l fetches the global chunk the
// swizzle puts there. Rows at or past S are read from row S - 1: finite data whose scores /
// products the masks zero. NW waves share the work; the caller waits with wait_vmcnt<>.
template <class E, int ROWS, int D, int NW>
__device__ __forceinline__ void dma_tile(char* lds, const typename E::T* __restrict__ src, int row0, int S) {
  typedef LdsTile<E, ROWS, D> Tile;
  constexpr int kBlocks = Tile::kBytes / 1024;
  static_assert(kBlocks % NW == 0, "tile must split into whole 1 KB blocks per wave");
  const int lane = lane_id();
  const int w = wave_id();
  const uint32_t base = lds_addr(lds);
  const char* tile = reinterpret_cast<const char*>(src + (size_t)row0 * D);
  if (row0 + ROWS <= S) {
    // Whole tile in range: per-lane byte offsets inside the tile do not depend on row0.
#pragma unroll
    for (int n = 0; n < kBlocks / NW; ++n) {
      const int blk = n * NW + w;
      const int c = blk * 64 + lane;
      const int r = c / Tile::kChunks;
      const int pos = c % Tile::kChunks;
      dma16(tile + r * Tile::kRowBytes + ((pos ^ Tile::swz(r)) << 4), base + blk * 1024);
    }
  } else {
#pragma unroll
    for (int n = 0; n < kBlocks / NW; ++n) {
      const int blk = n * NW + w;
      const int c = blk * 64 + lane;
      const int r = c / Tile::kChunks;
      const int pos = c % Tile::kChunks;
      const int gr = imin_(row0 + r, S - 1);
      const char* g = reinterpret_cast<const char*>(src + (size_t)gr * D) + ((pos ^ Tile::swz(r)) << 4);
      dma16(g, base + blk * 1024);
    }
  }
}
template <class E, int ROWS, int D, int NW>
constexpr int dma_tile_ops() { return LdsTile<E, ROWS, D>::kBytes / 1024 / NW; }

// The same copy for whole tiles with the global address split into a wave-uniform base (SGPRs)
// and a per-lane 32-bit offset that depends only on the lane and the 1 KB block: a tile row
// group of 64 * 16 / kRowBytes rows per block, and block n * NW + w of this wave lies
// n * NW * 1024 bytes further on in both the tile and LDS (the swizzle repeats every 16 rows).
// `lane_off` = dma_lane_off<Tile, NW>() computed once; no per-copy vector arithmetic. Rows at or
// past S need the clamped copy (dma_tile).
template <class Tile, int NW>
__device__ __forceinline__ uint32_t dma_lane_off() {
  const int c = wave_id() * 64 + lane_id();
  const int r = c / Tile::kChunks;
  const int pos = c % Tile::kChunks;
  return (uint32_t)(r * Tile::kRowBytes + ((pos ^ Tile::swz(r)) << 4));
}
// `sbase` must be the same for every lane of the wave; it is moved to scalar registers here.
// NT: a non-temporal (streaming) load, for data read exactly once.
template <bool NT = false>
__device__ __forceinline__ void dma16_s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  // (readfirstlane returns int: both halves are taken back to uint32_t before widening, so the
  // low half is zero-extended, not sign-extended)
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const uint64_t sa = ((uint64_t)hi << 32) | (uint64_t)lo;
  if constexpr (NT) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(voff), "s"(sa), "s"(lds_base) : "memory", "m0");
  } else {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sa), "s"(lds_base) : "memory", "m0");
  }
}
template <class E, int ROWS, int D, int NW>
constexpr bool dma_fast_ok() {
  return (LdsTile<E, ROWS, D>::kBytes / 1024) % NW == 0 && (NW * 1024) % (16 * LdsTile<E, ROWS, D>::kRowBytes) == 0;
}
template <class E, int ROWS, int D, int NW>
__device__ __forceinline__ void dma_tile_fast(char* lds, const typename E::T* __restrict__ src, int row0,
                                              uint32_t lane_off) {
  typedef LdsTile<E, ROWS, D> Tile;
  constexpr int kBlocks = Tile::kBytes / 1024;
  static_assert(kBlocks % NW == 0 && (NW * 1024) % (16 * Tile::kRowBytes) == 0, "blocks repeat the swizzle");
  const char* tile = reinterpret_cast<const char*>(src + (size_t)row0 * D);
  const uint32_t base = lds_addr(lds) + wave_id() * 1024;
#pragma unroll
  for (int n = 0; n < kBlocks / NW; ++n) dma16_s(lane_off, tile + n * NW * 1024, base + n * NW * 1024);
}

// The same copy from a paged cache: row t of the sequence lives in physical block tab[t >> shift]
// of a [nblocks, Hkv, 2^shift, D] pool, head g, slot t & (2^shift - 1). Block sizes are powers of
// two >= 16 and row0 is a multiple of ROWS, so the tile spans at most max(1, ROWS >> shift) <= 4
// blocks; their table entries are wave-uniform (scalar loads). Table indices are clamped to the
// entries that cover rows [0, S) and physical blocks to [0, nblocks): malformed tables cannot
// make the copy leave the pool. Rows at or past S are read from row S - 1, as in dma_tile.
template <class E, int ROWS, int D, int NW>
__device__ __forceinline__ void dma_tile_paged(char* lds, const typename E::T* __restrict__ pool,
                                               const int* __restrict__ tab, int g, int Hkv, int shift,
                                               int nblocks, int row0, int S) {
  typedef LdsTile<E, ROWS, D> Tile;
  constexpr int kBlocks = Tile::kBytes / 1024;
  static_assert(kBlocks % NW == 0, "tile must split into whole 1 KB blocks per wave");
  static_assert(ROWS <= 64, "at most 4 pool blocks of 16 rows per tile");
  const int lane = lane_id();
  const int w = wave_id();
  const uint32_t base = lds_addr(lds);
  const int lb0 = row0 >> shift;
  const int lb_last = (S - 1) >> shift;
  int ph[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lb = imin_(lb0 + i, lb_last);
    ph[i] = imin_(imax_(tab[lb], 0), nblocks - 1);
  }
#pragma unroll
  for (int n = 0; n < kBlocks / NW; ++n) {
    const int blk = n * NW + w;
    const int c = blk * 64 + lane;
    const int r = c / Tile::kChunks;
    const int pos = c % Tile::kChunks;
    const int gr = imin_(row0 + r, S - 1);
    const int rel = (gr >> shift) - lb0;  // 0 .. 3
    const int phys = rel == 0 ? ph[0] : (rel == 1 ? ph[1] : (rel == 2 ? ph[2] : ph[3]));
    const size_t row = ((((size_t)phys * Hkv + g) << shift) | (size_t)(gr & ((1 << shift) - 1)));
    const char* gp = reinterpret_cast<const char*>(pool + row * D) + ((pos ^ Tile::swz(r)) << 4);
    dma16(gp, base + blk * 1024);
  }
}

// 64 consecutive floats src[clamp(i0 + lane)] -> lds[0..63] (one wave, one instruction).
__device__ __forceinline__ void dma_row_floats(char* lds, const float* __restrict__ src, int i0, int S) {
  const int r = imin_(i0 + lane_id(), S - 1);
  dma4(src + r, lds_addr(lds));
}

// Runs steps 0 .. n-1 over an NST-stage ring of SB-byte LDS stages whose first NST-1 tiles were
// already issued (and waited for) by the caller. Step s: wait until this wave's copies of tile s
// have landed (OPS copy instructions per wave per tile; tiles s+1 .. s+NST-2 may stay in flight),
// workgroup barrier, issue tile s+NST-1 into the stage every wave finished with at step s-1, then
// compute on tile s. One barrier per step; tile s+NST-1 is fetched while tiles s.. are used.
template <int NST, int SB, int OPS, class Issue, class Compute>
__device__ __forceinline__ void ring_run(char* ring, int n, Issue&& issue, Compute&& compute) {
  static_assert(NST == 2 || NST == 3, "ring depth");
  auto one = [&](auto kc, int s) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    if constexpr (NST == 3) {
      if (s + 1 < n) wait_vmcnt<OPS>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    barrier_keep_vm();
    if (s + NST - 1 < n) issue(s + NST - 1, ring + ((k + NST - 1) % NST) * SB);
    compute(s, ring + k * SB);
  };
  for (int s0 = 0; s0 < n; s0 += NST) {
    one(IC<0>{}, s0);
    if (s0 + 1 < n) one(IC<1>{}, s0 + 1);
    if constexpr (NST == 3) {
      if (s0 + 2 < n) one(IC<2>{}, s0 + 2);
    }
  }
}

// Returns x through an empty volatile asm statement, inside a rarely taken branch: values derived
// from it cannot be hoisted out of the loop (where they would hold registers for the whole
// kernel), and the branch cannot be if-converted into the common path.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Copies the document boundaries cu[0..n] of one batch row into LDS, clamped to [0, S] (the whole
// workgroup takes part; the caller then synchronises the workgroup).
__device__ __forceinline__ void stage_docs(int* dst, const int* __restrict__ src, int n, int S) {
  for (int t = threadIdx.x; t <= n; t += blockDim.x) dst[t] = imin_(imax_(src[t], 0), S);
}

// Packed documents: at most this many key tiles are ranked by work in the dK/dV pass.
constexpr int kBalancedTiles = 256;

// Accumulator row index (within a 32 x 32 tile) held in register r by this lane.
__device__ __forceinline__ int acc_row(int r) { return 8 * (r >> 2) + 4 * (lane_id() >> 5) + (r & 3); }

}  // namespace fa

#endif  // ATTN_DEVICE_H_
