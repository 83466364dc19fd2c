// fa_common.hpp -- gfx950 building blocks shared by the attention kernels:
// matrix-core (MFMA) wrappers, LDS transpose reads, buffer loads with hardware
// range checking, conversions, and the workgroup -> tile mapping.
//
// Register layouts of v_mfma_f32_32x32x16_{f16,bf16} (wave64), confirmed by an
// on-device layout check before any kernel was built on them:
//   A (32 x 16):  lane l holds A[l % 32][8 * (l / 32) + i],  i = 0..7
//   B (16 x 32):  lane l holds B[8 * (l / 32) + i][l % 32],  i = 0..7
//   C (32 x 32):  lane l, register r holds
//                 C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32],  r = 0..15
// Only the pairing of A and B along k matters for the product, so any k
// permutation applied to both operands gives the same C.
//
// ds_read_b64_tr_b16 (LDS transpose read), per group of 16 lanes: lane
// j = 4a + b supplies the address of X[r0 + a][c0 + 4b .. 4b + 3] (row-major
// 16-bit storage); lane i of the group then receives X[r0 + a][c0 + i] for
// a = 0..3.  This turns a row-major tile into an MFMA operand whose k index
// runs along the rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

// Debug build (libfa_mi355x_debug.so, compiled with FA_DEBUG_BUILD=1): each
// tiled kernel fills its LDS with NaN before first use, so a read of LDS that
// was never written shows up in the outputs, and the forward and backward
// kernels count the tiles they load (see debug_visit).  The production library
// compiles both to nothing.
#ifndef FA_DEBUG_BUILD
#define FA_DEBUG_BUILD 0
#endif

namespace fa {

constexpr bool kDebugBuild = FA_DEBUG_BUILD != 0;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

template <typename T> struct Vec8;
template <> struct Vec8<_Float16> { typedef f16x8 type; };
template <> struct Vec8<__bf16> { typedef bf16x8 type; };

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even conversion of two floats into one packed 32-bit word
// (low half = a); one v_cvt_pk_{f16,bf16}_f32 on gfx950.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<_Float16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}
template <> __device__ __forceinline__ uint32_t pack2<__bf16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Sum of the two 16-bit values packed in w, added to acc (v_dot2 with (1, 1)).
template <typename T> __device__ __forceinline__ float add_pair(uint32_t w, float acc);
template <> __device__ __forceinline__ float add_pair<_Float16>(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), (f16x2){1, 1}, acc, false);
}
template <> __device__ __forceinline__ float add_pair<__bf16>(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), (bf16x2){1, 1}, acc, false);
}

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }

// Eight floats -> one MFMA operand of T.
template <typename T>
__device__ __forceinline__ typename Vec8<T>::type pack8(float x0, float x1, float x2, float x3,
                                                       float x4, float x5, float x6, float x7) {
  u32x4 w;
  w[0] = pack2<T>(x0, x1);
  w[1] = pack2<T>(x2, x3);
  w[2] = pack2<T>(x4, x5);
  w[3] = pack2<T>(x6, x7);
  return __builtin_bit_cast(typename Vec8<T>::type, w);
}

// ---- LDS access -----------------------------------------------------------
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ u32x2 lds_read_tr16(const char* lds_byte_ptr) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_byte_ptr));
  return __builtin_bit_cast(u32x2, v);
}

// A/B operand of 8 x 16-bit gathered by two transpose reads (rows r0..r0+3
// and r0+8..r0+11 of a row-major tile, pitch in bytes), see header comment.
template <typename T>
__device__ __forceinline__ typename Vec8<T>::type lds_tr_operand(const char* p0, const char* p1) {
  u32x2 lo = lds_read_tr16(p0);
  u32x2 hi = lds_read_tr16(p1);
  u32x4 w;
  w[0] = lo[0];
  w[1] = lo[1];
  w[2] = hi[0];
  w[3] = hi[1];
  return __builtin_bit_cast(typename Vec8<T>::type, w);
}

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type lds_read8(const char* p) {
  return __builtin_bit_cast(typename Vec8<T>::type, *(const u32x4*)p);
}

// ---- global memory through buffer resources -------------------------------
// Loads at byte offsets >= num_bytes return zeros (hardware range check), which
// is how ragged sequence tails are padded without branches.
struct Buf {
  __amdgpu_buffer_rsrc_t r;
};
__device__ __forceinline__ Buf make_buf(const void* base, uint32_t num_bytes) {
  Buf b;
  b.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)num_bytes, 0x00020000);
  return b;
}
__device__ __forceinline__ u32x4 buf_load16(const Buf& b, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(b.r, byte_off, 0, 0));
}

// ---- swizzled LDS tiles filled by direct global -> LDS copies --------------
// buffer_load_dwordx4 ... lds writes lane i's 16 bytes at (M0 base) + 16 i: one
// 1 KiB block of LDS per wave and instruction, whatever global offsets the
// lanes read; lanes whose offset is past the buffer's range write zeros
// (both confirmed on the device).  A tile of ROWS x D 16-bit elements is kept
// row-major in 16-byte chunks, chunk c of row r at position
// r * D/8 + (c ^ swz(r)).  The XOR pattern is a linear map of the four low row
// bits chosen (by exhaustive search over all such maps) so that both access
// patterns of the kernels are free of bank conflicts with 32 or with 64
// four-byte banks: 16 lanes reading 16 bytes each from 16 consecutive rows at
// one chunk (MFMA operands read by rows), and 32 lanes reading 8 bytes each
// from 4 rows x 64 bytes (transpose reads).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 64) {  // 8 chunks per row: bits r1, r0^r2, r0^r1^r3
    return ((r >> 1) & 1) | (((r ^ (r >> 2)) & 1) << 1) | (((r ^ (r >> 1) ^ (r >> 3)) & 1) << 2);
  } else {                   // 16 chunks per row: bits r0, r1, r0^r2, r1^r3
    return (r & 3) | (((r ^ (r >> 2)) & 1) << 2) | ((((r >> 1) ^ (r >> 3)) & 1) << 3);
  }
}
// byte offset of element column `col` of row r in a swizzled tile
template <int D>
__device__ __forceinline__ int swz_off(int r, int col) {
  return (r * (D / 8) + ((col >> 3) ^ swz<D>(r))) * 16 + (col & 7) * 2;
}

typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte-per-lane copy into the 1 KiB LDS block at `block`.  Written as
// inline assembly on purpose: the compiler's wait-count pass treats an LDS DMA
// it knows about as a store to all of LDS and waits for it before every later
// LDS read, including reads of the other buffer stage, which would stall each
// iteration until its prefetch lands.  The caller therefore waits for the
// copies itself (wait_all_memory) before the barrier that publishes them.
__device__ __forceinline__ void dma16(const Buf& b, uint32_t byte_off, char* block) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void*)block;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(byte_off), "s"(b.r)
               : "memory", "m0");
}
// The 4-byte form: lane i's dword lands at block + 4 i (256 bytes per wave);
// each lane's dword is range-checked on its own.
__device__ __forceinline__ void dma4(const Buf& b, uint32_t byte_off, char* block) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void*)block;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(byte_off), "s"(b.r)
               : "memory", "m0");
}

// Copy rows [r0, r0 + ROWS) of a row-major (rows x D) 16-bit tensor held by
// buffer b into the swizzled tile at `tile` (256 threads; each issues
// ROWS*D/2048 copies, copy n of wave w filling 1 KiB block 4n + w).
template <int D, int ROWS>
__device__ __forceinline__ void dma_tile(const Buf& b, int r0, char* tile, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int NI = ROWS * CPR / 256;
  static_assert(ROWS * CPR % 256 == 0, "tile must be a whole number of 1 KiB blocks per wave");
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int P = (n * 4 + wave) * 64 + lane;
    const int r = P / CPR, pc = P % CPR;
    // in 32-bit unsigned arithmetic: rows past N of the largest head reach 2^31 bytes
    const uint32_t off = (uint32_t)((r0 + r) * D + ((pc ^ swz<D>(r)) << 3)) * 2u;
    dma16(b, off, tile + (n * 4 + wave) * 1024);
  }
}

// A/B operand of 8 x 16-bit from two transpose reads of a swizzled tile:
// rows r and r + 8, element columns col .. col + 3 per lane (see header).
template <typename T, int D>
__device__ __forceinline__ typename Vec8<T>::type swz_tr_operand(const char* tile, int r, int col) {
  return lds_tr_operand<T>(tile + swz_off<D>(r, col), tile + swz_off<D>(r + 8, col));
}

// Per-lane byte offsets of the two operand reads of a swizzled tile, taken
// once before the tile loop.  The swizzle depends on the four low row bits
// only, so the same read 16 rows further down (the next k-step or 32-row
// block) or in another LDS stage is this offset plus a constant, which the
// read instruction carries as its immediate: no address arithmetic per read
// once the stage is known at compile time.
//   rows[t]:  lds_read8 at row l32, element columns 16 t + 8 g
//   tr[db][h]: the transpose reads of rows 4 g + (lane % 16) / 4 + 8 h,
//             element columns 32 db + 16 ((lane / 16) % 2) + 4 (lane % 4)
template <int D>
struct TileOffsets {
  int rows[D / 16];
  int tr[D / 32][2];
  __device__ __forceinline__ explicit TileOffsets(int lane) {
    const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) rows[t] = swz_off<D>(l32, t * 16 + g * 8);
    const int r0 = g * 4 + ((lane & 15) >> 2);
    const int c0 = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      tr[db][0] = swz_off<D>(r0, db * 32 + c0);
      tr[db][1] = swz_off<D>(r0 + 8, db * 32 + c0);
    }
  }
  // lds_read8 operand of rows row0 + l32 (row0 a multiple of 16), k-step t
  template <typename T>
  __device__ __forceinline__ typename Vec8<T>::type row_operand(const char* tile, int row0,
                                                                int t) const {
    return lds_read8<T>(tile + row0 * D * 2 + rows[t]);
  }
  // transpose-read operand of rows row0 .. row0 + 15 (row0 a multiple of 16),
  // column block db; equal to swz_tr_operand at row row0 + 4 g + (lane % 16) / 4
  template <typename T>
  __device__ __forceinline__ typename Vec8<T>::type tr_operand(const char* tile, int row0,
                                                               int db) const {
    return lds_tr_operand<T>(tile + row0 * D * 2 + tr[db][0], tile + row0 * D * 2 + tr[db][1]);
  }
};

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>)
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---- workgroup -> work-item mapping -----------------------------------------
// Workgroups are handed to the 8 XCDs round-robin by linear id.  Remap so that
// each XCD receives one contiguous range of the logical order (head-major):
// all tiles of a head then share one L2.  A bijection for any grid size.
__device__ __forceinline__ int xcd_remap(int linear, int total) {
  const int nx = 8;
  int x = linear % nx, slot = linear / nx;
  int per = total / nx, rem = total % nx;
  return x * per + (x < rem ? x : rem) + slot;
}

// Causal work on a small grid (every tile of the launch resident at once, one
// workgroup per tile): the time is the most loaded CU's, so spread the cost
// evenly over CUs.  Workgroup b goes to XCD b mod 8 and, within the XCD, the
// dispatcher fills its CUs in order; XCD x takes the tiles of heads
// [x hx, (x+1) hx) (hx = nheads / 8), sorted by cost (level 0 the costliest),
// and deals them to its cpx CUs in rounds that alternate direction, so that
// each CU's tiles add up to about the same number of key-tile steps.
// A bijection from [0, nheads * ntiles) onto (head, level) whenever
// nheads % 8 == 0.
__device__ __forceinline__ void spread_tile(int b, int nheads, int ntiles, int cpx, int& head,
                                            int& level) {
  const int hx = nheads >> 3, n = hx * ntiles;
  const int x = b & 7, j = b >> 3;
  const int r = j / cpx, k = j % cpx;
  // a last round that fills fewer than cpx CUs runs forward, so that i < n
  const bool reverse = (r & 1) && (r + 1) * cpx <= n;
  const int i = r * cpx + (reverse ? cpx - 1 - k : k);
  head = x * hx + i % hx;
  level = i / hx;
}

// IEEE maximum (NaN-propagating): v_maximum3_f32 on gfx950, no input
// canonicalisation as fmaxf needs.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// maximum of the 16 values of an accumulator block: eight 3-input maxima, depth 3
__device__ __forceinline__ float max16(const f32x16& x) {
  float m5[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) m5[i] = vmax(vmax(x[3 * i], x[3 * i + 1]), x[3 * i + 2]);
  return vmax(vmax(vmax(m5[0], m5[1]), m5[2]), vmax(vmax(m5[3], m5[4]), x[15]));
}

__device__ __forceinline__ float wave_max_pair(float v) {
  // lanes l and l ^ 32 hold the two halves of one query's row
  return vmax(v, __shfl_xor(v, 32, 64));
}

// Lanes l and l ^ 32 exchanged without LDS: v_permlane32_swap_b32 swaps the
// upper 32 lanes of its first operand with the lower 32 lanes of its second,
// so with both operands = v, lo holds v[l % 32] and hi holds v[l % 32 + 32] on
// every lane.  Sum and max of the pair, identical (same operand order) in both
// lanes.
struct LanePair {
  float lo, hi;
};
__device__ __forceinline__ LanePair lane_pair(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return LanePair{__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
}
__device__ __forceinline__ float pair_sum(float v) {
  const LanePair p = lane_pair(v);
  return p.lo + p.hi;
}
__device__ __forceinline__ float pair_max(float v) {
  const LanePair p = lane_pair(v);
  return vmax(p.lo, p.hi);
}

// Compile-time integer as a value (selects unrolled loop bodies).
template <int N>
struct IntC {
  static constexpr int value = N;
};

// Marks a rarely taken uniform branch so the compiler keeps it a branch
// instead of executing its body on every pass with selects.
#define FA_KEEP_BRANCH() __asm__ volatile("" ::: "memory")

// Wait for every outstanding memory operation of this wave.  Used once before
// a tile loop so that the compiler's wait tracking does not carry loads issued
// before the loop (operands kept in registers) into every iteration, where it
// would also wait for the prefetch of the next tile.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Scheduling hint for a block of N LDS operand reads feeding N matrix products
// (read i feeding product i): `ahead` reads first, then one product and one
// read alternately, then the last `ahead` products, so each read is issued
// `ahead` products before its use.  AHEAD = 0 leaves the block to the
// compiler.  Place it after the block's code (it orders that basic block).
template <int N, int AHEAD>
__device__ __forceinline__ void sched_reads_ahead() {
  if constexpr (AHEAD > 0) {
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // LDS reads
#pragma unroll
    for (int i = 0; i < N - AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // matrix products
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
  }
}

// s_waitcnt operand: at most n vector-memory operations of this wave still
// outstanding (they complete in issue order), no wait on the other counters.
constexpr int vmcnt_at_most(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wave index as a wave-uniform (scalar) value, so that branches on it stay
// scalar branches instead of being if-converted.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Debug build: fill `bytes` of LDS at `lds` with a quiet NaN (every thread
// of the workgroup calls it first thing; it ends with a barrier).
__device__ __forceinline__ void debug_fill_lds_nan(char* lds, int bytes) {
  if constexpr (kDebugBuild) {
    for (int i = (int)threadIdx.x * 4; i < bytes; i += (int)blockDim.x * 4)
      *(uint32_t*)(lds + i) = 0x7FC00000u;
    __syncthreads();
  }
}

// Debug build: add `amount` to visits[idx] once per workgroup (thread 0).
__device__ __forceinline__ void debug_visit(int32_t* visits, size_t idx, int amount) {
  if constexpr (kDebugBuild) {
    if (visits != nullptr && threadIdx.x == 0) atomicAdd(visits + idx, amount);
  }
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace fa
