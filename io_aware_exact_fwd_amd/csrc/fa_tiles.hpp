// fa_tiles.hpp -- which key tiles a query tile visits, and which query tiles a
// key tile visits.  Visibility is a band per row -- all keys, causal (key <=
// query: key tiles entirely in the future are never loaded, the causal-mask
// section of the marketmaker.cc article), a sliding window |i - j| < W (the
// practice problems of the lynx-cortex page) -- intersected with a block-sparse
// mask (only tiles inside kept mask blocks, block-sparse paragraph of the
// agihunt.info summary).  Lists are ascending and cover one contiguous range of
// the band, so the visited tiles are a contiguous run of the kept-block list.
#pragma once

#include "fa_kernels.hpp"

namespace fa {

// Band of visible positions, before the block mask.  Key j is visible to
// query i iff lo(i) <= j <= hi(i); equivalently query i sees key j iff
// qlo(j) <= i <= qhi(j).  All four are non-decreasing, so for a run of rows
// [a, b] the union of their bands is [lo(a), hi(b)] and the part common to all
// of them is [lo(b), hi(a)].
struct Band {
  int N;
  int window;  // 0: none
  bool causal;

  __device__ __forceinline__ int lo(int i) const { return window > 0 ? max(0, i - window + 1) : 0; }
  __device__ __forceinline__ int hi(int i) const {
    if (causal) return min(N - 1, i);
    return window > 0 ? min(N - 1, i + window - 1) : N - 1;
  }
  __device__ __forceinline__ int qlo(int j) const {
    if (causal) return j;
    return window > 0 ? max(0, j - window + 1) : 0;
  }
  __device__ __forceinline__ int qhi(int j) const {
    return window > 0 ? min(N - 1, j + window - 1) : N - 1;
  }
};

// Tiles of size TS that meet positions [lo, hi] (inclusive).  Dense: tiles
// first .. first + count - 1.  MASKED: entries first .. first + count - 1 of the
// flattened list "each kept block of `list`, split into mask_block / TS tiles".
// One entry of a compiled mask list.  Read through the constant address space
// so that it becomes a scalar load (the index is uniform across the wave): its
// wait counts scalar and LDS operations only, while a vector load's wait would
// also count the LDS copies of the next tile issued just before, and every
// step would then stall until its prefetch had landed.
__device__ __forceinline__ int32_t list_at(const int32_t* list, int i) {
  return ((const __attribute__((address_space(4))) int32_t*)list)[i];
}

template <int TS, bool MASKED>
struct TileRun {
  int count;
  int first;
  int base;  // MASKED: first entry of the block list
  int per;   // MASKED: tiles per mask block
  int mb;
  const int32_t* blocks;

  __device__ __forceinline__ void init(int lo, int hi, const int32_t* list, int list_base,
                                       int nblocks, int mask_block) {
    first = count = 0;
    blocks = list;
    base = list_base;
    mb = mask_block;
    per = MASKED ? mask_block / TS : 0;
    if (hi < lo) return;
    if constexpr (!MASKED) {
      first = lo / TS;
      count = hi / TS - first + 1;
    } else {
      int skip = 0, c = 0;
      for (int i = 0; i < nblocks; ++i) {
        const int t0 = list_at(blocks, base + i) * mb;
        if (t0 + mb - 1 < lo) {
          skip += per;
          continue;
        }
        if (t0 > hi) break;
        const int ta = (max(lo, t0) - t0) / TS;
        const int tb = (min(hi, t0 + mb - 1) - t0) / TS;
        if (c == 0) skip += ta;
        c += tb - ta + 1;
      }
      first = skip;
      count = c;
    }
  }
  // first position of the it-th visited tile
  __device__ __forceinline__ int pos0(int it) const {
    const int j = first + it;
    if constexpr (!MASKED) {
      return j * TS;
    } else {
      return list_at(blocks, base + j / per) * mb + (j % per) * TS;
    }
  }
};

// Key tiles of width KT for the query rows [q_lo, q_hi] (inclusive, q_hi < N).
template <int KT, bool MASKED>
__device__ __forceinline__ TileRun<KT, MASKED> key_tiles(const MaskLists& m, const Band& b,
                                                        int q_lo, int q_hi) {
  TileRun<KT, MASKED> t;
  if constexpr (MASKED) {
    const int qb = q_lo / m.mask_block;
    const int base = list_at(m.row_ptr, qb);
    t.init(b.lo(q_lo), b.hi(q_hi), m.col_idx, base, list_at(m.row_ptr, qb + 1) - base, m.mask_block);
  } else {
    t.init(b.lo(q_lo), b.hi(q_hi), nullptr, 0, 0, 0);
  }
  return t;
}

// Query tiles of height QT for the keys [k_lo, k_hi] (inclusive, k_lo < N).
template <int QT, bool MASKED>
__device__ __forceinline__ TileRun<QT, MASKED> query_tiles(const MaskLists& m, const Band& b,
                                                          int k_lo, int k_hi) {
  TileRun<QT, MASKED> t;
  k_hi = min(k_hi, b.N - 1);
  if constexpr (MASKED) {
    const int kb = k_lo / m.mask_block;
    const int base = list_at(m.col_ptr, kb);
    t.init(b.qlo(k_lo), b.qhi(k_hi), m.row_idx, base, list_at(m.col_ptr, kb + 1) - base, m.mask_block);
  } else {
    t.init(b.qlo(k_lo), b.qhi(k_hi), nullptr, 0, 0, 0);
  }
  return t;
}

}  // namespace fa
