// fa_tiles.hpp -- which key tiles a query tile visits, and which query tiles a
// key tile visits, under the three visibility rules: all keys, causal
// (key <= query; key tiles entirely in the future are never loaded -- the
// causal-mask section of the marketmaker.cc article), and block-sparse (only
// tiles inside kept mask blocks -- block-sparse paragraph of the agihunt.info
// summary).  Lists are ascending, so under causal the visible part is a prefix.
#pragma once

#include "fa_kernels.hpp"

namespace fa {

// Key tiles of width KT for the query rows [q_lo, q_hi] (inclusive, q_hi < N).
template <int KT, bool CAUSAL, bool MASKED>
struct KeyTileList {
  int count;
  int base;   // MASKED: first entry of the query block's kept-block list
  int per;    // MASKED: key tiles per mask block
  int start0; // dense: first key (always 0)
  const int32_t* cols;
  int mb;

  __device__ __forceinline__ void init(const MaskLists& m, int N, int q_lo, int q_hi) {
    const int nkt = (N + KT - 1) / KT;
    if constexpr (!MASKED) {
      count = CAUSAL ? min(nkt, q_hi / KT + 1) : nkt;
      cols = nullptr;
      base = per = mb = 0;
    } else {
      mb = m.mask_block;
      per = mb / KT;
      const int qb = q_lo / mb;
      base = m.row_ptr[qb];
      const int nk = m.row_ptr[qb + 1] - base;
      cols = m.col_idx;
      if constexpr (!CAUSAL) {
        count = nk * per;
      } else {
        int c = 0;
        for (int i = 0; i < nk; ++i) {
          const int k0 = cols[base + i] * mb;
          if (k0 > q_hi) break;
          c += min(per, (q_hi - k0) / KT + 1);
        }
        count = c;
      }
    }
    start0 = 0;
  }
  __device__ __forceinline__ int key0(int it) const {
    if constexpr (!MASKED) {
      return it * KT;
    } else {
      return cols[base + it / per] * mb + (it % per) * KT;
    }
  }
};

// Query tiles of height QT for the keys [k_lo, k_hi] (inclusive).
template <int QT, bool CAUSAL, bool MASKED>
struct QueryTileList {
  int count;
  int first;  // dense: first query tile
  int base;
  int per;
  const int32_t* rows;
  int mb;

  __device__ __forceinline__ void init(const MaskLists& m, int N, int k_lo) {
    const int nqt = (N + QT - 1) / QT;
    if constexpr (!MASKED) {
      first = CAUSAL ? k_lo / QT : 0;
      count = nqt - first;
      rows = nullptr;
      base = per = mb = 0;
    } else {
      mb = m.mask_block;
      per = mb / QT;
      const int kb = k_lo / mb;
      base = m.col_ptr[kb];
      const int nq = m.col_ptr[kb + 1] - base;
      rows = m.row_idx;
      first = 0;
      if constexpr (!CAUSAL) {
        count = nq * per;
      } else {
        // skip query tiles that end before k_lo; ascending, so they lead
        int skip = 0, total = nq * per;
        for (int i = 0; i < nq; ++i) {
          const int q0 = rows[base + i] * mb;
          if (q0 + mb - 1 < k_lo) { skip += per; continue; }
          if (q0 < k_lo) skip += (k_lo - q0) / QT;
          break;
        }
        first = skip;
        count = total - skip;
      }
    }
  }
  __device__ __forceinline__ int query0(int it) const {
    if constexpr (!MASKED) {
      return (first + it) * QT;
    } else {
      const int j = first + it;
      return rows[base + j / per] * mb + (j % per) * QT;
    }
  }
};

}  // namespace fa
