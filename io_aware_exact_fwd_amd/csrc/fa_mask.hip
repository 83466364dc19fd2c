// fa_mask.hip -- compile a dense block mask into the block lists the kernels
// walk: for each query block the kept key blocks (row lists, used by the
// forward and dQ kernels) and for each key block the query blocks that keep it
// (column lists, used by the dK/dV kernel).  Only kept blocks are ever loaded
// or computed, which is how block-sparse attention scales its IO by the
// non-zero fraction (block-sparse paragraph of the agihunt.info summary).
//
// One workgroup; the mask is small (N/128 blocks on a side).  Counts, then a
// serial prefix sum by one thread, then each thread fills whole rows/columns,
// so the lists come out in increasing order and identical on every run.
#include "fa_kernels.hpp"

namespace fa {

__global__ __launch_bounds__(256) void mask_compile_kernel(const uint8_t* mask, int nb,
                                                           int32_t* row_ptr, int32_t* col_idx,
                                                           int32_t* col_ptr, int32_t* row_idx) {
  const int tid = threadIdx.x;
  for (int r = tid; r < nb; r += blockDim.x) {
    int c_row = 0;
    for (int c = 0; c < nb; ++c) c_row += mask[(size_t)r * nb + c] != 0;
    row_ptr[r + 1] = c_row;
  }
  for (int c = tid; c < nb; c += blockDim.x) {
    int c_col = 0;
    for (int r = 0; r < nb; ++r) c_col += mask[(size_t)r * nb + c] != 0;
    col_ptr[c + 1] = c_col;
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    row_ptr[0] = 0;
    col_ptr[0] = 0;
    for (int i = 0; i < nb; ++i) {
      row_ptr[i + 1] += row_ptr[i];
      col_ptr[i + 1] += col_ptr[i];
    }
  }
  __threadfence();
  __syncthreads();
  for (int r = tid; r < nb; r += blockDim.x) {
    int pos = row_ptr[r];
    for (int c = 0; c < nb; ++c)
      if (mask[(size_t)r * nb + c] != 0) col_idx[pos++] = c;
  }
  for (int c = tid; c < nb; c += blockDim.x) {
    int pos = col_ptr[c];
    for (int r = 0; r < nb; ++r)
      if (mask[(size_t)r * nb + c] != 0) row_idx[pos++] = r;
  }
}

hipError_t launch_mask_compile(const uint8_t* mask, int nb, int32_t* row_ptr, int32_t* col_idx,
                               int32_t* col_ptr, int32_t* row_idx, hipStream_t s) {
  hipLaunchKernelGGL(mask_compile_kernel, dim3(1), dim3(256), 0, s, mask, nb, row_ptr, col_idx,
                     col_ptr, row_idx);
  return hipGetLastError();
}

}  // namespace fa
