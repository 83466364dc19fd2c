// fa_mask.hip -- compile a dense block mask into the block lists the kernels
// walk: for each query block the kept key blocks (row lists, used by the
// forward and dQ kernels) and for each key block the query blocks that keep it
// (column lists, used by the dK/dV kernel).  Only kept blocks are ever loaded
// or computed, which is how block-sparse attention scales its IO by the
// non-zero fraction (block-sparse paragraph of the agihunt.info summary).
//
// Three launches, each reading the nb x nb mask bytes at most twice:
//   count: workgroup g counts the kept blocks of row g and of column g;
//   scan:  one workgroup turns the counts into the offsets row_ptr, col_ptr;
//   fill:  workgroup g writes the lists of row g and column g, each thread a
//          contiguous chunk at the offset given by a scan of the chunk counts.
// The lists come out in increasing order and identical on every run.
#include "fa_kernels.hpp"

namespace fa {
namespace {

constexpr int kMaskThreads = 256;

// Sum over the workgroup (256 threads); every thread gets the total.
__device__ int block_sum(int v, int* lds) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[wave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kMaskThreads / 64; ++w) t += lds[w];
  return t;
}

// Exclusive prefix sum over the workgroup's threads in thread order: an
// inclusive scan inside each wave (log2 64 lane shifts), then each wave adds
// the totals of the waves before it (lds: kMaskThreads / 64 words).
__device__ int block_exclusive_scan(int v, int* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();  // earlier readers of lds are done
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += lds[w];
  return base + x - v;
}

__global__ __launch_bounds__(kMaskThreads) void mask_count_kernel(const uint8_t* mask, int nb,
                                                                  int32_t* row_ptr,
                                                                  int32_t* col_ptr) {
  __shared__ int lds[kMaskThreads / 64];
  const int g = blockIdx.x;
  int rc = 0, cc = 0;
  for (int c = threadIdx.x; c < nb; c += kMaskThreads) rc += mask[(size_t)g * nb + c] != 0;
  for (int r = threadIdx.x; r < nb; r += kMaskThreads) cc += mask[(size_t)r * nb + g] != 0;
  rc = block_sum(rc, lds);
  cc = block_sum(cc, lds);
  if (threadIdx.x == 0) {
    row_ptr[g + 1] = rc;
    col_ptr[g + 1] = cc;
  }
}

// a[1 .. nb] holds counts; afterwards a[i] = sum of the first i counts.
__device__ void offsets_in_place(int32_t* a, int nb, int* lds) {
  const int per = (nb + kMaskThreads - 1) / kMaskThreads;
  const int lo = min(nb, (int)threadIdx.x * per), hi = min(nb, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += a[i + 1];
  int run = block_exclusive_scan(local, lds);
  for (int i = lo; i < hi; ++i) {
    run += a[i + 1];
    a[i + 1] = run;
  }
  if (threadIdx.x == 0) a[0] = 0;
}

__global__ __launch_bounds__(kMaskThreads) void mask_scan_kernel(int nb, int32_t* row_ptr,
                                                                 int32_t* col_ptr) {
  __shared__ int lds[kMaskThreads / 64];
  offsets_in_place(row_ptr, nb, lds);
  offsets_in_place(col_ptr, nb, lds);
}

__global__ __launch_bounds__(kMaskThreads) void mask_fill_kernel(const uint8_t* mask, int nb,
                                                                 const int32_t* row_ptr,
                                                                 int32_t* col_idx,
                                                                 const int32_t* col_ptr,
                                                                 int32_t* row_idx) {
  __shared__ int lds[kMaskThreads / 64];
  const int g = blockIdx.x;
  const int per = (nb + kMaskThreads - 1) / kMaskThreads;
  const int lo = min(nb, (int)threadIdx.x * per), hi = min(nb, lo + per);
  // row g: its kept columns, in increasing order
  int n = 0;
  for (int c = lo; c < hi; ++c) n += mask[(size_t)g * nb + c] != 0;
  int pos = row_ptr[g] + block_exclusive_scan(n, lds);
  for (int c = lo; c < hi; ++c)
    if (mask[(size_t)g * nb + c] != 0) col_idx[pos++] = c;
  // column g: the rows that keep it, in increasing order
  n = 0;
  for (int r = lo; r < hi; ++r) n += mask[(size_t)r * nb + g] != 0;
  pos = col_ptr[g] + block_exclusive_scan(n, lds);
  for (int r = lo; r < hi; ++r)
    if (mask[(size_t)r * nb + g] != 0) row_idx[pos++] = r;
}

}  // namespace

hipError_t launch_mask_compile(const uint8_t* mask, int nb, int32_t* row_ptr, int32_t* col_idx,
                               int32_t* col_ptr, int32_t* row_idx, hipStream_t s) {
  hipLaunchKernelGGL(mask_count_kernel, dim3(nb), dim3(kMaskThreads), 0, s, mask, nb, row_ptr,
                     col_ptr);
  hipLaunchKernelGGL(mask_scan_kernel, dim3(1), dim3(kMaskThreads), 0, s, nb, row_ptr, col_ptr);
  hipLaunchKernelGGL(mask_fill_kernel, dim3(nb), dim3(kMaskThreads), 0, s, mask, nb, row_ptr,
                     col_idx, col_ptr, row_idx);
  return hipGetLastError();
}

}  // namespace fa
