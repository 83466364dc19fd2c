// fa_f32.hip -- float32 path (vector ALU, one query or one key per thread).
//
// gfx950's matrix cores do take float32 operands (v_mfma_f32_32x32x2_f32 and
// its 16x16x4 form), at about the rate of the packed float32 vector units; this
// path nevertheless computes on the vector units on purpose: it serves small
// float32 problems (a correctness workload, not a throughput one) and keeps the
// plainest per-thread form of the method -- key tiles staged in LDS, running
// row maximum and sum with rescaling, deferred normalisation, and a backward
// that rebuilds P from Q, K and the LSE with D_i = dO_i . O_i.  Visibility is
// tested per (query, key) pair; no tile is skipped.  It is not tuned.
#include <math.h>

#include "fa_common.hpp"
#include "fa_dropout.hpp"
#include "fa_kernels.hpp"

namespace fa {

constexpr int kF32Tile = 32;   // keys (or queries) staged per LDS step
constexpr int kF32Threads = 64;

__device__ __forceinline__ bool f32_visible(const F32Params& p, int qi, int kj) {
  if (kj >= p.N || qi >= p.N) return false;
  if (p.causal && kj > qi) return false;
  if (p.window > 0 && (kj - qi >= p.window || qi - kj >= p.window)) return false;
  if (p.block_mask) {
    const int nb = p.N / p.mask_block;
    return p.block_mask[(qi / p.mask_block) * nb + kj / p.mask_block] != 0;
  }
  return true;
}

// Dropout multiplier of weight (qi, kj) of query head `head`: 0 if dropped,
// the scale of kept weights otherwise (one generator evaluation per weight:
// this path is not tuned).
__device__ __forceinline__ float f32_drop(const F32Params& p, int head, int qi, int kj) {
  if (p.drop.t8 == 0) return 1.f;
  const u32x4 x = philox4x32_10((uint32_t)kj >> 2, (uint32_t)qi >> 2, (uint32_t)head,
                                p.drop.offset, p.drop.k0, p.drop.k1);
  return keep_byte(x[qi & 3], kj & 3, p.drop.t8) ? p.drop.mult : 0.f;
}

template <int D>
__global__ __launch_bounds__(kF32Threads) void f32_fwd_kernel(F32Params p) {
  __shared__ float ks[kF32Tile][D];
  __shared__ float vs[kF32Tile][D];
  const int head = blockIdx.x;
  const int q = blockIdx.y * kF32Threads + threadIdx.x;
  const size_t hoff = (size_t)head * p.N * D;
  const size_t kvoff = (size_t)(head / p.group) * p.N * D;
  float qv[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = q < p.N ? p.q[hoff + (size_t)q * D + c] : 0.f;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j0 = 0; j0 < p.N; j0 += kF32Tile) {
    __syncthreads();
    for (int e = threadIdx.x; e < kF32Tile * D; e += kF32Threads) {
      const int r = e / D, c = e % D;
      const bool in = j0 + r < p.N;
      ks[r][c] = in ? p.k[kvoff + (size_t)(j0 + r) * D + c] : 0.f;
      vs[r][c] = in ? p.v[kvoff + (size_t)(j0 + r) * D + c] : 0.f;
    }
    __syncthreads();
    // serial running max / sum over the staged keys (one key at a time)
#pragma unroll 1
    for (int jj = 0; jj < kF32Tile; ++jj) {
      if (!f32_visible(p, q, j0 + jj)) continue;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc = fmaf(qv[c], ks[jj][c], acc);
      const float sc = acc * p.c;
      if (sc > m) {
        const float alpha = exp2f(m - sc);
        l *= alpha;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] *= alpha;
        m = sc;
      }
      const float e = exp2f(sc - m);
      l += e;  // the row sum normalises P itself; dropout acts on the weights only
      const float ez = e * f32_drop(p, head, q, j0 + jj);
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(ez, vs[jj][c], o[c]);
    }
  }
  if (q < p.N) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) p.out_o[hoff + (size_t)q * D + c] = o[c] * inv;
    p.lse[(size_t)head * p.N + q] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D>
__global__ __launch_bounds__(kF32Threads) void f32_dq_kernel(F32Params p) {
  __shared__ float ks[kF32Tile][D];
  __shared__ float vs[kF32Tile][D];
  const int head = blockIdx.x;
  const int q = blockIdx.y * kF32Threads + threadIdx.x;
  const size_t hoff = (size_t)head * p.N * D;
  const size_t kvoff = (size_t)(head / p.group) * p.N * D;
  float qv[D], dov[D], dq[D];
  float dd = 0.f;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    const bool in = q < p.N;
    qv[c] = in ? p.q[hoff + (size_t)q * D + c] : 0.f;
    dov[c] = in ? p.dout[hoff + (size_t)q * D + c] : 0.f;
    dd = fmaf(dov[c], in ? p.o[hoff + (size_t)q * D + c] : 0.f, dd);
    dq[c] = 0.f;
  }
  float lse2 = INFINITY;
  if (q < p.N) {
    const float l = p.lse[(size_t)head * p.N + q];
    if (l != -INFINITY) lse2 = l * kLog2e;
    p.dvec[(size_t)head * p.N + q] = dd;
  }
  for (int j0 = 0; j0 < p.N; j0 += kF32Tile) {
    __syncthreads();
    for (int e = threadIdx.x; e < kF32Tile * D; e += kF32Threads) {
      const int r = e / D, c = e % D;
      const bool in = j0 + r < p.N;
      ks[r][c] = in ? p.k[kvoff + (size_t)(j0 + r) * D + c] : 0.f;
      vs[r][c] = in ? p.v[kvoff + (size_t)(j0 + r) * D + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 1
    for (int jj = 0; jj < kF32Tile; ++jj) {
      if (!f32_visible(p, q, j0 + jj)) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        s = fmaf(qv[c], ks[jj][c], s);
        dp = fmaf(dov[c], vs[jj][c], dp);
      }
      const float pr = exp2f(s * p.c - lse2);
      const float ds = pr * (dp * f32_drop(p, head, q, j0 + jj) - dd) * p.scale;
#pragma unroll
      for (int c = 0; c < D; ++c) dq[c] = fmaf(ds, ks[jj][c], dq[c]);
    }
  }
  if (q < p.N) {
#pragma unroll
    for (int c = 0; c < D; ++c) p.dq[hoff + (size_t)q * D + c] = dq[c];
  }
}

template <int D>
__global__ __launch_bounds__(kF32Threads) void f32_dkdv_kernel(F32Params p) {
  __shared__ float qs[kF32Tile][D];
  __shared__ float dos[kF32Tile][D];
  __shared__ float l2s[kF32Tile];
  __shared__ float dds[kF32Tile];
  const int kvh = blockIdx.x;  // K/V head; its query heads are kvh * group + r
  const int kj = blockIdx.y * kF32Threads + threadIdx.x;
  const size_t kvoff = (size_t)kvh * p.N * D;
  float kv[D], vv[D], dk[D], dv[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    const bool in = kj < p.N;
    kv[c] = in ? p.k[kvoff + (size_t)kj * D + c] : 0.f;
    vv[c] = in ? p.v[kvoff + (size_t)kj * D + c] : 0.f;
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  for (int r = 0; r < p.group; ++r) {
    const int head = kvh * p.group + r;
    const size_t hoff = (size_t)head * p.N * D;
    for (int i0 = 0; i0 < p.N; i0 += kF32Tile) {
      __syncthreads();
      for (int e = threadIdx.x; e < kF32Tile * D; e += kF32Threads) {
        const int rr = e / D, c = e % D;
        const bool in = i0 + rr < p.N;
        qs[rr][c] = in ? p.q[hoff + (size_t)(i0 + rr) * D + c] : 0.f;
        dos[rr][c] = in ? p.dout[hoff + (size_t)(i0 + rr) * D + c] : 0.f;
      }
      if (threadIdx.x < kF32Tile) {
        const int qi = i0 + threadIdx.x;
        float l2 = INFINITY, dd = 0.f;
        if (qi < p.N) {
          const float l = p.lse[(size_t)head * p.N + qi];
          if (l != -INFINITY) l2 = l * kLog2e;
          dd = p.dvec[(size_t)head * p.N + qi];
        }
        l2s[threadIdx.x] = l2;
        dds[threadIdx.x] = dd;
      }
      __syncthreads();
#pragma unroll 1
      for (int ii = 0; ii < kF32Tile; ++ii) {
        if (!f32_visible(p, i0 + ii, kj)) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
          s = fmaf(qs[ii][c], kv[c], s);
          dp = fmaf(dos[ii][c], vv[c], dp);
        }
        const float pr = exp2f(s * p.c - l2s[ii]);
        const float z = f32_drop(p, head, i0 + ii, kj);
        const float ds = pr * (dp * z - dds[ii]) * p.scale;
        const float pz = pr * z;
#pragma unroll
        for (int c = 0; c < D; ++c) {
          dv[c] = fmaf(pz, dos[ii][c], dv[c]);
          dk[c] = fmaf(ds, qs[ii][c], dk[c]);
        }
      }
    }
  }
  if (kj < p.N) {
#pragma unroll
    for (int c = 0; c < D; ++c) {
      p.dk[kvoff + (size_t)kj * D + c] = dk[c];
      p.dv[kvoff + (size_t)kj * D + c] = dv[c];
    }
  }
}

hipError_t launch_f32_fwd(const F32Params& p, hipStream_t s) {
  dim3 grid(p.nheads, (p.N + kF32Threads - 1) / kF32Threads), block(kF32Threads);
  if (p.d == 64) hipLaunchKernelGGL(f32_fwd_kernel<64>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(f32_fwd_kernel<128>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_f32_dq(const F32Params& p, hipStream_t s) {
  dim3 grid(p.nheads, (p.N + kF32Threads - 1) / kF32Threads), block(kF32Threads);
  if (p.d == 64) hipLaunchKernelGGL(f32_dq_kernel<64>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(f32_dq_kernel<128>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_f32_dkdv(const F32Params& p, hipStream_t s) {
  dim3 grid(p.nheads, (p.N + kF32Threads - 1) / kF32Threads), block(kF32Threads);
  if (p.d == 64) hipLaunchKernelGGL(f32_dkdv_kernel<64>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(f32_dkdv_kernel<128>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
