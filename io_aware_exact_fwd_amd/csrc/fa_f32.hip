// fa_f32.hip -- float32 path (vector ALU, 32 lanes per query or key).
//
// gfx950's matrix cores do take float32 operands (v_mfma_f32_32x32x2_f32 and
// its 16x16x4 form), at about the rate of the packed float32 vector units; this
// path nevertheless computes on the vector units on purpose: it serves small
// float32 problems (a correctness workload, not a throughput one) and keeps the
// plainest per-thread form of the method -- key tiles staged in LDS, running
// row maximum and sum with rescaling, deferred normalisation, and a backward
// that rebuilds P from Q, K and the LSE with D_i = dO_i . O_i.  Visibility is
// tested per (query, key) pair; no tile is skipped.
//
// Parallelism for small problems: 32 lanes share one query (forward, dQ) or
// one key (dK/dV), lane s taking keys (queries) s, s + 32, ... of every staged
// tile, so a 256-query head runs on 8192 threads instead of 256 (measured on
// the MI355X for N = 256: 16 lanes 1.3x and 8 lanes 1.9x slower, a whole wave
// 3x slower).  Each lane keeps a partial state -- the forward its own running
// maximum, sum and O, which is the online-softmax state of its share of the
// keys; the backward its partial dQ (dK, dV) sums -- and the 32 are merged at
// the end with lane exchanges: the forward takes the largest maximum and
// rescales every partial sum and O to it before adding them (the merge of two
// softmax states that the recurrence itself performs when a new maximum
// appears).
#include <math.h>

#include "fa_common.hpp"
#include "fa_dropout.hpp"
#include "fa_kernels.hpp"

namespace fa {

constexpr int kF32Tile = 128;    // keys (or queries) staged per LDS step
constexpr int kF32Threads = 256;
constexpr int kF32Split = 32;    // lanes per query (key), a power of two within a wave
constexpr int kF32Rows = kF32Threads / kF32Split;  // queries (keys) per workgroup
// Staged rows are padded by four floats: the lanes of a group read different
// rows at one column, and sixteen consecutive rows (one 16-byte read of 16
// lanes) then cover all 64 banks once.
constexpr int kF32Pad = 4;

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

// Sum of x over the kF32Split lanes of this lane's group (butterfly; every
// lane of the group receives the same total, added in the same order).
__device__ __forceinline__ float f32_group_sum(float x) {
#pragma unroll
  for (int w = 1; w < kF32Split; w <<= 1) x += __shfl_xor(x, w);
  return x;
}
__device__ __forceinline__ float f32_group_max(float x) {
#pragma unroll
  for (int w = 1; w < kF32Split; w <<= 1) x = fmaxf(x, __shfl_xor(x, w));
  return x;
}

// Stage rows r0 .. r0 + kF32Tile - 1 of two row-major N x D float tensors
// (rows >= N as zeros) into padded LDS tiles, all threads of the workgroup,
// 16 bytes per load (rows are 16-byte aligned in both).
template <int D>
__device__ __forceinline__ void f32_stage(float (*a)[D + kF32Pad], float (*b)[D + kF32Pad],
                                          const float* ga, const float* gb, int r0, int N) {
  constexpr int C4 = D / 4;
#pragma unroll
  for (int e = threadIdx.x; e < kF32Tile * C4; e += kF32Threads) {
    const int r = e / C4, c = (e % C4) * 4;
    const bool in = r0 + r < N;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    *(float4*)&a[r][c] = in ? *(const float4*)&ga[(size_t)(r0 + r) * D + c] : z;
    *(float4*)&b[r][c] = in ? *(const float4*)&gb[(size_t)(r0 + r) * D + c] : z;
  }
}

template <int D>
__global__ __launch_bounds__(kF32Threads) void f32_fwd_kernel(F32Params p) {
  __shared__ float ks[kF32Tile][D + kF32Pad];
  __shared__ float vs[kF32Tile][D + kF32Pad];
  debug_fill_lds_nan((char*)ks, sizeof(ks));
  debug_fill_lds_nan((char*)vs, sizeof(vs));
  const int head = blockIdx.x;
  const int sub = threadIdx.x % kF32Split;
  const int nrb = (p.N + kF32Rows - 1) / kF32Rows;
  for (int rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
    const int q = rb * kF32Rows + threadIdx.x / kF32Split;
    const size_t hoff = (size_t)head * p.N * D;
    const size_t kvoff = (size_t)(head / p.group) * p.N * D;
    float qv[D], o[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
      qv[c] = q < p.N ? p.q[hoff + (size_t)q * D + c] : 0.f;
      o[c] = 0.f;
    }
    // this lane's share of the row: running maximum and sum (base 2)
    float m = -INFINITY, l = 0.f;
    for (int j0 = 0; j0 < p.N; j0 += kF32Tile) {
      __syncthreads();
      f32_stage<D>(ks, vs, p.k + kvoff, p.v + kvoff, j0, p.N);
      __syncthreads();
#pragma unroll 1
      for (int jj = sub; jj < kF32Tile; jj += kF32Split) {
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
    // merge the group's states at the row's maximum (a lane that saw no
    // key, m = -inf, contributes nothing)
    const float mt = f32_group_max(m);
    const float a = m == -INFINITY ? 0.f : exp2f(m - mt);
    const float lt = f32_group_sum(l * a);
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] = f32_group_sum(o[c] * a);
    if (q < p.N) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      // lane s of the group stores columns s, s + 32, ...
#pragma unroll
      for (int c = 0; c < D; ++c)
        if (c % kF32Split == sub) p.out_o[hoff + (size_t)q * D + c] = o[c] * inv;
      // -inf for a row without a visible key; a NaN row sum stays NaN
      if (sub == 0) p.lse[(size_t)head * p.N + q] = !(lt <= 0.f) ? (mt + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kF32Threads) void f32_dq_kernel(F32Params p) {
  __shared__ float ks[kF32Tile][D + kF32Pad];
  __shared__ float vs[kF32Tile][D + kF32Pad];
  debug_fill_lds_nan((char*)ks, sizeof(ks));
  debug_fill_lds_nan((char*)vs, sizeof(vs));
  const int head = blockIdx.x;
  const int sub = threadIdx.x % kF32Split;
  const int nrb = (p.N + kF32Rows - 1) / kF32Rows;
  for (int rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
    const int q = rb * kF32Rows + threadIdx.x / kF32Split;
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
      if (sub == 0) p.dvec[(size_t)head * p.N + q] = dd;
    }
    for (int j0 = 0; j0 < p.N; j0 += kF32Tile) {
      __syncthreads();
      f32_stage<D>(ks, vs, p.k + kvoff, p.v + kvoff, j0, p.N);
      __syncthreads();
#pragma unroll 1
      for (int jj = sub; jj < kF32Tile; jj += kF32Split) {
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
#pragma unroll
    for (int c = 0; c < D; ++c) dq[c] = f32_group_sum(dq[c]);
    if (q < p.N) {
#pragma unroll
      for (int c = 0; c < D; ++c)
        if (c % kF32Split == sub) p.dq[hoff + (size_t)q * D + c] = dq[c];
    }
  }
}

template <int D>
__global__ __launch_bounds__(kF32Threads) void f32_dkdv_kernel(F32Params p) {
  __shared__ float qs[kF32Tile][D + kF32Pad];
  __shared__ float dos[kF32Tile][D + kF32Pad];
  __shared__ float l2s[kF32Tile];
  __shared__ float dds[kF32Tile];
  debug_fill_lds_nan((char*)qs, sizeof(qs));
  debug_fill_lds_nan((char*)dos, sizeof(dos));
  debug_fill_lds_nan((char*)l2s, sizeof(l2s));
  debug_fill_lds_nan((char*)dds, sizeof(dds));
  const int kvh = blockIdx.x;  // K/V head; its query heads are kvh * group + r
  const int sub = threadIdx.x % kF32Split;
  const int nrb = (p.N + kF32Rows - 1) / kF32Rows;
  for (int rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
    const int kj = rb * kF32Rows + threadIdx.x / kF32Split;
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
        f32_stage<D>(qs, dos, p.q + hoff, p.dout + hoff, i0, p.N);
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
        for (int ii = sub; ii < kF32Tile; ii += kF32Split) {
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
#pragma unroll
    for (int c = 0; c < D; ++c) {
      dk[c] = f32_group_sum(dk[c]);
      dv[c] = f32_group_sum(dv[c]);
    }
    if (kj < p.N) {
#pragma unroll
      for (int c = 0; c < D; ++c)
        if (c % kF32Split == sub) {
          p.dk[kvoff + (size_t)kj * D + c] = dk[c];
          p.dv[kvoff + (size_t)kj * D + c] = dv[c];
        }
    }
  }
}

// (heads, row blocks): the kernels loop over row blocks with a stride of
// gridDim.y, kept below 2^16 (the runtime's limit for that dimension); the
// debug build keeps it at 3, so that its tests run that loop many rounds
static dim3 f32_grid(const F32Params& p) {
  const int nrb = (p.N + kF32Rows - 1) / kF32Rows;
  const int cap = kDebugBuild ? 3 : 65535;
  return dim3(p.nheads, nrb < cap ? nrb : cap);
}

hipError_t launch_f32_fwd(const F32Params& p, hipStream_t s) {
  const dim3 grid = f32_grid(p), block(kF32Threads);
  if (p.d == 64) hipLaunchKernelGGL(f32_fwd_kernel<64>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(f32_fwd_kernel<128>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_f32_dq(const F32Params& p, hipStream_t s) {
  const dim3 grid = f32_grid(p), block(kF32Threads);
  if (p.d == 64) hipLaunchKernelGGL(f32_dq_kernel<64>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(f32_dq_kernel<128>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_f32_dkdv(const F32Params& p, hipStream_t s) {
  const dim3 grid = f32_grid(p), block(kF32Threads);
  if (p.d == 64) hipLaunchKernelGGL(f32_dkdv_kernel<64>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(f32_dkdv_kernel<128>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
