// fa_fwd.hip -- forward pass of tiled exact attention on gfx950 matrix cores.
//
// One workgroup = 4 waves = 128 query rows of one (b, h); each wave owns 32
// rows.  The workgroup walks the visible key tiles (64 keys each) in order;
// per tile it stages K and V in LDS (double-buffered, the next tile's global
// loads in flight while the current one is used) and every wave
//   1. computes its score block S^T = K_j Q_i^T (64 keys x 32 queries) on the
//      matrix cores, fp32 accumulate -- the block never leaves registers;
//   2. applies the causal / sequence-end mask on the tiles that need it;
//   3. runs the online-softmax update: new row maximum, rescale factor
//      alpha = 2^(m_old - m_new), P = 2^(S * scale * log2 e - m_new), running
//      row sum l <- alpha * l + rowsum(P), O <- alpha * O;
//   4. accumulates O^T += V_j^T P^T on the matrix cores (P rounded to the
//      input type, V read from LDS with transpose reads).
// After the last tile, O is divided by l once and LSE = (m + log2 l) * ln 2 is
// written (natural log).
//
// This is the query-outer order with the division deferred to the end, as in
// "02 -- FlashAttention como una optimizacion de roofline" (lynx-cortex),
// section "El algoritmo Flash (forward)", and the recurrence of the tonho.wtf
// digest, section "como funciona"; the running maximum and sum are kept in the
// base-2 exponential domain (a change of base, same result).
//
// Register layout: computing S^T (keys as rows) rather than S puts one query
// per lane (lanes l and l+32 share it), so row reductions are in-lane plus one
// exchange with lane l^32, and the probabilities are already laid out as the
// B operand of the P V product (see fa_common.hpp for the MFMA layouts).
#include "fa_common.hpp"
#include "fa_kernels.hpp"
#include "fa_tiles.hpp"

namespace fa {

template <int D>
struct FwdGeom {
  static constexpr int KT = kKeyTile;           // keys per tile
  static constexpr int KP = D * 2 + 16;         // K tile pitch (bytes)
  static constexpr int VP = D * 2 + 32;         // V tile pitch (bytes)
  static constexpr int KBYTES = KT * KP;
  static constexpr int VBYTES = KT * VP;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int CPT = KT * CPR / kThreads;  // chunks per thread per tensor
  static constexpr int NDB = D / 32;            // 32-wide blocks of the head dim
  static constexpr int NKS = D / 16;            // k-steps of the QK^T product
};

template <typename T, int D, bool CAUSAL, bool MASKED>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdParams p) {
  using G = FwdGeom<D>;
  using V8 = typename Vec8<T>::type;
  __shared__ __attribute__((aligned(16))) char smem[2 * G::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;        // which half of the wave
  const int l32 = lane & 31;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int head = logical / p.nqt;
  int qt = logical % p.nqt;
  if (CAUSAL) qt = p.nqt - 1 - qt;  // longest rows first
  const int N = p.N;
  const int q0 = qt * kFwdRows;
  const int qw0 = q0 + wave * 32;   // this wave's first query
  const int q = qw0 + l32;          // this lane's query
  const int q_hi = min(q0 + kFwdRows, N) - 1;

  const size_t head_off = (size_t)head * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * sizeof(T);
  const Buf bq = make_buf((const T*)p.q + head_off, head_bytes);
  const Buf bk = make_buf((const T*)p.k + head_off, head_bytes);
  const Buf bv = make_buf((const T*)p.v + head_off, head_bytes);

  KeyTileList<G::KT, CAUSAL, MASKED> tiles;
  tiles.init(p.m, N, q0, q_hi);

  // Q fragments: B operand of S^T = K Q^T (k = head dim), rows >= N read as 0.
  V8 qf[G::NKS];
#pragma unroll
  for (int t = 0; t < G::NKS; ++t)
    qf[t] = __builtin_bit_cast(V8, buf_load16(bq, (uint32_t)(q * D + t * 16 + g * 8) * sizeof(T)));

  f32x16 o[G::NDB];
#pragma unroll
  for (int i = 0; i < G::NDB; ++i) o[i] = f32x16{0};
  float m_run = kNegInf, l_run = 0.f;

  u32x4 pk[G::CPT], pv[G::CPT];
  auto gload = [&](int it) {
    const int k0 = tiles.key0(it);
#pragma unroll
    for (int i = 0; i < G::CPT; ++i) {
      const int ci = tid + i * kThreads;
      const int row = ci / G::CPR, cc = ci % G::CPR;
      const uint32_t off = (uint32_t)((k0 + row) * D * sizeof(T) + cc * 16);
      pk[i] = buf_load16(bk, off);
      pv[i] = buf_load16(bv, off);
    }
  };
  auto lstore = [&](int stage) {
    char* ks = smem + stage * G::STAGE;
    char* vs = ks + G::KBYTES;
#pragma unroll
    for (int i = 0; i < G::CPT; ++i) {
      const int ci = tid + i * kThreads;
      const int row = ci / G::CPR, cc = ci % G::CPR;
      *(u32x4*)(ks + row * G::KP + cc * 16) = pk[i];
      *(u32x4*)(vs + row * G::VP + cc * 16) = pv[i];
    }
  };

  const int ntiles = tiles.count;
  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < ntiles;
    if (more) gload(it + 1);

    const int k0 = tiles.key0(it);
    const char* ks = smem + cur * G::STAGE;
    const char* vs = ks + G::KBYTES;
    const bool active = !CAUSAL || k0 <= qw0 + 31;
    if (active) {
      // 1. S^T = K Q^T, two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{0};
#pragma unroll
        for (int t = 0; t < G::NKS; ++t) {
          const V8 a = lds_read8<T>(ks + (kb * 32 + l32) * G::KP + t * 32 + g * 16);
          s[kb] = mfma32(a, qf[t], s[kb]);
        }
      }
      // 2. mask keys in the future of the query, and keys past the end
      const bool need_mask = (CAUSAL && k0 + G::KT - 1 > qw0) || (k0 + G::KT > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
            const bool hide = (CAUSAL && key > q) || key >= N;
            if (hide) s[kb][r] = kNegInf;
          }
      }
      // 3. online softmax (base-2 domain)
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = wave_max_pair(mx);
      const float m_new = fmaxf(m_run, mx * p.c);
      const float ref = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - ref);
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(__builtin_fmaf(s[kb][r], p.c, -ref));
          s[kb][r] = e;
          lsum += e;
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < G::NDB; ++i) o[i] *= alpha;
      // 4. O^T += V^T P^T; k-step t covers keys 16t .. 16t+15
      V8 bp[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kb = t >> 1, r0 = (t & 1) * 8;
        bp[t] = pack8<T>(s[kb][r0 + 0], s[kb][r0 + 1], s[kb][r0 + 2], s[kb][r0 + 3],
                         s[kb][r0 + 4], s[kb][r0 + 5], s[kb][r0 + 6], s[kb][r0 + 7]);
      }
      const int tr_row = (lane & 15) >> 2;
      const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
#pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const char* p0 = vs + (t * 16 + g * 4 + tr_row) * G::VP + (db * 32 + tr_col) * 2;
          const V8 a = lds_tr_operand<T>(p0, p0 + 8 * G::VP);
          o[db] = mfma32(a, bp[t], o[db]);
        }
      }
    }
    if (more) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: deferred normalisation, natural-log LSE
  const float lt = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (q < N) {
    T* orow = (T*)p.o + head_off + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        u32x2 w;
        w[0] = pack2<T>(o[db][rr * 4 + 0] * inv, o[db][rr * 4 + 1] * inv);
        w[1] = pack2<T>(o[db][rr * 4 + 2] * inv, o[db][rr * 4 + 3] * inv);
        *(u32x2*)(orow + db * 32 + rr * 8 + g * 4) = w;
      }
    if (g == 0)
      p.lse[(size_t)head * N + q] = lt > 0.f ? (m_run + fast_log2(lt)) * kLn2 : kNegInf;
  }
}

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdParams& p, bool causal, bool masked, hipStream_t s) {
  dim3 grid(p.nheads * p.nqt), block(kThreads);
  if (causal && masked) hipLaunchKernelGGL((fwd_kernel<T, D, true, true>), grid, block, 0, s, p);
  else if (causal) hipLaunchKernelGGL((fwd_kernel<T, D, true, false>), grid, block, 0, s, p);
  else if (masked) hipLaunchKernelGGL((fwd_kernel<T, D, false, true>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((fwd_kernel<T, D, false, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int d, bool causal, bool masked,
                      hipStream_t s) {
  if (dtype == 1) {
    return d == 64 ? launch_fwd_t<_Float16, 64>(p, causal, masked, s)
                   : launch_fwd_t<_Float16, 128>(p, causal, masked, s);
  }
  return d == 64 ? launch_fwd_t<__bf16, 64>(p, causal, masked, s)
                 : launch_fwd_t<__bf16, 128>(p, causal, masked, s);
}

}  // namespace fa
