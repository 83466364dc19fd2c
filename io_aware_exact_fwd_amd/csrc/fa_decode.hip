// fa_decode.hip -- decode-shaped forward: a few queries per head (the last
// n_q positions of the sequence) against N keys and values, the keys split
// over workgroups and the partial results merged.
//
// With n_q queries there is too little work per head to fill the GPU from
// the query side, so the key range is cut into splits (split-K).  Each
// workgroup runs the forward recurrence of fa_fwd.hip over one split -- the
// running maximum / running sum of the online softmax ("como funciona",
// tonho.wtf digest) -- and leaves a partial (O_s normalised, LSE_s); a second
// kernel merges the splits with the same algebra that merges two key blocks
// of one row:  LSE = log sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s
// ("A recorrencia do softmax online", marketmaker.cc article).
//
// Rows.  Under grouped K/V heads the `group` query heads that read one K/V head
// share its keys, so one workgroup serves all of them: row r of K/V head kvh is
// query index r % n_q of query head kvh * group + r / n_q, i.e. row
// kvh * group * n_q + r of the (B, H, n_q) query layout.  Query i sits at
// position N - n_q + i; causal and window visibility use that position.
#include "fa_common.hpp"
#include "fa_kernels.hpp"
#include "fa_tiles.hpp"

namespace fa {

namespace {

constexpr float kDecTau = 8.0f;  // reference move threshold (base 2), as in the forward

// Split kernel: LDS stages (one computed, the others in flight) and waves per
// SIMD.  Measured on MI355X: one to three tiles in flight and two or three
// waves per SIMD ran the same (the kernel streams K and V near the HBM rate).
constexpr int kDecStages = 4;
constexpr int kDecWpe = 2;

template <int D>
struct DecGeom {
  static constexpr int KT = kDecKeys;          // keys per tile
  static constexpr int NST = kDecStages;       // LDS stages: one computed, NST - 1 in flight
  static_assert(NST >= 2, "at least one tile in flight");
  static constexpr int WPE = kDecWpe;           // waves per SIMD
  static constexpr int KBYTES = KT * D * 2;    // K tile, swizzled
  static constexpr int VBYTES = KT * D * 2;    // V tile, swizzled
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int NDB = D / 32;
  static constexpr int NKS = D / 16;
  static constexpr int COPIES = 2 * KT * D / 8 / 256;  // copies per thread per tile (K and V)
};

template <typename T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(DecGeom<D>::WPE, DecGeom<D>::WPE)))
void decode_split_kernel(DecParams p) {
  using G = DecGeom<D>;
  using V8 = typename Vec8<T>::type;
  __shared__ __attribute__((aligned(16))) char smem[G::NST * G::STAGE];
  debug_fill_lds_nan(smem, sizeof(smem));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int g = lane >> 5;
  const int l32 = lane & 31;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int per_kv = p.nrb * p.nsplit;
  const int kvh = logical / per_kv;
  const int rb = (logical % per_kv) / p.nsplit;
  const int sp = logical % p.nsplit;
  const int N = p.N;

  // this lane's row and its position in the key sequence
  const int r = rb * 128 + wave * 32 + l32;
  const bool row_ok = r < p.rows;
  const int pos = row_ok ? N - p.nq + r % p.nq : N - 1;
  const size_t row_g = (size_t)kvh * p.rows + r;  // row of the (B, H, n_q) layout

  const uint32_t kv_bytes = (uint32_t)N * D * sizeof(T);
  const Buf bq = make_buf((const T*)p.q + (size_t)kvh * p.rows * D, (uint32_t)p.rows * D * sizeof(T));
  const Buf bk = make_buf((const T*)p.k + (size_t)kvh * N * D, kv_bytes);
  const Buf bv = make_buf((const T*)p.v + (size_t)kvh * N * D, kv_bytes);

  // key tiles of this split; all rows of the problem lie in positions
  // [N - n_q, N - 1], which bounds the visible keys of every row
  const Band band{N, p.window, CAUSAL};
  const int t_begin = p.tile0 + sp * p.tiles_per_split;
  const int t_end = min(p.tile0 + p.ntiles, t_begin + p.tiles_per_split);
  const int p_lo = N - p.nq, p_hi = N - 1;
  const int w_lo = band.lo(p_lo), w_hi = band.hi(p_hi);  // keys some row sees
  const int c_lo = band.lo(p_hi), c_hi = band.hi(p_lo);  // keys every row sees
  const bool wave_rows = rb * 128 + wave * 32 < p.rows;  // wave has any row

  // Q fragments: B operands of S^T = K Q^T (rows past the head's rows read 0)
  V8 qf[G::NKS];
#pragma unroll
  for (int t = 0; t < G::NKS; ++t)
    qf[t] = __builtin_bit_cast(V8, buf_load16(bq, (uint32_t)(r * D + t * 16 + g * 8) * sizeof(T)));
  // Q has landed before any tile copy is issued, so no wait for Q remains
  // inside the loop (where it would also drain the copies in flight)
  wait_all_memory();

  f32x16 o[G::NDB];
#pragma unroll
  for (int i = 0; i < G::NDB; ++i) o[i] = f32x16{0};
  float m_ref = kNegInf, ref = 0.f, l_run = 0.f;

  // Tile `it` of the split goes to stage it % NST.  Every iteration issues
  // exactly one tile's copies (tiles past the split read beyond the buffer,
  // which writes zeros without touching memory), so the number of copies in
  // flight is a constant and the waits below are exact.
  const int ntl = t_end - t_begin;
  auto issue = [&](int it) {
    const int key0 = it < ntl ? (t_begin + it) * G::KT : N;
    char* ks = smem + (it % G::NST) * G::STAGE;
    dma_tile<D, G::KT>(bk, key0, ks, wave, lane);
    dma_tile<D, G::KT>(bv, key0, ks + G::KBYTES, wave, lane);
  };
#pragma unroll
  for (int it = 0; it < G::NST - 1; ++it) issue(it);

  const int tr_row = (lane & 15) >> 2;
  const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  for (int it = 0; it < ntl; ++it) {
    // tile it has landed (the NST - 2 younger tiles may still be in flight);
    // after the barrier every wave's copies are visible and no wave still
    // reads the stage of tile it - 1, which receives tile it + NST - 1
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most((G::NST - 2) * G::COPIES));
    __syncthreads();
    issue(it + G::NST - 1);
    const int k0 = (t_begin + it) * G::KT;
    const char* ks = smem + (it % G::NST) * G::STAGE;
    const char* vs = ks + G::KBYTES;
    if (!(wave_rows && k0 <= w_hi && k0 + G::KT - 1 >= w_lo)) continue;
    f32x16 s = f32x16{0};
#pragma unroll
    for (int t = 0; t < G::NKS; ++t)
      s = mfma32(lds_read8<T>(ks + swz_off<D>(l32, t * 16 + g * 8)), qf[t], s);
    // keys outside the row's band; key of register rr is k0 + g*4 + C,
    // C = (rr/4)*8 + rr%4
    if (k0 + G::KT - 1 > c_hi) {
      const int ub = band.hi(pos) - k0 - g * 4;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int C = (rr >> 2) * 8 + (rr & 3);
        s[rr] = C > ub ? kNegInf : s[rr];
      }
    }
    if (k0 < c_lo) {
      const int lb = band.lo(pos) - k0 - g * 4;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int C = (rr >> 2) * 8 + (rr & 3);
        s[rr] = C < lb ? kNegInf : s[rr];
      }
    }
    // online softmax and O^T += V^T P^T
    float m4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) m4[i] = vmax(s[i], s[i + 4]);
#pragma unroll
    for (int rr = 8; rr < 16; ++rr) m4[rr & 3] = vmax(m4[rr & 3], s[rr]);
    const float mx = vmax(vmax(m4[0], m4[1]), vmax(m4[2], m4[3])) * p.c;
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + kDecTau) != 0) {
      FA_KEEP_BRANCH();
      const float m_new = vmax(m_ref, pair_max(mx));
      const float r_new = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_ref - r_new);  // 0 while m_ref = -inf
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < G::NDB; ++i) o[i] *= alpha;
      m_ref = m_new;
      ref = r_new;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r0 = t * 8;
      u32x4 w;
      float lp = 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float e0 = fast_exp2(__builtin_fmaf(s[r0 + 2 * h], p.c, -ref));
        const float e1 = fast_exp2(__builtin_fmaf(s[r0 + 2 * h + 1], p.c, -ref));
        w[h] = pack2<T>(e0, e1);
        if constexpr (__is_same(T, _Float16)) {
          lp = add_pair<T>(w[h], lp);  // fp16: the rounded weights P V uses
        } else {
          lp += e0 + e1;  // bf16 rounding is too coarse for the LSE: fp32 sum
        }
      }
      l_run += lp;
      const V8 bp = __builtin_bit_cast(V8, w);
#pragma unroll
      for (int db = 0; db < G::NDB; ++db)
        o[db] = mfma32(swz_tr_operand<T, D>(vs, t * 16 + g * 4 + tr_row, db * 32 + tr_col), bp, o[db]);
    }
  }
  // the copies issued past the last tile must land before this workgroup's
  // LDS can be handed to another one
  wait_all_memory();

  // this split's part of the row: O / l and LSE (natural log), -inf if the
  // split holds no visible key of the row
  const float lt = pair_sum(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (m_ref + fast_log2(lt)) * kLn2 : kNegInf;
  if (!row_ok) return;
  if (p.nsplit == 1) {
    T* orow = (T*)p.o + row_g * D;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        u32x2 w;
        w[0] = pack2<T>(o[db][rr * 4 + 0] * inv, o[db][rr * 4 + 1] * inv);
        w[1] = pack2<T>(o[db][rr * 4 + 2] * inv, o[db][rr * 4 + 3] * inv);
        *(u32x2*)(orow + db * 32 + rr * 8 + g * 4) = w;
      }
    if (g == 0) p.lse[row_g] = lse;
  } else {
    const size_t slot = row_g * p.nsplit + sp;
    float* prow = p.part_o + slot * D;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = o[db][rr * 4 + e] * inv;
        *(f32x4*)(prow + db * 32 + rr * 8 + g * 4) = w;
      }
    if (g == 0) p.part_lse[slot] = lse;
  }
}

// Merge: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.  A row no
// split sees gets O = 0, LSE = -inf.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecParams p, int total_rows) {
  // one wave per output row: the wave reduces the splits' LSE (max, then sum
  // of exponentials), then each lane accumulates D / 64 columns
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave_id();
  if (row >= total_rows) return;
  const int ns = p.nsplit;
  const float* pl = p.part_lse + (size_t)row * ns;
  float m = kNegInf;
  for (int s = lane; s < ns; s += 64) m = vmax(m, pl[s]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = vmax(m, __shfl_xor(m, o, 64));
  float lse = kNegInf;
  float acc[D / 64];
#pragma unroll
  for (int j = 0; j < D / 64; ++j) acc[j] = 0.f;
  if (m != kNegInf) {
    float sum = 0.f;
    for (int s = lane; s < ns; s += 64) sum += fast_exp2((pl[s] - m) * kLog2e);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
    lse = m + fast_log2(sum) * kLn2;
    const float* po = p.part_o + (size_t)row * ns * D + lane;
    // eight splits' loads in flight at a time (5 % of the call on decode_gqa)
#pragma unroll 8
    for (int s = 0; s < ns; ++s) {
      const float w = fast_exp2((pl[s] - lse) * kLog2e);  // 0 for LSE_s = -inf
#pragma unroll
      for (int j = 0; j < D / 64; ++j) acc[j] += w * po[(size_t)s * D + j * 64];
    }
  }
  T* orow = (T*)p.o + (size_t)row * D + lane;
#pragma unroll
  for (int j = 0; j < D / 64; ++j) orow[j * 64] = (T)acc[j];
  if (lane == 0) p.lse[row] = lse;
}

template <typename T, int D>
hipError_t launch_decode_t(const DecParams& p, bool causal, hipStream_t s) {
  dim3 grid(p.nkv * p.nrb * p.nsplit), block(256);
  if (causal)
    hipLaunchKernelGGL((decode_split_kernel<T, D, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<T, D, false>), grid, block, 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  const int total_rows = p.nkv * p.rows;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((total_rows + 3) / 4), dim3(256), 0, s, p,
                     total_rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecParams& p, int dtype, int d, bool causal, hipStream_t s) {
  if (dtype == 1)
    return d == 64 ? launch_decode_t<_Float16, 64>(p, causal, s)
                   : launch_decode_t<_Float16, 128>(p, causal, s);
  return d == 64 ? launch_decode_t<__bf16, 64>(p, causal, s) : launch_decode_t<__bf16, 128>(p, causal, s);
}

}  // namespace fa
