// fa_fwd.hip -- forward pass of tiled exact attention on gfx950 matrix cores.
//
// One workgroup = 4 waves; each wave owns 32 query rows of one (b, h).  The
// workgroup walks the visible key tiles (64 keys each; 32 at head dim 128);
// per tile it stages K and V in LDS (double-buffered, the next tile's global
// loads in flight while the current one is used) and every wave
//   1. computes its score blocks S^T = K_j Q_i^T (32 keys x 32 queries each)
//      on the matrix cores, fp32 accumulate -- they never leave registers;
//   2. applies the causal / sequence-end mask on the tiles that need it;
//   3. runs the online-softmax update in the base-2 domain, 16 keys at a
//      time: P = 2^(S * scale * log2 e - m) against the row's reference m
//      (moved, with O and l rescaled, only when the weights would overflow;
//      see below), running row sum l += rowsum P;
//   4. accumulates O^T += V_j^T P^T on the matrix cores (P rounded to the
//      input type, V read from LDS with transpose reads).
// After the last tile, O is divided by l once and LSE = (m + log2 l) * ln 2 is
// written (natural log).
//
// This is the query-outer order with the division deferred to the end, as in
// "02 -- FlashAttention como una optimizacion de roofline" (lynx-cortex),
// section "El algoritmo Flash (forward)", and the running max / running sum
// recurrence of the tonho.wtf digest, section "como funciona".
//
// Reference maximum.  The recurrence rescales the accumulated O and l by
// 2^(m_old - m_new) whenever the row maximum grows.  Any reference value gives
// the same O / l and the same m + log2 l, as long as the exponentials stay in
// range; so no row maximum is computed on the common path: each 16-key step
// takes its weights against the row's current reference, and only when the
// new row sum overflows a limit (an fp16 weight above 65504 is infinite; see
// kRowSumLimit) -- or the row has no reference yet -- the step's scores give
// the new maximum, O and l are rescaled and the step's weights recomputed.
// The reference is always a maximum of scores the row has seen, so the
// largest weight so far is >= 1 and the sums keep their precision.  The move
// is decided per wave (any row over the limit moves all rows of the wave).
//
// Register layout: computing S^T (keys as rows) rather than S puts one query
// per lane (lanes l and l+32 share it), so row reductions are in-lane plus one
// exchange with lane l^32, and the probabilities are already laid out as the
// B operand of the P V product (see fa_common.hpp for the MFMA layouts).
#include <type_traits>

#include "fa_common.hpp"
#include "fa_dropout.hpp"
#include "fa_kernels.hpp"
#include "fa_tiles.hpp"

namespace fa {

// A step whose new row sum is not below kRowSumLimit moves the reference.
// fp16 weights above 65504 round to infinity, which the sum carries; bf16 and
// float32 weights stay finite, and the limit keeps each one (and the O
// accumulators, sums of them times V) far from float32 overflow.
constexpr float kRowSumLimit = 0x1p64f;
constexpr float kNoRef = __builtin_huge_valf();  // row sum while a row has no reference

// Workgroup shape: 4 waves, each owning 32 query rows (128 rows per
// workgroup); K and V tiles in a two-stage LDS ring.  Keys per tile: 64 at
// head dim 64, 32 at head dim 128 (two 32 KiB stages would leave room for only
// two workgroups per CU; with 32-key tiles three fit, and the kernel fits the
// 168 VGPRs of three waves) except under dropout, whose generator registers
// allow two waves per SIMD there.  Waves per SIMD that the register budget
// targets (measured on MI355X: 32 rows per wave at 4 waves per SIMD beats 64
// rows per wave at 2; under dropout head dim 64 still fits 4, 10 % faster than
// 2).
constexpr int kFwdWaves = 4;
constexpr int kFwdWpe64 = 4;
constexpr int kFwdWpe128 = 3;
constexpr int kFwdWpe128Drop = 2;

template <int D, int KT_>
struct FwdGeom {
  static constexpr int KT = KT_;                // keys per tile (64, or 32)
  static_assert(KT == 32 || KT == 64, "one or two 32-key halves per tile");
  static constexpr int KBYTES = KT * D * 2;    // K tile (read by rows), swizzled
  static constexpr int VBYTES = KT * D * 2;    // V tile (read by transpose), swizzled
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int NDB = D / 32;            // 32-wide blocks of the head dim
  static constexpr int NKS = D / 16;            // k-steps of the QK^T product
};

template <typename T, int D, bool CAUSAL, bool MASKED, bool DROP, int WPE, int KT, bool PERSIST>
__global__ __attribute__((amdgpu_flat_work_group_size(kFwdWaves * 64, kFwdWaves * 64),
                          amdgpu_waves_per_eu(WPE, WPE)))
void fwd_kernel(FwdParams p) {
  using G = FwdGeom<D, KT>;
  using V8 = typename Vec8<T>::type;
  constexpr int BR = kFwdWaves * 32;  // query rows per workgroup
  __shared__ __attribute__((aligned(16))) char smem[2 * G::STAGE + (DROP ? kFwdWaves * kDropLdsPerWave : 0)];
  debug_fill_lds_nan(smem, sizeof(smem));

  const int lane_ = threadIdx.x & 63;
  const int wave = wave_id();
  const int N = p.N;

  // one query tile of one head
  auto tile = [&](const int head, const int qt) __attribute__((always_inline)) {
    int lane = lane_;
    // in the persistent loop, lane-only values are recomputed per tile rather
    // than kept live across it (registers)
    if constexpr (PERSIST) __asm__ volatile("" : "+v"(lane));
    const int g = lane >> 5;  // which half of the wave
    const int l32 = lane & 31;
    const int q0 = qt * BR;
    const int qw0 = q0 + wave * 32;   // this wave's first query
    const int qw_last = qw0 + 31;
    const int q_hi = min(q0 + BR, N) - 1;

    const size_t head_off = (size_t)head * N * D;
    const size_t kv_off = (size_t)(head / p.group) * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * sizeof(T);
    const Buf bq = make_buf((const T*)p.q + head_off, head_bytes);
    const Buf bk = make_buf((const T*)p.k + kv_off, head_bytes);
    const Buf bv = make_buf((const T*)p.v + kv_off, head_bytes);

    const Band band{N, p.window, CAUSAL};
    const auto tiles = key_tiles<G::KT, MASKED>(p.m, band, q0, q_hi);
    const uint32_t bias = (0x8000u - p.drop.t8) * 0x10001u;  // dropout byte test, see keep_pair_mask

    // Q fragments: B operands of S^T = K Q^T (k = head dim), rows >= N read as 0.
    V8 qf[G::NKS];
#pragma unroll
    for (int t = 0; t < G::NKS; ++t)
      qf[t] = __builtin_bit_cast(V8, buf_load16(bq, (uint32_t)((qw0 + l32) * D + t * 16 + g * 8) * sizeof(T)));

    // The lane's row: m_ref, the reference maximum (-inf until the row has seen
    // a key); ref, the value the weights are taken against (m_ref, or 0 while
    // there is none); l_run, the running sum of the weights (kNoRef while there
    // is no reference, which sends the first step to the reference move).
    f32x16 o[G::NDB];
#pragma unroll
    for (int i = 0; i < G::NDB; ++i) o[i] = f32x16{0};
    float m_ref = kNegInf, ref = 0.f, l_run = kNoRef;

    // K and V tiles go straight from global memory to LDS
    const int nb128 = (N + 127) / 128;
    auto gload = [&](int it, int stage) {
      const int k0 = tiles.pos0(it);
      debug_visit(p.visits, ((size_t)head * p.nqt + qt) * nb128 + k0 / 128, G::KT);
      char* ks = smem + stage * G::STAGE;
      dma_tile<D, G::KT>(bk, k0, ks, wave, lane);
      dma_tile<D, G::KT>(bv, k0, ks + G::KBYTES, wave, lane);
    };

    const int ntiles = tiles.count;
    // The copies of tile it + 1 are issued at the start of step it; a step ends
    // once this thread's copies have landed, and the barrier publishes them.
    if (ntiles > 0) gload(0, 0);
    wait_all_memory();
    __syncthreads();

    const TileOffsets<D> toff(lane);

    // one key tile; the LDS stage is a compile-time constant (the loop below
    // runs two steps per iteration), so it joins the reads' immediate offsets
    auto step = [&](const int it, auto stage) __attribute__((always_inline)) {
      constexpr int cur = decltype(stage)::value;
      if (it + 1 < ntiles) gload(it + 1, 1 - cur);

      const int k0 = tiles.pos0(it);
      const char* ks = smem + cur * G::STAGE;
      const char* vs = ks + G::KBYTES;
      // the wave's rows [qw0, qw_last] see keys [lo(qw0), hi(qw_last)] between
      // them, and every row sees [lo(qw_last), hi(qw0)]
      const bool active = k0 <= band.hi(qw_last) && k0 + G::KT - 1 >= band.lo(qw0);
      if (active) {
        constexpr int NKB = G::KT / 32;  // 32-key halves of the tile
        // 1. S^T = K Q^T for each 32-key half
        f32x16 s[NKB];
#pragma unroll
        for (int j = 0; j < NKB; ++j) {
          s[j] = f32x16{0};
#pragma unroll
          for (int t = 0; t < G::NKS; ++t) s[j] = mfma32(toff.template row_operand<T>(ks, j * 32, t), qf[t], s[j]);
        }
        // head dim 128: the K operand reads issued four products ahead
        // (measured 3 % faster; no change at 64)
        sched_reads_ahead<NKB * G::NKS, D == 128 ? 4 : 0>();
        // 2. mask keys outside the row's band (future keys, keys outside the
        // window, keys past the end).  Key of register r is k0 + g*4 + C(j, r),
        // C = j*32 + (r/4)*8 + r%4; it is hidden iff C < lb or C > ub.
        const bool need_mask = k0 < band.lo(qw_last) || k0 + G::KT - 1 > band.hi(qw0);
        if (need_mask) {
          FA_KEEP_BRANCH();
          // one compare-and-select per bound on the VALU (an OR of the two
          // compares would route every element through the scalar unit)
          const int i = qw0 + l32;
          const int ub = band.hi(i) - k0 - g * 4;
#pragma unroll
          for (int j = 0; j < NKB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int C = j * 32 + (r >> 2) * 8 + (r & 3);
              s[j][r] = C > ub ? kNegInf : s[j][r];
            }
          if (p.window > 0) {
            const int lb = band.lo(i) - k0 - g * 4;
#pragma unroll
            for (int j = 0; j < NKB; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int C = j * 32 + (r >> 2) * 8 + (r & 3);
                s[j][r] = C < lb ? kNegInf : s[j][r];
              }
          }
        }
        // 3-4. per 16-key step: P = 2^(S c - ref) against the row's current
        // reference, packed to the input type, row sums, then O^T += V^T P^T.
        // The reference moves only when a step's weights would overflow (see
        // the header); one compare of the new row sum detects it.  With both
        // halves' scores computed first, the exponentials of half 0 overlap the
        // score products of half 1 still in flight, and those of half 1 the P V
        // products of half 0.
#pragma unroll
        for (int j = 0; j < NKB; ++j) {
          // dropout: generator bytes of this half's keys (byte e of kw[rr]
          // decides the key of register rr * 4 + e)
          u32x4 kw;
          if constexpr (DROP)
            kw = drop_bytes_query_lanes(p.drop, (uint32_t)head, k0 + j * 32, qw0,
                                        smem + 2 * G::STAGE + wave * kDropLdsPerWave, lane);
#pragma unroll
          for (int th = 0; th < 2; ++th) {
            const int r0 = th * 8;
            // the weights of the step's 16 keys and their sum (fp16: of the
            // rounded weights that P V uses; bf16: of the float32 weights, bf16
            // rounding being too coarse for the LSE)
            u32x4 w;
            auto weights = [&]() __attribute__((always_inline)) {
              float lp = 0.f;
#pragma unroll
              for (int h = 0; h < 4; ++h) {
                const float e0 = fast_exp2(__builtin_fmaf(s[j][r0 + 2 * h], p.c, -ref));
                const float e1 = fast_exp2(__builtin_fmaf(s[j][r0 + 2 * h + 1], p.c, -ref));
                w[h] = pack2<T>(e0, e1);
                if constexpr (__is_same(T, _Float16)) lp = add_pair<T>(w[h], lp);
                else lp += e0 + e1;
              }
              return l_run + lp;
            };
            float l_new = weights();
            if (__builtin_amdgcn_ballot_w64(!(l_new < kRowSumLimit)) != 0) {
              FA_KEEP_BRANCH();
              // move the row's reference to the maximum of the row so far (these
              // scores included) and redo the weights
              float mx = kNegInf;
#pragma unroll
              for (int r = 0; r < 8; ++r) mx = vmax(mx, s[j][r0 + r]);
              const float m_new = vmax(m_ref, pair_max(mx * p.c));
              const float r_new = m_new == kNegInf ? 0.f : m_new;
              const bool had = m_ref != kNegInf;
              float alpha = fast_exp2(had ? ref - r_new : kNegInf);  // 0 without a reference
              __asm__ volatile("" : "+v"(alpha));  // one rescale path, not one per case
#pragma unroll
              for (int i = 0; i < G::NDB; ++i) o[i] *= alpha;
              l_run = had ? l_run * alpha : (m_new == kNegInf ? kNoRef : 0.f);
              m_ref = m_new;
              ref = r_new;
              l_new = weights();
            }
            l_run = l_new;
            // dropout zeroes weights after the row sum: LSE normalises P itself
            if constexpr (DROP) {
#pragma unroll
              for (int h = 0; h < 4; ++h) w[h] &= keep_pair_mask(kw[th * 2 + (h >> 1)], h & 1, bias);
            }
            const V8 bp = __builtin_bit_cast(V8, w);
#pragma unroll
            for (int db = 0; db < G::NDB; ++db)
              o[db] = mfma32(toff.template tr_operand<T>(vs, (j * 2 + th) * 16, db), bp, o[db]);
          }
        }
      }
      wait_all_memory();  // this thread's copies of tile it + 1 have landed
      __syncthreads();
    };
    for (int it = 0; it < ntiles; it += 2) {
      step(it, std::integral_constant<int, 0>{});
      if (it + 1 < ntiles) step(it + 1, std::integral_constant<int, 1>{});
    }

    // epilogue: deferred normalisation (and the scale of kept weights under
    // dropout), natural-log LSE
    const int q = qw0 + l32;
    const float lt = pair_sum(m_ref == kNegInf ? 0.f : l_run);
    const float inv = lt > 0.f ? (DROP ? p.drop.mult : 1.f) / lt : 0.f;
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
      // -inf for a row without a visible key; a NaN row sum (a NaN score) stays NaN
      if (g == 0) p.lse[(size_t)head * N + q] = !(lt <= 0.f) ? (m_ref + fast_log2(lt)) * kLn2 : kNegInf;
    }
  };

  if constexpr (PERSIST) {
    // causal work units: the tile pair (nqt - 1 - u, u) of a head, the longer
    // rows first; every unit costs about the same
    const int units = (p.nqt + 1) / 2, total = p.nheads * units;
    for (int b = blockIdx.x; b < total; b += gridDim.x) {
      const int logical = xcd_remap(b, total);
      const int head = logical / units, u = logical % units;
      const int nsub = 2 * u + 1 != p.nqt ? 2 : 1;
      for (int e = 0; e < nsub; ++e) tile(head, e == 0 ? p.nqt - 1 - u : u);
    }
  } else {
    // causal: the longer rows first (one call of the tile body, so that it is
    // inlined once)
    int head, qt;
    if (CAUSAL && p.spread > 0) {
      spread_tile(blockIdx.x, p.nheads, p.nqt, p.spread, head, qt);
    } else {
      const int logical = xcd_remap(blockIdx.x, gridDim.x);
      head = logical / p.nqt;
      qt = logical % p.nqt;
    }
    tile(head, CAUSAL ? p.nqt - 1 - qt : qt);
  }
}

template <typename T, int D, bool MASKED, bool DROP>
static hipError_t launch_fwd_t(FwdParams p, bool causal, hipStream_t s) {
  constexpr int KT = (D == 64 || DROP) ? 64 : 32;
  constexpr int WPE = D == 64 ? kFwdWpe64 : (DROP ? kFwdWpe128Drop : kFwdWpe128);
  constexpr int BR = kFwdWaves * 32;
  p.nqt = (p.N + BR - 1) / BR;
  p.spread = 0;
  static_assert(kFwdWaves * 64 == kThreads, "one workgroup size for all launches");
  // causal work without a window or block mask: one workgroup per tile in the
  // spread order when all tiles fit on the GPU at once, else a persistent
  // grid over tile pairs; the rest one workgroup per tile
  if constexpr (!MASKED)
    if (causal && p.window == 0) {
      constexpr auto kTile = fwd_kernel<T, D, true, false, DROP, WPE, KT, false>;
      p.spread = spread_for<kTile>(p.nheads, p.nqt);
      if (p.spread > 0)
        launch_units<kTile>(p, p.nheads * p.nqt, false, s);
      else
        launch_units<fwd_kernel<T, D, true, false, DROP, WPE, KT, true>>(p, p.nheads * ((p.nqt + 1) / 2), true, s);
      return hipGetLastError();
    }
  if (causal)
    launch_units<fwd_kernel<T, D, true, MASKED, DROP, WPE, KT, false>>(p, p.nheads * p.nqt, false, s);
  else
    launch_units<fwd_kernel<T, D, false, MASKED, DROP, WPE, KT, false>>(p, p.nheads * p.nqt, false, s);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_fwd_dtype(const FwdParams& p, int d, bool causal, bool masked, bool drop,
                                   hipStream_t s) {
  if (d == 64) {
    if (drop) return masked ? launch_fwd_t<T, 64, true, true>(p, causal, s)
                            : launch_fwd_t<T, 64, false, true>(p, causal, s);
    return masked ? launch_fwd_t<T, 64, true, false>(p, causal, s)
                  : launch_fwd_t<T, 64, false, false>(p, causal, s);
  }
  if (drop) return masked ? launch_fwd_t<T, 128, true, true>(p, causal, s)
                          : launch_fwd_t<T, 128, false, true>(p, causal, s);
  return masked ? launch_fwd_t<T, 128, true, false>(p, causal, s)
                : launch_fwd_t<T, 128, false, false>(p, causal, s);
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int d, bool causal, bool masked,
                      hipStream_t s) {
  if (dtype == 1) return launch_fwd_dtype<_Float16>(p, d, causal, masked, false, s);
  return launch_fwd_dtype<__bf16>(p, d, causal, masked, false, s);
}

hipError_t launch_fwd_drop(const FwdParams& p, int dtype, int d, bool causal, bool masked,
                           hipStream_t s) {
  if (dtype == 1) return launch_fwd_dtype<_Float16>(p, d, causal, masked, true, s);
  return launch_fwd_dtype<__bf16>(p, d, causal, masked, true, s);
}

}  // namespace fa
