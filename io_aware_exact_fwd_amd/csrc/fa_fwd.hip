// fa_fwd.hip -- forward pass of tiled exact attention on gfx950 matrix cores.
//
// One workgroup = NW waves; each wave owns QB blocks of 32 query rows of one
// (b, h).  The workgroup walks the visible key tiles (64 keys each) in order;
// per tile it stages K and V in LDS (double-buffered, the next tile's global
// loads in flight while the current one is used) and every wave
//   1. computes its score blocks S^T = K_j Q_i^T (64 keys x 32 queries each)
//      on the matrix cores, fp32 accumulate -- they never leave registers;
//      every K fragment read from LDS feeds QB products;
//   2. applies the causal / sequence-end mask on the tiles that need it;
//   3. runs the online-softmax update in the base-2 domain, 16 keys at a
//      time: P = 2^(S * scale * log2 e - m) against the row's reference m
//      (moved, with O and l rescaled, only when the weights would overflow;
//      see below), running row sum l += rowsum P;
//   4. accumulates O^T += V_j^T P^T on the matrix cores (P rounded to the
//      input type, V read from LDS with transpose reads, each V fragment
//      feeding QB products).
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

// Tuning knobs of the dense head-dim-64 forward: waves per workgroup, 32-row
// query blocks per wave, waves per SIMD the register budget targets.  Measured
// on MI355X: 32 rows per wave at 4 waves per SIMD (112 VGPRs) beats 64 rows per
// wave at 2 waves per SIMD; latency hiding across waves matters more there than
// reusing each LDS fragment twice.
#ifndef FA_FWD64_NW
#define FA_FWD64_NW 4
#endif
#ifndef FA_FWD64_QB
#define FA_FWD64_QB 1
#endif
#ifndef FA_FWD_AHEAD
#define FA_FWD_AHEAD 0  // LDS reads issued ahead of the score products (0: compiler's order)
#endif
#ifndef FA_FWD_HALVES
#define FA_FWD_HALVES 0  // 1: each 32-key half of a tile runs scores to P V before the next
#endif
#ifndef FA_FWD64_WPE
#define FA_FWD64_WPE 4
#endif
#ifndef FA_FWD_CHECK_KEYS
#define FA_FWD_CHECK_KEYS 16
#endif
// Block-sparse, head dim 64: LDS stages and waves per SIMD.  Three stages keep
// the copies of two scattered key tiles in flight (48 KiB per workgroup, so
// three waves per SIMD); on the N = 65536 butterfly workload two stages at four
// waves measured 7 % faster.
// Head dim 128: keys per tile and waves per SIMD.  A 64-key tile pair of
// stages takes 64 KiB of LDS (two workgroups per CU); 32-key tiles take
// 32 KiB, so three fit, and the kernel fits the 168 VGPRs of three waves.
// Measured on MI355X: equal on the N = 8192 causal shape, 4 % faster with a
// 512-key window, 1.4 % faster with 64 query heads on 8 K/V heads.
#ifndef FA_FWD128_KT
#define FA_FWD128_KT 32
#endif
#ifndef FA_FWD128_WPE
#define FA_FWD128_WPE 3
#endif
#ifndef FA_FWD64_DROP_WPE
#define FA_FWD64_DROP_WPE 4  // dropout forward, head dim 64 (126 VGPRs; 10 % faster than 2)
#endif
#ifndef FA_FWD64_MASKED_NST
#define FA_FWD64_MASKED_NST 2
#endif
#ifndef FA_FWD64_MASKED_WPE
#define FA_FWD64_MASKED_WPE 4
#endif

template <int D, int NW, int KT_ = kKeyTile>
struct FwdGeom {
  static constexpr int KT = KT_;                // keys per tile (64, or 32)
  static_assert(KT == 32 || KT == 64, "one or two 32-key halves per tile");
  static constexpr int KBYTES = KT * D * 2;    // K tile (read by rows), swizzled
  static constexpr int VBYTES = KT * D * 2;    // V tile (read by transpose), swizzled
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int NDB = D / 32;            // 32-wide blocks of the head dim
  static constexpr int NKS = D / 16;            // k-steps of the QK^T product
  static_assert(NW == 4, "the tile copies assume 4 waves");
};

template <typename T, int D, bool CAUSAL, bool MASKED, bool DROP, int NW, int QB, int WPE, int NST,
          int KT>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(WPE, WPE)))
void fwd_kernel(FwdParams p) {
  using G = FwdGeom<D, NW, KT>;
  using V8 = typename Vec8<T>::type;
  constexpr int BR = NW * QB * 32;  // query rows per workgroup
  constexpr int WQ = QB * 32;       // query rows per wave
  static_assert(NST == 2 || NST == 3, "two or three LDS stages");
  __shared__ __attribute__((aligned(16))) char smem[NST * G::STAGE + (DROP ? NW * kDropLdsPerWave : 0)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int g = lane >> 5;        // which half of the wave
  const int l32 = lane & 31;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int head = logical / p.nqt;
  int qt = logical % p.nqt;
  if (CAUSAL) qt = p.nqt - 1 - qt;  // longest rows first
  const int N = p.N;
  const int q0 = qt * BR;
  const int qw0 = q0 + wave * WQ;   // this wave's first query
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
  V8 qf[QB][G::NKS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int t = 0; t < G::NKS; ++t)
      qf[qb][t] = __builtin_bit_cast(
          V8, buf_load16(bq, (uint32_t)((qw0 + qb * 32 + l32) * D + t * 16 + g * 8) * sizeof(T)));

  // Per row: m_ref, the reference maximum (-inf until the row has seen a
  // key); ref, the value the weights are taken against (m_ref, or 0 while
  // there is none); l_run, the running sum of the weights (kNoRef while there
  // is no reference, which sends the first step to the reference move).
  f32x16 o[QB][G::NDB];
  float m_ref[QB], ref[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int i = 0; i < G::NDB; ++i) o[qb][i] = f32x16{0};
    m_ref[qb] = kNegInf;
    ref[qb] = 0.f;
    l_run[qb] = kNoRef;
  }

  // K and V tiles go straight from global memory to LDS
  auto gload = [&](int it, int stage) {
    const int k0 = tiles.pos0(it);
    char* ks = smem + stage * G::STAGE;
    dma_tile<D, G::KT>(bk, k0, ks, wave, lane);
    dma_tile<D, G::KT>(bv, k0, ks + G::KBYTES, wave, lane);
  };

  const TileOffsets<D> toff(lane);
  const int ntiles = tiles.count;
  // With NST stages the copies of tile it + NST - 1 are issued at the start of
  // step it; a step ends once this thread's copies of the next tile have
  // landed (those of the tile after it may stay in flight: vector-memory
  // operations complete in issue order), and the barrier publishes them.
  constexpr int COPIES = 2 * (G::KT * D / 8 / 256);  // K and V copies per thread per tile
  auto land_next = [&](bool younger_in_flight) {
    if (NST > 2 && younger_in_flight)
      __builtin_amdgcn_s_waitcnt(vmcnt_at_most(COPIES));
    else
      wait_all_memory();
  };
  if (ntiles > 0) gload(0, 0);
  if (NST > 2 && ntiles > 1) gload(1, 1);
  land_next(ntiles > 1);
  __syncthreads();

  // one key tile; the LDS stage is a compile-time constant (the loop below
  // runs NST steps per iteration), so it joins the reads' immediate offsets
  auto step = [&](const int it, auto stage) __attribute__((always_inline)) {
    constexpr int cur = decltype(stage)::value;
    constexpr int pre = (cur + NST - 1) % NST;  // stage of tile it + NST - 1
    if (it + NST - 1 < ntiles) gload(it + NST - 1, pre);

    const int k0 = tiles.pos0(it);
    const char* ks = smem + cur * G::STAGE;
    const char* vs = ks + G::KBYTES;
    // the wave's rows [qw0, qw_last] see keys [lo(qw0), hi(qw_last)] between
    // them, and every row sees [lo(qw_last), hi(qw0)]
    const int qw_last = qw0 + WQ - 1;
    const bool active = k0 <= band.hi(qw_last) && k0 + G::KT - 1 >= band.lo(qw0);
    // key halves KB0 .. KB0 + NKB - 1 (32 keys each) of the tile
    auto key_halves = [&](auto kb0_c, auto nkb_c) __attribute__((always_inline)) {
      constexpr int KB0 = decltype(kb0_c)::value, NKB = decltype(nkb_c)::value;
      const int ka = k0 + KB0 * 32, kz = ka + NKB * 32 - 1;  // the halves' keys
      // halves no row of the wave sees add nothing
      if (NKB < 2 && (ka > band.hi(qw_last) || kz < band.lo(qw0))) return;
      // 1. S^T = K Q^T for each (key block kb, query block qb)
      f32x16 s[QB][NKB];
#pragma unroll
      for (int j = 0; j < NKB; ++j) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][j] = f32x16{0};
#pragma unroll
        for (int t = 0; t < G::NKS; ++t) {
          const V8 a = toff.template row_operand<T>(ks, (KB0 + j) * 32, t);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][j] = mfma32(a, qf[qb][t], s[qb][j]);
        }
      }
      if constexpr (QB == 1) sched_reads_ahead<NKB * G::NKS, FA_FWD_AHEAD>();
      // 2. mask keys outside the row's band (future keys, keys outside the
      // window, keys past the end).  Key of register r is k0 + g*4 + C(kb, r),
      // C = kb*32 + (r/4)*8 + r%4; it is hidden iff C < lb or C > ub.
      const bool need_mask = ka < band.lo(qw_last) || kz > band.hi(qw0);
      if (need_mask) {
        FA_KEEP_BRANCH();
        // one compare-and-select per bound on the VALU (an OR of the two
        // compares would route every element through the scalar unit)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int i = qw0 + qb * 32 + l32;
          const int ub = band.hi(i) - k0 - g * 4;
#pragma unroll
          for (int j = 0; j < NKB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int C = (KB0 + j) * 32 + (r >> 2) * 8 + (r & 3);
              s[qb][j][r] = C > ub ? kNegInf : s[qb][j][r];
            }
          if (p.window > 0) {
            const int lb = band.lo(i) - k0 - g * 4;
#pragma unroll
            for (int j = 0; j < NKB; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int C = (KB0 + j) * 32 + (r >> 2) * 8 + (r & 3);
                s[qb][j][r] = C < lb ? kNegInf : s[qb][j][r];
              }
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
        const int kb = KB0 + j;
        // dropout: generator bytes of this half's keys (byte e of kw[qb][rr]
        // decides the key of register rr * 4 + e)
        u32x4 kw[QB];
        if constexpr (DROP) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            kw[qb] = drop_bytes_query_lanes(p.drop, (uint32_t)head, k0 + kb * 32, qw0 + qb * 32,
                                            smem + NST * G::STAGE + wave * kDropLdsPerWave, lane);
        }
        // the weights of 16 keys (step th of the half), their sum (fp16: of
        // the rounded weights that P V uses; bf16: of the float32 weights,
        // bf16 rounding being too coarse for the LSE) added to lp
        u32x4 w[QB][2];
        auto weights = [&](int qb, int th, float& lp) __attribute__((always_inline)) {
          const int r0 = th * 8;
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const float e0 = fast_exp2(__builtin_fmaf(s[qb][j][r0 + 2 * h], p.c, -ref[qb]));
            const float e1 = fast_exp2(__builtin_fmaf(s[qb][j][r0 + 2 * h + 1], p.c, -ref[qb]));
            w[qb][th][h] = pack2<T>(e0, e1);
            if constexpr (__is_same(T, _Float16)) lp = add_pair<T>(w[qb][th][h], lp);
            else lp += e0 + e1;
          }
        };
        // CHK: keys whose weights are checked together (16: each step; 32:
        // the half)
        constexpr int CHK = FA_FWD_CHECK_KEYS;
#pragma unroll
        for (int c = 0; c < 32 / CHK; ++c) {
          const int th0 = c * (CHK / 16), nth = CHK / 16;
          float l_new[QB];
          bool bad = false;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            float lp = 0.f;
            for (int th = th0; th < th0 + nth; ++th) weights(qb, th, lp);
            l_new[qb] = l_run[qb] + lp;
            bad |= !(l_new[qb] < kRowSumLimit);
          }
          if (__builtin_amdgcn_ballot_w64(bad) != 0) {
            FA_KEEP_BRANCH();
            // move each row's reference to the maximum of the row so far
            // (these scores included) and redo the weights
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              float mx = kNegInf;
#pragma unroll
              for (int r = th0 * 8; r < (th0 + nth) * 8; ++r) mx = vmax(mx, s[qb][j][r]);
              const float m_new = vmax(m_ref[qb], pair_max(mx * p.c));
              const float r_new = m_new == kNegInf ? 0.f : m_new;
              const bool had = m_ref[qb] != kNegInf;
              float alpha = fast_exp2(had ? ref[qb] - r_new : kNegInf);  // 0 without a reference
              __asm__ volatile("" : "+v"(alpha));  // one rescale path, not one per case
#pragma unroll
              for (int i = 0; i < G::NDB; ++i) o[qb][i] *= alpha;
              l_run[qb] = had ? l_run[qb] * alpha : (m_new == kNegInf ? kNoRef : 0.f);
              m_ref[qb] = m_new;
              ref[qb] = r_new;
              float lp = 0.f;
              for (int th = th0; th < th0 + nth; ++th) weights(qb, th, lp);
              l_new[qb] = l_run[qb] + lp;
            }
          }
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) l_run[qb] = l_new[qb];
#pragma unroll
          for (int th = th0; th < th0 + nth; ++th) {
            const int t = kb * 2 + th;
            V8 bp[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              // dropout zeroes weights after the row sum: LSE normalises P itself
              if constexpr (DROP) {
#pragma unroll
                for (int h = 0; h < 4; ++h)
                  w[qb][th][h] &= keep_pair_mask(kw[qb][th * 2 + (h >> 1)], h & 1, bias);
              }
              bp[qb] = __builtin_bit_cast(V8, w[qb][th]);
            }
#pragma unroll
            for (int db = 0; db < G::NDB; ++db) {
              const V8 a = toff.template tr_operand<T>(vs, t * 16, db);
#pragma unroll
              for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(a, bp[qb], o[qb][db]);
            }
          }
        }
      }
    };
    if (active) {
      if constexpr (G::KT == 32) {
        key_halves(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
      } else if constexpr (FA_FWD_HALVES) {
        key_halves(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
        key_halves(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
      } else {
        key_halves(std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{});
      }
    }
    land_next(it + 2 < ntiles);  // this thread's copies of tile it + 1 have landed
    __syncthreads();
  };
  for (int it = 0; it < ntiles; it += NST) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < ntiles) step(it + 1, std::integral_constant<int, 1>{});
    if constexpr (NST > 2) {
      if (it + 2 < ntiles) step(it + 2, std::integral_constant<int, 2>{});
    }
  }

  // epilogue: deferred normalisation (and the scale of kept weights under
  // dropout), natural-log LSE
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qw0 + qb * 32 + l32;
    const float lt = pair_sum(m_ref[qb] == kNegInf ? 0.f : l_run[qb]);
    const float inv = lt > 0.f ? (DROP ? p.drop.mult : 1.f) / lt : 0.f;
    if (q < N) {
      T* orow = (T*)p.o + head_off + (size_t)q * D;
#pragma unroll
      for (int db = 0; db < G::NDB; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          u32x2 w;
          w[0] = pack2<T>(o[qb][db][rr * 4 + 0] * inv, o[qb][db][rr * 4 + 1] * inv);
          w[1] = pack2<T>(o[qb][db][rr * 4 + 2] * inv, o[qb][db][rr * 4 + 3] * inv);
          *(u32x2*)(orow + db * 32 + rr * 8 + g * 4) = w;
        }
      if (g == 0)
        p.lse[(size_t)head * N + q] = lt > 0.f ? (m_ref[qb] + fast_log2(lt)) * kLn2 : kNegInf;
    }
  }
}

template <typename T, int D, bool MASKED, bool DROP, int NW, int QB, int WPE, int NST = 2,
          int KT = kKeyTile>
static hipError_t launch_fwd_t(FwdParams p, bool causal, hipStream_t s) {
  constexpr int BR = NW * QB * 32;
  p.nqt = (p.N + BR - 1) / BR;
  dim3 grid(p.nheads * p.nqt), block(NW * 64);
  if (causal)
    hipLaunchKernelGGL((fwd_kernel<T, D, true, MASKED, DROP, NW, QB, WPE, NST, KT>), grid, block, 0,
                       s, p);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, false, MASKED, DROP, NW, QB, WPE, NST, KT>), grid, block, 0,
                       s, p);
  return hipGetLastError();
}

// Workgroup shapes.  A block mask needs the workgroup's rows inside one
// 128-row mask block.  Head dim 128 keeps 32 rows per wave at 2 waves per SIMD
// (register budget: the O accumulator alone is 64 registers); so does dropout
// at head dim 64 (the generator needs registers of its own).
template <typename T>
static hipError_t launch_fwd_dtype(const FwdParams& p, int d, bool causal, bool masked, bool drop,
                                   hipStream_t s) {
  if (drop) {
    if (d == 64)
      return masked ? launch_fwd_t<T, 64, true, true, 4, 1, FA_FWD64_DROP_WPE>(p, causal, s)
                    : launch_fwd_t<T, 64, false, true, 4, 1, FA_FWD64_DROP_WPE>(p, causal, s);
    return masked ? launch_fwd_t<T, 128, true, true, 4, 1, 2>(p, causal, s)
                  : launch_fwd_t<T, 128, false, true, 4, 1, 2>(p, causal, s);
  }
  if (d == 64) {
    if (masked)  // 128-row workgroups; copies two tiles ahead (see FA_FWD64_MASKED_NST)
      return launch_fwd_t<T, 64, true, false, 4, 1, FA_FWD64_MASKED_WPE, FA_FWD64_MASKED_NST>(
          p, causal, s);
    return launch_fwd_t<T, 64, false, false, FA_FWD64_NW, FA_FWD64_QB, FA_FWD64_WPE>(p, causal, s);
  }
  if (masked)
    return launch_fwd_t<T, 128, true, false, 4, 1, FA_FWD128_WPE, 2, FA_FWD128_KT>(p, causal, s);
  return launch_fwd_t<T, 128, false, false, 4, 1, FA_FWD128_WPE, 2, FA_FWD128_KT>(p, causal, s);
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
