// fa_bwd.hip -- backward pass of tiled exact attention on gfx950 matrix cores.
//
// The probabilities are never stored: both kernels rebuild each tile
// P = exp(scale * Q K^T - LSE) from Q, K and the LSE saved by the forward
// ("Passo para tras: recalcular em vez de armazenar", marketmaker.cc article;
// "como funciona", tonho.wtf digest).  With dP = dO V^T and
// D_i = dO_i . O_i (the d-length dot that replaces the N-length reduction
// sum_j P_ij dP_ij, "como funciona", tonho.wtf digest):
//     dS = P o (dP - D),   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO
// (the scale is applied once to the finished dQ and dK).
//
// Two kernels, so that every output is reduced inside one workgroup and
// written once (no atomics, no float32 dQ accumulator in memory, bitwise
// repeatable):
//   bwd_dq_kernel    query-outer (128 query rows per workgroup, 64-key steps,
//                    each run as two 32-key halves): computes D for its rows
//                    first, then per half S^T, dP^T, dS^T and dQ^T += K^T dS^T.
//                    It writes D for the second kernel.
//   bwd_dkdv_kernel  key-outer (128 keys per workgroup, 4 waves x 32 keys;
//                    64-query steps, each run as two 32-query blocks): per
//                    block S, dP, dS with one key per lane, then dV += P^T dO
//                    and dK += dS^T Q.  At head dim 64 the dP accumulators
//                    start at -D (see the kernel).
// The price is computing S and dP in both kernels: 14 d multiply-add FLOPs
// per visible pair instead of 10 d.
//
// The single-pass alternative (FA_BWD_ATOMIC_DQ) does the pages' own loop
// ("Passo para tras: recalcular em vez de armazenar", marketmaker.cc article):
// the key-outer kernel also forms dQ += dS K for its keys and adds it into a
// float32 accumulator in HBM with atomics, so S and dP are computed once
// (10 d FLOPs per pair).  A pre-pass writes D and clears the accumulator, and a
// last pass scales and converts it.  Each step the waves store their dS
// (one key per lane) into a shared 128-key x 64-query LDS tile; after a
// barrier each wave multiplies a 32-query x 32-column block of it by the
// workgroup's K tile (kept in LDS for the whole key tile), so its result is
// the workgroup's complete contribution, and adds it into HBM with one atomic
// add per element once the step's copies have landed (the adds then overlap
// the next step).  dQ depends on the order of the atomic adds (not bitwise
// repeatable); dK and dV are bitwise those of the two-kernel backward.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_dropout.hpp"
#include "fa_kernels.hpp"
#include "fa_tiles.hpp"

namespace fa {

// Waves per SIMD each kernel's register budget targets, measured on MI355X.
// dQ runs the two 32-key halves of a tile one after the other (scores to dQ),
// which keeps it within 124 VGPRs at head dim 64: four waves per SIMD, 3-4 %
// faster than both halves at once at three waves (150 VGPRs).  Likewise dK/dV
// handles the two 32-query blocks of a 64-query step one after the other: at
// head dim 64 it fits the 168 VGPRs of three waves (5 % faster than two), and
// at head dim 128 it runs 10 % faster at the same occupancy; 128-query steps
// (half the barriers) and a three-stage LDS ring measured slower.  At head dim
// 128, dQ under dropout fits two waves (19 % faster than one); dK/dV needs
// about 350 registers (VGPRs and AGPRs) and spills at two waves per SIMD.
constexpr int kDqWpe64 = 4;
constexpr int kDqWpe64DropDense = 4;  // dropout without a block mask: 128 VGPRs, 3.5 % faster than 3
constexpr int kDqWpe64DropMasked = 3; // dropout with a block mask: four waves would spill
constexpr int kDqWpe128 = 2;
constexpr int kDqWpe128Drop = 2;
constexpr int kDkdvWpe64 = 3;
constexpr int kDkdvWpe64Drop = 2;     // dropout's generator registers: three waves would spill
constexpr int kDkdvWpe128 = 1;
constexpr int kDkdvWpe64Adq = 2;      // single pass: K^T fragments and the dQ products
constexpr int kDkdvWpe128Adq = 1;
constexpr int kDkdvQueries = 64;      // queries per dK/dV step (two 32-query blocks)
// LDS operand reads issued ahead of the score products (head dim 64: six of
// the eight, 1-2 % faster than four; 128: four)
constexpr int kDkdvAhead64 = 6;
constexpr int kDkdvAhead128 = 4;
// dQ: LDS operand reads issued ahead of the score and dP products; at head dim
// 128 two ahead measured 2 % faster, at 64 no change (and 16 bytes of spill
// either way)
constexpr int kDqAhead128 = 2;

// ============================================================================
// dQ kernel
// ============================================================================
template <int D>
struct DqGeom {
  static constexpr int KT = kKeyTile;
  static constexpr int KBYTES = KT * D * 2;  // K tile (read by rows and by transpose), swizzled
  static constexpr int VBYTES = KT * D * 2;  // V tile (read by rows), swizzled
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int NDB = D / 32;
  static constexpr int NKS = D / 16;
  // waves per SIMD the registers allow
  static constexpr int wpe(bool drop, bool masked) {
    if (D == 128) return drop ? kDqWpe128Drop : kDqWpe128;
    if (drop) return masked ? kDqWpe64DropMasked : kDqWpe64DropDense;
    return kDqWpe64;
  }
};

template <typename T, int D, bool CAUSAL, bool MASKED, bool DROP, bool PERSIST>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(DqGeom<D>::wpe(DROP, MASKED),
                                              DqGeom<D>::wpe(DROP, MASKED))))
void bwd_dq_kernel(BwdParams p) {
  using G = DqGeom<D>;
  using V8 = typename Vec8<T>::type;
  __shared__ __attribute__((aligned(16))) char smem[2 * G::STAGE + (DROP ? 4 * kDropLdsPerWave : 0)];
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
    const int g = lane >> 5;
    const int l32 = lane & 31;
    const int q0 = qt * kFwdRows;
    const int qw0 = q0 + wave * 32;
    const int q = qw0 + l32;
    const int q_hi = min(q0 + kFwdRows, N) - 1;

    const size_t head_off = (size_t)head * N * D;
    const size_t kv_off = (size_t)(head / p.group) * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * sizeof(T);
    const Buf bq = make_buf((const T*)p.q + head_off, head_bytes);
    const Buf bk = make_buf((const T*)p.k + kv_off, head_bytes);
    const Buf bv = make_buf((const T*)p.v + kv_off, head_bytes);
    const Buf bo = make_buf((const T*)p.o + head_off, head_bytes);
    const Buf bdo = make_buf((const T*)p.dout + head_off, head_bytes);

    const Band band{N, p.window, CAUSAL};
    const auto tiles = key_tiles<G::KT, MASKED>(p.m, band, q0, q_hi);

    // Q and dO fragments (B operands, k = head dim); D_i = dO_i . O_i
    V8 qf[G::NKS], dof[G::NKS];
    float dpart = 0.f;
#pragma unroll
    for (int t = 0; t < G::NKS; ++t) {
      const uint32_t off = (uint32_t)(q * D + t * 16 + g * 8) * sizeof(T);
      qf[t] = __builtin_bit_cast(V8, buf_load16(bq, off));
      dof[t] = __builtin_bit_cast(V8, buf_load16(bdo, off));
      const V8 of = __builtin_bit_cast(V8, buf_load16(bo, off));
#pragma unroll
      for (int i = 0; i < 8; ++i) dpart += to_f32(dof[t][i]) * to_f32(of[i]);
    }
    const float dq_d = pair_sum(dpart);
    // Under dropout dS = mult * P o (keep o dP' - D / mult), dP' = dO V^T: the
    // mask selects dP', and mult joins the scale of the finished dQ.
    const float d_sub = DROP ? dq_d / p.drop.mult : dq_d;
    float lse2 = __builtin_huge_valf();  // rows past the end or with no visible key: P = 0
    if (q < N) {
      const float lse = p.lse[(size_t)head * N + q];
      if (lse != kNegInf) lse2 = lse * kLog2e;
      if (g == 0) p.dvec[(size_t)head * N + q] = dq_d;
    }

    f32x16 acc[G::NDB];
#pragma unroll
    for (int i = 0; i < G::NDB; ++i) acc[i] = f32x16{0};

    // K and V tiles go straight from global memory to LDS
    const int nb128 = (N + 127) / 128;
    auto gload = [&](int it, int stage) {
      const int k0 = tiles.pos0(it);
      // debug build: counters of the dQ kernel follow the forward's
      debug_visit(p.visits, ((size_t)(p.nheads + head) * p.ntiles + qt) * nb128 + k0 / 128, G::KT);
      char* ks = smem + stage * G::STAGE;
      dma_tile<D, G::KT>(bk, k0, ks, wave, lane);
      dma_tile<D, G::KT>(bv, k0, ks + G::KBYTES, wave, lane);
    };

    const int ntiles = tiles.count;
    if (ntiles > 0) gload(0, 0);
    wait_all_memory();
    __syncthreads();

    const TileOffsets<D> toff(lane);
    // The copies of tile it + 1 are issued at the start of step it, and a step
    // ends once this thread's copies have landed.  One key tile per step; the
    // LDS stage is a compile-time constant (two steps per iteration of the loop
    // below), so it joins the reads' immediate offsets.
    auto step = [&](const int it, auto stage) __attribute__((always_inline)) {
      constexpr int cur = decltype(stage)::value;
      if (it + 1 < ntiles) gload(it + 1, 1 - cur);

      const int k0 = tiles.pos0(it);
      const char* ks = smem + cur * G::STAGE;
      const char* vs = ks + G::KBYTES;
      const int qw_last = qw0 + 31;
      const bool active = k0 <= band.hi(qw_last) && k0 + G::KT - 1 >= band.lo(qw0);
      // key halves KB0 .. KB0 + NKB - 1 of the tile: scores, dP, dS, then dQ
      auto halves = [&](auto kb0_c, auto nkb_c) __attribute__((always_inline)) {
        constexpr int KB0 = decltype(kb0_c)::value, NKB = decltype(nkb_c)::value;
        static_assert(NKB == 1, "one 32-key half at a time");
        // a half no row of the wave sees adds nothing (the later half of a
        // causal diagonal tile)
        if (k0 + KB0 * 32 > band.hi(qw_last) || k0 + KB0 * 32 + 31 < band.lo(qw0)) return;
        f32x16 s[NKB], dp[NKB];
#pragma unroll
        for (int i = 0; i < NKB; ++i) {
          s[i] = f32x16{0};
          dp[i] = f32x16{0};
#pragma unroll
          for (int t = 0; t < G::NKS; ++t) {
            const V8 a = toff.template row_operand<T>(ks, (KB0 + i) * 32, t);
            s[i] = mfma32(a, qf[t], s[i]);
            const V8 b = toff.template row_operand<T>(vs, (KB0 + i) * 32, t);
            dp[i] = mfma32(b, dof[t], dp[i]);
          }
        }
        sched_reads_ahead<2 * NKB * G::NKS, D == 128 ? kDqAhead128 : 0>();
        // hide keys outside the row's band (future, outside the window, past
        // the end): key of register r is k0 + g*4 + C(kb, r) with
        // C = kb*32 + (r/4)*8 + r%4; hidden iff C < lb or C > ub
        // one compare-and-select per bound, each only where some row needs it
        // (an OR of the two compares would route every element through the
        // scalar unit)
        if (k0 + KB0 * 32 + NKB * 32 - 1 > band.hi(qw0)) {
          const int ub = band.hi(q) - k0 - g * 4;
#pragma unroll
          for (int i = 0; i < NKB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int C = (KB0 + i) * 32 + (r >> 2) * 8 + (r & 3);
              s[i][r] = C > ub ? kNegInf : s[i][r];
            }
        }
        if (k0 + KB0 * 32 < band.lo(qw_last)) {
          const int lb = band.lo(q) - k0 - g * 4;
#pragma unroll
          for (int i = 0; i < NKB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int C = (KB0 + i) * 32 + (r >> 2) * 8 + (r & 3);
              s[i][r] = C < lb ? kNegInf : s[i][r];
            }
        }
#pragma unroll
        for (int i = 0; i < NKB; ++i) {
          u32x4 kw;
          if constexpr (DROP)
            kw = drop_bytes_query_lanes(p.drop, (uint32_t)head, k0 + (KB0 + i) * 32, qw0,
                                        smem + 2 * G::STAGE + wave * kDropLdsPerWave, lane);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pr = fast_exp2(__builtin_fmaf(s[i][r], p.c, -lse2));
            float dpr = dp[i][r];
            if constexpr (DROP) dpr = keep_byte(kw[r >> 2], r & 3, p.drop.t8) ? dpr : 0.f;
            s[i][r] = pr * (dpr - d_sub);  // dS^T (scale applied to dQ at the end)
          }
        }
        // dQ^T += K^T dS^T : A = K^T via transpose reads of the K tile
        V8 bs[2 * NKB];
#pragma unroll
        for (int t = 0; t < 2 * NKB; ++t) {
          const int i = t >> 1, r0 = (t & 1) * 8;
          bs[t] = pack8<T>(s[i][r0 + 0], s[i][r0 + 1], s[i][r0 + 2], s[i][r0 + 3],
                           s[i][r0 + 4], s[i][r0 + 5], s[i][r0 + 6], s[i][r0 + 7]);
        }
#pragma unroll
        for (int db = 0; db < G::NDB; ++db)
#pragma unroll
          for (int t = 0; t < 2 * NKB; ++t) {
            const V8 a = toff.template tr_operand<T>(ks, (2 * KB0 + t) * 16, db);
            acc[db] = mfma32(a, bs[t], acc[db]);
          }
      };
      if (active) {
        halves(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
        halves(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
      }
      wait_all_memory();  // this thread's copies of tile it + 1 have landed
      __syncthreads();
    };
    for (int it = 0; it < ntiles; it += 2) {
      step(it, std::integral_constant<int, 0>{});
      if (it + 1 < ntiles) step(it + 1, std::integral_constant<int, 1>{});
    }

    if (q < N) {
      T* row = (T*)p.dq + head_off + (size_t)q * D;
      const float f = DROP ? p.scale * p.drop.mult : p.scale;
#pragma unroll
      for (int db = 0; db < G::NDB; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          u32x2 w;
          w[0] = pack2<T>(acc[db][rr * 4 + 0] * f, acc[db][rr * 4 + 1] * f);
          w[1] = pack2<T>(acc[db][rr * 4 + 2] * f, acc[db][rr * 4 + 3] * f);
          *(u32x2*)(row + db * 32 + rr * 8 + g * 4) = w;
        }
    }
  };

  if constexpr (PERSIST) {
    // causal work units: the tile pair (ntiles - 1 - u, u) of a head, the
    // longer rows first; every unit costs about the same
    const int units = (p.ntiles + 1) / 2, total = p.nheads * units;
    for (int b = blockIdx.x; b < total; b += gridDim.x) {
      const int logical = xcd_remap(b, total);
      const int head = logical / units, u = logical % units;
      const int nsub = 2 * u + 1 != p.ntiles ? 2 : 1;
      for (int e = 0; e < nsub; ++e) tile(head, e == 0 ? p.ntiles - 1 - u : u);
    }
  } else {
    // causal: the longer rows first (one call of the tile body, so that it is
    // inlined once)
    int head, qt;
    if (CAUSAL && p.spread > 0) {
      spread_tile(blockIdx.x, p.nheads, p.ntiles, p.spread, head, qt);
    } else {
      const int logical = xcd_remap(blockIdx.x, gridDim.x);
      head = logical / p.ntiles;
      qt = logical % p.ntiles;
    }
    tile(head, CAUSAL ? p.ntiles - 1 - qt : qt);
  }
}

// ============================================================================
// dK / dV kernel
// ============================================================================
template <int D>
struct DkvGeom {
  static constexpr int QT = kDkdvQueries;   // queries per step
  static constexpr int TBYTES = QT * D * 2;  // Q / dO tile, swizzled (no padding)
  static constexpr int LBYTES = 256;         // LSE (or D) of the step's rows, one dword per lane
  static constexpr int STAGE = 2 * TBYTES + 2 * LBYTES;  // Q, dO, LSE, D
  static_assert(QT == 64, "one 64-lane copy of LSE and D per step; two 32-query blocks");
  static constexpr int NDB = D / 32;
  static constexpr int NKS = D / 16;
  static constexpr int NQB = QT / 32;       // 32-query blocks per step
  // single pass: the workgroup's K tile and the step's dS^T (kBwdKeys x QT,
  // 16-bit), both swizzled tiles
  static constexpr int KTBYTES = kBwdKeys * D * 2;
  static constexpr int DSBYTES = kBwdKeys * QT * 2;
  // waves per SIMD the registers allow
  static constexpr int wpe(bool drop, bool adq) {
    if (adq) return D == 64 ? kDkdvWpe64Adq : kDkdvWpe128Adq;
    return D == 64 ? (drop ? kDkdvWpe64Drop : kDkdvWpe64) : kDkdvWpe128;
  }
};

template <typename T, int D, bool CAUSAL, bool MASKED, bool DROP, bool PERSIST, bool ADQ>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(DkvGeom<D>::wpe(DROP, ADQ), DkvGeom<D>::wpe(DROP, ADQ))))
void bwd_dkdv_kernel(BwdParams p) {
  using G = DkvGeom<D>;
  using V8 = typename Vec8<T>::type;
  // At head dim 64 without dropout the dP accumulators start at -D (an
  // exact float32 value), so dS = P o dp is one instruction.  The scale is
  // not folded into K: K c rounded to the input type moves every score by up
  // to |S c| 2^-11, which for large logits (|S c| ~ 100) breaks the
  // gradients' tolerance.
  constexpr bool kFoldD = D == 64 && !DROP;
  constexpr int kDropBytes = DROP ? 4 * kDropLdsPerWave : 0;
  __shared__ __attribute__((aligned(16))) char
      smem[2 * G::STAGE + kDropBytes + (ADQ ? G::KTBYTES + G::DSBYTES : 0)];
  debug_fill_lds_nan(smem, sizeof(smem));

  const int lane_ = threadIdx.x & 63;
  const int wave = wave_id();
  const int N = p.N;

  // single pass: the K tile and the dS^T tile
  char* const ktile = smem + 2 * G::STAGE + kDropBytes;
  char* const dstile = ktile + G::KTBYTES;

  // one key tile of one K/V head
  auto tile = [&](const int kvh, const int kt) __attribute__((always_inline)) {
    int lane = lane_;
    // in the persistent loop, lane-only values are recomputed per tile rather
    // than kept live across it (registers)
    if constexpr (PERSIST) __asm__ volatile("" : "+v"(lane));
    const int g = lane >> 5;
    const int l32 = lane & 31;
    const int k0 = kt * kBwdKeys;
    const int kw0 = k0 + wave * 32;
    const int key = kw0 + l32;          // this lane's key

    const size_t kv_off = (size_t)kvh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * sizeof(T);
    const Buf bk = make_buf((const T*)p.k + kv_off, head_bytes);
    const Buf bv = make_buf((const T*)p.v + kv_off, head_bytes);

    // The same query tiles are visited for each of the `group` query heads that
    // read this K/V head; iteration it covers head it / nqt, tile it % nqt, and
    // dK, dV sum over all of them in registers.
    const Band band{N, p.window, CAUSAL};
    const auto tiles = query_tiles<G::QT, MASKED>(p.m, band, k0, k0 + kBwdKeys - 1);
    const int nqt = tiles.count;

    // K and V fragments: B operands of S = Q K^T and dP = dO V^T (k = head dim)
    V8 kf[G::NKS], vf[G::NKS];
#pragma unroll
    for (int t = 0; t < G::NKS; ++t) {
      const uint32_t off = (uint32_t)(key * D + t * 16 + g * 8) * sizeof(T);
      kf[t] = __builtin_bit_cast(V8, buf_load16(bk, off));
      vf[t] = __builtin_bit_cast(V8, buf_load16(bv, off));
    }
    // Wait for these here: the copies below are invisible to the compiler's
    // own wait counting, which would otherwise wait inside the loop for loads
    // it still thinks pending -- and, counts being in issue order, for the
    // prefetch copies issued after them.
    wait_all_memory();
    f32x16 dka[G::NDB], dva[G::NDB];
#pragma unroll
    for (int i = 0; i < G::NDB; ++i) {
      dka[i] = f32x16{0};
      dva[i] = f32x16{0};
    }

    // Q, dO, LSE and D of a step go straight from global memory to LDS (no
    // registers, no store instructions): Q and dO by all waves, LSE and D by
    // wave 0, one row per lane (lanes past QT and rows past N read as zeros;
    // such rows are hidden by the masks).  The copies of step it + 1 are issued
    // at the start of step it.
    const int nb128 = (N + 127) / 128;
    auto gload = [&](int it, char* st) {
      const int r = it / nqt;
      const int qs = tiles.pos0(it - r * nqt);
      const size_t qh = (size_t)kvh * p.group + r;  // query head
      // debug build: counters of the dK/dV kernel follow those of the forward
      // and the dQ kernel (B*H_kv*group = B*H query heads each)
      debug_visit(p.visits, ((size_t)(2 * p.nheads * p.group + qh) * p.ntiles + kt) * nb128 + qs / 128, G::QT);
      const Buf bq = make_buf((const T*)p.q + qh * N * D, head_bytes);
      const Buf bdo = make_buf((const T*)p.dout + qh * N * D, head_bytes);
      dma_tile<D, G::QT>(bq, qs, st, wave, lane);
      dma_tile<D, G::QT>(bdo, qs, st + G::TBYTES, wave, lane);
      if (wave == 0) {
        const Buf bl = make_buf(p.lse + qh * N, (uint32_t)N * 4);
        const Buf bd = make_buf(p.dvec + qh * N, (uint32_t)N * 4);
        const uint32_t off = (uint32_t)(qs + lane) * 4;
        dma4(bl, off, st + 2 * G::TBYTES);
        dma4(bd, off, st + 2 * G::TBYTES + G::LBYTES);
      }
    };
    // Wait until this wave's copies of the next step have landed, then wave 0
    // converts that step's rows
    // in place: LSE -> LSE log2(e) (+inf for a row with no visible key, so P =
    // 0), D -> D / mult under dropout (see the dS step), D -> -D where the dP
    // accumulators start from it.  The barrier that follows publishes the stage.
    auto land_next = [&](char* st) {
      wait_all_memory();
      if (wave == 0) {
        float* ls = (float*)(st + 2 * G::TBYTES);
        float* ds = (float*)(st + 2 * G::TBYTES + G::LBYTES);
#pragma unroll
        for (int i = lane; i < G::QT; i += 64) {
          const float l = ls[i];
          ls[i] = l != kNegInf ? l * kLog2e : __builtin_huge_valf();
          if constexpr (DROP) ds[i] = ds[i] / p.drop.mult;
          if constexpr (kFoldD) ds[i] = -ds[i];  // dP accumulators start here
        }
      }
    };

    const int ntiles = nqt * p.group;
    if (ntiles > 0) gload(0, smem);
    // single pass: the workgroup's K tile, for the whole key tile
    if constexpr (ADQ) dma_tile<D, kBwdKeys>(bk, k0, ktile, wave, lane);
    land_next(smem);
    __syncthreads();

    const TileOffsets<D> toff(lane);
    // single pass: transpose-read offsets of the dS^T tile (64 columns), and
    // zeros for the rows of a 32-query block that this wave skips
    const TileOffsets<64> tds(lane);
    auto ds_zero = [&](const int qb) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < 32; c += 8)
        *(u32x2*)(dstile + swz_off<64>(wave * 32 + l32, qb * 32 + c + 4 * g)) = u32x2{0u, 0u};
    };
    // one query step; its LDS stage (it mod 2) is a compile-time constant (two
    // steps per iteration of the loop below), so stage addresses join the
    // reads' immediate offsets
    auto step = [&](const int it, auto stage) __attribute__((always_inline)) {
      constexpr int cur = decltype(stage)::value;
      constexpr int nxt = 1 - cur;  // stage of step it + 1
      if (it + 1 < ntiles) gload(it + 1, smem + nxt * G::STAGE);

      const int qs0 = tiles.pos0(it % nqt);
      const int qh = kvh * p.group + it / nqt;  // query head of this step
      const char* qsm = smem + cur * G::STAGE;
      const char* dsm = qsm + G::TBYTES;
      const float* lsm = (const float*)(dsm + G::TBYTES);
      // the wave's keys [kw0, kw_last] are seen by queries [qlo(kw0), qhi(kw_last)]
      // between them, and by all of them in [qlo(kw_last), qhi(kw0)]
      const int kw_last = kw0 + 31;
      const bool active = qs0 <= band.qhi(kw_last) && qs0 + G::QT - 1 >= band.qlo(kw0);
      // 32-query blocks QB0 .. QB0 + NQ - 1 of the step: scores, dP, softmax,
      // dS, then their dV and dK products
      auto qblocks = [&](auto qb0_c, auto nq_c) __attribute__((always_inline)) {
        constexpr int QB0 = decltype(qb0_c)::value, NQ = decltype(nq_c)::value;
        const int qa = qs0 + QB0 * 32, qz = qa + NQ * 32 - 1;  // the blocks' queries
        // blocks that see none of the wave's keys add nothing (single pass:
        // their dS^T rows are zeros)
        if (NQ < G::NQB && (qa > band.qhi(kw_last) || qz < band.qlo(kw0))) {
          if constexpr (ADQ) ds_zero(QB0);
          return;
        }
        f32x16 s[NQ], dp[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          s[i] = f32x16{0};
          if constexpr (kFoldD) {
            // register r of a block holds query row 8 (r / 4) + 4 g + r % 4
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const f32x4 d4 = *(const f32x4*)(lsm + G::LBYTES / 4 + (QB0 + i) * 32 + rr * 8 + g * 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) dp[i][rr * 4 + e] = d4[e];
            }
          } else {
            dp[i] = f32x16{0};
          }
#pragma unroll
          for (int t = 0; t < G::NKS; ++t) {
            const V8 a = toff.template row_operand<T>(qsm, (QB0 + i) * 32, t);
            s[i] = mfma32(a, kf[t], s[i]);
            const V8 b = toff.template row_operand<T>(dsm, (QB0 + i) * 32, t);
            dp[i] = mfma32(b, vf[t], dp[i]);
          }
        }
        sched_reads_ahead<2 * NQ * G::NKS, D == 64 ? kDkdvAhead64 : kDkdvAhead128>();
        // hide queries outside this lane's key band (before the key under
        // causal, outside the window, past the end).  Query of register r in
        // block qb is qs0 + g*4 + C(qb, r), C = qb*32 + (r/4)*8 + r%4; hidden
        // iff C < lb or C > ub
        if (qa < band.qlo(kw_last)) {
          const int lb = band.qlo(key) - qs0 - g * 4;
#pragma unroll
          for (int i = 0; i < NQ; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int C = (QB0 + i) * 32 + (r >> 2) * 8 + (r & 3);
              s[i][r] = C < lb ? kNegInf : s[i][r];
            }
        }
        if (qz > band.qhi(kw0)) {
          const int ub = band.qhi(key) - qs0 - g * 4;
#pragma unroll
          for (int i = 0; i < NQ; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int C = (QB0 + i) * 32 + (r >> 2) * 8 + (r & 3);
              s[i][r] = C > ub ? kNegInf : s[i][r];
            }
        }
        // Under dropout (keep mask Z01, scale mult): dV = mult (Z01 o P)^T dO and
        // dS = mult * P o (Z01 o dP' - D / mult); both mult factors join the
        // finished dV and dK, and the D loaded with the tile is already / mult.
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const int qb = QB0 + i;
          u32x4 kw;
          if constexpr (DROP)
            kw = drop_bytes_key_lanes(p.drop, (uint32_t)qh, kw0, qs0 + qb * 32,
                                      smem + 2 * G::STAGE + wave * kDropLdsPerWave, lane);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const f32x4 l4 = *(const f32x4*)(lsm + qb * 32 + rr * 8 + g * 4);
            f32x4 d4 = {0.f, 0.f, 0.f, 0.f};
            if (!kFoldD) d4 = *(const f32x4*)(lsm + G::LBYTES / 4 + qb * 32 + rr * 8 + g * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = rr * 4 + e;
              const float pr = fast_exp2(__builtin_fmaf(s[i][r], p.c, -l4[e]));
              if constexpr (DROP) {
                const bool keep = keep_byte(kw[rr], e, p.drop.t8);
                s[i][r] = keep ? pr : 0.f;                             // Z01 o P
                dp[i][r] = pr * ((keep ? dp[i][r] : 0.f) - d4[e]);  // dS / mult
              } else {
                s[i][r] = pr;  // P
                // dS (scale applied to dK at the end); dp may already hold dP - D
                dp[i][r] = kFoldD ? pr * dp[i][r] : pr * (dp[i][r] - d4[e]);
              }
            }
          }
        }
        // dV += P^T dO,  dK += dS^T Q ; k-step t covers queries 16t .. 16t+15
#pragma unroll
        for (int t = 0; t < 2 * NQ; ++t) {
          const int i = t >> 1, r0 = (t & 1) * 8;
          const V8 ap = pack8<T>(s[i][r0 + 0], s[i][r0 + 1], s[i][r0 + 2], s[i][r0 + 3],
                                 s[i][r0 + 4], s[i][r0 + 5], s[i][r0 + 6], s[i][r0 + 7]);
          const V8 ad = pack8<T>(dp[i][r0 + 0], dp[i][r0 + 1], dp[i][r0 + 2], dp[i][r0 + 3],
                                 dp[i][r0 + 4], dp[i][r0 + 5], dp[i][r0 + 6], dp[i][r0 + 7]);
#pragma unroll
          for (int db = 0; db < G::NDB; ++db) {
            const V8 bdo_ = toff.template tr_operand<T>(dsm, (2 * QB0 + t) * 16, db);
            dva[db] = mfma32(ap, bdo_, dva[db]);
            const V8 bq_ = toff.template tr_operand<T>(qsm, (2 * QB0 + t) * 16, db);
            dka[db] = mfma32(ad, bq_, dka[db]);
          }
          if constexpr (ADQ) {
            // dS^T row of this lane's key: words 0-1 of ad hold the block's
            // queries 16 (t % 2) + 4 g + 0..3, words 2-3 the same + 8
            const u32x4 w = __builtin_bit_cast(u32x4, ad);
            const int col = (QB0 + i) * 32 + 16 * (t & 1) + 4 * g;
            *(u32x2*)(dstile + swz_off<64>(wave * 32 + l32, col)) = u32x2{w[0], w[1]};
            *(u32x2*)(dstile + swz_off<64>(wave * 32 + l32, col + 8)) = u32x2{w[2], w[3]};
          }
        }
      };
      if (active) {
        qblocks(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
        qblocks(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
      } else if constexpr (ADQ) {
        ds_zero(0);
        ds_zero(1);
      }
      if constexpr (ADQ) {
        // dQ of the step's queries: wave w takes query block w / 2 and column
        // block(s) of w % 2; dS (k = the workgroup's 128 keys) times the K tile,
        // both read by transposes (k index: rows 4 g + 0..3 and + 8 of each
        // 16-row group, as TileOffsets lays out its transpose operands)
        __syncthreads();  // every wave's dS^T is in the tile
        const int qb = wave >> 1;
        f32x16 dqa[G::NDB / 2];
#pragma unroll
        for (int j = 0; j < G::NDB / 2; ++j) {
          const int db = (wave & 1) * (G::NDB / 2) + j;
          dqa[j] = f32x16{0};
#pragma unroll
          for (int kk = 0; kk < kBwdKeys / 16; ++kk)
            dqa[j] = mfma32(tds.template tr_operand<T>(dstile, kk * 16, qb),
                            toff.template tr_operand<T>(ktile, kk * 16, db), dqa[j]);
        }
        if (it + 1 < ntiles) land_next(smem + nxt * G::STAGE);
        // the atomic adds go out after this step's wait, so the next step's
        // computation overlaps them; register r is query qb*32 + 8 (r/4) + 4 g + r%4
        float* dst = p.dqacc + ((size_t)qh * N + qs0 + qb * 32) * D + l32;
#pragma unroll
        for (int j = 0; j < G::NDB / 2; ++j) {
          const int db = (wave & 1) * (G::NDB / 2) + j;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = (r >> 2) * 8 + g * 4 + (r & 3);
            if (dqa[j][r] != 0.f && qs0 + qb * 32 + row < N)
              unsafeAtomicAdd(dst + row * D + db * 32, dqa[j][r]);
          }
        }
      } else {
        if (it + 1 < ntiles) land_next(smem + nxt * G::STAGE);
      }
      __syncthreads();
    };
    for (int it = 0; it < ntiles; it += 2) {
      step(it, std::integral_constant<int, 0>{});
      if (it + 1 < ntiles) step(it + 1, std::integral_constant<int, 1>{});
    }

    // C layout: lane -> head-dim column, register -> key row.  Each wave turns
    // its 32 x D blocks of dK and dV into row-major order in LDS (the stages
    // are free once every wave has left the loop), then stores 16-byte pieces
    // of whole rows.
    static_assert(4 * 2 * 32 * D * (int)sizeof(T) <= 2 * G::STAGE, "epilogue fits the stages");
    const float fk = DROP ? p.scale * p.drop.mult : p.scale;
    const float fv = DROP ? p.drop.mult : 1.f;
    __syncthreads();
    T* ek = (T*)(smem + wave * 2 * 32 * D * sizeof(T));
    T* ev = ek + 32 * D;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (r >> 2) * 8 + g * 4 + (r & 3);
        ek[row * D + db * 32 + l32] = (T)(dka[db][r] * fk);
        ev[row * D + db * 32 + l32] = (T)(dva[db][r] * fv);
      }
    __syncthreads();
    constexpr int CPR = D / 8;  // 16-byte pieces per row
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
      const int c = i * 64 + lane, row = c / CPR, piece = c % CPR;
      if (kw0 + row < N) {
        const size_t idx = kv_off + (size_t)(kw0 + row) * D + piece * 8;
        *(u32x4*)((T*)p.dk + idx) = *(const u32x4*)(ek + row * D + piece * 8);
        *(u32x4*)((T*)p.dv + idx) = *(const u32x4*)(ev + row * D + piece * 8);
      }
    }
    // the next tile's copies overwrite the LDS this epilogue reads
    if constexpr (PERSIST) __syncthreads();
  };

  if constexpr (PERSIST) {
    // causal work units: the tile pair (u, ntiles - 1 - u) of a K/V head, the
    // longer columns first; every unit costs about the same
    const int units = (p.ntiles + 1) / 2, total = p.nheads * units;
    for (int b = blockIdx.x; b < total; b += gridDim.x) {
      const int logical = xcd_remap(b, total);
      const int kvh = logical / units, u = logical % units;
      const int nsub = 2 * u + 1 != p.ntiles ? 2 : 1;
      for (int e = 0; e < nsub; ++e) tile(kvh, e == 0 ? u : p.ntiles - 1 - u);
    }
  } else {
    // in order: under causal masking the longer columns first (key tile 0
    // sees every query); one call of the tile body, so that it is inlined once
    int kvh, kt;
    if (CAUSAL && p.spread > 0) {
      spread_tile(blockIdx.x, p.nheads, p.ntiles, p.spread, kvh, kt);
    } else {
      const int logical = xcd_remap(blockIdx.x, gridDim.x);
      kvh = logical / p.ntiles;
      kt = logical % p.ntiles;
    }
    tile(kvh, kt);
  }
}

template <typename T, int D, bool DROP>
static hipError_t launch_dq_t(const BwdParams& p_in, bool causal, bool masked, hipStream_t s) {
  BwdParams p = p_in;
  p.spread = 0;
  const int units = p.nheads * p.ntiles;
  // causal work without a window or block mask: one workgroup per tile in the
  // spread order when all tiles fit on the GPU at once, else a persistent grid
  // over tile pairs (not under dropout at head dim 64: the unit loop's
  // registers would spill); the rest one workgroup per tile
  if (causal && !masked && p.window == 0) {
    constexpr auto kTile = bwd_dq_kernel<T, D, true, false, DROP, false>;
    p.spread = spread_for<kTile>(p.nheads, p.ntiles);
    if (p.spread > 0) {
      launch_units<kTile>(p, units, false, s);
      return hipGetLastError();
    }
    if constexpr (!(DROP && D == 64)) {
      launch_units<bwd_dq_kernel<T, D, true, false, DROP, true>>(p, p.nheads * ((p.ntiles + 1) / 2), true, s);
      return hipGetLastError();
    }
  }
  if (causal && masked)
    launch_units<bwd_dq_kernel<T, D, true, true, DROP, false>>(p, units, false, s);
  else if (causal)
    launch_units<bwd_dq_kernel<T, D, true, false, DROP, false>>(p, units, false, s);
  else if (masked)
    launch_units<bwd_dq_kernel<T, D, false, true, DROP, false>>(p, units, false, s);
  else
    launch_units<bwd_dq_kernel<T, D, false, false, DROP, false>>(p, units, false, s);
  return hipGetLastError();
}

template <typename T, int D, bool DROP, bool ADQ = false>
static hipError_t launch_dkdv_t(const BwdParams& p_in, bool causal, bool masked, hipStream_t s) {
  BwdParams p = p_in;
  p.spread = 0;
  const int units = p.nheads * p.ntiles;
  // causal work without a window or block mask: one workgroup per tile in the
  // spread order when all tiles fit on the GPU at once, else a persistent grid
  // over tile pairs at head dim 64 (at 128, one wave per SIMD, one workgroup
  // per tile measured faster); the rest one workgroup per tile
  if (causal && !masked && p.window == 0) {
    constexpr auto kTile = bwd_dkdv_kernel<T, D, true, false, DROP, false, ADQ>;
    p.spread = spread_for<kTile>(p.nheads, p.ntiles);
    if (p.spread > 0) {
      launch_units<kTile>(p, units, false, s);
      return hipGetLastError();
    }
    if constexpr (D == 64) {
      launch_units<bwd_dkdv_kernel<T, D, true, false, DROP, true, ADQ>>(p, p.nheads * ((p.ntiles + 1) / 2), true, s);
      return hipGetLastError();
    }
  }
  if (causal && masked)
    launch_units<bwd_dkdv_kernel<T, D, true, true, DROP, false, ADQ>>(p, units, false, s);
  else if (causal)
    launch_units<bwd_dkdv_kernel<T, D, true, false, DROP, false, ADQ>>(p, units, false, s);
  else if (masked)
    launch_units<bwd_dkdv_kernel<T, D, false, true, DROP, false, ADQ>>(p, units, false, s);
  else
    launch_units<bwd_dkdv_kernel<T, D, false, false, DROP, false, ADQ>>(p, units, false, s);
  return hipGetLastError();
}

// ============================================================================
// Single-pass backward: pre-pass and conversion
// ============================================================================
// D_i = dO_i . O_i for every query row, and the row's float32 dQ accumulator
// cleared.  D / 8 threads per row, 8 elements each; rows = query heads x N.
// The sum runs in the dQ kernel's order (two chains of multiply-adds, over
// elements 16 t + 8 h + i for h = 0 and h = 1, then their sum), so D, and
// with it dK and dV, are bitwise those of the two-kernel backward.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p, size_t rows) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  const int part = threadIdx.x % TPR;
  const int base = (threadIdx.x & 63) - part;  // lane of part 0 of this row
  for (size_t row0 = (size_t)blockIdx.x * RPB; row0 < rows; row0 += (size_t)gridDim.x * RPB) {
    const size_t row = row0 + threadIdx.x / TPR;
    float x[8], y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = y[i] = 0.f;
    if (row < rows) {
      const size_t e = row * D + part * 8;
      const typename Vec8<T>::type ov = __builtin_bit_cast(typename Vec8<T>::type, *(const u32x4*)((const T*)p.o + e));
      const typename Vec8<T>::type gv = __builtin_bit_cast(typename Vec8<T>::type, *(const u32x4*)((const T*)p.dout + e));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[i] = to_f32(gv[i]);
        y[i] = to_f32(ov[i]);
      }
      *(f32x4*)(p.dqacc + e) = f32x4{0.f, 0.f, 0.f, 0.f};
      *(f32x4*)(p.dqacc + e + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // chain h = part % 2 passes through parts h, h + 2, h + 4, ...
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < TPR / 2; ++t) {
      float a = acc;
#pragma unroll
      for (int i = 0; i < 8; ++i) a += x[i] * y[i];
      acc = __shfl(a, base + 2 * t + (part & 1), 64);
    }
    const float lo = __shfl(acc, base, 64), hi = __shfl(acc, base + 1, 64);
    if (row < rows && part == 0) p.dvec[row] = lo + hi;
  }
}

// dq = f * accumulator, rounded to T; n8 groups of 8 elements.
template <typename T>
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* acc, T* dq, size_t n8, float f) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
    const f32x4 a = *(const f32x4*)(acc + 8 * i);
    const f32x4 b = *(const f32x4*)(acc + 8 * i + 4);
    u32x4 w;
    w[0] = pack2<T>(a[0] * f, a[1] * f);
    w[1] = pack2<T>(a[2] * f, a[3] * f);
    w[2] = pack2<T>(b[0] * f, b[1] * f);
    w[3] = pack2<T>(b[2] * f, b[3] * f);
    *(u32x4*)(dq + 8 * i) = w;
  }
}

template <typename T, int D, bool DROP>
static hipError_t single_pass_t(const BwdParams& p, bool causal, bool masked, hipStream_t s) {
  const size_t rows = (size_t)p.nheads * p.group * p.N;  // query rows
  constexpr int RPB = 256 / (D / 8);
  const unsigned pgrid = (unsigned)min((rows + RPB - 1) / RPB, (size_t)65536);
  hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3(pgrid), dim3(256), 0, s, p, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_dkdv_t<T, D, DROP, true>(p, causal, masked, s);
  if (e != hipSuccess) return e;
  const size_t n8 = rows * D / 8;
  const unsigned grid = (unsigned)min((n8 + 255) / 256, (size_t)65536);
  hipLaunchKernelGGL((dq_convert_kernel<T>), dim3(grid), dim3(256), 0, s, p.dqacc, (T*)p.dq, n8,
                     DROP ? p.scale * p.drop.mult : p.scale);
  return hipGetLastError();
}

hipError_t launch_bwd_single_pass(const BwdParams& p, int dtype, int d, bool causal, bool masked,
                                  hipStream_t s) {
  const bool drop = p.drop.t8 != 0;
  if (dtype == 1) {
    if (d == 64)
      return drop ? single_pass_t<_Float16, 64, true>(p, causal, masked, s)
                  : single_pass_t<_Float16, 64, false>(p, causal, masked, s);
    return drop ? single_pass_t<_Float16, 128, true>(p, causal, masked, s)
                : single_pass_t<_Float16, 128, false>(p, causal, masked, s);
  }
  if (d == 64)
    return drop ? single_pass_t<__bf16, 64, true>(p, causal, masked, s)
                : single_pass_t<__bf16, 64, false>(p, causal, masked, s);
  return drop ? single_pass_t<__bf16, 128, true>(p, causal, masked, s)
              : single_pass_t<__bf16, 128, false>(p, causal, masked, s);
}

template <bool DROP>
static hipError_t dq_dispatch(const BwdParams& p, int dtype, int d, bool causal, bool masked,
                              hipStream_t s) {
  if (dtype == 1)
    return d == 64 ? launch_dq_t<_Float16, 64, DROP>(p, causal, masked, s)
                   : launch_dq_t<_Float16, 128, DROP>(p, causal, masked, s);
  return d == 64 ? launch_dq_t<__bf16, 64, DROP>(p, causal, masked, s)
                 : launch_dq_t<__bf16, 128, DROP>(p, causal, masked, s);
}

template <bool DROP>
static hipError_t dkdv_dispatch(const BwdParams& p, int dtype, int d, bool causal, bool masked,
                                hipStream_t s) {
  if (dtype == 1)
    return d == 64 ? launch_dkdv_t<_Float16, 64, DROP>(p, causal, masked, s)
                   : launch_dkdv_t<_Float16, 128, DROP>(p, causal, masked, s);
  return d == 64 ? launch_dkdv_t<__bf16, 64, DROP>(p, causal, masked, s)
                 : launch_dkdv_t<__bf16, 128, DROP>(p, causal, masked, s);
}

hipError_t launch_bwd_dq(const BwdParams& p, int dtype, int d, bool causal, bool masked,
                         hipStream_t s) {
  return dq_dispatch<false>(p, dtype, d, causal, masked, s);
}

hipError_t launch_bwd_dkdv(const BwdParams& p, int dtype, int d, bool causal, bool masked,
                           hipStream_t s) {
  return dkdv_dispatch<false>(p, dtype, d, causal, masked, s);
}

hipError_t launch_bwd_dq_drop(const BwdParams& p, int dtype, int d, bool causal, bool masked,
                              hipStream_t s) {
  return dq_dispatch<true>(p, dtype, d, causal, masked, s);
}

hipError_t launch_bwd_dkdv_drop(const BwdParams& p, int dtype, int d, bool causal, bool masked,
                                hipStream_t s) {
  return dkdv_dispatch<true>(p, dtype, d, causal, masked, s);
}

}  // namespace fa
