// fa_fp8.hip -- FP8 forward with block scales and a random Hadamard rotation.
//
// The FP8 path of the FlashAttention-3 section of "Atencao Eficiente em
// Escala" (living-dl-book, section 10): Q, K and V are rotated by an orthogonal
// Hadamard-style matrix with random signs, which spreads outlier coordinates
// over the whole vector, then quantised to FP8 with one scale per tile; the
// rotation cancels inside Q K^T and is undone on the output after the P V
// product.
//
//   M = diag(s) H / sqrt(d)   (H the d x d Sylvester Hadamard matrix, s the
//                              caller's random signs; M is orthogonal)
//   Qr = Q M, Kr = K M, Vr = V M;  S = scale Qr Kr^T (= scale Q K^T);
//   O = softmax(S) Vr M^T.
//
// Formats.  E4M3 (bias 7, 3 mantissa bits, largest finite 448), round to
// nearest even (v_cvt_pk_fp8_f32; checked on the device against an encoder
// written from the format definition).  Every 64-row block of a head gets a
// power-of-two scale 2^e, e the smallest integer with max|y| <= 448 * 2^e, so
// the scales are exact E8M0 values that the matrix cores apply themselves:
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies row / column blocks of its
// operands by 2^(scale - 127) (layout and scales checked on the device: lane l
// holds row l % 32 and k = 32 (l / 32) .. + 31 of A, the mirror for B, and the
// 32 x 32 result in the layout of the 16-bit 32x32x16 product).
//
// Workspace layout (all from one caller buffer, regions 256-byte aligned; N64
// = N rounded up to a multiple of 64, rows past N quantised as zeros):
//   Q codes  (B H,    N64, d) uint8, row-major per head
//   K codes  (B H_kv, N64, d) uint8, row-major per head
//   V codes  (B H_kv, N64 / 64, d, 64) uint8: per 64-key tile, row c of the
//            tile holds column c of V; its byte p holds key kappa(p) of the
//            tile, kappa(p) = 32 (i / 16) + 8 ((i % 16) / 4) + 4 h + i % 4 with
//            h = p / 32, i = p % 32 -- the key order in which the probability
//            tile sits in a lane's registers, so that both operands of P V are
//            contiguous reads
//   Q, K, V exponents e (int8) per 64-row block
#include <math.h>

#include "fa_common.hpp"
#include "fa_kernels.hpp"
#include "fa_tiles.hpp"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kFp8Tau = 8.0f;  // reference move threshold: P <= 2^8 = 256 < 448

template <int D>
__device__ __forceinline__ float inv_sqrt_d() {
  // float32(1 / sqrt(d)), the constant the oracle uses
  return D == 64 ? 0.125f : (float)(1.0 / 11.313708498984761);
}

// XOR swizzle of the 16-byte chunks of an FP8 tile row (64 or 128 bytes), so
// that 16 lanes reading 16 consecutive rows at one chunk hit 16 different bank
// groups of 16 bytes.
template <int ROWBYTES>
__device__ __forceinline__ int swz8(int r) {
  return ROWBYTES == 64 ? (r >> 2) & 3 : (r >> 1) & 7;
}
template <int ROWBYTES>
__device__ __forceinline__ int swz8_off(int r, int chunk) {
  return (r * (ROWBYTES / 16) + (chunk ^ swz8<ROWBYTES>(r))) * 16;
}

// Copy ROWS rows of ROWBYTES bytes, starting at byte `base` of buffer b, into
// the swizzled LDS tile (256 threads; copy n of wave w fills 1 KiB block 4n+w).
template <int ROWBYTES, int ROWS>
__device__ __forceinline__ void dma_tile8(const Buf& b, uint32_t base, char* tile, int wave, int lane) {
  constexpr int CPR = ROWBYTES / 16;
  constexpr int NI = ROWS * CPR / 256;
  static_assert(ROWS * CPR % 256 == 0, "whole 1 KiB blocks per wave");
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int P = (n * 4 + wave) * 64 + lane;
    const int r = P / CPR, pc = P % CPR;
    dma16(b, base + (uint32_t)(r * ROWBYTES + ((pc ^ swz8<ROWBYTES>(r)) << 4)), tile + (n * 4 + wave) * 1024);
  }
}

// two floats -> E4M3 bytes in the low (HI = false) or high 16 bits of `old`
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// Smallest e >= -127 (the E8M0 range) with amax <= 448 * 2^e, from the float32
// bits; 0 for amax = 0.  A float32-subnormal amax reads as exponent -127 and
// lands on the -127 floor like every amax below 448 * 2^-128.
__device__ __forceinline__ int block_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  const uint32_t u = __builtin_bit_cast(uint32_t, amax);
  const int E = (int)((u >> 23) & 0xFF) - 127;
  return max(-127, E - 8 + ((u & 0x7FFFFF) > 0x600000 ? 1 : 0));  // mantissa above 1.75
}

__device__ __forceinline__ float exp2i(int k) {  // 2^k, -126 <= k <= 127
  return __builtin_bit_cast(float, (uint32_t)(k + 127) << 23);
}

// ---------------------------------------------------------------------------
// Quantisation: one workgroup of two waves per 64-row block of one head; a
// wave holds 32 rows, lane l the first half of its row and lane l + 32 the
// second half, so a lane keeps d/2 values in registers.  Q, K and V blocks
// share one launch.  The block's rows are copied into LDS with contiguous
// 1 KiB copies, each lane reads its half row (XOR-swizzled 16-byte chunks keep
// those reads free of bank conflicts), and the codes leave through LDS again
// so that the global stores are contiguous too.
template <int CPR>
__device__ __forceinline__ int swzq(int r) {  // chunk swizzle of a CPR-chunk row
  return CPR == 16 ? (r & 15) : CPR == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

template <typename T, int D>
__global__ __launch_bounds__(128) void fp8_quant_kernel(Fp8QuantParams p) {
  constexpr int RB = 2 * D;      // input row bytes
  constexpr int CPR = RB / 16;   // input chunks per row
  constexpr int OCPR = D / 16;   // code chunks per row
  constexpr int H = D / 2;       // values per lane
  __shared__ __attribute__((aligned(16))) char tile[64 * RB];
  __shared__ float wave_max[2];
  debug_fill_lds_nan(tile, sizeof(tile));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int g = lane >> 5;                 // which half of the row
  const int r = wave * 32 + (lane & 31);   // row within the block
  const int nblk = p.N64 / 64;
  // which tensor (uniform per workgroup): Q, then K, then V
  int idx = blockIdx.x;
  int t = 0;
  if (idx >= p.nq_wg) {
    idx -= p.nq_wg;
    t = 1;
    if (idx >= p.nk_wg) {
      idx -= p.nk_wg;
      t = 2;
    }
  }
  const void* x = t == 0 ? p.x0 : t == 1 ? p.x1 : p.x2;
  uint8_t* codes = t == 0 ? p.c0 : t == 1 ? p.c1 : p.c2;
  int8_t* exps = t == 0 ? p.e0 : t == 1 ? p.e1 : p.e2;
  const int head = idx / nblk;
  const int blk = idx % nblk;

  // rows blk*64 .. +63 of the head (rows past N read as zeros): CPR copies of
  // 1 KiB, copy n of wave w filling block 2n + w
  const Buf bx = make_buf((const char*)x + (size_t)head * p.N * RB, (uint32_t)p.N * RB);
#pragma unroll
  for (int n = 0; n < CPR / 2; ++n) {
    const int P = (2 * n + wave) * 64 + lane, rr = P / CPR, sl = P % CPR;
    dma16(bx, (uint32_t)(blk * 64 + rr) * RB + (uint32_t)((sl ^ swzq<CPR>(rr)) << 4), tile + (2 * n + wave) * 1024);
  }
  wait_all_memory();
  __syncthreads();

  float y[H];
#pragma unroll
  for (int c = 0; c < CPR / 2; ++c) {
    const int cc = g * (CPR / 2) + c;
    const u32x4 w = *(const u32x4*)(tile + r * RB + ((cc ^ swzq<CPR>(r)) << 4));
    const T* e = (const T*)&w;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[8 * c + i] = to_f32(e[i]) * p.signs[g * H + 8 * c + i];
  }
  // fast Walsh-Hadamard transform, pair distances 1, 2, ..., D/2: the stages
  // below D/2 inside the half row, the last one between the two halves
  // (element i with element i + D/2, held by lane l ^ 32)
#pragma unroll
  for (int h = 1; h < H; h <<= 1)
#pragma unroll
    for (int i = 0; i < H; ++i)
      if (!(i & h)) {
        const float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
  const float sgn = g == 0 ? 1.f : -1.f;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const LanePair pr = lane_pair(y[i]);
    y[i] = __builtin_fmaf(pr.hi, sgn, pr.lo);  // a + b or a - b, one rounding
  }
  // The rotated row is fl(y * c), c = float32(1 / sqrt(d)), and its codes are
  // E4M3(fl(y * c) * 2^-e).  Rounding is monotone, so the block maximum is
  // fl(max|y| * c).  For e >= -100, every element that E4M3 does not round
  // to zero has |y c| >= 2^-110 (normal), and c * 2^-e is an exact float32,
  // so fl(y * (c * 2^-e)) = fl(y * c) * 2^-e: one multiply per element gives
  // the same codes.  Smaller blocks (magnitudes near float32 underflow, where
  // fl(y * c) may be subnormal) take both roundings in turn.
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < H; ++i) amax = fmaxf(amax, fabsf(y[i]));
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if (lane == 0) wave_max[wave] = amax;
  __syncthreads();  // also: every lane has read its input row
  amax = fmaxf(wave_max[0], wave_max[1]);
  const int e = block_exponent(amax * inv_sqrt_d<D>());
  float mul = inv_sqrt_d<D>() * exp2i(-e);  // exact
  if (e < -100) {  // uniform over the workgroup
#pragma unroll
    for (int i = 0; i < H; ++i) y[i] *= inv_sqrt_d<D>();
    mul = exp2i(-e);
  }
  uint32_t w[H / 4];
#pragma unroll
  for (int j = 0; j < H / 4; ++j) {
    w[j] = fp8x2<false>(y[4 * j] * mul, y[4 * j + 1] * mul, 0u);
    w[j] = fp8x2<true>(y[4 * j + 2] * mul, y[4 * j + 3] * mul, w[j]);
  }
  if (tid == 0) exps[(size_t)head * nblk + blk] = (int8_t)e;

  // codes of the block, row-major with swizzled chunks, at the start of tile
#pragma unroll
  for (int j = 0; j < OCPR / 2; ++j) {
    const int cc = g * (OCPR / 2) + j;
    *(u32x4*)(tile + r * D + ((cc ^ swzq<OCPR>(r)) << 4)) = u32x4{w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]};
  }
  __syncthreads();
  if (t != 2) {
    uint8_t* out = codes + ((size_t)head * p.N64 + blk * 64) * D;
#pragma unroll
    for (int it = 0; it < OCPR / 2; ++it) {
      const int P = it * 128 + tid, rr = P / OCPR, pos = P % OCPR;
      *(u32x4*)(out + rr * D + ((pos ^ swzq<OCPR>(rr)) << 4)) = *(const u32x4*)(tile + P * 16);
    }
  } else {
    // V: row c of the output tile = column c of the codes, byte p of it the
    // code of key kappa(p); built in the second half of tile, then stored
    // contiguously
    char* otile = tile + 64 * D;
    for (int c = tid; c < D; c += 128) {
      uint32_t ow[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        uint32_t word = 0;
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          const int pp = q * 4 + bt, h = pp >> 5, i = pp & 31;
          const int key = (i >> 4) * 32 + ((i & 15) >> 2) * 8 + 4 * h + (i & 3);
          const int off = key * D + (((c >> 4) ^ swzq<OCPR>(key)) << 4) + (c & 15);
          word |= (uint32_t)(uint8_t)tile[off] << (8 * bt);
        }
        ow[q] = word;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(u32x4*)(otile + c * 64 + 16 * q) = u32x4{ow[4 * q], ow[4 * q + 1], ow[4 * q + 2], ow[4 * q + 3]};
    }
    __syncthreads();
    uint8_t* out = codes + ((size_t)head * nblk + blk) * D * 64;
#pragma unroll
    for (int it = 0; it < D / 32; ++it) {
      const int P = it * 128 + tid;
      *(u32x4*)(out + P * 16) = *(const u32x4*)(otile + P * 16);
    }
  }
}

// ---------------------------------------------------------------------------
// Attention on the quantised tensors: the tiling, masks and online softmax of
// fwd_kernel (fa_fwd.hip) with both products on the FP8 matrix cores.
template <int D>
struct Fp8Geom {
  static constexpr int KT = 64;
  static constexpr int KBYTES = KT * D;   // K codes tile, rows of D bytes
  static constexpr int VBYTES = D * KT;   // V codes tile, rows of 64 bytes
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int NDB = D / 32;
  static constexpr int NKS = D / 64;      // k-steps of the score product
};

// FP8 attention, head dim 128: 163 VGPRs, 32 KiB LDS, three waves per SIMD
// (measured 4 % faster than two)
constexpr int kFp8Wpe128 = 3;

template <typename T, int D, bool CAUSAL, int WPE, bool PERSIST>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(WPE, WPE)))
void fp8_fwd_kernel(Fp8FwdParams p) {
  using G = Fp8Geom<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * G::STAGE];
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
    const int q0 = qt * 128;
    const int qw0 = q0 + wave * 32;
    const int qw_last = qw0 + 31;
    const int q_hi = min(q0 + 128, N) - 1;
    const int kvh = head / p.group;
    const int nblk = p.N64 / 64;

    const Buf bq = make_buf(p.qc + (size_t)head * p.N64 * D, (uint32_t)p.N64 * D);
    const Buf bk = make_buf(p.kc + (size_t)kvh * p.N64 * D, (uint32_t)p.N64 * D);
    const Buf bv = make_buf(p.vc + (size_t)kvh * p.N64 * D, (uint32_t)p.N64 * D);
    // this wave's Q block scale (E8M0); a wave wholly past N64 (only in the last
    // query tile) reads zero codes and writes nothing
    const int sq = qw0 < p.N64 ? 127 + p.qe[(size_t)head * nblk + qw0 / 64] : 127;
    const int8_t* ke = p.ke + (size_t)kvh * nblk;
    const int8_t* ve = p.ve + (size_t)kvh * nblk;

    const Band band{N, p.window, CAUSAL};
    MaskLists none;
    none.row_ptr = none.col_idx = none.col_ptr = none.row_idx = nullptr;
    none.mask_block = 0;
    const auto tiles = key_tiles<G::KT, false>(none, band, q0, q_hi);
    const int ntiles = tiles.count;

    // Q codes: B operand of S^T = K Q^T, 32 consecutive head-dim bytes per lane
    i32x8 qf[G::NKS];
#pragma unroll
    for (int t = 0; t < G::NKS; ++t) {
      const uint32_t off = (uint32_t)((qw0 + l32) * D + 64 * t + 32 * g);
      const u32x4 lo = buf_load16(bq, off), hi = buf_load16(bq, off + 16);
      qf[t] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }

    f32x16 o[G::NDB];
#pragma unroll
    for (int i = 0; i < G::NDB; ++i) o[i] = f32x16{0};
    float m_ref = kNegInf, ref = 0.f, l_run = 0.f;

    auto gload = [&](int it, int stage) {
      const int k0 = tiles.pos0(it);
      char* ks = smem + stage * G::STAGE;
      dma_tile8<D, 64>(bk, (uint32_t)k0 * D, ks, wave, lane);
      dma_tile8<64, D>(bv, (uint32_t)(k0 / 64) * D * 64, ks + G::KBYTES, wave, lane);
    };
    if (ntiles > 0) gload(0, 0);
    wait_all_memory();
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
      const int cur = it & 1;
      if (it + 1 < ntiles) gload(it + 1, cur ^ 1);
      const int k0 = tiles.pos0(it);
      const char* ks = smem + cur * G::STAGE;
      const char* vs = ks + G::KBYTES;
      if (k0 <= band.hi(qw_last) && k0 + G::KT - 1 >= band.lo(qw0)) {
        const int sk = 127 + ke[k0 / 64];
        const int sv = 127 + ve[k0 / 64];
        // S^T = K Q^T, dequantised by the block scales inside the product
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb] = f32x16{0};
#pragma unroll
          for (int t = 0; t < G::NKS; ++t) {
            const int r = kb * 32 + l32;
            const u32x4 lo = *(const u32x4*)(ks + swz8_off<D>(r, 4 * t + 2 * g));
            const u32x4 hi = *(const u32x4*)(ks + swz8_off<D>(r, 4 * t + 2 * g + 1));
            const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[t], s[kb], 0, 0, 0, sk, 0, sq);
          }
        }
        // keys outside the row's band; key of register r of block kb is
        // k0 + g*4 + C, C = kb*32 + (r/4)*8 + r%4
        if (k0 + G::KT - 1 > band.hi(qw0)) {
          const int ub = band.hi(qw0 + l32) - k0 - g * 4;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int C = kb * 32 + (r >> 2) * 8 + (r & 3);
              s[kb][r] = C > ub ? kNegInf : s[kb][r];
            }
        }
        if (k0 < band.lo(qw_last)) {
          const int lb = band.lo(qw0 + l32) - k0 - g * 4;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int C = kb * 32 + (r >> 2) * 8 + (r & 3);
              s[kb][r] = C < lb ? kNegInf : s[kb][r];
            }
        }
        // online softmax over the whole tile, then one P V product per
        // 32-column block of O
        const float mx = vmax(max16(s[0]), max16(s[1])) * p.c;
        if (__builtin_amdgcn_ballot_w64(mx > m_ref + kFp8Tau) != 0) {
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
        // P = 2^(S c - ref) <= 256, rounded to E4M3; byte i = 16 kb + r of the
        // lane's operand is key kappa(g, i) of the tile
        uint32_t pw[8];
        float lp = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 4 * q;
            const float e0 = fast_exp2(__builtin_fmaf(s[kb][r], p.c, -ref));
            const float e1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], p.c, -ref));
            const float e2 = fast_exp2(__builtin_fmaf(s[kb][r + 2], p.c, -ref));
            const float e3 = fast_exp2(__builtin_fmaf(s[kb][r + 3], p.c, -ref));
            lp += (e0 + e1) + (e2 + e3);  // row sum of the unrounded weights
            pw[kb * 4 + q] = fp8x2<true>(e2, e3, fp8x2<false>(e0, e1, 0u));
          }
        l_run += lp;
        const i32x8 pb = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
        // O'^T += V^T P^T: row db*32 + l32 of the V codes tile, bytes 32 g ..
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
          const int r = db * 32 + l32;
          const u32x4 lo = *(const u32x4*)(vs + swz8_off<64>(r, 2 * g));
          const u32x4 hi = *(const u32x4*)(vs + swz8_off<64>(r, 2 * g + 1));
          const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, o[db], 0, 0, 0, sv, 0, 127);
        }
      }
      wait_all_memory();  // this thread's copies into the next stage have landed
      __syncthreads();
    }

    // epilogue: O' / l, then undo the rotation, O = O' H diag(s) / sqrt(d).
    // Register r of block db holds head-dim column db*32 + (r/4)*8 + 4g + r%4:
    // the Hadamard butterflies over bits 0, 1, 3, 4 (and 5, 6: db) of the column
    // pair registers of one lane; bit 2 pairs lane l with lane l ^ 32.
    const float lt = pair_sum(l_run);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= inv;
#pragma unroll
    for (int bit = 0; bit < 4; ++bit) {  // register bits r&1, r&2, r&4, r&8
      const int h = 1 << bit;
#pragma unroll
      for (int db = 0; db < G::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!(r & h)) {
            const float a = o[db][r], b = o[db][r + h];
            o[db][r] = a + b;
            o[db][r + h] = a - b;
          }
    }
#pragma unroll
    for (int h = 1; h < G::NDB; h <<= 1)  // column bits 5, 6: between blocks
#pragma unroll
      for (int db = 0; db < G::NDB; ++db)
        if (!(db & h))
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float a = o[db][r], b = o[db + h][r];
            o[db][r] = a + b;
            o[db + h][r] = a - b;
          }
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {  // column bit 2: across the lane halves
        const LanePair pr = lane_pair(o[db][r]);
        o[db][r] = g == 0 ? pr.lo + pr.hi : pr.lo - pr.hi;
      }
    const int q = qw0 + l32;
    if (q < N) {
      T* orow = (T*)p.o + ((size_t)head * N + q) * D;
#pragma unroll
      for (int db = 0; db < G::NDB; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int c = db * 32 + rr * 8 + g * 4;
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = o[db][rr * 4 + e] * inv_sqrt_d<D>() * p.signs[c + e];
          u32x2 w;
          w[0] = pack2<T>(x[0], x[1]);
          w[1] = pack2<T>(x[2], x[3]);
          *(u32x2*)(orow + c) = w;
        }
      if (g == 0) p.lse[(size_t)head * N + q] = lt > 0.f ? (m_ref + fast_log2(lt)) * kLn2 : kNegInf;
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
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int head = logical / p.nqt, qt = logical % p.nqt;
    tile(head, CAUSAL ? p.nqt - 1 - qt : qt);  // causal: the longer rows first
  }
}

template <typename T, int D>
hipError_t quant_t(const Fp8QuantParams& qp, int wgs, hipStream_t s) {
  hipLaunchKernelGGL((fp8_quant_kernel<T, D>), dim3(wgs), dim3(128), 0, s, qp);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t fwd8_t(const Fp8FwdParams& p, bool causal, hipStream_t s) {
  constexpr int WPE = D == 64 ? 4 : kFp8Wpe128;
  // causal work without a window: a persistent grid over tile pairs (as the
  // 16-bit forward); the rest one workgroup per tile
  if (causal && p.window == 0)
    launch_units<fp8_fwd_kernel<T, D, true, WPE, true>>(p, p.nheads * ((p.nqt + 1) / 2), true, s);
  else if (causal)
    launch_units<fp8_fwd_kernel<T, D, true, WPE, false>>(p, p.nheads * p.nqt, false, s);
  else
    launch_units<fp8_fwd_kernel<T, D, false, WPE, false>>(p, p.nheads * p.nqt, false, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_quantize(const Fp8QuantParams& qp, int dtype, int d, int wgs, hipStream_t s) {
  if (dtype == 1) return d == 64 ? quant_t<_Float16, 64>(qp, wgs, s) : quant_t<_Float16, 128>(qp, wgs, s);
  return d == 64 ? quant_t<__bf16, 64>(qp, wgs, s) : quant_t<__bf16, 128>(qp, wgs, s);
}

hipError_t launch_fp8_fwd(const Fp8FwdParams& p, int dtype, int d, bool causal, hipStream_t s) {
  if (dtype == 1) return d == 64 ? fwd8_t<_Float16, 64>(p, causal, s) : fwd8_t<_Float16, 128>(p, causal, s);
  return d == 64 ? fwd8_t<__bf16, 64>(p, causal, s) : fwd8_t<__bf16, 128>(p, causal, s);
}

}  // namespace fa
