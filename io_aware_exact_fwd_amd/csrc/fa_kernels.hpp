// fa_kernels.hpp -- parameter blocks and launchers of the attention kernels
// (host-visible declarations; the kernels live in fa_fwd.hip, fa_bwd.hip,
// fa_f32.hip and fa_mask.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace fa {

// Tile geometry of the matrix-core kernels.
constexpr int kFwdRows = 128;   // query rows per forward / dQ workgroup (4 waves x 32)
constexpr int kKeyTile = 64;    // keys per inner step of the forward / dQ loop
constexpr int kBwdKeys = 128;   // keys per dK/dV workgroup (4 waves x 32)
constexpr int kThreads = 256;
constexpr int kDecKeys = 32;   // keys per tile of the decode kernel

// Block-sparse lists compiled from the dense block mask (see fa_mask_compile).
struct MaskLists {
  const int32_t* row_ptr;  // [nb + 1]
  const int32_t* col_idx;  // kept key blocks per query block
  const int32_t* col_ptr;  // [nb + 1]
  const int32_t* row_idx;  // query blocks per key block
  int32_t mask_block;      // multiple of 128
};

// Dropout of P (see fa_dropout.hpp).  Active iff t8 > 0.
struct DropParams {
  uint32_t t8;      // floor(256 p): a weight is kept iff its generator byte >= t8
  float mult;       // 256 / (256 - t8), the scale of kept weights
  uint32_t k0, k1;  // generator key: seed mod 2^32, seed / 2^32
  uint32_t offset;  // counter word 3
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int N;
  int nheads;     // B * H (query heads)
  int nqt;        // query tiles per head
  int window;     // 0: none; W > 0: |i - j| < W
  int group;      // query heads per K/V head; K/V head of query head h is h / group
  float c;        // scale * log2(e)
  MaskLists m;
  DropParams drop;
  int32_t* visits;  // debug build: tile-visit counters (see fa_debug_set_tile_visits), else null
  int spread;       // set by the launcher: CUs per XCD for spread_tile, or 0
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;    // D_i = dO_i . O_i, float32 [B*H*N]
  float* dqacc;   // single-pass backward: float32 dQ accumulator [B*H*N*d], else null
  int N;
  int nheads;     // dQ kernel: query heads B*H; dK/dV kernel: K/V heads B*H_kv
  int ntiles;     // query tiles (dQ kernel) or key tiles (dK/dV kernel) per head
  int window;     // 0: none; W > 0: |i - j| < W
  int group;      // query heads per K/V head
  float c;        // scale * log2(e)
  float scale;
  MaskLists m;
  DropParams drop;
  int32_t* visits;  // debug build: tile-visit counters, else null
  int spread;       // set by the launcher: CUs per XCD for spread_tile, or 0
};

// Decode-shaped forward (fa_decode.hip): n_q queries per head at positions
// N - n_q .. N - 1, keys split over workgroups, partials merged.
struct DecParams {
  const void* q;     // (B, H, n_q, d)
  const void* k;     // (B, H_kv, N, d)
  const void* v;
  void* o;           // (B, H, n_q, d)
  float* lse;        // (B, H, n_q)
  float* part_o;     // [B*H*n_q][nsplit][d] float32 partial outputs (nsplit > 1)
  float* part_lse;   // [B*H*n_q][nsplit]
  int N;             // keys
  int nq;            // queries per head
  int rows;          // rows per K/V head: group * n_q
  int nrb;           // row blocks of 128 per K/V head
  int nkv;           // B * H_kv
  int nsplit;        // key splits
  int tiles_per_split;
  int tile0;         // first 64-key tile any row sees
  int ntiles;        // tiles from tile0 through the last one any row sees
  int window;        // 0: none; W > 0: |pos - j| < W
  float c;           // scale * log2(e)
};

// FP8 forward (fa_fp8.hip): rotation + block quantisation, then attention on
// the codes.
struct Fp8QuantParams {
  const void* x0;       // Q (B*H, N, d) in the problem dtype
  const void* x1;       // K (B*H_kv, N, d)
  const void* x2;       // V (B*H_kv, N, d)
  uint8_t* c0;          // Q codes, row-major (B*H, N64, d)
  uint8_t* c1;          // K codes, row-major (B*H_kv, N64, d)
  uint8_t* c2;          // V codes, tiles (B*H_kv, N64/64, d, 64)
  int8_t* e0;           // block exponents (heads, N64 / 64) of Q, K, V
  int8_t* e1;
  int8_t* e2;
  const float* signs;   // d random signs of the rotation
  int nq_wg;            // workgroups (64-row blocks) of Q
  int nk_wg;            // of K (V has as many)
  int N;
  int N64;              // N rounded up to a multiple of 64
};

struct Fp8FwdParams {
  const uint8_t* qc;    // Q codes (B*H, N64, d)
  const uint8_t* kc;    // K codes (B*H_kv, N64, d)
  const uint8_t* vc;    // V codes, tiles (B*H_kv, N64/64, d, 64)
  const int8_t* qe;     // block exponents
  const int8_t* ke;
  const int8_t* ve;
  const float* signs;
  void* o;              // (B, H, N, d) in the problem dtype
  float* lse;           // (B, H, N)
  int N;
  int N64;
  int nheads;           // B * H
  int nqt;              // 128-row query tiles per head
  int window;
  int group;            // query heads per K/V head
  float c;              // scale * log2(e)
};

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  const float* o;
  const float* dout;
  float* out_o;
  float* lse;       // forward output / backward input
  float* dq;
  float* dk;
  float* dv;
  float* dvec;
  const uint8_t* block_mask;
  int mask_block;
  int N;
  int nheads;       // forward / dQ: query heads; dK/dV: K/V heads
  int d;
  int causal;
  int window;
  int group;
  float c;
  float scale;
  DropParams drop;
};

// Each launcher returns hipSuccess or the launch error.
// ---- persistent grids ----------------------------------------------------------
// The forward and backward kernels launch at most as many workgroups as the GPU
// holds at once; each walks a static list of work units (unit b of the
// head-major order goes to workgroup b mod grid).  One workgroup per unit
// leaves CUs idle between workgroups: the dispatcher hands them out in order,
// one XCD after the other, and a workgroup whose XCD is full holds back all
// later ones.
// Compute units of the current device (cached per device; 1 if the query
// fails, which only narrows the grid).
inline int cu_count() {
  constexpr int kDevices = 64;
  static std::atomic<int> cache[kDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  if (dev >= 0 && dev < kDevices) {
    const int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
  }
  int n = 0;
  if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 1;
  if (dev >= 0 && dev < kDevices) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}
// Workgroups of Kernel resident on the GPU at once: CUs x workgroups per CU,
// the occupancy queried once per kernel.
template <auto Kernel>
inline long long resident_workgroups() {
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, Kernel, kThreads, 0) != hipSuccess || n < 1) n = 1;
    return n;
  }();
  return (long long)cu_count() * per_cu;
}
// Grid of a persistent launch: min(units, resident workgroups).
template <auto Kernel>
inline int persistent_grid(int units) {
  const long long g = resident_workgroups<Kernel>();
  return (int)(units < g ? units : g);
}
// Causal tiles of nheads heads, ntiles each, launched one workgroup per tile
// with Kernel: the CUs per XCD that spread_tile deals them over when they are
// all resident at once and the heads split evenly over the 8 XCDs (measured
// on GPT-2-small's forward: 32.4 -> 25.6 us against tile pairs, whose 384
// units load half the CUs twice), else 0.
template <auto Kernel>
inline int spread_for(int nheads, int ntiles) {
  const int cus = cu_count();
  if (nheads % 8 != 0 || cus % 8 != 0) return 0;
  return (long long)nheads * ntiles <= resident_workgroups<Kernel>() ? cus / 8 : 0;
}
// Launch Kernel over `units` work units: a persistent grid, or one workgroup
// per unit.  The kernels take persistent grids for causal work without a
// window or block mask, split into units of equal cost (the tile pairs t and
// n - 1 - t of a head); units of uneven cost (a block mask's, a window's)
// measured faster one workgroup each, balanced by the dispatcher.
template <auto Kernel, typename Params>
inline void launch_units(const Params& p, int units, bool persistent, hipStream_t s) {
  const int grid = persistent ? persistent_grid<Kernel>(units) : units;
  hipLaunchKernelGGL(Kernel, dim3(grid), dim3(kThreads), 0, s, p);
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int d, bool causal, bool masked,
                      hipStream_t s);
hipError_t launch_bwd_dq(const BwdParams& p, int dtype, int d, bool causal, bool masked,
                         hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdParams& p, int dtype, int d, bool causal, bool masked,
                           hipStream_t s);
// Dropout variants (p.drop.t8 > 0); same arguments.
hipError_t launch_fwd_drop(const FwdParams& p, int dtype, int d, bool causal, bool masked,
                           hipStream_t s);
hipError_t launch_bwd_dq_drop(const BwdParams& p, int dtype, int d, bool causal, bool masked,
                              hipStream_t s);
// Single-pass backward (FA_BWD_ATOMIC_DQ): D and the cleared accumulator,
// dK/dV with dQ added into p.dqacc by atomics, then dq = scale * accumulator.
// p as for launch_bwd_dkdv (K/V heads, key tiles), with dq and dqacc set.
hipError_t launch_bwd_single_pass(const BwdParams& p, int dtype, int d, bool causal, bool masked,
                                  hipStream_t s);
hipError_t launch_bwd_dkdv_drop(const BwdParams& p, int dtype, int d, bool causal, bool masked,
                                hipStream_t s);
hipError_t launch_decode(const DecParams& p, int dtype, int d, bool causal, hipStream_t s);
hipError_t launch_fp8_quantize(const Fp8QuantParams& qp, int dtype, int d, int wgs, hipStream_t s);
hipError_t launch_fp8_fwd(const Fp8FwdParams& p, int dtype, int d, bool causal, hipStream_t s);
hipError_t launch_f32_fwd(const F32Params& p, hipStream_t s);
hipError_t launch_f32_dq(const F32Params& p, hipStream_t s);
hipError_t launch_f32_dkdv(const F32Params& p, hipStream_t s);
hipError_t launch_mask_compile(const uint8_t* mask, int nb, int32_t* row_ptr, int32_t* col_idx,
                               int32_t* col_ptr, int32_t* row_idx, hipStream_t s);

}  // namespace fa
