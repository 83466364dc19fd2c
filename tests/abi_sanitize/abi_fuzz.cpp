// Host-only check of the C ABI's argument handling and workspace layout,
// built with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
// (see build_check.py).  The kernel launchers are stand-ins that record their
// parameters (launch_stubs.cpp), so no GPU is needed.
//
// For many problems drawn from edge values (sizes around tile and block
// boundaries, the largest accepted sizes and beyond, zero and negative
// values, non-finite scales, unknown dtypes and flags), every entry point is
// called with aligned fake device addresses.  Checked:
//   * a call that returns an error launched nothing;
//   * workspace sizes are multiples of 256, the backward's at least the
//     forward's, 0 for a problem the call rejects;
//   * every pointer a call derives from a workspace (block lists, D, decode
//     partials, FP8 regions) lies inside the size the matching
//     fa_*_workspace_size reported, and the regions do not overlap;
//   * null, misaligned or short arguments are rejected with the documented
//     status.
// Any memory error or undefined behaviour in the host code aborts the run.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <limits>

#include "../../include/fa.h"
#include "launch_stubs.h"

namespace {

uint64_t g_state = 0x243F6A8885A308D3ull;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
template <typename T, size_t N>
T pick(const T (&v)[N]) {
  return v[next_u64() % N];
}

long g_failures = 0;
#define CHECK(cond, ...)                                              \
  do {                                                                \
    if (!(cond)) {                                                    \
      if (g_failures < 20) {                                          \
        fprintf(stderr, "check failed (%s:%d): %s: ", __FILE__, __LINE__, #cond); \
        fprintf(stderr, __VA_ARGS__);                                 \
        fprintf(stderr, "\n");                                        \
      }                                                               \
      ++g_failures;                                                   \
    }                                                                 \
  } while (0)

// fake device addresses: 256-aligned, far apart, never dereferenced
char* fake(int i) { return (char*)(uintptr_t)(0x100000000000ull + (uint64_t)i * 0x1000000000ull); }

bool inside(const void* p, size_t bytes, const char* base, size_t size) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)base;
  return a >= b && bytes <= size && a - b <= size - bytes;
}

// half of the problems draw every field from accepted values only, so that
// the layout checks run often; the other half from all edge values
fa_problem valid_problem() {
  static const int32_t bh[] = {1, 2, 3, 4, 7, 16, 64};
  static const int32_t ns[] = {1, 63, 64, 65, 127, 128, 129, 256, 1000, 1024, 4096, 8192, 65536};
  static const int32_t ds[] = {64, 128};
  static const int32_t dts[] = {FA_F16, FA_BF16, FA_F32};
  static const int32_t mbs[] = {128, 256, 512};
  static const int32_t wins[] = {0, 0, 1, 300, 1 << 30};
  static const float drops[] = {0.f, 0.f, 0.1f, 0.5f};
  fa_problem p;
  p.B = pick(bh);
  p.H = pick(bh) * 2;
  p.N = pick(ns);
  p.d = pick(ds);
  p.dtype = pick(dts);
  p.causal = (int32_t)(next_u64() % 2);
  p.scale = 0.125f;
  const int32_t mb = pick(mbs);
  p.block_mask = (next_u64() % 2 == 0 && p.N % mb == 0) ? (const uint8_t*)fake(15) : nullptr;
  p.mask_block = p.block_mask ? mb : 0;
  p.window = pick(wins);
  const int32_t kvs[] = {0, 1, 2, p.H};
  p.H_kv = pick(kvs);
  p.dropout_p = pick(drops);
  p.seed = next_u64();
  p.offset = (uint32_t)next_u64();
  p.flags = (next_u64() % 3 == 0 ? FA_REUSE_LISTS : 0) | (next_u64() % 3 == 0 ? FA_BWD_ATOMIC_DQ : 0);
  return p;
}

fa_problem random_problem() {
  if (next_u64() % 2 == 0) return valid_problem();
  static const int32_t bh[] = {1, 2, 3, 7, 64, 1000, 1 << 16, std::numeric_limits<int32_t>::max(), 0, -1};
  static const int32_t ns[] = {1,    2,     63,       64,      65,      127,       128,
                               129,  1000,  1024,     8192,    65536,   1 << 20,   1 << 24,
                               8388607, std::numeric_limits<int32_t>::max(), 0, -5};
  static const int32_t ds[] = {64, 128, 64, 128, 32, 96, 0, -64, 256};
  static const int32_t dts[] = {FA_F16, FA_BF16, FA_F32, FA_F16, 3, -1};
  static const float scales[] = {0.125f, 0.088f, 1e-30f, 1e30f, 0.f, -1.f, INFINITY, NAN};
  static const int32_t mbs[] = {128, 256, 384, 64, 0, -128, 1 << 20};
  static const int32_t wins[] = {0, 0, 1, 300, 1 << 30, -1};
  static const float drops[] = {0.f, 0.f, 0.1f, 0.999f, 1.f, -0.1f, NAN};
  static const uint32_t flags[] = {0, 0, FA_REUSE_LISTS, FA_BWD_ATOMIC_DQ, 3, 4, 7, 0x80000000u};
  fa_problem p;
  p.B = pick(bh);
  p.H = pick(bh);
  p.N = pick(ns);
  p.d = pick(ds);
  p.dtype = pick(dts);
  p.causal = (int32_t)(next_u64() % 3 == 0 ? 2 : next_u64() % 2);
  p.scale = pick(scales);
  p.block_mask = next_u64() % 3 == 0 ? (const uint8_t*)fake(15) : nullptr;
  p.mask_block = pick(mbs);
  p.window = pick(wins);
  const int32_t kvs[] = {0, 1, 2, p.H, p.H < std::numeric_limits<int32_t>::max() ? p.H + 1 : 5, -1};
  p.H_kv = pick(kvs);
  p.dropout_p = pick(drops);
  p.seed = next_u64();
  p.offset = (uint32_t)next_u64();
  p.flags = pick(flags);
  return p;
}

// pointers of the compiled-list regions the last mask compile received lie in
// the workspace [ws, ws + size)
void check_lists(const fa_problem& p, const char* ws, size_t size, const char* what) {
  const size_t nb = (size_t)(p.N / p.mask_block);
  const size_t ext[4] = {(nb + 1) * 4, nb * nb * 4, (nb + 1) * 4, nb * nb * 4};
  for (int i = 0; i < 4; ++i)
    CHECK(inside(fa::g_rec.lists[i], ext[i], ws, size), "%s: list %d outside the workspace (N=%d mb=%d)",
          what, i, p.N, p.mask_block);
  CHECK(fa::g_rec.nb == (int)nb, "%s: block count", what);
}

void one(const fa_problem& p0) {
  fa_problem p = p0;
  const size_t w0 = fa_workspace_size(&p, 0), w1 = fa_workspace_size(&p, 1);
  CHECK(w0 % 256 == 0 && w1 % 256 == 0, "workspace sizes not 256-aligned");
  CHECK(w1 >= w0, "backward workspace smaller than the forward's");
  char *Q = fake(1), *K = fake(2), *V = fake(3), *O = fake(4), *L = fake(5), *DO = fake(6);
  char *DQ = fake(7), *DK = fake(8), *DV = fake(9), *WS = fake(10);
  const bool lists = p.block_mask && p.dtype != FA_F32;

  // forward
  long before = fa::g_rec.launches, mc = fa::g_rec.mask_compiles;
  int st = fa_fwd(&p, Q, K, V, O, (float*)L, WS, w0, nullptr);
  if (st != FA_OK) {
    CHECK(fa::g_rec.launches == before, "fa_fwd returned %d after launching", st);
  } else {
    CHECK(fa::g_rec.launches > before, "fa_fwd ok without a launch");
    if (lists && !(p.flags & FA_REUSE_LISTS)) check_lists(p, WS, w0, "fa_fwd");
    if (lists && (p.flags & FA_REUSE_LISTS)) CHECK(fa::g_rec.mask_compiles == mc, "fa_fwd compiled reused lists");
    if (lists) CHECK(inside(fa::g_rec.fwd.m.row_ptr, 4, WS, w0), "fa_fwd lists pointer");
    // the same call with a short or misaligned workspace
    if (w0 > 0) {
      before = fa::g_rec.launches;
      CHECK(fa_fwd(&p, Q, K, V, O, (float*)L, WS, w0 - 1, nullptr) == FA_ERR_WORKSPACE, "short fwd workspace");
      CHECK(fa_fwd(&p, Q, K, V, O, (float*)L, WS + 8, w0, nullptr) == FA_ERR_WORKSPACE, "misaligned fwd workspace");
      CHECK(fa_fwd(&p, Q, K, V, O, (float*)L, nullptr, w0, nullptr) == FA_ERR_WORKSPACE, "null fwd workspace");
      CHECK(fa::g_rec.launches == before, "rejected fwd calls launched");
    }
    before = fa::g_rec.launches;
    CHECK(fa_fwd(&p, nullptr, K, V, O, (float*)L, WS, w0, nullptr) == FA_ERR_ARG, "null q");
    CHECK(fa_fwd(&p, Q, K + 4, V, O, (float*)L, WS, w0, nullptr) == FA_ERR_ARG, "misaligned k");
    CHECK(fa_fwd(&p, Q, K, V, O, (float*)(L + 2), WS, w0, nullptr) == FA_ERR_ARG, "misaligned lse");
    CHECK(fa::g_rec.launches == before, "rejected fwd calls launched");
  }

  // backward (both stages)
  before = fa::g_rec.launches;
  st = fa_bwd(&p, Q, K, V, O, DO, (float*)L, DQ, DK, DV, WS, w1, nullptr);
  if (st != FA_OK) {
    CHECK(fa::g_rec.launches == before, "fa_bwd returned %d after launching", st);
  } else if (p.flags & FA_BWD_ATOMIC_DQ) {
    // single pass: D, then the float32 dQ accumulator, inside the workspace
    CHECK(p.dtype != FA_F32, "single-pass backward accepted float32");
    const fa::BwdParams& s = fa::g_rec.single;
    const size_t dbytes = (size_t)p.B * p.H * p.N * 4;
    CHECK(inside(s.dvec, dbytes, WS, w1), "single pass: D outside the workspace");
    CHECK(inside(s.dqacc, dbytes * (size_t)p.d, WS, w1),
          "single pass: dQ accumulator outside the workspace (B=%d H=%d N=%d d=%d w1=%zu)", p.B, p.H,
          p.N, p.d, w1);
    CHECK((const char*)s.dqacc >= (const char*)s.dvec + dbytes, "accumulator overlaps D");
    CHECK(s.dq == DQ && s.dk == DK && s.dv == DV, "single pass: output pointers");
    if (lists) {
      if (!(p.flags & FA_REUSE_LISTS)) check_lists(p, WS, w1, "fa_bwd single pass");
      const size_t nb = (size_t)(p.N / p.mask_block);
      CHECK((const char*)s.dvec >= (const char*)s.m.row_idx + nb * nb * 4, "D overlaps the block lists");
      CHECK((const char*)s.m.row_ptr == WS, "lists do not start the workspace");
    }
    before = fa::g_rec.launches;
    CHECK(fa_bwd(&p, Q, K, V, O, DO, (float*)L, DQ, DK, DV, WS, w1 - 4, nullptr) == FA_ERR_WORKSPACE, "short bwd ws");
    CHECK(fa_bwd_dq(&p, Q, K, V, O, DO, (float*)L, DQ, WS, w1, nullptr) == FA_ERR_ARG, "dq stage took the flag");
    CHECK(fa_bwd_dkdv(&p, Q, K, V, DO, (float*)L, DK, DV, WS, w1, nullptr) == FA_ERR_ARG, "dkdv stage took the flag");
    CHECK(fa::g_rec.launches == before, "rejected bwd calls launched");
  } else {
    const size_t dbytes = (size_t)p.B * p.H * p.N * 4;
    const float* dvec = p.dtype == FA_F32 ? fa::g_rec.f32.dvec : fa::g_rec.dq.dvec;
    CHECK(inside(dvec, dbytes, WS, w1),
          "D outside the workspace: B=%d H=%d N=%d d=%d dtype=%d mask=%p mb=%d w1=%zu D at +%td",
          p.B, p.H, p.N, p.d, p.dtype, (const void*)p.block_mask, p.mask_block, w1,
          (const char*)dvec - WS);
    if (p.dtype != FA_F32) CHECK(fa::g_rec.dq.dvec == fa::g_rec.dkdv.dvec, "stages disagree on D");
    if (lists) {
      if (!(p.flags & FA_REUSE_LISTS)) check_lists(p, WS, w1, "fa_bwd");
      const size_t nb = (size_t)(p.N / p.mask_block);
      const char* lend = (const char*)fa::g_rec.dq.m.row_idx + nb * nb * 4;
      CHECK((const char*)fa::g_rec.dq.dvec >= lend, "D overlaps the block lists");
      CHECK(fa::g_rec.dq.m.row_ptr == fa::g_rec.dkdv.m.row_ptr, "stages disagree on the lists");
      CHECK((const char*)fa::g_rec.dq.m.row_ptr == WS, "lists do not start the workspace");
    }
    before = fa::g_rec.launches;
    CHECK(fa_bwd(&p, Q, K, V, O, DO, (float*)L, DQ, DK, DV, WS, w1 - 4, nullptr) == FA_ERR_WORKSPACE, "short bwd ws");
    CHECK(fa_bwd(&p, Q, K, V, O, DO, (float*)L, DQ, DK, DV, WS + 16 + 8, w1, nullptr) == FA_ERR_WORKSPACE, "misaligned bwd ws");
    CHECK(fa_bwd_dq(&p, Q, K, V, nullptr, DO, (float*)L, DQ, WS, w1, nullptr) == FA_ERR_ARG, "null o");
    CHECK(fa_bwd_dkdv(&p, Q, K, V, DO, (float*)L, DK, nullptr, WS, w1, nullptr) == FA_ERR_ARG, "null dv");
    CHECK(fa::g_rec.launches == before, "rejected bwd calls launched");
  }

  // decode shape
  const int32_t nqs[] = {1, 3, p.N, (p.N > 0 && p.N < std::numeric_limits<int32_t>::max()) ? p.N + 1 : 1, 0};
  for (int32_t nq : nqs) {
    const size_t wd = fa_decode_workspace_size(&p, nq);
    CHECK(wd % 256 == 0, "decode workspace not 256-aligned");
    before = fa::g_rec.launches;
    st = fa_fwd_decode(&p, nq, Q, K, V, O, (float*)L, WS, wd, nullptr);
    if (st != FA_OK) {
      CHECK(fa::g_rec.launches == before, "fa_fwd_decode returned %d after launching", st);
      CHECK(wd == 0, "decode workspace size for a rejected problem");
      continue;
    }
    const fa::DecParams& d = fa::g_rec.dec;
    CHECK(d.nsplit >= 1 && d.tiles_per_split >= 1 && (int64_t)d.nsplit * d.tiles_per_split >= d.ntiles &&
              (int64_t)(d.nsplit - 1) * d.tiles_per_split < d.ntiles,
          "decode splits do not cover the tiles once");
    if (d.nsplit > 1) {
      const size_t rows = (size_t)p.B * p.H * nq;
      CHECK(inside(d.part_o, rows * d.nsplit * p.d * 4, WS, wd), "decode partials outside");
      CHECK(inside(d.part_lse, rows * d.nsplit * 4, WS, wd), "decode LSE partials outside");
      CHECK((const char*)d.part_lse >= (const char*)d.part_o + rows * d.nsplit * p.d * 4, "partials overlap");
      CHECK(fa_fwd_decode(&p, nq, Q, K, V, O, (float*)L, WS, wd - 4, nullptr) == FA_ERR_WORKSPACE, "short decode ws");
    } else {
      CHECK(wd == 0, "one split needs no workspace");
    }
    // the no-allocation entry: beyond the static scratch it must refuse
    // before touching the GPU; below it, it would need the device (not here)
    if (wd > ((size_t)64 << 20)) {
      before = fa::g_rec.launches;
      CHECK(fa_fwd_decode_noalloc(&p, nq, Q, K, V, O, (float*)L, nullptr) == FA_ERR_SCRATCH, "scratch limit");
      CHECK(fa::g_rec.launches == before, "noalloc launched past its limit");
    }
    CHECK(fa_fwd_decode_noalloc(&p, nq, nullptr, K, V, O, (float*)L, nullptr) == FA_ERR_ARG, "noalloc null q");
  }

  // FP8
  const size_t w8 = fa_fp8_workspace_size(&p);
  CHECK(w8 % 256 == 0, "fp8 workspace not 256-aligned");
  char* S = fake(11);
  before = fa::g_rec.launches;
  st = fa_fp8_quantize(&p, (const float*)S, Q, K, V, WS, w8, nullptr);
  if (st != FA_OK) {
    CHECK(fa::g_rec.launches == before, "fa_fp8_quantize returned %d after launching", st);
  } else {
    const fa::Fp8QuantParams& q = fa::g_rec.q8;
    const size_t n64 = (size_t)(p.N + 63) / 64 * 64, hq = (size_t)p.B * p.H;
    const size_t hk = (size_t)p.B * (p.H_kv ? p.H_kv : p.H);
    CHECK(inside(q.c0, hq * n64 * p.d, WS, w8) && inside(q.c1, hk * n64 * p.d, WS, w8) &&
              inside(q.c2, hk * n64 * p.d, WS, w8) && inside(q.e0, hq * n64 / 64, WS, w8) &&
              inside(q.e1, hk * n64 / 64, WS, w8) && inside(q.e2, hk * n64 / 64, WS, w8),
          "fp8 regions outside the workspace");
    CHECK((char*)q.c1 >= (char*)q.c0 + hq * n64 * p.d && (char*)q.c2 >= (char*)q.c1 + hk * n64 * p.d &&
              (char*)q.e0 >= (char*)q.c2 + hk * n64 * p.d && (char*)q.e1 >= (char*)q.e0 + hq * n64 / 64 &&
              (char*)q.e2 >= (char*)q.e1 + hk * n64 / 64,
          "fp8 regions overlap");
    CHECK(q.nq_wg + 2 * (int64_t)q.nk_wg == fa::g_rec.q8_wgs, "quantiser grid");
    before = fa::g_rec.launches;
    CHECK(fa_fwd_fp8(&p, (const float*)S, WS, w8, O, (float*)L, nullptr) == FA_OK, "fp8 attention");
    const fa::Fp8FwdParams& f = fa::g_rec.f8;
    CHECK(f.qc == q.c0 && f.kc == q.c1 && f.vc == q.c2 && f.qe == q.e0 && f.ke == q.e1 && f.ve == q.e2,
          "fp8 attention reads other regions than the quantiser wrote");
    CHECK(fa_fwd_fp8(&p, (const float*)S, WS, w8 - 1, O, (float*)L, nullptr) == FA_ERR_WORKSPACE, "short fp8 ws");
    CHECK(fa_fp8_quantize(&p, (const float*)(S + 2), Q, K, V, WS, w8, nullptr) == FA_ERR_ARG, "misaligned signs");
  }
}

}  // namespace

int main(int argc, char** argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 200000;
  long valid = 0;
  for (long i = 0; i < iters; ++i) {
    const fa_problem p = random_problem();
    const long before = fa::g_rec.launches;
    one(p);
    valid += fa::g_rec.launches > before;
  }
  printf("abi_fuzz: %ld problems, %ld with launches, %ld launches recorded, %ld failures\n", iters, valid,
         fa::g_rec.launches, g_failures);
  return g_failures == 0 ? 0 : 1;
}
