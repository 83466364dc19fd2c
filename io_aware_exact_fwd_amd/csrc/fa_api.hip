// fa_api.hip -- the C ABI of libfa_mi355x (declared in include/fa.h):
// argument checking, workspace layout, and dispatch to the kernels on the
// caller's stream.  No allocation, no synchronisation, no state.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace {

constexpr int kVersion = 1 * 10000 + 6 * 100 + 0;

// Size of the static scratch of fa_fwd_decode_noalloc (include/fa.h).
constexpr size_t kScratchBytes = (size_t)64 << 20;

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == FA_F32 ? 4 : 2; }

bool uses_lists(const fa_problem* p) { return p->block_mask != nullptr && p->dtype != FA_F32; }

int kv_heads(const fa_problem* p) { return p->H_kv == 0 ? p->H : p->H_kv; }

int group_of(const fa_problem* p) { return p->H / kv_heads(p); }

int check_problem(const fa_problem* p) {
  if (!p) return FA_ERR_ARG;
  if (p->B <= 0 || p->H <= 0 || p->N <= 0 || p->d <= 0) return FA_ERR_ARG;
  if (!isfinite(p->scale) || !(p->scale > 0.f)) return FA_ERR_ARG;
  if (p->causal != 0 && p->causal != 1) return FA_ERR_ARG;
  if (p->window < 0) return FA_ERR_ARG;
  if (p->H_kv < 0 || (p->H_kv > 0 && p->H % p->H_kv != 0)) return FA_ERR_ARG;
  if (!(p->dropout_p >= 0.f && p->dropout_p < 1.f)) return FA_ERR_ARG;
  if ((p->flags & ~(FA_REUSE_LISTS | FA_BWD_ATOMIC_DQ)) != 0) return FA_ERR_ARG;
  if (p->dtype != FA_F32 && p->dtype != FA_F16 && p->dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (p->d != 64 && p->d != 128) return FA_ERR_UNSUPPORTED;
  // one head must be addressable with 32-bit byte offsets
  if ((int64_t)p->N * p->d * elem_bytes(p->dtype) > (int64_t)INT32_MAX) return FA_ERR_UNSUPPORTED;
  // workgroup counts (heads x 64-row tiles) must fit a 32-bit grid; both
  // factors are below 2^31 here, so the product fits 64 bits
  const int64_t heads = (int64_t)p->B * p->H;
  if (heads > (int64_t)INT32_MAX || heads * ((p->N + 63) / 64) > (int64_t)INT32_MAX)
    return FA_ERR_UNSUPPORTED;
  if (p->block_mask) {
    if (p->mask_block <= 0 || p->mask_block % 128 != 0) return FA_ERR_UNSUPPORTED;
    if (p->N % p->mask_block != 0) return FA_ERR_UNSUPPORTED;
  }
  return FA_OK;
}

size_t lists_bytes(const fa_problem* p) {
  if (!uses_lists(p)) return 0;
  const size_t nb = (size_t)(p->N / p->mask_block);
  return align_up((nb + 1) * 4) * 2 + align_up(nb * nb * 4) * 2;
}

size_t dvec_bytes(const fa_problem* p) {
  return align_up((size_t)p->B * p->H * p->N * sizeof(float));
}

// single-pass backward: the float32 dQ accumulator after D
bool single_pass(const fa_problem* p) { return (p->flags & FA_BWD_ATOMIC_DQ) != 0; }
size_t dqacc_bytes(const fa_problem* p) {
  if (!single_pass(p) || p->dtype == FA_F32) return 0;
  return align_up((size_t)p->B * p->H * p->N * p->d * sizeof(float));
}

struct Lists {
  int32_t *row_ptr, *col_idx, *col_ptr, *row_idx;
};

Lists carve_lists(const fa_problem* p, char* base) {
  const size_t nb = (size_t)(p->N / p->mask_block);
  Lists l;
  l.row_ptr = (int32_t*)base;
  base += align_up((nb + 1) * 4);
  l.col_ptr = (int32_t*)base;
  base += align_up((nb + 1) * 4);
  l.col_idx = (int32_t*)base;
  base += align_up(nb * nb * 4);
  l.row_idx = (int32_t*)base;
  return l;
}

fa::MaskLists mask_lists(const fa_problem* p, const Lists& l) {
  fa::MaskLists m;
  m.row_ptr = l.row_ptr;
  m.col_idx = l.col_idx;
  m.col_ptr = l.col_ptr;
  m.row_idx = l.row_idx;
  m.mask_block = p->mask_block;
  return m;
}

// Dropout constants: t8 = floor(256 p) of the float32 p (exact: scaling by
// 256 is exact), keep scale 256 / (256 - t8).  t8 = 0 means no dropout.
fa::DropParams drop_params(const fa_problem* p) {
  fa::DropParams d;
  d.t8 = (uint32_t)floorf(p->dropout_p * 256.0f);
  d.mult = 256.0f / (float)(256u - d.t8);
  d.k0 = (uint32_t)(p->seed & 0xFFFFFFFFu);
  d.k1 = (uint32_t)(p->seed >> 32);
  d.offset = p->offset;
  return d;
}

// Debug build only: the tile-visit counter array set by
// fa_debug_set_tile_visits (see include/fa_debug.h); null in production.
int32_t* g_debug_visits = nullptr;
int32_t* debug_visits() { return fa::kDebugBuild ? g_debug_visits : nullptr; }

fa::MaskLists no_lists() {
  fa::MaskLists m;
  m.row_ptr = m.col_idx = m.col_ptr = m.row_idx = nullptr;
  m.mask_block = 0;
  return m;
}

}  // namespace

extern "C" {

size_t fa_workspace_size(const fa_problem* p, int pass) {
  if (check_problem(p) != FA_OK) return 0;
  if (pass == 0) return lists_bytes(p);
  return lists_bytes(p) + dvec_bytes(p) + dqacc_bytes(p);
}

int fa_fwd(const fa_problem* p, const void* q, const void* k, const void* v, void* o, float* lse,
           void* workspace, size_t ws_bytes, hipStream_t stream) {
  int st = check_problem(p);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o || !lse) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3u))
    return FA_ERR_ARG;
  const size_t need = fa_workspace_size(p, 0);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned16(workspace))) return FA_ERR_WORKSPACE;
  hipStream_t s = stream;
  const float c = p->scale * fa::kLog2e;
  const int nheads = p->B * p->H;

  if (p->dtype == FA_F32) {
    fa::F32Params f = {};
    f.q = (const float*)q;
    f.k = (const float*)k;
    f.v = (const float*)v;
    f.out_o = (float*)o;
    f.lse = lse;
    f.block_mask = p->block_mask;
    f.mask_block = p->mask_block;
    f.N = p->N;
    f.nheads = nheads;
    f.d = p->d;
    f.causal = p->causal;
    f.window = p->window;
    f.group = group_of(p);
    f.c = c;
    f.scale = p->scale;
    f.drop = drop_params(p);
    return fa::launch_f32_fwd(f, s) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
  }

  fa::FwdParams f;
  f.q = q;
  f.k = k;
  f.v = v;
  f.o = o;
  f.lse = lse;
  f.N = p->N;
  f.nheads = nheads;
  f.nqt = (p->N + fa::kFwdRows - 1) / fa::kFwdRows;
  f.window = p->window;
  f.group = group_of(p);
  f.c = c;
  f.m = no_lists();
  f.drop = drop_params(p);
  f.visits = debug_visits();
  const bool masked = p->block_mask != nullptr;
  if (masked) {
    Lists l = carve_lists(p, (char*)workspace);
    if (!(p->flags & FA_REUSE_LISTS) &&
        fa::launch_mask_compile(p->block_mask, p->N / p->mask_block, l.row_ptr, l.col_idx,
                                l.col_ptr, l.row_idx, s) != hipSuccess)
      return FA_ERR_LAUNCH;
    f.m = mask_lists(p, l);
  }
  const hipError_t e = f.drop.t8 ? fa::launch_fwd_drop(f, p->dtype, p->d, p->causal != 0, masked, s)
                                 : fa::launch_fwd(f, p->dtype, p->d, p->causal != 0, masked, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// Decode geometry: rows per K/V head, row blocks, key tiles (of kDecKeys) and splits.  The
// split count aims at >= 1024 workgroups (4 per CU, two rounds of the two that
// fit in LDS; 512 and 2048 measured 2 % slower on decode_gqa) and depends only
// on the problem, so the workspace size is known before any launch.
struct DecodeShape {
  int rows, nrb, nkv, tile0, ntiles, tps, nsplit;
};

DecodeShape decode_shape(const fa_problem* p, int n_q) {
  DecodeShape g;
  const int group = group_of(p);
  g.rows = group * n_q;
  g.nrb = (g.rows + 127) / 128;
  g.nkv = p->B * kv_heads(p);
  // keys some row sees: the rows sit at positions N - n_q .. N - 1
  const int lo = p->window > 0 ? (p->N - n_q - p->window + 1 > 0 ? p->N - n_q - p->window + 1 : 0) : 0;
  g.tile0 = lo / fa::kDecKeys;
  g.ntiles = (p->N - 1) / fa::kDecKeys - g.tile0 + 1;
  const int64_t wgs = (int64_t)g.nkv * g.nrb;
  int want = (int)((1024 + wgs - 1) / wgs);
  if (want < 1) want = 1;
  if (want > g.ntiles) want = g.ntiles;
  g.tps = (g.ntiles + want - 1) / want;
  g.nsplit = (g.ntiles + g.tps - 1) / g.tps;
  return g;
}

int check_decode(const fa_problem* p, int32_t n_q) {
  int st = check_problem(p);
  if (st != FA_OK) return st;
  if (n_q < 1 || n_q > p->N) return FA_ERR_ARG;
  if (p->dtype == FA_F32 || p->block_mask != nullptr || p->dropout_p != 0.f)
    return FA_ERR_UNSUPPORTED;
  if ((int64_t)p->B * p->H * n_q > (int64_t)INT32_MAX / 128) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Argument checks shared by the two decode entry points.
int check_decode_call(const fa_problem* p, int32_t n_q, const void* q, const void* k,
                      const void* v, const void* o, const float* lse) {
  int st = check_decode(p, n_q);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o || !lse) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3u))
    return FA_ERR_ARG;
  return FA_OK;
}

// Enqueue the split and merge kernels; `workspace` holds the float32
// partials (unused when one split suffices).  Every partial slot that the
// merge reads is written by the split kernel first, so nothing needs clearing.
int run_decode(const fa_problem* p, int32_t n_q, const void* q, const void* k, const void* v,
               void* o, float* lse, void* workspace, hipStream_t stream) {
  const DecodeShape g = decode_shape(p, n_q);
  fa::DecParams d;
  d.q = q;
  d.k = k;
  d.v = v;
  d.o = o;
  d.lse = lse;
  const size_t rows = (size_t)p->B * p->H * n_q;
  d.part_o = g.nsplit > 1 ? (float*)workspace : nullptr;
  d.part_lse = g.nsplit > 1 ? (float*)((char*)workspace + align_up(rows * g.nsplit * p->d * sizeof(float)))
                            : nullptr;
  d.N = p->N;
  d.nq = n_q;
  d.rows = g.rows;
  d.nrb = g.nrb;
  d.nkv = g.nkv;
  d.nsplit = g.nsplit;
  d.tiles_per_split = g.tps;
  d.tile0 = g.tile0;
  d.ntiles = g.ntiles;
  d.window = p->window;
  d.c = p->scale * fa::kLog2e;
  return fa::launch_decode(d, p->dtype, p->d, p->causal != 0, stream) == hipSuccess
             ? FA_OK
             : FA_ERR_LAUNCH;
}

}  // namespace

// Scratch of fa_fwd_decode_noalloc: the float32 split partials of callers that
// cannot allocate.  Each GPU the library runs on holds its own copy for the
// life of the process.  In host code `scratch` names a host-side stand-in, not
// the device memory: host code uses only the device address that
// hipGetSymbolAddress returns for the current device (scratch_of_stream_device).
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// This device's address of `scratch`, looked up once per device (with that
// device current) on the first call that needs it.  The stream must belong to
// the current device (NULL: the current device's default stream).
int scratch_of_stream_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return FA_ERR_ARG;
    if (sdev != dev) return FA_ERR_ARG;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return FA_ERR_LAUNCH;
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_decode_workspace_size(const fa_problem* p, int32_t n_q) {
  if (check_decode(p, n_q) != FA_OK) return 0;
  const DecodeShape g = decode_shape(p, n_q);
  if (g.nsplit == 1) return 0;
  const size_t rows = (size_t)p->B * p->H * n_q;
  return align_up(rows * g.nsplit * p->d * sizeof(float)) + align_up(rows * g.nsplit * sizeof(float));
}

int fa_fwd_decode(const fa_problem* p, int32_t n_q, const void* q, const void* k, const void* v,
                  void* o, float* lse, void* workspace, size_t ws_bytes, hipStream_t stream) {
  int st = check_decode_call(p, n_q, q, k, v, o, lse);
  if (st != FA_OK) return st;
  const size_t need = fa_decode_workspace_size(p, n_q);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned16(workspace))) return FA_ERR_WORKSPACE;
  return run_decode(p, n_q, q, k, v, o, lse, workspace, stream);
}

int fa_fwd_decode_noalloc(const fa_problem* p, int32_t n_q, const void* q, const void* k,
                          const void* v, void* o, float* lse, hipStream_t stream) {
  int st = check_decode_call(p, n_q, q, k, v, o, lse);
  if (st != FA_OK) return st;
  const size_t need = fa_decode_workspace_size(p, n_q);
  if (need > kScratchBytes) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_of_stream_device(stream, &ws);
    if (st != FA_OK) return st;
  }
  return run_decode(p, n_q, q, k, v, o, lse, ws, stream);
}

}  // extern "C"

namespace {

// FP8 workspace regions (see include/fa.h): codes of Q, K, V, then the block
// exponents of Q, K, V, each region 256-byte aligned.
struct Fp8Layout {
  size_t n64, qc, kc, vc, qe, ke, ve, total;
};

Fp8Layout fp8_layout(const fa_problem* p) {
  Fp8Layout l;
  l.n64 = (size_t)(p->N + 63) / 64 * 64;
  const size_t hq = (size_t)p->B * p->H, hk = (size_t)p->B * kv_heads(p);
  l.qc = 0;
  l.kc = l.qc + align_up(hq * l.n64 * p->d);
  l.vc = l.kc + align_up(hk * l.n64 * p->d);
  l.qe = l.vc + align_up(hk * l.n64 * p->d);
  l.ke = l.qe + align_up(hq * (l.n64 / 64));
  l.ve = l.ke + align_up(hk * (l.n64 / 64));
  l.total = l.ve + align_up(hk * (l.n64 / 64));
  return l;
}

int check_fp8(const fa_problem* p, const float* signs) {
  int st = check_problem(p);
  if (st != FA_OK) return st;
  if (!signs || ((uintptr_t)signs & 3u)) return FA_ERR_ARG;
  if (p->dtype == FA_F32 || p->block_mask != nullptr || p->dropout_p != 0.f) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_fp8_workspace_size(const fa_problem* p) {
  if (check_problem(p) != FA_OK || p->dtype == FA_F32 || p->block_mask || p->dropout_p != 0.f) return 0;
  return fp8_layout(p).total;
}

int fa_fp8_quantize(const fa_problem* p, const float* signs, const void* q, const void* k, const void* v,
                    void* workspace, size_t ws_bytes, hipStream_t stream) {
  int st = check_fp8(p, signs);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !aligned16(q) || !aligned16(k) || !aligned16(v)) return FA_ERR_ARG;
  const Fp8Layout l = fp8_layout(p);
  if (!workspace || ws_bytes < l.total || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  const int nblk = (int)(l.n64 / 64);
  fa::Fp8QuantParams qp;
  qp.x0 = q;
  qp.x1 = k;
  qp.x2 = v;
  qp.c0 = (uint8_t*)(ws + l.qc);
  qp.c1 = (uint8_t*)(ws + l.kc);
  qp.c2 = (uint8_t*)(ws + l.vc);
  qp.e0 = (int8_t*)(ws + l.qe);
  qp.e1 = (int8_t*)(ws + l.ke);
  qp.e2 = (int8_t*)(ws + l.ve);
  qp.signs = signs;
  qp.nq_wg = p->B * p->H * nblk;
  qp.nk_wg = p->B * kv_heads(p) * nblk;
  qp.N = p->N;
  qp.N64 = (int)l.n64;
  const int64_t wgs = (int64_t)qp.nq_wg + 2 * (int64_t)qp.nk_wg;
  if (wgs > (int64_t)INT32_MAX) return FA_ERR_UNSUPPORTED;
  return fa::launch_fp8_quantize(qp, p->dtype, p->d, (int)wgs, stream) == hipSuccess
             ? FA_OK
             : FA_ERR_LAUNCH;
}

int fa_fwd_fp8(const fa_problem* p, const float* signs, const void* workspace, size_t ws_bytes, void* o,
               float* lse, hipStream_t stream) {
  int st = check_fp8(p, signs);
  if (st != FA_OK) return st;
  if (!o || !lse || !aligned16(o) || ((uintptr_t)lse & 3u)) return FA_ERR_ARG;
  const Fp8Layout l = fp8_layout(p);
  if (!workspace || ws_bytes < l.total || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  const char* ws = (const char*)workspace;
  fa::Fp8FwdParams f;
  f.qc = (const uint8_t*)(ws + l.qc);
  f.kc = (const uint8_t*)(ws + l.kc);
  f.vc = (const uint8_t*)(ws + l.vc);
  f.qe = (const int8_t*)(ws + l.qe);
  f.ke = (const int8_t*)(ws + l.ke);
  f.ve = (const int8_t*)(ws + l.ve);
  f.signs = signs;
  f.o = o;
  f.lse = lse;
  f.N = p->N;
  f.N64 = (int)l.n64;
  f.nheads = p->B * p->H;
  f.nqt = (p->N + 127) / 128;
  f.window = p->window;
  f.group = group_of(p);
  f.c = p->scale * fa::kLog2e;
  return fa::launch_fp8_fwd(f, p->dtype, p->d, p->causal != 0, stream) == hipSuccess
             ? FA_OK
             : FA_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// Shared checks and parameter block of the backward entry points.  Pointers a
// stage does not use may be NULL; `need` lists which ones must be present.
int bwd_setup(const fa_problem* p, const void* q, const void* k, const void* v, const void* o,
              const void* dout, const float* lse, const void* dq, const void* dk, const void* dv,
              void* workspace, size_t ws_bytes, bool want_dq, bool want_dkdv,
              fa::BwdParams* b) {
  int st = check_problem(p);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !dout || !lse) return FA_ERR_ARG;
  if (want_dq && (!o || !dq)) return FA_ERR_ARG;
  if (want_dkdv && (!dk || !dv)) return FA_ERR_ARG;
  const void* ptrs[] = {q, k, v, dout, want_dq ? o : q, want_dq ? dq : q, want_dkdv ? dk : q,
                        want_dkdv ? dv : q};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA_ERR_ARG;
  if ((uintptr_t)lse & 3u) return FA_ERR_ARG;
  const size_t need = fa_workspace_size(p, 1);
  if (!workspace || ws_bytes < need || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  b->q = q;
  b->k = k;
  b->v = v;
  b->o = o;
  b->dout = dout;
  b->lse = lse;
  b->dq = const_cast<void*>(dq);
  b->dk = const_cast<void*>(dk);
  b->dv = const_cast<void*>(dv);
  b->dvec = (float*)((char*)workspace + lists_bytes(p));
  b->dqacc = dqacc_bytes(p) ? (float*)((char*)workspace + lists_bytes(p) + dvec_bytes(p)) : nullptr;
  b->N = p->N;
  b->nheads = p->B * p->H;
  b->window = p->window;
  b->group = group_of(p);
  b->c = p->scale * fa::kLog2e;
  b->scale = p->scale;
  b->m = no_lists();
  b->drop = drop_params(p);
  b->visits = debug_visits();
  if (p->block_mask) b->m = mask_lists(p, carve_lists(p, (char*)workspace));
  return FA_OK;
}

fa::F32Params f32_params(const fa_problem* p, const fa::BwdParams& b) {
  fa::F32Params f = {};
  f.q = (const float*)b.q;
  f.k = (const float*)b.k;
  f.v = (const float*)b.v;
  f.o = (const float*)b.o;
  f.dout = (const float*)b.dout;
  f.lse = (float*)b.lse;
  f.dq = (float*)b.dq;
  f.dk = (float*)b.dk;
  f.dv = (float*)b.dv;
  f.dvec = b.dvec;
  f.block_mask = p->block_mask;
  f.mask_block = p->mask_block;
  f.N = p->N;
  f.nheads = b.nheads;
  f.d = p->d;
  f.causal = p->causal;
  f.window = p->window;
  f.group = b.group;
  f.c = b.c;
  f.scale = p->scale;
  f.drop = b.drop;
  return f;
}

int run_dq(const fa_problem* p, fa::BwdParams b, hipStream_t s) {
  if (p->dtype == FA_F32)
    return fa::launch_f32_dq(f32_params(p, b), s) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
  const bool masked = p->block_mask != nullptr;
  if (masked && !(p->flags & FA_REUSE_LISTS) &&
      fa::launch_mask_compile(p->block_mask, p->N / p->mask_block,
                                        (int32_t*)b.m.row_ptr, (int32_t*)b.m.col_idx,
                                        (int32_t*)b.m.col_ptr, (int32_t*)b.m.row_idx,
                                        s) != hipSuccess)
    return FA_ERR_LAUNCH;
  b.ntiles = (p->N + fa::kFwdRows - 1) / fa::kFwdRows;
  const hipError_t e = b.drop.t8
                           ? fa::launch_bwd_dq_drop(b, p->dtype, p->d, p->causal != 0, masked, s)
                           : fa::launch_bwd_dq(b, p->dtype, p->d, p->causal != 0, masked, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// FA_BWD_ATOMIC_DQ: block lists (if any), then D, dK/dV with dQ by atomics,
// and the dQ conversion
int run_single_pass(const fa_problem* p, fa::BwdParams b, hipStream_t s) {
  if (p->dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  const bool masked = p->block_mask != nullptr;
  if (masked && !(p->flags & FA_REUSE_LISTS) &&
      fa::launch_mask_compile(p->block_mask, p->N / p->mask_block, (int32_t*)b.m.row_ptr,
                              (int32_t*)b.m.col_idx, (int32_t*)b.m.col_ptr,
                              (int32_t*)b.m.row_idx, s) != hipSuccess)
    return FA_ERR_LAUNCH;
  b.nheads = p->B * kv_heads(p);
  b.ntiles = (p->N + fa::kBwdKeys - 1) / fa::kBwdKeys;
  return fa::launch_bwd_single_pass(b, p->dtype, p->d, p->causal != 0, masked, s) == hipSuccess
             ? FA_OK
             : FA_ERR_LAUNCH;
}

int run_dkdv(const fa_problem* p, fa::BwdParams b, hipStream_t s) {
  b.nheads = p->B * kv_heads(p);  // one workgroup column per K/V head
  if (p->dtype == FA_F32)
    return fa::launch_f32_dkdv(f32_params(p, b), s) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
  b.ntiles = (p->N + fa::kBwdKeys - 1) / fa::kBwdKeys;
  const bool masked = p->block_mask != nullptr;
  const hipError_t e = b.drop.t8
                           ? fa::launch_bwd_dkdv_drop(b, p->dtype, p->d, p->causal != 0, masked, s)
                           : fa::launch_bwd_dkdv(b, p->dtype, p->d, p->causal != 0, masked, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_bwd(const fa_problem* p, const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv, void* workspace,
           size_t ws_bytes, hipStream_t stream) {
  fa::BwdParams b;
  int st = bwd_setup(p, q, k, v, o, dout, lse, dq, dk, dv, workspace, ws_bytes, true, true, &b);
  if (st != FA_OK) return st;
  if (single_pass(p)) return run_single_pass(p, b, stream);
  st = run_dq(p, b, stream);
  if (st != FA_OK) return st;
  return run_dkdv(p, b, stream);
}

int fa_bwd_dq(const fa_problem* p, const void* q, const void* k, const void* v, const void* o,
              const void* dout, const float* lse, void* dq, void* workspace, size_t ws_bytes,
              hipStream_t stream) {
  fa::BwdParams b;
  int st = bwd_setup(p, q, k, v, o, dout, lse, dq, nullptr, nullptr, workspace, ws_bytes, true,
                     false, &b);
  if (st != FA_OK) return st;
  if (single_pass(p)) return FA_ERR_ARG;  // a stage of the two-kernel backward only
  return run_dq(p, b, stream);
}

int fa_bwd_dkdv(const fa_problem* p, const void* q, const void* k, const void* v,
                const void* dout, const float* lse, void* dk, void* dv, void* workspace,
                size_t ws_bytes, hipStream_t stream) {
  fa::BwdParams b;
  int st = bwd_setup(p, q, k, v, nullptr, dout, lse, nullptr, dk, dv, workspace, ws_bytes, false,
                     true, &b);
  if (st != FA_OK) return st;
  if (single_pass(p)) return FA_ERR_ARG;  // a stage of the two-kernel backward only
  return run_dkdv(p, b, stream);
}

int fa_mask_compile(const uint8_t* mask, int32_t nb, int32_t* row_ptr, int32_t* col_idx,
                    int32_t* col_ptr, int32_t* row_idx, hipStream_t stream) {
  if (!mask || nb <= 0 || !row_ptr || !col_idx || !col_ptr || !row_idx) return FA_ERR_ARG;
  return fa::launch_mask_compile(mask, nb, row_ptr, col_idx, col_ptr, row_idx,
                                 stream) == hipSuccess
             ? FA_OK
             : FA_ERR_LAUNCH;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported problem";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_SCRATCH: return "problem needs more than the library's static scratch";
    default: return "unknown status";
  }
}

int fa_version(void) { return kVersion; }

#if FA_DEBUG_BUILD
int fa_debug_set_tile_visits(int32_t* visits) {
  g_debug_visits = visits;
  return FA_OK;
}
#endif

}  // extern "C"
