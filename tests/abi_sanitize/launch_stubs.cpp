// Stand-ins for the kernel launchers, for the host-only sanitizer build of
// the C ABI (fa_api.hip): each records the parameters it was given and
// returns success without touching a GPU, so a driver can check what the
// argument checks and workspace layout hand to the kernels.
#include "launch_stubs.h"

namespace fa {

Recorded g_rec;

hipError_t launch_fwd(const FwdParams& p, int, int, bool, bool, hipStream_t) {
  ++g_rec.launches;
  g_rec.fwd = p;
  return hipSuccess;
}
hipError_t launch_fwd_drop(const FwdParams& p, int, int, bool, bool, hipStream_t) {
  ++g_rec.launches;
  g_rec.fwd = p;
  return hipSuccess;
}
hipError_t launch_bwd_dq(const BwdParams& p, int, int, bool, bool, hipStream_t) {
  ++g_rec.launches;
  g_rec.dq = p;
  return hipSuccess;
}
hipError_t launch_bwd_dq_drop(const BwdParams& p, int, int, bool, bool, hipStream_t) {
  ++g_rec.launches;
  g_rec.dq = p;
  return hipSuccess;
}
hipError_t launch_bwd_dkdv(const BwdParams& p, int, int, bool, bool, hipStream_t) {
  ++g_rec.launches;
  g_rec.dkdv = p;
  return hipSuccess;
}
hipError_t launch_bwd_dkdv_drop(const BwdParams& p, int, int, bool, bool, hipStream_t) {
  ++g_rec.launches;
  g_rec.dkdv = p;
  return hipSuccess;
}
hipError_t launch_bwd_single_pass(const BwdParams& p, int, int, bool, bool, hipStream_t) {
  ++g_rec.launches;
  g_rec.single = p;
  return hipSuccess;
}
hipError_t launch_decode(const DecParams& p, int, int, bool, hipStream_t) {
  ++g_rec.launches;
  g_rec.dec = p;
  return hipSuccess;
}
hipError_t launch_fp8_quantize(const Fp8QuantParams& p, int, int, int wgs, hipStream_t) {
  ++g_rec.launches;
  g_rec.q8 = p;
  g_rec.q8_wgs = wgs;
  return hipSuccess;
}
hipError_t launch_fp8_fwd(const Fp8FwdParams& p, int, int, bool, hipStream_t) {
  ++g_rec.launches;
  g_rec.f8 = p;
  return hipSuccess;
}
hipError_t launch_f32_fwd(const F32Params& p, hipStream_t) {
  ++g_rec.launches;
  g_rec.f32 = p;
  return hipSuccess;
}
hipError_t launch_f32_dq(const F32Params& p, hipStream_t) {
  ++g_rec.launches;
  g_rec.f32 = p;
  return hipSuccess;
}
hipError_t launch_f32_dkdv(const F32Params& p, hipStream_t) {
  ++g_rec.launches;
  g_rec.f32 = p;
  return hipSuccess;
}
hipError_t launch_mask_compile(const uint8_t* mask, int nb, int32_t* row_ptr, int32_t* col_idx,
                               int32_t* col_ptr, int32_t* row_idx, hipStream_t) {
  ++g_rec.launches;
  ++g_rec.mask_compiles;
  g_rec.mask = mask;
  g_rec.nb = nb;
  g_rec.lists[0] = row_ptr;
  g_rec.lists[1] = col_idx;
  g_rec.lists[2] = col_ptr;
  g_rec.lists[3] = row_idx;
  return hipSuccess;
}

}  // namespace fa
