// Parameters recorded by the stand-in launchers (launch_stubs.cpp).
#pragma once

#include "../../io_aware_exact_fwd_amd/csrc/fa_kernels.hpp"

namespace fa {

struct Recorded {
  long launches = 0;
  long mask_compiles = 0;
  FwdParams fwd;
  BwdParams dq, dkdv, single;  // single: the single-pass backward's launch
  DecParams dec;
  Fp8QuantParams q8;
  int q8_wgs = 0;
  Fp8FwdParams f8;
  F32Params f32;
  const uint8_t* mask = nullptr;
  int nb = 0;
  int32_t* lists[4] = {nullptr, nullptr, nullptr, nullptr};
};

extern Recorded g_rec;

}  // namespace fa
