// Record of the last kernel launch the host side of the C ABI asked for, kept by
// the stand-in launchers in api_stubs.cpp.
#pragma once

#include "fa2_internal.h"

namespace stub {

struct Record {
  int calls = 0;            // launcher calls so far
  const char* kind = "";    // which launcher ran last
  fa2::FwdParams fwd{};     // launch_fwd, launch_splitkv_partial / _merge
  int config = -1;          // launch_fwd's configuration
  fa2::BwdParams bwd{};     // launch_bwd
  fa2::Fp8Params fp8{};     // launch_fwd_fp8, launch_decode_fp8
  fa2::QuantParams quant{}; // launch_quantize_fp8
  hipError_t result = hipSuccess;  // what every launcher returns
  int num_cus = 256;        // what the device query reports; <= 0: the query fails
};

extern Record rec;

}  // namespace stub
