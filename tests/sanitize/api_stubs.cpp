// Stand-ins for the kernel launchers and the two device queries that the host
// side of the C ABI calls, so that fa2_api.cpp builds with g++ under the
// address and undefined-behaviour sanitizers and runs without a GPU.  Each
// launcher records its parameter block and returns stub::rec.result.
#include "api_stubs.h"

namespace stub {
Record rec;
}

namespace fa2 {

hipError_t launch_fwd(const FwdParams& p, int config, hipStream_t) {
  stub::rec.kind = "fwd";
  stub::rec.fwd = p;
  stub::rec.config = config;
  ++stub::rec.calls;
  return stub::rec.result;
}

hipError_t launch_splitkv_partial(const FwdParams& p, hipStream_t) {
  stub::rec.kind = "splitkv_partial";
  stub::rec.fwd = p;
  ++stub::rec.calls;
  return stub::rec.result;
}

hipError_t launch_splitkv_merge(const FwdParams& p, hipStream_t) {
  stub::rec.kind = "splitkv_merge";
  stub::rec.fwd = p;
  ++stub::rec.calls;
  return stub::rec.result;
}

hipError_t launch_bwd(const BwdParams& p, hipStream_t) {
  stub::rec.kind = "bwd";
  stub::rec.bwd = p;
  ++stub::rec.calls;
  return stub::rec.result;
}

hipError_t launch_fwd_fp8(const Fp8Params& p, hipStream_t) {
  stub::rec.kind = "fwd_fp8";
  stub::rec.fp8 = p;
  ++stub::rec.calls;
  return stub::rec.result;
}

hipError_t launch_quantize_fp8(const QuantParams& p, hipStream_t) {
  stub::rec.kind = "quantize_fp8";
  stub::rec.quant = p;
  ++stub::rec.calls;
  return stub::rec.result;
}

hipError_t launch_decode_fp8(const Fp8Params& p, hipStream_t) {
  stub::rec.kind = "decode_fp8";
  stub::rec.fp8 = p;
  ++stub::rec.calls;
  return stub::rec.result;
}

hipError_t launch_fwd_blockmask(const FwdParams& p, hipStream_t) {
  stub::rec.kind = "fwd_blockmask";
  stub::rec.fwd = p;
  ++stub::rec.calls;
  return stub::rec.result;
}

hipError_t launch_xcc_probe(int*, int, hipStream_t) {
  stub::rec.kind = "xcc_probe";
  ++stub::rec.calls;
  return stub::rec.result;
}

}  // namespace fa2

extern "C" hipError_t hipGetDevice(int* device) {
  *device = 0;
  return stub::rec.num_cus > 0 ? hipSuccess : hipErrorNoDevice;
}

extern "C" hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int) {
  if (stub::rec.num_cus <= 0 || attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  *value = stub::rec.num_cus;
  return hipSuccess;
}
