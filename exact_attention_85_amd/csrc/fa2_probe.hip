// Dispatch-order probe: which XCD (chiplet) and which compute unit each
// workgroup of a launch runs on.  The forward kernels' XCD-aware renumbering
// (xcd_remap) assumes that workgroup ids are dealt to the 8 XCDs in turn; this
// records what the hardware does, so that the assumption can be checked.
#include <hip/hip_runtime.h>

#include "fa2_internal.h"

namespace fa2 {
namespace {

// Hardware registers read with s_getreg_b32: XCC_ID (id 20) bits 3:0 hold the
// XCD of the wave; HW_ID (id 4) holds the wave's slot, SIMD and compute unit.
constexpr int kHwregXccId = (3 << 11) | 20;
constexpr int kHwregHwId = (31 << 11) | 4;

__global__ void __launch_bounds__(64) xcc_probe_kernel(int* out, int n) {
  const int i = blockIdx.x;
  if (threadIdx.x == 0 && i < n) {
    out[2 * i] = __builtin_amdgcn_s_getreg(kHwregXccId);
    out[2 * i + 1] = __builtin_amdgcn_s_getreg(kHwregHwId);
  }
}

}  // namespace

hipError_t launch_xcc_probe(int* out, int n, hipStream_t stream) {
  hipLaunchKernelGGL(xcc_probe_kernel, dim3((unsigned)n), dim3(64), 0, stream, out, n);
  return hipGetLastError();
}

}  // namespace fa2
