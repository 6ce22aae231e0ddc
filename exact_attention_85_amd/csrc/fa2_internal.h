// Internal interface between the host API (argument validation, dispatch) and
// the HIP kernels.  Not installed; callers use include/fa2.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {

// Arguments of one forward (or split-KV partial) launch.  Pointers are device
// pointers; sizes were validated by the host API.
struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;       // bf16 output (forward mode)
  float* lse;        // fp32 natural-log LSE (forward mode)
  float* ws_acc;     // split mode: [S][R][d] unnormalised accumulators
  float* ws_m;       // split mode: [S][R] chunk reference maxima (natural-log units)
  float* ws_l;       // split mode: [S][R] sums of the probabilities as accumulated in acc
  float* ws_ll;      // split mode: [S][R] fp32 sums of the probabilities (for LSE)
  int B, H, n_q, n_k, d;
  int wl, wr;        // key band [i - wl, i + wr] of query i (top-left aligned); -1: unbounded.
                     // Plain attention is (-1, -1), the causal mask (-1, 0).
  float scale;
  int num_splits;    // 1 in forward mode
  int split_len;     // keys per chunk (N_k in forward mode)
};

// Forward: O, LSE.  Returns hipSuccess or the launch error.
hipError_t launch_fwd(const FwdParams& p, hipStream_t stream);

// Split-KV pass 1 (partials into the workspace) and pass 2 (merge into O, LSE).
hipError_t launch_splitkv_partial(const FwdParams& p, hipStream_t stream);
hipError_t launch_splitkv_merge(const FwdParams& p, hipStream_t stream);

}  // namespace fa2
