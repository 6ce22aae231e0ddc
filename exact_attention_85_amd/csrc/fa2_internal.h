// Internal interface between the host API (argument validation, dispatch) and
// the HIP kernels.  Not installed; callers use include/fa2.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {

// Workgroup order of the forward kernels (FwdParams::sched bits).
//   kSchedRemap   renumber workgroup ids with xcd_remap (each XCD a contiguous range);
//                 without it, id i runs on XCD i % 8 as dispatched.
//   kSchedQbMajor logical ids run over (query block, batch*head) with the query block
//                 slowest: under a causal-like band the heaviest block of every head
//                 is dispatched before any lighter one.  Without a remap and with
//                 B*H a multiple of 8, XCD x then serves the heads h = x (mod 8).
//                 Otherwise ids run head by head (all blocks of one head together).
constexpr int kSchedRemap = 1;
constexpr int kSchedQbMajor = 2;

// Arguments of one forward (or split-KV partial) launch.  Pointers are device
// pointers; sizes were validated by the host API.
struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;       // bf16 output (forward mode)
  float* lse;        // fp32 natural-log LSE (forward mode)
  float* ws_acc;     // split mode: [S][R][d] l * (the chunk's normalised output)
  float* ws_m;       // split mode: [S][R] chunk reference levels (natural-log units)
  float* ws_l;       // split mode: [S][R] fp32 sums of exp(s - m)
  int B, H, n_q, n_k, d;
  int wl, wr;        // key band [i - wl, i + wr] of query i (top-left aligned); -1: unbounded.
                     // Plain attention is (-1, -1), the causal mask (-1, 0).
  float scale;
  int num_splits;    // 1 in forward mode
  int split_len;     // keys per chunk (N_k in forward mode)
  int sched;         // workgroup order bits (kSchedRemap, kSchedQbMajor)
  // block-sparse forward: byte mask [Mb][Mh][ceil(N_q/128)][bm_n_kb], one entry per 128-row
  // query block and 64-key tile; strides in entries, 0 for a shared (size-1) dimension
  const uint8_t* bmask;
  long long bm_stride_b, bm_stride_h;
  int bm_n_kb;
};

// Rows and keys per block-mask entry (the 4-wave kernel's query block and key tile).
constexpr int kMaskBlockQ = 128;
constexpr int kMaskBlockK = 64;

// Forward kernel configurations (fa2_fwd_config): the kernel and the workgroup order.
//   kernel 0: 4 waves, 128 query rows per workgroup, two workgroups per compute unit
//   kernel 1: 8 waves, 256 query rows, ping-pong of matrix and vector phases
//   kernel 2: 8 waves, 256 query rows, the tile loop of kernel 0 (every wave in step)
struct FwdConfig {
  int kernel;
  int sched;
  const char* name;
};
constexpr int kNumFwdConfigs = 10;
extern const FwdConfig kFwdConfigs[kNumFwdConfigs];

// The configuration fa2_fwd takes for a shape (the measured table in fa2_tune_table.h).
int fwd_default_config(int d, bool banded, int n_q, long long n_bh);

// Arguments of the backward launches.  dq, dk, dv are bf16 outputs; the
// workspace holds l2vec [R] (LSE * log2 e) and dvec [R] (minus rowsum dO * O),
// R = B*H*N_q.
struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* l2vec;
  float* dvec;
  int B, H, n_q, n_k, d;
  int causal;
  float scale;
};

// Arguments of the FP8 forward: e4m3 codes of Q, K (row layout) and V
// (transposed, row stride vt_stride), per-(batch, head) descales.
struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* vt;  // forward: V transposed [B][H][d][vt_stride]
  const uint8_t* v;   // decode: V in row layout [B][H][N_k][d]
  const float* dsq;
  const float* dsk;
  const float* dsv;
  uint16_t* o;
  float* lse;
  int B, H, n_q, n_k, d, vt_stride;
  int wl, wr;
  float scale;
};

// Arguments of the quantiser; descale holds the amax bit patterns between its kernels.
struct QuantParams {
  const uint16_t* x;
  uint8_t* codes;
  float* descale;
  int B, H, n, d;
  int transposed;
  int vt_stride;
};

// Split-KV forward, host side (fa2_api.cpp): every check of fa2_fwd_splitkv except those of the
// workspace, with no HIP call (returns FA2_OK or a negative fa2_status); then the two passes
// over an fp32 workspace of fa2_splitkv_workspace_bytes() bytes (FA2_OK or FA2_ERR_HIP).
int splitkv_check_args(const void* Q, const void* K, const void* V, const void* O, const float* LSE, int B, int H,
                       int N_q, int N_k, int d, float scale, int num_splits);
int splitkv_run(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q, int N_k,
                int d, int causal, float scale, int num_splits, float* ws, void* stream);

// Forward: O, LSE, with configuration `config` (0 .. kNumFwdConfigs - 1; N_q == 1 always
// takes the decode kernel).  Returns hipSuccess or the launch error.
hipError_t launch_fwd(const FwdParams& p, int config, hipStream_t stream);

// Block-sparse forward (p.bmask set): the 4-wave kernel with the workgroup order in p.sched.
hipError_t launch_fwd_blockmask(const FwdParams& p, hipStream_t stream);

// Split-KV pass 1 (partials into the workspace) and pass 2 (merge into O, LSE).
hipError_t launch_splitkv_partial(const FwdParams& p, hipStream_t stream);
hipError_t launch_splitkv_merge(const FwdParams& p, hipStream_t stream);

// Backward: D and LSE*log2e, then dK and dV (one pass over the key blocks), then dQ (one
// pass over the query blocks).
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);

// Dispatch-order probe: out[2i] = XCD id, out[2i + 1] = hardware id word of workgroup i.
hipError_t launch_xcc_probe(int* out, int n, hipStream_t stream);

// FP8 forward and the quantiser that prepares its inputs.
hipError_t launch_fwd_fp8(const Fp8Params& p, hipStream_t stream);
hipError_t launch_quantize_fp8(const QuantParams& p, hipStream_t stream);
hipError_t launch_decode_fp8(const Fp8Params& p, hipStream_t stream);

}  // namespace fa2
