// Host side of the C ABI declared in include/fa2.h: argument validation (pure
// CPU, before any HIP call), kernel dispatch and status strings.
#include "fa2.h"

#include <math.h>
#include <stdint.h>

#include "fa2_internal.h"
#include "fa2_tune_table.h"

namespace {

constexpr long long kMaxGrid = (1LL << 31) - 1;
constexpr long long kMaxItems = (1LL << 32) - 1;  // work-items per grid dimension of one dispatch
constexpr long long kMaxHeadElems = (1LL << 30) - 1;  // one head's Q or K/V below 2^31 bytes
constexpr int kMaxWindow = 1 << 30;                   // keeps row +- window inside int

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range range_of(const void* p, long long bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

// Shapes, head dim and scale shared by both entry points.
int check_common(const void* Q, const void* K, const void* V, const void* O, const float* LSE, int B, int H,
                 int N_q, int N_k, int d, float scale) {
  if (!Q || !K || !V || !O || !LSE) return FA2_ERR_NULLPTR;
  if (B < 1 || H < 1 || N_q < 1 || N_k < 1) return FA2_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA2_ERR_HEAD_DIM;
  if ((long long)N_q * d > kMaxHeadElems || (long long)N_k * d > kMaxHeadElems) return FA2_ERR_BAD_SHAPE;
  if ((long long)B * H > kMaxGrid) return FA2_ERR_BAD_SHAPE;
  // |scale| * log2(e) must stay finite in fp32
  if (!isfinite(scale) || fabsf(scale) > 2.0e38f) return FA2_ERR_BAD_SCALE;
  return FA2_OK;
}

int check_alias(const void* Q, const void* K, const void* V, const void* O, const float* LSE, int B, int H, int N_q,
                int N_k, int d, const void* ws, size_t ws_bytes) {
  const long long bh = (long long)B * H;
  const Range q = range_of(Q, bh * N_q * d * 2), k = range_of(K, bh * N_k * d * 2),
              v = range_of(V, bh * N_k * d * 2);
  const Range o = range_of(O, bh * N_q * d * 2), l = range_of(LSE, bh * N_q * 4);
  if (overlap(o, q) || overlap(o, k) || overlap(o, v) || overlap(o, l)) return FA2_ERR_ALIAS;
  if (overlap(l, q) || overlap(l, k) || overlap(l, v)) return FA2_ERR_ALIAS;
  if (ws) {
    const Range w = range_of(ws, (long long)ws_bytes);
    if (overlap(w, q) || overlap(w, k) || overlap(w, v) || overlap(w, o) || overlap(w, l)) return FA2_ERR_ALIAS;
  }
  return FA2_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A 1-D launch of `blocks` workgroups of `threads` work-items fits one dispatch:
// below 2^31 workgroups and below 2^32 work-items (the dispatch packet's grid
// size is a 32-bit count of work-items).  blocks is checked first, so the
// product cannot overflow.
bool launch_fits(long long blocks, long long threads) { return blocks <= kMaxGrid && blocks * threads <= kMaxItems; }

// The launches of one forward (fa2_fwd, fa2_fwd_window, the FP8 forward): the
// 4-wave tile kernel takes ceil(N_q/128)*B*H workgroups of 256 work-items; the
// 8-wave kernel (256 rows, 512 work-items) and the single-row decode kernel
// (B*H workgroups of 256) never launch more work-items than that.
bool fwd_fits(int B, int H, int N_q) {
  return launch_fits((long long)((N_q + 127) / 128) * B * H, 256);
}

fa2::FwdParams make_params(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q,
                           int N_k, int d, int causal, float scale) {
  fa2::FwdParams p{};
  p.q = static_cast<const uint16_t*>(Q);
  p.k = static_cast<const uint16_t*>(K);
  p.v = static_cast<const uint16_t*>(V);
  p.o = static_cast<uint16_t*>(O);
  p.lse = LSE;
  p.B = B;
  p.H = H;
  p.n_q = N_q;
  p.n_k = N_k;
  p.d = d;
  p.wl = -1;
  p.wr = causal ? 0 : -1;
  p.scale = scale;
  p.num_splits = 1;
  p.split_len = N_k;
  p.sched = fa2::kSchedRemap;
  return p;
}

}  // namespace

namespace fa2 {

const FwdConfig kFwdConfigs[kNumFwdConfigs] = {
    {0, kSchedRemap, "tile128_remap_headmajor"},
    {0, kSchedRemap | kSchedQbMajor, "tile128_remap_qbmajor"},
    {0, 0, "tile128_noremap_headmajor"},
    {0, kSchedQbMajor, "tile128_noremap_qbmajor"},
    {1, kSchedRemap, "pingpong256_remap_headmajor"},
    {1, kSchedRemap | kSchedQbMajor, "pingpong256_remap_qbmajor"},
    {1, 0, "pingpong256_noremap_headmajor"},
    {1, kSchedQbMajor, "pingpong256_noremap_qbmajor"},
    {2, kSchedRemap, "tile256_remap_headmajor"},
    {2, kSchedQbMajor, "tile256_noremap_qbmajor"},
};

int fwd_default_config(int d, bool banded, int n_q, long long /*n_bh*/) {
  int best = 0, best_min = -1;
  for (const TuneRow& r : kTuneTable)
    if (r.d == d && r.banded == (banded ? 1 : 0) && r.nq_min <= n_q && r.nq_min > best_min) {
      best = r.config;
      best_min = r.nq_min;
    }
  return best;
}

int splitkv_check_args(const void* Q, const void* K, const void* V, const void* O, const float* LSE, int B, int H,
                       int N_q, int N_k, int d, float scale, int num_splits) {
  int rc = check_common(Q, K, V, O, LSE, B, H, N_q, N_k, d, scale);
  if (rc != FA2_OK) return rc;
  if (num_splits < 1 || num_splits > FA2_MAX_SPLITS || num_splits > N_k) return FA2_ERR_SPLITS;
  // partial pass: ceil(N_q/128)*B*H*S workgroups of 256 (tile kernel) or B*H*S of 256 (decode);
  // merge pass: one wave per query row, four rows per workgroup of 256
  if (!launch_fits((long long)((N_q + 127) / 128) * B * H * num_splits, 256) ||
      !launch_fits(((long long)B * H * N_q + 3) / 4, 256))
    return FA2_ERR_BAD_SHAPE;
  return check_alias(Q, K, V, O, LSE, B, H, N_q, N_k, d, nullptr, 0);
}

int splitkv_run(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q, int N_k,
                int d, int causal, float scale, int num_splits, float* ws, void* stream) {
  FwdParams p = make_params(Q, K, V, O, LSE, B, H, N_q, N_k, d, causal, scale);
  p.num_splits = num_splits;
  p.split_len = (N_k + num_splits - 1) / num_splits;
  const long long R = (long long)B * H * N_q;
  p.ws_acc = ws;
  p.ws_m = ws + (long long)num_splits * R * d;
  p.ws_l = p.ws_m + (long long)num_splits * R;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_splitkv_partial(p, s) != hipSuccess) return FA2_ERR_HIP;
  if (launch_splitkv_merge(p, s) != hipSuccess) return FA2_ERR_HIP;
  return FA2_OK;
}

}  // namespace fa2

extern "C" {

int fa2_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q, int N_k, int d,
            int causal, float scale, void* stream) {
  int rc = check_common(Q, K, V, O, LSE, B, H, N_q, N_k, d, scale);
  if (rc != FA2_OK) return rc;
  if (!fwd_fits(B, H, N_q)) return FA2_ERR_BAD_SHAPE;
  rc = check_alias(Q, K, V, O, LSE, B, H, N_q, N_k, d, nullptr, 0);
  if (rc != FA2_OK) return rc;
  const fa2::FwdParams p = make_params(Q, K, V, O, LSE, B, H, N_q, N_k, d, causal, scale);
  const int config = fa2::fwd_default_config(d, causal != 0, N_q, (long long)B * H);
  if (fa2::launch_fwd(p, config, static_cast<hipStream_t>(stream)) != hipSuccess) return FA2_ERR_HIP;
  return FA2_OK;
}

int fa2_fwd_window(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q,
                   int N_k, int d, int window_left, int window_right, float scale, void* stream) {
  int rc = check_common(Q, K, V, O, LSE, B, H, N_q, N_k, d, scale);
  if (rc != FA2_OK) return rc;
  if (window_left < -1 || window_right < -1 || window_left > kMaxWindow || window_right > kMaxWindow)
    return FA2_ERR_WINDOW;
  if (!fwd_fits(B, H, N_q)) return FA2_ERR_BAD_SHAPE;
  rc = check_alias(Q, K, V, O, LSE, B, H, N_q, N_k, d, nullptr, 0);
  if (rc != FA2_OK) return rc;
  fa2::FwdParams p = make_params(Q, K, V, O, LSE, B, H, N_q, N_k, d, 0, scale);
  p.wl = window_left;
  p.wr = window_right;
  const bool banded = window_left >= 0 || window_right >= 0;
  const int config = fa2::fwd_default_config(d, banded, N_q, (long long)B * H);
  if (fa2::launch_fwd(p, config, static_cast<hipStream_t>(stream)) != hipSuccess) return FA2_ERR_HIP;
  return FA2_OK;
}

int fa2_fwd_config(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q,
                   int N_k, int d, int window_left, int window_right, float scale, int config, void* stream) {
  int rc = check_common(Q, K, V, O, LSE, B, H, N_q, N_k, d, scale);
  if (rc != FA2_OK) return rc;
  if (window_left < -1 || window_right < -1 || window_left > kMaxWindow || window_right > kMaxWindow)
    return FA2_ERR_WINDOW;
  if (config < 0 || config >= fa2::kNumFwdConfigs) return FA2_ERR_CONFIG;
  if (!fwd_fits(B, H, N_q)) return FA2_ERR_BAD_SHAPE;
  rc = check_alias(Q, K, V, O, LSE, B, H, N_q, N_k, d, nullptr, 0);
  if (rc != FA2_OK) return rc;
  fa2::FwdParams p = make_params(Q, K, V, O, LSE, B, H, N_q, N_k, d, 0, scale);
  p.wl = window_left;
  p.wr = window_right;
  if (fa2::launch_fwd(p, config, static_cast<hipStream_t>(stream)) != hipSuccess) return FA2_ERR_HIP;
  return FA2_OK;
}

int fa2_fwd_blocksparse(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q,
                        int N_k, int d, const unsigned char* block_mask, int mask_batches, int mask_heads,
                        int window_left, int window_right, float scale, void* stream) {
  if (!block_mask) return FA2_ERR_NULLPTR;
  int rc = check_common(Q, K, V, O, LSE, B, H, N_q, N_k, d, scale);
  if (rc != FA2_OK) return rc;
  if (window_left < -1 || window_right < -1 || window_left > kMaxWindow || window_right > kMaxWindow)
    return FA2_ERR_WINDOW;
  if (!(mask_batches == 1 || mask_batches == B) || !(mask_heads == 1 || mask_heads == H)) return FA2_ERR_BAD_SHAPE;
  if (!fwd_fits(B, H, N_q)) return FA2_ERR_BAD_SHAPE;
  rc = check_alias(Q, K, V, O, LSE, B, H, N_q, N_k, d, nullptr, 0);
  if (rc != FA2_OK) return rc;
  const long long n_qb = (N_q + fa2::kMaskBlockQ - 1) / fa2::kMaskBlockQ;
  const long long n_kb = (N_k + fa2::kMaskBlockK - 1) / fa2::kMaskBlockK;
  const long long mask_bytes = (long long)mask_batches * mask_heads * n_qb * n_kb;
  const long long bh = (long long)B * H;
  const Range m = range_of(block_mask, mask_bytes);
  if (overlap(m, range_of(O, bh * N_q * d * 2)) || overlap(m, range_of(LSE, bh * N_q * 4))) return FA2_ERR_ALIAS;
  fa2::FwdParams p = make_params(Q, K, V, O, LSE, B, H, N_q, N_k, d, 0, scale);
  p.wl = window_left;
  p.wr = window_right;
  p.bmask = block_mask;
  p.bm_n_kb = (int)n_kb;
  p.bm_stride_h = mask_heads == 1 ? 0 : n_qb * n_kb;
  p.bm_stride_b = mask_batches == 1 ? 0 : (long long)mask_heads * n_qb * n_kb;
  // the workgroup order the tuned table picks for the shape (the masked kernel is the 4-wave one)
  const bool banded = window_left >= 0 || window_right >= 0;
  p.sched = fa2::kFwdConfigs[fa2::fwd_default_config(d, banded, N_q, bh)].sched;
  if (fa2::launch_fwd_blockmask(p, static_cast<hipStream_t>(stream)) != hipSuccess) return FA2_ERR_HIP;
  return FA2_OK;
}

int fa2_fwd_num_configs(void) { return fa2::kNumFwdConfigs; }

const char* fa2_fwd_config_name(int config) {
  if (config < 0 || config >= fa2::kNumFwdConfigs) return nullptr;
  return fa2::kFwdConfigs[config].name;
}

int fa2_fwd_default_config(int d, int banded, int N_q, int B, int H) {
  if (B < 1 || H < 1 || N_q < 1) return FA2_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA2_ERR_HEAD_DIM;
  return fa2::fwd_default_config(d, banded != 0, N_q, (long long)B * H);
}

size_t fa2_splitkv_workspace_bytes(int B, int H, int N_q, int d, int num_splits) {
  if (B < 1 || H < 1 || N_q < 1 || d < 1 || num_splits < 1 || num_splits > FA2_MAX_SPLITS) return 0;
  return (size_t)num_splits * (size_t)B * (size_t)H * (size_t)N_q * (size_t)(d + 2) * 4u;
}

int fa2_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q, int N_k,
                    int d, int causal, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                    void* stream) {
  int rc = fa2::splitkv_check_args(Q, K, V, O, LSE, B, H, N_q, N_k, d, scale, num_splits);
  if (rc != FA2_OK) return rc;
  const size_t need = fa2_splitkv_workspace_bytes(B, H, N_q, d, num_splits);
  if (!workspace || workspace_bytes < need) return FA2_ERR_WORKSPACE;
  rc = check_alias(Q, K, V, O, LSE, B, H, N_q, N_k, d, workspace, need);
  if (rc != FA2_OK) return rc;
  return fa2::splitkv_run(Q, K, V, O, LSE, B, H, N_q, N_k, d, causal, scale, num_splits,
                          static_cast<float*>(workspace), stream);
}

int fa2_num_splits(int B, int H, int N_q, int N_k, int d, int num_cus) {
  if (B < 1 || H < 1 || N_q < 1 || N_k < 1) return FA2_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA2_ERR_HEAD_DIM;
  if (num_cus <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || num_cus <= 0)
      return FA2_ERR_HIP;
  }
  // workgroups of the unsplit launch: one per (batch, head) for a single query
  // row (the streaming decode kernel), else one per 128-row query block
  const long long units = (long long)B * H * (N_q == 1 ? 1 : (N_q + 127) / 128);
  if (units >= num_cus) return 1;
  // split until the partial pass fills every compute unit once ...
  long long s = (num_cus + units - 1) / units;
  // ... or twice for the tile kernel (two workgroups share a compute unit),
  // which only pays while each chunk keeps at least 2048 keys
  const long long s2 = (2LL * num_cus + units - 1) / units;
  if (N_q > 1 && N_k / s2 >= 2048) s = s2;
  // chunks shorter than 512 keys spend more on the merge than they gain
  const long long cap = N_k / 512 > 1 ? N_k / 512 : 1;
  if (s > cap) s = cap;
  if (s > FA2_MAX_SPLITS) s = FA2_MAX_SPLITS;
  return (int)s;
}

size_t fa2_bwd_workspace_bytes(int B, int H, int N_q, int N_k, int d) {
  if (B < 1 || H < 1 || N_q < 1 || N_k < 1 || d < 1) return 0;
  const size_t R = (size_t)B * (size_t)H * (size_t)N_q;
  return 2 * R * 4u;  // LSE * log2(e) and D per query row
}

int fa2_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE, void* dQ,
            void* dK, void* dV, int B, int H, int N_q, int N_k, int d, int causal, float scale, void* workspace,
            size_t workspace_bytes, void* stream) {
  if (!dO || !dQ || !dK || !dV) return FA2_ERR_NULLPTR;
  // the forward's own checks on Q, K, V, O, LSE (LSE read-only here)
  int rc = check_common(Q, K, V, O, LSE, B, H, N_q, N_k, d, scale);
  if (rc != FA2_OK) return rc;
  // the two launches: the query blocks (one workgroup of 256 per 128 rows, or of 512 per 256
  // rows in the ping-pong form), then the key blocks (one workgroup of 512 per 128 keys)
  if (!launch_fits((long long)((N_k + 127) / 128) * B * H, 512) ||
      !launch_fits((long long)((N_q + 127) / 128) * B * H, 256) ||
      !launch_fits((long long)((N_q + 255) / 256) * B * H, 512))
    return FA2_ERR_BAD_SHAPE;
  const size_t need = fa2_bwd_workspace_bytes(B, H, N_q, N_k, d);
  if (!workspace || workspace_bytes < need) return FA2_ERR_WORKSPACE;
  // outputs must not overlap any input, each other or the workspace
  const long long bh = (long long)B * H;
  const Range in[6] = {range_of(Q, bh * N_q * d * 2), range_of(K, bh * N_k * d * 2), range_of(V, bh * N_k * d * 2),
                       range_of(O, bh * N_q * d * 2), range_of(dO, bh * N_q * d * 2), range_of(LSE, bh * N_q * 4)};
  const Range out[4] = {range_of(dQ, bh * N_q * d * 2), range_of(dK, bh * N_k * d * 2),
                        range_of(dV, bh * N_k * d * 2), range_of(workspace, (long long)need)};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlap(out[a], in[b])) return FA2_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (overlap(out[a], out[b])) return FA2_ERR_ALIAS;
  }
  fa2::BwdParams p{};
  p.q = static_cast<const uint16_t*>(Q);
  p.k = static_cast<const uint16_t*>(K);
  p.v = static_cast<const uint16_t*>(V);
  p.o = static_cast<const uint16_t*>(O);
  p.dout = static_cast<const uint16_t*>(dO);
  p.lse = LSE;
  p.dq = static_cast<uint16_t*>(dQ);
  p.dk = static_cast<uint16_t*>(dK);
  p.dv = static_cast<uint16_t*>(dV);
  const long long R = bh * N_q;
  float* ws = static_cast<float*>(workspace);
  p.l2vec = ws;
  p.dvec = ws + R;
  p.B = B;
  p.H = H;
  p.n_q = N_q;
  p.n_k = N_k;
  p.d = d;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  if (fa2::launch_bwd(p, static_cast<hipStream_t>(stream)) != hipSuccess) return FA2_ERR_HIP;
  return FA2_OK;
}

int fa2_fp8_vt_stride(int N_k) {
  if (N_k < 1 || N_k > (1 << 30)) return FA2_ERR_BAD_SHAPE;
  return (N_k + 15) / 16 * 16;
}

int fa2_quantize_fp8(const void* X, void* codes, float* descale, int B, int H, int N, int d, int transposed,
                     void* stream) {
  if (!X || !codes || !descale) return FA2_ERR_NULLPTR;
  if (B < 1 || H < 1 || N < 1) return FA2_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA2_ERR_HEAD_DIM;
  // two-dimensional launches (blocks per head, B*H): B*H is the y dimension, and with one head
  // below 2^30 elements no x dimension reaches 2^32 work-items
  if ((long long)N * d > kMaxHeadElems || (long long)B * H > 65535) return FA2_ERR_BAD_SHAPE;
  if (!aligned16(X) || !aligned16(codes) || !aligned16(descale)) return FA2_ERR_ALIGN;
  const long long bh = (long long)B * H;
  const int stride = fa2_fp8_vt_stride(N);
  const long long code_bytes = transposed ? bh * d * stride : bh * N * d;
  const Range x = range_of(X, bh * N * d * 2), c = range_of(codes, code_bytes), s = range_of(descale, bh * 4);
  if (overlap(c, x) || overlap(s, x) || overlap(s, c)) return FA2_ERR_ALIAS;
  fa2::QuantParams p{};
  p.x = static_cast<const uint16_t*>(X);
  p.codes = static_cast<uint8_t*>(codes);
  p.descale = descale;
  p.B = B;
  p.H = H;
  p.n = N;
  p.d = d;
  p.transposed = transposed ? 1 : 0;
  p.vt_stride = stride;
  if (fa2::launch_quantize_fp8(p, static_cast<hipStream_t>(stream)) != hipSuccess) return FA2_ERR_HIP;
  return FA2_OK;
}

int fa2_fwd_fp8(const void* Qc, const void* Kc, const void* Vt, const float* descale_q, const float* descale_k,
                const float* descale_v, void* O, float* LSE, int B, int H, int N_q, int N_k, int d, int causal,
                float scale, void* stream) {
  if (!descale_q || !descale_k || !descale_v) return FA2_ERR_NULLPTR;
  int rc = check_common(Qc, Kc, Vt, O, LSE, B, H, N_q, N_k, d, scale);
  if (rc != FA2_OK) return rc;
  if (!fwd_fits(B, H, N_q)) return FA2_ERR_BAD_SHAPE;
  const void* ptrs[8] = {Qc, Kc, Vt, descale_q, descale_k, descale_v, O, LSE};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA2_ERR_ALIGN;
  const long long bh = (long long)B * H;
  const int stride = fa2_fp8_vt_stride(N_k);
  const Range in[6] = {range_of(Qc, bh * N_q * d), range_of(Kc, bh * N_k * d), range_of(Vt, bh * d * stride),
                       range_of(descale_q, bh * 4), range_of(descale_k, bh * 4), range_of(descale_v, bh * 4)};
  const Range o = range_of(O, bh * N_q * d * 2), l = range_of(LSE, bh * N_q * 4);
  if (overlap(o, l)) return FA2_ERR_ALIAS;
  for (const Range& r : in)
    if (overlap(o, r) || overlap(l, r)) return FA2_ERR_ALIAS;
  fa2::Fp8Params p{};
  p.q = static_cast<const uint8_t*>(Qc);
  p.k = static_cast<const uint8_t*>(Kc);
  p.vt = static_cast<const uint8_t*>(Vt);
  p.dsq = descale_q;
  p.dsk = descale_k;
  p.dsv = descale_v;
  p.o = static_cast<uint16_t*>(O);
  p.lse = LSE;
  p.B = B;
  p.H = H;
  p.n_q = N_q;
  p.n_k = N_k;
  p.d = d;
  p.vt_stride = stride;
  p.wl = -1;
  p.wr = causal ? 0 : -1;
  p.scale = scale;
  if (fa2::launch_fwd_fp8(p, static_cast<hipStream_t>(stream)) != hipSuccess) return FA2_ERR_HIP;
  return FA2_OK;
}

int fa2_decode_fp8(const void* Qc, const void* Kc, const void* Vc, const float* descale_q, const float* descale_k,
                   const float* descale_v, void* O, float* LSE, int B, int H, int N_k, int d, float scale,
                   void* stream) {
  if (!descale_q || !descale_k || !descale_v) return FA2_ERR_NULLPTR;
  int rc = check_common(Qc, Kc, Vc, O, LSE, B, H, 1, N_k, d, scale);
  if (rc != FA2_OK) return rc;
  if (!launch_fits((long long)B * H, 256)) return FA2_ERR_BAD_SHAPE;
  const void* ptrs[8] = {Qc, Kc, Vc, descale_q, descale_k, descale_v, O, LSE};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA2_ERR_ALIGN;
  const long long bh = (long long)B * H;
  const Range in[6] = {range_of(Qc, bh * d), range_of(Kc, bh * N_k * d), range_of(Vc, bh * N_k * d),
                       range_of(descale_q, bh * 4), range_of(descale_k, bh * 4), range_of(descale_v, bh * 4)};
  const Range o = range_of(O, bh * d * 2), l = range_of(LSE, bh * 4);
  if (overlap(o, l)) return FA2_ERR_ALIAS;
  for (const Range& r : in)
    if (overlap(o, r) || overlap(l, r)) return FA2_ERR_ALIAS;
  fa2::Fp8Params p{};
  p.q = static_cast<const uint8_t*>(Qc);
  p.k = static_cast<const uint8_t*>(Kc);
  p.v = static_cast<const uint8_t*>(Vc);
  p.dsq = descale_q;
  p.dsk = descale_k;
  p.dsv = descale_v;
  p.o = static_cast<uint16_t*>(O);
  p.lse = LSE;
  p.B = B;
  p.H = H;
  p.n_q = 1;
  p.n_k = N_k;
  p.d = d;
  p.wl = -1;
  p.wr = -1;
  p.scale = scale;
  if (fa2::launch_decode_fp8(p, static_cast<hipStream_t>(stream)) != hipSuccess) return FA2_ERR_HIP;
  return FA2_OK;
}

int fa2_probe_xcc(int* out, int n_workgroups, void* stream) {
  if (!out) return FA2_ERR_NULLPTR;
  if (n_workgroups < 1 || !launch_fits(n_workgroups, 64)) return FA2_ERR_BAD_SHAPE;
  if (fa2::launch_xcc_probe(out, n_workgroups, static_cast<hipStream_t>(stream)) != hipSuccess) return FA2_ERR_HIP;
  return FA2_OK;
}

const char* fa2_status_string(int status) {
  switch (status) {
    case FA2_OK: return "FA2_OK: success";
    case FA2_ERR_NULLPTR: return "FA2_ERR_NULLPTR: a required pointer is NULL";
    case FA2_ERR_BAD_SHAPE: return "FA2_ERR_BAD_SHAPE: B, H, N_q, N_k must be >= 1 and within the size limits";
    case FA2_ERR_HEAD_DIM: return "FA2_ERR_HEAD_DIM: head dim d must be 64 or 128";
    case FA2_ERR_BAD_SCALE: return "FA2_ERR_BAD_SCALE: scale must be finite with |scale| <= 2e38";
    case FA2_ERR_WORKSPACE: return "FA2_ERR_WORKSPACE: split-KV workspace missing or too small";
    case FA2_ERR_ALIAS: return "FA2_ERR_ALIAS: an output overlaps an input, another output or the workspace";
    case FA2_ERR_SPLITS: return "FA2_ERR_SPLITS: num_splits must be in [1, min(N_k, FA2_MAX_SPLITS)]";
    case FA2_ERR_HIP: return "FA2_ERR_HIP: the HIP runtime rejected a kernel launch";
    case FA2_ERR_WINDOW: return "FA2_ERR_WINDOW: window sizes must be -1 (unbounded) or in [0, 2^30]";
    case FA2_ERR_ALIGN: return "FA2_ERR_ALIGN: FP8 entry points need 16-byte aligned tensor pointers";
    case FA2_ERR_CONFIG: return "FA2_ERR_CONFIG: config must be in [0, fa2_fwd_num_configs())";
    case FA2_ERR_SCRATCH:
      return "FA2_ERR_SCRATCH: the split-KV partials exceed the library's fixed scratch (FA2_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown fa2 status";
  }
}

}  // extern "C"
