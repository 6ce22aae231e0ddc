// Host side of the C ABI under the address and undefined-behaviour sanitizers:
// every entry point's validation, the parameter block it hands to the kernel
// launcher (recorded by the stand-ins in api_stubs.cpp), the workspace carving
// of the split-KV and backward entry points, and sizes at the documented
// limits, where a signed overflow in the size arithmetic would be caught.
// Device pointers are addresses that are never dereferenced.  Exit status:
// the number of failed checks.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "api_stubs.h"
#include "fa2.h"

static int failures = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

// distinct, far-apart fake device addresses (16-byte aligned)
static void* dev(int i) { return reinterpret_cast<void*>((uintptr_t)(0x100000000000ull + (uintptr_t)i * (1ull << 40))); }
static float* devf(int i) { return static_cast<float*>(dev(i)); }

static void test_status_strings() {
  for (int s = 0; s >= -12; --s) CHECK(strncmp(fa2_status_string(s), "FA2_", 4) == 0);
  CHECK(strcmp(fa2_status_string(1), "unknown fa2 status") == 0);
  CHECK(strcmp(fa2_status_string(-13), "unknown fa2 status") == 0);
}

static void test_fwd() {
  void *Q = dev(0), *K = dev(1), *V = dev(2), *O = dev(3);
  float* L = devf(4);
  const float sc = 0.125f;
  CHECK(fa2_fwd(nullptr, K, V, O, L, 1, 2, 256, 256, 64, 0, sc, nullptr) == FA2_ERR_NULLPTR);
  CHECK(fa2_fwd(Q, K, V, O, nullptr, 1, 2, 256, 256, 64, 0, sc, nullptr) == FA2_ERR_NULLPTR);
  CHECK(fa2_fwd(Q, K, V, O, L, 0, 2, 256, 256, 64, 0, sc, nullptr) == FA2_ERR_BAD_SHAPE);
  CHECK(fa2_fwd(Q, K, V, O, L, 1, -3, 256, 256, 64, 0, sc, nullptr) == FA2_ERR_BAD_SHAPE);
  CHECK(fa2_fwd(Q, K, V, O, L, 1, 2, 256, 0, 64, 0, sc, nullptr) == FA2_ERR_BAD_SHAPE);
  CHECK(fa2_fwd(Q, K, V, O, L, 1, 2, 256, 256, 96, 0, sc, nullptr) == FA2_ERR_HEAD_DIM);
  CHECK(fa2_fwd(Q, K, V, O, L, 1, 2, 256, 256, 64, 0, NAN, nullptr) == FA2_ERR_BAD_SCALE);
  CHECK(fa2_fwd(Q, K, V, O, L, 1, 2, 256, 256, 64, 0, INFINITY, nullptr) == FA2_ERR_BAD_SCALE);
  CHECK(fa2_fwd(Q, K, V, O, L, 1, 2, 256, 256, 64, 0, 3.0e38f, nullptr) == FA2_ERR_BAD_SCALE);
  // one head's Q or K/V must stay below 2^31 bytes: N*d <= 2^30 - 1
  CHECK(fa2_fwd(Q, K, V, O, L, 1, 1, (1 << 24), 256, 64, 0, sc, nullptr) == FA2_ERR_BAD_SHAPE);
  CHECK(fa2_fwd(Q, K, V, O, L, 1, 1, 256, (1 << 23), 128, 0, sc, nullptr) == FA2_ERR_BAD_SHAPE);
  CHECK(fa2_fwd(Q, K, V, O, L, 65536, 65536, 1, 1, 64, 0, sc, nullptr) == FA2_ERR_BAD_SHAPE);
  // extreme ints must be rejected without overflow
  CHECK(fa2_fwd(Q, K, V, O, L, INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX, 128, 0, sc, nullptr) == FA2_ERR_BAD_SHAPE);
  // aliasing: O over K, LSE over Q, O over LSE
  CHECK(fa2_fwd(Q, K, V, K, L, 1, 2, 256, 256, 64, 0, sc, nullptr) == FA2_ERR_ALIAS);
  CHECK(fa2_fwd(Q, K, V, O, static_cast<float*>(Q), 1, 2, 256, 256, 64, 0, sc, nullptr) == FA2_ERR_ALIAS);
  CHECK(fa2_fwd(Q, K, V, O, reinterpret_cast<float*>(static_cast<char*>(O) + 100), 1, 2, 256, 256, 64, 0, sc,
                nullptr) == FA2_ERR_ALIAS);
  // nothing was launched by a rejected call
  CHECK(stub::rec.calls == 0);

  // valid calls: the parameter block the launcher receives
  const int c0 = stub::rec.calls;
  CHECK(fa2_fwd(Q, K, V, O, L, 3, 5, 1000, 777, 128, 1, -0.5f, nullptr) == FA2_OK);
  CHECK(stub::rec.calls == c0 + 1 && strcmp(stub::rec.kind, "fwd") == 0);
  const fa2::FwdParams& p = stub::rec.fwd;
  CHECK(p.q == Q && p.k == K && p.v == V && p.o == O && p.lse == L);
  CHECK(p.B == 3 && p.H == 5 && p.n_q == 1000 && p.n_k == 777 && p.d == 128);
  CHECK(p.wl == -1 && p.wr == 0 && p.scale == -0.5f && p.num_splits == 1 && p.split_len == 777);
  CHECK(fa2_fwd(Q, K, V, O, L, 1, 1, 1, 1, 64, 0, 1.f, nullptr) == FA2_OK);
  CHECK(stub::rec.fwd.wl == -1 && stub::rec.fwd.wr == -1);
  // the largest head the API accepts
  CHECK(fa2_fwd(Q, K, V, O, L, 1, 1, (1 << 23) - 1, (1 << 23) - 1, 128, 0, sc, nullptr) == FA2_OK);
  CHECK(fa2_fwd(Q, K, V, O, L, 1, 1, (1 << 24) - 1, (1 << 24) - 1, 64, 1, sc, nullptr) == FA2_OK);
  // a launch error becomes FA2_ERR_HIP
  stub::rec.result = hipErrorLaunchFailure;
  CHECK(fa2_fwd(Q, K, V, O, L, 1, 2, 256, 256, 64, 0, sc, nullptr) == FA2_ERR_HIP);
  stub::rec.result = hipSuccess;
}

static void test_window() {
  void *Q = dev(0), *K = dev(1), *V = dev(2), *O = dev(3);
  float* L = devf(4);
  CHECK(fa2_fwd_window(Q, K, V, O, L, 1, 2, 256, 256, 64, -2, 0, 0.1f, nullptr) == FA2_ERR_WINDOW);
  CHECK(fa2_fwd_window(Q, K, V, O, L, 1, 2, 256, 256, 64, 0, (1 << 30) + 1, 0.1f, nullptr) == FA2_ERR_WINDOW);
  CHECK(fa2_fwd_window(Q, K, V, O, L, 1, 2, 256, 256, 64, 1 << 30, 1 << 30, 0.1f, nullptr) == FA2_OK);
  CHECK(stub::rec.fwd.wl == (1 << 30) && stub::rec.fwd.wr == (1 << 30));
  CHECK(fa2_fwd_window(Q, K, V, O, L, 2, 3, 300, 500, 128, 17, 0, 0.1f, nullptr) == FA2_OK);
  CHECK(stub::rec.fwd.wl == 17 && stub::rec.fwd.wr == 0 && stub::rec.fwd.n_k == 500);
}

static void test_configs() {
  void *Q = dev(0), *K = dev(1), *V = dev(2), *O = dev(3);
  float* L = devf(4);
  const int n = fa2_fwd_num_configs();
  CHECK(n == 10);
  for (int c = 0; c < n; ++c) {
    CHECK(fa2_fwd_config_name(c) != nullptr);
    CHECK(fa2_fwd_config(Q, K, V, O, L, 2, 3, 300, 400, 128, -1, 0, 0.1f, c, nullptr) == FA2_OK);
    CHECK(stub::rec.config == c && stub::rec.fwd.wl == -1 && stub::rec.fwd.wr == 0);
  }
  CHECK(fa2_fwd_config_name(-1) == nullptr && fa2_fwd_config_name(n) == nullptr);
  CHECK(fa2_fwd_config(Q, K, V, O, L, 2, 3, 300, 400, 128, -1, 0, 0.1f, n, nullptr) == FA2_ERR_CONFIG);
  CHECK(fa2_fwd_config(Q, K, V, O, L, 2, 3, 300, 400, 128, -1, 0, 0.1f, -1, nullptr) == FA2_ERR_CONFIG);
  CHECK(fa2_fwd_config(Q, K, V, O, L, 2, 3, 300, 400, 128, -3, 0, 0.1f, 0, nullptr) == FA2_ERR_WINDOW);
  // fa2_fwd and fa2_fwd_window take the table's configuration for the shape
  CHECK(fa2_fwd(Q, K, V, O, L, 1, 32, 16384, 16384, 128, 0, 0.1f, nullptr) == FA2_OK);
  CHECK(stub::rec.config == fa2_fwd_default_config(128, 0, 16384, 1, 32));
  CHECK(fa2_fwd(Q, K, V, O, L, 8, 16, 2048, 2048, 64, 1, 0.1f, nullptr) == FA2_OK);
  CHECK(stub::rec.config == fa2_fwd_default_config(64, 1, 2048, 8, 16));
  CHECK(fa2_fwd_window(Q, K, V, O, L, 1, 2, 9000, 9000, 128, 100, 0, 0.1f, nullptr) == FA2_OK);
  CHECK(stub::rec.config == fa2_fwd_default_config(128, 1, 9000, 1, 2));
  CHECK(fa2_fwd_default_config(96, 0, 100, 1, 1) == FA2_ERR_HEAD_DIM);
  CHECK(fa2_fwd_default_config(64, 0, 0, 1, 1) == FA2_ERR_BAD_SHAPE);
  for (int nq = 1; nq < (1 << 24); nq *= 3)
    for (int d = 64; d <= 128; d += 64)
      for (int b = 0; b < 2; ++b) {
        const int c = fa2_fwd_default_config(d, b, nq, 1, 1);
        CHECK(c >= 0 && c < n);
      }
}

static void test_blocksparse() {
  void *Q = dev(0), *K = dev(1), *V = dev(2), *O = dev(3);
  float* L = devf(4);
  const unsigned char* M = static_cast<const unsigned char*>(dev(10));
  CHECK(fa2_fwd_blocksparse(Q, K, V, O, L, 2, 3, 300, 700, 64, nullptr, 1, 1, -1, -1, 0.1f, nullptr) ==
        FA2_ERR_NULLPTR);
  CHECK(fa2_fwd_blocksparse(Q, K, V, O, L, 2, 3, 300, 700, 64, M, 3, 1, -1, -1, 0.1f, nullptr) == FA2_ERR_BAD_SHAPE);
  CHECK(fa2_fwd_blocksparse(Q, K, V, O, L, 2, 3, 300, 700, 64, M, 1, 2, -1, -1, 0.1f, nullptr) == FA2_ERR_BAD_SHAPE);
  // per-(batch, head) mask: 3 query blocks x 11 key blocks each
  CHECK(fa2_fwd_blocksparse(Q, K, V, O, L, 2, 3, 300, 700, 64, M, 2, 3, 50, 0, 0.1f, nullptr) == FA2_OK);
  const fa2::FwdParams& p = stub::rec.fwd;
  CHECK(p.bmask == M && p.bm_n_kb == 11 && p.bm_stride_h == 33 && p.bm_stride_b == 99 && p.wl == 50 && p.wr == 0);
  CHECK(strcmp(stub::rec.kind, "fwd_blockmask") == 0);
  // shared over batches and heads: zero strides
  CHECK(fa2_fwd_blocksparse(Q, K, V, O, L, 2, 3, 300, 700, 64, M, 1, 1, -1, -1, 0.1f, nullptr) == FA2_OK);
  CHECK(stub::rec.fwd.bm_stride_h == 0 && stub::rec.fwd.bm_stride_b == 0);
  // the largest head: N_k * d just under 2^30
  CHECK(fa2_fwd_blocksparse(Q, K, V, O, L, 1, 1, 1 << 10, (1 << 24) - 1, 64, M, 1, 1, -1, -1, 0.1f, nullptr) ==
        FA2_OK);
  CHECK(stub::rec.fwd.bm_n_kb == (1 << 18));
}

static void test_splitkv() {
  void *Q = dev(0), *K = dev(1), *V = dev(2), *O = dev(3), *W = dev(5);
  float* L = devf(4);
  CHECK(fa2_splitkv_workspace_bytes(64, 32, 1, 128, 16) == (size_t)16 * 64 * 32 * 130 * 4);
  CHECK(fa2_splitkv_workspace_bytes(1, 1, 1, 64, 0) == 0);
  CHECK(fa2_splitkv_workspace_bytes(1, 1, 1, 64, FA2_MAX_SPLITS + 1) == 0);
  CHECK(fa2_splitkv_workspace_bytes(INT32_MAX, INT32_MAX, INT32_MAX, 128, FA2_MAX_SPLITS) > 0);
  const size_t need = fa2_splitkv_workspace_bytes(2, 4, 3, 64, 5);
  CHECK(fa2_fwd_splitkv(Q, K, V, O, L, 2, 4, 3, 100, 64, 0, 0.1f, 0, W, need, nullptr) == FA2_ERR_SPLITS);
  CHECK(fa2_fwd_splitkv(Q, K, V, O, L, 2, 4, 3, 4, 64, 0, 0.1f, 5, W, need, nullptr) == FA2_ERR_SPLITS);
  CHECK(fa2_fwd_splitkv(Q, K, V, O, L, 2, 4, 3, 100, 64, 0, 0.1f, 5, W, need - 1, nullptr) == FA2_ERR_WORKSPACE);
  CHECK(fa2_fwd_splitkv(Q, K, V, O, L, 2, 4, 3, 100, 64, 0, 0.1f, 5, nullptr, need, nullptr) == FA2_ERR_WORKSPACE);
  CHECK(fa2_fwd_splitkv(Q, K, V, O, L, 2, 4, 3, 100, 64, 0, 0.1f, 5, K, need, nullptr) == FA2_ERR_ALIAS);
  const int c0 = stub::rec.calls;
  CHECK(fa2_fwd_splitkv(Q, K, V, O, L, 2, 4, 3, 100, 64, 1, 0.1f, 5, W, need, nullptr) == FA2_OK);
  CHECK(stub::rec.calls == c0 + 2 && strcmp(stub::rec.kind, "splitkv_merge") == 0);
  const fa2::FwdParams& p = stub::rec.fwd;
  const long long R = 2 * 4 * 3;
  float* ws = static_cast<float*>(W);
  CHECK(p.num_splits == 5 && p.split_len == 20 && p.wr == 0);
  // acc [S][R][d], then m and l [S][R] each, ending exactly at the workspace size
  CHECK(p.ws_acc == ws && p.ws_m == ws + 5 * R * 64 && p.ws_l == p.ws_m + 5 * R);
  CHECK((size_t)((char*)(p.ws_l + 5 * R) - (char*)ws) == need);
  // 2^20 heads of one query row in 16 chunks: 2^24 decode workgroups of 256 work-items, one past
  // the 2^32 work-items of a dispatch; 2^20 - 1 heads fit
  const int c1 = stub::rec.calls;
  CHECK(fa2_fwd_splitkv(Q, K, V, O, L, 1 << 10, 1 << 10, 1, 16, 128, 0, 0.1f, 16, W,
                        fa2_splitkv_workspace_bytes(1 << 10, 1 << 10, 1, 128, 16), nullptr) == FA2_ERR_BAD_SHAPE);
  CHECK(stub::rec.calls == c1);
  CHECK(fa2_fwd_splitkv(Q, K, V, O, L, (1 << 20) - 1, 1, 1, 16, 128, 0, 0.1f, 16, W,
                        fa2_splitkv_workspace_bytes((1 << 20) - 1, 1, 1, 128, 16), nullptr) == FA2_OK);
}

static void test_num_splits() {
  stub::rec.num_cus = 256;
  CHECK(fa2_num_splits(64, 32, 1, 8192, 128, 0) == 1);  // units >= CUs
  CHECK(fa2_num_splits(1, 8, 1, 131072, 128, 0) == 32);
  CHECK(fa2_num_splits(1, 8, 1, 131072, 128, 64) == 8);
  CHECK(fa2_num_splits(1, 1, 1, 100, 64, 0) == 1);      // capped by N_k / 512
  CHECK(fa2_num_splits(1, 1, 1, INT32_MAX, 64, 0) == FA2_MAX_SPLITS);
  CHECK(fa2_num_splits(0, 1, 1, 100, 64, 0) == FA2_ERR_BAD_SHAPE);
  CHECK(fa2_num_splits(1, 1, 1, 100, 32, 0) == FA2_ERR_HEAD_DIM);
  stub::rec.num_cus = 0;  // the device query fails
  CHECK(fa2_num_splits(1, 1, 1, 100000, 64, 0) == FA2_ERR_HIP);
  CHECK(fa2_num_splits(1, 1, 1, 100000, 64, 100) >= 1);  // an explicit CU count needs no query
  stub::rec.num_cus = 256;
}

static void test_bwd() {
  void *Q = dev(0), *K = dev(1), *V = dev(2), *O = dev(3), *dO = dev(6), *dQ = dev(7), *dK = dev(8), *dV = dev(9),
       *W = dev(5);
  float* L = devf(4);
  const long long R = 1 * 2 * 256;
  // LSE*log2e and D per query row, whatever N_k and d (and no overflow at the limits)
  CHECK(fa2_bwd_workspace_bytes(1, 2, 256, 200, 64) == (size_t)(2 * R) * 4);
  CHECK(fa2_bwd_workspace_bytes(1, 2, 256, 300, 128) == (size_t)(2 * R) * 4);
  CHECK(fa2_bwd_workspace_bytes(1, 32, 16384, 16384, 128) == (size_t)2 * 32 * 16384 * 4);
  CHECK(fa2_bwd_workspace_bytes(INT32_MAX, INT32_MAX, 1, INT32_MAX, 128) > 0);
  CHECK(fa2_bwd_workspace_bytes(0, 2, 256, 200, 64) == 0);
  const size_t need = fa2_bwd_workspace_bytes(1, 2, 256, 200, 64);
  CHECK(fa2_bwd(Q, K, V, O, nullptr, L, dQ, dK, dV, 1, 2, 256, 200, 64, 0, 0.1f, W, need, nullptr) == FA2_ERR_NULLPTR);
  CHECK(fa2_bwd(Q, K, V, O, dO, L, dQ, dK, dV, 1, 2, 256, 200, 96, 0, 0.1f, W, need, nullptr) == FA2_ERR_HEAD_DIM);
  CHECK(fa2_bwd(Q, K, V, O, dO, L, dQ, dK, dV, 1, 2, 256, 200, 64, 0, 0.1f, W, need - 4, nullptr) == FA2_ERR_WORKSPACE);
  CHECK(fa2_bwd(Q, K, V, O, dO, L, dQ, dK, dK, 1, 2, 256, 200, 64, 0, 0.1f, W, need, nullptr) == FA2_ERR_ALIAS);
  CHECK(fa2_bwd(Q, K, V, O, dO, L, dQ, dK, dV, 1, 2, 256, 200, 64, 0, 0.1f, dO, need, nullptr) == FA2_ERR_ALIAS);
  CHECK(fa2_bwd(Q, K, V, O, dO, L, dQ, dK, dV, 1, 2, 256, 200, 64, 1, 0.1f, W, need, nullptr) == FA2_OK);
  CHECK(strcmp(stub::rec.kind, "bwd") == 0);
  const fa2::BwdParams& p = stub::rec.bwd;
  float* ws = static_cast<float*>(W);
  CHECK(p.dout == dO && p.dq == dQ && p.dk == dK && p.dv == dV && p.lse == L && p.causal == 1);
  // LSE*log2e [R], then D [R], ending at the workspace size
  CHECK(p.l2vec == ws && p.dvec == ws + R);
  CHECK((size_t)((char*)(p.dvec + R) - (char*)ws) == need);
}

static void test_fp8() {
  void *Q = dev(0), *K = dev(1), *V = dev(2), *O = dev(3);
  float *L = devf(4), *dq = devf(10), *dk = devf(11), *dv = devf(12);
  CHECK(fa2_fp8_vt_stride(1) == 16 && fa2_fp8_vt_stride(16) == 16 && fa2_fp8_vt_stride(17) == 32);
  CHECK(fa2_fp8_vt_stride(0) == FA2_ERR_BAD_SHAPE && fa2_fp8_vt_stride((1 << 30) + 1) == FA2_ERR_BAD_SHAPE);
  CHECK(fa2_fp8_vt_stride(1 << 30) == (1 << 30));
  CHECK(fa2_quantize_fp8(Q, K, dq, 1, 2, 100, 64, 1, nullptr) == FA2_OK);
  CHECK(strcmp(stub::rec.kind, "quantize_fp8") == 0 && stub::rec.quant.vt_stride == 112 &&
        stub::rec.quant.transposed == 1);
  CHECK(fa2_quantize_fp8(Q, static_cast<char*>(K) + 8, dq, 1, 2, 100, 64, 0, nullptr) == FA2_ERR_ALIGN);
  CHECK(fa2_quantize_fp8(Q, Q, dq, 1, 2, 100, 64, 0, nullptr) == FA2_ERR_ALIAS);
  CHECK(fa2_quantize_fp8(Q, K, dq, 256, 256, 100, 64, 0, nullptr) == FA2_ERR_BAD_SHAPE);
  CHECK(fa2_fwd_fp8(Q, K, V, nullptr, dk, dv, O, L, 1, 2, 256, 256, 128, 0, 0.1f, nullptr) == FA2_ERR_NULLPTR);
  CHECK(fa2_fwd_fp8(Q, K, V, dq, dk, dv, O, L, 1, 2, 256, 256, 128, 1, 0.1f, nullptr) == FA2_OK);
  CHECK(strcmp(stub::rec.kind, "fwd_fp8") == 0 && stub::rec.fp8.vt == V && stub::rec.fp8.vt_stride == 256 &&
        stub::rec.fp8.wr == 0);
  CHECK(fa2_fwd_fp8(Q, K, V, dq, dk, dv, O, reinterpret_cast<float*>(static_cast<char*>(O) + 16), 1, 2, 256, 256,
                    128, 0, 0.1f, nullptr) == FA2_ERR_ALIAS);
  CHECK(fa2_decode_fp8(Q, K, V, dq, dk, dv, O, L, 4, 8, 1000, 64, 0.1f, nullptr) == FA2_OK);
  CHECK(strcmp(stub::rec.kind, "decode_fp8") == 0 && stub::rec.fp8.n_q == 1 && stub::rec.fp8.n_k == 1000 &&
        stub::rec.fp8.v == V);
  CHECK(fa2_decode_fp8(Q, K, V, dq, dk, dv, O, L, 4, 8, 1000, 64, NAN, nullptr) == FA2_ERR_BAD_SCALE);
}

int main() {
  test_status_strings();
  test_fwd();
  test_window();
  test_configs();
  test_blocksparse();
  test_splitkv();
  test_num_splits();
  test_bwd();
  test_fp8();
  if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
  else printf("host API checks passed\n");
  return failures;
}
