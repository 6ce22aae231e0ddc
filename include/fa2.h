/*
 * fa2.h — FlashAttention-2 style exact-attention forward for AMD MI355X (gfx950).
 *
 * C ABI.  Every tensor argument is a DEVICE pointer owned by the caller
 * (for example the data pointer of a torch tensor); the library never
 * allocates, frees or synchronises, keeps no state between calls and only
 * enqueues work on `stream` (a hipStream_t passed as void*; NULL = the
 * default stream).  Calls return as soon as the work is enqueued.
 *
 * Layouts (contiguous, row-major):
 *   Q   [B][H][N_q][d]   bf16 (raw 16-bit storage)
 *   K,V [B][H][N_k][d]   bf16
 *   O   [B][H][N_q][d]   bf16, rounded to nearest even from fp32
 *   LSE [B][H][N_q]      fp32, natural logarithm
 *
 * What is computed (the FlashAttention-2 source walkthrough page, "kernel main
 * loop" section: the online-softmax pseudocode, whose result is exact
 * attention; the epilogue writes O and the log-sum-exp):
 *   s_ij   = scale * sum_c Q[i][c] * K[j][c]
 *   key j is visible to query i iff j < N_k and, when causal != 0, j <= i
 *            (top-left alignment, so every query row sees key 0)
 *   O[i]   = sum_j softmax_j(s_ij) * V[j]      over visible keys
 *   LSE[i] = log(sum_j exp(s_ij))              over visible keys
 * Products are formed from the bf16 inputs and accumulated in fp32.  The
 * probabilities are rounded to bf16 for the P.V product; O is divided by the
 * sum of those rounded probabilities (so each output row is an exact convex
 * combination of V rows), and LSE uses the sum of the fp32 probabilities.
 *
 * Errors: every argument is validated on the host BEFORE any HIP call, and a
 * negative fa2_status is returned with nothing enqueued.  FA2_ERR_HIP means
 * a launch was rejected by the runtime (hipGetLastError).  Faults during
 * execution surface at the caller's next synchronisation.  No C++ exception
 * crosses this interface.  Overlapping calls on different streams that share
 * output buffers race; the library does not detect that.
 */
#ifndef FA2_H_
#define FA2_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa2_status {
  FA2_OK = 0,
  FA2_ERR_NULLPTR = -1,   /* a required pointer is NULL */
  FA2_ERR_BAD_SHAPE = -2, /* B, H, N_q, N_k < 1, or a size beyond the limits below */
  FA2_ERR_HEAD_DIM = -3,  /* d is not 64 or 128 */
  FA2_ERR_BAD_SCALE = -4, /* scale is not finite */
  FA2_ERR_WORKSPACE = -5, /* split-KV workspace NULL or smaller than fa2_splitkv_workspace_bytes() */
  FA2_ERR_ALIAS = -6,     /* an output overlaps an input, another output or the workspace */
  FA2_ERR_HIP = -7,       /* the HIP runtime rejected a kernel launch */
  FA2_ERR_SPLITS = -8,    /* num_splits outside [1, min(N_k, FA2_MAX_SPLITS)] */
  FA2_ERR_WINDOW = -9,    /* a window size below -1 or above 2^30 */
  FA2_ERR_ALIGN = -10,    /* an FP8 entry point's tensor pointer is not 16-byte aligned */
  FA2_ERR_SCRATCH = -11,  /* fa2_fwd_splitkv_noalloc: the partials exceed FA2_NOALLOC_SCRATCH_BYTES */
  FA2_ERR_CONFIG = -12    /* fa2_fwd_config: config outside [0, fa2_fwd_num_configs()) */
} fa2_status;

/* Size limits (validated): N_k * d and N_q * d below 2^30 per head (one
 * head's Q, K or V under 2 GiB); every launch below 2^31 workgroups and
 * below 2^32 work-items in all (workgroups x threads per workgroup).
 * Shapes beyond them return FA2_ERR_BAD_SHAPE with nothing enqueued. */
#define FA2_MAX_SPLITS 256

/*
 * fa2_fwd — exact attention forward (the FlashAttention-2 forward pass).
 *
 * Launch shape (the walkthrough page, "launch grid" section: one workgroup
 * per query block, batch and head, with the query sequence split into
 * blocks): ceil(N_q / B_r) * B * H workgroups, B_r query rows each; every
 * workgroup streams the K/V blocks its rows can see (the synthesis page,
 * section 2 item 2: queries on the outer loop, keys/values on the inner loop,
 * no inter-workgroup communication).  With causal != 0, key blocks above the
 * diagonal are skipped and only diagonal blocks are masked.  N_q == 1 (one
 * decode step) runs one workgroup per (batch, head) that streams all N_k keys
 * with fp32 probabilities, so O there is divided by the same fp32 sum as LSE.
 *
 * Q, K, V, O, LSE: device pointers as laid out above.  O and LSE must not
 * overlap Q, K, V or each other.
 * B, H, N_q, N_k: >= 1.   d: 64 or 128.   causal: 0 or non-zero.
 * scale: finite multiplier of q.k (callers usually pass fp32(1/sqrt(d))).
 * stream: hipStream_t or NULL.
 * Returns FA2_OK or a negative fa2_status.
 */
int fa2_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
            int B, int H, int N_q, int N_k, int d, int causal, float scale, void* stream);

/*
 * fa2_fwd_window — sliding-window (banded) attention forward (the synthesis
 * page, section 5 item 4: the causal block skip generalised to a window).
 *
 * Key j is visible to query i iff j < N_k and
 *   (window_left  < 0 or j >= i - window_left)  and
 *   (window_right < 0 or j <= i + window_right),
 * top-left aligned like the causal mask.  (-1, -1) is plain attention and
 * (-1, 0) is fa2_fwd's causal mask; (w - 1, 0) is causal attention over the
 * last w positions.  Each workgroup streams only the key tiles its rows can
 * see; tiles wholly inside every row's band run unmasked, tiles crossing an
 * edge are masked.  A row that sees no key (possible when N_q > N_k or the
 * band misses every key) gets O = 0 and LSE = -inf.
 *
 * Arguments, layouts and errors as fa2_fwd, plus window_left, window_right:
 * -1 (unbounded) or 0 .. 2^30, else FA2_ERR_WINDOW.  A single query row
 * (N_q == 1) sees keys 0 .. window_right.
 */
int fa2_fwd_window(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   int B, int H, int N_q, int N_k, int d, int window_left, int window_right,
                   float scale, void* stream);

/*
 * fa2_fwd_blocksparse — attention forward under a block mask (the synthesis
 * page, section 5 item 4: the causal block skip extended to sliding windows
 * and dilated patterns as one sparse-block-skip mechanism).
 *
 * block_mask: device bytes [mask_batches][mask_heads][ceil(N_q/128)][ceil(N_k/64)],
 * mask_batches in {1, B}, mask_heads in {1, H} (a size-1 dimension is shared by
 * every batch or head).  One entry per (128-row query block, 64-key block):
 * key j is visible to query i of (b, h) iff j < N_k, the entry
 * [b mod mask_batches][h mod mask_heads][i / 128][j / 64] is non-zero, and the
 * band admits it: (window_left < 0 or j >= i - window_left) and
 * (window_right < 0 or j <= i + window_right), as fa2_fwd_window.  Each
 * workgroup streams only the key tiles its mask row marks, and masks inside a
 * tile only at the band's edges and the key tail.  A row that sees no key
 * gets O = 0 and LSE = -inf.  A dilated pattern is a mask whose entries skip
 * key blocks at a stride; the all-ones mask is fa2_fwd_window.
 *
 * The mask is read in aligned 4-byte words (never past the aligned word that
 * holds its last byte).
 *
 * Other arguments, layouts and errors as fa2_fwd_window; FA2_ERR_NULLPTR for
 * a NULL mask, FA2_ERR_BAD_SHAPE for mask dimensions other than 1 or B / H,
 * FA2_ERR_ALIAS when O or LSE overlaps the mask.
 */
#define FA2_MASK_BLOCK_Q 128
#define FA2_MASK_BLOCK_K 64
int fa2_fwd_blocksparse(const void* Q, const void* K, const void* V, void* O, float* LSE,
                        int B, int H, int N_q, int N_k, int d, const unsigned char* block_mask,
                        int mask_batches, int mask_heads, int window_left, int window_right,
                        float scale, void* stream);

/*
 * Forward configurations (the synthesis page, section 3 item 3: FA2 picks its
 * block sizes by hand from a few candidates; section 5 item 1: search block
 * sizes, warp counts and stages per shape instead).  A configuration is a
 * kernel plus a workgroup order; every configuration computes the same result
 * (the kernels share their arithmetic, so outputs agree bit for bit between
 * configurations of one kernel, and to rounding between kernels):
 *   kernel   "tile128":     4 waves, 128 query rows per workgroup, two
 *                           workgroups per compute unit;
 *            "pingpong256": 8 waves, 256 query rows, waves sharing a SIMD
 *                           alternate matrix and vector phases;
 *            "tile256":     8 waves, 256 query rows, the tile128 loop with every
 *                           wave in step (K/V tiles shared by twice the rows);
 *   order    "remap":       workgroup ids renumbered so that each of the 8
 *                           XCDs (chiplets) runs a contiguous range of blocks
 *                           (the synthesis page, section 2, Chiplet FA
 *                           paragraph: K/V reuse in one chiplet's L2);
 *            "noremap":     ids as dispatched (id i on XCD i mod 8);
 *            "headmajor":   all query blocks of one (batch, head) together;
 *            "qbmajor":     query block slowest, (batch, head) fastest, so that
 *                           under a causal or banded mask the heaviest block of
 *                           every head is dispatched before any lighter one.
 * fa2_fwd and fa2_fwd_window take the configuration a measured table picks
 * for (d, banded, N_q) (fa2_fwd_default_config); fa2_fwd_config runs a chosen
 * one (for measuring, and for parity tests of every configuration).
 *
 * fa2_fwd_num_configs: the number of configurations.
 * fa2_fwd_config_name: a static name for config, or NULL when out of range.
 * fa2_fwd_default_config: the configuration fa2_fwd (banded = causal) or
 *   fa2_fwd_window (banded = a window side >= 0) takes for the shape, or
 *   FA2_ERR_BAD_SHAPE / FA2_ERR_HEAD_DIM.  No HIP call.
 * fa2_fwd_config: fa2_fwd_window with the given configuration; arguments and
 *   errors as fa2_fwd_window, plus FA2_ERR_CONFIG.  N_q == 1 always runs the
 *   single-row decode kernel, whatever the configuration.
 */
int fa2_fwd_num_configs(void);
const char* fa2_fwd_config_name(int config);
int fa2_fwd_default_config(int d, int banded, int N_q, int B, int H);
int fa2_fwd_config(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   int B, int H, int N_q, int N_k, int d, int window_left, int window_right,
                   float scale, int config, void* stream);

/*
 * fa2_splitkv_workspace_bytes — bytes of caller-owned device workspace that
 * fa2_fwd_splitkv needs: num_splits * B * H * N_q * (d + 2) * 4.
 * Returns 0 when an argument is out of range.
 */
size_t fa2_splitkv_workspace_bytes(int B, int H, int N_q, int d, int num_splits);

/*
 * fa2_fwd_splitkv — the same result as fa2_fwd, computed by splitting the key
 * sequence into num_splits chunks (the synthesis page, section 5 item 5: for
 * single-query decode the query-block parallelism vanishes, so parallelise
 * over the key/value sequence and merge the partial results).
 *
 * Chunk c covers keys [c*L, min((c+1)*L, N_k)), L = ceil(N_k / num_splits);
 * a chunk may be empty.  Pass 1 writes, per chunk and query row, the fp32
 * partial (acc, m, l) into the workspace:
 *   m   = a reference level in natural-log units: the running maximum of the
 *         chunk's visible scaled scores s_ij at its last refresh (at most the
 *         true maximum; -inf exactly when the chunk holds no visible key);
 *   l   = sum over the chunk of exp(s_ij - m), in fp32           (0 when empty);
 *   acc = l * (the chunk's normalised output): acc / l is the chunk's
 *         attention output exactly as the P.V product formed it, a convex
 *         combination of the chunk's V rows                        (0 when empty).
 * So acc / l and m + log(l) (the chunk's log-sum-exp) do not depend on the
 * reference m.  Pass 2 merges them in chunk order: M = max_c m_c,
 * w_c = exp(m_c - M) (0 for an empty chunk), O = (sum_c w_c acc_c) /
 * (sum_c w_c l_c), LSE = M + log(sum_c w_c l_c) — the same rescaling as the
 * online softmax (walkthrough page, main-loop pseudocode).
 *
 * Workspace layout (fp32, R = B*H*N_q rows, row = (b*H + h)*N_q + i):
 *   acc [num_splits][R][d], then m and l, each [num_splits][R].
 * Its contents after the call are the partials above; it must not overlap
 * any input or output.  Both passes run in order on `stream`.
 *
 * Other arguments and errors as fa2_fwd, plus:
 * num_splits: 1 <= num_splits <= min(N_k, FA2_MAX_SPLITS).
 * workspace, workspace_bytes: device buffer of at least
 *   fa2_splitkv_workspace_bytes(B, H, N_q, d, num_splits) bytes.
 */
int fa2_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE,
                    int B, int H, int N_q, int N_k, int d, int causal, float scale,
                    int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa2_bwd_workspace_bytes — bytes of caller-owned device workspace fa2_bwd
 * needs: 2 * B * H * N_q * 4 (LSE * log2(e) and D for every query row).
 * Returns 0 when an argument is out of range.
 */
size_t fa2_bwd_workspace_bytes(int B, int H, int N_q, int N_k, int d);

/*
 * fa2_bwd — gradients of the attention forward (the synthesis page, section 3
 * item 1: FA2's backward as five matrix products from the stored LSE; section
 * 5 item 2: a deterministic variant without atomic adds, in two passes).
 *
 * For an upstream gradient dO of O = fa2_fwd(Q, K, V, causal, scale) and that
 * call's LSE:
 *   P_ij  = exp(scale q_i . k_j - LSE_i) over visible keys (0 elsewhere)
 *   D_i   = sum_c dO_ic O_ic
 *   dV_j  = sum_i P_ij dO_i
 *   dS_ij = P_ij (dO_i . v_j - D_i)
 *   dK_j  = scale * sum_i dS_ij q_i
 *   dQ_i  = scale * sum_j dS_ij k_j
 * P is rounded to bf16 for dV, dS to bf16 for dK and dQ; products accumulate
 * in fp32; dQ, dK, dV are written as bf16 (RNE).
 *
 * Passes: (1) one workgroup per 128-row query block forms D and LSE*log2(e)
 * of its rows (stored in the workspace), streams the key blocks and
 * accumulates dQ for its rows; (2) one workgroup per 128-key block streams
 * the query blocks and accumulates dK and dV for its keys.  Both passes
 * recompute S and dP (seven products in all); every
 * gradient element is accumulated by one wave in a fixed order, with no
 * partial sums in memory and no atomics: results are bit-reproducible.
 *
 * Q, K, V, O, dO: bf16 [B][H][N][d] as in fa2_fwd; LSE: fp32 [B][H][N_q]
 * (natural log, as fa2_fwd writes it).  dQ [B][H][N_q][d], dK and dV
 * [B][H][N_k][d]: bf16 outputs that must not overlap any input, each other
 * or the workspace.  workspace: device buffer of at least
 * fa2_bwd_workspace_bytes(B, H, N_q, N_k, d) bytes (its contents on return
 * are scratch).  causal, scale, stream and the remaining errors as fa2_fwd.
 */
int fa2_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
            const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int N_q, int N_k,
            int d, int causal, float scale, void* workspace, size_t workspace_bytes,
            void* stream);

/*
 * fa2_fwd_splitkv_noalloc — fa2_fwd_splitkv without a caller workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It allocates nothing
 * and calls no allocating routine.
 *
 * The partials go to a fixed array of FA2_NOALLOC_SCRATCH_BYTES bytes of device
 * memory that the library owns (one per GPU, held until the process ends), in
 * the workspace layout of fa2_fwd_splitkv; the same two kernels run, so O and
 * LSE equal fa2_fwd_splitkv's bit for bit.  Problems whose partials
 * (fa2_splitkv_workspace_bytes()) exceed that size return FA2_ERR_SCRATCH
 * with nothing enqueued.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's partials: calls that overlap on one GPU (different
 * streams, or host threads) race, and the caller must order them.  The
 * array's device address is looked up on the first call for each device; the
 * kernels run on `stream`'s device (the current device for NULL).
 *
 * Arguments and the remaining errors as fa2_fwd_splitkv, without the workspace.
 */
#define FA2_NOALLOC_SCRATCH_BYTES (32u << 20)
int fa2_fwd_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int B, int H, int N_q, int N_k, int d, int causal, float scale,
                            int num_splits, void* stream);

/*
 * fa2_num_splits — a key-chunk count for fa2_fwd_splitkv that fills the chip
 * (the walkthrough page, "launch grid" section: the first version derives the
 * split count from batch x heads and the multiprocessor count so that
 * occupancy stays high, while too many splits add HBM traffic and merge work;
 * the synthesis page, section 5 item 5).  Split the key sequence only when the
 * batch x head x query-block grid leaves compute units idle.
 *
 * units = B*H for N_q == 1, else B*H*ceil(N_q/128) (the workgroups of the
 * unsplit launch).  Returns 1 when units >= num_cus; otherwise the smallest
 * count that gives every compute unit one workgroup, or two for N_q > 1 when
 * each chunk still holds >= 2048 keys, capped at max(1, N_k/512) and
 * FA2_MAX_SPLITS.  A return of 1 with N_q > 1 means fa2_fwd is the better call
 * (no merge pass); fa2_fwd with N_q == 1 already streams the keys at full
 * bandwidth when B*H fills the chip.
 *
 * num_cus: compute units of the target device; <= 0 queries the current HIP
 * device (the only case that makes a HIP call).
 * Returns the split count (>= 1) or a negative fa2_status: FA2_ERR_BAD_SHAPE,
 * FA2_ERR_HEAD_DIM, or FA2_ERR_HIP when the device query fails.  Nothing is
 * enqueued.
 */
int fa2_num_splits(int B, int H, int N_q, int N_k, int d, int num_cus);

/*
 * FP8 forward (the improvements page: section 三 credits FlashAttention-3 with
 * FP8 tensor-core support, and section 四 point ③ says FP8 doubles matrix
 * throughput while its precision loss must be held in check by scaling; the
 * pages give no scaling recipe).  The recipe here: each (batch, head) slice of
 * Q, K and V is scaled so that its largest magnitude becomes 448, the largest
 * OCP e4m3 (e4m3fn) value, and rounded to nearest even; descale = amax / 448
 * per slice is applied back in fp32.  Both products run on the 8-bit matrix
 * unit; the probabilities are scaled by 2^7 and rounded to e4m3 for the P.V
 * product, O is divided by the sum of those rounded probabilities, and LSE
 * uses the sum of the fp32 probabilities.  The result approximates exact
 * attention of the dequantised inputs decode(code) * descale.
 *
 * Codes are bytes (e4m3fn: sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; 0x7f and 0xff are NaN and must not appear).  Every tensor pointer of
 * these entry points must be 16-byte aligned (FA2_ERR_ALIGN otherwise).
 */

/*
 * fa2_fp8_vt_stride — row stride, in bytes (= keys), of a transposed V code
 * tensor: N_k rounded up to a multiple of 16.  Returns FA2_ERR_BAD_SHAPE for
 * N_k < 1 or N_k > 2^30.
 */
int fa2_fp8_vt_stride(int N_k);

/*
 * fa2_quantize_fp8 — per-(batch, head) e4m3 quantisation of a bf16 tensor.
 *
 * X: bf16 [B][H][N][d].  descale: fp32 [B][H] output, fp32(amax / 448) of the
 * slice (1 for an all-zero slice).  codes: output, code = e4m3 RNE of
 * fp32(x) * fp32(448 / amax):
 *   transposed == 0: [B][H][N][d]                     (layout of Q and K)
 *   transposed != 0: [B][H][d][fa2_fp8_vt_stride(N)]  (layout of V for
 *                    fa2_fwd_fp8; columns N .. stride-1 are written as 0)
 * X must hold finite values.  codes and descale must not overlap X or each
 * other.  d: 64 or 128; B, H, N >= 1 with N * d below 2^30 and B * H at most
 * 65535 (FA2_ERR_BAD_SHAPE otherwise).  Four kernels are
 * enqueued on `stream`; descale holds intermediate values until the last.
 * Returns FA2_OK or a negative fa2_status.
 */
int fa2_quantize_fp8(const void* X, void* codes, float* descale, int B, int H, int N, int d,
                     int transposed, void* stream);

/*
 * fa2_fwd_fp8 — attention forward on FP8 inputs.
 *
 * Qc [B][H][N_q][d] and Kc [B][H][N_k][d] codes; Vt [B][H][d][stride] codes of
 * V transposed, stride = fa2_fp8_vt_stride(N_k) (fa2_quantize_fp8 with
 * transposed != 0 writes it).  descale_q, descale_k, descale_v: fp32 [B][H],
 * positive and finite.  O bf16 [B][H][N_q][d] and LSE fp32 [B][H][N_q] as in
 * fa2_fwd, with
 *   s_ij = scale * (descale_q * descale_k) * sum_c decode(Qc[i][c]) decode(Kc[j][c])
 *   O[i] = descale_v * sum_j softmax_j(s_ij) decode(V[j])
 * over the visible keys (causal as in fa2_fwd).  Rows are never empty; O and
 * LSE must not overlap any input or each other.  Launch shape, work order and
 * the remaining errors as fa2_fwd.
 */
int fa2_fwd_fp8(const void* Qc, const void* Kc, const void* Vt, const float* descale_q,
                const float* descale_k, const float* descale_v, void* O, float* LSE, int B, int H,
                int N_q, int N_k, int d, int causal, float scale, void* stream);

/*
 * fa2_decode_fp8 — one decode step (a single query row per head) over an FP8
 * K/V cache (the walkthrough page, "launch grid" section, and the synthesis
 * page, section 5 item 5, single-query decode; FP8 inputs as above).
 *
 * Qc [B][H][1][d], Kc and Vc [B][H][N_k][d] e4m3 codes, all in row layout
 * (fa2_quantize_fp8 with transposed == 0 writes them); descales fp32 [B][H],
 * positive and finite.  O bf16 [B][H][1][d], LSE fp32 [B][H][1].  Every key
 * is visible.  One workgroup per (batch, head) streams that head's codes once;
 * the codes are decoded to fp32 in registers and the probabilities stay fp32,
 * so only the inputs are 8-bit.  Pointers 16-byte aligned; O and LSE must not
 * overlap any input or each other; the remaining errors as fa2_fwd.
 */
int fa2_decode_fp8(const void* Qc, const void* Kc, const void* Vc, const float* descale_q,
                   const float* descale_k, const float* descale_v, void* O, float* LSE, int B, int H,
                   int N_k, int d, float scale, void* stream);

/*
 * fa2_probe_xcc — where the workgroups of a launch run (a diagnostic behind
 * the forward's XCD-aware workgroup order; the synthesis page, section 2,
 * Chiplet FA paragraph).  Launches n_workgroups workgroups of one wave; for
 * workgroup i it writes out[2i] = the XCD (chiplet) id and out[2i + 1] = the
 * wave's hardware id word (HW_ID register: wave slot, SIMD, compute unit,
 * shader array and engine fields).  out: device int[2 * n_workgroups].
 * Returns FA2_OK, FA2_ERR_NULLPTR, FA2_ERR_BAD_SHAPE (n_workgroups < 1 or
 * beyond a launch's limits) or FA2_ERR_HIP.
 */
int fa2_probe_xcc(int* out, int n_workgroups, void* stream);

/* fa2_status_string — static, human-readable text for a status code. */
const char* fa2_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H_ */
