// FP8 (OCP e4m3) attention forward for gfx950, and the per-head quantiser that
// produces its inputs.
//
// The improvements page (section 三 on FlashAttention-3, section 四 point ③)
// says FP8 matrix units double the throughput and that the precision lost has
// to be controlled by scaling.  Here every (batch, head) slice of Q, K and V is
// scaled so that its largest magnitude maps to 448, the largest e4m3 value, and
// rounded to nearest even; the slice's descale = amax / 448 is applied back in
// fp32 (scores: descale_q * descale_k folded into the softmax multiplier;
// output: descale_v in the epilogue).
//
// The forward keeps the structure of the bf16 kernel (one 32-row query block
// per wave, 64-key K/V tiles streamed through two LDS stages, S computed
// transposed so that one lane column holds one query row), with both products
// on v_mfma_f32_32x32x64_f8f6f4:
//   S^T = K Q^T      K rows from LDS, Q codes resident in VGPRs
//   P   = 2^7 exp2(s*sl2 - m)  rounded to e4m3 (v_cvt_pk_fp8_f32, RNE)
//   O^T += V^T P^T   V^T from LDS (V is stored transposed by the quantiser)
//   l   += 1^T P^T   a third product against a block of ones: the exact sum of
//                    the rounded probabilities, so that each output row is a
//                    convex combination of V rows
// and LSE from the fp32 sum of the unrounded probabilities.
//
// Operand layout of the 32x32x64 fp8 product (lane l, byte j): A holds row
// l%32, k = 32*(l/32) + j; B holds column l%32, the same k; C as in the bf16
// 32x32 products (register r: row 8*(r/4) + 4*(l/32) + r%4, column l%32).  For
// the probabilities of a lane to be the B operand of the second product with
// keys in natural order, the K rows are read from LDS permuted: A row
// rho = 8g + 4h + e (g < 4, h < 2, e < 4) of key block kb holds key
// 32h + 16kb + 4g + e.  Score register r of s_kb in lane half hf is then key
// 32*hf + 16*kb + r, and bytes 0..31 of the packed probabilities are keys
// 32*hf + 0..31 of the tile.
#include "fa2_device.h"
#include "fa2_internal.h"

#include <float.h>
#include <math.h>

namespace fa2 {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kBC8 = 64;             // keys per tile
constexpr float kPLog2 = 7.f;        // probabilities are scaled by 2^7 before rounding
constexpr unsigned kOnes = 0x38383838u;  // four e4m3 ones

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// K tile: 64 rows (keys) of D bytes in 16-byte chunks; chunk c of row r is
// stored at slot c ^ kswz(r).  The 16 lanes of one LDS read phase read one
// chunk of rows {0..7, 32..39} (+8, +16 or +24); the XOR spreads them over
// all 16 slots of a 256-byte bank row.
template <int D> __device__ __forceinline__ int kswz(int r);
template <> __device__ __forceinline__ int kswz<128>(int r) { return ((r >> 1) & 3) | (((r >> 5) & 1) << 2); }
template <> __device__ __forceinline__ int kswz<64>(int r) { return ((r >> 2) & 1) | (((r >> 5) & 1) << 1); }
// V^T tile: D rows (feature) of 64 bytes (keys); 16 consecutive rows at one chunk.
__device__ __forceinline__ int vswz(int r) { return (r >> 2) & 3; }

template <int D>
__device__ __forceinline__ int kperm(int col) {  // tile row read by A row `col` of key block 0
  return 32 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
}

template <int D>
struct Fp8Rows {
  i32x8 qf[D / 64];  // Q codes: qf[t] bytes j = Q[row][64t + 32hf + j]
  f32x16 acc[D / 32];
  f32x16 lsum;       // sum of the rounded probabilities (every register holds the row total)
  float m_run;       // reference maximum of the scaled scores (log2 units)
  float l_run;       // fp32 sum of the unrounded probabilities (this lane's share)
};

template <int D>
struct Fp8Addr {
  unsigned ka[D / 32];  // K: chunk 4t + 2hf + h of tile row kperm(col), j = 2t + h
  unsigned va[2];       // V^T: chunk 2hf + h of tile row col
};

// One K tile and one V^T tile (keys k0 .. k0 + 63) into LDS; each has 4*D
// 16-byte slots and lane `lane` of wave `wave` fills slot (i*NW + wave)*64 + lane.
// V^T chunks at or beyond the row stride would read the next feature row, so
// they get an offset past the buffer and load zero.
template <int D, int NW>
__device__ __forceinline__ void issue_tile8(i32x4 krs, i32x4 vrs, unsigned vbytes, int vt_stride, const char* kdst,
                                            const char* vdst, int k0, int wave, int lane) {
  constexpr int CPR = D / 16;
  constexpr int NLD = 4 * D / (64 * NW);
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int s = (i * NW + wave) * 64 + lane;
    const int kr = s / CPR;
    const int kc = (s % CPR) ^ kswz<D>(kr);
    const unsigned koff = (unsigned)((k0 + kr) * D + 16 * kc);
    const int vr = s >> 2;
    const int vc = (s & 3) ^ vswz(vr);
    const int key = k0 + 16 * vc;
    const unsigned voff = key < vt_stride ? (unsigned)(vr * vt_stride + key) : vbytes;
    const int sbase = (i * NW + wave) * 64 * 16;
    lds_dma16(krs, kdst + sbase, koff);
    lds_dma16(vrs, vdst + sbase, voff);
  }
}

__device__ __forceinline__ i32x8 cat8(u32x4 lo, u32x4 hi) {
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// S^T = K Q^T for one 64-key tile: s{kb}[r] is the score of this lane's query
// row against key k0 + 32hf + 16kb + r.
template <int D, unsigned KOFF>
__device__ __forceinline__ void qk8(const Fp8Rows<D>& w, const Fp8Addr<D>& la, f32x16& s0, f32x16& s1) {
  s0 = f32x16{};
  s1 = f32x16{};
#pragma unroll
  for (int t = 0; t < D / 64; ++t) {
    const i32x8 a0 = cat8(lds_load<u32x4>(la.ka[2 * t] + KOFF), lds_load<u32x4>(la.ka[2 * t + 1] + KOFF));
    const i32x8 a1 = cat8(lds_load<u32x4>(la.ka[2 * t] + KOFF + 16 * D),
                          lds_load<u32x4>(la.ka[2 * t + 1] + KOFF + 16 * D));
    s0 = mfma8(a0, w.qf[t], s0);
    s1 = mfma8(a1, w.qf[t], s1);
  }
}

// -inf outside this lane's key band [row_lo, row_hi].
__device__ __forceinline__ void mask8(f32x16& s0, f32x16& s1, int k0, int row_lo, int row_hi, int hf) {
  const int hi = row_hi - k0 - 32 * hf;
  const int lo = row_lo - k0 - 32 * hf;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r > hi || r < lo) s0[r] = -INFINITY;
    if (r + 16 > hi || r + 16 < lo) s1[r] = -INFINITY;
  }
}

// exp2(s * sl2 - mref) in place; returns this lane's fp32 sum.
__device__ __forceinline__ float exp8(f32x16& s0, f32x16& s1, float sl2, float mref) {
  float rs = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], sl2, -mref));
    rs += s0[r];
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], sl2, -mref));
    rs += s1[r];
  }
  return rs;
}

__device__ __forceinline__ int pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// One 64-key tile for one wave.  The probabilities are formed against the
// reference maximum m_run and scaled by 2^7; to be representable they must not
// exceed 448, i.e. no score may exceed the reference by more than log2(3.5).
// The tile's row maxima are taken from the raw scores first; only when some
// row of the wave exceeds its reference by more than kHead (and while a row
// has no reference yet) are the references raised to the tile maxima and the
// accumulators and sums rescaled.  Each probability is then at most
// 2^(7 + kHead) < 448, and the exponentials are computed once.
constexpr float kHead = 1.75f;

// Softmax of one tile from its raw scores: P (scaled by 2^7, rounded to e4m3)
// packed as the B operand of the second product.
template <int D>
__device__ __forceinline__ void softmax8(Fp8Rows<D>& w, f32x16& s0, f32x16& s1, i32x8& pw, bool need_mask, int k0,
                                         int row_lo, int row_hi, float sl2, int lane) {
  constexpr int NB = D / 32;
  const int hf = lane >> 5;
  if (need_mask) mask8(s0, s1, k0, row_lo, row_hi, hf);
  // IEEE maximum (NaN-propagating): gfx950 folds it into v_maximum3_f32 without the
  // canonicalising copies that fmaxf needs on matrix-product results
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s0[r], s1[r]));
  mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 32)) * sl2;
  if (__ballot(mx > w.m_run + kHead)) {
    const float m_new = fmaxf(w.m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(w.m_run - m_use);
    w.l_run *= alpha;
    w.lsum *= alpha;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) w.acc[nb] *= alpha;
    w.m_run = m_new;
  }
  const float m_use = w.m_run == -INFINITY ? 0.f : w.m_run;  // all scores so far masked: they stay -inf
  w.l_run += exp8(s0, s1, sl2, m_use - kPLog2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pw[i] = pack4(s0[4 * i], s0[4 * i + 1], s0[4 * i + 2], s0[4 * i + 3]);
    pw[4 + i] = pack4(s1[4 * i], s1[4 * i + 1], s1[4 * i + 2], s1[4 * i + 3]);
  }
}

// O^T += V^T P^T and the row sums of the rounded P (against a block of ones).
template <int D, unsigned VOFF>
__device__ __forceinline__ void pv8(Fp8Rows<D>& w, const Fp8Addr<D>& la, i32x8 ones, const i32x8& pw) {
  w.lsum = mfma8(ones, pw, w.lsum);
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
    const i32x8 a = cat8(lds_load<u32x4>(la.va[0] + VOFF + nb * 32 * 64),
                         lds_load<u32x4>(la.va[1] + VOFF + nb * 32 * 64));
    w.acc[nb] = mfma8(a, pw, w.acc[nb]);
  }
}

template <int D, unsigned KOFF, unsigned VOFF>
__device__ __forceinline__ void tile8(Fp8Rows<D>& w, const Fp8Addr<D>& la, i32x8 ones, bool need_mask, int k0,
                                      int row_lo, int row_hi, float sl2, int lane) {
  f32x16 s0, s1;
  i32x8 pw;
  qk8<D, KOFF>(w, la, s0, s1);
  softmax8(w, s0, s1, pw, need_mask, k0, row_lo, row_hi, sl2, lane);
  pv8<D, VOFF>(w, la, ones, pw);
}

// Forward kernel.  Workgroup = NW waves = 32*NW query rows of one (batch, head);
// same work order, band handling and LDS double buffering as the bf16 kernel.
template <int D, int NW>
__global__ void __launch_bounds__(64 * NW, 8 / NW) fwd_fp8_kernel(Fp8Params p) {
  constexpr int BR = 32 * NW;
  constexpr int NB = D / 32;
  constexpr int TILE = kBC8 * D;  // bytes of one K tile (= one V^T tile)
  static_assert((4 * D) % (64 * NW) == 0, "tile must split evenly over the threads");

  __shared__ __attribute__((aligned(1024))) char lds[2][2][TILE];  // [stage][K=0 / V^T=1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;
  const int col = lane & 31;

  const int n_qb = (p.n_q + BR - 1) / BR;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / n_qb;
  int qb = L % n_qb;
  const int wl = p.wl, wr = p.wr;
  if (wl < 0 && wr >= 0) qb = n_qb - 1 - qb;  // causal-like band: heaviest query blocks first
  const int q0 = qb * BR;
  const int q0w = q0 + wave * 32;
  const int row = q0w + col;

  int klo = 0, khi = p.n_k, klo_w = 0, khi_w = p.n_k, row_lo = 0, row_hi = p.n_k - 1;
  if (wr >= 0) {
    khi = min(khi, q0 + BR + wr);
    khi_w = min(khi_w, q0w + 32 + wr);
    row_hi = min(row_hi, row + wr);
  }
  if (wl >= 0) {
    klo = max(klo, q0 - wl);
    klo_w = max(klo_w, q0w - wl);
    row_lo = max(row_lo, row - wl);
  }
  const int kfirst = klo / kBC8 * kBC8;
  const int n_tiles = khi > kfirst ? (khi - kfirst + kBC8 - 1) / kBC8 : 0;

  const float dsq = p.dsq[bh], dsk = p.dsk[bh], dsv = p.dsv[bh];
  const float sl2 = fmaxf(fabsf(p.scale) * kLog2e * dsq * dsk, FLT_MIN);

  const i32x4 krs = raw_rsrc(p.k + (long long)bh * p.n_k * D, (long long)khi * D);
  const unsigned vbytes = (unsigned)(D * p.vt_stride);
  const i32x4 vrs = raw_rsrc(p.vt + (long long)bh * D * p.vt_stride, vbytes);

  Fp8Rows<D> w;
  {
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q + (long long)bh * p.n_q * D, (long long)p.n_q * D);
    const unsigned sg = p.scale < 0.f ? 0x80808080u : 0u;  // negate Q so the multiplier stays positive
    const u32x4 sign = {sg, sg, sg, sg};
#pragma unroll
    for (int t = 0; t < D / 64; ++t) {
      const unsigned off = (unsigned)(row * D + 64 * t + 32 * hf);
      const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0)) ^ sign;
      const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off + 16, 0, 0)) ^ sign;
      w.qf[t] = cat8(lo, hi);
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) w.acc[nb] = f32x16{};
  w.lsum = f32x16{};
  w.m_run = -INFINITY;
  w.l_run = 0.f;

  Fp8Addr<D> la;
  {
    const unsigned kbase = (unsigned)(uintptr_t)(const lds_void*)&lds[0][0][0];
    const unsigned vbase = (unsigned)(uintptr_t)(const lds_void*)&lds[0][1][0];
    const int kr = kperm<D>(col);
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const int c = 4 * (j >> 1) + 2 * hf + (j & 1);
      la.ka[j] = kbase + kr * D + 16 * (c ^ kswz<D>(kr));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) la.va[h] = vbase + col * 64 + 16 * ((2 * hf + h) ^ vswz(col));
#pragma unroll
    for (int j = 0; j < D / 32; ++j) asm volatile("" : "+v"(la.ka[j]));
    asm volatile("" : "+v"(la.va[0]), "+v"(la.va[1]));
  }
  constexpr unsigned STAGE = 2 * TILE;
  i32x8 ones = {(int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes};
  asm volatile("" : "+v"(ones));  // kept in registers rather than rebuilt per tile

#define FA2_STEP8(STG, k0_)                                                                            \
  do {                                                                                               \
    const int kk = (k0_);                                                                            \
    if (kk < khi_w && kk + kBC8 > klo_w)                                                             \
      tile8<D, STG * STAGE, STG * STAGE>(                                                            \
          w, la, ones,                                                                               \
          (kk + kBC8 > p.n_k) || (wr >= 0 && kk + kBC8 - 1 > q0w + wr) || (wl >= 0 && kk < q0w + 31 - wl), \
          kk, row_lo, row_hi, sl2, lane);                                                            \
  } while (0)

  if (n_tiles > 0) issue_tile8<D, NW>(krs, vrs, vbytes, p.vt_stride, lds[0][0], lds[0][1], kfirst, wave, lane);
  for (int j = 0; j < n_tiles; j += 2) {
    const int k0 = kfirst + j * kBC8;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < n_tiles)
      issue_tile8<D, NW>(krs, vrs, vbytes, p.vt_stride, lds[1][0], lds[1][1], k0 + kBC8, wave, lane);
    FA2_STEP8(0, k0);
    if (j + 1 < n_tiles) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (j + 2 < n_tiles)
        issue_tile8<D, NW>(krs, vrs, vbytes, p.vt_stride, lds[0][0], lds[0][1], k0 + 2 * kBC8, wave, lane);
      FA2_STEP8(1, k0 + kBC8);
    }
  }
#undef FA2_STEP8

  // ---- epilogue ----
  const float l_tot = w.l_run + __shfl_xor(w.l_run, 32);
  const float lq = w.lsum[0];
  // O = dsv * acc / lq (a row with no visible key: O = 0), staged in the tiles' space once every
  // wave is done with it and written as whole rows
  static_assert(NW * kStagedRows<D> <= (int)sizeof(lds), "the staged rows fit");
  u32x2 out[NB][4];
  scaled_rows<D>(w.acc, lq > 0.f ? dsv / lq : 0.f, out);
  __syncthreads();
  write_rows<D>(out, (unsigned)(uintptr_t)(const lds_void*)&lds[0][0][0] + (unsigned)(wave * kStagedRows<D>),
                p.o + ((long long)bh * p.n_q + q0w) * D, p.n_q - q0w, lane);
  if (row >= p.n_q) return;
  if (hf == 0)
    p.lse[(long long)bh * p.n_q + row] = l_tot > 0.f ? (w.m_run + __log2f(l_tot) - kPLog2) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Single-query decode over an FP8 K/V cache: one workgroup (4 waves) per
// (batch, head) streams the head's K and V codes (both in row layout) from HBM.
// With one query row both products are matrix-vector shaped, so the kernel
// uses VALU dot products in fp32 on the decoded codes, like the bf16 decode
// kernel: D/16 lanes share one key row (16 codes each), every lane keeps
// kDec8U keys' K and V loads in flight, each wave runs its own online softmax
// over the steps it owns, and the four wave partials are merged at the end.
// The probabilities stay fp32 (only the inputs are 8-bit).
constexpr int kDec8Threads = 256;
constexpr int kDec8U = 16;
constexpr int kNt = 2;  // buffer-load cache policy: non-temporal (each code is read once)

__device__ __forceinline__ void decode16(u32x4 w, float (&f)[16]) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned wi = w[i];  // named copy: bit-casting a vector element in place reads element 0
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wi, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wi, true);
    f[4 * i] = lo.x;
    f[4 * i + 1] = lo.y;
    f[4 * i + 2] = hi.x;
    f[4 * i + 3] = hi.y;
  }
}

template <int D>
__global__ void __launch_bounds__(kDec8Threads) decode_fp8_kernel(Fp8Params p) {
  constexpr int LPK = D / 16;          // lanes per key row
  constexpr int KPW = 64 / LPK;        // key rows per wave-wide load
  constexpr int STEP = KPW * kDec8U;   // keys per wave step
  constexpr int NWAVE = kDec8Threads / 64;
  __shared__ float part_acc[NWAVE][D];
  __shared__ float part_m[NWAVE], part_l[NWAVE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane % LPK, kg = lane / LPK;
  const int bh = xcd_remap(blockIdx.x, gridDim.x);
  const int kend = p.n_k;

  const float sl2 = fmaxf(fabsf(p.scale) * kLog2e * p.dsq[bh] * p.dsk[bh], FLT_MIN);
  const float dsv = p.dsv[bh];
  // loads past key kend return zero (range check on the per-lane offset)
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + (long long)bh * p.n_k * D, (long long)kend * D);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + (long long)bh * p.n_k * D, (long long)kend * D);

  float qv[16];
  decode16(*reinterpret_cast<const u32x4*>(p.q + (long long)bh * D + sub * 16), qv);
  if (p.scale < 0.f) {
#pragma unroll
    for (int e = 0; e < 16; ++e) qv[e] = -qv[e];  // keep the folded multiplier positive
  }

  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  float m_run = -INFINITY;  // log2 units, uniform over the wave
  float l_run = 0.f;        // this key group's share

  for (int k0 = wave * STEP; k0 < kend; k0 += NWAVE * STEP) {
    u32x4 kr[kDec8U], vr[kDec8U];
#pragma unroll
    for (int u = 0; u < kDec8U; ++u) {
      const unsigned off = (unsigned)((k0 + u * KPW + kg) * D + sub * 16);
      kr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, kNt));
      vr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, kNt));
    }
    float sc[kDec8U];
    float mloc = -INFINITY;
#pragma unroll
    for (int u = 0; u < kDec8U; ++u) {
      float kf[16];
      decode16(kr[u], kf);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) dot = __builtin_fmaf(qv[e], kf[e], dot);
#pragma unroll
      for (int x = LPK / 2; x >= 1; x >>= 1) dot += __shfl_xor(dot, x);
      sc[u] = (k0 + u * KPW + kg < kend) ? dot * sl2 : -INFINITY;
      mloc = fmaxf(mloc, sc[u]);
    }
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, x));
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kDec8U; ++u) {
      const float pk = __builtin_amdgcn_exp2f(sc[u] - m_use);
      ps += pk;
      float vf[16];
      decode16(vr[u], vf);
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = __builtin_fmaf(pk, vf[e], acc[e]);
    }
    l_run = l_run * alpha + ps;
  }

  // fold the key groups of the wave (lanes with equal `sub`)
#pragma unroll
  for (int x = LPK; x < 64; x <<= 1) {
    l_run += __shfl_xor(l_run, x);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] += __shfl_xor(acc[e], x);
  }
  if (kg == 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) part_acc[wave][sub * 16 + e] = acc[e];
  }
  if (lane == 0) {
    part_m[wave] = m_run;
    part_l[wave] = l_run;
  }
  __syncthreads();

  // merge the wave partials (log2 units); the single query row sees key 0, so lsum > 0
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < NWAVE; ++v) M = fmaxf(M, part_m[v]);
  float wgt[NWAVE];
  float lsum = 0.f;
#pragma unroll
  for (int v = 0; v < NWAVE; ++v) {
    wgt[v] = part_m[v] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(part_m[v] - M);
    lsum += wgt[v] * part_l[v];
  }
  const float inv = dsv / lsum;
  for (int dd = tid; dd < D; dd += kDec8Threads) {
    float t = 0.f;
#pragma unroll
    for (int v = 0; v < NWAVE; ++v) t += wgt[v] * part_acc[v][dd];
    p.o[(long long)bh * D + dd] = __builtin_bit_cast(uint16_t, (__bf16)(t * inv));
  }
  if (tid == 0) p.lse[bh] = (M + __log2f(lsum)) * kLn2;
}

// ---------------------------------------------------------------------------
// Quantiser.  Four launches on the caller's stream:
//   clear     amax[bh] = 0 (the descale array holds amax bit patterns until the end)
//   amax      per-workgroup max |x| of a chunk, folded in with an atomic max on the
//             bit pattern (non-negative floats order like their bit patterns)
//   quantise  code = e4m3 RNE of fp32(x) * fp32(448 / amax), row layout or transposed
//   finalise  descale[bh] = fp32(amax / 448), 1 for an all-zero slice
constexpr int kQThreads = 256;
constexpr int kAmaxElems = kQThreads * 64;  // bf16 elements per amax workgroup

__global__ void __launch_bounds__(kQThreads) q8_clear(unsigned* amax_bits, int n) {
  const int i = blockIdx.x * kQThreads + threadIdx.x;
  if (i < n) amax_bits[i] = 0u;
}

__global__ void __launch_bounds__(kQThreads) q8_amax(const uint16_t* x, unsigned* amax_bits, long long per_head) {
  const int bh = blockIdx.y;
  const uint16_t* xh = x + (long long)bh * per_head;
  const long long base = (long long)blockIdx.x * kAmaxElems;
  unsigned m = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const long long e = base + (long long)(i * kQThreads + threadIdx.x) * 8;
    if (e < per_head) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xh + e);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const unsigned wv = v[c];
        m = max(m, (wv & 0x7fffu) << 16);
        m = max(m, (wv >> 16 & 0x7fffu) << 16);
      }
    }
  }
#pragma unroll
  for (int x2 = 32; x2 >= 1; x2 >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, x2));
  __shared__ unsigned wm[kQThreads / 64];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = wm[0];
    for (int i = 1; i < kQThreads / 64; ++i) t = max(t, wm[i]);
    atomicMax(amax_bits + bh, t);
  }
}

__device__ __forceinline__ float q8_inv(unsigned amax_bits) {
  const float amax = __builtin_bit_cast(float, amax_bits);
  return amax > 0.f ? 448.f / amax : 1.f;
}

__device__ __forceinline__ float bf16f(unsigned h) { return __builtin_bit_cast(float, h << 16); }

// Row layout: 16 elements per thread.
__global__ void __launch_bounds__(kQThreads) q8_rows(const uint16_t* x, uint8_t* codes, const unsigned* amax_bits,
                                                     long long per_head) {
  const int bh = blockIdx.y;
  const long long e = ((long long)blockIdx.x * kQThreads + threadIdx.x) * 16;
  if (e >= per_head) return;
  const float inv = q8_inv(amax_bits[bh]);
  const uint16_t* xp = x + (long long)bh * per_head + e;
  const u32x4 a = *reinterpret_cast<const u32x4*>(xp);
  const u32x4 b = *reinterpret_cast<const u32x4*>(xp + 8);
  float f[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const unsigned wa = a[c], wb = b[c];
    f[2 * c] = bf16f(wa & 0xffffu) * inv;
    f[2 * c + 1] = bf16f(wa >> 16) * inv;
    f[8 + 2 * c] = bf16f(wb & 0xffffu) * inv;
    f[8 + 2 * c + 1] = bf16f(wb >> 16) * inv;
  }
  u32x4 out;
#pragma unroll
  for (int c = 0; c < 4; ++c) out[c] = (unsigned)pack4(f[4 * c], f[4 * c + 1], f[4 * c + 2], f[4 * c + 3]);
  *reinterpret_cast<u32x4*>(codes + (long long)bh * per_head + e) = out;
}

// Transposed: one workgroup per (batch*head, 64-key block) writes
// codes[bh][d][k0 .. k0 + 63] (row stride vt_stride, keys >= N coded as 0).
template <int D>
__global__ void __launch_bounds__(kQThreads) q8_vt(const uint16_t* x, uint8_t* codes, const unsigned* amax_bits,
                                                   int n, int vt_stride) {
  constexpr int KPT = 64 * D / kQThreads;  // keys per thread: 32 (D = 128) or 16 (D = 64)
  __shared__ uint16_t tile[64][D + 8];     // +8: row starts on a different bank
  const int bh = blockIdx.y;
  const int k0 = blockIdx.x * 64;
  const float inv = q8_inv(amax_bits[bh]);
  const uint16_t* xh = x + (long long)bh * n * D;
  for (int s = threadIdx.x; s < 64 * D / 8; s += kQThreads) {
    const int r = s / (D / 8), c = s % (D / 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k0 + r < n) v = *reinterpret_cast<const u32x4*>(xh + (long long)(k0 + r) * D + 8 * c);
    *reinterpret_cast<u32x4*>(&tile[r][8 * c]) = v;
  }
  __syncthreads();
  const int dcol = threadIdx.x % D;
  const int kg = threadIdx.x / D;
  uint8_t* out = codes + ((long long)bh * D + dcol) * vt_stride;
#pragma unroll
  for (int c = 0; c < KPT / 16; ++c) {
    const int key = k0 + kg * KPT + 16 * c;
    if (key >= vt_stride) break;
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kk = kg * KPT + 16 * c + 4 * q;
      o[q] = (unsigned)pack4(bf16f(tile[kk][dcol]) * inv, bf16f(tile[kk + 1][dcol]) * inv,
                             bf16f(tile[kk + 2][dcol]) * inv, bf16f(tile[kk + 3][dcol]) * inv);
    }
    *reinterpret_cast<u32x4*>(out + key) = o;
  }
}

__global__ void __launch_bounds__(kQThreads) q8_finalise(float* descale, int n) {
  const int i = blockIdx.x * kQThreads + threadIdx.x;
  if (i >= n) return;
  const float amax = descale[i];  // still the amax bit pattern, read as a float
  descale[i] = amax > 0.f ? amax / 448.f : 1.f;
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Params& p, hipStream_t stream) {
  constexpr int NW = 4;
  const int n_qb = (p.n_q + 32 * NW - 1) / (32 * NW);
  const dim3 grid((unsigned)((long long)n_qb * p.B * p.H));
  if (p.d == 128)
    hipLaunchKernelGGL((fwd_fp8_kernel<128, NW>), grid, dim3(64 * NW), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<64, NW>), grid, dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_fp8(const Fp8Params& p, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)p.B * p.H));
  if (p.d == 128)
    hipLaunchKernelGGL(decode_fp8_kernel<128>, grid, dim3(kDec8Threads), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_fp8_kernel<64>, grid, dim3(kDec8Threads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const QuantParams& p, hipStream_t stream) {
  const int nbh = p.B * p.H;
  const long long per_head = (long long)p.n * p.d;
  unsigned* amax_bits = reinterpret_cast<unsigned*>(p.descale);
  const dim3 blk(kQThreads);
  hipLaunchKernelGGL(q8_clear, dim3((nbh + kQThreads - 1) / kQThreads), blk, 0, stream, amax_bits, nbh);
  hipLaunchKernelGGL(q8_amax, dim3((unsigned)((per_head + kAmaxElems - 1) / kAmaxElems), nbh), blk, 0, stream, p.x,
                     amax_bits, per_head);
  if (!p.transposed) {
    const long long per_block = (long long)kQThreads * 16;
    hipLaunchKernelGGL(q8_rows, dim3((unsigned)((per_head + per_block - 1) / per_block), nbh), blk, 0, stream, p.x,
                       p.codes, amax_bits, per_head);
  } else if (p.d == 128) {
    hipLaunchKernelGGL(q8_vt<128>, dim3((p.n + 63) / 64, nbh), blk, 0, stream, p.x, p.codes, amax_bits, p.n,
                       p.vt_stride);
  } else {
    hipLaunchKernelGGL(q8_vt<64>, dim3((p.n + 63) / 64, nbh), blk, 0, stream, p.x, p.codes, amax_bits, p.n,
                       p.vt_stride);
  }
  hipLaunchKernelGGL(q8_finalise, dim3((nbh + kQThreads - 1) / kQThreads), blk, 0, stream, p.descale, nbh);
  return hipGetLastError();
}

}  // namespace fa2
