// FlashAttention-2 style exact-attention forward for gfx950 (MI355X).
//
// One workgroup owns a block of query rows of one (batch, head) and streams the
// key/value blocks it can see through LDS (FlashAttention-2 walkthrough page,
// "launch grid" and "kernel main loop" sections; synthesis page, section 2
// items 1-3).  Each wave owns 32 query rows and runs both products on its own
// (split-Q, no inter-wave exchange of partial results); every wave computes
// (synthesis page, section 2, HipKittens paragraph: no producer-only waves
// under static register allocation).
//
// Per 64-key tile, each wave:
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, K from LDS, Q resident in VGPRs
//   mask             only on tiles that cross the diagonal or the key tail
//   online softmax   per-row reference maximum and sums, base-2 exponent with
//                    scale*log2(e) folded into one FMA; P stays in registers
//   O^T += V^T P^T   v_mfma_f32_32x32x16_bf16, V read transposed from LDS with
//                    ds_read_b64_tr_b16, P converted to bf16 (RNE)
// and the epilogue divides once per row (deferred normalisation, synthesis
// page, section 2 item 1) and writes O (bf16) and LSE = m + ln l (fp32).
//
// Computing S transposed puts one query row in each lane column, so the
// accumulator of S^T is directly the B operand of the second product and every
// per-row statistic lives in one lane pair (lanes c and c+32).
#include "fa2_device.h"
#include "fa2_internal.h"

#include <math.h>

#include <type_traits>

namespace fa2 {
namespace {

constexpr int kBC = 64;  // keys per K/V tile

// Per-wave state of one 32-row query block: the Q fragment (B operand of
// S^T = K Q^T; lane holds Q[row][16t + 8hf .. +7]), the O^T accumulator
// (acc[nb][4g + i] = O^T[32nb + 8g + 4hf + i][row]), the reference maximum of
// the scaled scores in log2 units, and this lane's shares of the two sums.
template <int D>
struct WaveRows {
  bf16x8 qf[D / 16];
  f32x16 acc[D / 32];
  float m_run;
  float l_run;   // sum of fp32 probabilities (for LSE)
  float l16;     // sum of the bf16-rounded probabilities (normalises O)
};

// Issue the loads of one K tile and one V tile (kBC rows from key k0) into
// LDS.  Load i of a wave fills physical slots (i*NW + wave)*64 .. +63; the
// lane owning slot s fetches the (row, chunk) that the swizzle stores there.
// The whole byte offset goes in the per-lane voffset, which the buffer range
// check applies to.
template <int D, int NW>
__device__ __forceinline__ void issue_tile(i32x4 krs, i32x4 vrs, const char* kdst, const char* vdst, int k0,
                                           int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int NLD = kBC * CPR / (64 * NW);
  const unsigned toff = (unsigned)k0 * D * 2;
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int s = (i * NW + wave) * 64 + lane;
    const int r = s / CPR;
    const int c = (s % CPR) ^ (swz<D>(r, 0) - r * CPR);
    const unsigned off = (unsigned)((r * D + c * 8) * 2) + toff;
    const int sbase = (i * NW + wave) * 64 * 16;
    lds_dma16(krs, kdst + sbase, off);
    lds_dma16(vrs, vdst + sbase, off);
  }
}

// S^T = K Q^T for one kBC-key tile (two 32-key blocks, two interleaved
// accumulation chains).  KOFF: byte offset of the tile's K buffer relative to
// the addresses in `la`.  s{kb}[r] is the score of query `row` against key
// k0 + kb*32 + 8*(r/4) + 4*hf + r%4.
template <int D, unsigned KOFF>
__device__ __forceinline__ void qk_tile(const WaveRows<D>& w, const LdsAddr<D>& la, f32x16& s0, f32x16& s1) {
  constexpr unsigned ROW = D * 2;
  s0 = f32x16{};
  s1 = f32x16{};
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const bf16x8 a0 = lds_load<bf16x8>(la.ka[t] + KOFF);
    const bf16x8 a1 = lds_load<bf16x8>(la.ka[t] + KOFF + 32 * ROW);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, w.qf[t], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, w.qf[t], s1, 0, 0, 0);
  }
}


// S^T = K Q^T with the K operands read PF pairs ahead of their products.  Left
// to itself the scheduler keeps one pair in flight, and an LDS read takes longer
// than the two products it feeds (64 cycles), so every pair stalled; the
// scheduling-group barriers pin the order (PF pairs of reads, then per step two
// products and the next pair of reads).
template <int D, unsigned KOFF, int PF>
__device__ __forceinline__ void qk_tile_pf(const WaveRows<D>& w, const LdsAddr<D>& la, f32x16& s0, f32x16& s1) {
  constexpr unsigned ROW = D * 2;
  constexpr int KT = D / 16;
  bf16x8 a[PF][2];
#pragma unroll
  for (int t = 0; t < PF; ++t) {
    a[t][0] = lds_load<bf16x8>(la.ka[t] + KOFF);
    a[t][1] = lds_load<bf16x8>(la.ka[t] + KOFF + 32 * ROW);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
  s0 = f32x16{};
  s1 = f32x16{};
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t % PF][0], w.qf[t], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t % PF][1], w.qf[t], s1, 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    if (t + PF < KT) {
      a[t % PF][0] = lds_load<bf16x8>(la.ka[t + PF] + KOFF);
      a[t % PF][1] = lds_load<bf16x8>(la.ka[t + PF] + KOFF + 32 * ROW);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  }
}

// -inf for keys outside this lane's row band [row_lo, row_hi] (the band already
// clipped to the key tail).  Key k0 + 4hf + c is visible iff lo <= c <= hi; c is
// a compile-time constant per register.
__device__ __forceinline__ void mask_scores(f32x16& s0, f32x16& s1, int k0, int row_lo, int row_hi, int hf) {
  const int hi = row_hi - k0 - 4 * hf;
  const int lo = row_lo - k0 - 4 * hf;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int c = 8 * (r >> 2) + (r & 3);
    if (c > hi || c < lo) s0[r] = -INFINITY;
    if (c + 32 > hi || c + 32 < lo) s1[r] = -INFINITY;
  }
}

// Probabilities exp2(s * sl2 - m_use) in place; returns this lane's fp32 sum.
__device__ __forceinline__ float exp_tile(f32x16& s0, f32x16& s1, float sl2, float m_use) {
  float rs = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], sl2, -m_use));
    rs += s0[r];
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], sl2, -m_use));
    rs += s1[r];
  }
  return rs;
}

// acc + the sum of the 32 bf16 probabilities in pb (v_dot2 against (1, 1)).
// Dwords are copied into named values first: bit-casting a vector element in
// place reads element 0.
__device__ __forceinline__ float sum_bf16(const bf16x8 (&pb)[4], float acc) {
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = __builtin_bit_cast(u32x4, pb[i]);
    const unsigned v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v0), ones, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v1), ones, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v2), ones, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v3), ones, acc, false);
  }
  return acc;
}

// One kBC-key tile for one wave: S^T = K Q^T, mask (only when need_mask),
// online softmax, O^T += V^T P^T.  KOFF / VOFF: byte offsets of this stage's K
// and V tiles relative to the addresses in `la`.
//
// Softmax against a reference maximum.  The probabilities are first formed
// against the current reference m_run, with no max pass and no rescale of O.
// Only when a lane's tile sum exceeds kLazyBound (so no probability can exceed
// it), or when some row has no reference yet, is the tile redone exactly: new
// maximum, rescale of O and of both sums, probabilities again.  The result does
// not depend on the reference: O = acc / l16 with l16 the sum of the bf16
// probabilities exactly as accumulated (each O row is an exact convex
// combination of V rows), and LSE = m_run + log2(l_run) with l_run the fp32 sum.
constexpr float kLazyBound = 2048.f;

template <int D, unsigned KOFF, unsigned VOFF>
__device__ __forceinline__ void tile_step(WaveRows<D>& w, const LdsAddr<D>& la, bool need_mask, int k0, int row_lo,
                                          int row_hi, float sl2, int lane) {
  constexpr int NB = D / 32;
  constexpr unsigned ROW = D * 2;
  const int hf = lane >> 5;
  f32x16 s0, s1;
  qk_tile_pf<D, KOFF, 2>(w, la, s0, s1);
  // d = 64: the softmax is the longer part of a tile, and the four resident waves of a SIMD
  // (different workgroups) drift into the same phase; raising the priority of whichever wave
  // is in its softmax keeps the vector unit fed while the others issue their products
  // (measured +2 to +6 % at B8 H16 N2048; no gain at d = 128)
  if (D == 64) __builtin_amdgcn_s_setprio(3);
  if (need_mask) mask_scores(s0, s1, k0, row_lo, row_hi, hf);

  bool exact = __ballot(w.m_run == -INFINITY) != 0;  // some row has no reference yet
  float rs = 0.f;
  if (!exact) {
    rs = exp_tile(s0, s1, sl2, w.m_run);
    if (__ballot(rs > kLazyBound)) {
      exact = true;
      qk_tile<D, KOFF>(w, la, s0, s1);  // scores again (the K tile is still in LDS)
      if (need_mask) mask_scores(s0, s1, k0, row_lo, row_hi, hf);
    }
  }
  if (exact) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
    const float m_new = fmaxf(w.m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(w.m_run - m_use);
    w.l_run *= alpha;
    w.l16 *= alpha;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) w.acc[nb] *= alpha;
    w.m_run = m_new;
    rs = exp_tile(s0, s1, sl2, m_use);
  }
  w.l_run += rs;
  bf16x8 pb[4];
  pb[0] = cvt_bf16x8(slice8(s0, 0));
  pb[1] = cvt_bf16x8(slice8(s0, 1));
  pb[2] = cvt_bf16x8(slice8(s1, 0));
  pb[3] = cvt_bf16x8(slice8(s1, 1));
  w.l16 = sum_bf16(pb, w.l16);
  if (D == 64) __builtin_amdgcn_s_setprio(0);

#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const unsigned roff = VOFF + (kb * 32 + 16 * t) * ROW;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<lds_i16x4*>((uintptr_t)(la.va[2 * nb] + roff)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<lds_i16x4*>((uintptr_t)(la.va[2 * nb + 1] + roff)));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        w.acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[2 * kb + t], w.acc[nb], 0, 0, 0);
      }
    }
}

// Forward / split-KV partial kernel.
//   D   head dim (64 or 128)
//   NW  waves per workgroup; the query block is B_r = 32*NW rows
//   SPLIT  false: write O and LSE;  true: write the fp32 partial (acc, m, l)
//          of the key chunk selected by the workgroup id.
// Kernel arguments beyond FwdParams: sl2 = max(|scale| * log2 e, FLT_MIN) and
// qsign = 0x80008000 when scale < 0 (Q is negated in registers so that the
// folded multiplier stays positive), else 0.
//
// K/V tiles go straight from HBM/L2 into LDS (buffer_load ... lds).  Two LDS
// stages, each its own __shared__ object so that the compiler can see that
// reading one stage does not depend on the loads in flight into the other:
// tile j+1 streams in while tile j computes, and one barrier per tile both
// publishes tile j and retires the buffer of tile j-1.
//   MASK   stream only the key tiles that the block mask row of the workgroup's
//          query block marks (p.bmask; 128-row workgroups, NW == 4, one mask row each)
// Tile t of a wave's key range (keys kfirst + kBC t ..): live when ja <= t < jb, and
// masked when t >= jmh (it reaches past kend or past the band's upper edge) or t < jml
// (it starts before the lower edge).  Taken once per wave, so that each tile costs two
// comparisons; >> 6 is a floor division by kBC, negative values included.
struct TileBounds {
  int ja, jb, jmh, jml;
};
__device__ __forceinline__ TileBounds tile_bounds(int kfirst, int n_tiles, int klo_w, int khi_w, int kend, int q0w,
                                                  int wl, int wr) {
  static_assert(kBC == 64, "tile bounds divide by 64");
  TileBounds b;
  b.ja = (klo_w - kfirst) >> 6;
  b.jb = min(n_tiles, (khi_w - kfirst + 63) >> 6);
  b.jmh = wr >= 0 ? min((kend - kfirst) >> 6, ((q0w + wr - 63 - kfirst) >> 6) + 1) : (kend - kfirst) >> 6;
  b.jml = wl >= 0 ? (q0w + 31 - wl - kfirst + 63) >> 6 : -(1 << 30);
  return b;
}

template <int D, int NW, bool SPLIT, bool MASK = false>
__global__ void __launch_bounds__(64 * NW, 8 / NW) fwd_kernel(FwdParams p, float sl2, unsigned qsign) {
  static_assert(!MASK || (NW == 4 && !SPLIT), "block masks are read per 128-row workgroup");
  constexpr int BR = 32 * NW;
  constexpr int KT = D / 16;
  constexpr int NB = D / 32;
  constexpr int TILE_BYTES = kBC * D * 2;
  static_assert((kBC * D / 8) % (64 * NW) == 0, "tile must split evenly over the threads");

  __shared__ __attribute__((aligned(1024))) char lds[2][2][TILE_BYTES];  // [stage][K=0 / V=1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;           // which 8-wide k half of an MFMA operand this lane holds
  const int col = lane & 31;          // query row (within the wave) of this lane

  // ---- workgroup -> (batch*head, query block, key chunk) ----
  const int n_qb = (p.n_q + BR - 1) / BR;
  int L = wg_logical(p.sched);
  int split = 0;
  if (SPLIT) {
    split = L % p.num_splits;
    L /= p.num_splits;
  }
  const int wl = p.wl, wr = p.wr;  // key band [i - wl, i + wr] of query i; -1: unbounded
  int bh, qb;
  // causal-like band: heaviest query blocks first
  wg_coords(L, n_qb, p.B * p.H, p.sched, wl < 0 && wr >= 0, bh, qb);
  const int q0 = qb * BR;
  const int q0w = q0 + wave * 32;
  const int row = q0w + col;

  int kbeg = 0, kend = p.n_k;
  if (SPLIT) {
    const long long b = (long long)split * p.split_len;
    kbeg = b < p.n_k ? (int)b : p.n_k;
    kend = kbeg + p.split_len < p.n_k ? kbeg + p.split_len : p.n_k;
  }
  // Keys in [klo, khi) are visible to some row of the workgroup, keys in
  // [klo_w, khi_w) to some row of this wave, keys in [row_lo, row_hi] to this
  // lane's row.  Tiles stay aligned to kbeg; the first one holds klo.
  int klo = kbeg, khi = kend, klo_w = kbeg, khi_w = kend, row_lo = kbeg, row_hi = kend - 1;
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
  const int kfirst = kbeg + (klo - kbeg) / kBC * kBC;
  const int n_tiles = khi > kfirst ? (khi - kfirst + kBC - 1) / kBC : 0;

  const uint16_t* Qh = p.q + (long long)bh * p.n_q * D;
  const i32x4 krs = raw_rsrc(p.k + (long long)bh * p.n_k * D, (long long)khi * D * 2);
  const i32x4 vrs = raw_rsrc(p.v + (long long)bh * p.n_k * D, (long long)khi * D * 2);

  WaveRows<D> w;
  {
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qh, (long long)p.n_q * D * 2);
    const u32x4 sign = {qsign, qsign, qsign, qsign};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const u32x4 raw = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, ((unsigned)row * D + 16 * t + 8 * hf) * 2u, 0, 0));
      w.qf[t] = as_bf16x8(raw ^ sign);
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) w.acc[nb] = f32x16{};
  w.m_run = -INFINITY;
  w.l_run = 0.f;
  w.l16 = 0.f;

  LdsAddr<D> la;
  make_lds_addr<D>(la, (unsigned)(uintptr_t)(const lds_void*)&lds[0][0][0], lane);
  constexpr unsigned STAGE = 2 * TILE_BYTES;

  // A tile is skipped when no row of this wave sees any of its keys, and
  // masked when it crosses either edge of the wave's band or the key tail.
  const TileBounds bnd = tile_bounds(kfirst, n_tiles, klo_w, khi_w, kend, q0w, wl, wr);
#define FA2_STEP(STG, t_)                                                                  \
  do {                                                                                     \
    const int t = (t_);                                                                    \
    if (t >= bnd.ja && t < bnd.jb)                                                         \
      tile_step<D, STG * STAGE, STG * STAGE + TILE_BYTES>(w, la, t >= bnd.jmh || t < bnd.jml, \
                                                          kfirst + t * kBC, row_lo, row_hi, sl2, lane); \
  } while (0)

  if (MASK) {
    // Block-sparse: tile t holds key block kfirst/kBC + t, streamed only when the mask row of
    // this query block marks it.  The tile after the current one is found by a scan that every
    // lane makes alike; the two-stage ring and its barriers are those of the dense loop below.
    // The mask row is read through the constant address space, so the reads are scalar loads
    // (scalar cache, lgkmcnt): a read never waits for the tile loads in flight (vmcnt).  The
    // current dword of the row stays in a register; most steps need no load at all.
    typedef __attribute__((address_space(4))) const unsigned cu32;
    const unsigned long long mrow =
        (unsigned long long)(uintptr_t)p.bmask + (unsigned long long)(bh / p.H) * p.bm_stride_b +
        (unsigned long long)(bh % p.H) * p.bm_stride_h + (unsigned long long)qb * p.bm_n_kb + kfirst / kBC;
    unsigned long long word_at = ~0ull;  // byte address of the dword held in `word`
    unsigned word = 0;
    auto next_active = [&](int t) {
      for (; t < n_tiles; ++t) {
        const unsigned long long a = mrow + (unsigned long long)t;
        if ((a & ~3ull) != word_at) {
          word_at = a & ~3ull;
          word = *reinterpret_cast<cu32*>(word_at);
        }
        if ((word >> (8 * (a & 3))) & 0xffu) break;
      }
      return t;
    };
    int ta = next_active(0);
    if (ta < n_tiles) issue_tile<D, NW>(krs, vrs, lds[0][0], lds[0][1], kfirst + ta * kBC, wave, lane);
    while (ta < n_tiles) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int tb = next_active(ta + 1);
      if (tb < n_tiles) issue_tile<D, NW>(krs, vrs, lds[1][0], lds[1][1], kfirst + tb * kBC, wave, lane);
      FA2_STEP(0, ta);
      if (tb >= n_tiles) break;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      ta = next_active(tb + 1);
      if (ta < n_tiles) issue_tile<D, NW>(krs, vrs, lds[0][0], lds[0][1], kfirst + ta * kBC, wave, lane);
      FA2_STEP(1, tb);
    }
  }
  // unrolled by two so that each stage's LDS offsets are compile-time constants
  if (!MASK && n_tiles > 0) issue_tile<D, NW>(krs, vrs, lds[0][0], lds[0][1], kfirst, wave, lane);
  for (int j = 0; !MASK && j < n_tiles; j += 2) {
    const int k0 = kfirst + j * kBC;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < n_tiles) issue_tile<D, NW>(krs, vrs, lds[1][0], lds[1][1], k0 + kBC, wave, lane);
    FA2_STEP(0, j);
    if (j + 1 < n_tiles) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (j + 2 < n_tiles) issue_tile<D, NW>(krs, vrs, lds[0][0], lds[0][1], k0 + 2 * kBC, wave, lane);
      FA2_STEP(1, j + 1);
    }
  }
#undef FA2_STEP

  // ---- epilogue ----
  const float l_tot = w.l_run + __shfl_xor(w.l_run, 32);
  const float l16_tot = w.l16 + __shfl_xor(w.l16, 32);
  if (!SPLIT) {
    // O = acc / l16 (a row with no visible key: O = 0), staged in the tiles' space once every
    // wave is done with it and written as whole rows
    static_assert(NW * kStagedRows<D> <= (int)sizeof(lds), "the staged rows fit");
    u32x2 out[NB][4];
    scaled_rows<D>(w.acc, l16_tot > 0.f ? 1.f / l16_tot : 0.f, out);
    __syncthreads();
    write_rows<D>(out, (unsigned)(uintptr_t)(const lds_void*)&lds[0][0][0] + (unsigned)(wave * kStagedRows<D>),
                  p.o + ((long long)bh * p.n_q + q0w) * D, p.n_q - q0w, lane);
    if (hf == 0 && row < p.n_q)
      p.lse[(long long)bh * p.n_q + row] = l_tot > 0.f ? (w.m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    if (row >= p.n_q) return;
    // partial (acc, m, l) with l the fp32 sum: acc is rescaled by l / l16 so that acc / l is
    // the chunk's output exactly as normalised by its bf16 probabilities (0 for an empty chunk)
    const long long R = (long long)p.B * p.H * p.n_q;
    const long long rg = (long long)bh * p.n_q + row;
    const float rescale = l16_tot > 0.f ? l_tot / l16_tot : 0.f;
    float* wa = p.ws_acc + ((long long)split * R + rg) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 o4 = {w.acc[nb][4 * g] * rescale, w.acc[nb][4 * g + 1] * rescale,
                          w.acc[nb][4 * g + 2] * rescale, w.acc[nb][4 * g + 3] * rescale};
        *reinterpret_cast<f32x4*>(wa + 32 * nb + 8 * g + 4 * hf) = o4;
      }
    if (hf == 0) {
      p.ws_m[split * R + rg] = w.m_run == -INFINITY ? -INFINITY : w.m_run * kLn2;
      p.ws_l[split * R + rg] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-KV partial for single-query decode (N_q == 1).  One workgroup (4
// waves) per (batch*head, key chunk).  With a single query row both products
// are matrix-vector shaped and the kernel is bound by streaming K and V from
// HBM, so it uses VALU dot products: D/8 lanes share one key row (16 bytes
// each), a wave covers 64*8/D keys per load, and each lane keeps kDecU keys'
// K and V loads in flight per step.  Every wave runs its own online softmax
// over the steps it owns (steps are dealt round-robin to the waves), so the
// stream never waits at a workgroup barrier; the four wave partials are merged
// once at the end with the same rescaling.
constexpr int kDecThreads = 256;
constexpr int kNonTemporal = 2;  // buffer-load cache policy bit: nt
constexpr int kDecU = 16;

// DIRECT: a single chunk (num_splits == 1) whose result is final, so the
// workgroup writes O and LSE itself instead of a workspace partial.
template <int D, bool DIRECT>
__global__ void __launch_bounds__(kDecThreads) decode_partial_kernel(FwdParams p, float sl2, unsigned qsign) {
  constexpr int LPK = D / 8;        // lanes per key row
  constexpr int KPW = 64 / LPK;     // key rows per wave-wide load
  constexpr int STEP = KPW * kDecU; // keys per wave step
  constexpr int NWAVE = kDecThreads / 64;
  __shared__ float part_acc[NWAVE][D];
  __shared__ float part_m[NWAVE], part_l[NWAVE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane % LPK, kg = lane / LPK;

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int split = L % p.num_splits;
  const int bh = L / p.num_splits;
  const long long b0 = (long long)split * p.split_len;
  const int kbeg = b0 < p.n_k ? (int)b0 : p.n_k;
  int kend = kbeg + p.split_len < p.n_k ? kbeg + p.split_len : p.n_k;
  if (p.wr >= 0) kend = min(kend, p.wr + 1);  // the single query row 0 sees keys 0 .. wr

  // loads past key kend return zero (range check on the per-lane offset)
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + (long long)bh * p.n_k * D, (long long)kend * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + (long long)bh * p.n_k * D, (long long)kend * D * 2);

  bf16x2 q2[4];
  {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(p.q + (long long)bh * D + sub * 8) ^
                      u32x4{qsign, qsign, qsign, qsign};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned qw = raw[i];
      q2[i] = __builtin_bit_cast(bf16x2, qw);
    }
  }

  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float m_run = -INFINITY;  // log2 units, uniform over the wave
  float l_run = 0.f;        // this key group's share

  for (int k0 = kbeg + wave * STEP; k0 < kend; k0 += NWAVE * STEP) {
    u32x4 kr[kDecU], vr[kDecU];
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      const unsigned off = ((unsigned)(k0 + u * KPW + kg) * D + sub * 8) * 2u;
      // non-temporal: each K/V byte is read once, so keep it from displacing cached lines
      // (measured +12 % on the 8.6 GB decode stream)
      kr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, kNonTemporal));
      vr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, kNonTemporal));
    }
    float sc[kDecU];
    float mloc = -INFINITY;
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned kw = kr[u][i];  // named copy: bit-casting a vector element in place reads element 0
        dot = __builtin_amdgcn_fdot2_f32_bf16(q2[i], __builtin_bit_cast(bf16x2, kw), dot, false);
      }
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
    for (int i = 0; i < 8; ++i) acc[i] *= alpha;
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      const float pk = __builtin_amdgcn_exp2f(sc[u] - m_use);
      ps += pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(pk, __builtin_bit_cast(float, vr[u][i] << 16), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(pk, __builtin_bit_cast(float, vr[u][i] & 0xffff0000u), acc[2 * i + 1]);
      }
    }
    l_run = l_run * alpha + ps;
  }

  // fold the key groups of the wave (lanes with equal `sub`)
#pragma unroll
  for (int x = LPK; x < 64; x <<= 1) {
    l_run += __shfl_xor(l_run, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], x);
  }
  if (kg == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) part_acc[wave][sub * 8 + i] = acc[i];
  }
  if (lane == 0) {
    part_m[wave] = m_run;
    part_l[wave] = l_run;
  }
  __syncthreads();

  // merge the wave partials (log2 units) and write the chunk partial
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
  if (DIRECT) {
    // every query row sees key 0, so lsum > 0
    const float inv = 1.f / lsum;
    for (int dd = tid; dd < D; dd += kDecThreads) {
      float t = 0.f;
#pragma unroll
      for (int v = 0; v < NWAVE; ++v) t += wgt[v] * part_acc[v][dd];
      p.o[(long long)bh * D + dd] = __builtin_bit_cast(uint16_t, (__bf16)(t * inv));
    }
    if (tid == 0) p.lse[bh] = (M + __log2f(lsum)) * kLn2;
    return;
  }
  const long long R = (long long)p.B * p.H;  // N_q == 1
  for (int dd = tid; dd < D; dd += kDecThreads) {
    float t = 0.f;
#pragma unroll
    for (int v = 0; v < NWAVE; ++v) t += wgt[v] * part_acc[v][dd];
    p.ws_acc[((long long)split * R + bh) * D + dd] = t;
  }
  if (tid == 0) {
    p.ws_m[split * R + bh] = M == -INFINITY ? -INFINITY : M * kLn2;
    p.ws_l[split * R + bh] = lsum;   // P is used in fp32 here, so acc / lsum is the chunk's output
  }
}

// ---------------------------------------------------------------------------
// Split-KV merge: one wave per query row, chunks combined in order 0..S-1:
// O = sum_c w_c acc_c / sum_c w_c l_c, LSE = M + ln sum_c w_c l_c, w_c = exp(m_c - M).
template <int D>
__global__ void __launch_bounds__(256) splitkv_merge_kernel(FwdParams p) {
  constexpr int PER = D / 64;  // head-dim elements per lane
  const int lane = threadIdx.x & 63;
  const long long R = (long long)p.B * p.H * p.n_q;
  const long long rg = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rg >= R) return;
  const int S = p.num_splits;
  float M = -INFINITY;
  for (int c = lane; c < S; c += 64) M = fmaxf(M, p.ws_m[c * R + rg]);
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) M = fmaxf(M, __shfl_xor(M, w));
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  float lsum = 0.f;
  for (int c = 0; c < S; ++c) {
    const float mc = p.ws_m[c * R + rg];
    if (mc == -INFINITY) continue;  // empty chunk
    const float w = __builtin_amdgcn_exp2f((mc - M) * kLog2e);
    lsum += w * p.ws_l[c * R + rg];
    const float* a = p.ws_acc + (c * R + rg) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] += w * a[lane + 64 * i];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;  // no visible key in any chunk: O = 0, LSE = -inf
  uint16_t* orow = p.o + rg * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const __bf16 b = (__bf16)(o[i] * inv);
    orow[lane + 64 * i] = __builtin_bit_cast(uint16_t, b);
  }
  if (lane == 0) p.lse[rg] = lsum > 0.f ? M + __logf(lsum) : -INFINITY;
}

// ---------------------------------------------------------------------------
// Ping-pong forward: 8 waves, 256 query rows (synthesis page, section 2: the
// HipKittens paragraph replaces producer/consumer wave specialisation by an
// 8-wave ping-pong in which every wave computes and wave priorities order the
// two halves; the FlashAttention-3 paragraph credits its speedup to
// overlapping matrix work with the softmax).  Waves w and w+4 share a SIMD;
// group 0 (waves 0-3) runs one phase ahead of group 1 (waves 4-7), so that on
// every SIMD one wave issues its matrix products (at raised priority) while
// the other computes its softmax.  Per tile j and wave, the phases are
//   matrix phase:  O += P_{j-1} V_{j-1};  S_j = K_j Q^T
//   vector phase:  P_j from S_j (online softmax)
// and every phase ends at a workgroup barrier.  Group 0 runs the matrix phase
// of tile j in global phase 2j and the vector phase in 2j+1; group 1 one phase
// later.  K and V each have a three-stage LDS ring (tile j in stage j % 3):
// the matrix phase of tile j issues the loads of K_{j+2} and V_{j+1} among its
// products, and the wait at the end of iteration j+1 retires them, so every
// load has one to two phases to arrive.  The raw scores stay in registers
// through the vector phase, so the exact redo of a tile never reads K again.

// O += P_{j-1} V_{j-1} followed by S_j = K_j Q^T as one stream of products whose A
// operands (V^T read transposed, then K rows) come from one ring of PF registers, each
// read issued PF products ahead: the score products start without an LDS round trip
// at the hand-over.  The scheduling groups hold the compiler to that issue order.
template <int D, unsigned VOFF, unsigned KOFF, int PF, int NDMA, typename Dma>
__device__ __forceinline__ void pv_qk_tile(WaveRows<D>& w, const LdsAddr<D>& la, const bf16x8 (&pb)[4], f32x16& s0,
                                           f32x16& s1, Dma&& dma) {
  constexpr int NB = D / 32;
  constexpr int KT = D / 16;
  constexpr int NPV = 4 * NB;        // products of P.V: (kb, t, nb)
  constexpr int NM = NPV + 2 * KT;   // then the score products: (t, block)
  constexpr unsigned ROW = D * 2;
  bf16x8 a[PF];
  auto load = [&](int m) {
    if (m < NPV) {
      const int kb = m / (2 * NB), t = (m / NB) % 2, nb = m % NB;
      const unsigned roff = VOFF + (kb * 32 + 16 * t) * ROW;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<lds_i16x4*>((uintptr_t)(la.va[2 * nb] + roff)));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<lds_i16x4*>((uintptr_t)(la.va[2 * nb + 1] + roff)));
      a[m % PF] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      const int i = m - NPV;
      a[m % PF] = lds_load<bf16x8>(la.ka[i / 2] + KOFF + (i % 2) * 32 * ROW);
    }
  };
#pragma unroll
  for (int m = 0; m < PF; ++m) load(m);
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
  s0 = f32x16{};
  s1 = f32x16{};
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    if (m < NPV) {
      const int kb = m / (2 * NB), t = (m / NB) % 2, nb = m % NB;
      w.acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % PF], pb[2 * kb + t], w.acc[nb], 0, 0, 0);
    } else {
      const int i = m - NPV, t = i / 2;
      if (i % 2 == 0)
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % PF], w.qf[t], s0, 0, 0, 0);
      else
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % PF], w.qf[t], s1, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (m + PF < NPV) {
      load(m + PF);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    } else if (m + PF < NM) {
      load(m + PF);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    // the next tiles' buffer->LDS loads, spread over the stream (issued together they
    // queue in the address unit and stall the issuing wave)
#pragma unroll
    for (int i = 0; i < NDMA; ++i)
      if (m == i * NM / NDMA + 1) dma(i);
  }
}

// exp2(s * sl2 - m) of one 8-register slice, converted to bf16; adds to the sums
__device__ __forceinline__ bf16x8 exp_slice(const f32x16& s, int half, float sl2, float m, float& rs) {
  f32x8 e;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * half + r], sl2, -m));
    rs += e[r];
  }
  return cvt_bf16x8(e);
}

template <int D>
__device__ __forceinline__ void softmax_pp(WaveRows<D>& w, f32x16& s0, f32x16& s1, bf16x8 (&pb)[4], bool need_mask,
                                           int k0, int row_lo, int row_hi, float sl2, int lane) {
  constexpr int NB = D / 32;
  const int hf = lane >> 5;
  if (need_mask) mask_scores(s0, s1, k0, row_lo, row_hi, hf);
  bool exact = __ballot(w.m_run == -INFINITY) != 0;
  float rs = 0.f;
  if (!exact) {
    pb[0] = exp_slice(s0, 0, sl2, w.m_run, rs);
    pb[1] = exp_slice(s0, 1, sl2, w.m_run, rs);
    pb[2] = exp_slice(s1, 0, sl2, w.m_run, rs);
    pb[3] = exp_slice(s1, 1, sl2, w.m_run, rs);
    exact = __ballot(rs > kLazyBound) != 0;
  }
  if (exact) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
    const float m_new = fmaxf(w.m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(w.m_run - m_use);
    w.l_run *= alpha;
    w.l16 *= alpha;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) w.acc[nb] *= alpha;
    w.m_run = m_new;
    rs = 0.f;
    pb[0] = exp_slice(s0, 0, sl2, m_use, rs);
    pb[1] = exp_slice(s0, 1, sl2, m_use, rs);
    pb[2] = exp_slice(s1, 0, sl2, m_use, rs);
    pb[3] = exp_slice(s1, 1, sl2, m_use, rs);
  }
  w.l_run += rs;
  w.l16 = sum_bf16(pb, w.l16);
}

template <int D>
__global__ void __launch_bounds__(512, 1) fwd_pp_kernel(FwdParams p, float sl2, unsigned qsign) {
  constexpr int NW = 8;
  constexpr int BR = 32 * NW;
  constexpr int KT = D / 16;
  constexpr int NB = D / 32;
  constexpr int TILE_BYTES = kBC * D * 2;
  constexpr int CPR = D / 8;
  constexpr int NLD = kBC * CPR / (64 * NW);  // buffer->LDS loads per tile and wave

  // three-stage rings: tile j of K (V) in stage j % 3, loaded two (one) iterations ahead
  __shared__ __attribute__((aligned(1024))) char ldsk[3][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char ldsv[3][TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int hf = lane >> 5;
  const int col = lane & 31;

  const int n_qb = (p.n_q + BR - 1) / BR;
  const int wl = p.wl, wr = p.wr;
  int bh, qb;
  wg_coords(wg_logical(p.sched), n_qb, p.B * p.H, p.sched, wl < 0 && wr >= 0, bh, qb);
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
  const int kfirst = klo / kBC * kBC;
  const int n_tiles = khi > kfirst ? (khi - kfirst + kBC - 1) / kBC : 0;

  const uint16_t* Qh = p.q + (long long)bh * p.n_q * D;
  const i32x4 krs = raw_rsrc(p.k + (long long)bh * p.n_k * D, (long long)khi * D * 2);
  const i32x4 vrs = raw_rsrc(p.v + (long long)bh * p.n_k * D, (long long)khi * D * 2);

  WaveRows<D> w;
  {
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qh, (long long)p.n_q * D * 2);
    const u32x4 sign = {qsign, qsign, qsign, qsign};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const u32x4 raw = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, ((unsigned)row * D + 16 * t + 8 * hf) * 2u, 0, 0));
      w.qf[t] = as_bf16x8(raw ^ sign);
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) w.acc[nb] = f32x16{};
  w.m_run = -INFINITY;
  w.l_run = 0.f;
  w.l16 = 0.f;

  LdsAddr<D> la;  // K-row addresses over the K ring, transposed-V addresses over the V ring
  {
    LdsAddr<D> lv;
    make_lds_addr<D>(la, (unsigned)(uintptr_t)(const lds_void*)&ldsk[0][0], lane);
    make_lds_addr<D>(lv, (unsigned)(uintptr_t)(const lds_void*)&ldsv[0][0], lane);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) la.va[i] = lv.va[i];
  }
  // this lane's byte offset within a tile for each of its NLD loads (swizzled slots)
  unsigned offp[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int sl = (i * NW + wave) * 64 + lane;
    const int r = sl / CPR;
    const int c = (sl % CPR) ^ (swz<D>(r, 0) - r * CPR);
    offp[i] = (unsigned)((r * D + c * 8) * 2);
  }
  // load part i (0 .. 2 NLD - 1) of iteration j's prefetch: K_{j+2} into stage (KS + 2) % 3,
  // then V_{j+1} into stage (KS + 1) % 3.  Tiles past the last one read past the buffer
  // range and fill their stage with zeros, which no phase reads.
  auto dma = [&](int j, auto kst, int i) {
    constexpr unsigned KS = decltype(kst)::value;
    if (i < NLD)
      lds_dma16(krs, &ldsk[(KS + 2) % 3][(i * NW + wave) * 64 * 16],
                offp[i] + (unsigned)(kfirst + (j + 2) * kBC) * D * 2);
    else
      lds_dma16(vrs, &ldsv[(KS + 1) % 3][((i - NLD) * NW + wave) * 64 * 16],
                offp[i - NLD] + (unsigned)(kfirst + (j + 1) * kBC) * D * 2);
  };

  f32x16 s0 = {}, s1 = {};
  bf16x8 pb[4] = {};
  // the first matrix phase multiplies P = 0 with V stage 2, which no load has written
  // yet: zero it (published by the barrier before the loop)
  {
    constexpr int PER = TILE_BYTES / (64 * NW);
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < PER / 16; ++i)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
          (uintptr_t)(const lds_void*)&ldsv[2][(tid * (PER / 16) + i) * 16]) = z;
  }

  const TileBounds bnd = tile_bounds(kfirst, n_tiles, klo_w, khi_w, p.n_k, q0w, wl, wr);
  auto act = [&](int j) { return j >= bnd.ja && j < bnd.jb; };
  auto need_mask = [&](int j) { return j >= bnd.jmh || j < bnd.jml; };
  // matrix phase of tile j: O += P_{j-1} V_{j-1}, then S_j = K_j Q^T, with the loads of
  // K_{j+2} and V_{j+1} issued among the products.  KST = j % 3: stage of K_j.
  auto mat = [&](int j, auto kst) {
    constexpr unsigned KS = decltype(kst)::value;
    // one straight-line stream whenever either half is live: an inactive previous tile
    // left P = 0 (and V finite), an inactive current tile's scores are never used
    __builtin_amdgcn_s_setprio(1);
    if (act(j - 1) || act(j)) {
      pv_qk_tile<D, ((KS + 2) % 3) * TILE_BYTES, KS * TILE_BYTES, 4, 2 * NLD>(w, la, pb, s0, s1,
                                                                             [&](int i) { dma(j, kst, i); });
    } else {
#pragma unroll
      for (int i = 0; i < 2 * NLD; ++i) dma(j, kst, i);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto vec = [&](int j) {
    if (act(j))
      softmax_pp(w, s0, s1, pb, need_mask(j), kfirst + j * kBC, row_lo, row_hi, sl2, lane);
    else
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = bf16x8{};
  };
  // The loads a wave issues in iteration j are waited for at the end of iteration j + 1:
  // the wait leaves this iteration's 2 NLD loads in flight (each wave's loads complete in
  // order).  Both groups issue in their matrix phase.
  auto wait_prev = [&]() {
    if constexpr (NLD == 2)
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  };
  // tile iteration j: phases 2j and 2j+1.  KST = j % 3.  Group 0 runs (matrix j, vector j),
  // group 1 (vector j-1, matrix j); each group has its own loop so that its phases are
  // straight-line code.  Both execute the same barriers.
  auto iter0 = [&](int j, auto kst) {
    mat(j, kst);
    __syncthreads();
    vec(j);
    wait_prev();
    __syncthreads();
  };
  auto iter1 = [&](int j, auto kst) {
    vec(j - 1);
    __syncthreads();
    mat(j, kst);
    wait_prev();
    __syncthreads();
  };

  // K_0, K_1 and V_0 before the loop
  {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      lds_dma16(krs, &ldsk[0][(i * NW + wave) * 64 * 16], offp[i] + (unsigned)kfirst * D * 2);
      lds_dma16(krs, &ldsk[1][(i * NW + wave) * 64 * 16], offp[i] + (unsigned)(kfirst + kBC) * D * 2);
      lds_dma16(vrs, &ldsv[0][(i * NW + wave) * 64 * 16], offp[i] + (unsigned)kfirst * D * 2);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (grp == 0) {
    for (int j = 0; j <= n_tiles; j += 3) {
      iter0(j, std::integral_constant<unsigned, 0>{});
      if (j + 1 <= n_tiles) iter0(j + 1, std::integral_constant<unsigned, 1>{});
      if (j + 2 <= n_tiles) iter0(j + 2, std::integral_constant<unsigned, 2>{});
    }
  } else {
    for (int j = 0; j <= n_tiles; j += 3) {
      iter1(j, std::integral_constant<unsigned, 0>{});
      if (j + 1 <= n_tiles) iter1(j + 1, std::integral_constant<unsigned, 1>{});
      if (j + 2 <= n_tiles) iter1(j + 2, std::integral_constant<unsigned, 2>{});
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const float l_tot = w.l_run + __shfl_xor(w.l_run, 32);
  const float l16_tot = w.l16 + __shfl_xor(w.l16, 32);
  // O staged in the K rings (group 0) and the V rings (group 1) once every wave is done with them
  static_assert(4 * kStagedRows<D> <= (int)sizeof(ldsk), "the staged rows fit");
  u32x2 out[NB][4];
  scaled_rows<D>(w.acc, l16_tot > 0.f ? 1.f / l16_tot : 0.f, out);
  __syncthreads();
  const unsigned stage = (unsigned)(uintptr_t)(const lds_void*)(wave < 4 ? &ldsk[0][0] : &ldsv[0][0]) +
                         (unsigned)((wave & 3) * kStagedRows<D>);
  write_rows<D>(out, stage, p.o + ((long long)bh * p.n_q + q0w) * D, p.n_q - q0w, lane);
  if (hf == 0 && row < p.n_q)
    p.lse[(long long)bh * p.n_q + row] = l_tot > 0.f ? (w.m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

// scale handling shared by all launches: fold |scale|*log2(e) into one positive
// multiplier and move the sign into Q
void fold_scale(float scale, float* sl2, unsigned* qsign) {
  const float a = fabsf(scale) * kLog2e;
  *sl2 = a > 1.17549435e-38f ? a : 1.17549435e-38f;  // scale 0 -> tiny positive: every score weighs 1
  *qsign = scale < 0.f ? 0x80008000u : 0u;
}

template <int D, int NW, bool SPLIT, bool MASK = false>
hipError_t launch_tile(const FwdParams& p, hipStream_t stream) {
  constexpr int BR = 32 * NW;
  const long long n_qb = (p.n_q + BR - 1) / BR;
  const long long grid = n_qb * p.B * p.H * (SPLIT ? p.num_splits : 1);
  float sl2;
  unsigned qsign;
  fold_scale(p.scale, &sl2, &qsign);
  hipLaunchKernelGGL((fwd_kernel<D, NW, SPLIT, MASK>), dim3((unsigned)grid), dim3(64 * NW), 0, stream, p, sl2,
                     qsign);
  return hipGetLastError();
}

template <bool DIRECT>
hipError_t launch_decode(const FwdParams& p, hipStream_t stream) {
  float sl2;
  unsigned qsign;
  fold_scale(p.scale, &sl2, &qsign);
  const unsigned grid = (unsigned)((long long)p.B * p.H * p.num_splits);
  if (p.d == 128)
    hipLaunchKernelGGL((decode_partial_kernel<128, DIRECT>), dim3(grid), dim3(kDecThreads), 0, stream, p, sl2, qsign);
  else
    hipLaunchKernelGGL((decode_partial_kernel<64, DIRECT>), dim3(grid), dim3(kDecThreads), 0, stream, p, sl2, qsign);
  return hipGetLastError();
}

template <int D>
hipError_t launch_pp(const FwdParams& p, hipStream_t stream) {
  float sl2;
  unsigned qsign;
  fold_scale(p.scale, &sl2, &qsign);
  const unsigned grid = (unsigned)((long long)((p.n_q + 255) / 256) * p.B * p.H);
  hipLaunchKernelGGL(fwd_pp_kernel<D>, dim3(grid), dim3(512), 0, stream, p, sl2, qsign);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p_in, int config, hipStream_t stream) {
  // one query row per head: the streaming decode kernel over the whole key range
  if (p_in.n_q == 1) return launch_decode<true>(p_in, stream);
  const FwdConfig& c = kFwdConfigs[config];
  FwdParams p = p_in;
  p.sched = c.sched;
  if (c.kernel == 1) return p.d == 128 ? launch_pp<128>(p, stream) : launch_pp<64>(p, stream);
  if (c.kernel == 2) return p.d == 128 ? launch_tile<128, 8, false>(p, stream) : launch_tile<64, 8, false>(p, stream);
  return p.d == 128 ? launch_tile<128, 4, false>(p, stream) : launch_tile<64, 4, false>(p, stream);
}

hipError_t launch_fwd_blockmask(const FwdParams& p, hipStream_t stream) {
  return p.d == 128 ? launch_tile<128, 4, false, true>(p, stream) : launch_tile<64, 4, false, true>(p, stream);
}

hipError_t launch_splitkv_partial(const FwdParams& p, hipStream_t stream) {
  if (p.n_q == 1) return launch_decode<false>(p, stream);
  if (p.d == 128) return launch_tile<128, 4, true>(p, stream);
  return launch_tile<64, 4, true>(p, stream);
}

hipError_t launch_splitkv_merge(const FwdParams& p, hipStream_t stream) {
  const long long R = (long long)p.B * p.H * p.n_q;
  const unsigned grid = (unsigned)((R + 3) / 4);
  if (p.d == 128)
    hipLaunchKernelGGL(splitkv_merge_kernel<128>, dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(splitkv_merge_kernel<64>, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa2
