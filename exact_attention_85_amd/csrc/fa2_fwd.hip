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
//   online softmax   running max m and sum l per row, base-2 exponent with
//                    scale*log2(e) folded into one FMA; P stays in registers
//   O^T += V^T P^T   v_mfma_f32_32x32x16_bf16, V read transposed from LDS with
//                    ds_read_b64_tr_b16, P converted to bf16 (RNE)
// and the epilogue divides by l once (deferred normalisation, synthesis page,
// section 2 item 1) and writes O (bf16) and LSE = m + ln l (fp32).
//
// Computing S transposed puts one query row in each lane column, so the
// accumulator of S^T is directly the B operand of the second product and every
// per-row statistic lives in one lane pair (lanes c and c+32).
#include "fa2_internal.h"

#include <math.h>

namespace fa2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kBC = 64;  // keys per K/V tile

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ---------------------------------------------------------------------------
// LDS tile layout.  A K or V tile is kBC rows of D bf16, stored as 16-byte
// slots; row r, chunk c (elements 8c..8c+7) lives in slot swz<D>(r, c).  The
// XOR keeps both read patterns free of bank conflicts on a 256-byte bank row:
// 16 consecutive rows at one chunk (K operand reads) and 4 consecutive rows x
// 4 consecutive chunks (transposed V reads).
template <int D> __device__ __forceinline__ int swz(int r, int c);
template <> __device__ __forceinline__ int swz<128>(int r, int c) {
  return r * 16 + (c ^ (((r & 3) << 2) | ((r >> 2) & 3)));
}
template <> __device__ __forceinline__ int swz<64>(int r, int c) {
  const int br = r >> 1;
  return r * 8 + (c ^ (((br & 1) << 2) | ((br >> 1) & 3)));
}

// Workgroup ids are dealt round-robin to the 8 XCDs.  Renumber them so that
// each XCD receives a contiguous range of logical ids: consecutive logical
// ids share a (batch, head), so the K/V blocks they stream are reused in that
// XCD's L2 (synthesis page, section 2, Chiplet FA paragraph).  Bijective on
// [0, G) for any G.
__device__ __forceinline__ int xcd_remap(int w, int G) {
  constexpr int X = 8;
  const int per = (G + X - 1) / X;
  const int tall = G - (per - 1) * X;  // XCDs that receive `per` ids
  const int x = w % X, i = w / X;
  return x < tall ? x * per + i : tall * per + (x - tall) * (per - 1) + i;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x8 cvt_bf16x8(f32x8 v) { return __builtin_convertvector(v, bf16x8); }

__device__ __forceinline__ f32x8 slice8(const f32x16& s, int t) {
  return t == 0 ? __builtin_shufflevector(s, s, 0, 1, 2, 3, 4, 5, 6, 7)
                : __builtin_shufflevector(s, s, 8, 9, 10, 11, 12, 13, 14, 15);
}

// ---------------------------------------------------------------------------
// Buffer resource over [base, base + bytes): loads whose per-lane offset lies
// beyond `bytes` return zero, which is how ragged query/key tails are
// zero-filled without branches.  The host limits one head to < 2^31 bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void;

// Forward / split-KV partial kernel.
//   D   head dim (64 or 128)
//   NW  waves per workgroup; the query block is B_r = 32*NW rows
//   SPLIT  false: write O and LSE;  true: write the fp32 partial (acc, m, l)
//          of the key chunk selected by the workgroup id.
// Kernel arguments beyond FwdParams: sl2 = max(|scale| * log2 e, FLT_MIN) and
// qsign = 0x80008000 when scale < 0 (Q is negated in registers so that the
// folded multiplier stays positive), else 0.
//
// K/V tiles go straight from HBM/L2 into LDS (buffer_load ... lds): lane i of
// a load writes LDS slot (M0 + 16 i), so each lane fetches the (row, chunk)
// whose swizzled slot it owns.  Tile j+1 is in flight while tile j computes;
// one barrier per tile both publishes tile j and retires tile j-1's buffer.
//
// The O accumulator is rescaled only on tiles where some row of the wave
// finds a new maximum (alpha = 1 for every row otherwise); the running maximum
// itself stays exact, so the largest probability of each row is exactly 1
// before its conversion to bf16.

template <int D, int NW, bool SPLIT>
__global__ void __launch_bounds__(64 * NW, 8 / NW) fwd_kernel(FwdParams p, float sl2, unsigned qsign) {
  constexpr int T = 64 * NW;
  constexpr int BR = 32 * NW;
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int SLOTS = kBC * CPR;    // slots per tile per tensor
  constexpr int NLD = SLOTS / T;      // buffer->LDS loads per thread per tensor per tile
  constexpr int KT = D / 16;          // k-steps of Q K^T
  constexpr int NB = D / 32;          // 32-wide blocks of the head dim in O^T
  constexpr int TILE_BYTES = SLOTS * 16;
  static_assert(SLOTS % T == 0, "tile must split evenly over the threads");

  __shared__ __attribute__((aligned(1024))) char lds[2][2][TILE_BYTES];  // [stage][K=0 / V=1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;           // which 8-wide k half of an MFMA operand this lane holds
  const int col = lane & 31;          // query row (within the wave) of this lane
  const int j16 = lane & 15, cg = (lane >> 4) & 1;

  // ---- workgroup -> (batch*head, query block, key chunk) ----
  const int n_qb = (p.n_q + BR - 1) / BR;
  int L = xcd_remap(blockIdx.x, gridDim.x);
  int split = 0;
  if (SPLIT) {
    split = L % p.num_splits;
    L /= p.num_splits;
  }
  const int bh = L / n_qb;
  int qb = L % n_qb;
  if (p.causal) qb = n_qb - 1 - qb;  // heaviest query blocks are dispatched first
  const int q0 = qb * BR;
  const int q0w = q0 + wave * 32;
  const int row = q0w + col;

  int kbeg = 0, kend = p.n_k;
  if (SPLIT) {
    const long long b = (long long)split * p.split_len;
    kbeg = b < p.n_k ? (int)b : p.n_k;
    kend = kbeg + p.split_len < p.n_k ? kbeg + p.split_len : p.n_k;
  }
  // keys below khi are visible to some row of the workgroup, below khi_w to some row of this wave
  int khi = kend, khi_w = kend;
  if (p.causal) {
    khi = min(khi, q0 + BR);
    khi_w = min(khi_w, q0w + 32);
  }
  const int n_tiles = khi > kbeg ? (khi - kbeg + kBC - 1) / kBC : 0;

  const uint16_t* Qh = p.q + (long long)bh * p.n_q * D;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + (long long)bh * p.n_k * D, (long long)khi * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + (long long)bh * p.n_k * D, (long long)khi * D * 2);

  // ---- Q fragment: B operand of S^T = K Q^T; lane holds Q[row][16t + 8hf .. +7] ----
  bf16x8 qf[KT];
  {
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qh, (long long)p.n_q * D * 2);
    const u32x4 sign = {qsign, qsign, qsign, qsign};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const u32x4 raw = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, (unsigned)((row * D + 16 * t + 8 * hf) * 2), 0, 0));
      qf[t] = as_bf16x8(raw ^ sign);
    }
  }

  // ---- buffer->LDS tile loads ----
  // Load i of this wave fills physical slots (i*NW + wave)*64 .. +63; the lane
  // owning slot s fetches the (row, chunk) that the swizzle stores there.  The
  // whole byte offset goes in the per-lane voffset, which the range check uses.
  auto issue_tile = [&](int k0, int st) {
    const unsigned toff = (unsigned)k0 * D * 2;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int s = (i * NW + wave) * 64 + lane;
      const int r = s / CPR;
      const int c = (s % CPR) ^ (swz<D>(r, 0) - r * CPR);
      const unsigned off = (unsigned)((r * D + c * 8) * 2) + toff;
      const int sbase = (i * NW + wave) * 64 * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(&lds[st][0][sbase]), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(&lds[st][1][sbase]), 16, off, 0, 0, 0);
    }
  };

  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};
  float m_run = -INFINITY;  // reference maximum of the scaled scores, log2 units
  float l_run = 0.f;        // this lane's share of the running denominator

  if (n_tiles > 0) issue_tile(kbeg, 0);

  for (int j = 0; j < n_tiles; ++j) {
    const int k0 = kbeg + j * kBC;
    const int st = j & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < n_tiles) issue_tile(k0 + kBC, st ^ 1);

    if (k0 < khi_w) {
      const char* Kt = lds[st][0];
      const char* Vt = lds[st][1];

      // S^T = K Q^T : two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kt + swz<D>(kb * 32 + col, 2 * t + hf) * 16);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[kb], 0, 0, 0);
        }
      }
      // s[kb][r] is the score of query `row` against key k0 + kb*32 + 8*(r/4) + 4*hf + r%4

      const bool need_mask = (k0 + kBC > kend) || (p.causal && k0 + kBC - 1 > q0w);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (key >= kend || (p.causal && key > row)) s[kb][r] = -INFINITY;
          }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      if (__ballot(m_new > m_run)) {  // some row of this wave has a new maximum
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        l_run *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] *= alpha;
      }
      m_run = m_new;

      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], sl2, -m_use));
          s[kb][r] = e;
          rs += e;
        }
      l_run += rs;

      // O^T += V^T P^T.  k-step (kb, t) contracts keys kb*32 + 16t + {4hf..4hf+3, 8+4hf..8+4hf+3}
      // (the keys this lane's S^T registers 8t..8t+7 hold); the A operand is read transposed.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 pb = cvt_bf16x8(slice8(s[kb], t));
          const int kr = kb * 32 + 16 * t + 4 * hf + (j16 >> 2);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int dd = 32 * nb + 16 * cg + 4 * (j16 & 3);
            const int boff = (dd & 7) * 2;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(Vt + swz<D>(kr, dd >> 3) * 16 + boff));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(Vt + swz<D>(kr + 8, dd >> 3) * 16 + boff));
            const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[nb], 0, 0, 0);
          }
        }
    }
  }

  // ---- epilogue ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row >= p.n_q) return;
  // acc[nb][4g + i] = O^T[32nb + 8g + 4hf + i][row]
  if (!SPLIT) {
    const float inv = 1.f / l_tot;
    uint16_t* Orow = p.o + ((long long)bh * p.n_q + row) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 o4 = {acc[nb][4 * g] * inv, acc[nb][4 * g + 1] * inv, acc[nb][4 * g + 2] * inv,
                          acc[nb][4 * g + 3] * inv};
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 b4 = __builtin_convertvector(o4, bf16x4);
        *reinterpret_cast<u32x2*>(Orow + 32 * nb + 8 * g + 4 * hf) = __builtin_bit_cast(u32x2, b4);
      }
    if (hf == 0) p.lse[(long long)bh * p.n_q + row] = (m_run + __log2f(l_tot)) * kLn2;
  } else {
    const long long R = (long long)p.B * p.H * p.n_q;
    const long long rg = (long long)bh * p.n_q + row;
    float* wa = p.ws_acc + ((long long)split * R + rg) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 o4 = {acc[nb][4 * g], acc[nb][4 * g + 1], acc[nb][4 * g + 2], acc[nb][4 * g + 3]};
        *reinterpret_cast<f32x4*>(wa + 32 * nb + 8 * g + 4 * hf) = o4;
      }
    if (hf == 0) {
      p.ws_m[split * R + rg] = m_run == -INFINITY ? -INFINITY : m_run * kLn2;
      p.ws_l[split * R + rg] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-KV partial for single-query decode (N_q == 1).  One workgroup per
// (batch*head, chunk).  With a single query row the products are matrix-vector
// shaped and the kernel is bound by streaming K and V from HBM, so it uses
// plain fp32 dot products: D/8 lanes share one key row (16 bytes each) and
// the chunk is walked in blocks of kDecBlock keys with the same running-max
// rescaling as the tile kernel.
constexpr int kDecThreads = 256;
constexpr int kDecBlock = 128;

template <int D>
__global__ void __launch_bounds__(kDecThreads) decode_partial_kernel(FwdParams p, float sl2, unsigned qsign) {
  constexpr int LPK = D / 8;                 // lanes per key row
  constexpr int KPI = kDecThreads / LPK;     // key rows per workgroup-wide load
  constexpr int NIT = kDecBlock / KPI;       // loads per thread per block
  __shared__ float sc[kDecBlock];
  __shared__ float red[kDecThreads / 64];
  __shared__ float accs[KPI][D + 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = tid % LPK, kslot = tid / LPK;

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int split = L % p.num_splits;
  const int bh = L / p.num_splits;
  const long long b0 = (long long)split * p.split_len;
  const int kbeg = b0 < p.n_k ? (int)b0 : p.n_k;
  int kend = kbeg + p.split_len < p.n_k ? kbeg + p.split_len : p.n_k;
  if (p.causal) kend = min(kend, 1);  // the single query row 0 sees key 0 only

  const uint16_t* Kh = p.k + (long long)bh * p.n_k * D;
  const uint16_t* Vh = p.v + (long long)bh * p.n_k * D;

  float q[8];
  {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(p.q + (long long)bh * D + sub * 8) ^
                      u32x4{qsign, qsign, qsign, qsign};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[2 * i] = __builtin_bit_cast(float, raw[i] << 16);
      q[2 * i + 1] = __builtin_bit_cast(float, raw[i] & 0xffff0000u);
    }
  }

  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float m_run = -INFINITY, l_run = 0.f;

  for (int kb0 = kbeg; kb0 < kend; kb0 += kDecBlock) {
    u32x4 kr[NIT], vr[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int key = kb0 + it * KPI + kslot;
      if (key < kend) {
        const long long off = (long long)key * D + sub * 8;
        kr[it] = *reinterpret_cast<const u32x4*>(Kh + off);
        vr[it] = *reinterpret_cast<const u32x4*>(Vh + off);
      } else {
        kr[it] = u32x4{0, 0, 0, 0};
        vr[it] = u32x4{0, 0, 0, 0};
      }
    }
    // scores
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dot = __builtin_fmaf(q[2 * i], __builtin_bit_cast(float, kr[it][i] << 16), dot);
        dot = __builtin_fmaf(q[2 * i + 1], __builtin_bit_cast(float, kr[it][i] & 0xffff0000u), dot);
      }
#pragma unroll
      for (int w = LPK / 2; w >= 1; w >>= 1) dot += __shfl_xor(dot, w);
      const int key = kb0 + it * KPI + kslot;
      if (sub == 0) sc[it * KPI + kslot] = key < kend ? dot * sl2 : -INFINITY;
    }
    __syncthreads();
    // block max
    float mx = tid < kDecBlock ? sc[tid] : -INFINITY;
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) mx = fmaxf(mx, __shfl_xor(mx, w));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < kDecThreads / 64; ++w) mx = fmaxf(mx, red[w]);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    __syncthreads();  // everyone has read red[] before it is reused
    float pe = 0.f;
    if (tid < kDecBlock) {
      pe = __builtin_amdgcn_exp2f(sc[tid] - m_use);
      sc[tid] = pe;
    }
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) pe += __shfl_xor(pe, w);
    if (lane == 0) red[wave] = pe;
    __syncthreads();
    float bsum = 0.f;
#pragma unroll
    for (int w = 0; w < kDecThreads / 64; ++w) bsum += red[w];
    l_run = l_run * alpha + bsum;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= alpha;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const float pk = sc[it * KPI + kslot];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(pk, __builtin_bit_cast(float, vr[it][i] << 16), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(pk, __builtin_bit_cast(float, vr[it][i] & 0xffff0000u), acc[2 * i + 1]);
      }
    }
    __syncthreads();  // sc[] and red[] are rewritten by the next block
  }

  // sum the KPI key slots' accumulators
#pragma unroll
  for (int i = 0; i < 8; ++i) accs[kslot][sub * 8 + i] = acc[i];
  __syncthreads();
  const long long R = (long long)p.B * p.H;  // N_q == 1
  for (int dd = tid; dd < D; dd += kDecThreads) {
    float t = 0.f;
    for (int s = 0; s < KPI; ++s) t += accs[s][dd];
    p.ws_acc[((long long)split * R + bh) * D + dd] = t;
  }
  if (tid == 0) {
    p.ws_m[split * R + bh] = m_run == -INFINITY ? -INFINITY : m_run * kLn2;
    p.ws_l[split * R + bh] = l_run;
  }
}

// ---------------------------------------------------------------------------
// Split-KV merge: one wave per query row, chunks combined in order 0..S-1.
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
  const float inv = 1.f / lsum;
  uint16_t* orow = p.o + rg * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const __bf16 b = (__bf16)(o[i] * inv);
    orow[lane + 64 * i] = __builtin_bit_cast(uint16_t, b);
  }
  if (lane == 0) p.lse[rg] = M + __logf(lsum);
}

// scale handling shared by all launches: fold |scale|*log2(e) into one positive
// multiplier and move the sign into Q
void fold_scale(float scale, float* sl2, unsigned* qsign) {
  const float a = fabsf(scale) * kLog2e;
  *sl2 = a > 1.17549435e-38f ? a : 1.17549435e-38f;  // scale 0 -> tiny positive: every score weighs 1
  *qsign = scale < 0.f ? 0x80008000u : 0u;
}

template <int D, int NW, bool SPLIT>
hipError_t launch_tile(const FwdParams& p, hipStream_t stream) {
  constexpr int BR = 32 * NW;
  const long long n_qb = (p.n_q + BR - 1) / BR;
  const long long grid = n_qb * p.B * p.H * (SPLIT ? p.num_splits : 1);
  float sl2;
  unsigned qsign;
  fold_scale(p.scale, &sl2, &qsign);
  hipLaunchKernelGGL((fwd_kernel<D, NW, SPLIT>), dim3((unsigned)grid), dim3(64 * NW), 0, stream, p, sl2, qsign);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  if (p.d == 128) return launch_tile<128, 4, false>(p, stream);
  return launch_tile<64, 4, false>(p, stream);
}

hipError_t launch_splitkv_partial(const FwdParams& p, hipStream_t stream) {
  if (p.n_q == 1) {
    float sl2;
    unsigned qsign;
    fold_scale(p.scale, &sl2, &qsign);
    const unsigned grid = (unsigned)((long long)p.B * p.H * p.num_splits);
    if (p.d == 128)
      hipLaunchKernelGGL(decode_partial_kernel<128>, dim3(grid), dim3(kDecThreads), 0, stream, p, sl2, qsign);
    else
      hipLaunchKernelGGL(decode_partial_kernel<64>, dim3(grid), dim3(kDecThreads), 0, stream, p, sl2, qsign);
    return hipGetLastError();
  }
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
