// Backward pass of exact attention for gfx950 (MI355X), deterministic.
//
// Gradients for an upstream gradient dO of O, from the forward's stored LSE
// (the synthesis page: section 3 item 1 lists FA2's backward as five matrix
// products; section 5 item 2 proposes a deterministic version that replaces
// the cross-block atomic add of dQ by two passes: per-K/V-block local dQ
// contributions, then a reduction):
//   P_ij  = exp(s_ij - LSE_i),  s_ij = scale q_i . k_j     (0 where masked)
//   D_i   = sum_c dO_ic O_ic
//   dV_j  = sum_i P_ij dO_i
//   dS_ij = P_ij (dO_i . v_j - D_i)
//   dK_j  = scale sum_i dS_ij q_i
//   dQ_i  = scale sum_j dS_ij k_j
//
// Three launches:
//   bwd_prep_kernel    D_i and LSE_i * log2(e) for every query row
//   bwd_kv_kernel      one workgroup per group of up to 8 128-key blocks,
//                      taken one after the other (one wave per 32 keys):
//                      streams 64-row query blocks through LDS and runs the
//                      five products on the matrix cores; dK and dV stay in
//                      registers.  The group shares one workspace slot for its
//                      dQ contribution: the first block stores it, and for each
//                      later block each thread's dQ accumulators start from the
//                      values it stored itself, so the slot ends up holding the
//                      group's sum and the reduction reads one partial per
//                      group instead of one per block
//   bwd_dq_kernel      dQ_i = scale * sum over the slots, in slot order
// No atomics: every output element is written by exactly one thread (a slot
// value twice, by the same thread, in program order), and the dQ sum runs in a
// fixed order, so the result is bit-reproducible.
//
// Within a wave the scores are computed as S = Q K^T (query rows x 32 keys),
// so every lane owns one key column: P and dS in accumulator layout are then
// directly the B operands of dV^T += dO^T P and dK^T += Q^T dS.  The dQ
// product needs dS with query rows on the lanes, so dS goes through LDS
// (stored key-major, read back transposed) once per query block.
#include "fa2_device.h"
#include "fa2_internal.h"

#include <math.h>

#include <type_traits>

namespace fa2 {
namespace {

constexpr int kBK = 128;  // keys per block (a workgroup takes a group of them)
constexpr int kBQ = 64;   // query rows per step
// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt fields at their maxima)
constexpr int kWaitVm0 = 0x0F70;

// ---------------------------------------------------------------------------
// D_i = sum_c dO_ic O_ic and LSE_i * log2(e).  D/8 lanes per row.
template <int D>
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdParams p) {
  constexpr int LPR = D / 8;
  const long long R = (long long)p.B * p.H * p.n_q;
  const long long row = (long long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < R) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p.dout + row * D + sub * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p.o + row * D + sub * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned x = a[i], y = b[i];
      acc = __builtin_fmaf(__builtin_bit_cast(float, x << 16), __builtin_bit_cast(float, y << 16), acc);
      acc = __builtin_fmaf(__builtin_bit_cast(float, x & 0xffff0000u), __builtin_bit_cast(float, y & 0xffff0000u),
                           acc);
    }
  }
#pragma unroll
  for (int x = LPR / 2; x >= 1; x >>= 1) acc += __shfl_xor(acc, x);
  if (sub == 0 && row < R) {
    p.dvec[row] = acc;
    p.l2vec[row] = p.lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// Transposed-read addresses for operands whose contraction index must run in
// natural order (k = 8*hf + e): supplying lane j16 of a 16-lane group loads
// the 4 elements (row rbase + 8hf + j16/4 + 4h, cols cbase + 16cg + 4(j16%4))
// of a row-major swizzled tile, so that the receiving lane gets rows
// rbase + 8hf + 4h + 0..3 at column cbase + 16cg + (lane % 16).
template <int RL>
__device__ __forceinline__ unsigned tr_nat_addr(unsigned base, int lane, int rbase, int cbase, int h) {
  const int hf = lane >> 5, cg = (lane >> 4) & 1, j16 = lane & 15;
  const int r = rbase + 8 * hf + (j16 >> 2) + 4 * h;
  const int c = cbase + 16 * cg + 4 * (j16 & 3);
  return base + swz<RL>(r, c >> 3) * 16 + (c & 7) * 2;
}

__device__ __forceinline__ bf16x8 tr_pair(unsigned a0, unsigned a1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4*>((uintptr_t)a0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4*>((uintptr_t)a1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Loads of one 64-row tile (Q or dO) into LDS with the swizzled slot layout.
template <int D>
__device__ __forceinline__ void issue_rows(i32x4 rs, const char* dst, int r0, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int NLD = kBQ * CPR / 256;
  const unsigned toff = (unsigned)r0 * D * 2;
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int s = (i * 4 + wave) * 64 + lane;
    const int r = s / CPR;
    const int c = (s % CPR) ^ (swz<D>(r, 0) - r * CPR);
    lds_dma16(rs, dst + (i * 4 + wave) * 64 * 16, (unsigned)((r * D + c * 8) * 2) + toff);
  }
}

template <int D>
__global__ void __launch_bounds__(256, 1) bwd_kv_kernel(BwdParams p, float sl2) {
  constexpr int NB = D / 32;
  constexpr int KT = D / 16;
  constexpr int ROW = D * 2;                    // bytes per tile row
  constexpr int TILE = kBQ * D * 2;             // one 64-row Q or dO tile

  // [stage][Q=0 / dO=1] row tiles, then the row vectors, the key block, dS^T
  __shared__ __attribute__((aligned(1024))) char qdo[2][2][TILE];
  __shared__ __attribute__((aligned(1024))) char kblk[kBK * D * 2];
  __shared__ __attribute__((aligned(1024))) char dst_t[kBK * kBQ * 2];  // dS^T [128 keys][64 rows]
  __shared__ __attribute__((aligned(16))) float rowv[2][2][kBQ];        // [stage][L2=0 / D=1][row]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;
  const int col = lane & 31;

  // One workgroup per group of G key blocks sharing a dQ slot s: with n = n_slot, the pairs
  // (2jn + s, 2jn + 2n - 1 - s) for j < G / 2 (G = 1: block s alone), which gives every
  // slot the same causal work.  They are taken in decreasing order (blocks past the last
  // key are skipped), so that each block sees a superset of the query rows the blocks
  // before it saw.
  const int n_kb = (p.n_k + kBK - 1) / kBK;
  const int G = bwd_blocks_per_group(p.B, p.H, p.n_k);
  const int n_slot = (int)bwd_num_slots(p.B, p.H, p.n_k);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / n_slot;
  const int slot = L % n_slot;
  const int n_qb = (p.n_q + kBQ - 1) / kBQ;

  const long long hq = (long long)bh * p.n_q, hk = (long long)bh * p.n_k;
  const i32x4 qrs = raw_rsrc(p.q + hq * D, (long long)p.n_q * D * 2);
  const i32x4 dors = raw_rsrc(p.dout + hq * D, (long long)p.n_q * D * 2);
  const i32x4 l2rs = raw_rsrc(p.l2vec + hq, (long long)p.n_q * 4);
  const i32x4 dvrs = raw_rsrc(p.dvec + hq, (long long)p.n_q * 4);

  LdsAddr<D> la;  // over qdo: ka = A operand of S / dP (rows x d), va = A operand of dV^T / dK^T
  make_lds_addr<D>(la, (unsigned)(uintptr_t)(const lds_void*)&qdo[0][0][0], lane);

  // dQ product: wave w computes rows 32rb .. +31 (rb over RB), d columns 32cb .. +31
  constexpr int RB = D == 128 ? 2 : 1;
  const int cb = D == 128 ? wave : (wave & 1);
  const int rb0 = D == 128 ? 0 : (wave >> 1);
  unsigned da[RB][2], kba[2];
  {
    const unsigned dsb = (unsigned)(uintptr_t)(const lds_void*)dst_t;
    const unsigned kbb = (unsigned)(uintptr_t)(const lds_void*)kblk;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int r = 0; r < RB; ++r) da[r][h] = tr_nat_addr<kBQ>(dsb, lane, 0, 32 * (rb0 + r), h);
      kba[h] = tr_nat_addr<D>(kbb, lane, 0, 32 * cb, h);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      asm volatile("" : "+v"(kba[h]));
#pragma unroll
      for (int r = 0; r < RB; ++r) asm volatile("" : "+v"(da[r][h]));
    }
  }
  // this lane's dS^T store address: key row (key - k0), query rows 8g + 4hf (+32qh) in chunk 4qh + g
  const unsigned dsw = (unsigned)(uintptr_t)(const lds_void*)dst_t;

  int qb_add = n_qb;  // query blocks from here on already hold earlier blocks' contributions
  for (int pass = 0; pass < G; ++pass) {
    const int kb = G == 1 ? slot : (G / 2 - 1 - pass / 2) * 2 * n_slot + ((pass & 1) ? slot : 2 * n_slot - 1 - slot);
    if (kb >= n_kb) continue;  // uniform over the workgroup
    const int k0 = kb * kBK;
    const int kw0 = k0 + 32 * wave;     // this wave's keys kw0 .. kw0 + 31
    const int key = kw0 + col;          // this lane's key column
    // causal: rows below the block's first key see none of its keys
    const int qb0 = p.causal ? min(k0 / kBQ, n_qb) : 0;
    // every wave is done with the previous block's LDS buffers
    if (pass > 0) __syncthreads();

    // this wave's keys and values as B operands (lane = key, k = d): zero past n_k
    bf16x8 kf[KT], vf[KT];
    {
      const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + hk * D, (long long)p.n_k * D * 2);
      const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + hk * D, (long long)p.n_k * D * 2);
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const unsigned off = ((unsigned)key * D + 16 * t + 8 * hf) * 2u;
        kf[t] = as_bf16x8(__builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0)));
        vf[t] = as_bf16x8(__builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0)));
      }
    }
    // the whole key block, row-major swizzled, for the dQ product
    {
      constexpr int CPR = D / 8;
      const i32x4 krs = raw_rsrc(p.k + hk * D, (long long)p.n_k * D * 2);
#pragma unroll
      for (int i = 0; i < kBK * CPR / 256; ++i) {
        const int s = (i * 4 + wave) * 64 + lane;
        const int r = s / CPR;
        const int c = (s % CPR) ^ (swz<D>(r, 0) - r * CPR);
        lds_dma16(krs, kblk + (i * 4 + wave) * 64 * 16, ((unsigned)(k0 + r) * D + c * 8) * 2u);
      }
    }

    f32x16 dvt[NB], dkt[NB];  // dV^T, dK^T: rows d, columns this wave's keys
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      dvt[nb] = f32x16{};
      dkt[nb] = f32x16{};
    }

    auto issue_q = [&](int stage, int qi) {
      const int r0 = qi * kBQ;
      issue_rows<D>(qrs, qdo[stage][0], r0, wave, lane);
      issue_rows<D>(dors, qdo[stage][1], r0, wave, lane);
      // lanes 0-15 of wave 0 bring the 64 L2 values, lanes 16-31 the 64 D values
      // (lane l writes 16 bytes at the LDS base + 16 l)
      if (wave == 0 && lane < 16)
        lds_dma16(l2rs, reinterpret_cast<const char*>(&rowv[stage][0][0]), (unsigned)(r0 * 4 + lane * 16));
      else if (wave == 0 && lane < 32)
        lds_dma16(dvrs, reinterpret_cast<const char*>(&rowv[stage][1][0]) - 256, (unsigned)(r0 * 4 + (lane - 16) * 16));
    };

    // K^T fragments of this wave's d columns for the dQ product: the key block is the
    // same for every query block, so they are read from LDS once and kept in registers
    bf16x8 kTr[kBK / 16];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // the key block is in LDS
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) kTr[ks] = tr_pair(kba[0] + ks * 16 * ROW, kba[1] + ks * 16 * ROW);

    // the key/value fragments have arrived (waited for here once, not inside the query loop)
#pragma unroll
    for (int t = 0; t < KT; ++t) asm volatile("" ::"v"(kf[t]), "v"(vf[t]));

    if (qb0 < n_qb) issue_q(0, qb0);

    // one query block; STG is the LDS stage (compile-time so that offsets are immediates)
    auto step = [&](auto stg_c, int qi) {
      constexpr int STG = decltype(stg_c)::value;
      constexpr unsigned QOFF = STG * 2 * TILE, DOFF = QOFF + TILE;
      const int i0 = qi * kBQ;
      // masking: causal diagonal, query rows past n_q, keys past n_k
      const bool need_mask = (p.causal && i0 < kw0 + 31) || (i0 + kBQ > p.n_q) || (kw0 + 32 > p.n_k);
      // In the second pass the dQ accumulators of this query block start from what this same
      // thread stored for it in the first pass (read now, so that the step's products hide the
      // latency; rows past n_q read as zero through the range check); otherwise from zero.
      const long long R = (long long)p.B * p.H * p.n_q;
      f32x16 dq0[RB];
      if (qi >= qb_add) {
        const __amdgpu_buffer_rsrc_t srs =
            make_rsrc(p.ws_dq + ((long long)slot * R + hq) * D, (long long)p.n_q * D * 4);
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const unsigned off = ((unsigned)(i0 + 32 * (rb0 + r) + col) * D + 32 * cb + 8 * g + 4 * hf) * 4u;
            const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(srs, off, 0, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) dq0[r][4 * g + e] = v[e];
          }
      } else {
#pragma unroll
        for (int r = 0; r < RB; ++r) dq0[r] = f32x16{};
      }

      // S = Q K^T and dP = dO V^T for two 32-row halves
      f32x16 s[2], dp[2];
      {
        // operands read PF steps ahead of their products (LDS latency exceeds two products)
        constexpr int PF = 2;
        constexpr int NST = 2 * KT;  // steps (qh, t)
        bf16x8 ra[PF][2];
#pragma unroll
        for (int st = 0; st < PF; ++st) {
          ra[st][0] = lds_load<bf16x8>(la.ka[st % KT] + QOFF + (st / KT) * 32 * ROW);
          ra[st][1] = lds_load<bf16x8>(la.ka[st % KT] + DOFF + (st / KT) * 32 * ROW);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          const int qh = st / KT, t = st % KT;
          if (t == 0) {
            s[qh] = f32x16{};
            dp[qh] = f32x16{};
          }
          s[qh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[st % PF][0], kf[t], s[qh], 0, 0, 0);
          dp[qh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[st % PF][1], vf[t], dp[qh], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          if (st + PF < NST) {
            const int s2 = st + PF;
            ra[st % PF][0] = lds_load<bf16x8>(la.ka[s2 % KT] + QOFF + (s2 / KT) * 32 * ROW);
            ra[st % PF][1] = lds_load<bf16x8>(la.ka[s2 % KT] + DOFF + (s2 / KT) * 32 * ROW);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
        }
      }
      // P = exp2(s * scale*log2e - LSE*log2e), dS = P (dP - D); row of register r:
      // 32qh + 8(r/4) + 4hf + r%4
      bf16x8 pb[2][2], db[2][2];
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        f32x16 pv, dsv;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int rl = 32 * qh + 8 * g + 4 * hf;  // first of this lane's 4 rows in the tile
          const f32x4 l2 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
              (uintptr_t)(const lds_void*)&rowv[STG][0][rl]);
          const f32x4 dd = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
              (uintptr_t)(const lds_void*)&rowv[STG][1][rl]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qh][r], sl2, -l2[e]));
            if (need_mask) {
              const int row = i0 + rl + e;
              const bool ok = row < p.n_q && key < p.n_k && (!p.causal || key <= row);
              pr = ok ? pr : 0.f;
            }
            pv[r] = pr;
            dsv[r] = pr * (dp[qh][r] - dd[e]);
          }
        }
        pb[qh][0] = cvt_bf16x8(slice8(pv, 0));
        pb[qh][1] = cvt_bf16x8(slice8(pv, 1));
        db[qh][0] = cvt_bf16x8(slice8(dsv, 0));
        db[qh][1] = cvt_bf16x8(slice8(dsv, 1));
        // dS^T to LDS: 4 consecutive rows (8 bytes) per g
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = 4 * qh + g;  // chunk of 8 rows
          const unsigned addr = dsw + swz<kBQ>(key - k0, c) * 16 + hf * 8;
          const u32x4 w4 = __builtin_bit_cast(u32x4, g < 2 ? db[qh][0] : db[qh][1]);
          const u32x2 w2 = (g & 1) ? u32x2{w4.z, w4.w} : u32x2{w4.x, w4.y};
          *reinterpret_cast<__attribute__((address_space(3))) u32x2*>((uintptr_t)addr) = w2;
        }
      }
      // every wave's dS^T is in LDS
      __syncthreads();
      // dQ contribution of this key block, computed transposed (dQ^T = K^T dS^T)
      // so that each lane holds one query row and 4 consecutive d per register
      // group: rows 32(rb0 + r) + lane%32, d columns 32cb + 8g + 4hf + 0..3
      // Steps (ks, r): consecutive products accumulate into different row groups, and
      // the dS^T operands are read PF steps ahead.
      {
        constexpr int NST = (kBK / 16) * RB;
        constexpr int PF = 3;
        f32x16 dqt[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) dqt[r] = dq0[r];
        bf16x8 rds[PF];
        auto load = [&](int st) {
          const int ks = st / RB, r = st % RB;
          rds[st % PF] = tr_pair(da[r][0] + ks * 16 * kBQ * 2, da[r][1] + ks * 16 * kBQ * 2);
        };
#pragma unroll
        for (int st = 0; st < PF; ++st) load(st);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          const int ks = st / RB, r = st % RB;
          dqt[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kTr[ks], rds[st % PF], dqt[r], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (st + PF < NST) {
            load(st + PF);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const int row = i0 + 32 * (rb0 + r) + col;
          if (row < p.n_q) {
            float* ws = p.ws_dq + ((long long)slot * R + hq + row) * D + 32 * cb + 4 * hf;
#pragma unroll
            for (int g = 0; g < 4; ++g)
              __builtin_nontemporal_store(
                  f32x4{dqt[r][4 * g], dqt[r][4 * g + 1], dqt[r][4 * g + 2], dqt[r][4 * g + 3]},
                  reinterpret_cast<f32x4*>(ws + 8 * g));
          }
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the 64 rows (4 k-steps of 16), steps
      // (qh, t, nb) in that order; the transposed operands are read PF steps ahead of
      // their products (one LDS read outlasts the two products it feeds).  These come
      // after the dQ products: the dQ stores then complete while they run, instead of
      // holding up the wait at the top of the next step (one counter covers loads and
      // stores).
      {
        constexpr int NST = 4 * NB;
        constexpr int PF = 3;
        bf16x8 rdo[PF], rq[PF];
        auto load = [&](int st) {
          const int qh = st / (2 * NB), t = (st / NB) % 2, nb = st % NB;
          const unsigned roff = (32 * qh + 16 * t) * ROW;
          rdo[st % PF] = tr_pair(la.va[2 * nb] + DOFF + roff, la.va[2 * nb + 1] + DOFF + roff);
          rq[st % PF] = tr_pair(la.va[2 * nb] + QOFF + roff, la.va[2 * nb + 1] + QOFF + roff);
        };
#pragma unroll
        for (int st = 0; st < PF; ++st) load(st);
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * PF, 0);
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          const int qh = st / (2 * NB), t = (st / NB) % 2, nb = st % NB;
          dvt[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rdo[st % PF], pb[qh][t], dvt[nb], 0, 0, 0);
          dkt[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rq[st % PF], db[qh][t], dkt[nb], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          if (st + PF < NST) {
            load(st + PF);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          }
        }
      }
    };

    // two LDS stages, unrolled by two so that every offset is an immediate
    for (int qi = qb0; qi < n_qb; qi += 2) {
      // keep the dV^T / dK^T accumulators in AGPRs across iterations: otherwise the
      // loop-carried values are assigned VGPRs and each iteration copies all 128 of
      // them out of and back into the AGPRs the products accumulate in
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+a"(dvt[nb]), "+a"(dkt[nb]));
      // vmcnt(0) through the builtin, which the compiler's own wait tracking sees: it then
      // knows that no earlier load is outstanding inside the step
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();  // stage 0 published; dS^T and stage 1 free
      if (qi + 1 < n_qb) issue_q(1, qi + 1);
      step(std::integral_constant<int, 0>{}, qi);
      if (qi + 1 < n_qb) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
        if (qi + 2 < n_qb) issue_q(0, qi + 2);
        step(std::integral_constant<int, 1>{}, qi + 1);
      }
    }

    // dK = scale * dK, dV, rows d 32nb + 8g + 4hf + 0..3 of this lane's key
    if (key < p.n_k) {
      uint16_t* dkr = p.dk + (hk + key) * D;
      uint16_t* dvr = p.dv + (hk + key) * D;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          const f32x4 k4 = {dkt[nb][4 * g] * p.scale, dkt[nb][4 * g + 1] * p.scale, dkt[nb][4 * g + 2] * p.scale,
                            dkt[nb][4 * g + 3] * p.scale};
          const f32x4 v4 = {dvt[nb][4 * g], dvt[nb][4 * g + 1], dvt[nb][4 * g + 2], dvt[nb][4 * g + 3]};
          const int d0 = 32 * nb + 8 * g + 4 * hf;
          *reinterpret_cast<u32x2*>(dkr + d0) = __builtin_bit_cast(u32x2, __builtin_convertvector(k4, bf16x4));
          *reinterpret_cast<u32x2*>(dvr + d0) = __builtin_bit_cast(u32x2, __builtin_convertvector(v4, bf16x4));
        }
    }
    // this block's partial stores have completed before the next block reads them back
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    qb_add = qb0;
  }  // pass
}

// ---------------------------------------------------------------------------
// dQ_i = scale * sum over slots s of the partials, in slot order; under the
// causal mask slot s holds rows from s*128 on only.  One thread per
// 4 elements.
template <int D>
__global__ void __launch_bounds__(256) bwd_dq_kernel(BwdParams p) {
  const long long R = (long long)p.B * p.H * p.n_q;
  const long long idx = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (idx >= R * D) return;
  const long long rg = idx / D;
  const int i = (int)(rg % p.n_q);
  const int n_slot = (int)bwd_num_slots(p.B, p.H, p.n_k);
  // the lowest key block of slot s is block s; under the causal mask query block qi was
  // processed by it (and so the slot written) iff s*128 <= qi*64 + 63
  const int s_end = p.causal ? min(n_slot, (i / kBQ * kBQ + kBQ - 1) / kBK + 1) : n_slot;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // the partials are written once and read once: non-temporal on both sides
#pragma unroll 4
  for (int s = 0; s < s_end; ++s)
    acc += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.ws_dq + (long long)s * R * D + idx));
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<u32x2*>(p.dq + idx) = __builtin_bit_cast(u32x2, __builtin_convertvector(acc * p.scale, bf16x4));
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  const long long R = (long long)p.B * p.H * p.n_q;
  const float sl2 = p.scale * kLog2e;
  const unsigned g0 = (unsigned)((R + (256 / (p.d / 8)) - 1) / (256 / (p.d / 8)));
  const unsigned g1 = (unsigned)((long long)p.B * p.H * bwd_num_slots(p.B, p.H, p.n_k));
  const unsigned g2 = (unsigned)((R * p.d / 4 + 255) / 256);
  if (p.d == 128) {
    hipLaunchKernelGGL(bwd_prep_kernel<128>, dim3(g0), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(bwd_kv_kernel<128>, dim3(g1), dim3(256), 0, stream, p, sl2);
    hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3(g2), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(bwd_prep_kernel<64>, dim3(g0), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(bwd_kv_kernel<64>, dim3(g1), dim3(256), 0, stream, p, sl2);
    hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3(g2), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace fa2
