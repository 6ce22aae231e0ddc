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
// Two launches, the dQ pass first:
//   bwd_dq_kernel      one workgroup per 128-row query block (one wave per 32
//                      rows): forms -D_i and LSE_i * log2(e) of its rows (kept
//                      in registers and stored for the key pass), streams
//                      64-key K/V tiles through LDS as the forward does and
//                      runs three products (S, dP, then dQ += dS K); dQ stays
//                      in registers.  From 2048 query rows at d = 128,
//                      bwd_dq_pp_kernel does the same work with 8 waves in the
//                      ping-pong schedule of the forward
//   bwd_kv_pp_kernel   one workgroup of 8 waves per 128-key block: two waves per
//                      32 keys, each over half of every 64-row query block
//                      streamed through LDS; four products on the matrix cores
//                      (S, dP, then dV and dK); K and V of the block stay in
//                      LDS, dK and dV in registers, and the two halves' sums
//                      are added at the end.  The two waves of a SIMD run one
//                      phase apart (ping-pong schedule)
// This is the deterministic form of the synthesis page's section 5 item 2
// without any partial sums in memory: every gradient element is accumulated
// by exactly one wave, in a fixed order, and written once, so the result is
// bit-reproducible.  S and dP are computed twice (once per pass): seven
// products instead of five, against no dQ workspace and no reduction pass.
//
// In the key pass the scores are computed as S = Q K^T (query rows x 32
// keys), so every lane owns one key column: P and dS in accumulator layout
// are then directly the B operands of dV^T += dO^T P and dK^T += Q^T dS.  In
// bwd_dq_kernel they are computed transposed (S^T = K Q^T, as the forward),
// so every lane owns one query row and dS^T is the B operand of
// dQ^T += K^T dS^T, with K^T read transposed from LDS.
#include "fa2_device.h"
#include "fa2_internal.h"

#include <math.h>

#include <type_traits>

namespace fa2 {
namespace {

constexpr int kBK = 128;  // keys per workgroup of the key pass
constexpr int kBQ = 64;   // query rows per step
// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt fields at their maxima)
constexpr int kWaitVm0 = 0x0F70;

// ---------------------------------------------------------------------------
// Two transposed 8-byte LDS reads forming one 16-byte MFMA operand.
__device__ __forceinline__ bf16x8 tr_pair(unsigned a0, unsigned a1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4*>((uintptr_t)a0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4*>((uintptr_t)a1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------------------
// Key pass: one workgroup of 8 waves per (batch, head, 128-key block).  Wave w owns keys
// 32 (w % 4) .. + 31 of the block and rows 32 (w / 4) .. + 31 of every 64-row query
// block, so the two waves of a SIMD share their keys and split the rows; each
// accumulates its own dV^T, dK^T (registers) and the pair is summed through LDS at the
// end.  K and V of the block stay in LDS for the whole pass and serve as the B operands
// of S and dP.  The two waves of a SIMD run one phase apart as in the ping-pong forward:
// group 0 (waves 0-3) one phase ahead of group 1 (waves 4-7).  Per query block j and wave:
//   matrix phase:  dV^T += dO_{j-1}^T P_{j-1};  dK^T += Q_{j-1}^T dS_{j-1};
//                  S_j = Q_j K^T;  dP_j = dO_j V^T
//   vector phase:  P_j = exp2(s * scale*log2e - L2) (0 where masked), dS_j = P_j (dP_j - D)
// so that one wave of a SIMD issues 32 products while its partner does the vector work.
// The Q/dO tiles have two stages, each filled half by half: a group loads its rows of
// its next block at the start of its vector phase, into the place of the block its
// matrix phase has just finished with, and retires the loads before the phase ends, so
// that neither the issue of the loads nor the wait for them falls in a matrix phase.
template <int D>
__global__ void __launch_bounds__(512, 1) bwd_kv_pp_kernel(BwdParams p, float sl2, int sched) {
  constexpr int NW = 8;
  constexpr int NB = D / 32;
  constexpr int KT = D / 16;
  constexpr int ROW = D * 2;         // bytes per row
  constexpr int TILE = kBQ * D * 2;  // one 64-row Q or dO tile
  constexpr int HALF = TILE / 2;     // its 32 rows of one group
  constexpr int BLK = kBK * D * 2;   // the 128-key K or V block
  constexpr int CPR = D / 8;

  __shared__ __attribute__((aligned(1024))) char kvb[2][BLK];       // K = 0, V = 1
  __shared__ __attribute__((aligned(1024))) char qdo[2][2][TILE];   // [stage][Q = 0 / dO = 1]
  __shared__ __attribute__((aligned(16))) float rowv[2][2][kBQ];     // [stage][L2 = 0 / D = 1][row]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = wave & 3;   // key slice
  const int rh = wave >> 2;  // row half, and the group
  const int hf = lane >> 5;
  const int col = lane & 31;

  const int n_kb = (p.n_k + kBK - 1) / kBK;
  int bh, kb;  // under the causal mask key block 0 sees the most query blocks: it goes first
  wg_coords(wg_logical(sched), n_kb, p.B * p.H, sched, false, bh, kb);
  const int n_qb = (p.n_q + kBQ - 1) / kBQ;

  const long long hq = (long long)bh * p.n_q, hk = (long long)bh * p.n_k;
  const i32x4 qrs = raw_rsrc(p.q + hq * D, (long long)p.n_q * D * 2);
  const i32x4 dors = raw_rsrc(p.dout + hq * D, (long long)p.n_q * D * 2);
  const i32x4 l2rs = raw_rsrc(p.l2vec + hq, (long long)p.n_q * 4);
  const i32x4 dvrs = raw_rsrc(p.dvec + hq, (long long)p.n_q * 4);
  const i32x4 krs = raw_rsrc(p.k + hk * D, (long long)p.n_k * D * 2);
  const i32x4 vrs = raw_rsrc(p.v + hk * D, (long long)p.n_k * D * 2);

  LdsAddr<D> la, lk;  // la over qdo from this wave's first row, lk over K from its first key
  make_lds_addr<D>(la, (unsigned)(uintptr_t)(const lds_void*)&qdo[0][0][0] + (unsigned)(32 * rh) * ROW, lane);
  make_lds_addr<D>(lk, (unsigned)(uintptr_t)(const lds_void*)&kvb[0][0] + (unsigned)(32 * ks) * ROW, lane);

  const int k0 = kb * kBK;
  const int kw0 = k0 + 32 * ks;  // this wave's keys kw0 .. kw0 + 31
  const int key = kw0 + col;     // this lane's key column
  const int qb0 = p.causal ? min(k0 / kBQ, n_qb) : 0;
  const int n_t = n_qb - qb0;    // query blocks this key block sees

  // slot offsets: the K/V block takes NLDB loads per wave and array, a half tile NLDH per
  // wave of the loading group (the swizzle repeats every 16 rows)
  constexpr int NLDB = kBK * CPR / (64 * NW);
  constexpr int NLDH = 32 * CPR / (64 * 4);
  constexpr int NDMA = 2 * NLDH;  // Q parts, then dO parts
  unsigned offh[NLDH];
#pragma unroll
  for (int i = 0; i < NLDH; ++i) {
    const int sl = (i * 4 + ks) * 64 + lane;
    const int r = sl / CPR;
    const int c = (sl % CPR) ^ (swz<D>(r, 0) - r * CPR);
    offh[i] = (unsigned)((r * D + c * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < NLDB; ++i) {
    const int sl = (i * NW + wave) * 64 + lane;
    const int r = sl / CPR;
    const int c = (sl % CPR) ^ (swz<D>(r, 0) - r * CPR);
    const unsigned o = (unsigned)((r * D + c * 8) * 2) + (unsigned)k0 * D * 2;
    lds_dma16(krs, &kvb[0][(i * NW + wave) * 64 * 16], o);
    lds_dma16(vrs, &kvb[1][(i * NW + wave) * 64 * 16], o);
  }
  // part i of this wave's share of half h of query block qi, into stage st; part 0 of a
  // key-slice-0 wave also brings the half's 32 L2 and 32 D values
  auto dma_half = [&](int st, int h, int qi, int i) {
    if (qi >= n_qb) return;
    const unsigned goff = (unsigned)(qi * kBQ + 32 * h) * ROW;
    const int a = i / NLDH, ii = i % NLDH;
    lds_dma16(a ? dors : qrs, &qdo[st][a][h * HALF + (ii * 4 + ks) * 64 * 16], offh[ii] + goff);
    if (i == 0 && ks == 0) {
      const unsigned roff = (unsigned)(qi * kBQ + 32 * h) * 4;
      if (lane < 8)
        lds_dma16(l2rs, reinterpret_cast<const char*>(&rowv[st][0][32 * h]), roff + lane * 16);
      else if (lane < 16)
        lds_dma16(dvrs, reinterpret_cast<const char*>(&rowv[st][1][32 * h]) - 128, roff + (lane - 8) * 16);
    }
  };
  if (rh == 0) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) dma_half(0, 0, qb0, i);
  }
  // the first matrix phase of each group multiplies P = dS = 0 with stage 1, which no
  // load has written yet: zero it
  {
    constexpr int PER = 2 * TILE / (64 * NW);
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < PER / 16; ++i)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
          (uintptr_t)(const lds_void*)&qdo[1][0][(tid * (PER / 16) + i) * 16]) = z;
  }

  f32x16 dvt[NB], dkt[NB];  // dV^T, dK^T over this wave's rows: rows d, columns its keys
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    dvt[nb] = f32x16{};
    dkt[nb] = f32x16{};
  }
  f32x16 s = {}, dp = {};
  bf16x8 pb[2] = {}, db[2] = {};
  f32x4 l2r[4];  // LSE*log2e of this lane's rows of the block in S, read by the matrix phase

  // matrix phase of block j, whose tiles sit in stage STG (block j - 1 in the other): one
  // stream of 32 products, dV^T and dK^T of block j - 1 (16-row k-step t, d block nb)
  // then S and dP of block j (k-step t), each product's operands read PD products ahead
  auto mat = [&](int j, auto stg_c) {
    constexpr int STG = decltype(stg_c)::value;
    constexpr unsigned QC = STG * 2 * TILE, DC = QC + TILE;
    constexpr unsigned QP = (1 - STG) * 2 * TILE, DP = QP + TILE;
    constexpr int NG = 4 * NB;  // gradient products
    constexpr int NM = NG + 2 * KT;
    constexpr int PD = 4;
    bf16x8 oa[PD], ob[PD];
    f32x4 nd[4];  // -D of this lane's rows of block j: the start of the dP accumulator
    auto load = [&](int m) {
      if (m < NG) {
        const int st = m / 2, t = st / NB, nb = st % NB;
        const unsigned o = (m % 2 ? QP : DP) + 16 * t * ROW;
        oa[m % PD] = tr_pair(la.va[2 * nb] + o, la.va[2 * nb + 1] + o);
      } else {
        const int i = m - NG, t = i / 2;
        oa[m % PD] = lds_load<bf16x8>(la.ka[t] + (i % 2 ? DC : QC));
        ob[m % PD] = lds_load<bf16x8>(lk.ka[t] + (i % 2 ? BLK : 0));
      }
    };
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int m = 0; m < PD; ++m) load(m);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PD, 0);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m < NG) {
        const int st = m / 2, t = st / NB, nb = st % NB;
        if (m % 2 == 0)
          dvt[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[m % PD], pb[t], dvt[nb], 0, 0, 0);
        else
          dkt[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[m % PD], db[t], dkt[nb], 0, 0, 0);
      } else {
        const int i = m - NG, t = i / 2;
        if (i % 2 == 0)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[m % PD], ob[m % PD], t ? s : f32x16{}, 0, 0, 0);
        else
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              oa[m % PD], ob[m % PD],
              t ? dp
                : __builtin_shufflevector(__builtin_shufflevector(nd[0], nd[1], 0, 1, 2, 3, 4, 5, 6, 7),
                                          __builtin_shufflevector(nd[2], nd[3], 0, 1, 2, 3, 4, 5, 6, 7), 0, 1,
                                          2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15),
              0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m + PD < NM) {
        load(m + PD);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      if (m == NG - 4) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          nd[g] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
              (uintptr_t)(const lds_void*)&rowv[STG][1][32 * rh + 8 * g + 4 * hf]);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
      if (m == NM - 4) {  // and LSE*log2e of the rows for the vector phase
#pragma unroll
        for (int g = 0; g < 4; ++g)
          l2r[g] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
              (uintptr_t)(const lds_void*)&rowv[STG][0][32 * rh + 8 * g + 4 * hf]);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // vector phase of block j (stage STG): P and dS (bf16) for the next matrix phase; the
  // group's loads (dma(i), i < NDMA) are issued first.  dp holds dP - D already.
  auto vec = [&](int j, auto stg_c, auto&& dma) {
    constexpr int STG = decltype(stg_c)::value;
#pragma unroll
    for (int i = 0; i < NDMA; ++i) dma(i);
    if (j < 0 || j >= n_t) {
      pb[0] = pb[1] = db[0] = db[1] = bf16x8{};
      return;
    }
    const int i0 = (qb0 + j) * kBQ + 32 * rh;  // first row
    // element (8g + e) is row i0 + 8g + 4hf + e: visible to this lane's key when
    // lo <= 8g + e < hi
    const int lo = (p.causal ? key - i0 : 0) - 4 * hf;
    const int hi = (key < p.n_k ? p.n_q - i0 : 0) - 4 * hf;
    auto softmax = [&](auto mask_c) {
      constexpr bool MASKED = decltype(mask_c)::value;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l2 = l2r[g];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -l2[e]));
          if (MASKED) {
            const int c = 8 * g + e;
            pr = (c >= lo && c < hi) ? pr : 0.f;
          }
          dp[r] = pr * dp[r];  // dS over dP - D (the products started from -D) and P over S
          s[r] = pr;
        }
      }
      pb[0] = cvt_bf16x8(slice8(s, 0));
      pb[1] = cvt_bf16x8(slice8(s, 1));
      db[0] = cvt_bf16x8(slice8(dp, 0));
      db[1] = cvt_bf16x8(slice8(dp, 1));
    };
    // masking: causal diagonal, query rows past n_q, keys past n_k (uniform per wave)
    if ((p.causal && i0 < kw0 + 31) || (i0 + 32 > p.n_q) || (kw0 + 32 > p.n_k))
      softmax(std::true_type{});
    else
      softmax(std::false_type{});
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // group 0 loads the first half of block j + 1 in its vector phase on block j, group 1
  // the second half of block j in its vector phase on block j - 1: places last read by
  // the group's matrix phase just before
  auto iter0 = [&](int j, auto stg_c) {
    constexpr int STG = decltype(stg_c)::value;
    mat(j, stg_c);
    __syncthreads();
    vec(j, stg_c, [&](int i) { dma_half(1 - STG, 0, qb0 + j + 1, i); });
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  };
  auto iter1 = [&](int j, auto stg_c) {
    constexpr int STG = decltype(stg_c)::value;
    vec(j - 1, std::integral_constant<int, 1 - STG>{}, [&](int i) { dma_half(STG, 1, qb0 + j, i); });
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    mat(j, stg_c);
    __syncthreads();
  };

  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();  // the K/V block, the first half tile and the zeroed stage published
  if (rh == 0) {
    for (int j = 0; j <= n_t; j += 2) {
      iter0(j, S0{});
      if (j + 1 <= n_t) iter0(j + 1, S1{});
    }
  } else {
    for (int j = 0; j <= n_t; j += 2) {
      iter1(j, S0{});
      if (j + 1 <= n_t) iter1(j + 1, S1{});
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();  // every wave is done with the tiles: their space takes the partial sums

  // The workgroup 256 ids later runs on this XCD next (ids go round the 8 XCDs, 32 units each):
  // touch one dword of each 128-byte line of its K and V block, so that its prologue finds them
  // in L2.  Waves 0-3 take K, 4-7 V, 64 lines each; the value is only kept until the end.
  unsigned pref = 0;
  if (blockIdx.x + 256 < gridDim.x) {
    int nbh, nkb;
    wg_coords((sched & kSchedRemap) ? xcd_remap(blockIdx.x + 256, gridDim.x) : (int)blockIdx.x + 256, n_kb,
              p.B * p.H, sched, false, nbh, nkb);
    const long long nhk = (long long)nbh * p.n_k;
    const int nk0 = nkb * kBK;
    const __amdgpu_buffer_rsrc_t prs = make_rsrc((wave < 4 ? p.k : p.v) + (nhk + nk0) * D, (long long)(p.n_k - nk0) * D * 2);
    pref = __builtin_amdgcn_raw_buffer_load_b32(prs, (unsigned)(((wave & 3) * 64 + lane) * 128) % (unsigned)BLK, 0, 0);
  }

  // The two waves of a key slice hold partial dV^T and dK^T of the same keys.  The second row
  // half hands over its dV^T (in the Q/dO tiles' space), the first half its dK^T (in the K/V
  // block's space); after one barrier the first half finishes dV and the second dK, staging its
  // rows for write_rows in its own slice of that space once it has read the partner's sums.
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  constexpr int SLICE = NB * 16 * 64 * 4;  // bytes of one wave's partial sums
  static_assert(4 * SLICE <= (int)sizeof(qdo) && 4 * SLICE <= (int)sizeof(kvb), "partials fit");
  static_assert(kStagedRows<D> <= SLICE, "the staged rows fit in the slice");
  const unsigned xv = (unsigned)(uintptr_t)(const lds_void*)&qdo[0][0][0] + (unsigned)(ks * SLICE);
  const unsigned xk = (unsigned)(uintptr_t)(const lds_void*)&kvb[0][0] + (unsigned)(ks * SLICE);
  auto slot = [&](unsigned base, int nb, int q) { return base + (unsigned)(((nb * 4 + q) * 64 + lane) * 16); };
  auto hand_over = [&](const f32x16(&acc)[NB], unsigned base) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {acc[nb][4 * q], acc[nb][4 * q + 1], acc[nb][4 * q + 2], acc[nb][4 * q + 3]};
        *reinterpret_cast<lds_f32x4*>((uintptr_t)slot(base, nb, q)) = v;
      }
  };
  auto finish = [&](const f32x16(&acc)[NB], unsigned base, uint16_t* grad, float sc) {
    u32x2 out[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 o = *reinterpret_cast<const lds_f32x4*>((uintptr_t)slot(base, nb, q));
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (acc[nb][4 * q + e] + o[e]) * sc;
        out[nb][q] = __builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4));
      }
    write_rows<D>(out, base, grad + (hk + kw0) * D, p.n_k - kw0, lane);
  };
  if (rh) hand_over(dvt, xv);
  else hand_over(dkt, xk);
  __syncthreads();
  if (rh) finish(dkt, xk, p.dk, p.scale);
  else finish(dvt, xv, p.dv, 1.f);
  asm volatile("" ::"v"(pref));
}

// ---------------------------------------------------------------------------
// dQ pass: one workgroup of 4 waves per (batch, head, 128-row query block), the K and
// V tiles of 64 keys streamed through a two-stage LDS ring as in the forward.  Per wave
// (32 query rows, one per lane column) and tile:
//   S^T  = K Q^T      A = K rows from LDS, B = Q in registers
//   dP^T = V dO^T     A = V rows from LDS, B = dO in registers
//   P = exp2(s * scale*log2e - LSE*log2e) (0 where masked), dS = P (dP - D)
//   dQ^T += K^T dS^T  A = K^T read transposed from LDS, B = dS^T (bf16) in registers
// and at the end dQ = scale * dQ, rounded to bf16.
constexpr int kBC = 64;  // keys per tile of bwd_dq_kernel

template <int D>
__device__ __forceinline__ void issue_kv(i32x4 krs, i32x4 vrs, const char* kdst, const char* vdst, int k0, int wave,
                                         int lane) {
  constexpr int CPR = D / 8;
  constexpr int NLD = kBC * CPR / 256;
  const unsigned toff = (unsigned)k0 * D * 2;
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int s = (i * 4 + wave) * 64 + lane;
    const int r = s / CPR;
    const int c = (s % CPR) ^ (swz<D>(r, 0) - r * CPR);
    const unsigned off = (unsigned)((r * D + c * 8) * 2) + toff;
    const int sbase = (i * 4 + wave) * 64 * 16;
    lds_dma16(krs, kdst + sbase, off);
    lds_dma16(vrs, vdst + sbase, off);
  }
}

// acc[0..1] = A B over the tile's two 32-key blocks: A rows from the LDS tile at OFF,
// B = this wave's fragments bf (row operand), k-steps of 16; operands read two ahead
template <int D, unsigned OFF, typename Dma>
__device__ __forceinline__ void rows_product(const LdsAddr<D>& la, const bf16x8 (&bf)[D / 16], f32x16& a0,
                                             f32x16& a1, float start, Dma&& dma) {
  constexpr unsigned ROW = D * 2;
  constexpr int KT = D / 16;
  constexpr int PF = 2;
  bf16x8 a[PF][2];
#pragma unroll
  for (int t = 0; t < PF; ++t) {
    a[t][0] = lds_load<bf16x8>(la.ka[t] + OFF);
    a[t][1] = lds_load<bf16x8>(la.ka[t] + OFF + 32 * ROW);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) {  // every element of this lane's row starts at `start`
    a0[r] = start;
    a1[r] = start;
  }
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t % PF][0], bf[t], a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t % PF][1], bf[t], a1, 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    if (t + PF < KT) {
      a[t % PF][0] = lds_load<bf16x8>(la.ka[t + PF] + OFF);
      a[t % PF][1] = lds_load<bf16x8>(la.ka[t + PF] + OFF + 32 * ROW);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    dma(t);
  }
}

template <int D>
__global__ void __launch_bounds__(256, 2) bwd_dq_kernel(BwdParams p, float sl2, int sched) {
  constexpr int BR = 128;
  constexpr int KT = D / 16;
  constexpr int NB = D / 32;
  constexpr unsigned ROW = D * 2;
  constexpr int TILE = kBC * D * 2;
  constexpr unsigned STAGE = 2 * TILE;

  __shared__ __attribute__((aligned(1024))) char lds[2][2][TILE];  // [stage][K=0 / V=1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;
  const int col = lane & 31;

  const int n_qb = (p.n_q + BR - 1) / BR;
  int bh, qb;
  // under the causal mask the last query blocks see the most keys: heaviest first
  wg_coords(wg_logical(sched), n_qb, p.B * p.H, sched, p.causal != 0, bh, qb);
  const int q0 = qb * BR;
  const int q0w = q0 + 32 * wave;
  const int row = q0w + col;
  // keys seen by some row of the workgroup [0, khi), of this wave [0, khi_w)
  const int khi = p.causal ? min(p.n_k, q0 + BR) : p.n_k;
  const int khi_w = p.causal ? min(p.n_k, q0w + 32) : p.n_k;
  const int n_tiles = (khi + kBC - 1) / kBC;

  const long long hq = (long long)bh * p.n_q, hk = (long long)bh * p.n_k;
  const i32x4 krs = raw_rsrc(p.k + hk * D, (long long)khi * D * 2);
  const i32x4 vrs = raw_rsrc(p.v + hk * D, (long long)khi * D * 2);

  // Q and dO rows of this lane as B operands (k = d), zero past n_q; the row's LSE*log2e and D
  bf16x8 qf[KT], dof[KT];
  float l2 = 0.f, dd = 0.f;
  {
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q + hq * D, (long long)p.n_q * D * 2);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(p.dout + hq * D, (long long)p.n_q * D * 2);
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const unsigned off = ((unsigned)row * D + 16 * t + 8 * hf) * 2u;
      qf[t] = as_bf16x8(__builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0)));
      dof[t] = as_bf16x8(__builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(drs, off, 0, 0)));
    }
    // -D = -sum_c dO_c O_c of the row (its two halves in lanes c and c + 32) and LSE*log2e,
    // kept in registers and stored for the key pass
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(p.o + hq * D, (long long)p.n_q * D * 2);
    float dpart = 0.f;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const unsigned off = ((unsigned)row * D + 16 * t + 8 * hf) * 2u;
      const u32x4 ov = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ors, off, 0, 0));
      const u32x4 dv = __builtin_bit_cast(u32x4, dof[t]);
      const unsigned o0 = ov.x, o1 = ov.y, o2 = ov.z, o3 = ov.w, d0 = dv.x, d1 = dv.y, d2 = dv.z, d3 = dv.w;
      dpart = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d0), __builtin_bit_cast(bf16x2, o0), dpart, false);
      dpart = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d1), __builtin_bit_cast(bf16x2, o1), dpart, false);
      dpart = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d2), __builtin_bit_cast(bf16x2, o2), dpart, false);
      dpart = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d3), __builtin_bit_cast(bf16x2, o3), dpart, false);
    }
    const float dsum = dpart + __shfl_xor(dpart, 32);
    if (row < p.n_q) {
      l2 = p.lse[hq + row] * kLog2e;
      dd = -dsum;
      if (hf == 0) {
        p.dvec[hq + row] = dd;
        p.l2vec[hq + row] = l2;
      }
    }
  }
  f32x16 dq[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) dq[nb] = f32x16{};

  LdsAddr<D> la;
  make_lds_addr<D>(la, (unsigned)(uintptr_t)(const lds_void*)&lds[0][0][0], lane);
  constexpr int NLDK = kBC * (D / 8) / 256;  // loads per tile and wave, for K and again for V
  static_assert(2 * NLDK == KT, "one load per score product pair");
  unsigned offk[NLDK];  // this lane's byte offset within a tile for each of its loads
#pragma unroll
  for (int i = 0; i < NLDK; ++i) {
    const int sl = (i * 4 + wave) * 64 + lane;
    const int r = sl / (D / 8);
    const int c = (sl % (D / 8)) ^ (swz<D>(r, 0) - r * (D / 8));
    offk[i] = (unsigned)((r * D + c * 8) * 2);
  }

  auto step = [&](auto stg_c, int k0) {
    constexpr unsigned KOFF = decltype(stg_c)::value * STAGE, VOFF = KOFF + TILE;
    // the next tile's K and V loads into the other stage, one per score product pair (a
    // tile past the last one reads past the buffers' range: zeros that no step reads)
    auto dma = [&](int t) {
      constexpr unsigned NS = KOFF ? 0 : 1;
      if (t < NLDK)
        lds_dma16(krs, lds[NS][0] + (t * 4 + wave) * 64 * 16, offk[t] + (unsigned)(k0 + kBC) * D * 2);
      else
        lds_dma16(vrs, lds[NS][1] + ((t - NLDK) * 4 + wave) * 64 * 16, offk[t - NLDK] + (unsigned)(k0 + kBC) * D * 2);
    };
    if (k0 >= khi_w) {  // no row of this wave sees the tile
#pragma unroll
      for (int t = 0; t < KT; ++t) dma(t);
      return;
    }
    f32x16 s0, s1, d0, d1;
    rows_product<D, KOFF>(la, qf, s0, s1, 0.f, dma);
    rows_product<D, VOFF>(la, dof, d0, d1, dd, [](int) {});  // dP^T - D: the products start at -D
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x16& s = kb ? s1 : s0;
      f32x16& dp = kb ? d1 : d0;  // dS replaces dP in place
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -l2)) * dp[r];
    }
    // masked pairs (keys past n_k, or past the row under the causal mask) get dS = 0,
    // selected over whatever the unmasked formula gave; only tiles that reach past n_k or
    // the diagonal (uniform per wave) take this branch
    if ((k0 + kBC > p.n_k) || (p.causal && k0 + kBC - 1 > q0w)) {
      // register r of block kb holds key k0 + 32kb + 8(r/4) + 4hf + r%4 of this lane's row
      const int hi = min(p.n_k - 1, p.causal ? row : p.n_k - 1) - k0 - 4 * hf;  // last visible offset
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 8 * (r >> 2) + (r & 3);
        d0[r] = c > hi ? 0.f : d0[r];
        d1[r] = c + 32 > hi ? 0.f : d1[r];
      }
    }
    bf16x8 db[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x16& dp = kb ? d1 : d0;
      db[2 * kb] = cvt_bf16x8(slice8(dp, 0));
      db[2 * kb + 1] = cvt_bf16x8(slice8(dp, 1));
    }
    // dQ^T += K^T dS^T: K^T read transposed from the K tile, keys in the order of db
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const unsigned roff = KOFF + (kb * 32 + 16 * t) * ROW;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const bf16x8 a = tr_pair(la.va[2 * nb] + roff, la.va[2 * nb + 1] + roff);
          dq[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, db[2 * kb + t], dq[nb], 0, 0, 0);
        }
      }
  };

  // two LDS stages, unrolled by two so that each stage's offsets are immediates; one
  // barrier per tile publishes it and retires the buffer read two tiles back
  if (n_tiles > 0) issue_kv<D>(krs, vrs, lds[0][0], lds[0][1], 0, wave, lane);
  for (int j = 0; j < n_tiles; j += 2) {
    const int k0 = j * kBC;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // (the step loads tile j + 1 into stage 1)
    step(std::integral_constant<unsigned, 0>{}, k0);
    if (j + 1 < n_tiles) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      // (the step loads tile j + 2 into stage 0)
      step(std::integral_constant<unsigned, 1>{}, k0 + kBC);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last step's loads land before the workgroup ends

  // dQ = scale * dQ^T^T, staged in the tiles' space once every wave is done with it
  static_assert(4 * kStagedRows<D> <= (int)sizeof(lds), "the staged rows fit");
  u32x2 out[NB][4];
  scaled_rows<D>(dq, p.scale, out);
  __syncthreads();
  write_rows<D>(out, (unsigned)(uintptr_t)(const lds_void*)&lds[0][0][0] + (unsigned)(wave * kStagedRows<D>),
                p.dq + (hq + q0w) * D, p.n_q - q0w, lane);
}

// ---------------------------------------------------------------------------
// dQ pass, ping-pong form: one workgroup of 8 waves per (batch, head, 256-row query
// block), waves w and w + 4 on one SIMD, group 0 (waves 0-3) one phase ahead of group 1,
// as in the ping-pong forward.  Per tile j and wave:
//   matrix phase:  dQ^T += K_{j-1}^T dS_{j-1}^T;  S_j^T = K_j Q^T;  dP_j^T = V_j dO^T
//   vector phase:  P_j = exp2(s * scale*log2e - LSE*log2e) (0 where masked), dS_j = P_j (dP_j - D),
//                  dP_j - D coming from products that start at -D
// so that on each SIMD one wave issues 48 products while its partner runs the vector
// work of the previous tile.  K and V each have a four-stage LDS ring (tile j in stage
// j % 4): the matrix phase reads K_{j-1}, K_j and V_j and issues the loads of K_{j+2}
// and V_{j+2} among its products; the wait at the end of iteration j + 1 retires them.
template <int D, unsigned KPREV, unsigned KCUR, unsigned VCUR, int PF, int NDMA, typename Dma>
__device__ __forceinline__ void dq_mat_stream(const LdsAddr<D>& la, unsigned vdelta, const bf16x8 (&qf)[D / 16],
                                              const bf16x8 (&dof)[D / 16], const bf16x8 (&db)[4], f32x16 (&dq)[D / 32],
                                              f32x16& s0, f32x16& s1, f32x16& d0, f32x16& d1, float nd, Dma&& dma) {
  constexpr int NB = D / 32;
  constexpr int KT = D / 16;
  constexpr unsigned ROW = D * 2;
  constexpr int NQ = 4 * NB;         // dQ products (kb, t, nb)
  constexpr int NS = 2 * KT;         // score products (t, block), then as many for dP
  constexpr int NM = NQ + 2 * NS;
  bf16x8 a[PF];
  auto load = [&](int m) {
    if (m < NQ) {
      const int kb = m / (2 * NB), t = (m / NB) % 2, nb = m % NB;
      const unsigned roff = KPREV + (kb * 32 + 16 * t) * ROW;
      a[m % PF] = tr_pair(la.va[2 * nb] + roff, la.va[2 * nb + 1] + roff);
    } else if (m < NQ + NS) {
      const int i = m - NQ;
      a[m % PF] = lds_load<bf16x8>(la.ka[i / 2] + KCUR + (i % 2) * 32 * ROW);
    } else {
      const int i = m - NQ - NS;
      a[m % PF] = lds_load<bf16x8>(la.ka[i / 2] + vdelta + VCUR + (i % 2) * 32 * ROW);
    }
  };
#pragma unroll
  for (int m = 0; m < PF; ++m) load(m);
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
  s0 = f32x16{};
  s1 = f32x16{};
  // dP^T accumulates on -D of this lane's row, so that the vector phase gets dP - D
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    d0[r] = nd;
    d1[r] = nd;
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    if (m < NQ) {
      const int kb = m / (2 * NB), t = (m / NB) % 2, nb = m % NB;
      dq[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % PF], db[2 * kb + t], dq[nb], 0, 0, 0);
    } else if (m < NQ + NS) {
      const int i = m - NQ, t = i / 2;
      if (i % 2 == 0)
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % PF], qf[t], s0, 0, 0, 0);
      else
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % PF], qf[t], s1, 0, 0, 0);
    } else {
      const int i = m - NQ - NS, t = i / 2;
      if (i % 2 == 0)
        d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % PF], dof[t], d0, 0, 0, 0);
      else
        d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % PF], dof[t], d1, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (m + PF < NQ) {
      load(m + PF);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    } else if (m + PF < NM) {
      load(m + PF);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < NDMA; ++i)
      if (m == i * NM / NDMA + 1) dma(i);
  }
}

template <int D>
__global__ void __launch_bounds__(512, 1) bwd_dq_pp_kernel(BwdParams p, float sl2, int sched) {
  constexpr int NW = 8;
  constexpr int BR = 32 * NW;
  constexpr int KT = D / 16;
  constexpr int NB = D / 32;
  constexpr int TILE = kBC * D * 2;
  constexpr int CPR = D / 8;
  constexpr int NLD = kBC * CPR / (64 * NW);  // loads per tile and wave, for K and again for V

  __shared__ __attribute__((aligned(1024))) char ldsk[4][TILE];
  __shared__ __attribute__((aligned(1024))) char ldsv[4][TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int hf = lane >> 5;
  const int col = lane & 31;

  const int n_qb = (p.n_q + BR - 1) / BR;
  int bh, qb;
  wg_coords(wg_logical(sched), n_qb, p.B * p.H, sched, p.causal != 0, bh, qb);
  const int q0 = qb * BR;
  const int q0w = q0 + 32 * wave;
  const int row = q0w + col;
  // keys seen by some row of the workgroup [0, khi), of this wave [0, khi_w)
  const int khi = p.causal ? min(p.n_k, q0 + BR) : p.n_k;
  const int khi_w = p.causal ? min(p.n_k, q0w + 32) : p.n_k;
  const int n_tiles = (khi + kBC - 1) / kBC;

  const long long hq = (long long)bh * p.n_q, hk = (long long)bh * p.n_k;
  const i32x4 krs = raw_rsrc(p.k + hk * D, (long long)khi * D * 2);
  const i32x4 vrs = raw_rsrc(p.v + hk * D, (long long)khi * D * 2);

  bf16x8 qf[KT], dof[KT];
  float l2 = 0.f, dd = 0.f;
  {
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q + hq * D, (long long)p.n_q * D * 2);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(p.dout + hq * D, (long long)p.n_q * D * 2);
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const unsigned off = ((unsigned)row * D + 16 * t + 8 * hf) * 2u;
      qf[t] = as_bf16x8(__builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0)));
      dof[t] = as_bf16x8(__builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(drs, off, 0, 0)));
    }
    // -D = -sum_c dO_c O_c of the row (its two halves in lanes c and c + 32) and LSE*log2e,
    // kept in registers and stored for the key pass
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(p.o + hq * D, (long long)p.n_q * D * 2);
    float dpart = 0.f;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const unsigned off = ((unsigned)row * D + 16 * t + 8 * hf) * 2u;
      const u32x4 ov = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ors, off, 0, 0));
      const u32x4 dv = __builtin_bit_cast(u32x4, dof[t]);
      const unsigned o0 = ov.x, o1 = ov.y, o2 = ov.z, o3 = ov.w, d0 = dv.x, d1 = dv.y, d2 = dv.z, d3 = dv.w;
      dpart = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d0), __builtin_bit_cast(bf16x2, o0), dpart, false);
      dpart = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d1), __builtin_bit_cast(bf16x2, o1), dpart, false);
      dpart = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d2), __builtin_bit_cast(bf16x2, o2), dpart, false);
      dpart = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d3), __builtin_bit_cast(bf16x2, o3), dpart, false);
    }
    const float dsum = dpart + __shfl_xor(dpart, 32);
    if (row < p.n_q) {
      l2 = p.lse[hq + row] * kLog2e;
      dd = -dsum;
      if (hf == 0) {
        p.dvec[hq + row] = dd;
        p.l2vec[hq + row] = l2;
      }
    }
  }
  f32x16 dq[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) dq[nb] = f32x16{};

  LdsAddr<D> la;  // K rows and K^T over the K ring; V rows at the same places of the V ring
  make_lds_addr<D>(la, (unsigned)(uintptr_t)(const lds_void*)&ldsk[0][0], lane);
  const unsigned vdelta = (unsigned)(uintptr_t)(const lds_void*)&ldsv[0][0] -
                          (unsigned)(uintptr_t)(const lds_void*)&ldsk[0][0];
  unsigned offp[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int sl = (i * NW + wave) * 64 + lane;
    const int r = sl / CPR;
    const int c = (sl % CPR) ^ (swz<D>(r, 0) - r * CPR);
    offp[i] = (unsigned)((r * D + c * 8) * 2);
  }
  // part i of iteration j's loads: K_{j+2} then V_{j+2}, into stage (j + 2) % 4
  auto dma = [&](int j, auto ks, int i) {
    constexpr unsigned S2 = (decltype(ks)::value + 2) % 4;
    const unsigned toff = (unsigned)((j + 2) * kBC) * D * 2;
    if (i < NLD)
      lds_dma16(krs, &ldsk[S2][(i * NW + wave) * 64 * 16], offp[i] + toff);
    else
      lds_dma16(vrs, &ldsv[S2][((i - NLD) * NW + wave) * 64 * 16], offp[i - NLD] + toff);
  };

  f32x16 s0 = {}, s1 = {}, d0 = {}, d1 = {};
  bf16x8 db[4] = {};
  // the first matrix phase multiplies dS = 0 with K stage 3, which no load has written
  // yet: zero it (published by the barrier before the loop)
  {
    constexpr int PER = TILE / (64 * NW);
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < PER / 16; ++i)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
          (uintptr_t)(const lds_void*)&ldsk[3][(tid * (PER / 16) + i) * 16]) = z;
  }

  auto act = [&](int j) { return j >= 0 && j < n_tiles && j * kBC < khi_w; };
  auto mat = [&](int j, auto ks) {
    constexpr unsigned KS = decltype(ks)::value;
    __builtin_amdgcn_s_setprio(1);
    if (act(j - 1) || act(j)) {
      dq_mat_stream<D, ((KS + 3) % 4) * TILE, KS * TILE, KS * TILE, 4, 2 * NLD>(
          la, vdelta, qf, dof, db, dq, s0, s1, d0, d1, dd, [&](int i) { dma(j, ks, i); });
    } else {
#pragma unroll
      for (int i = 0; i < 2 * NLD; ++i) dma(j, ks, i);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto vec = [&](int j) {
    if (!act(j)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) db[i] = bf16x8{};
      return;
    }
    const int k0 = j * kBC;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x16& s = kb ? s1 : s0;
      f32x16& dp = kb ? d1 : d0;  // dS replaces dP in place
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -l2)) * dp[r];
    }
    // masked pairs (keys past n_k, or past the row under the causal mask) get dS = 0,
    // selected over whatever the unmasked formula gave; only tiles that reach past n_k or
    // the diagonal (uniform per wave) take this branch
    if ((k0 + kBC > p.n_k) || (p.causal && k0 + kBC - 1 > q0w)) {
      // register r of block kb holds key k0 + 32kb + 8(r/4) + 4hf + r%4 of this lane's row
      const int hi = min(p.n_k - 1, p.causal ? row : p.n_k - 1) - k0 - 4 * hf;  // last visible offset
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 8 * (r >> 2) + (r & 3);
        d0[r] = c > hi ? 0.f : d0[r];
        d1[r] = c + 32 > hi ? 0.f : d1[r];
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x16& dp = kb ? d1 : d0;
      db[2 * kb] = cvt_bf16x8(slice8(dp, 0));
      db[2 * kb + 1] = cvt_bf16x8(slice8(dp, 1));
    }
  };
  auto wait_prev = [&]() {
    if constexpr (NLD == 2)
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  };
  auto iter0 = [&](int j, auto ks) {
    mat(j, ks);
    __syncthreads();
    vec(j);
    wait_prev();
    __syncthreads();
  };
  auto iter1 = [&](int j, auto ks) {
    vec(j - 1);
    __syncthreads();
    mat(j, ks);
    wait_prev();
    __syncthreads();
  };

  // K_0, K_1, V_0, V_1 before the loop
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int sl = (i * NW + wave) * 64 * 16;
    lds_dma16(krs, &ldsk[0][sl], offp[i]);
    lds_dma16(krs, &ldsk[1][sl], offp[i] + (unsigned)kBC * D * 2);
    lds_dma16(vrs, &ldsv[0][sl], offp[i]);
    lds_dma16(vrs, &ldsv[1][sl], offp[i] + (unsigned)kBC * D * 2);
  }
  // vmcnt(0) through the builtin, which the compiler's own wait tracking sees: the Q and
  // dO fragments have then arrived, and it adds no waits of its own inside the loop
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if (grp == 0) {
    for (int j = 0; j <= n_tiles; j += 4) {
      iter0(j, std::integral_constant<unsigned, 0>{});
      if (j + 1 <= n_tiles) iter0(j + 1, std::integral_constant<unsigned, 1>{});
      if (j + 2 <= n_tiles) iter0(j + 2, std::integral_constant<unsigned, 2>{});
      if (j + 3 <= n_tiles) iter0(j + 3, std::integral_constant<unsigned, 3>{});
    }
  } else {
    for (int j = 0; j <= n_tiles; j += 4) {
      iter1(j, std::integral_constant<unsigned, 0>{});
      if (j + 1 <= n_tiles) iter1(j + 1, std::integral_constant<unsigned, 1>{});
      if (j + 2 <= n_tiles) iter1(j + 2, std::integral_constant<unsigned, 2>{});
      if (j + 3 <= n_tiles) iter1(j + 3, std::integral_constant<unsigned, 3>{});
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last loads land before the workgroup ends

  // dQ staged in the K rings (waves 0-3) and the V rings (waves 4-7) once every wave is done
  static_assert(4 * kStagedRows<D> <= (int)sizeof(ldsk), "the staged rows fit");
  u32x2 out[NB][4];
  scaled_rows<D>(dq, p.scale, out);
  __syncthreads();
  const unsigned stage = (unsigned)(uintptr_t)(const lds_void*)(wave < 4 ? &ldsk[0][0] : &ldsv[0][0]) +
                         (unsigned)((wave & 3) * kStagedRows<D>);
  write_rows<D>(out, stage, p.dq + (hq + q0w) * D, p.n_q - q0w, lane);
}

}  // namespace

// the dQ pass takes the ping-pong kernel from this many query rows (d = 128); under the causal
// mask its 256-row workgroups split the triangle too coarsely below 4096 rows
constexpr int kDqPingPongMinRows = 2048;
constexpr int kDqPingPongMinRowsCausal = 4096;

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  const float sl2 = p.scale * kLog2e;
  const unsigned g1 = (unsigned)((long long)p.B * p.H * ((p.n_k + kBK - 1) / kBK));
  const unsigned g2 = (unsigned)((long long)p.B * p.H * ((p.n_q + 127) / 128));
  // both passes take the forward's workgroup orders: block-major without the renumbering under
  // the causal mask, the heaviest blocks of every head first; renumbered head-major otherwise
  const int sched = p.causal ? kSchedQbMajor : kSchedRemap;
  const unsigned g3 = (unsigned)((long long)p.B * p.H * ((p.n_q + 255) / 256));
  const bool pp = p.d == 128 && p.n_q >= (p.causal ? kDqPingPongMinRowsCausal : kDqPingPongMinRows);
  // the dQ pass first: it forms -D and LSE*log2e of its rows and stores them for the key pass
  if (p.d == 128) {
    if (pp)
      hipLaunchKernelGGL(bwd_dq_pp_kernel<128>, dim3(g3), dim3(512), 0, stream, p, sl2, sched);
    else
      hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3(g2), dim3(256), 0, stream, p, sl2, sched);
    hipLaunchKernelGGL(bwd_kv_pp_kernel<128>, dim3(g1), dim3(512), 0, stream, p, sl2, sched);
  } else {
    if (pp)
      hipLaunchKernelGGL(bwd_dq_pp_kernel<64>, dim3(g3), dim3(512), 0, stream, p, sl2, sched);
    else
      hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3(g2), dim3(256), 0, stream, p, sl2, sched);
    hipLaunchKernelGGL(bwd_kv_pp_kernel<64>, dim3(g1), dim3(512), 0, stream, p, sl2, sched);
  }
  return hipGetLastError();
}

}  // namespace fa2
