// Device helpers shared by the forward and backward kernels: vector types,
// the LDS tile swizzle, the XCD-aware workgroup renumbering, buffer
// descriptors and the buffer->LDS load.  Internal; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa2_internal.h"

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

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ---------------------------------------------------------------------------
// LDS tile layout.  A tile is a block of rows of D bf16, stored as 16-byte
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

// (batch*head, query block) of logical workgroup L among n_qb query blocks per head
// and n_bh heads; heavy_first reverses the block order (the heaviest block of a
// causal-like band is the last one).
__device__ __forceinline__ void wg_coords(int L, int n_qb, int n_bh, int sched, bool heavy_first, int& bh,
                                          int& qb) {
  if (sched & kSchedQbMajor) {
    qb = L / n_bh;
    bh = L % n_bh;
  } else {
    bh = L / n_qb;
    qb = L % n_qb;
  }
  if (heavy_first) qb = n_qb - 1 - qb;
}

__device__ __forceinline__ int wg_logical(int sched) {
  return (sched & kSchedRemap) ? xcd_remap(blockIdx.x, gridDim.x) : (int)blockIdx.x;
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

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (stride 0) over [base, base + bytes): loads whose
// per-lane offset lies at or beyond `bytes` return zero.
__device__ __forceinline__ i32x4 raw_rsrc(const void* base, long long bytes) {
  const unsigned long long a = (unsigned long long)base;
  return i32x4{(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// 16 bytes per lane from buffer `rs` at byte offset voff into LDS at
// dst + 16*lane (buffer_load_dwordx4 ... lds; M0 holds the LDS base and is
// restored afterwards).  Issued through asm so that the compiler does not
// order later LDS reads of the other stage behind it; the kernel waits for
// these loads itself (s_waitcnt vmcnt(0) before the barrier that publishes a
// tile).
//
// Built with FA2_POISON_LDS (the race-check build), each lane first fills its
// 16 destination bytes with 0x7fff7fff, a NaN as bf16, fp32 and e4m3 alike, and
// waits for that store.  A read of the slot that is not ordered after the load's
// wait and barrier then sees NaN (or the load's data where an overwrite races a
// reader), so a missing wait or barrier shows up as NaN or as a changed result.
__device__ __forceinline__ void lds_dma16(i32x4 rs, const char* dst, unsigned voff) {
  const unsigned m0v = (unsigned)(uintptr_t)(const lds_void*)dst;
#ifdef FA2_POISON_LDS
  *reinterpret_cast<__attribute__((address_space(3))) u32x4*>((uintptr_t)(m0v + 16u * (threadIdx.x & 63u))) =
      u32x4{0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu};
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#endif
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0v), "v"(voff), "s"(rs)
      : "memory");
}

template <typename T>
__device__ __forceinline__ T lds_load(unsigned addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>((uintptr_t)addr);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// LDS byte addresses a lane reads from, computed once per kernel.  With the
// XOR swizzle the address of (row, chunk) is not affine in the chunk, so each
// lane keeps one register per distinct pattern and every other index (key
// block, k-step, stage) becomes an immediate offset:
//   ka[t]       K operand: key row col, chunk 2t + hf            (+ kb*32 rows)
//   va[2nb + h] V^T operand: rows 4hf + j16/4 + 8h, d 32nb + 16cg + 4(j16%4)
//               (+ kb*32 + 16t rows).  The swizzle repeats every 16 rows, so
//               whole 16-row steps are plain offsets.
template <int D>
struct LdsAddr {
  unsigned ka[D / 16];
  unsigned va[D / 16];
};

template <int D>
__device__ __forceinline__ void make_lds_addr(LdsAddr<D>& a, unsigned base, int lane) {
  const int hf = lane >> 5, col = lane & 31;
  const int j16 = lane & 15, cg = (lane >> 4) & 1;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) a.ka[t] = base + swz<D>(col, 2 * t + hf) * 16;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kr = 4 * hf + (j16 >> 2) + 8 * h;
      const int dd = 32 * nb + 16 * cg + 4 * (j16 & 3);
      a.va[2 * nb + h] = base + swz<D>(kr, dd >> 3) * 16 + (dd & 7) * 2;
    }
  // opaque to the optimiser: keep these in registers instead of recomputing them per tile
#pragma unroll
  for (int i = 0; i < D / 16; ++i) asm volatile("" : "+v"(a.ka[i]), "+v"(a.va[i]));
}

// ---------------------------------------------------------------------------
// Output rows.  The kernels hold a wave's 32 output rows transposed: lane column c owns row c,
// and register 4q + e of 32-column block nb is element 32 nb + 8 q + 4 hf + e of it (hf the
// lane half).  Written straight out, every store would cover 16 bytes of 32 rows.  write_rows
// stages the rows in LDS instead (row-major, 2D bytes per row, the 16-byte chunks of row r
// placed at chunk index c ^ (r mod 16) so that the 32 rows written by one instruction spread
// over the banks) and reads them back so that each store writes whole rows, 16 bytes per lane.
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <int D>
constexpr int kStagedRows = 32 * D * 2;  // LDS bytes write_rows takes per wave

// out[nb][q] = bf16(acc[nb][4q .. 4q + 3] * sc), round to nearest even
template <int D>
__device__ __forceinline__ void scaled_rows(const f32x16 (&acc)[D / 32], float sc, u32x2 (&out)[D / 32][4]) {
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = {acc[nb][4 * q] * sc, acc[nb][4 * q + 1] * sc, acc[nb][4 * q + 2] * sc, acc[nb][4 * q + 3] * sc};
      out[nb][q] = __builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4));
    }
}

// Row r (r < 32) goes to dst + r * D when r < n_valid.  `stage`: kStagedRows<D> bytes of LDS
// that no other wave touches until this call returns.
template <int D>
__device__ __forceinline__ void write_rows(const u32x2 (&out)[D / 32][4], unsigned stage, uint16_t* dst, int n_valid,
                                           int lane) {
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  constexpr int ROW = D * 2;
  constexpr int LPR = ROW / 16;  // 16-byte chunks per row = lanes per row in the write-out
  constexpr int RPI = 64 / LPR;  // rows per store
  const int col = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = (4 * nb + q) ^ (col & 15 & (LPR - 1));
      *reinterpret_cast<lds_u32x2*>((uintptr_t)(stage + (unsigned)(col * ROW + c * 16 + hf * 8))) = out[nb][q];
    }
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / LPR, c = lane % LPR;
    const u32x4 v =
        *reinterpret_cast<const lds_u32x4*>((uintptr_t)(stage + (unsigned)(r * ROW + (c ^ (r & 15 & (LPR - 1))) * 16)));
    if (r < n_valid) *reinterpret_cast<u32x4*>(dst + (long long)r * D + c * 8) = v;
  }
}

}  // namespace
}  // namespace fa2
