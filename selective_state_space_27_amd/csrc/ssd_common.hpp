// Device helpers shared by the SSD forward and backward kernels (gfx950):
// the 32x32x16 bf16 matrix-core product and its register layouts, bf16 hi/lo
// splitting of fp32 operands, the time-contiguous LDS staging layout, a
// fixed-order wave prefix sum and 32x32 state-tile loads and stores.
#pragma once

#include "common.hpp"

namespace mss {
namespace ssd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kP = 64;      // headdim
constexpr int kN = 128;     // dstate
constexpr int kSub = 64;    // steps per block
constexpr int kPadH = 8;    // bf16 row padding (16 bytes)
constexpr int kTRow = kSub + kPadH;  // row length of the time-contiguous (transposed) stagings

// Element (row, step j) of a time-contiguous staging [rows][kTRow]: the eight
// 16-byte blocks of a row are permuted by (row >> 4) so that the staging
// writes (two steps of many rows per instruction) spread over all LDS banks,
// while a 16-byte operand read (8 consecutive steps of one row) stays whole.
__device__ __forceinline__ int tsw(int row, int j) {
  return row * kTRow + ((((j >> 3) ^ (row >> 4)) & 7) << 3) + (j & 7);
}

// D += A B with A 32x16 (lane l: row l%32, k = 8(l/32)+t), B 16x32 (lane l:
// k = 8(l/32)+t, column l%32), t the bf16 index in the 8-vector.
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Row (within a 32x32 tile) of accumulator register r of lane l; the column is l%32.
__device__ __forceinline__ int acc_row(int r, int l) { return 8 * (r >> 2) + 4 * (l >> 5) + (r & 3); }

// Rows 16S..16S+15 of an accumulator tile in operand form: lane l gets rows
// 16S + 8(l/32) + t, t = 0..7, of column l%32.  Registers 8S+q hold rows
// 16S+q (lanes 0-31) and 16S+4+q (lanes 32-63), registers 8S+4+q rows 16S+8+q
// and 16S+12+q; swapping the upper half of the first with the lower half of
// the second puts every row where the operand layout wants it.
template <int S>
__device__ __forceinline__ void acc_kslice(const f32x16& acc, float* v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[8 * S + q]),
                                                    __float_as_uint(acc[8 * S + 4 + q]), false, false);
    v[q] = __uint_as_float(r[0]);
    v[4 + q] = __uint_as_float(r[1]);
  }
}

// fp32 pair -> (hi, lo) bf16 pairs with hi + lo = value to ~16 mantissa bits.
// The residuals value - hi come from v_dot2_f32_bf16 of the packed hi pair
// with (-1, 0) or (0, -1), plus the value: one instruction each instead of
// unpacking hi and subtracting, and exact (the products are exact and the
// residual of a round-to-nearest is representable).  The two masks live in
// registers: folded into an inline constant, (-1, 0) is read as (0, -1).
struct Dot2Masks {
  bf16x2_t lo, hi;
};
__device__ __forceinline__ Dot2Masks dot2_masks() {
  uint32_t lo = 0x0000bf80u, hi = 0xbf800000u;
  asm volatile("" : "+v"(lo));
  asm volatile("" : "+v"(hi));
  return {__builtin_bit_cast(bf16x2_t, lo), __builtin_bit_cast(bf16x2_t, hi)};
}
__device__ __forceinline__ float dot2_bf16(uint32_t h, bf16x2_t m, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, h), m, c, false);
}
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo, const Dot2Masks& m) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(dot2_bf16(hi, m.lo, a), dot2_bf16(hi, m.hi, b));
}
__device__ __forceinline__ void split8(const float* v, u32x4& hi, u32x4& lo, const Dot2Masks& m) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t h, l;
    split2(v[2 * q], v[2 * q + 1], h, l, m);
    hi[q] = h;
    lo[q] = l;
  }
}

// x plus lane (lane - S) of its 16-lane row (0 for the first S lanes of a row).
template <int S>
__device__ __forceinline__ float add_row_shr(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + S, 0xf, 0xf,
                                                                   false));
}

// Inclusive prefix sum over the 64 lanes of a wave in a fixed order: scans
// inside each 16-lane row (DPP row_shr 1, 2, 4, 8), then row 0's total is
// added to row 1 and row 2's to row 3 (row_bcast:15), then the total of rows
// 0-1 to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x = add_row_shr<1>(x);
  x = add_row_shr<2>(x);
  x = add_row_shr<4>(x);
  x = add_row_shr<8>(x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xa, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xc, 0xf, false));
  return x;
}


// One 32x32 tile of S^T (rows n = nt*32.., columns p = pt*32..) from a
// state whose row p starts at S + p*ld (columns n < nmax valid, the rest
// zero; nmax a multiple of 16): each lane moves 4 consecutive n of its column.
__device__ __forceinline__ void load_stateT(f32x16& acc, const float* S, int nt, int pt, int ld = kN,
                                            int nmax = kN) {
  const int lane = threadIdx.x & 63;
  const int p = pt * 32 + (lane & 31);
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    const int n = nt * 32 + 8 * g4 + 4 * (lane >> 5);
    const f32x4 v = (S && n < nmax) ? *reinterpret_cast<const f32x4*>(&S[(size_t)p * ld + n])
                                    : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[4 * g4 + q] = v[q];
  }
}

// The inverse: a 32x32 tile of S^T written back (columns n < nmax only).
__device__ __forceinline__ void store_stateT(const f32x16& acc, float* S, int nt, int pt, int ld = kN,
                                             int nmax = kN) {
  const int lane = threadIdx.x & 63;
  const int p = pt * 32 + (lane & 31);
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    const int n = nt * 32 + 8 * g4 + 4 * (lane >> 5);
    if (n < nmax)
      *reinterpret_cast<f32x4*>(&S[(size_t)p * ld + n]) =
          f32x4{acc[4 * g4], acc[4 * g4 + 1], acc[4 * g4 + 2], acc[4 * g4 + 3]};
  }
}

// The same state as an S tile: headdim rows p = pt*32 + 8(r >> 2) + 4hf +
// (r & 3) in register r, states n = nt*32 + lane % 32 in the lanes (the
// accumulator layout of a product with the headdim rows as its A operand).
// A register is one row segment of 32 states: whole 128-byte lines.
__device__ __forceinline__ void load_stateS(f32x16& acc, const float* S, int nt, int pt, int ld = kN,
                                            int nmax = kN) {
  const int lane = threadIdx.x & 63;
  const int n = nt * 32 + (lane & 31), p0 = pt * 32 + 4 * (lane >> 5);
#pragma unroll
  for (int r = 0; r < 16; ++r)
    acc[r] = (S && n < nmax) ? S[(size_t)(p0 + 8 * (r >> 2) + (r & 3)) * ld + n] : 0.f;
}

__device__ __forceinline__ void store_stateS(const f32x16& acc, float* S, int nt, int pt, int ld = kN,
                                             int nmax = kN) {
  const int lane = threadIdx.x & 63;
  const int n = nt * 32 + (lane & 31), p0 = pt * 32 + 4 * (lane >> 5);
  if (n < nmax) {
#pragma unroll
    for (int r = 0; r < 16; ++r) S[(size_t)(p0 + 8 * (r >> 2) + (r & 3)) * ld + n] = acc[r];
  }
}

}  // namespace ssd
}  // namespace mss
