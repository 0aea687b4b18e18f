// Device helpers shared by the libmambascan kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mss {

constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Exact widening of bf16 (stored in the low/high half of a 32-bit word).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Hardware base-2 exponential (v_exp_f32) and reciprocal (v_rcp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// silu(z) = z / (1 + exp(-z)); the limits z -> -inf (exp overflows to inf,
// rcp gives 0) and z -> +inf come out right without branches.
__device__ __forceinline__ float silu(float z) { return z * rcp_fast(1.0f + exp2_fast(-z * kLog2e)); }

}  // namespace mss

namespace mss {

// Raw buffer descriptors: an access whose byte offset is at or beyond
// `bytes` reads 0 and a store there is dropped, so tails and inactive lanes
// need no branches (branch-free loads keep the in-order vmcnt bookkeeping
// precise, which lets loads issued several tiles ahead stay in flight).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;
// An offset at or past the end of every descriptor used here: the host checks
// keep each descriptor at most 2^32 - 256 bytes long (a 64-channel block of
// fp32 scan rows reaches exactly that at seqlen 2^24 - 1), and the largest
// access (16 bytes) from this offset does not wrap 32 bits.
constexpr uint32_t kOffNone = 0xFFFFFF00u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ uint32_t buf_load_u32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint16_t buf_load_u16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 buf_load_u32x2(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x4 buf_load_u32x4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store_u32(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store_u16(rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store_u32x2(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store_u32x4(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

// Broadcast lane P of each row of 16 lanes to the whole row (DPP row_newbcast).
// Used as the first operand of a multiply, the move folds into v_mul_f32_dpp.
// Every lane has a valid source, so bound_ctrl is set: the move then needs no
// zeroed destination register when it cannot be folded.
template <int P>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + P, 0xf, 0xf, true));
}


// acc + (lane P of each 16-lane row of v, broadcast) * h as one
// v_fmac_f32_dpp, which the compiler does not form from a DPP move and a
// multiply-add.  The broadcast operand v must not have been written by a VALU
// instruction in the two wait states before (the compiler inserts none around
// inline assembly); the build checks the disassembly of every kernel for it.
template <int P>
__device__ __forceinline__ float fmac_row_bcast(float acc, float v, float h) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "+v"(acc)
      : "v"(v), "v"(h), "i"(P));
  return acc;
}

}  // namespace mss
