// Device helpers shared by the libmambascan kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mss {

constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Loads through the constant address space: with a wave-uniform address the
// compiler emits scalar (s_load) reads, so per-timestep values shared by all
// lanes (B and C rows) arrive in SGPRs without touching the vector memory path.
typedef const __attribute__((address_space(4))) float* cfloat_ptr;
__device__ __forceinline__ cfloat_ptr as_const(const float* p) { return (cfloat_ptr)(p); }

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
