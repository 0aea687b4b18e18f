// Layouts and row helpers shared by the selective scan's forward
// (scan.hip) and backward (scan_bwd.hip) kernels: the 8-way split of the
// d_state states over waves, 16-step tiles, the fp32 B/C workspace written by
// bc_transpose_kernel, DPP row broadcasts of B/C values, and branch-free loads
// and stores of four consecutive steps of one [b, d, L] row.
#pragma once

#include "common.hpp"

namespace mss {
namespace {

constexpr int kWaves = 8;          // waves the d_state states are split across
constexpr int kLanes = 64;         // channels per block (one per lane)
constexpr int kTile = 16;          // time steps per tile
constexpr int kBlk = kTile / 4;    // float4 blocks per tile

// B/C values a wave needs per 4-step block: 4 steps x (SPW B values, SPW C
// values) = 8*SPW, spread over NV VGPRs of 16 row positions each.
template <int SPW>
struct BCShape {
  static constexpr int kPerBlk = 8 * SPW;
  static constexpr int kNV = kPerBlk <= 16 ? 1 : kPerBlk / 16;
  static constexpr int kPerTile = kNV * 16 * kBlk;  // floats per (batch, wave, tile)
  static constexpr bool kBlockLayout = kNV >= 8;    // see bc_index
};

// Workspace B/C layout, per [batch][wave g][tile]: value i = v*16 + p of
// block blk (step i / (2*SPW), quantity i % (2*SPW): B of states g*SPW..,
// then C) belongs to row position p, and
//   tile layout  [v][p][blk]:        lane p loads the float4 over blk, so the
//                                    value sits in component blk of VGPR v;
//   block layout [blk][v/4][p][v%4]: lane p loads, per block, the float4 over
//                                    v%4, so it sits in component v%4 of
//                                    VGPR v/4 of that block's load.
template <int SPW>
__device__ __forceinline__ size_t bc_index(int b, int g, int tile, int ntiles, int v, int p, int blk) {
  using S = BCShape<SPW>;
  return ((((size_t)b * kWaves + g) * ntiles + tile) * S::kNV + v) * 64 + p * 4 + blk;
}

__device__ __forceinline__ float fmac_row_bcast_rt(float acc, float v, float h, int p) {
  switch (p) {
    case 0: return fmac_row_bcast<0>(acc, v, h);
    case 1: return fmac_row_bcast<1>(acc, v, h);
    case 2: return fmac_row_bcast<2>(acc, v, h);
    case 3: return fmac_row_bcast<3>(acc, v, h);
    case 4: return fmac_row_bcast<4>(acc, v, h);
    case 5: return fmac_row_bcast<5>(acc, v, h);
    case 6: return fmac_row_bcast<6>(acc, v, h);
    case 7: return fmac_row_bcast<7>(acc, v, h);
    case 8: return fmac_row_bcast<8>(acc, v, h);
    case 9: return fmac_row_bcast<9>(acc, v, h);
    case 10: return fmac_row_bcast<10>(acc, v, h);
    case 11: return fmac_row_bcast<11>(acc, v, h);
    case 12: return fmac_row_bcast<12>(acc, v, h);
    case 13: return fmac_row_bcast<13>(acc, v, h);
    case 14: return fmac_row_bcast<14>(acc, v, h);
    default: return fmac_row_bcast<15>(acc, v, h);
  }
}

__device__ __forceinline__ float row_bcast_rt(float v, int p) {
  switch (p) {
    case 0: return row_bcast<0>(v);
    case 1: return row_bcast<1>(v);
    case 2: return row_bcast<2>(v);
    case 3: return row_bcast<3>(v);
    case 4: return row_bcast<4>(v);
    case 5: return row_bcast<5>(v);
    case 6: return row_bcast<6>(v);
    case 7: return row_bcast<7>(v);
    case 8: return row_bcast<8>(v);
    case 9: return row_bcast<9>(v);
    case 10: return row_bcast<10>(v);
    case 11: return row_bcast<11>(v);
    case 12: return row_bcast<12>(v);
    case 13: return row_bcast<13>(v);
    case 14: return row_bcast<14>(v);
    default: return row_bcast<15>(v);
  }
}

// Raw (undecoded) words of four consecutive steps of one row.
template <bool BF16>
struct Raw4;
template <>
struct Raw4<true> {
  u32x2 w;
};
template <>
struct Raw4<false> {
  u32x4 w;
};

// Branch-free load of steps t..t+3 of this lane's row; out-of-range steps read 0.
template <bool BF16, bool VEC>
__device__ __forceinline__ Raw4<BF16> load_raw4(rsrc_t r, uint32_t lane_off, int t, int L, bool ok) {
  constexpr uint32_t es = BF16 ? 2 : 4;
  Raw4<BF16> res;
  if constexpr (VEC) {  // L % 4 == 0: the four steps are all in range or all out
    const uint32_t o = (ok && t < L) ? lane_off + (uint32_t)t * es : kOffNone;
    if constexpr (BF16) res.w = buf_load_u32x2(r, o);
    else res.w = buf_load_u32x4(r, o);
  } else {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (ok && t + i < L) ? lane_off + (uint32_t)(t + i) * es : kOffNone;
    if constexpr (BF16) {
      res.w.x = (uint32_t)buf_load_u16(r, o[0]) | ((uint32_t)buf_load_u16(r, o[1]) << 16);
      res.w.y = (uint32_t)buf_load_u16(r, o[2]) | ((uint32_t)buf_load_u16(r, o[3]) << 16);
    } else {
      res.w.x = buf_load_u32(r, o[0]);
      res.w.y = buf_load_u32(r, o[1]);
      res.w.z = buf_load_u32(r, o[2]);
      res.w.w = buf_load_u32(r, o[3]);
    }
  }
  return res;
}

__device__ __forceinline__ f32x4 decode4(const Raw4<true>& r) {
  return f32x4{bf16_lo(r.w.x), bf16_hi(r.w.x), bf16_lo(r.w.y), bf16_hi(r.w.y)};
}
__device__ __forceinline__ f32x4 decode4(const Raw4<false>& r) { return __builtin_bit_cast(f32x4, r.w); }

template <bool BF16, bool VEC>
__device__ __forceinline__ void store4(rsrc_t r, uint32_t lane_off, int t, int L, bool ok, f32x4 v) {
  constexpr uint32_t es = BF16 ? 2 : 4;
  if constexpr (VEC) {
    const uint32_t o = (ok && t < L) ? lane_off + (uint32_t)t * es : kOffNone;
    if constexpr (BF16) {
      buf_store_u32x2(r, o, u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)});
    } else {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)o, 0, 0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t o = (ok && t + i < L) ? lane_off + (uint32_t)(t + i) * es : kOffNone;
      if constexpr (BF16) buf_store_u16(r, o, f32_to_bf16(v[i]));
      else buf_store_u32(r, o, __float_as_uint(v[i]));
    }
  }
}

// The forward's workspace opens with its flags block: [0] the call's status
// word (nonzero when a bounded wait between workgroups gave up), [1] the
// ticket, [2 ..) the carry flags of up to kMaxScanWG workgroups; the fp32 B/C
// arrangement follows.
constexpr int kMaxScanWG = 512;
inline size_t align256(size_t x);
inline size_t scan_flags_bytes() { return align256((size_t)(kMaxScanWG + 2) * sizeof(int)); }

inline int states_per_wave(int64_t N) { return N <= 8 ? 1 : N <= 16 ? 2 : N <= 32 ? 4 : N <= 64 ? 8 : 16; }
inline int64_t num_tiles(int64_t L) { return (L + kTile - 1) / kTile; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t bc_floats(int spw, int64_t batch, int64_t L) {
  const int per_tile = spw == 1 ? BCShape<1>::kPerTile : spw == 2 ? BCShape<2>::kPerTile
                     : spw == 4 ? BCShape<4>::kPerTile : spw == 8 ? BCShape<8>::kPerTile
                     : BCShape<16>::kPerTile;
  return (size_t)batch * kWaves * num_tiles(L) * per_tile;
}

}  // namespace
}  // namespace mss
