// Mamba-3 state update (one generation step) for gfx950.
//
// What is computed (see include/mambascan.h): the Mamba-2 head structure (one
// decay exp(delta*A_h) per head, heads of a group sharing B and C) with the
// three changes "Mamba-1/2/3 visual guide" section 4 gives Mamba-3's
// recurrence: an exponential-trapezoidal input rule (the step's input taken
// at both of its ends), a complex state that rotates while it decays
// (angle delta*theta_n per state), and MIMO (R input vectors and R B/C pairs
// per head: a rank-R update and R outputs).  Per (b, head h, row p, state n):
//   alpha = exp(delta A_h) [* e^{i delta theta[h,n]}]
//   u     = sum_r x[r,p] B[r,n];   u' = sum_r x_prev[r,p] B_prev[r,n]
//   h    <- alpha h + (delta/2)(alpha u' + u)    (trapezoid; else + delta u)
//   y[r,p] = (sum_n C[r,n] Re h[p,n] + D_h x[r,p]) * silu(z[r,p])
//
// Decode streams the state once (read, update, write), so the layout is the
// state update's: a workgroup takes 16 consecutive rows of one head, 16 lanes
// per row, each lane a contiguous slice of SPL states (2*SPL floats when
// complex), so a wave touches 4 whole rows.  Everything a row shares with the
// other rows of its head is formed once per workgroup into LDS: the rotation
// (cos, sin)(delta theta_n) of every state, B, C and B_prev of every rank.
// The R readouts of a row are summed over its 16 lanes in a fixed butterfly
// (bitwise deterministic).  Rank R raises the work per state byte R-fold
// (2R multiply-adds per state for the update and the readout) at the same
// state traffic: the point of MIMO for decode.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace mss {
namespace {

constexpr int kM3Threads = 256;
constexpr int kM3LanesPerRow = 16;
constexpr int kM3Rows = kM3Threads / kM3LanesPerRow;  // rows per workgroup
constexpr int kM3MaxR = 8;
constexpr int kM3MaxN = 256;

template <bool BF16>
__device__ __forceinline__ float ld_io(const void* p, size_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

// RPT rows per thread (2 when headdim is a multiple of 32: rows `row` and
// `row + 16` of a 32-row workgroup), so that each wave keeps twice the state
// bytes in flight; the per-state values staged in LDS serve both rows.
template <int SPL, int RPT, bool CPLX, bool TRAP, bool BF16>
__global__ void __launch_bounds__(kM3Threads) mamba3_step_kernel(Mamba3Params a) {
  constexpr int F = CPLX ? 2 * SPL : SPL;  // floats of state per lane and row
  constexpr int kRowsWG = kM3Rows * RPT;
  __shared__ __attribute__((aligned(16))) float s_cs[kM3MaxN][2];  // (cos, sin)(delta theta_n)
  __shared__ __attribute__((aligned(16))) float s_B[kM3MaxR][kM3MaxN];
  __shared__ __attribute__((aligned(16))) float s_C[kM3MaxR][kM3MaxN];
  __shared__ __attribute__((aligned(16))) float s_Bp[TRAP ? kM3MaxR : 1][TRAP ? kM3MaxN : 1];
  __shared__ float s_x[kM3MaxR][kRowsWG], s_xp[TRAP ? kM3MaxR : 1][kRowsWG];

  const int H = (int)a.nheads, P = (int)a.headdim, N = (int)a.dstate, R = (int)a.rank;
  const int hd = blockIdx.y, b = blockIdx.z;
  const int g = hd / (H / (int)a.ngroups);
  const int p0 = blockIdx.x * kRowsWG;
  const int row = threadIdx.x / kM3LanesPerRow, q = threadIdx.x % kM3LanesPerRow;
  const int n0 = q * SPL;
  const size_t bh = (size_t)b * H + hd;
  const size_t bg = (size_t)b * a.ngroups + g;
  const float dl = a.delta[bh];
  const float dec = exp2_fast(dl * a.A[hd] * kLog2e);  // exp(delta A_h)

  // Shared per workgroup: rotations, B, C (and B_prev) of every rank, x (and
  // x_prev) of this workgroup's rows.
  for (int i = threadIdx.x; i < N; i += kM3Threads) {
    if constexpr (CPLX) {
      float sn, cs;
      sincosf(dl * a.theta[(size_t)hd * N + i], &sn, &cs);
      s_cs[i][0] = cs;
      s_cs[i][1] = sn;
    }
  }
  for (int i = threadIdx.x; i < R * N; i += kM3Threads) {
    const int r = i / N, n = i % N;
    const size_t o = (bg * R + r) * N + n;
    s_B[r][n] = ld_io<BF16>(a.B, o);
    s_C[r][n] = ld_io<BF16>(a.C, o);
    if constexpr (TRAP) s_Bp[r][n] = ld_io<BF16>(a.B_prev, o);
  }
  if (threadIdx.x < R * kRowsWG) {
    const int r = threadIdx.x / kRowsWG, rr = threadIdx.x % kRowsWG;
    const size_t o = (bh * R + r) * P + p0 + rr;
    s_x[r][rr] = ld_io<BF16>(a.x, o);
    if constexpr (TRAP) s_xp[r][rr] = ld_io<BF16>(a.x_prev, o);
  }

  // This lane's slice of each of its state rows (whole 16-byte groups: F is a
  // multiple of 4), loaded before the barrier.
  float* hrow[RPT];
  float hv[RPT][F];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    hrow[k] = a.h + ((bh * P + p0 + row + k * kM3Rows) * N + n0) * (CPLX ? 2 : 1);
#pragma unroll
    for (int j = 0; j < F; j += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(hrow[k] + j);
      hv[k][j] = v[0], hv[k][j + 1] = v[1], hv[k][j + 2] = v[2], hv[k][j + 3] = v[3];
    }
  }
  __syncthreads();

  const float wcur = TRAP ? 0.5f * dl : dl;  // weight of the current input (trapezoid: delta/2)
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    const int n = n0 + j;
    float u[RPT], up[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) u[k] = up[k] = 0.f;
    for (int r = 0; r < R; ++r) {
      const float bn = s_B[r][n];
      const float bpn = TRAP ? s_Bp[r][n] : 0.f;
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        u[k] = __builtin_fmaf(s_x[r][row + k * kM3Rows], bn, u[k]);
        if constexpr (TRAP) up[k] = __builtin_fmaf(s_xp[r][row + k * kM3Rows], bpn, up[k]);
      }
    }
    if constexpr (CPLX) {
      const float ar = dec * s_cs[n][0], ai = dec * s_cs[n][1];
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const float re = hv[k][2 * j], im = hv[k][2 * j + 1];
        float nre = __builtin_fmaf(ar, re, -ai * im);
        float nim = __builtin_fmaf(ar, im, ai * re);
        if constexpr (TRAP) {
          nre = __builtin_fmaf(wcur, __builtin_fmaf(ar, up[k], u[k]), nre);
          nim = __builtin_fmaf(wcur * ai, up[k], nim);
        } else {
          nre = __builtin_fmaf(wcur, u[k], nre);
        }
        hv[k][2 * j] = nre;
        hv[k][2 * j + 1] = nim;
      }
    } else {
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        float nh = dec * hv[k][j];
        if constexpr (TRAP) nh = __builtin_fmaf(wcur, __builtin_fmaf(dec, up[k], u[k]), nh);
        else nh = __builtin_fmaf(wcur, u[k], nh);
        hv[k][j] = nh;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < RPT; ++k)
#pragma unroll
    for (int j = 0; j < F; j += 4)
      __builtin_nontemporal_store(f32x4{hv[k][j], hv[k][j + 1], hv[k][j + 2], hv[k][j + 3]},
                                  reinterpret_cast<f32x4*>(hrow[k] + j));

  // R readouts of the real part per row, each summed over the row's 16 lanes
  // in a fixed butterfly; lane r of the row finishes output r.
  const float dh = a.D != nullptr ? a.D[hd] : 0.f;
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int rw = row + k * kM3Rows;
    float mine = 0.f;
    for (int r = 0; r < R; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < SPL; ++j) acc = __builtin_fmaf(s_C[r][n0 + j], hv[k][CPLX ? 2 * j : j], acc);
#pragma unroll
      for (int m = 1; m < kM3LanesPerRow; m <<= 1) acc += __shfl_xor(acc, m, kM3LanesPerRow);
      if (q == r) mine = acc;
    }
    if (q < R) {
      const float xv = s_x[q][rw];
      float out = __builtin_fmaf(dh, xv, mine);
      const size_t o = (bh * R + q) * P + p0 + rw;
      if (a.z != nullptr) out *= silu(ld_io<BF16>(a.z, o));
      if constexpr (BF16) static_cast<uint16_t*>(a.y)[o] = f32_to_bf16(out);
      else static_cast<float*>(a.y)[o] = out;
    }
  }
}

template <int SPL, bool CPLX, bool TRAP>
hipError_t launch_m3_typed(const Mamba3Params& p, hipStream_t stream) {
  // Two rows per thread when the headdim allows 32-row workgroups.
  if (p.headdim % (2 * kM3Rows) == 0) {
    const dim3 grid((unsigned)(p.headdim / (2 * kM3Rows)), (unsigned)p.nheads, (unsigned)p.batch);
    if (p.bf16) hipLaunchKernelGGL((mamba3_step_kernel<SPL, 2, CPLX, TRAP, true>), grid, dim3(kM3Threads), 0, stream, p);
    else hipLaunchKernelGGL((mamba3_step_kernel<SPL, 2, CPLX, TRAP, false>), grid, dim3(kM3Threads), 0, stream, p);
  } else {
    const dim3 grid((unsigned)(p.headdim / kM3Rows), (unsigned)p.nheads, (unsigned)p.batch);
    if (p.bf16) hipLaunchKernelGGL((mamba3_step_kernel<SPL, 1, CPLX, TRAP, true>), grid, dim3(kM3Threads), 0, stream, p);
    else hipLaunchKernelGGL((mamba3_step_kernel<SPL, 1, CPLX, TRAP, false>), grid, dim3(kM3Threads), 0, stream, p);
  }
  return hipGetLastError();
}

template <int SPL>
hipError_t launch_m3_spl(const Mamba3Params& p, hipStream_t stream) {
  const bool cplx = p.theta != nullptr, trap = p.x_prev != nullptr;
  if (cplx) return trap ? launch_m3_typed<SPL, true, true>(p, stream) : launch_m3_typed<SPL, true, false>(p, stream);
  return trap ? launch_m3_typed<SPL, false, true>(p, stream) : launch_m3_typed<SPL, false, false>(p, stream);
}

}  // namespace

hipError_t launch_mamba3_step(const Mamba3Params& p, hipStream_t stream) {
  // dstate is 64, 128 or 256 (validated on the host): 4, 8 or 16 states per
  // lane, whole 16-byte groups of the state row.
  switch (p.dstate / kM3LanesPerRow) {
    case 4: return launch_m3_spl<4>(p, stream);
    case 8: return launch_m3_spl<8>(p, stream);
    default: return launch_m3_spl<16>(p, stream);
  }
}

}  // namespace mss
