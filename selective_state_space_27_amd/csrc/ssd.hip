// Mamba-2 SSD layer, chunked, on the CDNA4 matrix cores (gfx950).
//
// What is computed (see include/mambascan.h): per batch b and head h, with the
// heads of a group sharing B and C and one scalar A_h per head ("Mamba-1/2/3
// visual guide", section 3 comparison table),
//   S_t = exp(delta_t A_h) S_{t-1} + delta_t x_t B_t^T       (P x N state)
//   y_t = S_t C_t (+ D_h x_t) (* silu(z_t))
// evaluated the way the same page's chunk figures describe: dense products
// inside a chunk, the state handed from chunk to chunk.  For a block of steps
// with in-block decay sums s_i = A_h * sum_{k<=i} delta_k:
//   y_i   = exp(s_i) C_i S_in^T                                (off-diagonal)
//         + sum_{j<=i} (C_i . B_j) exp(s_i - s_j) delta_j x_j  (diagonal block)
//   S_out = exp(s_last) S_in + sum_j exp(s_last - s_j) delta_j x_j B_j^T
// which is the recurrence above summed over the block (exact up to rounding).
//
// Two kernels:
//   ssd_state_kernel: one workgroup per (batch, head) walks the chunks in
//     order with the 64 x 128 state in MFMA accumulators (fp32) and writes the
//     state entering every chunk to the workspace (and, on request, the state
//     after every chunk and the final state).
//   ssd_scan_kernel: one workgroup per (batch, chunk, head) starts from the
//     state entering its chunk and walks the chunk in 64-step blocks: C B^T,
//     the decay-masked diagonal block times x, exp(s) C S^T, all on
//     v_mfma_f32_32x32x16_bf16 with fp32 accumulation, then the block's state
//     update, kept in accumulators.  Every operand that is not an exact bf16
//     input (the state in C S^T, the decay-weighted diagonal block, x scaled
//     by the decay weights) enters as a bf16 hi/lo pair (two products), so it
//     keeps ~16 bits of mantissa; accumulation is fp32 throughout.
// Operands that the matrix cores read along time (x and B for the state
// update, x for the diagonal block) are staged transposed in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace mss {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kP = 64;      // headdim
constexpr int kN = 128;     // dstate
constexpr int kSub = 64;    // steps per block inside the scan kernel
constexpr int kT = 256;     // threads per workgroup (4 waves)
constexpr int kPadH = 8;    // bf16 row padding (16 bytes)

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Row (within a 32x32 tile) of accumulator register r of lane l.
__device__ __forceinline__ int acc_row(int r, int l) { return 8 * (r >> 2) + 4 * (l >> 5) + (r & 3); }


// fp32 pair -> (hi, lo) bf16 pairs with hi + lo = value to ~16 mantissa bits.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - bf16_lo(hi), b - bf16_hi(hi));
}
__device__ __forceinline__ float lo16(uint32_t w) { return bf16_lo(w); }
__device__ __forceinline__ float hi16(uint32_t w) { return bf16_hi(w); }

struct SSDArgs {
  const uint16_t* x;   // [b, L, H, P] bf16
  const float* delta;  // [b, L, H]
  const float* A;      // [H]
  const uint16_t* B;   // [b, L, G, N] bf16
  const uint16_t* C;   // [b, L, G, N] bf16
  const float* D;      // [H] or null
  const uint16_t* z;   // [b, L, H, P] bf16 or null
  const float* h0;     // [b, H, P, N] or null
  float* y;            // [b, L, H, P]
  float* chunk_states; // [b, nchunks, H, P, N] or null
  float* h_last;       // [b, H, P, N] or null
  float* s_in;         // workspace [b, nchunks, H, P, N]: state entering each chunk
  int batch, L, H, G, Q, nchunks;
};

// Inclusive prefix sum of delta over steps [l0, l0 + n) of head h, computed by
// wave 0 (n <= 64) into cum[]; also stores the deltas.  Out-of-range steps
// count as zero.  Fixed shuffle order: deterministic.
__device__ __forceinline__ void block_cumsum64(const SSDArgs& a, int b, int h, int l0, float* dl, float* cum) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    const int l = l0 + lane;
    float d = (l < a.L) ? a.delta[((size_t)b * a.L + l) * a.H + h] : 0.f;
    float s = d;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t = __shfl_up(s, o, 64);
      if (lane >= o) s += t;
    }
    dl[lane] = d;
    cum[lane] = s;
  }
}

// Stages x^T (bf16, [P][kSub + pad]) for steps [l0, l0 + 64) of head h.
// One thread per (step pair, 8 headdim values): two 16-byte row loads, eight
// packed (step, step+1) words written along time.
__device__ __forceinline__ void stage_xT(const SSDArgs& a, int b, int h, int l0, uint16_t (*xT)[kSub + kPadH]) {
  const int t = threadIdx.x;
  const int pg = t & 7, jp = t >> 3;  // 8 groups of 8 headdim values, 32 step pairs
  const int j = 2 * jp;
  const rsrc_t rx = make_rsrc(a.x + (size_t)b * a.L * a.H * kP, (uint32_t)((size_t)a.L * a.H * kP * 2));
  const uint32_t o0 = (l0 + j < a.L) ? (uint32_t)((((size_t)(l0 + j) * a.H + h) * kP + pg * 8) * 2) : kOffNone;
  const uint32_t o1 = (l0 + j + 1 < a.L) ? (uint32_t)((((size_t)(l0 + j + 1) * a.H + h) * kP + pg * 8) * 2) : kOffNone;
  const u32x4 r0 = buf_load_u32x4(rx, o0);
  const u32x4 r1 = buf_load_u32x4(rx, o1);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w0 = r0[k], w1 = r1[k];
    *reinterpret_cast<uint32_t*>(&xT[pg * 8 + 2 * k][j]) = (w0 & 0xffffu) | (w1 << 16);
    *reinterpret_cast<uint32_t*>(&xT[pg * 8 + 2 * k + 1][j]) = (w0 >> 16) | (w1 & 0xffff0000u);
  }
}

// Stages B (or C) of group g for steps [l0, l0 + 64): row-major copy
// rm[step][N + pad] and/or transposed copy tr[N][kSub + pad].
template <bool ROWMAJOR, bool TRANSPOSED>
__device__ __forceinline__ void stage_bc(const SSDArgs& a, const uint16_t* src, int b, int g, int l0,
                                         uint16_t (*rm)[kN + kPadH], uint16_t (*tr)[kSub + kPadH]) {
  const rsrc_t rs = make_rsrc(src + (size_t)b * a.L * a.G * kN, (uint32_t)((size_t)a.L * a.G * kN * 2));
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int u = threadIdx.x + kT * it;    // 512 units: 32 step pairs x 16 groups of 8 states
    const int ng = u & 15, jp = u >> 4;
    const int j = 2 * jp;
    const uint32_t o0 = (l0 + j < a.L) ? (uint32_t)((((size_t)(l0 + j) * a.G + g) * kN + ng * 8) * 2) : kOffNone;
    const uint32_t o1 = (l0 + j + 1 < a.L) ? (uint32_t)((((size_t)(l0 + j + 1) * a.G + g) * kN + ng * 8) * 2) : kOffNone;
    const u32x4 r0 = buf_load_u32x4(rs, o0);
    const u32x4 r1 = buf_load_u32x4(rs, o1);
    if constexpr (ROWMAJOR) {
      *reinterpret_cast<u32x4*>(&rm[j][ng * 8]) = r0;
      *reinterpret_cast<u32x4*>(&rm[j + 1][ng * 8]) = r1;
    }
    if constexpr (TRANSPOSED) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w0 = r0[k], w1 = r1[k];
        *reinterpret_cast<uint32_t*>(&tr[ng * 8 + 2 * k][j]) = (w0 & 0xffffu) | (w1 << 16);
        *reinterpret_cast<uint32_t*>(&tr[ng * 8 + 2 * k + 1][j]) = (w0 >> 16) | (w1 & 0xffff0000u);
      }
    }
  }
}

// State update over one staged 64-step block, for this wave's two state tiles
// (headdim tile pt, state tiles nt0, nt0+1):
//   S <- decay * S + sum_j w_j x_j B_j^T,  w_j = delta_j exp(s_last - s_j)
// A operand: x^T rows scaled by w_j, as a bf16 hi/lo pair (two products);
// B operand: B^T (exact bf16 inputs).
__device__ __forceinline__ void state_update_block(f32x16* acc, float decay, const float* w,
                                                   const uint16_t (*xT)[kSub + kPadH],
                                                   const uint16_t (*BT)[kSub + kPadH], int pt, int nt0) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < 2; ++t) acc[t] *= decay;
#pragma unroll
  for (int kk = 0; kk < kSub / 16; ++kk) {
    const int j0 = kk * 16 + 8 * (lane >> 5);
    const u32x4 xr = *reinterpret_cast<const u32x4*>(&xT[pt * 32 + (lane & 31)][j0]);
    u32x4 ah, al;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t hh, ll;
      split2(lo16(xr[q]) * w[j0 + 2 * q], hi16(xr[q]) * w[j0 + 2 * q + 1], hh, ll);
      ah[q] = hh;
      al[q] = ll;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 bv = *reinterpret_cast<const u32x4*>(&BT[(nt0 + t) * 32 + (lane & 31)][j0]);
      acc[t] = mfma(ah, bv, acc[t]);
      acc[t] = mfma(al, bv, acc[t]);
    }
  }
}

// Per-block decay quantities from the prefix sums (wave 0): e_i = exp(s_i),
// w_j = delta_j exp(s_last - s_j), and the block decay exp(s_last).
__device__ __forceinline__ void block_weights(float a2, const float* dl, const float* cum, float* e, float* w,
                                              float* decay) {
  if (threadIdx.x < 64) {
    const int i = threadIdx.x;
    const float last = cum[63];
    e[i] = exp2_fast(a2 * cum[i]);
    w[i] = dl[i] * exp2_fast(a2 * (last - cum[i]));
    if (i == 0) *decay = exp2_fast(a2 * last);
  }
}

// Loads/stores one wave's two 32x32 state tiles (headdim tile pt, state tiles
// nt0, nt0+1) of a [P][N] fp32 state.
__device__ __forceinline__ void load_state(f32x16* acc, const float* S, int pt, int nt0) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      acc[t][r] = S ? S[(pt * 32 + acc_row(r, lane)) * kN + (nt0 + t) * 32 + (lane & 31)] : 0.f;
}
__device__ __forceinline__ void store_state(const f32x16* acc, float* S, int pt, int nt0) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) S[(pt * 32 + acc_row(r, lane)) * kN + (nt0 + t) * 32 + (lane & 31)] = acc[t][r];
}

// ---------------------------------------------------------------------------
// Chunk states.  grid (H, batch), 256 threads.
__global__ void __launch_bounds__(kT) ssd_state_kernel(SSDArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xT[kP][kSub + kPadH];
  __shared__ __attribute__((aligned(16))) uint16_t BT[kN][kSub + kPadH];
  __shared__ float s_dl[kSub], s_cum[kSub], s_e[kSub], s_w[kSub];
  __shared__ float s_decay;

  const int h = blockIdx.x, b = blockIdx.y;
  const int g = h / (a.H / a.G);
  const int w = threadIdx.x >> 6;
  const int pt = w & 1, nt0 = 2 * (w >> 1);
  const float a2 = a.A[h] * kLog2e;
  const size_t state_stride = (size_t)kP * kN;

  f32x16 acc[2];
  load_state(acc, a.h0 ? a.h0 + ((size_t)b * a.H + h) * state_stride : nullptr, pt, nt0);

  const int sub_per_chunk = a.Q / kSub;
  const int nsub = (a.L + kSub - 1) / kSub;
  for (int sb = 0; sb < nsub; ++sb) {
    const int l0 = sb * kSub;
    const int c = sb / sub_per_chunk;
    if (sb % sub_per_chunk == 0)  // state entering chunk c
      store_state(acc, a.s_in + (((size_t)b * a.nchunks + c) * a.H + h) * state_stride, pt, nt0);
    block_cumsum64(a, b, h, l0, s_dl, s_cum);
    stage_xT(a, b, h, l0, xT);
    stage_bc<false, true>(a, a.B, b, g, l0, nullptr, BT);
    __syncthreads();
    block_weights(a2, s_dl, s_cum, s_e, s_w, &s_decay);
    __syncthreads();
    state_update_block(acc, s_decay, s_w, xT, BT, pt, nt0);
    const bool chunk_end = (sb % sub_per_chunk == sub_per_chunk - 1) || sb == nsub - 1;
    if (chunk_end && a.chunk_states)
      store_state(acc, a.chunk_states + (((size_t)b * a.nchunks + c) * a.H + h) * state_stride, pt, nt0);
    __syncthreads();
  }
  if (a.h_last) store_state(acc, a.h_last + ((size_t)b * a.H + h) * state_stride, pt, nt0);
}

// ---------------------------------------------------------------------------
// Chunk outputs.  grid (nchunks, H, batch), 256 threads; wave w owns output
// tile (row tile w>>1, headdim tile w&1) and state tiles (w&1, 2*(w>>1)+{0,1}).
__global__ void __launch_bounds__(kT) ssd_scan_kernel(SSDArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xT[kP][kSub + kPadH];
  __shared__ __attribute__((aligned(16))) uint16_t BT[kN][kSub + kPadH];
  __shared__ __attribute__((aligned(16))) uint16_t Cs[kSub][kN + kPadH];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kSub][kN + kPadH];
  __shared__ __attribute__((aligned(16))) uint16_t Shi[kP][kN + kPadH];
  __shared__ __attribute__((aligned(16))) uint16_t Slo[kP][kN + kPadH];
  __shared__ __attribute__((aligned(16))) float Gb[kSub][kSub + 4];
  __shared__ float s_dl[kSub], s_cum[kSub], s_e[kSub], s_w[kSub];
  __shared__ float s_decay;

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.H / a.G);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rt = w >> 1, pt = w & 1;        // output tile
  const int spt = w & 1, snt0 = 2 * (w >> 1);  // state tiles
  const float a2 = a.A[h] * kLog2e;
  const float dh = a.D ? a.D[h] : 0.f;
  const size_t state_stride = (size_t)kP * kN;

  f32x16 st[2];
  load_state(st, a.s_in + (((size_t)b * a.nchunks + c) * a.H + h) * state_stride, spt, snt0);

  const int lbeg = c * a.Q;
  const int lend = min(a.L, lbeg + a.Q);
  for (int l0 = lbeg; l0 < lend; l0 += kSub) {
    // Stage the block and the current state (hi/lo bf16 split of fp32).
    block_cumsum64(a, b, h, l0, s_dl, s_cum);
    stage_xT(a, b, h, l0, xT);
    stage_bc<true, true>(a, a.B, b, g, l0, Bs, BT);
    stage_bc<true, false>(a, a.C, b, g, l0, Cs, nullptr);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = spt * 32 + acc_row(r, lane), n = (snt0 + t) * 32 + (lane & 31);
        const float v = st[t][r];
        const uint16_t hv = f32_to_bf16(v);
        Shi[p][n] = hv;
        Slo[p][n] = f32_to_bf16(v - bf16_to_f32(hv));
      }
    __syncthreads();
    block_weights(a2, s_dl, s_cum, s_e, s_w, &s_decay);

    // G = C B^T for this wave's 32x32 tile (row tile rt, column tile pt).
    {
      f32x16 gacc = {};
#pragma unroll
      for (int kk = 0; kk < kN / 16; ++kk) {
        const int k0 = kk * 16 + 8 * (lane >> 5);
        const u32x4 av = *reinterpret_cast<const u32x4*>(&Cs[rt * 32 + (lane & 31)][k0]);
        const u32x4 bv = *reinterpret_cast<const u32x4*>(&Bs[pt * 32 + (lane & 31)][k0]);
        gacc = mfma(av, bv, gacc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Gb[rt * 32 + acc_row(r, lane)][pt * 32 + (lane & 31)] = gacc[r];
    }

    // Off-diagonal part: exp(s_i) * C_i S^T, state as hi + lo.
    f32x16 yacc = {};
#pragma unroll
    for (int kk = 0; kk < kN / 16; ++kk) {
      const int k0 = kk * 16 + 8 * (lane >> 5);
      const u32x4 av = *reinterpret_cast<const u32x4*>(&Cs[rt * 32 + (lane & 31)][k0]);
      const u32x4 bh = *reinterpret_cast<const u32x4*>(&Shi[pt * 32 + (lane & 31)][k0]);
      const u32x4 bl = *reinterpret_cast<const u32x4*>(&Slo[pt * 32 + (lane & 31)][k0]);
      yacc = mfma(av, bh, yacc);
      yacc = mfma(av, bl, yacc);
    }
    __syncthreads();  // G tiles and block weights complete
#pragma unroll
    for (int r = 0; r < 16; ++r) yacc[r] *= s_e[rt * 32 + acc_row(r, lane)];

    // Diagonal block: M = mask o G o exp(s_i - s_j) delta_j, times x.
    {
      const int i = rt * 32 + (lane & 31);
      const float ci = s_cum[i];
      for (int kk = 0; kk < 2 * (rt + 1); ++kk) {
        const int j0 = kk * 16 + 8 * (lane >> 5);
        const float4 g0 = *reinterpret_cast<const float4*>(&Gb[i][j0]);
        const float4 g1 = *reinterpret_cast<const float4*>(&Gb[i][j0 + 4]);
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        float m[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = j0 + q;
          const float dec = exp2_fast(fminf(a2 * (ci - s_cum[j]), 0.f));
          m[q] = (j <= i) ? gv[q] * dec * s_dl[j] : 0.f;
        }
        u32x4 ah, al;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t hh, ll;
          split2(m[2 * q], m[2 * q + 1], hh, ll);
          ah[q] = hh;
          al[q] = ll;
        }
        const u32x4 bv = *reinterpret_cast<const u32x4*>(&xT[pt * 32 + (lane & 31)][j0]);
        yacc = mfma(ah, bv, yacc);
        yacc = mfma(al, bv, yacc);
      }
    }

    // Skip term, gate, store: element (row i, headdim p).
    {
      const int p = pt * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = rt * 32 + acc_row(r, lane);
        const int l = l0 + i;
        if (l < lend) {
          float v = yacc[r];
          const size_t off = (((size_t)b * a.L + l) * a.H + h) * kP + p;
          if (a.D) v = __builtin_fmaf(dh, bf16_to_f32(xT[p][i]), v);
          if (a.z) v *= silu(bf16_to_f32(a.z[off]));
          a.y[off] = v;
        }
      }
    }

    // State after the block.
    state_update_block(st, s_decay, s_w, xT, BT, spt, snt0);
    __syncthreads();
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t ssd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                           int64_t dstate, int64_t chunk) {
  (void)ngroups;
  const int64_t nchunks = (seqlen + chunk - 1) / chunk;
  return align256((size_t)batch * nchunks * nheads * headdim * dstate * sizeof(float));
}

hipError_t launch_ssd(const SSDParams& p, hipStream_t stream) {
  SSDArgs a;
  a.x = static_cast<const uint16_t*>(p.x);
  a.delta = p.delta;
  a.A = p.A;
  a.B = static_cast<const uint16_t*>(p.B);
  a.C = static_cast<const uint16_t*>(p.C);
  a.D = p.D;
  a.z = static_cast<const uint16_t*>(p.z);
  a.h0 = p.h0;
  a.y = p.y;
  a.chunk_states = p.chunk_states;
  a.h_last = p.h_last;
  a.s_in = static_cast<float*>(p.workspace);
  a.batch = (int)p.batch;
  a.L = (int)p.seqlen;
  a.H = (int)p.nheads;
  a.G = (int)p.ngroups;
  a.Q = (int)p.chunk;
  a.nchunks = (int)((p.seqlen + p.chunk - 1) / p.chunk);
  hipLaunchKernelGGL(ssd_state_kernel, dim3((unsigned)a.H, (unsigned)a.batch), dim3(kT), 0, stream, a);
  hipLaunchKernelGGL(ssd_scan_kernel, dim3((unsigned)a.nchunks, (unsigned)a.H, (unsigned)a.batch), dim3(kT), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace mss
