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
// Three kernels; the two big ones on v_mfma_f32_32x32x16_bf16 with fp32
// accumulation:
//   ssd_cumsum_kernel: delta transposed to head-major rows and its prefix
//     sums inside every 64-step block, scaled by A log2(e), into the
//     workspace (the decay factors of both other kernels come from these).
//   ssd_state_kernel: one workgroup per (batch, head, 32-wide headdim tile),
//     eight waves (four 32-row tiles of S^T, each over half of every block's
//     steps, the halves added where a state is written), walks the sequence
//     in 64-step blocks with the next block staged while the current one is
//     multiplied, and writes the state entering every chunk to the workspace
//     (and, on request, the state after every chunk and the final state).
//   ssd_scan_kernel: one workgroup per (batch, chunk, head) starts from the
//     state entering its chunk and walks the chunk in 64-step blocks.  Each
//     wave owns one 32 x 32 output tile and holds S^T for its headdim tile in
//     accumulators; C S^T, G^T = B C^T, the decay-masked diagonal block times
//     x and the state update all run on the matrix cores.  Accumulator tiles
//     become MFMA operands in registers: a K slice of 16 rows is gathered by
//     swapping lane halves of register pairs (v_permlane32_swap), so neither
//     the state nor G passes through LDS.
// Every operand that is not an exact bf16 input (the state in C S^T, the
// decay-weighted diagonal block, x scaled by the decay weights) enters as a
// bf16 hi/lo pair (two products), keeping ~16 bits of mantissa.  Operands the
// matrix cores read along time (x and B) are staged transposed in LDS.
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "ssd_common.hpp"

namespace mss {
namespace {

using namespace ssd;
constexpr int kT = 256;     // threads per workgroup (4 waves)

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
  float* dlT;          // workspace [b, H, Lp]: delta, head-major (0 past L)
  float* lsT;          // workspace [b, H, Lp]: A log2(e) times the prefix sum of delta inside each 64-step block
  float* pend;         // workspace [b, Hv, npieces, 64, 128]: state at the end of each piece, from the piece's start
  float* pstart;       // workspace [b, Hv, npieces, 64, 128]: exact state entering each piece (pieces 1..)
  float* pdec;         // workspace [b, Hv, npieces]: A log2(e) sum of delta over each piece
  int* status;         // workspace: the call's status word (first 4 bytes)
  int batch, L, H, G, Q, nchunks, Lp;
  // Heads of headdim P run as P/64 "virtual heads" of 64 (the rows p of a
  // head's state evolve independently under the head's delta and A): virtual
  // head v is rows (v % ph)*64.. of head v / ph.  States wider than 128 run as
  // 128-wide halves, one launch sequence each: states noff .. noff+127 here
  // (columns past N read and stay zero).
  int P, ph, Hv, N, noff;
  int accumulate;      // y += this half's part (second half of N > 128)
  int npieces, cpp;    // the sequence is cut into npieces pieces of cpp chunks (the last may be shorter)
};

__device__ __forceinline__ int head_of(const SSDArgs& a, int vh) { return vh / a.ph; }
// Element offset of (virtual head vh, its row p) inside one step's [H, P] row.
__device__ __forceinline__ size_t row_el(const SSDArgs& a, int vh, int p) {
  return (size_t)(vh / a.ph) * a.P + (size_t)(vh % a.ph) * kP + p;
}
// Element offset of state row p, column noff of virtual head vh in a
// [b, H, P, N] tensor (state_el(a, b, vh) + p*N + n, n < N - noff).
__device__ __forceinline__ size_t state_el(const SSDArgs& a, int b, int vh) {
  return (((size_t)b * a.H + vh / a.ph) * a.P + (size_t)(vh % a.ph) * kP) * a.N + a.noff;
}


// Head-major delta rows and their scaled prefix sums, per (64-step block,
// 64-head tile, batch): ls_i = A log2(e) sum_{j<=i} delta_j inside the block,
// so that inside a block exp(s_i - s_j) = exp2(ls_i - ls_j), the decay over a
// whole block is exp2(ls_63) and steps past L (delta 0) leave ls unchanged.
__global__ void __launch_bounds__(256) ssd_cumsum_kernel(SSDArgs a) {
  __shared__ float tile[kSub][65];
  const int l0 = blockIdx.x * kSub, h0 = blockIdx.y * 64, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // The workspace's status word (no kernel here waits on another workgroup).
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *a.status = 0;
#pragma unroll
  for (int i = 0; i < kSub / 4; ++i) {
    const int j = w + 4 * i, l = l0 + j, hh = h0 + lane;
    tile[j][lane] = (l < a.L && hh < a.H) ? a.delta[((size_t)b * a.L + l) * a.H + hh] : 0.f;
  }
  __syncthreads();
  for (int k = 0; k < 16; ++k) {
    const int h = h0 + w * 16 + k;
    if (h >= a.H) break;
    const float d = tile[lane][w * 16 + k];
    const float ls = a.A[h] * kLog2e * wave_prefix_sum(d);
    const size_t o = ((size_t)b * a.H + h) * a.Lp + l0 + lane;
    a.dlT[o] = d;
    a.lsT[o] = ls;
  }
}

// B or C rows of group g for steps (l0 + j, l0 + j + 1), 8 states from
// noff + ng*8: two 16-byte loads per unit, 2 units per thread.  The
// descriptor starts at step l0, so each thread's offsets are fixed; steps past
// L lie beyond it and read zero, and so do states past N.
struct BCRegs {
  u32x4 r[2][2];
};
struct BCOffsets {
  uint32_t o[2][2];
};
__device__ __forceinline__ BCOffsets bc_offsets(const SSDArgs& a, int g) {
  BCOffsets r;
  const uint32_t row = (uint32_t)(a.G * a.N * 2);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int u = threadIdx.x + kT * it;  // 512 units: 32 step pairs x 16 groups of 8 states
    const int ng = u & 15, j = 2 * (u >> 4);
    const bool nok = a.noff + ng * 8 < a.N;
    const uint32_t col = (uint32_t)((g * a.N + a.noff + ng * 8) * 2);
#pragma unroll
    for (int e = 0; e < 2; ++e) r.o[it][e] = nok ? (uint32_t)(j + e) * row + col : kOffNone;
  }
  return r;
}
__device__ __forceinline__ void load_bc_rows(const SSDArgs& a, const uint16_t* src, int b, int l0,
                                             const BCOffsets& off, BCRegs& o) {
  const uint32_t left = (uint32_t)max(a.L - l0, 0);
  const rsrc_t rs = make_rsrc(src + ((size_t)b * a.L + l0) * a.G * a.N, left * (uint32_t)(a.G * a.N * 2));
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int e = 0; e < 2; ++e) o.r[it][e] = buf_load_u32x4(rs, off.o[it][e]);
}
// Row-major copy rm[step][N + pad] and/or time-contiguous copy tr (tsw layout, N rows).
template <bool ROWMAJOR, bool TRANSPOSED>
__device__ __forceinline__ void store_bc_rows(const BCRegs& o, uint16_t (*rm)[kN + kPadH], uint16_t* tr) {
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int u = threadIdx.x + kT * it;
    const int ng = u & 15, j = 2 * (u >> 4);
    const u32x4 r0 = o.r[it][0], r1 = o.r[it][1];
    if constexpr (ROWMAJOR) {
      *reinterpret_cast<u32x4*>(&rm[j][ng * 8]) = r0;
      *reinterpret_cast<u32x4*>(&rm[j + 1][ng * 8]) = r1;
    }
    if constexpr (TRANSPOSED) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w0 = r0[k], w1 = r1[k];
        *reinterpret_cast<uint32_t*>(&tr[tsw(ng * 8 + 2 * k, j)]) = (w0 & 0xffffu) | (w1 << 16);
        *reinterpret_cast<uint32_t*>(&tr[tsw(ng * 8 + 2 * k + 1, j)]) = (w0 >> 16) | (w1 & 0xffff0000u);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Piece states.  grid (2 Hv, batch, npieces - 1), 512 threads: workgroup (b, vh,
// pt, piece) owns headdim tile pt of virtual head vh over the chunks of one
// piece of the sequence and runs them from a zero state (piece 0 from h0),
// writing only the piece's end state and its decay; ssd_chain_kernel then
// makes the exact state entering each piece, from which the scan kernel walks
// the piece's chunks.  Cutting the sequence keeps every CU equally busy.
// Wave w owns S^T rows (w&3)*32.. over half of every block's steps (k-half
// w>>2): the state is the sum of the two halves' partial states, which decay
// alike, so they are only added where the state is written out.  Each thread
// forms the decay weights of its own steps from the head-major delta rows;
// the weighted x (w_j x_j) is staged once per block as bf16 hi/lo pairs.
// Stagings are double-buffered: one barrier per block.
constexpr int kTS = 512;

__global__ void __launch_bounds__(kTS, 4) ssd_state_kernel(SSDArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xh[2][32 * kTRow];  // tsw layout: hi part of w o x, headdim rows
  __shared__ __attribute__((aligned(16))) uint16_t xl[2][32 * kTRow];  // lo part
  __shared__ __attribute__((aligned(16))) uint16_t BT[2][kN * kTRow];  // tsw layout, state rows
  // The 32 x 128 state slice [p][n] of this headdim tile on its way out (rows
  // padded to 132 floats: a b128 access of 16 lanes of one n and 16 rows p
  // covers 16 distinct bank groups).
  constexpr int kSRow = kN + 4;
  __shared__ __attribute__((aligned(16))) float sout[32 * kSRow];

  // Both headdim tiles of a virtual head on one XCD (workgroups are dealt to
  // the XCDs round-robin), so that each x row is fetched from HBM once.
  const int i = blockIdx.x;
  const bool pair = (a.Hv & 7) == 0;
  const int pt = pair ? (i >> 3) & 1 : i & 1;
  const int vh = pair ? ((i >> 4) << 3) | (i & 7) : i >> 1;
  const int h = head_of(a, vh);
  const int b = blockIdx.y;
  const int piece = blockIdx.z;
  const int g = h / (a.H / a.G);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave id, uniform
  const int lc = lane & 31, hf = lane >> 5;
  const int nt = w & 3, kh = w >> 2;
  const size_t state_stride = (size_t)kP * kN;
  const Dot2Masks dm = dot2_masks();
  // This piece's 64-step blocks [sb0, sb1).
  const int sub_per_chunk = a.Q / kSub;
  const int nsub = (a.L + kSub - 1) / kSub;
  const int c0 = piece * a.cpp;
  const int sb0 = c0 * sub_per_chunk;
  const int sb1 = min(nsub, min(a.nchunks, c0 + a.cpp) * sub_per_chunk);

  // Staging map: thread -> step pair (jx, jx+1); headdim values pq*2, pq*2+1
  // of x, states noff + ng*8 .. +7 of B.
  const int pq = threadIdx.x & 15, ng = pq, jx = 2 * (threadIdx.x >> 4);
  // Each block's loads go through descriptors based at the block's first
  // step, so the per-lane offsets are fixed; rows past L (or past the padded
  // delta rows) lie beyond the descriptor and read 0, and so do the B columns
  // past N.  Byte offsets inside one batch entry fit 32 bits (checked by the
  // caller).
  const uint32_t x_row = (uint32_t)(a.H * a.P * 2), b_row = (uint32_t)(a.G * a.N * 2);
  const uint32_t xo0 = (uint32_t)jx * x_row + (uint32_t)(row_el(a, vh, pt * 32 + pq * 2) * 2), xo1 = xo0 + x_row;
  const bool bok = a.noff + ng * 8 < a.N;
  const uint32_t bcol = (uint32_t)((g * a.N + a.noff + ng * 8) * 2);
  const uint32_t bo0 = bok ? (uint32_t)jx * b_row + bcol : kOffNone;
  const uint32_t bo1 = bok ? (uint32_t)(jx + 1) * b_row + bcol : kOffNone;
  const uint32_t dlo = (uint32_t)jx * 4u;
  const size_t row_bh = ((size_t)b * a.H + h) * a.Lp;

  // Loads of one block: x and the delta rows (from HBM) four blocks ahead of
  // their staging, B (shared by every head, so mostly an L2 hit) two ahead.
  // All of them are vector loads, waited for through vmcnt in issue order: a
  // scalar-cache load would share lgkmcnt with the LDS traffic, and the
  // lgkmcnt(0) in front of every barrier would wait for it right away.
  struct XSlot {
    uint32_t xr[2];
    u32x2 dl, ls;
    float last;
  };
  struct BSlot {
    u32x4 br[2];
  };
  auto load_x = [&](int blk, XSlot& sl) {
    const int l0 = blk * kSub;
    const uint32_t left = (uint32_t)max(a.L - l0, 0), left_p = (uint32_t)max(a.Lp - l0, 0);
    const rsrc_t rx = make_rsrc(a.x + ((size_t)b * a.L + l0) * a.H * a.P, left * x_row);
    const rsrc_t rd = make_rsrc(a.dlT + row_bh + l0, left_p * 4u);
    const rsrc_t rl = make_rsrc(a.lsT + row_bh + l0, left_p * 4u);
    sl.xr[0] = buf_load_u32(rx, xo0);
    sl.xr[1] = buf_load_u32(rx, xo1);
    sl.dl = buf_load_u32x2(rd, dlo);
    sl.ls = buf_load_u32x2(rl, dlo);
    // Prefix sum at the block's last step, the same address in every lane
    // (blocks past the padded rows read 0; they are staged as zeros and their
    // decay is never applied).
    sl.last = __uint_as_float(buf_load_u32(rl, (uint32_t)(kSub - 1) * 4u));
  };
  auto load_b = [&](int blk, BSlot& sl) {
    const int l0 = blk * kSub;
    const uint32_t left = (uint32_t)max(a.L - l0, 0);
    const rsrc_t rb = make_rsrc(a.B + ((size_t)b * a.L + l0) * a.G * a.N, left * b_row);
    sl.br[0] = buf_load_u32x4(rb, bo0);
    sl.br[1] = buf_load_u32x4(rb, bo1);
  };
  // w o x for steps (jx, jx+1) of headdim rows pq*2, pq*2+1 as hi/lo pairs,
  // w_j = delta_j exp(s_last - s_j); B transposed to state rows.
  auto stage = [&](const XSlot& sl, const BSlot& sb_, int buf) {
    const float w0 = __uint_as_float(sl.dl[0]) * exp2_fast(sl.last - __uint_as_float(sl.ls[0]));
    const float w1 = __uint_as_float(sl.dl[1]) * exp2_fast(sl.last - __uint_as_float(sl.ls[1]));
    uint32_t hi, lo;
    split2(bf16_lo(sl.xr[0]) * w0, bf16_lo(sl.xr[1]) * w1, hi, lo, dm);
    *reinterpret_cast<uint32_t*>(&xh[buf][tsw(pq * 2, jx)]) = hi;
    *reinterpret_cast<uint32_t*>(&xl[buf][tsw(pq * 2, jx)]) = lo;
    split2(bf16_hi(sl.xr[0]) * w0, bf16_hi(sl.xr[1]) * w1, hi, lo, dm);
    *reinterpret_cast<uint32_t*>(&xh[buf][tsw(pq * 2 + 1, jx)]) = hi;
    *reinterpret_cast<uint32_t*>(&xl[buf][tsw(pq * 2 + 1, jx)]) = lo;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t v0 = sb_.br[0][k], v1 = sb_.br[1][k];
      *reinterpret_cast<uint32_t*>(&BT[buf][tsw(ng * 8 + 2 * k, jx)]) = (v0 & 0xffffu) | (v1 << 16);
      *reinterpret_cast<uint32_t*>(&BT[buf][tsw(ng * 8 + 2 * k + 1, jx)]) = (v0 >> 16) | (v1 & 0xffff0000u);
    }
  };

  // The state is the sum of both k-halves' partials: k-half 0 of piece 0
  // starts from h0, everything else from zero.
  f32x16 st;
  load_stateT(st, (a.h0 && kh == 0 && piece == 0) ? a.h0 + state_el(a, b, vh) : nullptr, nt, pt, a.N,
              a.N - a.noff);
  // Writes the full state slice (rows pt*32.., all 128 n) of a [64][128]
  // state: k-half 1 puts its partial in LDS, k-half 0 adds its own, then the
  // workgroup copies the 16 KB slice out with whole-row stores.
  auto write_state = [&](float* S) {
    const int sp = lc;  // headdim row of this lane's accumulator column
    if (kh == 1) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int n = nt * 32 + 8 * g4 + 4 * hf;
        *reinterpret_cast<f32x4*>(&sout[sp * kSRow + n]) =
            f32x4{st[4 * g4], st[4 * g4 + 1], st[4 * g4 + 2], st[4 * g4 + 3]};
      }
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int n = nt * 32 + 8 * g4 + 4 * hf;
        f32x4* q = reinterpret_cast<f32x4*>(&sout[sp * kSRow + n]);
        *q = *q + f32x4{st[4 * g4], st[4 * g4 + 1], st[4 * g4 + 2], st[4 * g4 + 3]};
      }
    }
    __syncthreads();
    float* dst = S + (size_t)pt * 32 * kN;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int e = (threadIdx.x + it * kTS) * 4;  // element of the 32 x 128 slice
      const int row = e / kN, col = e % kN;
      *reinterpret_cast<f32x4*>(&dst[e]) = *reinterpret_cast<const f32x4*>(&sout[row * kSRow + col]);
    }
  };

  // Software pipeline: iteration rel runs block sb0+rel's products from
  // staging buffer rel&1 while it stages the next block into the other buffer
  // (whose last readers finished before the previous barrier), one barrier
  // per block.  The next block sits in x slot (rel+1)%4 and B slot (rel+1)%2
  // (loop unrolled by four so the slots are compile-time constants).  Loads
  // that run past the piece read the next piece's steps (or zeros past the
  // end) and are never multiplied.
  XSlot xring[4];
  BSlot bring[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) load_x(sb0 + k, xring[k]);
  load_b(sb0, bring[0]);
  load_b(sb0 + 1, bring[1]);
  stage(xring[0], bring[0], 0);
  float lcur = xring[0].last;  // s_last (log2 units) of the block being multiplied
  float lsum = 0.f;            // the same summed over the piece's earlier blocks
  load_b(sb0 + 2, bring[0]);
  load_x(sb0 + 4, xring[0]);
  __syncthreads();

  auto step = [&](auto x_tag, auto b_tag, int rel) {
    constexpr int SX = decltype(x_tag)::value;  // (rel + 1) % 4
    constexpr int SB = decltype(b_tag)::value;  // (rel + 1) % 2
    const int sb = sb0 + rel;
    const int buf = rel & 1;
    st *= exp2_fast(lcur);
    lsum += lcur;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int j0 = (kh * 2 + kk) * 16 + 8 * hf;
      const u32x4 bh = *reinterpret_cast<const u32x4*>(&xh[buf][tsw(lc, j0)]);
      const u32x4 bl = *reinterpret_cast<const u32x4*>(&xl[buf][tsw(lc, j0)]);
      const u32x4 av = *reinterpret_cast<const u32x4*>(&BT[buf][tsw(nt * 32 + lc, j0)]);
      st = mfma(av, bh, st);
      st = mfma(av, bl, st);
    }
    stage(xring[SX], bring[SB], buf ^ 1);
    lcur = xring[SX].last;
    // Every read of the two slots happens before their next loads are issued,
    // so the loads can land in the same registers: otherwise the unrolled
    // loop ends in register copies that wait for loads still in flight.
    asm volatile("" ::"v"(lcur) : "memory");
    // B first: loads return in issue order, so the wait for this B two steps
    // from now covers only the x loads issued before it (three steps old).
    load_b(sb + 3, bring[SB]);
    load_x(sb + 5, xring[SX]);
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  const int nrel = sb1 - sb0;
  int rel = 0;
  for (; rel + 4 <= nrel; rel += 4) {
    step(I1{}, I1{}, rel);
    step(I2{}, I0{}, rel + 1);
    step(I3{}, I1{}, rel + 2);
    step(I0{}, I0{}, rel + 3);
  }
  if (rel < nrel) step(I1{}, I1{}, rel);
  if (rel + 1 < nrel) step(I2{}, I0{}, rel + 1);
  if (rel + 2 < nrel) step(I3{}, I1{}, rel + 2);
  // The piece's end state (from its start) and decay for the chain; the last
  // piece's are not needed (the scan kernel walks that piece to the end).
  if (piece < a.npieces - 1) {
    write_state(a.pend + (((size_t)b * a.Hv + vh) * a.npieces + piece) * state_stride);
    if (threadIdx.x == 0 && pt == 0) a.pdec[((size_t)b * a.Hv + vh) * a.npieces + piece] = lsum;
  }
}

// The exact state entering every piece after the first:
// S(k+1) = exp(A sum of delta over piece k) S(k) + pend(k), S(1) = pend(0)
// (piece 0 ran from h0).  grid (8 slices of the state, Hv, batch), 256
// threads, 4 state elements per thread.
constexpr int kMaxPieces = 64;
__global__ void __launch_bounds__(256) ssd_chain_kernel(SSDArgs a) {
  const int h = blockIdx.y, b = blockIdx.z;
  const size_t state_stride = (size_t)kP * kN;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
  const size_t base = ((size_t)b * a.Hv + h) * a.npieces * state_stride + e;
  const float* pdec = a.pdec + ((size_t)b * a.Hv + h) * a.npieces;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int k = 1; k < a.npieces; ++k) {
    const f32x4 pe = *reinterpret_cast<const f32x4*>(&a.pend[base + (size_t)(k - 1) * state_stride]);
    s = s * exp2_fast(pdec[k - 1]) + pe;
    *reinterpret_cast<f32x4*>(&a.pstart[base + (size_t)k * state_stride]) = s;
  }
}

// ---------------------------------------------------------------------------
// Outputs.  grid (npieces x Hv x batch), 256 threads: one workgroup per
// (batch, virtual head, piece) starts from the exact state entering its piece
// and walks the piece's chunks in 64-step blocks, the running state staying
// in the matrix cores' accumulators; the state after each chunk is written
// when requested (it is exact), and the final state by the last piece.  Wave
// w = (rt, pt) with rt = w>>1, pt = w&1 owns output tile (row tile rt,
// headdim tile pt) and the two S^T tiles (state rows 64*rt .. +64, headdim
// tile pt).  C S^T is split by state rows: each wave forms it over its own
// two state tiles for both row tiles and hands the other row tile's partial
// sum to its partner wave (1-rt, pt) through LDS, already scaled by exp(s_i).
// Of the masked decay block's three 32x32 tiles (0,0), (1,0), (1,1), the full
// tile (1,0) is split by k-slice between the two row tiles, so that every wave
// forms three slices; the rows-0 wave hands its slice's product over with the
// C S^T part.
// Part of the masked decay block: the G^T tile (rows j of tile JT, columns i
// of tile RT) = B C^T on the matrix cores, then k-slices [S0, S1) of
// M = mask o G o exp(s_i - s_j) delta_j as the A operand (rows i, k = j),
// times x (headdim tile pt) accumulated into yacc.  Masked elements (j > i)
// are dropped by a select, so whatever their exponent gives is harmless.
// FACTORED: the block's prefix sums fall (A <= 0) by less than 200 (log2
// units), and exp(s_i - s_j) delta_j is taken as ei[i] * fd[j] with
// ei = exp2(ls - mid), fd = delta exp2(mid - ls) (each factor within 2^100,
// the unmasked products at most delta); otherwise one exp2 per element.
template <int RT, int JT, int S0, int S1, bool FACTORED>
__device__ __forceinline__ void diag_part(f32x16& yacc, const uint16_t (*Cs)[kN + kPadH],
                                          const uint16_t (*Bs)[kN + kPadH], const uint16_t* xT, const float* s_ls,
                                          const float* s_dl, const float* s_ei, const float* s_fd, int pt,
                                          const Dot2Masks& dm) {
  const int lane = threadIdx.x & 63, lc = lane & 31, hf = lane >> 5;
  const int i = RT * 32 + lc;
  const float rowv = FACTORED ? s_ei[i] : s_ls[i];  // ei[i], or ls_i
  f32x16 gacc = {};
#pragma unroll
  for (int kk = 0; kk < kN / 16; ++kk) {
    const u32x4 bop = *reinterpret_cast<const u32x4*>(&Bs[JT * 32 + lc][kk * 16 + 8 * hf]);
    const u32x4 cop = *reinterpret_cast<const u32x4*>(&Cs[RT * 32 + lc][kk * 16 + 8 * hf]);
    gacc = mfma(bop, cop, gacc);
  }
  auto slice = [&](auto s_tag) {
    constexpr int S = decltype(s_tag)::value;
    float gv[8];
    acc_kslice<S>(gacc, gv);
    const int j0 = JT * 32 + 16 * S + 8 * hf;
    float m[8];
    if constexpr (FACTORED) {
      const f32x4 f0 = *reinterpret_cast<const f32x4*>(&s_fd[j0]);
      const f32x4 f1 = *reinterpret_cast<const f32x4*>(&s_fd[j0 + 4]);
      const float fj[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float v = gv[t] * rowv * fj[t];
        m[t] = (JT < RT || j0 + t <= i) ? v : 0.f;
      }
    } else {
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(&s_ls[j0]);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(&s_ls[j0 + 4]);
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(&s_dl[j0]);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(&s_dl[j0 + 4]);
      const float cj[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
      const float dj[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float dec = exp2_fast(rowv - cj[t]);
        const float v = gv[t] * dec * dj[t];
        m[t] = (JT < RT || j0 + t <= i) ? v : 0.f;
      }
    }
    u32x4 mh, ml;
    split8(m, mh, ml, dm);
    const u32x4 xb = *reinterpret_cast<const u32x4*>(&xT[tsw(pt * 32 + lc, j0)]);
    yacc = mfma(mh, xb, yacc);
    yacc = mfma(ml, xb, yacc);
  };
  if constexpr (S0 <= 0 && S1 > 0) slice(std::integral_constant<int, 0>{});
  if constexpr (S0 <= 1 && S1 > 1) slice(std::integral_constant<int, 1>{});
}

// Y = false: the states only (chunk_states, h_last), no output: the block
// products that form y are skipped, and C is not read.
template <bool HAS_Z, bool HAS_D, bool ACCUM, bool Y = true>
__global__ void __launch_bounds__(kT, 2) ssd_scan_kernel(SSDArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xT[kP * kTRow];  // tsw layout, headdim rows
  __shared__ __attribute__((aligned(16))) uint16_t BT[kN * kTRow];  // tsw layout, state rows
  __shared__ __attribute__((aligned(16))) uint16_t Cs[kSub][kN + kPadH];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kSub][kN + kPadH];
  __shared__ __attribute__((aligned(16))) float xbuf[4][16][64];  // partial C S^T handed to the partner wave
  __shared__ __attribute__((aligned(16))) float s_dl[kSub];
  __shared__ __attribute__((aligned(16))) float s_ls[kSub];
  __shared__ __attribute__((aligned(16))) float s_e[kSub];
  __shared__ __attribute__((aligned(16))) float s_w[kSub];
  __shared__ __attribute__((aligned(16))) float s_ei[kSub];  // exp2(ls - mid) (factored decay block)
  __shared__ __attribute__((aligned(16))) float s_fd[kSub];  // delta exp2(mid - ls)
  __shared__ float s_decay;
  __shared__ int s_factored;

  // Workgroups are dealt to the 8 XCDs round-robin; XCD x takes a contiguous
  // run of (piece, batch, virtual head) items in piece-major order, so the B
  // and C rows of a piece, shared by all heads of its group, are read into one
  // L2.
  int piece, vh, b;
  {
    const int nwg = a.npieces * a.batch * a.Hv;
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int q = nwg >> 3, r = nwg & 7;
    const int t = x * q + min(x, r) + j;
    piece = t / (a.batch * a.Hv);
    b = (t / a.Hv) % a.batch;
    vh = t % a.Hv;
  }
  const int h = head_of(a, vh);
  const int g = h / (a.H / a.G);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave id, uniform: branches on it are scalar
  const int lc = lane & 31, hf = lane >> 5;
  const int rt = w >> 1, pt = w & 1;
  const Dot2Masks dm = dot2_masks();
  const int partner = w ^ 2;
  const float dh = a.D ? a.D[h] : 0.f;
  const size_t state_stride = (size_t)kP * kN;
  const int p = pt * 32 + lc;  // headdim row (within the virtual head) of this lane's output column
  const int nvalid = a.N - a.noff;  // state columns of this half that exist (the rest stay zero)

  // x staging: thread -> (step pair j, 8 headdim values pg*8..), through a
  // descriptor starting at the block's first step (fixed per-thread offsets;
  // steps past L read zero).
  const int pg = threadIdx.x & 7, jx = 2 * (threadIdx.x >> 3);
  const uint32_t x_row = (uint32_t)(a.H * a.P * 2);
  const uint32_t xo0 = (uint32_t)jx * x_row + (uint32_t)(row_el(a, vh, pg * 8) * 2);
  auto load_x = [&](int l0, u32x4* xr) {
    const uint32_t left = (uint32_t)max(a.L - l0, 0);
    const rsrc_t rx = make_rsrc(a.x + ((size_t)b * a.L + l0) * a.H * a.P, left * x_row);
    xr[0] = buf_load_u32x4(rx, xo0);
    xr[1] = buf_load_u32x4(rx, xo0 + x_row);
  };
  const BCOffsets bco = bc_offsets(a, g);
  auto store_x = [&](const u32x4* xr) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w0 = xr[0][k], w1 = xr[1][k];
      *reinterpret_cast<uint32_t*>(&xT[tsw(pg * 8 + 2 * k, jx)]) = (w0 & 0xffffu) | (w1 << 16);
      *reinterpret_cast<uint32_t*>(&xT[tsw(pg * 8 + 2 * k + 1, jx)]) = (w0 >> 16) | (w1 & 0xffff0000u);
    }
  };

  // This wave's two state tiles: state rows (2*rt + t)*32.., headdim tile pt,
  // from the exact state entering the piece (piece 0: h0 or zero); as S^T
  // tiles (the operand of C S^T), or with no output as S tiles (stored in
  // whole lines).
  f32x16 st[2];
  auto load_st = [&](f32x16& acc, const float* S, int nt, int ld, int nmax) {
    if constexpr (Y)
      load_stateT(acc, S, nt, pt, ld, nmax);
    else
      load_stateS(acc, S, nt, pt, ld, nmax);
  };
  auto store_st = [&](const f32x16& acc, float* S, int nt) {
    if constexpr (Y)
      store_stateT(acc, S, nt, pt, a.N, nvalid);
    else
      store_stateS(acc, S, nt, pt, a.N, nvalid);
  };
  if (piece == 0) {
    const float* s0 = a.h0 ? a.h0 + state_el(a, b, vh) : nullptr;
#pragma unroll
    for (int t = 0; t < 2; ++t) load_st(st[t], s0, 2 * rt + t, a.N, nvalid);
  } else {
    const float* ps = a.pstart + (((size_t)b * a.Hv + vh) * a.npieces + piece) * state_stride;
#pragma unroll
    for (int t = 0; t < 2; ++t) load_st(st[t], ps, 2 * rt + t, kN, kN);
  }

  // Output of the previous block, finished at the start of the next one (the
  // partner's part is in xbuf then): accumulator and x of this lane's 16 rows.
  const int lbeg = piece * a.cpp * a.Q;
  const int lend = min(a.L, lbeg + a.cpp * a.Q);
  f32x16 yprev = {};
  float xprev[16];
  int lprev = -1;  // first step of the block yprev belongs to
  // y and z rows of this batch entry and virtual head: element (step l,
  // headdim p) at l*H*P + p; steps outside the piece are dropped (store) or
  // read as 0 (z, and y when accumulating).
  const uint32_t row = (uint32_t)(a.H * a.P);
  const size_t hoff = row_el(a, vh, 0);
  const size_t bh_el = (size_t)b * a.L * a.H * a.P + hoff;
  const uint32_t ybytes = (uint32_t)(((size_t)a.L * a.H * a.P - hoff) * 4);
  // y is null only in the states-only instantiation (the backward's state
  // pass without a gate needs no output), which stores none.
  const rsrc_t ry = make_rsrc(a.y ? a.y + bh_el : nullptr, a.y ? ybytes : 0u);
  const rsrc_t rz = make_rsrc(a.z ? a.z + bh_el : nullptr, a.z ? ybytes / 2 : 0u);
  // Row r of this lane's accumulator tile is step lprev + rt*32 + 4*hf +
  // 8*(r>>2) + (r&3): a per-lane base plus a compile-time multiple of the row.
  auto finish = [&]() {
    if (lprev < 0) return;
    const int l_lane = lprev + rt * 32 + 4 * hf;
    const uint32_t o_lane = (uint32_t)l_lane * row + (uint32_t)p;
    float zv[16], yv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dr = 8 * (r >> 2) + (r & 3);
      const bool in = l_lane + dr < lend;
      const uint32_t o = o_lane + (uint32_t)dr * row;
      if constexpr (HAS_Z) zv[r] = bf16_to_f32(buf_load_u16(rz, in ? o * 2u : kOffNone));
      if constexpr (ACCUM) yv[r] = __uint_as_float(buf_load_u32(ry, in ? o * 4u : kOffNone));
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dr = 8 * (r >> 2) + (r & 3);
      float v = xbuf[partner][r][lane] + yprev[r];
      if constexpr (ACCUM) v += yv[r];
      if constexpr (HAS_D) v = __builtin_fmaf(dh, xprev[r], v);
      if constexpr (HAS_Z) v *= silu(zv[r]);
      const uint32_t yo = (l_lane + dr < lend) ? (o_lane + (uint32_t)dr * row) * 4u : kOffNone;
      buf_store_u32(ry, yo, __float_as_uint(v));
    }
  };

  // Head-major delta and its block prefix sums: lane j holds step l0 + j.
  const size_t row_bh = ((size_t)b * a.H + h) * a.Lp;
  const rsrc_t rd = make_rsrc(a.dlT + row_bh, (uint32_t)a.Lp * 4u);
  const rsrc_t rl = make_rsrc(a.lsT + row_bh, (uint32_t)a.Lp * 4u);
  auto load_dls = [&](int l0, float& d, float& ls) {
    d = __uint_as_float(buf_load_u32(rd, (uint32_t)(l0 + lane) * 4u));
    ls = __uint_as_float(buf_load_u32(rl, (uint32_t)(l0 + lane) * 4u));
  };

  u32x4 xr[2];
  BCRegs br, cr;
  float d, ls;
  load_x(lbeg, xr);
  load_bc_rows(a, a.B, b, lbeg, bco, br);
  if constexpr (Y) load_bc_rows(a, a.C, b, lbeg, bco, cr);
  load_dls(lbeg, d, ls);  // every wave loads them (no branch around loads); wave 0 uses them
  for (int l0 = lbeg; l0 < lend; l0 += kSub) {
    if constexpr (Y) finish();  // the previous block (its xbuf entries were written before the last barrier)
    store_x(xr);
    if constexpr (Y) {
      store_bc_rows<true, true>(br, Bs, BT);
      store_bc_rows<true, false>(cr, Cs, nullptr);
    } else {
      store_bc_rows<false, true>(br, nullptr, BT);
    }
    if (w == 0) {
      // e_i = exp(s_i), w_j = delta_j exp(s_last - s_j), decay = exp(s_last).
      const float last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ls), 63));
      s_dl[lane] = d;
      s_ls[lane] = ls;
      s_e[lane] = exp2_fast(ls);
      s_w[lane] = d * exp2_fast(last - ls);
      if (lane == 0) s_decay = exp2_fast(last);
      // Factors of exp(s_i - s_j) about the block's middle prefix sum, used
      // when the prefix sums fall (A <= 0) by less than 200 over the block.
      const float first = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ls), 0));
      const float mid = 0.5f * (first + last);
      s_ei[lane] = exp2_fast(ls - mid);
      s_fd[lane] = d * exp2_fast(mid - ls);
      if (lane == 0) s_factored = (first - last >= 0.f && first - last < 200.f) ? 1 : 0;
    }
    load_dls(l0 + kSub, d, ls);
    __syncthreads();

    if constexpr (Y) {
    // C S^T over this wave's state rows for both row tiles, the state as hi + lo.
    f32x16 yown = {}, yoth = {};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      auto slice = [&](auto s_tag) {
        constexpr int S = decltype(s_tag)::value;
        float v[8];
        acc_kslice<S>(st[t], v);
        u32x4 bh, bl;
        split8(v, bh, bl, dm);
        const int k0 = (2 * rt + t) * 32 + 16 * S + 8 * hf;
        const u32x4 c_own = *reinterpret_cast<const u32x4*>(&Cs[rt * 32 + lc][k0]);
        const u32x4 c_oth = *reinterpret_cast<const u32x4*>(&Cs[(1 - rt) * 32 + lc][k0]);
        yown = mfma(c_own, bh, yown);
        yown = mfma(c_own, bl, yown);
        yoth = mfma(c_oth, bh, yoth);
        yoth = mfma(c_oth, bl, yoth);
      };
      slice(std::integral_constant<int, 0>{});
      slice(std::integral_constant<int, 1>{});
    }

    // exp(s_i) on both row tiles' C S^T parts (registers 4k..4k+3 hold four
    // consecutive rows: one 16-byte read each), then the masked decay block.
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 eo = *reinterpret_cast<const f32x4*>(&s_e[rt * 32 + 8 * k + 4 * hf]);
      const f32x4 et = *reinterpret_cast<const f32x4*>(&s_e[(1 - rt) * 32 + 8 * k + 4 * hf]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        yown[4 * k + q] *= eo[q];
        yoth[4 * k + q] *= et[q];
      }
    }
    auto diag = [&](auto factored_tag) {
      constexpr bool F = decltype(factored_tag)::value;
      if (rt == 0) {
        diag_part<0, 0, 0, 2, F>(yown, Cs, Bs, xT, s_ls, s_dl, s_ei, s_fd, pt, dm);
        diag_part<1, 0, 0, 1, F>(yoth, Cs, Bs, xT, s_ls, s_dl, s_ei, s_fd, pt, dm);
      } else {
        diag_part<1, 1, 0, 2, F>(yown, Cs, Bs, xT, s_ls, s_dl, s_ei, s_fd, pt, dm);
        diag_part<1, 0, 1, 2, F>(yown, Cs, Bs, xT, s_ls, s_dl, s_ei, s_fd, pt, dm);
      }
    };
    if (__builtin_amdgcn_readfirstlane(s_factored))
      diag(std::true_type{});
    else
      diag(std::false_type{});
#pragma unroll
    for (int r = 0; r < 16; ++r) xbuf[w][r][lane] = yoth[r];
    // The next block's loads, issued once the products that need the most
    // registers are done (the block after the piece's last is read and
    // ignored; past L reads zero).
    load_x(l0 + kSub, xr);
    load_bc_rows(a, a.B, b, l0 + kSub, bco, br);
    load_bc_rows(a, a.C, b, l0 + kSub, bco, cr);
    yprev = yown;
    if constexpr (HAS_D) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int i0 = rt * 32 + 8 * g4 + 4 * hf;
        const u32x2 xx = *reinterpret_cast<const u32x2*>(&xT[tsw(p, i0)]);
        xprev[4 * g4] = bf16_lo(xx[0]);
        xprev[4 * g4 + 1] = bf16_hi(xx[0]);
        xprev[4 * g4 + 2] = bf16_lo(xx[1]);
        xprev[4 * g4 + 3] = bf16_hi(xx[1]);
      }
    }
    lprev = l0;
    } else {  // the next block's loads
      load_x(l0 + kSub, xr);
      load_bc_rows(a, a.B, b, l0 + kSub, bco, br);
    }

    // State after the block: S^T <- decay S^T + B^T (w o x).
    const float decay = s_decay;
#pragma unroll
    for (int t = 0; t < 2; ++t) st[t] *= decay;
#pragma unroll
    for (int kk = 0; kk < kSub / 16; ++kk) {
      const int j0 = kk * 16 + 8 * hf;
      const u32x4 xv = *reinterpret_cast<const u32x4*>(&xT[tsw(p, j0)]);
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&s_w[j0]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&s_w[j0 + 4]);
      const float v[8] = {bf16_lo(xv[0]) * w0[0], bf16_hi(xv[0]) * w0[1], bf16_lo(xv[1]) * w0[2],
                          bf16_hi(xv[1]) * w0[3], bf16_lo(xv[2]) * w1[0], bf16_hi(xv[2]) * w1[1],
                          bf16_lo(xv[3]) * w1[2], bf16_hi(xv[3]) * w1[3]};
      u32x4 bh, bl;
      split8(v, bh, bl, dm);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(&BT[tsw((2 * rt + t) * 32 + lc, j0)]);
        if constexpr (Y) {
          st[t] = mfma(av, bh, st[t]);
          st[t] = mfma(av, bl, st[t]);
        } else {  // S <- S + (w o x)^T B
          st[t] = mfma(bh, av, st[t]);
          st[t] = mfma(bl, av, st[t]);
        }
      }
    }
    // The state after a chunk (exact: the piece started from the exact
    // state).  A chunk ends with a block (chunks hold whole 64-step blocks);
    // the last chunk may stop at L, where the block's later steps (delta 0)
    // left the state unchanged.
    if (a.chunk_states && ((l0 + kSub) % a.Q == 0 || l0 + kSub >= lend)) {
      const int c = l0 / a.Q;
      float* cs = a.chunk_states + ((size_t)b * a.nchunks + c) * a.H * a.P * a.N +
                  (state_el(a, b, vh) - (size_t)b * a.H * a.P * a.N);
#pragma unroll
      for (int t = 0; t < 2; ++t) store_st(st[t], cs, 2 * rt + t);
    }
    __syncthreads();
  }
  if constexpr (Y) finish();
  if (a.h_last && piece == a.npieces - 1) {
    float* hl = a.h_last + state_el(a, b, vh);
#pragma unroll
    for (int t = 0; t < 2; ++t) store_st(st[t], hl, 2 * rt + t);
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Pieces per sequence: the scan kernel runs one workgroup per (batch, virtual
// head, piece), two per CU, so about five of them per CU over all pieces (and
// twice as many state-kernel workgroups), at most kMaxPieces and one per
// chunk; pieces hold whole chunks, cpp each.  Fewer, longer pieces leave the
// state kernel less to do (it runs every piece but the last) and each scan
// workgroup fewer pipeline fills; ten per CU measured 5% slower on a
// 160-stream, 64-chunk layer.  The environment variable
// MSS_SSD_CHUNKS_PER_PIECE, when it holds a positive count, overrides the
// piece length within the same limits (tuning and tests); the workspace
// query and the call must see the same value.
void ssd_pieces(int64_t batch, int64_t vheads, int64_t nchunks, int& npieces, int& cpp) {
  const int64_t streams = vheads * batch;
  int64_t np = (1280 + streams - 1) / streams;
  np = std::max<int64_t>(1, std::min<int64_t>({np, (int64_t)kMaxPieces, nchunks}));
  cpp = (int)((nchunks + np - 1) / np);
  if (const char* e = std::getenv("MSS_SSD_CHUNKS_PER_PIECE")) {
    const long v = std::strtol(e, nullptr, 10);
    const int64_t min_cpp = (nchunks + kMaxPieces - 1) / kMaxPieces;  // at most kMaxPieces pieces
    if (v >= 1) cpp = (int)std::max<int64_t>(min_cpp, std::min<int64_t>(v, nchunks));
  }
  npieces = (int)((nchunks + cpp - 1) / cpp);
}

struct SSDLayout {
  size_t dlT, lsT, pend, pstart, pdec, total;
};

SSDLayout ssd_layout(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t chunk) {
  const int64_t nchunks = (seqlen + chunk - 1) / chunk;
  const int64_t lp = (seqlen + kSub - 1) / kSub * kSub;
  const int64_t vheads = nheads * (headdim / kP);
  int np, cpp;
  ssd_pieces(batch, vheads, nchunks, np, cpp);
  const size_t state = (size_t)kP * kN * sizeof(float);
  SSDLayout l;
  l.dlT = 256;  // after the status word
  l.lsT = l.dlT + align256((size_t)batch * nheads * lp * sizeof(float));
  l.pend = l.lsT + align256((size_t)batch * nheads * lp * sizeof(float));
  l.pstart = l.pend + align256((size_t)batch * vheads * np * state);
  l.pdec = l.pstart + align256((size_t)batch * vheads * np * state);
  l.total = l.pdec + align256((size_t)batch * vheads * np * sizeof(float));
  return l;
}

}  // namespace

size_t ssd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                           int64_t dstate, int64_t chunk) {
  (void)ngroups;
  (void)dstate;
  return ssd_layout(batch, seqlen, nheads, headdim, chunk).total;
}

void ssd_delta_rows(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t chunk, size_t& dlT,
                    size_t& lsT) {
  const SSDLayout l = ssd_layout(batch, seqlen, nheads, headdim, chunk);
  dlT = l.dlT;
  lsT = l.lsT;
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
  a.batch = (int)p.batch;
  a.L = (int)p.seqlen;
  a.H = (int)p.nheads;
  a.G = (int)p.ngroups;
  a.Q = (int)p.chunk;
  a.P = (int)p.headdim;
  a.ph = (int)(p.headdim / kP);
  a.Hv = a.H * a.ph;
  a.N = (int)p.dstate;
  a.nchunks = (int)((p.seqlen + p.chunk - 1) / p.chunk);
  const int nsub = (a.L + kSub - 1) / kSub;
  a.Lp = nsub * kSub;
  const SSDLayout l = ssd_layout(p.batch, p.seqlen, p.nheads, p.headdim, p.chunk);
  char* ws = static_cast<char*>(p.workspace);
  a.status = reinterpret_cast<int*>(ws);
  a.dlT = reinterpret_cast<float*>(ws + l.dlT);
  a.lsT = reinterpret_cast<float*>(ws + l.lsT);
  a.pend = reinterpret_cast<float*>(ws + l.pend);
  a.pstart = reinterpret_cast<float*>(ws + l.pstart);
  a.pdec = reinterpret_cast<float*>(ws + l.pdec);
  ssd_pieces(a.batch, a.Hv, a.nchunks, a.npieces, a.cpp);
  hipLaunchKernelGGL(ssd_cumsum_kernel, dim3((unsigned)nsub, (unsigned)((a.H + 63) / 64), (unsigned)a.batch), dim3(256),
                     0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // States wider than 128 run as two 128-wide halves; the second adds its
  // part of y to the first's and applies D and the gate.
  const int halves = (a.N + kN - 1) / kN;
  for (int hv = 0; hv < halves; ++hv) {
    a.noff = hv * kN;
    a.accumulate = hv > 0 ? 1 : 0;
    const bool last = hv == halves - 1;
    // The last piece's end state is not needed (the scan kernel walks that
    // piece to the end), nor is any with a single piece.
    if (a.npieces > 1)
      hipLaunchKernelGGL(ssd_state_kernel, dim3((unsigned)(2 * a.Hv), (unsigned)a.batch, (unsigned)(a.npieces - 1)),
                         dim3(kTS), 0, stream, a);
    if (a.npieces > 1)
      hipLaunchKernelGGL(ssd_chain_kernel, dim3((unsigned)(kP * kN / 1024), (unsigned)a.Hv, (unsigned)a.batch),
                         dim3(256), 0, stream, a);
    const dim3 grid((unsigned)a.npieces * (unsigned)a.Hv * (unsigned)a.batch);
    const bool hz = last && a.z != nullptr, hd = last && a.D != nullptr;
    auto go = [&](auto accum_tag) {
      constexpr bool ACC = decltype(accum_tag)::value;
      if (hz && hd) hipLaunchKernelGGL((ssd_scan_kernel<true, true, ACC>), grid, dim3(kT), 0, stream, a);
      else if (hz) hipLaunchKernelGGL((ssd_scan_kernel<true, false, ACC>), grid, dim3(kT), 0, stream, a);
      else if (hd) hipLaunchKernelGGL((ssd_scan_kernel<false, true, ACC>), grid, dim3(kT), 0, stream, a);
      else hipLaunchKernelGGL((ssd_scan_kernel<false, false, ACC>), grid, dim3(kT), 0, stream, a);
    };
    if (a.y == nullptr)
      hipLaunchKernelGGL((ssd_scan_kernel<false, false, false, false>), grid, dim3(kT), 0, stream, a);
    else if (a.accumulate)
      go(std::true_type{});
    else
      go(std::false_type{});
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace mss
