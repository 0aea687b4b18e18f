// Selective scan forward (Mamba-1 selective SSM layer) for gfx950.
//
// What is computed (per batch b and channel d, see include/mambascan.h):
//   h[n] <- exp(delta*A[d,n]) * h[n] + delta*B[b,n,l]*u      (recurrence)
//   y    <- (sum_n C[b,n,l]*h[n] + D[d]*u) * silu(z)          (readout, skip, gate)
// following the discretised recurrence of "Mamba (deep learning)" (state-space
// paragraph: Abar = exp(Delta*A)) and "Mamba-1/2/3 visual guide" (section 1 SSM
// equation; section 2 selectivity table and block diagram).  The expanded state
// stays in registers (section 2 figure: many steps combined on-chip, only the
// outputs written back).
//
// Mapping on CDNA4.  One workgroup = 8 wave64s = one block of 64 channels of
// one batch row.  Lanes are channels; the d_state states are split across the
// 8 waves (SPW = ceil(N/8) states per wave), so 8 waves (2 per SIMD) share one
// channel block and each wave's sequential chain is 1/8 of the work.  Time is
// processed in tiles of 16 steps with one barrier per tile:
//   prologue (all 512 threads, one (channel, 2 steps) item each): widen u and
//     delta, x = delta*u and the decay table for the tile into LDS;
//   core (each wave, its SPW states, 16 sequential steps): B and C of the step
//     come in through SGPRs from a pre-transposed fp32 copy; partial readouts
//     go to LDS;
//   epilogue (all threads, same items as the prologue): sum the 8 partial
//     readouts in a fixed order, add D*u, gate with silu(z), store y.
// The prologue of tile k+1 and the epilogue of tile k run in the same loop
// iteration as the core of tile k; global loads are issued three tiles ahead.
//
// Decay.  Where every channel of the block has A[d,n] == (n+1)*A[d,0] (the
// S4D-real structure, checked on the device), the prologue computes one
// r = exp2(delta*A[d,0]*log2 e) per (d,l) and the start power r^(g*SPW+1) of
// each wave's states; the waves continue the power chain with multiplies.
// Elsewhere each wave evaluates exp2(delta*A[d,n]*log2 e) per state.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mss {
namespace {

constexpr int kWaves = 8;
constexpr int kLanes = 64;
constexpr int kThreads = kWaves * kLanes;
constexpr int kTile = 16;          // time steps per tile
constexpr int kBlk = kTile / 4;    // float4 blocks per tile
constexpr int kQMax = 2 + kWaves;  // LDS quantities per (d,l): x, r, 8 start powers
constexpr int kPrefetch = 3;       // tiles of global loads in flight

struct ScanArgs {
  const void* u;
  const void* delta;
  const float* A;
  const float* D;
  const void* z;
  const float* h0;
  void* y;
  float* h_last;
  const float* bc;     // [batch][8][lpad][2*SPW]: B then C of each wave's states, fp32
  const int* s4d_ok;   // [nblocks]
  int batch, dim, dstate, seqlen, lpad;
  int force_general;
};

// Raw (undecoded) loads of two consecutive steps of one row.
template <bool BF16>
struct Raw;
template <>
struct Raw<true> {
  uint32_t w;
};
template <>
struct Raw<false> {
  float2 w;
};

template <bool BF16, bool VEC>
__device__ __forceinline__ Raw<BF16> load_raw(const void* base, size_t row, int t, int L, bool ok) {
  Raw<BF16> r;
  if constexpr (BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + row;
    if (VEC) {
      r.w = (ok && t < L) ? *reinterpret_cast<const uint32_t*>(p + t) : 0u;  // L even: t+1 < L too
    } else {
      uint32_t lo = (ok && t < L) ? p[t] : 0u;
      uint32_t hi = (ok && t + 1 < L) ? p[t + 1] : 0u;
      r.w = lo | (hi << 16);
    }
  } else {
    const float* p = static_cast<const float*>(base) + row;
    if (VEC) {
      r.w = (ok && t < L) ? *reinterpret_cast<const float2*>(p + t) : make_float2(0.f, 0.f);
    } else {
      r.w.x = (ok && t < L) ? p[t] : 0.f;
      r.w.y = (ok && t + 1 < L) ? p[t + 1] : 0.f;
    }
  }
  return r;
}

__device__ __forceinline__ float2 decode(const Raw<true>& r) { return make_float2(bf16_lo(r.w), bf16_hi(r.w)); }
__device__ __forceinline__ float2 decode(const Raw<false>& r) { return r.w; }

template <bool BF16>
__device__ __forceinline__ void store_pair(void* base, size_t row, int t, int L, bool ok, float v0, float v1) {
  if (!ok || t >= L) return;
  if constexpr (BF16) {
    uint16_t* p = static_cast<uint16_t*>(base) + row;
    if (t + 1 < L && ((row + t) & 1) == 0) {
      *reinterpret_cast<uint32_t*>(p + t) = pack_bf16x2(v0, v1);
    } else {
      p[t] = f32_to_bf16(v0);
      if (t + 1 < L) p[t + 1] = f32_to_bf16(v1);
    }
  } else {
    float* p = static_cast<float*>(base) + row;
    if (t + 1 < L && ((row + t) & 1) == 0) {
      *reinterpret_cast<float2*>(p + t) = make_float2(v0, v1);
    } else {
      p[t] = v0;
      if (t + 1 < L) p[t + 1] = v1;
    }
  }
}

// LDS: per buffer, kQMax quantities x kBlk x 64 lanes x float4 (4 steps), and
// 8 waves x kBlk x 64 lanes x float4 of partial readouts.
constexpr int kQFloats = kQMax * kBlk * kLanes * 4;
constexpr int kPFloats = kWaves * kBlk * kLanes * 4;

__device__ __forceinline__ int q_off(int q, int blk, int lane) { return ((q * kBlk + blk) * kLanes + lane) * 4; }

template <bool BF16, int SPW, bool VEC>
__global__ void __launch_bounds__(kThreads, 1) scan_kernel(ScanArgs a) {
  __shared__ __attribute__((aligned(16))) float qbuf[2][kQFloats];
  __shared__ __attribute__((aligned(16))) float pbuf[2][kPFloats];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave id, uniform
  const int blk_id = blockIdx.x;
  const int b = blockIdx.y;
  const int c = blk_id * kLanes + lane;  // channel of this lane
  const bool cok = c < a.dim;
  const int L = a.seqlen, N = a.dstate;
  const size_t row = ((size_t)b * a.dim + (cok ? c : 0)) * (size_t)L;
  const bool s4d = !a.force_general && a.s4d_ok[blk_id] != 0;

  // Per-lane constants.
  const float a20 = cok ? a.A[(size_t)c * N] * kLog2e : 0.f;
  const float dskip = (a.D != nullptr && cok) ? a.D[c] : 0.f;
  float A2[SPW];
  float h[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int n = w * SPW + j;
    A2[j] = (cok && n < N) ? a.A[(size_t)c * N + n] * kLog2e : 0.f;
    h[j] = (a.h0 != nullptr && cok && n < N) ? a.h0[((size_t)b * a.dim + c) * N + n] : 0.f;
  }

  const int ntiles = (L + kTile - 1) / kTile;
  // Item of this thread in prologue/epilogue: channel `c`, steps t0 + 2w, t0 + 2w + 1.
  const int tt = 2 * w;

  Raw<BF16> ru[kPrefetch], rd[kPrefetch], rz[kPrefetch];
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) {
    const int t = k * kTile + tt;
    ru[k] = load_raw<BF16, VEC>(a.u, row, t, L, cok);
    rd[k] = load_raw<BF16, VEC>(a.delta, row, t, L, cok);
    if (a.z) rz[k] = load_raw<BF16, VEC>(a.z, row, t, L, cok);
  }

  float2 u_keep = make_float2(0.f, 0.f), z_keep = make_float2(0.f, 0.f);

  // Prologue of one tile from the oldest prefetched raw values into qbuf[buf].
  auto prologue = [&](int buf) {
    const float2 uu = decode(ru[0]);
    const float2 dd = decode(rd[0]);
    float* q = qbuf[buf];
    const int blk = tt >> 2, sub = tt & 3;
    const float2 x = make_float2(dd.x * uu.x, dd.y * uu.y);
    *reinterpret_cast<float2*>(&q[q_off(0, blk, lane) + sub]) = x;
    if (s4d) {
      const float2 r = make_float2(exp2_fast(dd.x * a20), exp2_fast(dd.y * a20));
      *reinterpret_cast<float2*>(&q[q_off(1, blk, lane) + sub]) = r;
      float2 step = r;  // r^SPW
#pragma unroll
      for (int j = 1; j < SPW; ++j) step = make_float2(step.x * r.x, step.y * r.y);
      float2 s = r;     // r^(g*SPW + 1)
#pragma unroll
      for (int g = 0; g < kWaves; ++g) {
        *reinterpret_cast<float2*>(&q[q_off(2 + g, blk, lane) + sub]) = s;
        s = make_float2(s.x * step.x, s.y * step.y);
      }
    } else {
      *reinterpret_cast<float2*>(&q[q_off(1, blk, lane) + sub]) = dd;
    }
    u_keep = uu;
    if (a.z) z_keep = decode(rz[0]);
  };

  // Rotate the prefetch ring and issue the loads for tile `tile`.
  auto advance = [&](int tile) {
#pragma unroll
    for (int k = 0; k + 1 < kPrefetch; ++k) {
      ru[k] = ru[k + 1];
      rd[k] = rd[k + 1];
      if (a.z) rz[k] = rz[k + 1];
    }
    const int t = tile * kTile + tt;
    ru[kPrefetch - 1] = load_raw<BF16, VEC>(a.u, row, t, L, cok);
    rd[kPrefetch - 1] = load_raw<BF16, VEC>(a.delta, row, t, L, cok);
    if (a.z) rz[kPrefetch - 1] = load_raw<BF16, VEC>(a.z, row, t, L, cok);
  };

  const float* bc_wave = a.bc + ((size_t)b * kWaves + w) * (size_t)a.lpad * (2 * SPW);

  // Core: this wave's SPW states over the 16 steps of one tile.  B and C of
  // four steps (4 * 2 * SPW floats) are fetched with wide scalar loads.
  auto core_tile = [&](auto guard_tag, int buf, int t0) {
    constexpr bool GUARD = decltype(guard_tag)::value;
    const float* q = qbuf[buf];
    float* pp = pbuf[buf];
    typedef float f4 __attribute__((ext_vector_type(4)));
    typedef const __attribute__((address_space(4))) f4* cf4_ptr;
    cf4_ptr bcs = (cf4_ptr)(bc_wave + (size_t)t0 * (2 * SPW));
#pragma unroll
    for (int blk = 0; blk < kBlk; ++blk) {
      f4 bcv[2 * SPW];  // 4 steps x (B[SPW], C[SPW])
#pragma unroll
      for (int i = 0; i < 2 * SPW; ++i) bcv[i] = bcs[blk * 2 * SPW + i];
      const float* bcf = reinterpret_cast<const float*>(bcv);
      const float4 xv = *reinterpret_cast<const float4*>(&q[q_off(0, blk, lane)]);
      const float4 rv = *reinterpret_cast<const float4*>(&q[q_off(1, blk, lane)]);
      float4 sv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s4d) sv = *reinterpret_cast<const float4*>(&q[q_off(2 + w, blk, lane)]);
      float part[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const float x = (&xv.x)[kk];
        const float r = (&rv.x)[kk];  // r (S4D) or delta (general)
        const float* bt = bcf + kk * 2 * SPW;
        float p = 0.f;
        if (!GUARD || t0 + blk * 4 + kk < L) {
          if (s4d) {
            float dec = (&sv.x)[kk];
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
              if (j > 0) dec *= r;
              h[j] = __builtin_fmaf(dec, h[j], x * bt[j]);
              p = __builtin_fmaf(bt[SPW + j], h[j], p);
            }
          } else {
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
              const float dec = exp2_fast(r * A2[j]);
              h[j] = __builtin_fmaf(dec, h[j], x * bt[j]);
              p = __builtin_fmaf(bt[SPW + j], h[j], p);
            }
          }
        }
        part[kk] = p;
      }
      *reinterpret_cast<float4*>(&pp[q_off(w, blk, lane)]) = make_float4(part[0], part[1], part[2], part[3]);
    }
  };

  prologue(0);
  float2 u_cur = u_keep, z_cur = z_keep;
  advance(kPrefetch);
  __syncthreads();

  for (int k = 0; k < ntiles; ++k) {
    const int buf = k & 1;
    const int t0 = k * kTile;
    if (k + 1 < ntiles) {
      prologue(buf ^ 1);
      advance(k + 1 + kPrefetch);
    }

    // ---- core: this wave's states over the 16 steps of tile k ----
    if (t0 + kTile <= L)
      core_tile(std::false_type{}, buf, t0);
    else
      core_tile(std::true_type{}, buf, t0);
    __syncthreads();

    // ---- epilogue of tile k: items (c, t0 + tt, t0 + tt + 1) ----
    {
      const float* pp = pbuf[buf];
      const int blk = tt >> 2, sub = tt & 3;
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int g = 0; g < kWaves; ++g) {
        const float2 v = *reinterpret_cast<const float2*>(&pp[q_off(g, blk, lane) + sub]);
        s0 += v.x;
        s1 += v.y;
      }
      float o0 = __builtin_fmaf(dskip, u_cur.x, s0);
      float o1 = __builtin_fmaf(dskip, u_cur.y, s1);
      if (a.z) {
        o0 *= silu(z_cur.x);
        o1 *= silu(z_cur.y);
      }
      store_pair<BF16>(a.y, row, t0 + tt, L, cok, o0, o1);
    }
    u_cur = u_keep;
    z_cur = z_keep;
  }

  if (a.h_last != nullptr && cok) {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int n = w * SPW + j;
      if (n < N) a.h_last[((size_t)b * a.dim + c) * N + n] = h[j];
    }
  }
}

// B, C [batch, N, L] (bf16 or fp32) -> fp32 [batch][8][lpad][2*SPW] with zero
// padding for n >= N and l >= L.  One thread per (b, wave group, l).
template <bool BF16, int SPW>
__global__ void bc_transpose_kernel(const void* __restrict__ B, const void* __restrict__ C,
                                    float* __restrict__ out, int batch, int N, int L, int lpad) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)batch * kWaves * lpad;
  if (idx >= total) return;
  const int l = (int)(idx % lpad);
  const int g = (int)((idx / lpad) % kWaves);
  const int b = (int)(idx / ((size_t)lpad * kWaves));
  float* o = out + idx * (2 * SPW);
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int n = g * SPW + j;
    float bv = 0.f, cv = 0.f;
    if (n < N && l < L) {
      const size_t off = ((size_t)b * N + n) * L + l;
      if (BF16) {
        bv = bf16_to_f32(static_cast<const uint16_t*>(B)[off]);
        cv = bf16_to_f32(static_cast<const uint16_t*>(C)[off]);
      } else {
        bv = static_cast<const float*>(B)[off];
        cv = static_cast<const float*>(C)[off];
      }
    }
    o[j] = bv;
    o[SPW + j] = cv;
  }
}

// s4d_ok[blk] = 1 when A[d,n] == (n+1)*A[d,0] (exactly, in fp32) for every
// channel d of the 64-channel block.  One wave per block.
__global__ void s4d_check_kernel(const float* __restrict__ A, int* __restrict__ ok_out, int dim, int N) {
  const int c = blockIdx.x * kLanes + threadIdx.x;
  bool ok = true;
  if (c < dim) {
    const float a0 = A[(size_t)c * N];
    for (int n = 1; n < N; ++n) ok = ok && (A[(size_t)c * N + n] == (float)(n + 1) * a0);
  }
  const bool all = __all(ok);
  if (threadIdx.x == 0) ok_out[blockIdx.x] = all ? 1 : 0;
}

int states_per_wave(int64_t N) { return N <= 8 ? 1 : N <= 16 ? 2 : N <= 32 ? 4 : 8; }
int64_t padded_len(int64_t L) { return (L + kTile - 1) / kTile * kTile; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <bool BF16, int SPW>
hipError_t launch_typed(const ScanParams& p, hipStream_t stream) {
  const int64_t lpad = padded_len(p.seqlen);
  const int nblocks = (int)((p.dim + kLanes - 1) / kLanes);
  char* ws = static_cast<char*>(p.workspace);
  float* bc = reinterpret_cast<float*>(ws);
  int* ok = reinterpret_cast<int*>(ws + align256((size_t)p.batch * kWaves * lpad * 2 * SPW * sizeof(float)));

  {
    const size_t total = (size_t)p.batch * kWaves * lpad;
    const unsigned grid = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL((bc_transpose_kernel<BF16, SPW>), dim3(grid), dim3(256), 0, stream, p.B, p.C, bc,
                       (int)p.batch, (int)p.dstate, (int)p.seqlen, (int)lpad);
  }
  hipLaunchKernelGGL(s4d_check_kernel, dim3(nblocks), dim3(kLanes), 0, stream, p.A, ok, (int)p.dim,
                     (int)p.dstate);

  ScanArgs a;
  a.u = p.u;
  a.delta = p.delta;
  a.A = p.A;
  a.D = p.D;
  a.z = p.z;
  a.h0 = p.h0;
  a.y = p.y;
  a.h_last = p.h_last;
  a.bc = bc;
  a.s4d_ok = ok;
  a.batch = (int)p.batch;
  a.dim = (int)p.dim;
  a.dstate = (int)p.dstate;
  a.seqlen = (int)p.seqlen;
  a.lpad = (int)lpad;
  a.force_general = p.force_general ? 1 : 0;
  const dim3 grid(nblocks, (unsigned)p.batch);
  if (p.seqlen % 2 == 0)
    hipLaunchKernelGGL((scan_kernel<BF16, SPW, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((scan_kernel<BF16, SPW, false>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const ScanParams& p, hipStream_t stream) {
  switch (states_per_wave(p.dstate)) {
    case 1: return launch_typed<BF16, 1>(p, stream);
    case 2: return launch_typed<BF16, 2>(p, stream);
    case 4: return launch_typed<BF16, 4>(p, stream);
    default: return launch_typed<BF16, 8>(p, stream);
  }
}

}  // namespace

size_t scan_workspace_bytes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen) {
  const int spw = states_per_wave(dstate);
  const int64_t lpad = padded_len(seqlen);
  const int64_t nblocks = (dim + kLanes - 1) / kLanes;
  return align256((size_t)batch * kWaves * lpad * 2 * spw * sizeof(float)) + align256((size_t)nblocks * sizeof(int));
}

hipError_t launch_scan(const ScanParams& p, hipStream_t stream) {
  return p.bf16 ? launch_dtype<true>(p, stream) : launch_dtype<false>(p, stream);
}

}  // namespace mss
