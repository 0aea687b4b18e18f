// Backward of the selective scan fed by its prologue (the short causal
// convolution forming u, softplus forming delta; see scan.hip's fused form).
//
// "Mamba (deep learning)" (paragraph on the block: a convolution in front of
// the SSM on the input branch) and "Mamba State-Space Models" (usage example,
// kernel size 4) give the prologue; the gradient is the chain rule through it
// around the scan's own gradient:
//   c = conv_b + sum_k w_k x[t-3+k] (zeros before step 0),  u = c or silu(c),
//   v = delta_raw + delta_bias,  delta = v or softplus(v);
//   dc = du silu'(c) (du without silu),  silu'(c) = s (1 + c (1 - s)),
//   s = sigmoid(c);  dv = ddelta sigmoid(v) (ddelta without softplus);
//   dx[s] = sum_k w_k dc[s+3-k] (terms past L dropped);
//   dconv_w[d,k] = sum_{b,t} dc[t] x[t-3+k];  dconv_b = sum dc;
//   ddelta_raw = dv;  ddelta_bias = sum dv.
// Passes: u and delta formed once in fp32 (they never exist outside the
// forward kernel, so the scan's gradient is taken at their fp32 values), the
// other [b, d, L] and [b, N, L] inputs widened to fp32, the scan's backward in
// fp32 (by slices of 32 states above 32), then the prologue's chain rule:
// one pass over the steps (dc, dx, dv, ddelta_raw) and one workgroup per
// channel for the tap and bias sums (a fixed order: bitwise repeatable).
// Gradients in the I/O type are rounded once.
//
// Workspace: a 256-byte head (word 0: the call's status), the scan backward's
// workspace, then the fp32 buffers of the layout below.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace mss {
namespace {

constexpr size_t kMaxFbGrid = 16384;
inline unsigned fb_grid(size_t items) {
  return (unsigned)std::max<size_t>(1, std::min<size_t>((items + 1023) / 1024, kMaxFbGrid));
}
inline size_t al256f(size_t x) { return (x + 255) & ~(size_t)255; }

__device__ __forceinline__ float ld_io(const void* p, size_t i, int bf16) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}
__device__ __forceinline__ void st_io(void* p, size_t i, float v, int bf16) {
  if (bf16) static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  else static_cast<float*>(p)[i] = v;
}
// The forward kernel's forms: sigmoid by the hardware exp2 and reciprocal,
// softplus(v) = max(v, 0) + log1p(exp(-|v|)) with log1p(e) taken as
// log(w) e / (w - 1), w = 1 + e rounded (e itself when w rounds to 1), so
// that u and delta here are bitwise those the forward formed.
__device__ __forceinline__ float sigmoid_f(float v) { return rcp_fast(1.0f + exp2_fast(-v * kLog2e)); }
__device__ __forceinline__ float softplus_fwd(float v) {
  constexpr float kLn2f = 0.6931471805599453f;
  const float e = exp2_fast(-fabsf(v) * kLog2e);
  const float w = 1.0f + e;
  const float l = (w == 1.0f) ? e : __builtin_amdgcn_logf(w) * kLn2f * (e * rcp_fast(w - 1.0f));
  return fmaxf(v, 0.f) + l;
}

// Groups of four consecutive elements: the per-element passes move 8 (bf16)
// or 16 (fp32) bytes per lane and access, where one element per lane left
// them far below the HBM rate.  V: the group is whole and starts at a
// multiple of 4 elements from a 16-byte-aligned base (one vector access);
// otherwise elements k < n are accessed one by one and the rest read as 0.
template <bool V>
__device__ __forceinline__ void ld4(const void* p, size_t i, int n, int bf16, float (&v)[4]) {
  if (V) {
    if (bf16) {
      const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
      v[0] = __uint_as_float(q.x << 16);
      v[1] = __uint_as_float(q.x & 0xffff0000u);
      v[2] = __uint_as_float(q.y << 16);
      v[3] = __uint_as_float(q.y & 0xffff0000u);
    } else {
      const float4 q = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
      v[0] = q.x;
      v[1] = q.y;
      v[2] = q.z;
      v[3] = q.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = k < n ? ld_io(p, i + k, bf16) : 0.f;
  }
}
template <bool V>
__device__ __forceinline__ void ld4f(const float* p, size_t i, int n, float (&v)[4]) {
  ld4<V>(p, i, n, 0, v);
}
template <bool V>
__device__ __forceinline__ void st4(void* p, size_t i, int n, int bf16, const float (&v)[4]) {
  if (V) {
    if (bf16) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = make_uint2(pack_bf16x2(v[0], v[1]),
                                                                            pack_bf16x2(v[2], v[3]));
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = make_float4(v[0], v[1], v[2], v[3]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < n) st_io(p, i + k, v[k], bf16);
  }
}

// The convolution's pre-activations at steps t0..t0+3 of a row from the
// window win[m] = x[t0-4+m] (m = 0..7; steps before 0 are skipped, as the
// filter sees zeros there).
__device__ __forceinline__ void conv4(const float (&win)[8], int t0, const float* w, float cb, float (&c)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float a = cb;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (t0 + k - 3 + q >= 0) a = __builtin_fmaf(w[q], win[k + 1 + q], a);
    c[k] = a;
  }
}

// x over steps t0-4..t0+3 of the row at base (t0 a multiple of 4, so the
// group before a non-first group is whole).
template <bool V>
__device__ __forceinline__ void x_window(const void* x, size_t base, int t0, int n, int bf16, float (&win)[8]) {
  float prev[4] = {0.f, 0.f, 0.f, 0.f}, cur[4];
  if (t0 > 0) ld4<V>(x, base + t0 - 4, 4, bf16, prev);
  ld4<V>(x, base + t0, n, bf16, cur);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    win[k] = prev[k];
    win[4 + k] = cur[k];
  }
}

// Grid of the per-row passes: groups of 4 steps of a row along x, rows along
// y (each loop strides over its grid dimension, so any size fits).
inline dim3 fb_grid2(size_t rows, int L) {
  const int groups = (L + 3) / 4;
  const unsigned gx = (unsigned)std::min<int64_t>(((int64_t)groups + 255) / 256, 16);
  const unsigned gy = (unsigned)std::max<size_t>(1, std::min<size_t>(rows, (size_t)(8192 / gx)));
  return dim3(gx, gy);
}

// u, delta in fp32 from x, delta_raw (four steps of one row per thread).
template <bool V>
__global__ void __launch_bounds__(256) fb_prologue(const void* __restrict__ x, const void* __restrict__ delta_raw,
                                                   const float* __restrict__ conv_w, const float* __restrict__ conv_b,
                                                   const float* __restrict__ delta_bias, float* __restrict__ u,
                                                   float* __restrict__ delta, size_t rows, int dim, int L, int silu_on,
                                                   int softplus_on, int bf16) {
  const int groups = (L + 3) / 4;
  for (size_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const int d = (int)(r % (size_t)dim);
    const float w[4] = {conv_w[4 * d], conv_w[4 * d + 1], conv_w[4 * d + 2], conv_w[4 * d + 3]};
    const float cb = conv_b ? conv_b[d] : 0.f, db = delta_bias ? delta_bias[d] : 0.f;
    const size_t base = r * (size_t)L;
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < groups; j += gridDim.x * blockDim.x) {
      const int t0 = 4 * j, n = std::min(4, L - t0);
      float win[8], c[4], v[4], uo[4], dl[4];
      x_window<V>(x, base, t0, n, bf16, win);
      conv4(win, t0, w, cb, c);
      ld4<V>(delta_raw, base + t0, n, bf16, v);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uo[k] = silu_on ? silu(c[k]) : c[k];
        const float vv = v[k] + db;
        dl[k] = softplus_on ? softplus_fwd(vv) : vv;
      }
      st4<V>(u, base + t0, n, 0, uo);
      st4<V>(delta, base + t0, n, 0, dl);
    }
  }
}

// Flat widening and narrowing, four elements per thread and step (the bases
// are 16-byte aligned; a partial last group goes element by element).
__global__ void __launch_bounds__(256) fb_to_f32(const void* __restrict__ src, float* __restrict__ dst, size_t n,
                                                 int bf16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
  for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    float v[4];
    if (i + 4 <= n) {
      ld4<true>(src, i, 4, bf16, v);
      st4<true>(dst, i, 4, 0, v);
    } else {
      const int m = (int)(n - i);
      ld4<false>(src, i, m, bf16, v);
      st4<false>(dst, i, m, 0, v);
    }
  }
}

__global__ void __launch_bounds__(256) fb_from_f32(const float* __restrict__ src, void* __restrict__ dst, size_t n,
                                                   int bf16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
  for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    float v[4];
    if (i + 4 <= n) {
      ld4f<true>(src, i, 4, v);
      st4<true>(dst, i, 4, bf16, v);
    } else {
      const int m = (int)(n - i);
      ld4f<false>(src, i, m, v);
      st4<false>(dst, i, m, bf16, v);
    }
  }
}

// dc = du silu'(c) (du itself without silu) into dc_out, dx[s] = sum_k w_k
// dc[s+3-k] (terms past L dropped), dv = ddelta sigmoid(v) in place of
// ddelta, and ddelta_raw = dv in the I/O type.  A thread's dx needs dc three
// steps into the next group: it forms those from du and x as that group's
// thread does (the same operations, so the same values).
template <bool V>
__global__ void __launch_bounds__(256) fb_chain(const void* __restrict__ x, const void* __restrict__ delta_raw,
                                                const float* __restrict__ conv_w, const float* __restrict__ conv_b,
                                                const float* __restrict__ delta_bias, const float* __restrict__ du,
                                                float* __restrict__ dc_out, float* __restrict__ dd_dv,
                                                void* __restrict__ ddelta_raw, void* __restrict__ dx, size_t rows,
                                                int dim, int L, int silu_on, int softplus_on, int bf16) {
  const int groups = (L + 3) / 4;
  for (size_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const int d = (int)(r % (size_t)dim);
    const float w[4] = {conv_w[4 * d], conv_w[4 * d + 1], conv_w[4 * d + 2], conv_w[4 * d + 3]};
    const float cb = conv_b ? conv_b[d] : 0.f, db = delta_bias ? delta_bias[d] : 0.f;
    const size_t base = r * (size_t)L;
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < groups; j += gridDim.x * blockDim.x) {
      const int t0 = 4 * j, n = std::min(4, L - t0);
      const int nn = t0 + 4 < L ? std::min(4, L - t0 - 4) : 0;  // steps of the next group
      const size_t i = base + t0;
      // g[m] = dc at step t0+m, m = 0..7 (0 past L)
      float g[8], a4[4], b4[4] = {0.f, 0.f, 0.f, 0.f};
      ld4f<V>(du, i, n, a4);
      if (nn > 0) {
        if (V) ld4f<true>(du, i + 4, 4, b4);
        else ld4f<false>(du, i + 4, nn, b4);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        g[k] = a4[k];
        g[4 + k] = b4[k];
      }
      if (silu_on) {
        // xw[m] = x at step t0-4+m, m = 0..11 (zeros outside the row)
        float xw[12], p4[4] = {0.f, 0.f, 0.f, 0.f}, c4[4], n4[4] = {0.f, 0.f, 0.f, 0.f};
        if (t0 > 0) ld4<V>(x, base + t0 - 4, 4, bf16, p4);
        ld4<V>(x, i, n, bf16, c4);
        if (nn > 0) {
          if (V) ld4<true>(x, i + 4, 4, bf16, n4);
          else ld4<false>(x, i + 4, nn, bf16, n4);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          xw[k] = p4[k];
          xw[4 + k] = c4[k];
          xw[8 + k] = n4[k];
        }
#pragma unroll
        for (int m = 0; m < 7; ++m) {
          float c = cb;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (t0 + m - 3 + q >= 0) c = __builtin_fmaf(w[q], xw[m + 1 + q], c);
          const float s = sigmoid_f(c);
          g[m] *= s * (1.0f + c * (1.0f - s));
        }
      }
      const float dcv[4] = {g[0], g[1], g[2], g[3]};
      st4<V>(dc_out, i, n, 0, dcv);
      float out[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (t0 + m + 3 - k < L) acc = __builtin_fmaf(w[k], g[m + 3 - k], acc);
        out[m] = acc;
      }
      st4<V>(dx, i, n, bf16, out);
      float dv[4];
      ld4f<V>(dd_dv, i, n, dv);
      if (softplus_on) {
        float v[4];
        ld4<V>(delta_raw, i, n, bf16, v);
#pragma unroll
        for (int k = 0; k < 4; ++k) dv[k] *= sigmoid_f(v[k] + db);
        st4<V>(dd_dv, i, n, 0, dv);
      }
      st4<V>(ddelta_raw, i, n, bf16, dv);
    }
  }
}

// One workgroup per channel d: dconv_w[d, k] = sum_{b,t} dc x[t-3+k],
// dconv_b[d] = sum dc, ddelta_bias[d] = sum dv; each thread sums fixed
// groups of four steps of every batch row, then a fixed tree over the
// threads.
template <bool V>
__global__ void __launch_bounds__(256) fb_channel_sums(const void* __restrict__ x, const float* __restrict__ dc,
                                                       const float* __restrict__ dv, float* __restrict__ dconv_w,
                                                       float* __restrict__ dconv_b, float* __restrict__ ddelta_bias,
                                                       int batch, int dim, int L, int bf16) {
  __shared__ float red[6][256];
  const int d = blockIdx.x;
  const int groups = (L + 3) / 4;
  float acc[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < batch; ++b) {
    const size_t base = ((size_t)b * dim + d) * (size_t)L;
    for (int j = threadIdx.x; j < groups; j += blockDim.x) {
      const int t0 = 4 * j, n = std::min(4, L - t0);
      float win[8], g[4], h[4];
      x_window<V>(x, base, t0, n, bf16, win);
      ld4f<V>(dc, base + t0, n, g);
      ld4f<V>(dv, base + t0, n, h);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m < n) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (t0 + m - 3 + k >= 0) acc[k] = __builtin_fmaf(g[m], win[m + 1 + k], acc[k]);
          acc[4] += g[m];
          acc[5] += h[m];
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 6; ++q) red[q][threadIdx.x] = acc[q];
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) {
#pragma unroll
      for (int q = 0; q < 6; ++q) red[q][threadIdx.x] += red[q][threadIdx.x + h];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) dconv_w[4 * d + k] = red[k][0];
    if (dconv_b) dconv_b[d] = red[4][0];
    if (ddelta_bias) ddelta_bias[d] = red[5][0];
  }
}

// Status: mode 0 clears the call's word, 1 copies the scan backward's into it.
__global__ void fb_status(int* __restrict__ head, const int* __restrict__ inner, int mode) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  head[0] = mode == 0 ? 0 : *inner;
}

struct FbLayout {
  size_t head, inner, u, delta, z, dy, B, C, du, dd, dz, dB, dC, total;
};

FbLayout fb_layout(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen) {
  const size_t bdl = (size_t)batch * dim * seqlen * 4;
  const size_t bnl = (size_t)batch * dstate * seqlen * 4;
  FbLayout l;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += al256f(bytes);
    return at;
  };
  l.head = take(256);
  l.inner = take(dstate > 32 ? scan_bwd_wide_workspace_bytes(batch, dim, seqlen)
                             : scan_bwd_workspace_bytes(batch, dim, dstate, seqlen));
  l.u = take(bdl);
  l.delta = take(bdl);
  l.z = take(bdl);
  l.dy = take(bdl);
  l.B = take(bnl);
  l.C = take(bnl);
  l.du = take(bdl);
  l.dd = take(bdl);
  l.dz = take(bdl);
  l.dB = take(bnl);
  l.dC = take(bnl);
  l.total = o;
  return l;
}

}  // namespace

size_t scan_fused_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen) {
  return fb_layout(batch, dim, dstate, seqlen).total;
}

hipError_t launch_scan_fused_bwd(const ScanFusedBwdParams& p, hipStream_t stream) {
  const FbLayout l = fb_layout(p.batch, p.dim, p.dstate, p.seqlen);
  char* ws = static_cast<char*>(p.workspace);
  auto fp = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const int bf16 = p.bf16 ? 1 : 0;
  const size_t rows = (size_t)p.batch * p.dim;
  const size_t bdl = rows * (size_t)p.seqlen;
  const size_t bnl = (size_t)p.batch * p.dstate * p.seqlen;
  const int dim = (int)p.dim, L = (int)p.seqlen;
  hipError_t err = hipSuccess;
  auto check = [&]() {
    err = hipGetLastError();
    return err == hipSuccess;
  };

  int* head = reinterpret_cast<int*>(ws + l.head);
  hipLaunchKernelGGL(fb_status, dim3(1), dim3(64), 0, stream, head, head, 0);
  // Whole groups of four steps start at 16-byte-aligned addresses when L is a
  // multiple of 4 (every buffer base is 16-byte aligned).
  const bool vec = L % 4 == 0;
  hipLaunchKernelGGL(vec ? fb_prologue<true> : fb_prologue<false>, fb_grid2(rows, L), dim3(256), 0, stream, p.x,
                     p.delta_raw, p.conv_w, p.conv_b, p.delta_bias, fp(l.u), fp(l.delta), rows, dim, L,
                     p.conv_silu ? 1 : 0, p.softplus ? 1 : 0, bf16);
  if (p.z) hipLaunchKernelGGL(fb_to_f32, dim3(fb_grid(bdl)), dim3(256), 0, stream, p.z, fp(l.z), bdl, bf16);
  hipLaunchKernelGGL(fb_to_f32, dim3(fb_grid(bdl)), dim3(256), 0, stream, p.dy, fp(l.dy), bdl, bf16);
  hipLaunchKernelGGL(fb_to_f32, dim3(fb_grid(bnl)), dim3(256), 0, stream, p.B, fp(l.B), bnl, bf16);
  hipLaunchKernelGGL(fb_to_f32, dim3(fb_grid(bnl)), dim3(256), 0, stream, p.C, fp(l.C), bnl, bf16);
  if (!check()) return err;

  ScanBwdParams q;
  q.fwd.u = fp(l.u);
  q.fwd.delta = fp(l.delta);
  q.fwd.A = p.A;
  q.fwd.B = fp(l.B);
  q.fwd.C = fp(l.C);
  q.fwd.D = p.D;
  q.fwd.z = p.z ? fp(l.z) : nullptr;
  q.fwd.h0 = p.h0;
  q.fwd.y = nullptr;
  q.fwd.h_last = nullptr;
  q.fwd.batch = p.batch;
  q.fwd.dim = p.dim;
  q.fwd.dstate = p.dstate;
  q.fwd.seqlen = p.seqlen;
  q.fwd.bf16 = false;
  q.fwd.force_general = p.force_general;
  q.fwd.workspace = ws + l.inner;
  q.dy = fp(l.dy);
  q.dh_last = p.dh_last;
  q.du = fp(l.du);
  q.ddelta = fp(l.dd);
  q.dA = p.dA;
  q.dB = fp(l.dB);
  q.dC = fp(l.dC);
  q.dD = p.dD;
  q.dz = p.z ? fp(l.dz) : nullptr;
  q.dh0 = p.dh0;
  err = p.dstate > 32 ? launch_scan_bwd_wide(q, stream) : launch_scan_bwd(q, stream);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(fb_status, dim3(1), dim3(64), 0, stream, head, reinterpret_cast<const int*>(ws + l.inner), 1);

  // dc goes where u was: u is read only by the scan's backward, done by now.
  hipLaunchKernelGGL(vec ? fb_chain<true> : fb_chain<false>, fb_grid2(rows, L), dim3(256), 0, stream, p.x,
                     p.delta_raw, p.conv_w, p.conv_b, p.delta_bias, fp(l.du), fp(l.u), fp(l.dd), p.ddelta_raw, p.dx,
                     rows, dim, L, p.conv_silu ? 1 : 0, p.softplus ? 1 : 0, bf16);
  hipLaunchKernelGGL(vec ? fb_channel_sums<true> : fb_channel_sums<false>, dim3((unsigned)p.dim), dim3(256), 0,
                     stream, p.x, fp(l.u), fp(l.dd), p.dconv_w, p.dconv_b, p.ddelta_bias, (int)p.batch, dim, L,
                     bf16);
  hipLaunchKernelGGL(fb_from_f32, dim3(fb_grid(bnl)), dim3(256), 0, stream, fp(l.dB), p.dB, bnl, bf16);
  hipLaunchKernelGGL(fb_from_f32, dim3(fb_grid(bnl)), dim3(256), 0, stream, fp(l.dC), p.dC, bnl, bf16);
  if (p.z) hipLaunchKernelGGL(fb_from_f32, dim3(fb_grid(bdl)), dim3(256), 0, stream, fp(l.dz), p.dz, bdl, bf16);
  check();
  return err;
}

}  // namespace mss
