// The layer's short convolution before the forward: SiLU of a causal depthwise
// convolution over time, per channel, applied to q, k and v.
//
//   y[t, c] = silu(bias[c] + sum_{j<W} w[c, j] * x[t - (W-1) + j, c]),  silu(z) = z sigmoid(z)
//
// with tokens before the first token of t's sequence counting as zero (the
// left zero padding of W-1 tokens, taken per row, or per document of a packed
// row); W = 0 is SiLU alone.  Definition: hyper_parallel coverage page for
// context_parallel/kimi_delta_attention.py, `_run_causal_short_conv` and
// `_validate_layer_short_conv` (depthwise conv1d, stride 1, dilation 1, zero
// padding of kernel_size - 1, output cut to the sequence length, SiLU), and
// the forward of KimiDeltaAttentionUlyssesCP (SiLU alone without the
// convolution).
//
// HBM-bound streaming: every thread owns 16 bytes of channels (8 bf16 or 4
// fp32) over a run of kRun consecutive tokens and carries the previous W-1
// inputs in registers, so each input element is read once plus a halo of W-1
// rows per run; 64 lanes of a wave read 1 KiB of one token row.  One launch
// covers the three tensors (grid.y).
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kConvThreads = 256;
constexpr int kRun = 32;    // tokens per thread
constexpr int kGroup = 8;   // token rows loaded together

__device__ __forceinline__ void load16(const float* p, float* out) {
  const float4 v = *(const float4*)p;
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}
__device__ __forceinline__ void load16(const bf16* p, float* out) {
  const uint4 v = *(const uint4*)p;
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(u[i] << 16);
    out[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void store16(float* p, const float* v) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store16(bf16* p, const float* v) {
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
  *(uint4*)p = make_uint4(u[0], u[1], u[2], u[3]);
}

// z sigmoid(z) with the hardware exponential and reciprocal (each about 1 ulp
// in fp32; the result is rounded to the input dtype).  The matrix-core forward
// that convolves on load computes the same expression, so both agree bit for bit.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

// Sequence bounds of flat token t: [s0, s1) is the part of t's sequence from
// its first token on.  Packed rows search cu_seqlens (largest n with
// cu[n] <= t); malformed device offsets are clamped so that s0 <= t and
// s1 > t, which keeps every access inside the buffers.
struct SeqCursor {
  int64_t s0, s1;
  int n;
};

__device__ __forceinline__ SeqCursor seq_find(const ConvArgs& a, int64_t t, int64_t tot) {
  SeqCursor c;
  if (!a.cu) {
    c.s0 = t / a.T * a.T;
    c.s1 = c.s0 + a.T;
    c.n = 0;
    return c;
  }
  int lo = 0, hi = a.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  c.n = lo;
  const int64_t b0 = a.cu[lo], b1 = a.cu[lo + 1];
  c.s0 = b0 < 0 ? 0 : (b0 > t ? t : b0);
  c.s1 = b1 > t ? b1 : tot;
  return c;
}

// Move the cursor to the sequence that starts at t (t >= s1).
__device__ __forceinline__ void seq_advance(const ConvArgs& a, SeqCursor& c, int64_t t, int64_t tot) {
  if (!a.cu) {
    c.s0 = t;
    c.s1 = t + a.T;
    return;
  }
  while (c.n < a.N - 1 && a.cu[c.n + 1] <= t) ++c.n;
  const int64_t b1 = a.cu[c.n + 1];
  c.s0 = t;
  c.s1 = b1 > t ? b1 : tot;
}

template <typename T, int W>
__global__ __launch_bounds__(kConvThreads) void k_short_conv(ConvArgs a) {
  constexpr int NV = 16 / (int)sizeof(T);  // channels per thread
  constexpr int WT = W > 0 ? W : 1;
  const ConvTensor& z = a.t[blockIdx.y];
  const int nvec = z.C / NV;
  const int64_t gid = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
  const int64_t run = gid / nvec;
  const int cv = (int)(gid - run * nvec);
  const int64_t tot = (int64_t)a.B * a.T;
  const int64_t t0 = run * kRun;
  if (t0 >= tot) return;
  const int64_t C = z.C;
  const T* x = (const T*)z.x + (int64_t)cv * NV;
  T* y = (T*)z.y + (int64_t)cv * NV;

  float wt[WT][NV], bias[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int64_t c = (int64_t)cv * NV + e;
    bias[e] = (W > 0 && z.bias) ? z.bias[c] : 0.f;
#pragma unroll
    for (int j = 0; j < WT; ++j) wt[j][e] = W > 0 ? z.w[c * W + j] : 0.f;
  }

  SeqCursor sc = seq_find(a, t0, tot);
  // win[s-1]: input of token t-s (s = 1..W-1), zero before the sequence start
  float win[WT][NV];
#pragma unroll
  for (int s = 1; s < WT; ++s) {
    if (t0 - s >= sc.s0) {
      load16(x + (t0 - s) * C, win[s - 1]);
    } else {
#pragma unroll
      for (int e = 0; e < NV; ++e) win[s - 1][e] = 0.f;
    }
  }

  for (int g0 = 0; g0 < kRun; g0 += kGroup) {
    if (t0 + g0 >= tot) break;
    float xr[kGroup][NV];
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
      const int64_t t = t0 + g0 + r < tot ? t0 + g0 + r : tot - 1;
      load16(x + t * C, xr[r]);
    }
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
      const int64_t t = t0 + g0 + r;
      if (t >= tot) break;
      if (t >= sc.s1) {  // a new sequence starts at t: its padding is zero
        seq_advance(a, sc, t, tot);
#pragma unroll
        for (int s = 0; s < WT; ++s)
#pragma unroll
          for (int e = 0; e < NV; ++e) win[s][e] = 0.f;
      }
      float out[NV];
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        float acc;
        if (W == 0) {
          acc = xr[r][e];
        } else {
          acc = fmaf(wt[W - 1][e], xr[r][e], bias[e]);
#pragma unroll
          for (int s = 1; s < W; ++s) acc = fmaf(wt[W - 1 - s][e], win[s - 1][e], acc);
        }
        out[e] = silu(acc);
      }
      store16(y + t * C, out);
#pragma unroll
      for (int s = WT - 1; s >= 2; --s)
#pragma unroll
        for (int e = 0; e < NV; ++e) win[s - 1][e] = win[s - 2][e];
      if (W > 1)
#pragma unroll
        for (int e = 0; e < NV; ++e) win[0][e] = xr[r][e];
    }
  }
}

template <typename T>
hipError_t launch_typed(const ConvArgs& a, int W, dim3 grid, hipStream_t s) {
  switch (W) {
    case 0: hipLaunchKernelGGL((k_short_conv<T, 0>), grid, dim3(kConvThreads), 0, s, a); break;
    case 1: hipLaunchKernelGGL((k_short_conv<T, 1>), grid, dim3(kConvThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_short_conv<T, 2>), grid, dim3(kConvThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_short_conv<T, 3>), grid, dim3(kConvThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_short_conv<T, 4>), grid, dim3(kConvThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_short_conv(const ConvArgs& a, hipStream_t s) {
  const int64_t tot = (int64_t)a.B * a.T;
  if (tot == 0 || a.count == 0) return hipSuccess;
  const int nv = a.dtype == 1 ? 8 : 4;
  int64_t maxvec = 0;
  for (int i = 0; i < a.count; ++i) maxvec = a.t[i].C / nv > maxvec ? a.t[i].C / nv : maxvec;
  const int64_t runs = (tot + kRun - 1) / kRun;
  const int64_t blocks = (runs * maxvec + kConvThreads - 1) / kConvThreads;
  const dim3 grid((unsigned)blocks, (unsigned)a.count);
  return a.dtype == 1 ? launch_typed<bf16>(a, a.width, grid, s)
                      : launch_typed<float>(a, a.width, grid, s);
}

}  // namespace kda
