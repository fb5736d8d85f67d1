// The gated output norm after the forward, o_norm(o, output_gate) of the layer:
// per (token, value head) row of V values,
//
//     y[v] = o[v] / sqrt(mean_v(o^2) + eps) * weight[v] * act(gate[v]),
//     act = sigmoid or SiLU (x sigmoid(x)),
//
// with the mean reduced in fp32.  Source: the hyper_parallel coverage page for
// context_parallel/kimi_delta_attention.py (the forward of
// KimiDeltaAttentionUlyssesCP: the output gate projection reshaped to
// [B, T, HV, V], then o_norm(output, output_gate)) and the torchtitan PR #4025
// review (the model's RMSNorm reduces in fp32).  The pages print neither the
// norm nor the gate's activation; this is the gated RMSNorm reading.
//
// HBM-bound: every lane holds 16 bytes of one row (8 bf16 or 4 fp32 values)
// for kNormRows rows; the V / 8 (or V / 4) lanes of a row sum their squares
// with xor shuffles; the gate's sigmoid uses the hardware exponential and
// reciprocal (about one ulp each).
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kNormThreads = 256;
constexpr int kNormRows = 4;  // rows per thread

template <typename T> __device__ __forceinline__ void ld16(const T* p, float* out);
template <> __device__ __forceinline__ void ld16<float>(const float* p, float* out) {
  const float4 v = *(const float4*)p;
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}
template <> __device__ __forceinline__ void ld16<bf16>(const bf16* p, float* out) {
  const uint4 v = *(const uint4*)p;
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(u[i] << 16);
    out[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void st16(float* p, const float* v) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st16(bf16* p, const float* v) {
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
  *(uint4*)p = make_uint4(u[0], u[1], u[2], u[3]);
}

template <typename T, int V, int ACT>
__global__ __launch_bounds__(kNormThreads) void k_gated_rms_norm(NormArgs a) {
  constexpr int NV = 16 / (int)sizeof(T), LPR = V / NV;  // values per lane, lanes per row
  constexpr int RPB = kNormThreads / LPR;                 // rows per block and round
  static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "a row's lanes sit in one wave");
  const int part = threadIdx.x % LPR;
  const int64_t row0 = (int64_t)blockIdx.x * RPB * kNormRows + threadIdx.x / LPR;
  // all of a thread's rows are loaded before any arithmetic; rows past the end
  // read row 0 and store nothing (whole row groups stay together for the shuffles)
  float x[kNormRows][NV], g[kNormRows][NV];
#pragma unroll
  for (int k = 0; k < kNormRows; ++k) {
    const int64_t row = row0 + (int64_t)k * RPB;
    const int64_t off = (row < a.rows ? row : 0) * V + part * NV;
    ld16((const T*)a.o + off, x[k]);
    ld16((const T*)a.gate + off, g[k]);
  }
  float w[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) w[e] = a.w ? a.w[part * NV + e] : 1.f;
#pragma unroll
  for (int k = 0; k < kNormRows; ++k) {
    const int64_t row = row0 + (int64_t)k * RPB;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < NV; ++e) ss = fmaf(x[k][e], x[k][e], ss);
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float inv = 1.f / sqrtf(ss / V + a.eps);
    float y[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const float s = __builtin_amdgcn_rcpf(1.f + __expf(-g[k][e]));  // sigmoid
      const float act = ACT == 0 ? s : g[k][e] * s;
      y[e] = x[k][e] * inv * w[e] * act;
    }
    if (row < a.rows) st16((T*)a.y + row * V + part * NV, y);
  }
}

template <typename T, int V>
hipError_t launch_v(const NormArgs& a, dim3 grid, hipStream_t s) {
  if (a.act == 0) hipLaunchKernelGGL((k_gated_rms_norm<T, V, 0>), grid, dim3(kNormThreads), 0, s, a);
  else hipLaunchKernelGGL((k_gated_rms_norm<T, V, 1>), grid, dim3(kNormThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_rms_norm(const NormArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  const int nv = a.dtype == 1 ? 8 : 4;
  const int64_t rows_per_block = (int64_t)(kNormThreads / (a.V / nv)) * kNormRows;
  const dim3 grid((unsigned)((a.rows + rows_per_block - 1) / rows_per_block));
  if (a.dtype == 1) {
    if (a.V == 64) return launch_v<bf16, 64>(a, grid, s);
    return a.V == 128 ? launch_v<bf16, 128>(a, grid, s) : launch_v<bf16, 256>(a, grid, s);
  }
  if (a.V == 64) return launch_v<float, 64>(a, grid, s);
  return a.V == 128 ? launch_v<float, 128>(a, grid, s) : launch_v<float, 256>(a, grid, s);
}

}  // namespace kda
