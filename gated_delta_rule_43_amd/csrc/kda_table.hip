// Chunk table and state-summary application kernels.
//
// Chunk table: every sequence (a row b, or a document [cu[n], cu[n+1]) of the
// single packed row) is cut into chunks of C tokens that start at the
// sequence's own first token, so a document that ends mid-chunk ends with a
// partial chunk and the next document starts a fresh one (document resets of
// cu_seqlens, NeMo AutoModel page "nemo_automodel.components.models.kimi_k3.cp",
// module introduction and `segment_cu_seqlens`).
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kTableThreads = 1024;

// Inclusive block scan over one int per thread (Hillis-Steele in LDS).
template <bool kMax>
__device__ int block_scan(int x, int* sh) {
  const int t = threadIdx.x;
  sh[t] = x;
  __syncthreads();
  for (int off = 1; off < kTableThreads; off <<= 1) {
    int y = (t >= off) ? sh[t - off] : (kMax ? INT32_MIN : 0);
    __syncthreads();
    if (t >= off) sh[t] = kMax ? max(sh[t], y) : sh[t] + y;
    __syncthreads();
  }
  int r = sh[t];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kTableThreads) void k_chunk_table(const int32_t* __restrict__ cu, int N,
                                                               int B, int T, int C, int nt_max,
                                                               int32_t* __restrict__ tok,
                                                               int32_t* __restrict__ len,
                                                               int32_t* __restrict__ seq0,
                                                               int32_t* __restrict__ nt_out,
                                                               int32_t* __restrict__ zero_out,
                                                               int32_t* __restrict__ cseq) {
  __shared__ int sh[kTableThreads];
  const int tid = threadIdx.x;
  if (zero_out && tid == 0) *zero_out = 0;  // counter the later kernels append to
  if (cu == nullptr) {
    const int nc = (T + C - 1) / C;
    for (int n = tid; n <= B; n += kTableThreads) seq0[n] = n * nc;
    for (int j = tid; j < B * nc; j += kTableThreads) {
      int b = j / nc, t0 = (j - b * nc) * C;
      tok[j] = b * T + t0;
      len[j] = min(C, T - t0);
      if (cseq) cseq[j] = b;
    }
    if (tid == 0) *nt_out = B * nc;
    return;
  }
  // Document n spans [m(n), m(n+1)) with m(0) = 0, m(N) = T and, in between,
  // m(e) = clamp(max(cu[0..e]), 0, T): equal to cu for valid offsets, and always
  // monotone and inside the row, so no chunk can leave the buffers.
  const int per = (N + kTableThreads - 1) / kTableThreads;
  const int d0 = min(tid * per, N), d1 = min(d0 + per, N);
  int lmax = INT32_MIN;
  for (int e = d0; e < d1; ++e) lmax = max(lmax, (int)cu[e]);
  const int incl_max = block_scan<true>(lmax, sh);
  sh[tid] = incl_max;
  __syncthreads();
  const int excl_max = tid > 0 ? sh[tid - 1] : INT32_MIN;
  __syncthreads();
  auto bound = [&](int e, int pm) { return e == 0 ? 0 : (e == N ? T : min(max(pm, 0), T)); };

  int cnt = 0;
  if (d0 < d1) {
    int pm = max(excl_max, (int)cu[d0]);
    int m_prev = bound(d0, pm);
    for (int e = d0 + 1; e <= d1; ++e) {
      pm = max(pm, (int)cu[e]);
      const int m = bound(e, pm);
      cnt += (m - m_prev + C - 1) / C;
      m_prev = m;
    }
  }
  const int incl_cnt = block_scan<false>(cnt, sh);
  if (d0 < d1) {
    int j = incl_cnt - cnt;
    int pm = max(excl_max, (int)cu[d0]);
    int m_prev = bound(d0, pm);
    for (int e = d0 + 1; e <= d1; ++e) {
      pm = max(pm, (int)cu[e]);
      const int m = bound(e, pm);
      seq0[e - 1] = min(j, nt_max);
      for (int t0 = m_prev; t0 < m; t0 += C, ++j) {
        if (j < nt_max) {
          tok[j] = t0;
          len[j] = min(C, m - t0);
          if (cseq) cseq[j] = e - 1;
        }
      }
      m_prev = m;
    }
  }
  if (tid == kTableThreads - 1) {
    seq0[N] = min(incl_cnt, nt_max);
    *nt_out = min(incl_cnt, nt_max);
  }
}

__global__ __launch_bounds__(256) void k_apply_summary(int64_t total, int K, int V,
                                                       const float* __restrict__ E,
                                                       const float* __restrict__ P,
                                                       const float* __restrict__ S0,
                                                       float* F) {
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int64_t kv = (int64_t)K * V;
  const int64_t bh = idx / kv;
  const int i = (int)((idx / V) % K);
  const int jv = (int)(idx % V);
  float acc = E[idx];
  if (S0) {
    const float* Pr = P + bh * K * K + (int64_t)i * K;
    const float* Sc = S0 + bh * kv + jv;
    for (int c = 0; c < K; ++c) acc = fmaf(Pr[c], Sc[(int64_t)c * V], acc);
  }
  F[idx] = acc;
}

}  // namespace

hipError_t launch_chunk_table(const FwdArgs& a, hipStream_t s) {
  mark(a, kStageTable, 0, s);
  hipLaunchKernelGGL(k_chunk_table, dim3(1), dim3(kTableThreads), 0, s, a.cu, a.N, a.B, a.T, a.C,
                     a.NT, a.chunk_tok, a.chunk_len, a.seq_chunk0, a.nt_dev, a.exact_count,
                     a.chunk_seq);
  hipError_t e = hipGetLastError();
  mark(a, kStageTable, 1, s);
  return e;
}

hipError_t launch_apply_summary(int B, int H, int K, int V, const float* E, const float* P,
                                const float* S0, float* F, hipStream_t s) {
  int64_t total = (int64_t)B * H * K * V;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_apply_summary, dim3((unsigned)blocks), dim3(256), 0, s, total, K, V, E, P,
                     S0, F);
  return hipGetLastError();
}

}  // namespace kda
