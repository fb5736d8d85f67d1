// fp32 path of the KDA chunked forward.
//
// It serves fp32 inputs and every chunk size, and recomputes the chunk factors
// for the backward.  Three kernels, all fp32 arithmetic (for 64-token chunks
// the chunk kernel's off-diagonal Akk/Aqk blocks, the off-diagonal blocks of
// Tm and its W, U products run on fp32 matrix cores, v_mfma_f32_16x16x4f32;
// everything else on VALU):
//
//   1. k_prologue_valu   one wave per token-head: q^, k^ (L2 norm), the
//                        per-key-channel log-decay g from the raw gate logits,
//                        a_log and dt_bias, and beta = sigmoid(logit);
//   2. k_chunk_valu      one workgroup per chunk-head: the chunk-local factors
//                        of the WY/UT form (below);
//   3. k_state_valu      one workgroup per (sequence, head, column tile):
//                        the sequential pass over the sequence's chunks that
//                        carries the fp32 state and writes the output.
//
// Chunk algebra (derived from the token recurrence; the pages name the chunked
// kernel, chunk_kda, but print no algorithm).  For a chunk of L tokens entering
// with state S0, gamma = chunk-local inclusive cumulative sum of g:
//   Akk[r,i] = sum_c k^_rc k^_ic exp(gamma_rc - gamma_ic)       (i < r)
//   Aqk[r,i] = sum_c q^_rc k^_ic exp(gamma_rc - gamma_ic)       (i <= r)
//   Tm = (I + Diag(beta) Akk)^-1                                 (forward substitution)
//   W  = Tm Diag(beta) (K^ . exp(gamma)),   U = Tm Diag(beta) V
//   Delta = U - W S0
//   O     = scale (Q^ . exp(gamma)) S0 + scale Aqk Delta
//   S_L   = Diag(exp(gamma_L)) S0 + (K^ . exp(gamma_L - gamma))^T Delta
// All exponents above are <= 0 because g <= 0, so nothing overflows.
#include "kda_internal.h"

namespace kda {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
// The chunk-factor kernel's workgroup: its LDS (about 50 KB for C = 64) leaves
// room for three workgroups per CU, so 512 threads give each SIMD six waves.
constexpr int kChunkThreads = 512;
constexpr int kMaxD = 128;  // largest head dimension of the default instantiations
constexpr int kWideD = 256; // the wide instantiations (head dim 256, chunks of 16 or 32)

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ inline float softplus_f(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }
__device__ inline float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }

// In-kernel gate: g = -exp(a_log) softplus(x + dt_bias), or with a lower bound
// lb < 0: g = lb * sigmoid(exp(a_log) (x + dt_bias)) (gate 1) or the clamp
// g = max(lb, -exp(a_log) softplus(x + dt_bias)) (gate 2).  g is floored at -110:
// exp(-110) is already below the smallest fp32 denormal, so no decay factor
// representable in fp32 changes, and the chunk-local cumulative sums stay
// small enough for their differences to keep full precision.
constexpr float kGateFloor = -110.f;
__device__ inline float gate_value(float x, float A, int gate, float lb) {
  const float g = gate == 1 ? lb * sigmoid_f(A * x) : -A * softplus_f(x);
  return fmaxf(gate == 2 ? fmaxf(g, lb) : g, kGateFloor);
}

// Token-heads per wave in the prologue: a wave issues the loads of all of them
// before it uses any, so each wave keeps several rows in flight (the kernel is
// bound by the bytes in flight per CU, not by its arithmetic).
constexpr int kProTPW = 4;

template <typename Tin, int KM>
__global__ __launch_bounds__(kThreads) void k_prologue_valu(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ gate,
    const Tin* __restrict__ beta, const float* __restrict__ a_log,
    const float* __restrict__ dt_bias, int64_t n_th, int H, int HK, int K, int gate_form, float lb,
    float* __restrict__ qn, float* __restrict__ kn, float* __restrict__ g,
    float* __restrict__ bt, float* __restrict__ rqo, float* __restrict__ rko) {
  const int lane = threadIdx.x & 63;
  const int64_t th0 = ((int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * kProTPW;
  if (th0 >= n_th) return;
  constexpr int M = KM / 64;
  float vq[kProTPW][M], vk[kProTPW][M], vx[kProTPW][M], bl[kProTPW];
  // every load of the wave's token-heads is issued up front (past the end,
  // the last token-head is read again and nothing is stored)
#pragma unroll
  for (int t = 0; t < kProTPW; ++t) {
    const int64_t th = th0 + t < n_th ? th0 + t : n_th - 1;
    const int h = (int)(th % H);
    const int64_t base = th * K;  // value-head token-head (outputs, gate)
    // q and k of the key head this value head reads
    const int64_t kbase = ((th / H) * HK + h / (H / HK)) * K;
    bl[t] = load_f32(beta + th);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int c = lane + 64 * m < K ? lane + 64 * m : 0;
      vq[t][m] = load_f32(q + kbase + c);
      vk[t][m] = load_f32(k + kbase + c);
      vx[t][m] = load_f32(gate + base + c) + dt_bias[(int64_t)h * K + c];
    }
  }
#pragma unroll
  for (int t = 0; t < kProTPW; ++t) {
    const int64_t th = th0 + t;
    if (th >= n_th) break;
    const int h = (int)(th % H);
    const int64_t base = th * K;
    float ssq = 0.f, ssk = 0.f;
    const float A = expf(a_log[h]);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (lane + 64 * m >= K) break;
      ssq = fmaf(vq[t][m], vq[t][m], ssq);
      ssk = fmaf(vk[t][m], vk[t][m], ssk);
    }
    ssq = wave_sum(ssq);
    ssk = wave_sum(ssk);
    const float rq = 1.f / sqrtf(ssq + 1e-6f), rk = 1.f / sqrtf(ssk + 1e-6f);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int c = lane + 64 * m;
      if (c >= K) break;
      qn[base + c] = vq[t][m] * rq;
      kn[base + c] = vk[t][m] * rk;
      g[base + c] = gate_value(vx[t][m], A, gate_form, lb);
    }
    if (lane == 0) {
      bt[th] = sigmoid_f(bl[t]);
      if (rqo) {
        rqo[th] = rq;
        rko[th] = rk;
      }
    }
  }
}

// One workgroup per chunk-head (flattened j*H + h).  The decay factors use the
// hardware exponential (__expf, about one ulp; all arguments are <= 0).  gamma's rows are padded
// to K+1 floats: the pairwise products read gamma of row i with lanes over i.
template <typename Tin, int C, int KM>
__global__ __launch_bounds__(kChunkThreads) void k_chunk_valu(FwdArgs a) {
  constexpr int kThreads = kChunkThreads;  // the loops below stride by the workgroup
  const int H = a.H, K = a.K, V = a.V;
  const int64_t wid = blockIdx.x;
  const int j = (int)(wid / H), h = (int)(wid % H);
  if (j >= *a.nt_dev) return;
  const int tid = threadIdx.x;
  const int tok0 = a.chunk_tok[j], L = a.chunk_len[j];

  __shared__ float sG[C][KM + 1];  // gamma, later X = beta k^ exp(gamma)
  __shared__ float sA[C][C + 1];   // Akk, then Tm in place
  __shared__ float sB[C];
  __shared__ float sGL[KM];     // gamma_L, the chunk's last row of gamma
  __shared__ float sDg[2][C == 64 ? C : 1];  // halves of the diagonal Aqk sums
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  auto tok_off = [&](int r) { return ((int64_t)(tok0 + r) * H + h); };
  const int64_t chb = (int64_t)j * H + h;  // chunk-head index

  // gamma: chunk-local inclusive cumsum; rows >= L repeat gamma_{L-1}.  The
  // chunk's g values reach LDS first, every thread issuing all of its 16-byte
  // loads before the first store (one memory latency), then each channel's
  // thread adds down its column in LDS.  Loads here and below read a clamped,
  // valid address and select zero afterwards, so none sits in a branch of its
  // own waiting for its data.
  for (int p0 = 0; p0 < C * K; p0 += 16 * kThreads) {
    f32x4 gv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + 4 * (tid + u * kThreads), r = p / K, c = p % K;
      const bool in = p < C * K && r < L;
      const f32x4 x = *(const f32x4*)(a.g + (in ? tok_off(r) * K + c : tok_off(0) * K));
      gv[u] = in ? x : zero4;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + 4 * (tid + u * kThreads);
      if (p < C * K)
#pragma unroll
        for (int e = 0; e < 4; ++e) sG[p / K][p % K + e] = gv[u][e];
    }
  }
  for (int r = tid; r < C; r += kThreads) {
    const float x = a.bt[tok_off(r < L ? r : 0)];
    sB[r] = r < L ? x : 0.f;
  }
  __syncthreads();
  for (int c = tid; c < K; c += kThreads) {
    float acc = 0.f;
    for (int r = 0; r < C; ++r) {
      acc += sG[r][c];
      sG[r][c] = acc;
    }
    sGL[c] = acc;
    a.gL[chb * K + c] = __expf(acc);
  }
  __syncthreads();

  float* Aqk = (float*)a.Aqk + chb * C * C;
  if constexpr (C == 64) {
    // Off-diagonal 16 x 16 blocks (R > I) on fp32 matrix cores: with the
    // per-channel reference gamma_ref = gamma_{16R-1} (the last row before block
    // R), e^{gamma_r - gamma_i} = e^{gamma_r - gamma_ref} e^{gamma_ref - gamma_i},
    // both factors <= 1 for r >= 16R > i, so the decayed products become
    //   Akk_RI = (K^_R . e^{gamma_R - gamma_ref}) (K^_I . e^{gamma_ref - gamma_I})^T
    // (and Aqk with Q^_R), one wave per block, lane l holding A[l%16][l/16],
    // B[l/16][l%16] and D[4(l/16)+e][l%16] (v_mfma_f32_16x16x4f32).  The four
    // diagonal blocks keep the per-pair sums; rows past the chunk end are zero.
    const int w = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    if (w < 6) {
      const int R = w < 1 ? 1 : w < 3 ? 2 : 3, I = w - R * (R - 1) / 2;
      const int r = 16 * R + ln, i = 16 * I + ln;   // this lane's A row and B column
      const bool rin = r < L, iin = i < L;
      // Lane group lg takes the channels [lg K/4, (lg + 1) K/4): its k-step s
      // is channel lg K/4 + s, so each lane reads 16-byte pieces of its rows,
      // the next piece in flight while the current one is multiplied.
      const int KQ = K / 4, c0 = KQ * lg;
      const float* kr = a.kn + tok_off(rin ? r : 0) * K + c0;
      const float* qr = a.qn + tok_off(rin ? r : 0) * K + c0;
      const float* ki = a.kn + tok_off(iin ? i : 0) * K + c0;
      f32x4 ak = zero4, aq = zero4;
      f32x4 nk = *(const f32x4*)kr, nq = *(const f32x4*)qr, ni = *(const f32x4*)ki;
      for (int s0 = 0; s0 < KQ; s0 += 4) {
        const f32x4 k4 = nk, q4 = nq, i4 = ni;
        const int sn = s0 + 4 < KQ ? s0 + 4 : s0;
        nk = *(const f32x4*)(kr + sn);
        nq = *(const f32x4*)(qr + sn);
        ni = *(const f32x4*)(ki + sn);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = c0 + s0 + e;
          const float gref = sG[16 * R - 1][c];
          const float er = __expf(sG[r][c] - gref), ei = __expf(gref - sG[i][c]);
          const float xk = rin ? k4[e] * er : 0.f, xq = rin ? q4[e] * er : 0.f;
          const float yk = iin ? i4[e] * ei : 0.f;
          ak = __builtin_amdgcn_mfma_f32_16x16x4f32(xk, yk, ak, 0, 0, 0);
          aq = __builtin_amdgcn_mfma_f32_16x16x4f32(xq, yk, aq, 0, 0, 0);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ro = 16 * R + 4 * lg + e, io = 16 * I + ln, pp = ro * C + io;
        const bool in = ro < L;
        sA[ro][io] = in ? ak[e] : 0.f;
        Aqk[pp] = in ? a.scale * aq[e] : 0.f;
        if (a.Akk_out) a.Akk_out[chb * C * C + pp] = in ? ak[e] : 0.f;
      }
    } else {
      // The 64 diagonal Aqk elements (decay 1): lane r takes row r, wave 6 the
      // first half of the channels and wave 7 the second; the two partial sums
      // wait in sDg until the solve below adds them.
      const int r = lane, c0 = (w - 6) * (K / 2);
      const float* kr = a.kn + tok_off(r < L ? r : 0) * K + c0;
      const float* qr = a.qn + tok_off(r < L ? r : 0) * K + c0;
      float aqk = 0.f;
      f32x4 nk = *(const f32x4*)kr, nq = *(const f32x4*)qr;
      for (int c = 0; c < K / 2; c += 4) {
        const f32x4 k4 = nk, q4 = nq;
        const int cn = c + 4 < K / 2 ? c + 4 : c;
        nk = *(const f32x4*)(kr + cn);
        nq = *(const f32x4*)(qr + cn);
#pragma unroll
        for (int e = 0; e < 4; ++e) aqk = fmaf(q4[e], k4[e], aqk);
      }
      sDg[w - 6][r] = aqk;
      if (w == 6) {
        sA[r][r] = 0.f;
        if (a.Akk_out) a.Akk_out[chb * C * C + r * C + r] = 0.f;
      }
    }
    // Diagonal blocks: the 4 x 120 strictly lower pairs, one per thread, rows
    // read in 16-byte pieces, the next piece in flight.
    static_assert(kThreads >= 4 * 120, "one thread per diagonal-block pair");
    if (tid < 4 * 120) {
      const int bk = tid / 120, q = tid % 120;   // q = rl (rl - 1) / 2 + il, il < rl
      int rl = (int)((sqrtf(8.f * q + 1.f) + 1.f) * 0.5f);
      while (rl * (rl - 1) / 2 > q) --rl;
      while ((rl + 1) * rl / 2 <= q) ++rl;
      const int il = q - rl * (rl - 1) / 2;
      const int r = 16 * bk + rl, i = 16 * bk + il, pp = r * C + i;
      float akk = 0.f, aqk = 0.f;
      if (r < L) {
        const float* kr = a.kn + tok_off(r) * K;
        const float* qr = a.qn + tok_off(r) * K;
        const float* ki = a.kn + tok_off(i) * K;
        f32x4 nk = *(const f32x4*)kr, nq = *(const f32x4*)qr, ni = *(const f32x4*)ki;
        for (int c = 0; c < K; c += 4) {
          const f32x4 k4 = nk, q4 = nq, i4 = ni;
          const int cn = c + 4 < K ? c + 4 : c;
          nk = *(const f32x4*)(kr + cn);
          nq = *(const f32x4*)(qr + cn);
          ni = *(const f32x4*)(ki + cn);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float d = __expf(sG[r][c + e] - sG[i][c + e]);
            const float kd = i4[e] * d;
            akk = fmaf(k4[e], kd, akk);
            aqk = fmaf(q4[e], kd, aqk);
          }
        }
      }
      sA[r][i] = akk;
      Aqk[pp] = (r < L) ? a.scale * aqk : 0.f;
      if (a.Akk_out) a.Akk_out[chb * C * C + pp] = akk;
    }
    // above the diagonal: zero
    for (int pp = tid; pp < C * C; pp += kThreads) {
      const int r = pp / C, i = pp % C;
      if (i > r) {
        sA[r][i] = 0.f;
        Aqk[pp] = 0.f;
        if (a.Akk_out) a.Akk_out[chb * C * C + pp] = 0.f;
      }
    }
    __syncthreads();
  } else {
  float* Aqk = (float*)a.Aqk + chb * C * C;
  for (int p = tid; p < C * C; p += kThreads) {
    const int r = p / C, i = p % C;
    float akk = 0.f, aqk = 0.f;
    if (r < L && i <= r) {
      const float* kr = a.kn + tok_off(r) * K;
      const float* qr = a.qn + tok_off(r) * K;
      const float* ki = a.kn + tok_off(i) * K;
      for (int c = 0; c < K; ++c) {
        const float d = __expf(sG[r][c] - sG[i][c]);
        const float kd = ki[c] * d;
        akk = fmaf(kr[c], kd, akk);
        aqk = fmaf(qr[c], kd, aqk);
      }
    }
    sA[r][i] = (i < r) ? akk : 0.f;
    Aqk[p] = (i <= r && r < L) ? a.scale * aqk : 0.f;
    if (a.Akk_out) a.Akk_out[chb * C * C + p] = (i < r) ? akk : 0.f;
  }
  __syncthreads();

  }
  // Tm = (I + Diag(beta) Akk)^-1 in 16 x 16 blocks.  Diagonal blocks: lane s of
  // wave b solves column s of block b by forward substitution (independent
  // lanes, no barriers).  Off-diagonal blocks, block row by block row:
  // Tm_RI = -Tm_RR Diag(beta_R) sum_{I <= J < R} Akk_RJ Tm_JI.
  {
    constexpr int NB = C / 16;
    __shared__ float sM[NB > 1 ? NB - 1 : 1][16][17];
    const int wv = tid >> 6, ln = tid & 63;
    if constexpr (C == 64) {
      if (wv == 4) Aqk[ln * C + ln] = (ln < L) ? a.scale * (sDg[0][ln] + sDg[1][ln]) : 0.f;
    }
    float col[16];
    if (wv < NB && ln < 16) {
      const int o = 16 * wv;
      // col[u] is 0 for u < s, so every lane may sum from u = 0 (fixed
      // register indices, the same sums)
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < t; ++u) acc = fmaf(sA[o + t][o + u], col[u], acc);
        col[t] = t == ln ? 1.f : (t > ln ? -sB[o + t] * acc : 0.f);
      }
    }
    __syncthreads();
    if (wv < NB && ln < 16)
#pragma unroll
      for (int t = 0; t < 16; ++t) sA[16 * wv + t][16 * wv + ln] = col[t];
    __syncthreads();
    for (int R = 1; R < NB; ++R) {
      if constexpr (C == 64) {
        // On fp32 matrix cores, wave I < R taking block I (lane l holds
        // A[l%16][l/16], B[l/16][l%16] and D[4(l/16)+e][l%16] of each
        // 16 x 16 x 4 step): first M_I, then Tm_RI = -(Tm_RR Diag(beta_R)) M_I,
        // summed over all 16 columns of Tm_RR (zero above its diagonal).
        const int lq = ln & 15, lg = ln >> 4;
        if (wv < R) {
          f32x4 acc = zero4;
          for (int u0 = 16 * wv; u0 < 16 * R; u0 += 4)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[16 * R + lq][u0 + lg], sA[u0 + lg][16 * wv + lq],
                                                       acc, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) sM[wv][4 * lg + e][lq] = acc[e];
        }
        __syncthreads();
        if (wv < R) {
          f32x4 acc = zero4;
#pragma unroll
          for (int u0 = 0; u0 < 16; u0 += 4)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(
                sA[16 * R + lq][16 * R + u0 + lg] * sB[16 * R + u0 + lg], sM[wv][u0 + lg][lq], acc, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) sA[16 * R + 4 * lg + e][16 * wv + lq] = -acc[e];
        }
        __syncthreads();
      } else {
      // M_I = sum_{I <= J < R} Akk_RJ Tm_JI for every I < R
      for (int e = tid; e < R * 256; e += kThreads) {
        const int I = e >> 8, t = (e >> 4) & 15, sc = e & 15;
        float acc = 0.f;
        for (int u = 16 * I; u < 16 * R; ++u) acc = fmaf(sA[16 * R + t][u], sA[u][16 * I + sc], acc);
        sM[I][t][sc] = acc;
      }
      __syncthreads();
      for (int e = tid; e < R * 256; e += kThreads) {
        const int I = e >> 8, t = (e >> 4) & 15, sc = e & 15;
        float acc = 0.f;
        for (int u = 0; u <= t; ++u)
          acc = fmaf(sA[16 * R + t][16 * R + u] * sB[16 * R + u], sM[I][u][sc], acc);
        sA[16 * R + t][16 * I + sc] = -acc;
      }
      __syncthreads();
      }
    }
    // strictly upper blocks of Tm are zero
    for (int e = tid; e < C * C; e += kThreads) {
      const int r = e / C, i = e % C;
      if ((i >> 4) > (r >> 4)) sA[r][i] = 0.f;
    }
    __syncthreads();
  }
  if (a.Tm_out)
    for (int p = tid; p < C * C; p += kThreads) a.Tm_out[chb * C * C + p] = sA[p / C][p % C];

  // Qt = scale q^ exp(gamma), Kb = k^ exp(gamma_L - gamma) and, in gamma's
  // place, X = beta k^ exp(gamma).  Each thread owns 16-byte pieces of rows
  // (no other thread reads gamma there; gamma_L comes from sGL) and issues
  // every load before its first store.
  float* Qt = (float*)a.Qt + chb * C * K;
  float* Kb = (float*)a.Kb + chb * C * K;
  {
    constexpr int NP = (C * KM / 4 + kThreads - 1) / kThreads;
    f32x4 q4[NP], k4[NP];
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int p = 4 * (tid + u * kThreads), r = p / K, c = p % K;
      const int64_t off = (p < C * K && r < L) ? tok_off(r) * K + c : tok_off(0) * K;
      q4[u] = *(const f32x4*)(a.qn + off);
      k4[u] = *(const f32x4*)(a.kn + off);
    }
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int p = 4 * (tid + u * kThreads), r = p / K, c = p % K;
      if (p >= C * K) break;
      const bool in = r < L;
      f32x4 qt, kb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float gm = sG[r][c + e], eg = __expf(gm);
        qt[e] = in ? a.scale * q4[u][e] * eg : 0.f;
        kb[e] = in ? k4[u][e] * __expf(sGL[c + e] - gm) : 0.f;
        sG[r][c + e] = in ? sB[r] * k4[u][e] * eg : 0.f;
      }
      *(f32x4*)(Qt + p) = qt;
      *(f32x4*)(Kb + p) = kb;
    }
  }
  __syncthreads();
  // W = Tm X, U = Tm Diag(beta) V   (Tm lower triangular with unit diagonal).
  // A thread's elements share one column (c = tid % D, rows tid / D + (256/D) m):
  // that column of X and of Diag(beta) V is read into registers once.
  float* W = (float*)a.W + chb * C * K;
  // Tm (lower triangular, in sA) times the C x D matrix in sG, written to out
  // [C][D]: for 64-token chunks on fp32 matrix cores, one 16 x 16 output tile
  // per accumulator, k-steps up to the tile's diagonal block.
  auto tm_product = [&](float* out, int D) {
    const int w = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int nct = D / 16;
    for (int t = w; t < (C / 16) * nct; t += kThreads / 64) {
      const int rt = t / nct, ct = t % nct;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int i0 = 0; i0 < 16 * (rt + 1); i0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[16 * rt + ln][i0 + lg], sG[i0 + lg][16 * ct + ln],
                                                   acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) out[(int64_t)(16 * rt + 4 * lg + e) * D + 16 * ct + ln] = acc[e];
    }
  };
  if constexpr (C == 64) {
    tm_product(W, K);
  } else {
    const int c = tid % K, r0 = tid / K, rs = kThreads / K;
    float xc[C];
#pragma unroll
    for (int i = 0; i < C; ++i) xc[i] = sG[i][c];
    for (int r = r0; r < C; r += rs) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < C; ++i) acc = (i <= r) ? fmaf(sA[r][i], xc[i], acc) : acc;
      W[(int64_t)r * K + c] = acc;
    }
  }
  float* U = (float*)a.U + chb * C * V;
  // Diag(beta) V to LDS in X's place (every load issued before the first
  // store), then U's rows read it from there
  const Tin* v = (const Tin*)a.v;
  constexpr int NV = (C * KM + kThreads - 1) / kThreads;
  float vv[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int p = tid + u * kThreads, i = p / V;
    const bool in = p < C * V && i < L;
    const float x = load_f32(v + (in ? tok_off(i) * V + p % V : tok_off(0) * V));
    vv[u] = in ? x : 0.f;
  }
  __syncthreads();  // X is no longer read
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int p = tid + u * kThreads, i = p / V;
    if (p < C * V) sG[i][p % V] = i < L ? sB[i] * vv[u] : 0.f;
  }
  __syncthreads();
  if constexpr (C == 64) {
    tm_product(U, V);
  } else {
    const int c = tid % V, r0 = tid / V, rs = kThreads / V;
    for (int r = r0; r < C; r += rs) {
      float acc = 0.f;
      for (int i = 0; i <= r; ++i) acc = fmaf(sA[r][i], sG[i][c], acc);
      U[(int64_t)r * V + c] = acc;
    }
  }
}

// One workgroup per (sequence n, head h, tile of VT state columns).  Columns
// [0, V) are the value columns of the state; in summary mode columns
// [V, V+K) carry the transition (its values are zero, it starts as I).
// Each chunk's operands (W, Qt, Kbar, Aqk, the tile's U columns, gL) are first
// copied into LDS with coalesced 16-byte loads; the products then read LDS
// only, 4 channels (or rows) per step.
template <typename Tin, int C, int KD, int VT, bool SUM>
__global__ __launch_bounds__(kThreads) void k_state_valu(FwdArgs a) {
  static_assert(VT == 32 && kThreads == 256, "thread layouts below");
  constexpr int NR = C / 8;            // rows per thread in the row phases
  constexpr int TPC = kThreads / KD;   // threads per channel in the state update
  constexpr int JPT = VT / TPC;        // columns per thread in the state update
  constexpr int KP = KD + 4, CP = C + 4;  // padded rows: the two half-waves hit other banks
  const int H = a.H, V = a.V;
  const int ncols = SUM ? V + KD : V;
  const int ntile = ncols / VT;
  const int64_t wid = blockIdx.x;
  const int tile = (int)(wid % ntile);
  const int64_t nh = wid / ntile;
  const int h = (int)(nh % H), n = (int)(nh / H);
  const int col0 = tile * VT;
  const int tid = threadIdx.x;
  constexpr bool out = !SUM;  // summary mode writes no output

  __shared__ __attribute__((aligned(16))) float sS[KD][VT];
  __shared__ __attribute__((aligned(16))) float sD[C][VT];
  __shared__ __attribute__((aligned(16))) float sW[C][KP];
  __shared__ __attribute__((aligned(16))) float sQ[C][KP];
  __shared__ __attribute__((aligned(16))) float sKb[C][KD];
  __shared__ __attribute__((aligned(16))) float sA[C][CP];
  __shared__ __attribute__((aligned(16))) float sU[C][VT];
  __shared__ float sG[KD];

  const int64_t sbase = ((int64_t)n * H + h) * KD * V;
  for (int e = tid; e < KD * VT; e += kThreads) {
    const int c = e / VT, jj = e % VT, col = col0 + jj;
    float s;
    if (col < V)
      s = (a.init && out) ? a.init[sbase + (int64_t)c * V + col] : 0.f;
    else
      s = (c == col - V) ? 1.f : 0.f;
    sS[c][jj] = s;
  }
  const int jj = tid % VT, rg = tid / VT;           // row phases: column jj, rows rg + 8m
  const int cs = tid / TPC, j0 = (tid % TPC) * JPT;  // state update: channel cs, columns j0..
  const int jc0 = a.seq_chunk0[n], jc1 = a.seq_chunk0[n + 1];
  for (int j = jc0; j < jc1; ++j) {
    const int64_t chb = (int64_t)j * H + h;
    const float4* W = (const float4*)((const float*)a.W + chb * C * KD);
    const float4* Qt = (const float4*)((const float*)a.Qt + chb * C * KD);
    const float4* Kb = (const float4*)((const float*)a.Kb + chb * C * KD);
    const float4* Aqk = (const float4*)((const float*)a.Aqk + chb * C * C);
    const float* U = (const float*)a.U + chb * C * V;
    const int tok0 = a.chunk_tok[j], L = a.chunk_len[j];
    __syncthreads();  // the previous chunk is done with every LDS operand
    {
      constexpr int N4 = C * KD / 4 / kThreads;
      float4 wv[N4], qv[N4];
#pragma unroll
      for (int u = 0; u < N4; ++u) {
        wv[u] = W[tid + kThreads * u];
        if constexpr (out) qv[u] = Qt[tid + kThreads * u];
      }
#pragma unroll
      for (int u = 0; u < N4; ++u) {
        const int idx = tid + kThreads * u, r = idx / (KD / 4), c = 4 * (idx % (KD / 4));
        *(float4*)&sW[r][c] = wv[u];
        if constexpr (out) *(float4*)&sQ[r][c] = qv[u];
      }
      constexpr int NA = (C * C / 4 + kThreads - 1) / kThreads;
      constexpr int NU = (C * VT / 4 + kThreads - 1) / kThreads;
      float4 kv[N4], av[NA], uv[NU];
#pragma unroll
      for (int u = 0; u < N4; ++u) kv[u] = Kb[tid + kThreads * u];
#pragma unroll
      for (int u = 0; u < NA; ++u) {
        const int idx = tid + kThreads * u;
        av[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (out)
          if (idx < C * C / 4) av[u] = Aqk[idx];
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int idx = tid + kThreads * u, r = idx / (VT / 4), c = col0 + 4 * (idx % (VT / 4));
        uv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (idx < C * VT / 4 && c < V) uv[u] = *(const float4*)(U + (int64_t)r * V + c);
      }
      const float gl = tid < KD ? a.gL[chb * KD + tid] : 0.f;
#pragma unroll
      for (int u = 0; u < N4; ++u) {
        const int idx = tid + kThreads * u, r = idx / (KD / 4), c = 4 * (idx % (KD / 4));
        *(float4*)&sKb[r][c] = kv[u];
      }
#pragma unroll
      for (int u = 0; u < NA; ++u) {
        const int idx = tid + kThreads * u, r = idx / (C / 4), c = 4 * (idx % (C / 4));
        if constexpr (out)
          if (idx < C * C / 4) *(float4*)&sA[r][c] = av[u];
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int idx = tid + kThreads * u, r = idx / (VT / 4), c = 4 * (idx % (VT / 4));
        if (idx < C * VT / 4) *(float4*)&sU[r][c] = uv[u];
      }
      if (tid < KD) sG[tid] = gl;
    }
    __syncthreads();
    // X = W S and Y = Qt S for rows rg + 8m, column jj; Delta = U - X
    float xs[NR], ys[NR];
#pragma unroll
    for (int m = 0; m < NR; ++m) xs[m] = ys[m] = 0.f;
    for (int c = 0; c < KD; c += 4) {
      const float s0 = sS[c][jj], s1 = sS[c + 1][jj], s2 = sS[c + 2][jj], s3 = sS[c + 3][jj];
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        const int r = rg + 8 * m;
        const float4 w4 = *(const float4*)&sW[r][c];
        xs[m] = fmaf(w4.x, s0, fmaf(w4.y, s1, fmaf(w4.z, s2, fmaf(w4.w, s3, xs[m]))));
        if constexpr (out) {
          const float4 q4 = *(const float4*)&sQ[r][c];
          ys[m] = fmaf(q4.x, s0, fmaf(q4.y, s1, fmaf(q4.z, s2, fmaf(q4.w, s3, ys[m]))));
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NR; ++m) sD[rg + 8 * m][jj] = sU[rg + 8 * m][jj] - xs[m];
    __syncthreads();
    // O = Qt S + Aqk Delta  (scale folded into Qt and Aqk; Aqk is zero above the diagonal)
    if constexpr (out) {
      Tin* o = (Tin*)a.o;
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        const int r = rg + 8 * m;
        if (r >= L) continue;
        float acc = ys[m];
        for (int i = 0; i <= r; i += 4) {
          const float4 a4 = *(const float4*)&sA[r][i];
          acc = fmaf(a4.x, sD[i][jj], fmaf(a4.y, sD[i + 1][jj],
                fmaf(a4.z, sD[i + 2][jj], fmaf(a4.w, sD[i + 3][jj], acc))));
        }
        store_as(o + ((int64_t)(tok0 + r) * H + h) * V + col0 + jj, acc);
      }
    }
    __syncthreads();
    // S = Diag(gL) S + Kb^T Delta for channel cs, columns j0 .. j0 + JPT - 1
    {
      float acc[JPT];
      const float gc = sG[cs];
#pragma unroll
      for (int t = 0; t < JPT; t += 4) {
        const float4 s4 = *(const float4*)&sS[cs][j0 + t];
        acc[t] = gc * s4.x; acc[t + 1] = gc * s4.y; acc[t + 2] = gc * s4.z; acc[t + 3] = gc * s4.w;
      }
      for (int r = 0; r < L; ++r) {
        const float kb = sKb[r][cs];
#pragma unroll
        for (int t = 0; t < JPT; t += 4) {
          const float4 d4 = *(const float4*)&sD[r][j0 + t];
          acc[t] = fmaf(kb, d4.x, acc[t]);
          acc[t + 1] = fmaf(kb, d4.y, acc[t + 1]);
          acc[t + 2] = fmaf(kb, d4.z, acc[t + 2]);
          acc[t + 3] = fmaf(kb, d4.w, acc[t + 3]);
        }
      }
#pragma unroll
      for (int t = 0; t < JPT; t += 4)
        *(float4*)&sS[cs][j0 + t] = make_float4(acc[t], acc[t + 1], acc[t + 2], acc[t + 3]);
    }
  }
  __syncthreads();
  for (int e = tid; e < KD * VT; e += kThreads) {
    const int c = e / VT, jj2 = e % VT, col = col0 + jj2;
    if constexpr (out) {
      if (a.fin) a.fin[sbase + (int64_t)c * V + col] = sS[c][jj2];
    } else if (col < V) {
      a.state_ext[sbase + (int64_t)c * V + col] = sS[c][jj2];
    } else {
      a.transition[((int64_t)n * H + h) * KD * KD + (int64_t)c * KD + (col - V)] = sS[c][jj2];
    }
  }
}

template <typename Tin, int C>
hipError_t run_prep(const FwdArgs& a, hipStream_t s) {
  const int64_t n_th = (int64_t)a.B * a.T * a.H;
  if (n_th > 0) {
    const int64_t per_block = (kThreads / 64) * kProTPW;
    const int64_t blocks = (n_th + per_block - 1) / per_block;
    hipLaunchKernelGGL((k_prologue_valu<Tin, kMaxD>), dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.gate, (const Tin*)a.beta,
                       a.a_log, a.dt_bias, n_th, a.H, a.HK, a.K, a.gate_form, a.lb, a.qn, a.kn, a.g, a.bt,
                       a.rq, a.rk);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  if (a.NT > 0) {
    hipLaunchKernelGGL((k_chunk_valu<Tin, C, kMaxD>), dim3((unsigned)((int64_t)a.NT * a.H)),
                       dim3(kChunkThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  return hipSuccess;
}

// KM: the widest head dimension the instantiation handles (kMaxD, or kWideD
// for head dim 256 with chunks of 16 or 32, whose state pass stages fit LDS)
template <typename Tin, int C, int KM>
hipError_t run(const FwdArgs& a, hipStream_t s) {
  const int64_t n_th = (int64_t)a.B * a.T * a.H;
  mark(a, kStagePrologue, 0, s);
  if (n_th > 0) {
    const int64_t per_block = (kThreads / 64) * kProTPW;
    const int64_t blocks = (n_th + per_block - 1) / per_block;
    hipLaunchKernelGGL((k_prologue_valu<Tin, KM>), dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.gate, (const Tin*)a.beta,
                       a.a_log, a.dt_bias, n_th, a.H, a.HK, a.K, a.gate_form, a.lb, a.qn, a.kn, a.g, a.bt,
                       a.rq, a.rk);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  mark(a, kStagePrologue, 1, s);
  mark(a, kStageChunk, 0, s);
  if (a.NT > 0) {
    hipLaunchKernelGGL((k_chunk_valu<Tin, C, KM>), dim3((unsigned)((int64_t)a.NT * a.H)),
                       dim3(kChunkThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  mark(a, kStageChunk, 1, s);
  constexpr int VT = 32;
  const int ncols = a.summary ? a.V + a.K : a.V;
  const int64_t wgs = (int64_t)a.N * a.H * (ncols / VT);
  mark(a, kStageState, 0, s);
  if (wgs > 0 && (a.summary || a.fin || a.NT > 0)) {
    auto launch = [&](auto kd, auto sum) {
      hipLaunchKernelGGL((k_state_valu<Tin, C, decltype(kd)::value, VT, decltype(sum)::value>),
                         dim3((unsigned)wgs), dim3(kThreads), 0, s, a);
    };
    using K64 = std::integral_constant<int, 64>;
    using K128 = std::integral_constant<int, 128>;
    using K256 = std::integral_constant<int, 256>;
    using S0 = std::false_type;
    using S1 = std::true_type;
    if constexpr (KM == kWideD) {
      if (a.K == 256) a.summary ? launch(K256{}, S1{}) : launch(K256{}, S0{});
      else if (a.K == 64) a.summary ? launch(K64{}, S1{}) : launch(K64{}, S0{});
      else a.summary ? launch(K128{}, S1{}) : launch(K128{}, S0{});
    } else {
      if (a.K == 64) a.summary ? launch(K64{}, S1{}) : launch(K64{}, S0{});
      else a.summary ? launch(K128{}, S1{}) : launch(K128{}, S0{});
    }
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  mark(a, kStageState, 1, s);
  return hipSuccess;
}

template <typename Tin>
hipError_t run_c(const FwdArgs& a, hipStream_t s) {
  if (a.K > kMaxD || a.V > kMaxD) {
    // head dim 256: chunks of 16 or 32 only (the host rejects 64)
    if (a.C == 16) return run<Tin, 16, kWideD>(a, s);
    return run<Tin, 32, kWideD>(a, s);
  }
  switch (a.C) {
    case 16: return run<Tin, 16, kMaxD>(a, s);
    case 32: return run<Tin, 32, kMaxD>(a, s);
    default: return run<Tin, 64, kMaxD>(a, s);
  }
}

}  // namespace

hipError_t launch_valu_path(const FwdArgs& a, hipStream_t s) {
  return a.dtype == 0 ? run_c<float>(a, s) : run_c<bf16>(a, s);
}

// The prologue and chunk-factor kernels alone (no state pass): the
// recomputation the backward starts from.
hipError_t launch_valu_prep(const FwdArgs& a, hipStream_t s) {
  if (a.dtype == 0) {
    switch (a.C) {
      case 16: return run_prep<float, 16>(a, s);
      case 32: return run_prep<float, 32>(a, s);
      default: return run_prep<float, 64>(a, s);
    }
  }
  switch (a.C) {
    case 16: return run_prep<bf16, 16>(a, s);
    case 32: return run_prep<bf16, 32>(a, s);
    default: return run_prep<bf16, 64>(a, s);
  }
}

}  // namespace kda
