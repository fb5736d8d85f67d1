// Backward of the KDA chunked forward: gradients of
//     L = sum(d_o * o) + sum(d_final * final_state)
// for q, k, v, the gate logits, the beta logits, a_log, dt_bias and the
// initial state, through the in-kernel L2 norm, gate and beta sigmoid.  What is
// differentiated: the chunk_kda call that the torchtitan PR #4025 commit note
// tests forward and backward together, whose state gradient the hyper_parallel
// coverage page routes between slices (the backward of _RecvKDAInitialState).
//
// Plain VALU fp32 arithmetic for both input dtypes.  The forward's chunk
// factors are recomputed first (the VALU prologue and chunk kernels, which
// here also keep Akk and Tm); then, per chunk of L rows entering with state
// S0 and with Q~ = q^ e^gamma, K~ = k^ e^gamma, Kbar = k^ e^(gamma_L - gamma),
// Aqk_s = scale Aqk, Qt_s = scale Q~ (the forward's stored operands):
//
//   forward state pass     S0 per chunk, Delta = U - W S0, S <- e^gamma_L S + Kbar^T Delta
//   reverse state pass     dS_L per chunk (the gradient of the state leaving it),
//                          dDelta = Aqk_s^T dO + Kbar dS_L,
//                          dS0 = Qt_s^T dO + e^gamma_L dS_L - W^T dDelta
//   chunk-local gradients  dW = -dDelta S0^T; Y = dW K~^T + dDelta V^T (lower);
//                          dT = Y Diag(beta) (strictly lower); dN = -Tm^T dT Tm^T;
//                          dAkk = Diag(beta) dN; dbeta = diag(Tm^T Y) + rowsum(dN . Akk);
//                          dV = Diag(beta) Tm^T dDelta; P = scale dO Delta^T (lower);
//                          then q^, k^, gamma through Q~ S0, Kbar, K~ and the two
//                          pairwise products Akk, Aqk (exp(gamma_r - gamma_i) per pair,
//                          never a factor larger than one), gamma -> g by a reverse
//                          cumulative sum, and g through the gate;
//   reductions             dq, dk: sum over the value heads that share a key head,
//                          then the L2 norm's Jacobian; da_log, ddt_bias: sums over
//                          chunks in a fixed order (deterministic).
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxD = 128;
constexpr float kGateFloor = -110.f;

__device__ inline float softplus_f(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }
__device__ inline float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }

// dg/dx and dg/da_log of the in-kernel gate at x = gate + dt_bias; zero where
// the forward clamped g at the bound or floored it at -110.
__device__ inline void gate_grad(float x, float alog, int form, float lb, float* dgdx, float* dgda) {
  const float A = expf(alog);
  float g, gx, ga;
  if (form == 1) {
    const float s = sigmoid_f(A * x);
    g = lb * s;
    gx = lb * s * (1.f - s) * A;
    ga = gx * x;
  } else {
    g = -A * softplus_f(x);
    gx = -A * sigmoid_f(x);
    ga = g;
    if (form == 2 && !(g > lb)) gx = ga = 0.f;
  }
  if (!(g > kGateFloor)) gx = ga = 0.f;
  *dgdx = gx;
  *dgda = ga;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Forward state pass keeping S0 and Delta of every chunk.  One workgroup per
// (sequence, head, tile of VT columns).
template <int C, int VT>
__global__ __launch_bounds__(kThreads) void k_bwd_fstate(BwdArgs b) {
  const FwdArgs& a = b.f;
  const int H = a.H, K = a.K, V = a.V;
  const int ntile = V / VT;
  const int64_t wid = blockIdx.x;
  const int tile = (int)(wid % ntile);
  const int64_t nh = wid / ntile;
  const int h = (int)(nh % H), n = (int)(nh / H);
  const int col0 = tile * VT;
  const int tid = threadIdx.x;
  __shared__ float sS[kMaxD][VT];
  __shared__ float sD[C][VT];
  const int64_t sbase = ((int64_t)n * H + h) * K * V;
  for (int e = tid; e < K * VT; e += kThreads) {
    const int c = e / VT, jj = e % VT;
    sS[c][jj] = a.init ? a.init[sbase + (int64_t)c * V + col0 + jj] : 0.f;
  }
  const int jc0 = a.seq_chunk0[n], jc1 = a.seq_chunk0[n + 1];
  for (int j = jc0; j < jc1; ++j) {
    const int64_t chb = (int64_t)j * H + h;
    const float* W = (const float*)a.W + chb * C * K;
    const float* U = (const float*)a.U + chb * C * V;
    const float* Kb = (const float*)a.Kb + chb * C * K;
    const float* gL = a.gL + chb * K;
    float* hc = b.hc + chb * K * V;
    float* Dc = b.Dc + chb * C * V;
    const int L = a.chunk_len[j];
    __syncthreads();
    for (int e = tid; e < K * VT; e += kThreads) {
      const int c = e / VT, jj = e % VT;
      hc[(int64_t)c * V + col0 + jj] = sS[c][jj];
    }
    for (int e = tid; e < C * VT; e += kThreads) {
      const int r = e / VT, jj = e % VT, col = col0 + jj;
      float acc = U[(int64_t)r * V + col];
      for (int c = 0; c < K; ++c) acc = fmaf(-W[(int64_t)r * K + c], sS[c][jj], acc);
      sD[r][jj] = acc;
      Dc[(int64_t)r * V + col] = acc;
    }
    __syncthreads();
    for (int e = tid; e < K * VT; e += kThreads) {
      const int c = e / VT, jj = e % VT;
      float acc = gL[c] * sS[c][jj];
      for (int r = 0; r < L; ++r) acc = fmaf(Kb[(int64_t)r * K + c], sD[r][jj], acc);
      sS[c][jj] = acc;
    }
  }
}

// Reverse state pass: dS_L and dDelta of every chunk, and the initial state's
// gradient.  One workgroup per (sequence, head, tile of VT columns).
template <typename Tin, int C, int VT>
__global__ __launch_bounds__(kThreads) void k_bwd_dstate(BwdArgs b) {
  const FwdArgs& a = b.f;
  const int H = a.H, K = a.K, V = a.V;
  const int ntile = V / VT;
  const int64_t wid = blockIdx.x;
  const int tile = (int)(wid % ntile);
  const int64_t nh = wid / ntile;
  const int h = (int)(nh % H), n = (int)(nh / H);
  const int col0 = tile * VT;
  const int tid = threadIdx.x;
  __shared__ float sS[kMaxD][VT];  // dS
  __shared__ float sD[C][VT];      // dDelta
  __shared__ float sO[C][VT];      // dO
  const int64_t sbase = ((int64_t)n * H + h) * K * V;
  for (int e = tid; e < K * VT; e += kThreads) {
    const int c = e / VT, jj = e % VT;
    sS[c][jj] = b.d_fin ? b.d_fin[sbase + (int64_t)c * V + col0 + jj] : 0.f;
  }
  const Tin* dO = (const Tin*)b.d_o;
  const int jc0 = a.seq_chunk0[n], jc1 = a.seq_chunk0[n + 1];
  for (int j = jc1 - 1; j >= jc0; --j) {
    const int64_t chb = (int64_t)j * H + h;
    const float* W = (const float*)a.W + chb * C * K;
    const float* Qt = (const float*)a.Qt + chb * C * K;
    const float* Kb = (const float*)a.Kb + chb * C * K;
    const float* Aqk = (const float*)a.Aqk + chb * C * C;
    const float* gL = a.gL + chb * K;
    float* dhc = b.dhc + chb * K * V;
    float* dDc = b.dDc + chb * C * V;
    const int tok0 = a.chunk_tok[j], L = a.chunk_len[j];
    __syncthreads();
    for (int e = tid; e < K * VT; e += kThreads) {
      const int c = e / VT, jj = e % VT;
      dhc[(int64_t)c * V + col0 + jj] = sS[c][jj];
    }
    for (int e = tid; e < C * VT; e += kThreads) {
      const int r = e / VT, jj = e % VT;
      sO[r][jj] = r < L ? load_f32(dO + ((int64_t)(tok0 + r) * H + h) * V + col0 + jj) : 0.f;
    }
    __syncthreads();
    // dDelta = Aqk_s^T dO + Kbar dS_L
    for (int e = tid; e < C * VT; e += kThreads) {
      const int r = e / VT, jj = e % VT;
      float acc = 0.f;
      for (int rr = r; rr < L; ++rr) acc = fmaf(Aqk[(int64_t)rr * C + r], sO[rr][jj], acc);
      for (int c = 0; c < K; ++c) acc = fmaf(Kb[(int64_t)r * K + c], sS[c][jj], acc);
      sD[r][jj] = acc;
      dDc[(int64_t)r * V + col0 + jj] = acc;
    }
    __syncthreads();
    // dS0 = Qt_s^T dO + e^gamma_L dS_L - W^T dDelta (each element reads only its own dS)
    for (int e = tid; e < K * VT; e += kThreads) {
      const int c = e / VT, jj = e % VT;
      float acc = gL[c] * sS[c][jj];
      for (int r = 0; r < L; ++r) {
        acc = fmaf(Qt[(int64_t)r * K + c], sO[r][jj], acc);
        acc = fmaf(-W[(int64_t)r * K + c], sD[r][jj], acc);
      }
      sS[c][jj] = acc;
    }
  }
  __syncthreads();
  if (b.dinit)
    for (int e = tid; e < K * VT; e += kThreads) {
      const int c = e / VT, jj = e % VT;
      b.dinit[sbase + (int64_t)c * V + col0 + jj] = sS[c][jj];
    }
}

// Chunk-local gradients.  One workgroup per chunk-head.
template <typename Tin, int C>
__global__ __launch_bounds__(kThreads) void k_bwd_chunk(BwdArgs b) {
  const FwdArgs& a = b.f;
  const int H = a.H, K = a.K, V = a.V;
  const int64_t wid = blockIdx.x;
  const int j = (int)(wid / H), h = (int)(wid % H);
  if (j >= *a.nt_dev) return;
  const int tid = threadIdx.x;
  const int tok0 = a.chunk_tok[j], L = a.chunk_len[j];
  const int64_t chb = (int64_t)j * H + h;
  auto th = [&](int r) { return (int64_t)(tok0 + r) * H + h; };
  const float* Tm = a.Tm_out + chb * C * C;
  const float* Akk = a.Akk_out + chb * C * C;
  const float* S0 = b.hc + chb * K * V;
  const float* dSL = b.dhc + chb * K * V;
  const float* Dl = b.Dc + chb * C * V;
  const float* dDl = b.dDc + chb * C * V;
  const Tin* dO = (const Tin*)b.d_o;
  const Tin* v = (const Tin*)a.v;
  const float scale = a.scale;

  __shared__ float sGam[C][kMaxD];  // gamma (rows >= L repeat gamma_{L-1})
  __shared__ float sDW[C][kMaxD];   // dW = -dDelta S0^T
  __shared__ float sT[C][C + 1];    // Tm
  __shared__ float sP[C][C + 1];    // gradient of the unscaled Aqk (i <= r)
  __shared__ float sY[C][C + 1];    // Y = dW K~^T + dDelta V^T (i <= r), later dAkk (i < r)
  __shared__ float sZ[C][C + 1];    // Z = Tm^T dT (b < r)
  __shared__ float sB[C], sDb[C];   // beta, d(beta)
  __shared__ float sRed[kMaxD];

  for (int c = tid; c < K; c += kThreads) {
    float acc = 0.f;
    for (int r = 0; r < C; ++r) {
      if (r < L) acc += a.g[th(r) * K + c];
      sGam[r][c] = acc;
    }
  }
  for (int r = tid; r < C; r += kThreads) {
    sB[r] = r < L ? a.bt[th(r)] : 0.f;
    sDb[r] = 0.f;
  }
  for (int p = tid; p < C * C; p += kThreads) sT[p / C][p % C] = Tm[p];
  __syncthreads();

  // dW and P
  for (int p = tid; p < C * K; p += kThreads) {
    const int r = p / K, c = p % K;
    float acc = 0.f;
    if (r < L)
      for (int jv = 0; jv < V; ++jv) acc = fmaf(dDl[(int64_t)r * V + jv], S0[(int64_t)c * V + jv], acc);
    sDW[r][c] = -acc;
  }
  for (int p = tid; p < C * C; p += kThreads) {
    const int r = p / C, i = p % C;
    float acc = 0.f;
    if (i <= r && r < L)
      for (int jv = 0; jv < V; ++jv)
        acc = fmaf(load_f32(dO + th(r) * V + jv), Dl[(int64_t)i * V + jv], acc);
    sP[r][i] = scale * acc;
  }
  __syncthreads();

  // Y[a][i] = sum_c dW[a][c] K~[i][c] + sum_j dDelta[a][j] v[i][j]   (i <= a < L)
  for (int p = tid; p < C * C; p += kThreads) {
    const int r = p / C, i = p % C;
    float acc = 0.f;
    if (i <= r && r < L) {
      const float* ki = a.kn + th(i) * K;
      for (int c = 0; c < K; ++c) acc = fmaf(sDW[r][c], ki[c] * expf(sGam[i][c]), acc);
      for (int jv = 0; jv < V; ++jv)
        acc = fmaf(dDl[(int64_t)r * V + jv], load_f32(v + th(i) * V + jv), acc);
    }
    sY[r][i] = acc;
  }
  __syncthreads();

  // dbeta, first part: diag(Tm^T Y); Z[r][bb] = beta_bb sum_{a >= r} Tm[a][r] Y[a][bb] (bb < r)
  for (int r = tid; r < L; r += kThreads) {
    float acc = 0.f;
    for (int aa = r; aa < L; ++aa) acc = fmaf(sT[aa][r], sY[aa][r], acc);
    sDb[r] = acc;
  }
  for (int p = tid; p < C * C; p += kThreads) {
    const int r = p / C, bb = p % C;
    float acc = 0.f;
    if (bb < r && r < L)
      for (int aa = r; aa < L; ++aa) acc = fmaf(sT[aa][r], sY[aa][bb], acc);
    sZ[r][bb] = sB[bb] * acc;
  }
  __syncthreads();

  // dN[r][i] = -sum_{bb <= i} Z[r][bb] Tm[i][bb] (i < r); dAkk = beta_r dN -> sY;
  // dbeta, second part: sum_i dN[r][i] Akk[r][i]
  for (int r = tid; r < C; r += kThreads) {
    float db = 0.f;
    for (int i = 0; i < C; ++i) {
      float dAkk = 0.f;
      if (i < r && r < L) {
        float dn = 0.f;
        for (int bb = 0; bb <= i; ++bb) dn = fmaf(-sZ[r][bb], sT[i][bb], dn);
        db = fmaf(dn, Akk[(int64_t)r * C + i], db);
        dAkk = sB[r] * dn;
      }
      sY[r][i] = dAkk;
    }
    sDb[r] += db;
  }
  __syncthreads();

  // per element (r, c): the gradients of q^, k^ and gamma
  for (int p = tid; p < L * K; p += kThreads) {
    const int r = p / K, c = p % K;
    const float q = a.qn[th(r) * K + c], kk = a.kn[th(r) * K + c];
    const float gm = sGam[r][c], egm = expf(gm), ekb = expf(sGam[L - 1][c] - gm);
    float dqt = 0.f, dkb = 0.f;
    for (int jv = 0; jv < V; ++jv) {
      const float s0 = S0[(int64_t)c * V + jv];
      dqt = fmaf(load_f32(dO + th(r) * V + jv), s0, dqt);
      dkb = fmaf(Dl[(int64_t)r * V + jv], dSL[(int64_t)c * V + jv], dkb);
    }
    dqt *= scale;
    float dxk = 0.f;
    for (int aa = r; aa < L; ++aa) dxk = fmaf(sT[aa][r], sDW[aa][c], dxk);
    const float dkt = sB[r] * dxk;
    float r1 = 0.f, r2 = 0.f;
    for (int i = 0; i <= r; ++i) {
      const float ke = a.kn[th(i) * K + c] * expf(gm - sGam[i][c]);
      r1 = fmaf(sP[r][i], ke, r1);
      r2 = fmaf(sY[r][i], ke, r2);  // zero on the diagonal
    }
    float c12 = 0.f;
    for (int rr = r; rr < L; ++rr) {
      const float e = expf(sGam[rr][c] - gm);
      c12 = fmaf(sP[rr][r] * a.qn[th(rr) * K + c] + sY[rr][r] * a.kn[th(rr) * K + c], e, c12);
    }
    const float tkb = kk * ekb * dkb;
    b.dqh[th(r) * K + c] = egm * dqt + r1;
    b.dkh[th(r) * K + c] = egm * dkt + ekb * dkb + r2 + c12;
    b.dgam[th(r) * K + c] = q * egm * dqt + kk * egm * dkt - tkb + q * r1 + kk * r2 - kk * c12;
    b.tkb[th(r) * K + c] = tkb;
  }
  // dV = Diag(beta) Tm^T dDelta
  Tin* dv = (Tin*)b.dv;
  for (int p = tid; p < L * V; p += kThreads) {
    const int r = p / V, jv = p % V;
    float acc = 0.f;
    for (int aa = r; aa < L; ++aa) acc = fmaf(sT[aa][r], dDl[(int64_t)aa * V + jv], acc);
    store_as(dv + th(r) * V + jv, sB[r] * acc);
  }
  __syncthreads();

  // gamma -> g (reverse cumulative sum; gamma_L also collects the Kbar terms and
  // the state decay), then through the gate
  Tin* dgate = (Tin*)b.dgate;
  const Tin* gate = (const Tin*)a.gate;
  for (int c = tid; c < K; c += kThreads) {
    float cst = 0.f;
    for (int r = 0; r < L; ++r) cst += b.tkb[th(r) * K + c];
    float sd = 0.f;
    for (int jv = 0; jv < V; ++jv) sd = fmaf(dSL[(int64_t)c * V + jv], S0[(int64_t)c * V + jv], sd);
    cst = fmaf(expf(sGam[L - 1][c]), sd, cst);
    float run = cst, ddt = 0.f, da = 0.f;
    const float alog = a.a_log[h], db = a.dt_bias[(int64_t)h * K + c];
    for (int r = L - 1; r >= 0; --r) {
      run += b.dgam[th(r) * K + c];
      float gx, ga;
      gate_grad(load_f32(gate + th(r) * K + c) + db, alog, a.gate_form, a.lb, &gx, &ga);
      const float dg = run * gx;
      store_as(dgate + th(r) * K + c, dg);
      ddt += dg;
      da = fmaf(run, ga, da);
    }
    b.ddt_part[chb * K + c] = ddt;
    sRed[c] = da;
  }
  // beta logit
  Tin* dbeta = (Tin*)b.dbeta;
  for (int r = tid; r < L; r += kThreads) store_as(dbeta + th(r), sDb[r] * sB[r] * (1.f - sB[r]));
  __syncthreads();
  if (tid == 0) {
    float s = 0.f;
    for (int c = 0; c < K; ++c) s += sRed[c];
    b.da_part[chb] = s;
  }
}

// dq, dk: sum over the value heads of a group, then the L2 norm's Jacobian.
// One wave per (token, key head).
template <typename Tin>
__global__ __launch_bounds__(kThreads) void k_bwd_qk(BwdArgs b) {
  const FwdArgs& a = b.f;
  const int H = a.H, HK = a.HK, K = a.K, G = H / HK;
  const int lane = threadIdx.x & 63;
  const int64_t tk = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (tk >= (int64_t)a.B * a.T * HK) return;
  const int64_t tok = tk / HK;
  const int hk = (int)(tk % HK);
  for (int which = 0; which < 2; ++which) {
    const Tin* x = (const Tin*)(which ? a.k : a.q) + tk * K;
    const float* dxh = which ? b.dkh : b.dqh;
    Tin* out = (Tin*)(which ? b.dk : b.dq) + tk * K;
    float ss = 0.f, dot = 0.f;
    float dn[kMaxD / 64];
    for (int m = 0; m < K / 64; ++m) {
      const int c = lane + 64 * m;
      float s = 0.f;
      for (int gi = 0; gi < G; ++gi) s += dxh[(tok * H + (int64_t)hk * G + gi) * K + c];
      dn[m] = s;
      const float xv = load_f32(x + c);
      ss = fmaf(xv, xv, ss);
      dot = fmaf(xv, s, dot);
    }
    ss = wave_sum(ss);
    dot = wave_sum(dot);
    const float rn = 1.f / sqrtf(ss + 1e-6f);
    const float r3 = rn * rn * rn;
    for (int m = 0; m < K / 64; ++m) {
      const int c = lane + 64 * m;
      store_as(out + c, dn[m] * rn - load_f32(x + c) * dot * r3);
    }
  }
}

// da_log, ddt_bias: sums over chunks in chunk order.
__global__ __launch_bounds__(kThreads) void k_bwd_params(BwdArgs b) {
  const FwdArgs& a = b.f;
  const int H = a.H, K = a.K;
  const int nt = *a.nt_dev;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t < (int64_t)H * K) {
    const int h = (int)(t / K), c = (int)(t % K);
    float s = 0.f;
    for (int j = 0; j < nt; ++j) s += b.ddt_part[((int64_t)j * H + h) * K + c];
    b.ddt_bias[t] = s;
  }
  if (t < H) {
    float s = 0.f;
    for (int j = 0; j < nt; ++j) s += b.da_part[(int64_t)j * H + t];
    b.da_log[t] = s;
  }
}

template <typename Tin, int C>
hipError_t run(const BwdArgs& b, hipStream_t s) {
  const FwdArgs& a = b.f;
  hipError_t e = launch_valu_prep(a, s);
  if (e != hipSuccess) return e;
  constexpr int VT = 32;
  const int64_t wgs = (int64_t)a.N * a.H * (a.V / VT);
  if (wgs > 0) {
    if (a.NT > 0) {
      hipLaunchKernelGGL((k_bwd_fstate<C, VT>), dim3((unsigned)wgs), dim3(kThreads), 0, s, b);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    hipLaunchKernelGGL((k_bwd_dstate<Tin, C, VT>), dim3((unsigned)wgs), dim3(kThreads), 0, s, b);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  if (a.NT > 0) {
    hipLaunchKernelGGL((k_bwd_chunk<Tin, C>), dim3((unsigned)((int64_t)a.NT * a.H)), dim3(kThreads), 0, s, b);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  const int64_t tk = (int64_t)a.B * a.T * a.HK;
  if (tk > 0) {
    hipLaunchKernelGGL((k_bwd_qk<Tin>), dim3((unsigned)((tk + 3) / 4)), dim3(kThreads), 0, s, b);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  const int64_t hk = (int64_t)a.H * a.K;
  hipLaunchKernelGGL(k_bwd_params, dim3((unsigned)((hk + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, b);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  return hipSuccess;
}

template <typename Tin>
hipError_t run_c(const BwdArgs& b, hipStream_t s) {
  switch (b.f.C) {
    case 16: return run<Tin, 16>(b, s);
    case 32: return run<Tin, 32>(b, s);
    default: return run<Tin, 64>(b, s);
  }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& b, hipStream_t s) {
  hipError_t e = launch_chunk_table(b.f, s);
  if (e != hipSuccess) return e;
  return b.f.dtype == 0 ? run_c<float>(b, s) : run_c<bf16>(b, s);
}

}  // namespace kda
