// Backward of the KDA chunked forward: gradients of
//     L = sum(d_o * o) + sum(d_final * final_state)
// for q, k, v, the gate logits, the beta logits, a_log, dt_bias and the
// initial state, through the in-kernel L2 norm, gate and beta sigmoid.  What is
// differentiated: the chunk_kda call that the torchtitan PR #4025 commit note
// tests forward and backward together, whose state gradient the hyper_parallel
// coverage page routes between slices (the backward of _RecvKDAInitialState).
//
// fp32 arithmetic after the recomputation.  For 64-token chunks the dense
// per-chunk products (the two state passes, the value-dimension, Y, Z and dN
// products and the pairwise sums of the chunk kernel) run on matrix cores:
// for fp32 inputs on fp32 ones (v_mfma_f32_16x16x4f32); for bf16 inputs the
// state passes and the value-dimension products on bf16 ones
// (v_mfma_f32_16x16x32_bf16) with every fp32 operand split into bf16 hi + lo
// (within about 2^-16 of the fp32 product), fp32 accumulation throughout;
// the per-element work, and chunks of 16 or 32, stay on VALU.  The
// decay factors and the gate's derivative use the hardware exponential,
// logarithm and reciprocal (about one ulp on the result).  The forward's chunk
// factors are recomputed first, with Akk and Tm kept: for fp32 inputs by the
// fp32 prologue and chunk kernels; for bf16 inputs by the forward's
// matrix-core chunk kernel (bf16 operands, fp32 accumulation, as in the
// forward) writing the same fp32 arrays, or by the fp32 kernels when
// KDA_BWD_RECOMPUTE=valu.  Then,
// per chunk of L rows entering with state
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
//                          split through 16-row block boundaries while no block
//                          decays by more than kBlockSafe, exact per pair inside
//                          a block otherwise), gamma -> g by a reverse
//                          cumulative sum, and g through the gate;
//   reductions             dq, dk: sum over the value heads that share a key head,
//                          then the L2 norm's Jacobian; da_log, ddt_bias: sums over
//                          chunks in a fixed order (deterministic).
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
// Workgroup size of the chunk-gradient kernel per (C, K): its LDS (up to 160 KiB)
// allows one workgroup per CU, so the widest size that compiles without
// register spills gives the most waves to hide LDS latency.
constexpr int chunk_threads(int C, int K) { return C == 64 ? (K == 128 ? 1024 : 512) : C == 32 ? 256 : 512; }
constexpr int kMaxD = 128;
constexpr float kGateFloor = -110.f;
// Largest decay of a 16-row block (in a channel) for which the chunk-gradient
// kernel splits in-block pair factors through the block boundary.  The inner
// factor (up to e^kBlockSafe) multiplies P or dAkk before the sum is scaled
// back, and those are not bounded by one as the forward's k^ k^ products are:
// e^70 (about 2.5e30) leaves such a sum about eight orders of magnitude below
// the fp32 range for any realistic P.
constexpr float kBlockSafe = 70.f;

// Hardware exponential and logarithm (v_exp_f32 / v_log_f32 after a scaling,
// about one ulp) and reciprocal: the gate's derivatives enter sums whose fp32
// tolerance is far above their error.  softplus(x) = max(x, 0) + log(1 + e),
// sigmoid(x) = 1 / (1 + e) for x >= 0 and e / (1 + e) otherwise, e = e^{-|x|}
// (log(1 + e) loses e below half an ulp of 1, an absolute error under 6e-8).
__device__ inline void softplus_sigmoid(float x, float* sp, float* sg) {
  const float e = __expf(-fabsf(x));
  const float r = __builtin_amdgcn_rcpf(1.f + e);
  *sp = fmaxf(x, 0.f) + __logf(1.f + e);
  *sg = x >= 0.f ? r : e * r;
}

// The in-kernel gate at x = gate + dt_bias (A = e^a_log), the same arithmetic
// as gate_grad's value: -A softplus(x) (form 0), lb sigmoid(A x) (form 1),
// max(lb, -A softplus(x)) (form 2), floored at -110.
__device__ inline float gate_value(float x, float A, int form, float lb) {
  float sp, s, g;
  if (form == 1) {
    softplus_sigmoid(A * x, &sp, &s);
    g = lb * s;
  } else {
    softplus_sigmoid(x, &sp, &s);
    g = -A * sp;
    if (form == 2) g = fmaxf(g, lb);
  }
  return fmaxf(g, kGateFloor);
}

// dg/dx and dg/da_log of the in-kernel gate at x = gate + dt_bias (A = e^a_log);
// zero where the forward clamped g at the bound or floored it at -110.
__device__ inline void gate_grad(float x, float A, int form, float lb, float* dgdx, float* dgda) {
  float g, gx, ga;
  if (form == 1) {
    float sp, s;
    softplus_sigmoid(A * x, &sp, &s);
    g = lb * s;
    gx = lb * s * (1.f - s) * A;
    ga = gx * x;
  } else {
    float sp, s;
    softplus_sigmoid(x, &sp, &s);
    g = -A * sp;
    gx = -A * s;
    ga = g;
    if (form == 2 && !(g > lb)) gx = ga = 0.f;
  }
  if (!(g > kGateFloor)) gx = ga = 0.f;
  *dgdx = gx;
  *dgda = ga;
}

// The (sequence, head) chain and value-column tile of a state-pass workgroup.
// Workgroups go to the chip's eight XCDs in turn (id % 8), each XCD with its
// own L2, and the column tiles of one chain read the same per-chunk K-side
// operands at about the same time: so all tiles of a chain take ids on one
// XCD, 8 apart.  Ids past the last whole group of 8 chains map in order.
__device__ __forceinline__ void chain_tile(int64_t wid, int64_t wgs, int ntile, int& tile, int64_t& nh) {
  constexpr int kX = 8;
  if (ntile == 1) {
    tile = 0;
    nh = wid;
    return;
  }
  const int64_t full = wgs / (kX * ntile) * (kX * ntile);
  if (wid < full) {
    const int64_t x = wid % kX, q = wid / kX;
    tile = (int)(q % ntile);
    nh = (q / ntile) * kX + x;
  } else {
    tile = (int)(wid % ntile);
    nh = wid / ntile;
  }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// fp32 matrix-core product of one 16 x 4 by 4 x 16 step into a 16 x 16 tile
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// bf16 matrix-core product of one 16 x 32 by 32 x 16 step into a 16 x 16 fp32
// tile: lane l holds A[l%16][8(l/16) .. +7] and B[8(l/16) .. +7][l%16]
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// x = hi + lo: hi = bf16(x), lo = bf16(x - hi); hi + lo is within 2^-17 |x|
// of x, and a product of two such pairs without the lo * lo term within about
// 2^-16 of the fp32 product
__device__ __forceinline__ void split_bf16(float x, bf16& hi, bf16& lo) {
  const __bf16 h = (__bf16)x;
  hi = __builtin_bit_cast(bf16, h);
  lo = __builtin_bit_cast(bf16, (__bf16)(x - (float)h));
}
__device__ __forceinline__ bf16 to_bf16(float x) { return __builtin_bit_cast(bf16, (__bf16)x); }
// 8 consecutive bf16 of an LDS row (16-byte aligned)
__device__ __forceinline__ bf16x8 frag8(const bf16* p) { return *(const bf16x8*)p; }
// Column of element (row, col) in a bf16 LDS array whose rows are read as
// 16-byte chunks of 8 and written transposed (lanes stepping 4 rows, rows 72
// or 136 bf16 long): the chunk index is XORed with bits 3..5 of the row, so
// that 32 such lanes reach 8 of the 32 banks instead of 2, while a chunk stays
// 16 contiguous bytes.  For columns below 64.
// With two 4-column pieces per thread (a C x K bf16 operand, K = 128, 1024
// threads), the thread's pieces u = 0, 1: rows 2 (tid / 32) + u, columns
// 4 (tid % 32) .. + 3, so that its transposed writes pair two adjacent rows.
__device__ __forceinline__ int pair_piece(int tid, int u) { return (2 * (tid >> 5) + u) * 32 + (tid & 31); }
__device__ __forceinline__ int swz8(int row, int col) { return (((col >> 3) ^ ((row >> 3) & 7)) << 3) | (col & 7); }

// Sum over the 64 lanes on the VALU (DPP): inclusive prefix sums inside each
// 16-lane row (row_shr 1, 2, 4, 8, zero fill), then row 0's total into row 1
// and row 2's into row 3 (row_bcast:15), then row 1's into rows 2 and 3
// (row_bcast:31); lane 63 then holds the total, which is broadcast.
template <int CTRL, int ROWS, bool ZERO>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, ZERO));
}
__device__ inline float wave_sum_dpp(float x) {
  x += dpp_f<0x111, 0xF, true>(x);
  x += dpp_f<0x112, 0xF, true>(x);
  x += dpp_f<0x114, 0xF, true>(x);
  x += dpp_f<0x118, 0xF, true>(x);
  x += dpp_f<0x142, 0xA, false>(x);
  x += dpp_f<0x143, 0xC, false>(x);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Copy n floats (n a multiple of 4, 16-byte aligned) from global memory to LDS
// with a workgroup of nt threads.
__device__ inline void stage(float* dst, const float* src, int n, int nt) {
  for (int e = threadIdx.x; e < n / 4; e += nt) ((float4*)dst)[e] = ((const float4*)src)[e];
}

// Waves per workgroup of the state passes: as many as keep the row groups
// (C/NW rows of Delta per wave) multiples of four.
constexpr int state_waves(int C) { return C >= 64 ? 16 : C >= 32 ? 8 : 4; }

// Forward state pass keeping S0 and Delta of every chunk.  One workgroup per
// (sequence, head, tile of 64 columns): lane = column, wave w owns the state
// rows [w K/4, (w+1) K/4) in registers; W and Kbar of each chunk are staged in
// LDS and read as float4 broadcasts.
template <int C, int K>
__global__ __launch_bounds__(64 * state_waves(C)) void k_bwd_fstate(BwdArgs b) {
  constexpr int NW = state_waves(C), NT = 64 * NW;
  constexpr int VT = 64, RS = K / NW, RD = C / NW;
  const FwdArgs& a = b.f;
  const int H = a.H, V = a.V;
  const int ntile = V / VT;
  int tile;
  int64_t nh;
  chain_tile(blockIdx.x, gridDim.x, ntile, tile, nh);
  const int h = (int)(nh % H), n = (int)(nh / H);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = tile * VT + lane;
  __shared__ float sS[K][VT];
  __shared__ float sD[C][VT];
  __shared__ __attribute__((aligned(16))) float sW[C][K];
  __shared__ __attribute__((aligned(16))) float sKb[C][K];
  const int64_t sbase = ((int64_t)n * H + h) * K * V;
  float st[RS];
#pragma unroll
  for (int m = 0; m < RS; ++m) {
    st[m] = a.init ? a.init[sbase + (int64_t)(w * RS + m) * V + col] : 0.f;
    sS[w * RS + m][lane] = st[m];
  }
  const int jc0 = a.seq_chunk0[n], jc1 = a.seq_chunk0[n + 1];
  for (int j = jc0; j < jc1; ++j) {
    const int64_t chb = (int64_t)j * H + h;
    const float* U = (const float*)a.U + chb * C * V;
    const float* gL = a.gL + chb * K;
    float* hc = b.hc + chb * K * V;
    float* Dc = b.Dc + chb * C * V;
    const int L = a.chunk_len[j];
    __syncthreads();  // the previous chunk is done with sW, sKb; sS holds the state
    stage(&sW[0][0], (const float*)a.W + chb * C * K, C * K, NT);
    stage(&sKb[0][0], (const float*)a.Kb + chb * C * K, C * K, NT);
#pragma unroll
    for (int m = 0; m < RS; ++m) hc[(int64_t)(w * RS + m) * V + col] = st[m];
    __syncthreads();
    // Delta = U - W S for rows [w C/4, (w+1) C/4)
    float d[RD];
#pragma unroll
    for (int m = 0; m < RD; ++m) d[m] = U[(int64_t)(w * RD + m) * V + col];
    for (int c = 0; c < K; c += 4) {
      const float s0 = sS[c][lane], s1 = sS[c + 1][lane], s2 = sS[c + 2][lane], s3 = sS[c + 3][lane];
#pragma unroll
      for (int m = 0; m < RD; ++m) {
        const float4 wv = *(const float4*)&sW[w * RD + m][c];
        d[m] -= wv.x * s0 + wv.y * s1 + wv.z * s2 + wv.w * s3;
      }
    }
#pragma unroll
    for (int m = 0; m < RD; ++m) {
      sD[w * RD + m][lane] = d[m];
      Dc[(int64_t)(w * RD + m) * V + col] = d[m];
    }
    __syncthreads();
    // S = Diag(gL) S + Kbar^T Delta for the wave's rows
#pragma unroll
    for (int m = 0; m < RS; ++m) st[m] *= gL[w * RS + m];
    for (int r = 0; r < L; ++r) {
      const float dv = sD[r][lane];
#pragma unroll
      for (int m = 0; m < RS; m += 4) {
        const float4 kb = *(const float4*)&sKb[r][w * RS + m];
        st[m] = fmaf(kb.x, dv, st[m]);
        st[m + 1] = fmaf(kb.y, dv, st[m + 1]);
        st[m + 2] = fmaf(kb.z, dv, st[m + 2]);
        st[m + 3] = fmaf(kb.w, dv, st[m + 3]);
      }
    }
#pragma unroll
    for (int m = 0; m < RS; ++m) sS[w * RS + m][lane] = st[m];
  }
}

// The forward state pass for 64-token chunks on fp32 matrix cores, same
// arithmetic as k_bwd_fstate up to the order of additions: the state (K x 64
// columns) lives in accumulator tiles, K/64 per wave; per chunk, wave w
// computes one 16 x 16 tile of Delta (row tile w/4, column tile w%4).
template <int K>
__global__ __launch_bounds__(1024) void k_bwd_fstate_mfma(BwdArgs b) {
  constexpr int C = 64, NT = 1024, VT = 64;
  constexpr int TPW = K / 64;
  constexpr int SP = VT + 16, KP = K + 4;
  const FwdArgs& a = b.f;
  const int H = a.H, V = a.V;
  const int ntile = V / VT;
  int tile;
  int64_t nh;
  chain_tile(blockIdx.x, gridDim.x, ntile, tile, nh);
  const int h = (int)(nh % H), n = (int)(nh / H);
  const int col0 = tile * VT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
  __shared__ __attribute__((aligned(16))) float sS[K][SP];
  __shared__ __attribute__((aligned(16))) float sD[C][SP];
  __shared__ __attribute__((aligned(16))) float sW[C][KP];
  __shared__ __attribute__((aligned(16))) float sKb[C][KP];
  // W and Kbar of each chunk reach registers one chunk ahead (their loads are
  // in flight while the previous chunk's products run)
  constexpr int NF4 = C * K / 4 / NT;
  static_assert(NF4 * NT * 4 == C * K && NF4 <= 2, "one or two float4 pieces per thread");
  float4 pw0, pw1, pk0, pk1;  // named, so that they stay in registers
  f32x4 pu;                   // the chunk's U tile of this wave's Delta tile
  float pgl[TPW][4];          // its gL entries of this wave's state tiles
  const int drt = w >> 2, dct = w & 3;  // this wave's Delta tile
  auto fetch_wk = [&](int64_t chb) __attribute__((always_inline)) {
    const float* U = (const float*)a.U + chb * C * V;
    const float* gL = a.gL + chb * K;
#pragma unroll
    for (int e = 0; e < 4; ++e) pu[e] = U[(int64_t)(16 * drt + 4 * lg + e) * V + col0 + 16 * dct + ln];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) pgl[t][e] = gL[16 * ((w * TPW + t) >> 2) + 4 * lg + e];
    const float4* W4 = (const float4*)((const float*)a.W + chb * C * K);
    const float4* K4 = (const float4*)((const float*)a.Kb + chb * C * K);
    pw0 = W4[tid];
    pk0 = K4[tid];
    if constexpr (NF4 == 2) {
      pw1 = W4[tid + NT];
      pk1 = K4[tid + NT];
    }
  };
  const int64_t sbase = ((int64_t)n * H + h) * K * V;
  f32x4 st[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 16 * srt + 4 * lg + e, col = col0 + 16 * sct + ln;
      st[t][e] = a.init ? a.init[sbase + (int64_t)c * V + col] : 0.f;
    }
  }
  const int jc0 = a.seq_chunk0[n], jc1 = a.seq_chunk0[n + 1];
  if (jc0 < jc1) fetch_wk((int64_t)jc0 * H + h);
  for (int j = jc0; j < jc1; ++j) {
    const int64_t chb = (int64_t)j * H + h;
    float* hc = b.hc + chb * K * V;
    float* Dc = b.Dc + chb * C * V;
    // this chunk's U tile and gL came with its W and Kbar, a chunk ahead
    f32x4 acc = pu;
    float gl[TPW][4];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) gl[t][e] = pgl[t][e];
    __syncthreads();  // the previous chunk is done with sW, sKb, sS, sD
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * srt + 4 * lg + e, cc = 16 * sct + ln;
        hc[(int64_t)c * V + col0 + cc] = st[t][e];
        sS[c][cc] = st[t][e];
      }
    }
    {
      const int r0 = tid / (K / 4), c0 = 4 * (tid % (K / 4));
      *(float4*)&sW[r0][c0] = pw0;
      *(float4*)&sKb[r0][c0] = pk0;
      if constexpr (NF4 == 2) {
        const int r1 = (tid + NT) / (K / 4), c1 = 4 * ((tid + NT) % (K / 4));
        *(float4*)&sW[r1][c1] = pw1;
        *(float4*)&sKb[r1][c1] = pk1;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // the next chunk of this sequence; unconditional (the last chunk reads
    // itself again, unused) so that the waits can count it
    fetch_wk(j + 1 < jc1 ? chb + H : chb);
    __syncthreads();
    // Delta = U - W S
#pragma unroll 8
    for (int c = 0; c < K; c += 4)
      acc = mfma_f32(-sW[16 * drt + ln][c + lg], sS[c + lg][16 * dct + ln], acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * drt + 4 * lg + e, cc = 16 * dct + ln;
      sD[r][cc] = acc[e];
      Dc[(int64_t)r * V + col0 + cc] = acc[e];
    }
    __syncthreads();
    // S = Diag(gL) S + Kbar^T Delta (rows past the chunk end are zero)
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) st[t][e] *= gl[t][e];
#pragma unroll 4
    for (int r = 0; r < C; r += 4) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
        st[t] = mfma_f32(sKb[r + lg][16 * srt + ln], sD[r + lg][16 * sct + ln], st[t]);
      }
    }
  }
}

// Reverse state pass: dS_L and dDelta of every chunk, and the initial state's
// gradient.  Same layout as the forward pass; Aqk and Kbar, then Qt and W,
// take turns in one LDS region.
template <typename Tin, int C, int K>
__global__ __launch_bounds__(64 * state_waves(C)) void k_bwd_dstate(BwdArgs b) {
  constexpr int NW = state_waves(C), NT = 64 * NW;
  constexpr int VT = 64, RS = K / NW, RD = C / NW;
  const FwdArgs& a = b.f;
  const int H = a.H, V = a.V;
  const int ntile = V / VT;
  int tile;
  int64_t nh;
  chain_tile(blockIdx.x, gridDim.x, ntile, tile, nh);
  const int h = (int)(nh % H), n = (int)(nh / H);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = tile * VT + lane;
  __shared__ float sS[K][VT];   // dS
  __shared__ float sO[C][VT];   // dO
  __shared__ float sD[C][VT];   // dDelta
  __shared__ __attribute__((aligned(16))) float sR[2 * C * K];  // Aqk | Kbar, then Qt | W
  float (*sA)[C] = (float(*)[C])sR;
  float (*sKb)[K] = (float(*)[K])(sR + C * C);
  float (*sQt)[K] = (float(*)[K])sR;
  float (*sW)[K] = (float(*)[K])(sR + C * K);
  const int64_t sbase = ((int64_t)n * H + h) * K * V;
  float ds[RS];
#pragma unroll
  for (int m = 0; m < RS; ++m) ds[m] = b.d_fin ? b.d_fin[sbase + (int64_t)(w * RS + m) * V + col] : 0.f;
  const Tin* dO = (const Tin*)b.d_o;
  const int jc0 = a.seq_chunk0[n], jc1 = a.seq_chunk0[n + 1];
  for (int j = jc1 - 1; j >= jc0; --j) {
    const int64_t chb = (int64_t)j * H + h;
    const float* gL = a.gL + chb * K;
    float* dhc = b.dhc + chb * K * V;
    float* dDc = b.dDc + chb * C * V;
    const int tok0 = a.chunk_tok[j], L = a.chunk_len[j];
    __syncthreads();  // the previous chunk is done with sR, sO, sD, sS
#pragma unroll
    for (int m = 0; m < RS; ++m) {
      dhc[(int64_t)(w * RS + m) * V + col] = ds[m];
      sS[w * RS + m][lane] = ds[m];
    }
#pragma unroll
    for (int m = 0; m < RD; ++m) {
      const int r = w * RD + m;
      const float x = load_f32(dO + ((int64_t)(tok0 + (r < L ? r : 0)) * H + h) * V + col);
      sO[r][lane] = r < L ? x : 0.f;
    }
    stage(sR, (const float*)a.Aqk + chb * C * C, C * C, NT);
    stage(sR + C * C, (const float*)a.Kb + chb * C * K, C * K, NT);
    __syncthreads();
    // dDelta = Aqk_s^T dO + Kbar dS_L (Aqk_s is zero above the diagonal)
    float d[RD];
#pragma unroll
    for (int m = 0; m < RD; ++m) d[m] = 0.f;
    for (int rr = 0; rr < L; ++rr) {
      const float o = sO[rr][lane];
#pragma unroll
      for (int m = 0; m < RD; m += 4) {
        const float4 av = *(const float4*)&sA[rr][w * RD + m];
        d[m] = fmaf(av.x, o, d[m]);
        d[m + 1] = fmaf(av.y, o, d[m + 1]);
        d[m + 2] = fmaf(av.z, o, d[m + 2]);
        d[m + 3] = fmaf(av.w, o, d[m + 3]);
      }
    }
    for (int c = 0; c < K; c += 4) {
      const float s0 = sS[c][lane], s1 = sS[c + 1][lane], s2 = sS[c + 2][lane], s3 = sS[c + 3][lane];
#pragma unroll
      for (int m = 0; m < RD; ++m) {
        const float4 kv = *(const float4*)&sKb[w * RD + m][c];
        d[m] += kv.x * s0 + kv.y * s1 + kv.z * s2 + kv.w * s3;
      }
    }
#pragma unroll
    for (int m = 0; m < RD; ++m) {
      sD[w * RD + m][lane] = d[m];
      dDc[(int64_t)(w * RD + m) * V + col] = d[m];
    }
    __syncthreads();  // dDelta complete; Aqk and Kbar are no longer read
    stage(sR, (const float*)a.Qt + chb * C * K, C * K, NT);
    stage(sR + C * K, (const float*)a.W + chb * C * K, C * K, NT);
    __syncthreads();
    // dS0 = Diag(gL) dS_L + Qt_s^T dO - W^T dDelta
#pragma unroll
    for (int m = 0; m < RS; ++m) ds[m] *= gL[w * RS + m];
    for (int r = 0; r < L; ++r) {
      const float o = sO[r][lane], dd = sD[r][lane];
#pragma unroll
      for (int m = 0; m < RS; m += 4) {
        const float4 qv = *(const float4*)&sQt[r][w * RS + m];
        const float4 wv = *(const float4*)&sW[r][w * RS + m];
        ds[m] = fmaf(qv.x, o, fmaf(-wv.x, dd, ds[m]));
        ds[m + 1] = fmaf(qv.y, o, fmaf(-wv.y, dd, ds[m + 1]));
        ds[m + 2] = fmaf(qv.z, o, fmaf(-wv.z, dd, ds[m + 2]));
        ds[m + 3] = fmaf(qv.w, o, fmaf(-wv.w, dd, ds[m + 3]));
      }
    }
  }
  if (b.dinit)
#pragma unroll
    for (int m = 0; m < RS; ++m) b.dinit[sbase + (int64_t)(w * RS + m) * V + col] = ds[m];
}

// The reverse state pass for 64-token chunks on fp32 matrix cores
// (v_mfma_f32_16x16x4f32), same arithmetic as k_bwd_dstate up to the order of
// additions.  One workgroup of 16 waves per (sequence, head, 64 columns); the
// state gradient dS (K x 64) lives in accumulator tiles, K/64 per wave (state
// row tile (w*TPW+t)/4, column tile (w*TPW+t)%4); per chunk, wave w computes
// one 16 x 16 tile of dDelta (row tile w/4, column tile w%4).  Operands come
// from LDS rows padded so that the 16 lanes of a fragment column hit
// different banks.
template <typename Tin, int K>
__global__ __launch_bounds__(1024) void k_bwd_dstate_mfma(BwdArgs b) {
  constexpr int C = 64, NT = 1024, VT = 64;
  constexpr int TPW = K / 64;                     // state tiles per wave
  constexpr int SP = VT + 16, AP = C + 4, KP = K + 4;
  const FwdArgs& a = b.f;
  const int H = a.H, V = a.V;
  const int ntile = V / VT;
  int tile;
  int64_t nh;
  chain_tile(blockIdx.x, gridDim.x, ntile, tile, nh);
  const int h = (int)(nh % H), n = (int)(nh / H);
  const int col0 = tile * VT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
  __shared__ __attribute__((aligned(16))) float sS[K][SP];   // dS
  __shared__ __attribute__((aligned(16))) float sO[C][SP];   // dO
  __shared__ __attribute__((aligned(16))) float sD[C][SP];   // dDelta
  __shared__ __attribute__((aligned(16))) float sR[2 * C * KP];  // Aqk | Kbar, then Qt | W
  float (*sA)[AP] = (float(*)[AP])sR;
  float (*sKb)[KP] = (float(*)[KP])(sR + C * AP);
  float (*sQt)[KP] = (float(*)[KP])sR;
  float (*sW)[KP] = (float(*)[KP])(sR + C * KP);
  static_assert(C * AP + C * KP <= 2 * C * KP, "Aqk and Kbar fit the operand region");
  // Aqk, Kbar, Qt and W of each chunk reach registers one chunk ahead (named,
  // so that they stay in registers): their loads are in flight while the
  // previous chunk's products run
  static_assert(C * C / 4 == NT && C * K / 4 <= 2 * NT, "one Aqk piece, one or two of the others");
  constexpr bool TWO = C * K / 4 == 2 * NT;
  float4 pa, pk0, pk1, pq0, pq1, pw0, pw1;
  // dO of the prefetched chunk, raw (rows past its end are masked when staged)
  constexpr int NO = C * VT / NT;
  static_assert(NO * NT == C * VT, "whole dO tiles per thread");
  const Tin* dO = (const Tin*)b.d_o;
  float po[NO];
  auto fetch = [&](int jn) __attribute__((always_inline)) {
    const int64_t chb = (int64_t)jn * H + h;
    const int tokn = a.chunk_tok[jn], Ln = a.chunk_len[jn];
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const int e = tid + u * NT, r = e / VT, cc = e % VT;
      po[u] = load_f32(dO + ((int64_t)(tokn + (r < Ln ? r : 0)) * H + h) * V + col0 + cc);
    }
    const float4* A4 = (const float4*)((const float*)a.Aqk + chb * C * C);
    const float4* K4 = (const float4*)((const float*)a.Kb + chb * C * K);
    const float4* Q4 = (const float4*)((const float*)a.Qt + chb * C * K);
    const float4* W4 = (const float4*)((const float*)a.W + chb * C * K);
    pa = A4[tid];
    pk0 = K4[tid];
    pq0 = Q4[tid];
    pw0 = W4[tid];
    if constexpr (TWO) {
      pk1 = K4[tid + NT];
      pq1 = Q4[tid + NT];
      pw1 = W4[tid + NT];
    }
  };
  // a [C][K] matrix held as pieces tid (and tid + NT) into LDS rows of stride KP
  auto put_k = [&](float (*dst)[KP], const float4& v0, const float4& v1) __attribute__((always_inline)) {
    *(float4*)&dst[tid / (K / 4)][4 * (tid % (K / 4))] = v0;
    if constexpr (TWO) *(float4*)&dst[(tid + NT) / (K / 4)][4 * ((tid + NT) % (K / 4))] = v1;
  };
  const int64_t sbase = ((int64_t)n * H + h) * K * V;
  f32x4 st[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 16 * srt + 4 * lg + e, col = col0 + 16 * sct + ln;
      st[t][e] = b.d_fin ? b.d_fin[sbase + (int64_t)c * V + col] : 0.f;
    }
  }
  const int drt = w >> 2, dct = w & 3;  // this wave's dDelta tile
  const int jc0 = a.seq_chunk0[n], jc1 = a.seq_chunk0[n + 1];
  if (jc0 < jc1) fetch(jc1 - 1);
  for (int j = jc1 - 1; j >= jc0; --j) {
    const int64_t chb = (int64_t)j * H + h;
    const float* gL = a.gL + chb * K;
    float* dhc = b.dhc + chb * K * V;
    float* dDc = b.dDc + chb * C * V;
    const int L = a.chunk_len[j];
    __syncthreads();  // the previous chunk is done with sR, sO, sD, sS
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * srt + 4 * lg + e, cc = 16 * sct + ln;
        dhc[(int64_t)c * V + col0 + cc] = st[t][e];
        sS[c][cc] = st[t][e];
      }
    }
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const int e = tid + u * NT, r = e / VT, cc = e % VT;
      sO[r][cc] = r < L ? po[u] : 0.f;
    }
    *(float4*)&sA[tid / (C / 4)][4 * (tid % (C / 4))] = pa;
    put_k(sKb, pk0, pk1);
    __syncthreads();
    // dDelta = Aqk_s^T dO + Kbar dS_L (Aqk_s is zero above the diagonal, so
    // rows rr below the tile's first row contribute nothing)
    {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int rr = 16 * drt; rr < C; rr += 4)
        acc = mfma_f32(sA[rr + lg][16 * drt + ln], sO[rr + lg][16 * dct + ln], acc);
#pragma unroll 8
      for (int c = 0; c < K; c += 4)
        acc = mfma_f32(sKb[16 * drt + ln][c + lg], sS[c + lg][16 * dct + ln], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * drt + 4 * lg + e, cc = 16 * dct + ln;
        sD[r][cc] = acc[e];
        dDc[(int64_t)r * V + col0 + cc] = acc[e];
      }
    }
    __syncthreads();  // dDelta complete; Aqk and Kbar are no longer read
    put_k(sQt, pq0, pq1);
    put_k(sW, pw0, pw1);
    float gl[TPW][4];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) gl[t][e] = gL[16 * ((w * TPW + t) >> 2) + 4 * lg + e];
    // The previous chunk of this sequence (its operands and its dO tile),
    // issued after gL's loads (held there by the scheduling barrier) so that
    // waiting for gL leaves it in flight; unconditional (the first chunk reads
    // itself again, unused) so that the wait can count it.
    __builtin_amdgcn_sched_barrier(0);
    fetch(j - 1 >= jc0 ? j - 1 : j);
    __syncthreads();
    // dS0 = Diag(gL) dS_L + Qt_s^T dO - W^T dDelta (rows past the chunk end are zero)
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) st[t][e] *= gl[t][e];
#pragma unroll 4
    for (int r = 0; r < C; r += 4) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
        st[t] = mfma_f32(sQt[r + lg][16 * srt + ln], sO[r + lg][16 * sct + ln], st[t]);
        st[t] = mfma_f32(-sW[r + lg][16 * srt + ln], sD[r + lg][16 * sct + ln], st[t]);
      }
    }
  }
  if (b.dinit) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        b.dinit[sbase + (int64_t)(16 * srt + 4 * lg + e) * V + col0 + 16 * sct + ln] = st[t][e];
    }
  }
}

// ---------------------------------------------------------------------------
// State passes on bf16 matrix cores (FwdArgs::ws_bf16: W, U, Qt, Kbar and Aqk
// recomputed as bf16).  Those operands enter the products exactly; the fp32
// state (or state gradient) and Delta (or dDelta) enter as bf16 hi + lo pairs
// (hi = bf16(x), lo = bf16(x - hi): within 2^-17 of x), so each product is
// two v_mfma_f32_16x16x32_bf16 per 32-long k-step with fp32 accumulation,
// against eight fp32 steps of 4.  Operands are staged in LDS so that every
// lane's 8 k-consecutive elements are one 16-byte read: row-major where the
// k index runs along a row, transposed otherwise.  Layout as in the fp32
// passes: one workgroup of 16 waves per (sequence, head, 64 columns), the
// K x 64 state in accumulator tiles (K/64 per wave: state row tile
// (w*TPW+t)/4, column tile (w*TPW+t)%4), wave w owning the (w/4, w%4) tile of
// the chunk's Delta.
// ---------------------------------------------------------------------------
// 4 fp32 -> 4 bf16 hi and 4 bf16 lo (as two 32-bit words each)
__device__ __forceinline__ void split4_bf16(f32x4 x, uint2& hi, uint2& lo) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  bf16x4_t h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = (__bf16)x[e];
    l[e] = (__bf16)(x[e] - (float)h[e]);
  }
  const u32x2 hu = __builtin_bit_cast(u32x2, h), lu = __builtin_bit_cast(u32x2, l);
  hi = make_uint2(hu.x, hu.y);
  lo = make_uint2(lu.x, lu.y);
}
// element q of 4 bf16 held as two 32-bit words
__device__ __forceinline__ bf16 elem4(uint2 u, int q) {
  return (bf16)(((q < 2 ? u.x : u.y) >> (16 * (q & 1))) & 0xffffu);
}

template <int K>
__global__ __launch_bounds__(1024) void k_bwd_fstate_bf(BwdArgs b) {
  constexpr int C = 64, NT = 1024, VT = 64;
  constexpr int TPW = K / 64;
  constexpr int WP = K + 8, TP = C + 8;  // bf16 row strides, multiples of 16 bytes
  const FwdArgs& a = b.f;
  const int H = a.H, V = a.V;
  const int ntile = V / VT;
  int tile;
  int64_t nh;
  chain_tile(blockIdx.x, gridDim.x, ntile, tile, nh);
  const int h = (int)(nh % H), n = (int)(nh / H);
  const int col0 = tile * VT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
  __shared__ __attribute__((aligned(16))) bf16 sWn[C][WP];             // -W
  __shared__ __attribute__((aligned(16))) bf16 sKbT[K][TP];            // Kbar^T
  __shared__ __attribute__((aligned(16))) bf16 sSh[VT][WP], sSl[VT][WP];  // S^T hi, lo
  __shared__ __attribute__((aligned(16))) bf16 sDh[VT][TP], sDl[VT][TP];  // Delta^T hi, lo
  // W and Kbar (4 bf16 per piece, two pieces per thread), this wave's U tile
  // and gL entries: one chunk ahead, in named registers
  constexpr int NP = C * K / 4 / NT;
  static_assert(NP == 1 || NP == 2, "one or two pieces per thread");
  struct Pre { uint2 pw0, pw1, pk0, pk1; uint2 u4; float pgl[TPW][4]; };
  Pre P0, P1;
  const int drt = w >> 2, dct = w & 3;
  auto fetch = [&](Pre& x, int64_t chb) __attribute__((always_inline)) {
    // U as 16 x 16 accumulator tiles of bf16 ([row tile][column tile][lane][4])
    x.u4 = ((const uint2*)a.U)[((chb * 4 + drt) * (V / 16) + col0 / 16 + dct) * 64 + lane];
    const float* gL = a.gL + chb * K;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) x.pgl[t][e] = gL[16 * ((w * TPW + t) >> 2) + 4 * lg + e];
    const uint2* W4 = (const uint2*)((const bf16*)a.W + chb * C * K);
    const uint2* K4 = (const uint2*)((const bf16*)a.Kb + chb * C * K);
    if constexpr (NP == 2) {
      x.pw0 = W4[pair_piece(tid, 0)];
      x.pk0 = K4[pair_piece(tid, 0)];
      x.pw1 = W4[pair_piece(tid, 1)];
      x.pk1 = K4[pair_piece(tid, 1)];
    } else {
      x.pw0 = W4[tid];
      x.pk0 = K4[tid];
    }
  };
  auto put = [&](int p, uint2 wv, uint2 kv) __attribute__((always_inline)) {
    const int r = p / (K / 4), c = 4 * (p % (K / 4));
    *(uint2*)&sWn[r][c] = make_uint2(wv.x ^ 0x80008000u, wv.y ^ 0x80008000u);
#pragma unroll
    for (int q = 0; q < 4; ++q) sKbT[c + q][swz8(c + q, r)] = elem4(kv, q);
  };
  // two pieces of rows r (even) and r + 1: the transposed elements as pairs
  auto put2 = [&](uint2 wv0, uint2 kv0, uint2 wv1, uint2 kv1) __attribute__((always_inline)) {
    const int p = pair_piece(tid, 0), r = p / (K / 4), c = 4 * (p % (K / 4));
    *(uint2*)&sWn[r][c] = make_uint2(wv0.x ^ 0x80008000u, wv0.y ^ 0x80008000u);
    *(uint2*)&sWn[r + 1][c] = make_uint2(wv1.x ^ 0x80008000u, wv1.y ^ 0x80008000u);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(uint32_t*)&sKbT[c + q][swz8(c + q, r)] = (uint32_t)elem4(kv0, q) | ((uint32_t)elem4(kv1, q) << 16);
  };
  const int64_t sbase = ((int64_t)n * H + h) * K * V;
  f32x4 st[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 16 * srt + 4 * lg + e, col = col0 + 16 * sct + ln;
      st[t][e] = a.init ? a.init[sbase + (int64_t)c * V + col] : 0.f;
    }
  }
  const int jc0 = a.seq_chunk0[n], jc1 = a.seq_chunk0[n + 1];
  auto chunk = [&](Pre& cur, const int j) __attribute__((always_inline)) {
    const int64_t chb = (int64_t)j * H + h;
    float* hc = b.hc + chb * K * V;
    float* Dc = b.Dc + chb * C * V;
    f32x4 acc = {__uint_as_float(cur.u4.x << 16), __uint_as_float(cur.u4.x & 0xffff0000u),
                 __uint_as_float(cur.u4.y << 16), __uint_as_float(cur.u4.y & 0xffff0000u)};
    float gl[TPW][4];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) gl[t][e] = cur.pgl[t][e];
    __syncthreads();  // the previous chunk is done with the LDS operands
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hc[(int64_t)(16 * srt + 4 * lg + e) * V + col0 + 16 * sct + ln] = st[t][e];
      uint2 hi, lo;
      split4_bf16(st[t], hi, lo);
      *(uint2*)&sSh[16 * sct + ln][16 * srt + 4 * lg] = hi;
      *(uint2*)&sSl[16 * sct + ln][16 * srt + 4 * lg] = lo;
    }
    if constexpr (NP == 2) put2(cur.pw0, cur.pk0, cur.pw1, cur.pk1);
    else put(tid, cur.pw0, cur.pk0);
    __builtin_amdgcn_sched_barrier(0);
    // the chunk two after this one (near the sequence end a chunk reads itself
    // again, unused)
    fetch(cur, j + 2 < jc1 ? chb + 2 * H : chb);
    __syncthreads();
    // Delta = U - W S
#pragma unroll
    for (int c0 = 0; c0 < K; c0 += 32) {
      const bf16x8 wa = frag8(&sWn[16 * drt + ln][c0 + 8 * lg]);
      acc = mfma_bf16(wa, frag8(&sSh[16 * dct + ln][c0 + 8 * lg]), acc);
      acc = mfma_bf16(wa, frag8(&sSl[16 * dct + ln][c0 + 8 * lg]), acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) Dc[(int64_t)(16 * drt + 4 * lg + e) * V + col0 + 16 * dct + ln] = acc[e];
    {
      uint2 hi, lo;
      split4_bf16(acc, hi, lo);
      *(uint2*)&sDh[16 * dct + ln][16 * drt + 4 * lg] = hi;
      *(uint2*)&sDl[16 * dct + ln][16 * drt + 4 * lg] = lo;
    }
    __syncthreads();
    // S = Diag(gL) S + Kbar^T Delta (rows past the chunk end are zero)
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) st[t][e] *= gl[t][e];
#pragma unroll
    for (int r0 = 0; r0 < C; r0 += 32) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
        const bf16x8 ka = frag8(&sKbT[16 * srt + ln][swz8(16 * srt + ln, r0 + 8 * lg)]);
        st[t] = mfma_bf16(ka, frag8(&sDh[16 * sct + ln][r0 + 8 * lg]), st[t]);
        st[t] = mfma_bf16(ka, frag8(&sDl[16 * sct + ln][r0 + 8 * lg]), st[t]);
      }
    }
  };
  if (jc0 < jc1) fetch(P0, (int64_t)jc0 * H + h);
  if (jc0 + 1 < jc1) fetch(P1, (int64_t)(jc0 + 1) * H + h);
  int j = jc0;
  for (; j + 1 < jc1; j += 2) {
    chunk(P0, j);
    chunk(P1, j + 1);
  }
  if (j < jc1) chunk(P0, j);
}

template <int K>
__global__ __launch_bounds__(1024) void k_bwd_dstate_bf(BwdArgs b) {
  constexpr int C = 64, NT = 1024, VT = 64;
  constexpr int TPW = K / 64;
  constexpr int WP = K + 8, TP = C + 8;
  const FwdArgs& a = b.f;
  const int H = a.H, V = a.V;
  const int ntile = V / VT;
  int tile;
  int64_t nh;
  chain_tile(blockIdx.x, gridDim.x, ntile, tile, nh);
  const int h = (int)(nh % H), n = (int)(nh / H);
  const int col0 = tile * VT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
  __shared__ __attribute__((aligned(16))) bf16 sAT[C][TP];   // Aqk_s^T
  __shared__ __attribute__((aligned(16))) bf16 sKb[C][WP];   // Kbar
  __shared__ __attribute__((aligned(16))) bf16 sQT[K][TP];   // Qt_s^T
  __shared__ __attribute__((aligned(16))) bf16 sWT[K][TP];   // -W^T
  __shared__ __attribute__((aligned(16))) bf16 sOT[VT][TP];  // dO^T (rows past the chunk end zero)
  __shared__ __attribute__((aligned(16))) bf16 sSh[VT][WP], sSl[VT][WP];  // dS^T hi, lo
  __shared__ __attribute__((aligned(16))) bf16 sDh[VT][TP], sDl[VT][TP];  // dDelta^T hi, lo
  constexpr int NP = C * K / 4 / NT;
  static_assert(NP == 1 || NP == 2, "one or two pieces per thread");
  static_assert(C * C / 4 == NT, "one Aqk piece per thread");
  uint2 pa, pk0, pk1, pq0, pq1, pw0, pw1;
  constexpr int NO = C * VT / NT;
  static_assert(NO * NT == C * VT, "whole dO tiles per thread");
  const bf16* dO = (const bf16*)b.d_o;
  bf16 po[NO];
  auto fetch = [&](int jn) __attribute__((always_inline)) {
    const int64_t chb = (int64_t)jn * H + h;
    const int tokn = a.chunk_tok[jn], Ln = a.chunk_len[jn];
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const int e = tid + u * NT, r = e / VT, cc = e % VT;
      po[u] = dO[((int64_t)(tokn + (r < Ln ? r : 0)) * H + h) * V + col0 + cc];
    }
    const uint2* A4 = (const uint2*)((const bf16*)a.Aqk + chb * C * C);
    const uint2* K4 = (const uint2*)((const bf16*)a.Kb + chb * C * K);
    const uint2* Q4 = (const uint2*)((const bf16*)a.Qt + chb * C * K);
    const uint2* W4 = (const uint2*)((const bf16*)a.W + chb * C * K);
    pa = A4[tid];
    if constexpr (NP == 2) {
      pk0 = K4[pair_piece(tid, 0)];
      pq0 = Q4[pair_piece(tid, 0)];
      pw0 = W4[pair_piece(tid, 0)];
      pk1 = K4[pair_piece(tid, 1)];
      pq1 = Q4[pair_piece(tid, 1)];
      pw1 = W4[pair_piece(tid, 1)];
    } else {
      pk0 = K4[tid];
      pq0 = Q4[tid];
      pw0 = W4[tid];
    }
  };
  auto put = [&](int p, uint2 kv, uint2 qv, uint2 wv) __attribute__((always_inline)) {
    const int r = p / (K / 4), c = 4 * (p % (K / 4));
    *(uint2*)&sKb[r][c] = kv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sQT[c + q][swz8(c + q, r)] = elem4(qv, q);
      sWT[c + q][swz8(c + q, r)] = elem4(wv, q) ^ 0x8000u;
    }
  };
  // two pieces of rows r (even) and r + 1: the transposed elements as pairs
  auto put2 = [&](uint2 kv0, uint2 qv0, uint2 wv0, uint2 kv1, uint2 qv1, uint2 wv1) __attribute__((always_inline)) {
    const int p = pair_piece(tid, 0), r = p / (K / 4), c = 4 * (p % (K / 4));
    *(uint2*)&sKb[r][c] = kv0;
    *(uint2*)&sKb[r + 1][c] = kv1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *(uint32_t*)&sQT[c + q][swz8(c + q, r)] = (uint32_t)elem4(qv0, q) | ((uint32_t)elem4(qv1, q) << 16);
      *(uint32_t*)&sWT[c + q][swz8(c + q, r)] = ((uint32_t)elem4(wv0, q) | ((uint32_t)elem4(wv1, q) << 16)) ^ 0x80008000u;
    }
  };
  const int64_t sbase = ((int64_t)n * H + h) * K * V;
  f32x4 st[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 16 * srt + 4 * lg + e, col = col0 + 16 * sct + ln;
      st[t][e] = b.d_fin ? b.d_fin[sbase + (int64_t)c * V + col] : 0.f;
    }
  }
  const int drt = w >> 2, dct = w & 3;
  const int jc0 = a.seq_chunk0[n], jc1 = a.seq_chunk0[n + 1];
  if (jc0 < jc1) fetch(jc1 - 1);
  for (int j = jc1 - 1; j >= jc0; --j) {
    const int64_t chb = (int64_t)j * H + h;
    const float* gL = a.gL + chb * K;
    float* dhc = b.dhc + chb * K * V;
    float* dDc = b.dDc + chb * C * V;
    const int L = a.chunk_len[j];
    __syncthreads();  // the previous chunk is done with the LDS operands
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dhc[(int64_t)(16 * srt + 4 * lg + e) * V + col0 + 16 * sct + ln] = st[t][e];
      uint2 hi, lo;
      split4_bf16(st[t], hi, lo);
      *(uint2*)&sSh[16 * sct + ln][16 * srt + 4 * lg] = hi;
      *(uint2*)&sSl[16 * sct + ln][16 * srt + 4 * lg] = lo;
    }
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const int e = tid + u * NT, r = e / VT, cc = e % VT;
      sOT[cc][swz8(cc, r)] = r < L ? po[u] : (bf16)0;
    }
    {
      const int rr = tid / (C / 4), i = 4 * (tid % (C / 4));
#pragma unroll
      for (int q = 0; q < 4; ++q) sAT[i + q][swz8(i + q, rr)] = elem4(pa, q);
    }
    if constexpr (NP == 2) put2(pk0, pq0, pw0, pk1, pq1, pw1);
    else put(tid, pk0, pq0, pw0);
    float gl[TPW][4];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) gl[t][e] = gL[16 * ((w * TPW + t) >> 2) + 4 * lg + e];
    // the previous chunk of this sequence, after gL's loads (held there by the
    // scheduling barrier) so that waiting for gL leaves it in flight; the
    // first chunk reads itself again, unused
    __builtin_amdgcn_sched_barrier(0);
    fetch(j - 1 >= jc0 ? j - 1 : j);
    __syncthreads();
    // dDelta = Aqk_s^T dO + Kbar dS_L (Aqk_s[rr][r] is zero for rr < r: the
    // row tiles from 32 on skip the first k-step)
    {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r0 = 0; r0 < C; r0 += 32)
        if (16 * drt < r0 + 32)
          acc = mfma_bf16(frag8(&sAT[16 * drt + ln][swz8(16 * drt + ln, r0 + 8 * lg)]),
                          frag8(&sOT[16 * dct + ln][swz8(16 * dct + ln, r0 + 8 * lg)]), acc);
#pragma unroll
      for (int c0 = 0; c0 < K; c0 += 32) {
        const bf16x8 ka = frag8(&sKb[16 * drt + ln][c0 + 8 * lg]);
        acc = mfma_bf16(ka, frag8(&sSh[16 * dct + ln][c0 + 8 * lg]), acc);
        acc = mfma_bf16(ka, frag8(&sSl[16 * dct + ln][c0 + 8 * lg]), acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) dDc[(int64_t)(16 * drt + 4 * lg + e) * V + col0 + 16 * dct + ln] = acc[e];
      uint2 hi, lo;
      split4_bf16(acc, hi, lo);
      *(uint2*)&sDh[16 * dct + ln][16 * drt + 4 * lg] = hi;
      *(uint2*)&sDl[16 * dct + ln][16 * drt + 4 * lg] = lo;
    }
    __syncthreads();
    // dS0 = Diag(gL) dS_L + Qt_s^T dO - W^T dDelta (rows past the chunk end are zero)
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) st[t][e] *= gl[t][e];
#pragma unroll
    for (int r0 = 0; r0 < C; r0 += 32) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
        st[t] = mfma_bf16(frag8(&sQT[16 * srt + ln][swz8(16 * srt + ln, r0 + 8 * lg)]),
                          frag8(&sOT[16 * sct + ln][swz8(16 * sct + ln, r0 + 8 * lg)]), st[t]);
        const bf16x8 wa = frag8(&sWT[16 * srt + ln][swz8(16 * srt + ln, r0 + 8 * lg)]);
        st[t] = mfma_bf16(wa, frag8(&sDh[16 * sct + ln][r0 + 8 * lg]), st[t]);
        st[t] = mfma_bf16(wa, frag8(&sDl[16 * sct + ln][r0 + 8 * lg]), st[t]);
      }
    }
  }
  if (b.dinit) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int s = w * TPW + t, srt = s >> 2, sct = s & 3;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        b.dinit[sbase + (int64_t)(16 * srt + 4 * lg + e) * V + col0 + 16 * sct + ln] = st[t][e];
    }
  }
}

// Chunk-local gradients.  One workgroup per chunk-head.
//
// Thread layouts (NT threads): C x K elements (r, c) are owned as c = tid % K,
// r = tid / K + (NT / K) m, so a wave shares its rows (broadcast LDS reads) and
// its lanes hold consecutive channels (coalesced global access); C x C
// elements (r, i) likewise with i = tid % C (a row's C lanes sit in one wave).
// The products over the value dimension (dW, dQ~, dKbar, P, the V half of Y,
// and dV) run in two sweeps over 32-column tiles of S0, dS_L, dDelta, dO,
// Delta and V staged in LDS; everything after that reads LDS, and each
// element's partial terms stay in its owner's registers between phases.
template <typename Tin, int C, int K, int NT>
__global__ __launch_bounds__(NT) void k_bwd_chunk(BwdArgs b) {
  constexpr int VTL = 32, TS = VTL + 4;  // value tile and its padded row stride
  constexpr int NE1 = C * K / NT, NE2 = (C * C + NT - 1) / NT;
  constexpr int RSTEP1 = NT / K, RSTEP2 = NT / C;
  constexpr int NEV = (C * VTL + NT - 1) / NT;  // dV elements per thread and tile
  // bf16 inputs at 64-token chunks: the value-dimension products on bf16
  // matrix cores with split operands (see phase B)
  constexpr bool BF = std::is_same<Tin, bf16>::value && C == 64;
  const FwdArgs& a = b.f;
  const int H = a.H, V = a.V;
  const int64_t wid = blockIdx.x;
  const int j = (int)(wid / H), h = (int)(wid % H);
  if (j >= *a.nt_dev) return;
  const int tid = threadIdx.x;
  const int tok0 = a.chunk_tok[j], L = a.chunk_len[j];
  const int64_t chb = (int64_t)j * H + h;
  auto th = [&](int r) { return (int64_t)(tok0 + r) * H + h; };
  // q^ and k^ rebuilt from the raw q and k of the key head this value head
  // reads and the recomputation's norm scales (the same fp32 product as there):
  // one element, or the 4 channels 4 c4 .. 4 c4 + 3 (one 8- or 16-byte load
  // when the inputs allow it)
  const int64_t hk = h / (H / a.HK);
  auto thk = [&](int r) { return (int64_t)(tok0 + r) * a.HK + hk; };
  auto khat = [&](int r, int c) { return load_f32((const Tin*)a.k + thk(r) * K + c) * a.rk[th(r)]; };
  const bool vec_in = (((uintptr_t)a.q | (uintptr_t)a.k) % (4 * sizeof(Tin))) == 0;
  auto hat4 = [&](const Tin* x, const float* rs, int r, int c4) {
    const Tin* p = x + thk(r) * K + 4 * c4;
    float f[4];
    if constexpr (std::is_same<Tin, bf16>::value) {
      if (vec_in) {
        const uint2 u = *(const uint2*)p;
        f[0] = __uint_as_float(u.x << 16);
        f[1] = __uint_as_float(u.x & 0xffff0000u);
        f[2] = __uint_as_float(u.y << 16);
        f[3] = __uint_as_float(u.y & 0xffff0000u);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = load_f32(p + e);
      }
    } else {
      if (vec_in) {
        const float4 u = *(const float4*)p;
        f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = p[e];
      }
    }
    const float s = rs[th(r)];
    return make_float4(f[0] * s, f[1] * s, f[2] * s, f[3] * s);
  };
  const float* Akk = a.Akk_out + chb * C * C;
  const float* S0 = b.hc + chb * K * V;
  const float* dSL = b.dhc + chb * K * V;
  const float* Dl = b.Dc + chb * C * V;
  const float* dDl = b.dDc + chb * C * V;
  const Tin* dO = (const Tin*)b.d_o;
  const Tin* v = (const Tin*)a.v;
  const float scale = a.scale;

  // LDS: gamma and Tm for the whole kernel; one region reused by phase.
  // dW's rows are padded to DWS floats: phase C's matrix-core loop reads it
  // down columns (16 rows per k-step), which a 128-float stride puts in one
  // bank; 4 extra floats spread them and keep rows 16-byte aligned
  constexpr int DWS = K + 4;
  constexpr int kTiles = C * DWS + 2 * K * (VTL + 1) + 4 * C * TS;
  constexpr int kAfter = C * DWS + 2 * C * (C + 1) + K * (C + 1);
  constexpr int kRegion = kTiles > kAfter ? kTiles : kAfter;
  __shared__ float sGam[C][K];
  __shared__ float sT[C][C + 1];
  __shared__ __attribute__((aligned(16))) float sReg[kRegion];
  __shared__ float sB[C], sDb[C], sSd[K], sRed[K];
  // phase B, first sweep's tiles
  float (*tS0)[VTL + 1] = (float(*)[VTL + 1])sReg;
  float (*tdD)[TS] = (float(*)[TS])(sReg + K * (VTL + 1));
  float (*tdO)[TS] = (float(*)[TS])(sReg + K * (VTL + 1) + C * TS);
  // after phase B: dW | P | Y (then dAkk) | K~ transposed (then Z); after phase
  // D, q^ takes dW's place; after phase E, k^ takes Z's; after phase F, dgamma
  // and the Kbar term take those two places
  float (*sDW)[DWS] = (float(*)[DWS])sReg;
  float (*sP)[C + 1] = (float(*)[C + 1])(sReg + C * DWS);
  float (*sY)[C + 1] = (float(*)[C + 1])(sReg + C * DWS + C * (C + 1));
  float* sR4 = sReg + C * DWS + 2 * C * (C + 1);
  float (*sKtT)[C + 1] = (float(*)[C + 1])sR4;
  float (*sZ)[C + 1] = (float(*)[C + 1])sR4;
  float (*sQn)[K] = (float(*)[K])sReg;
  float (*sKn)[K] = (float(*)[K])sR4;
  float (*sDg)[K] = (float(*)[K])sReg;
  float (*sTk)[K] = (float(*)[K])sR4;

  // ---- phase A: gamma, beta, Tm ----
  // The chunk's gate g = gate(x + dt_bias) reaches LDS first, every thread
  // taking 4-channel pieces of the raw gate (rows past the chunk end are zero);
  // then each channel's thread adds down its column.  Loads under a row
  // condition read a clamped, valid row and select afterwards: a load under a
  // condition of its own is waited for on the spot.
  {
    constexpr int NP = (C * K / 4 + NT - 1) / NT;
    const float Ag = expf(a.a_log[h]);  // as in the gate's derivative below
    const float* dbh = a.dt_bias + (int64_t)h * K;
    const bool vec_g = ((uintptr_t)a.gate % (4 * sizeof(Tin))) == 0 && ((uintptr_t)dbh % 16) == 0;
    float4 gq[NP];
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int p = 4 * (tid + u * NT), r = p / K, c = p % K;
      const bool in = p < C * K && r < L;
      const Tin* gp = (const Tin*)a.gate + th(in ? r : 0) * K + (in ? c : 0);
      float x[4];
      if constexpr (std::is_same<Tin, bf16>::value) {
        if (vec_g) {
          const uint2 w = *(const uint2*)gp;
          x[0] = __uint_as_float(w.x << 16);
          x[1] = __uint_as_float(w.x & 0xffff0000u);
          x[2] = __uint_as_float(w.y << 16);
          x[3] = __uint_as_float(w.y & 0xffff0000u);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = load_f32(gp + e);
        }
      } else {
        if (vec_g) {
          const float4 w = *(const float4*)gp;
          x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = gp[e];
        }
      }
      const int cc = in ? c : 0;
      const float4 db = vec_g ? *(const float4*)(dbh + cc) : make_float4(dbh[cc], dbh[cc + 1], dbh[cc + 2], dbh[cc + 3]);
      gq[u] = in ? make_float4(gate_value(x[0] + db.x, Ag, a.gate_form, a.lb),
                               gate_value(x[1] + db.y, Ag, a.gate_form, a.lb),
                               gate_value(x[2] + db.z, Ag, a.gate_form, a.lb),
                               gate_value(x[3] + db.w, Ag, a.gate_form, a.lb))
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int r = tid; r < C; r += NT) {
      const float x = a.bt[th(r < L ? r : 0)];
      sB[r] = r < L ? x : 0.f;
      sDb[r] = 0.f;
    }
    for (int p = tid; p < C * C; p += NT) sT[p / C][p % C] = a.Tm_out[chb * C * C + p];
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int p = 4 * (tid + u * NT), r = p / K, c = p % K;
      if (p < C * K) {
        sGam[r][c] = gq[u].x;
        sGam[r][c + 1] = gq[u].y;
        sGam[r][c + 2] = gq[u].z;
        sGam[r][c + 3] = gq[u].w;
      }
    }
  }
  __syncthreads();
  // each channel's column: all C rows read first (independent LDS reads),
  // then summed down in registers and written back
  for (int c = tid; c < K; c += NT) {
    float col[C];
#pragma unroll
    for (int r = 0; r < C; ++r) col[r] = sGam[r][c];
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      acc += col[r];
      sGam[r][c] = acc;
    }
  }

  // ---- phase B: products over the value dimension, and dV, over 32-column
  //      value tiles staged in LDS (dW, dQ~, dKbar, P, the V half of Y and
  //      dV).  For C = 64 the products run on the matrix cores, each wave
  //      owning fixed 16 x 16 output tiles, the results reaching the thread
  //      layouts below through LDS: for bf16 inputs in one sweep on bf16
  //      matrix cores with split operands (below); for fp32 inputs in two
  //      sweeps (dW and dQ~; then dKbar, P, Y and dV) in fp32
  //      (v_mfma_f32_16x16x4f32: lane l holds A[l%16][l/16], B[l/16][l%16] and
  //      D[4(l/16)+e][l%16]).  Smaller chunks keep per-thread VALU accumulators.
  const int c1 = tid % K, rb1 = tid / K;       // C x K layout
  const int i2 = tid % C, rb2 = tid / C;       // C x C layout
  Tin* dv = (Tin*)b.dv;
  float dqs[NE1];  // scale dO S0^T, kept until phase F
  float dkb[NE1], sd = 0.f;
  if constexpr (BF) {
    // bf16 inputs: one sweep over 32-column value tiles.  Each tile of S0,
    // dS_L, Delta and dDelta reaches LDS as bf16 hi + lo pairs (dO and V
    // exactly), rows padded to BP (16-byte fragment reads), and is one k-step
    // of every product on the bf16 matrix cores (hi*hi + hi*lo + lo*hi per
    // pair of split operands, fp32 accumulation):
    //   M1 = dDelta S0^T (-> -dW), M2 = dO S0^T (-> dQ~), M3 = Delta dS_L^T (-> dKbar),
    //   P = dO Delta^T and Yv = dDelta V^T (lower tiles); dV = Diag(beta) Tm^T dDelta
    //   on the fp32 matrix cores with dDelta from its pair.
    // Each tile reaches registers one tile ahead of its products, every thread
    // taking one 4-column piece of a row of S0 and dS_L and one NR-column piece
    // of a row of Delta, dDelta, dO and V (16-, 8- and 4-byte loads, 8- and
    // 4-byte LDS writes); rowsum(S0 . dS_L) comes from those registers.
    constexpr int NW = NT / 64;
    const int lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
    static_assert(2 * NW * 16 * 16 == C * K, "two output tiles per wave and product");
    static_assert(VTL == 32, "one bf16 k-step per value tile");
    const int rt = w & 3, ct0 = 2 * (w >> 2);  // M1..M3 tiles: row tile rt, column tiles ct0, ct0 + 1
    constexpr int NS = K * VTL / NT, NR = C * VTL / NT;
    static_assert(NS * NT == K * VTL && NR * NT == C * VTL, "whole tiles per thread");
    static_assert(NS == 4 && (NR == 2 || NR == 4), "one piece of each operand per thread");
    // this thread's pieces: S0 / dS_L row sc, columns sj .. sj + 3; Delta,
    // dDelta, dO, V row rr, columns rj .. rj + NR - 1 (of the value tile)
    const int sc = tid / (VTL / 4), sj = 4 * (tid % (VTL / 4));
    const int rr = tid / (VTL / NR), rj = NR * (tid % (VTL / NR));
    const bool vec_ov = ((uintptr_t)dO % (NR * sizeof(Tin))) == 0 && ((uintptr_t)v % (NR * sizeof(Tin))) == 0;
    constexpr int BP = VTL + 8;
    bf16 (*hS0)[BP] = (bf16(*)[BP])sReg;
    bf16 (*lS0)[BP] = hS0 + K;
    bf16 (*hSL)[BP] = lS0 + K;
    bf16 (*lSL)[BP] = hSL + K;
    bf16 (*hD)[BP] = lSL + K;
    bf16 (*lD)[BP] = hD + C;
    bf16 (*hdD)[BP] = lD + C;
    bf16 (*ldD)[BP] = hdD + C;
    bf16 (*hdO)[BP] = ldD + C;
    bf16 (*hv)[BP] = hdO + C;
    static_assert((4 * K + 6 * C) * BP * 2 <= kRegion * 4, "the tiles fit the region");
    constexpr int NTRI = 10;                  // lower 16 x 16 tiles (rt >= it) of a 64 x 64 matrix
    constexpr int NPY = (NTRI + NW - 1) / NW;  // P and Yv tile pairs per wave
    auto tri_tile = [](int t, int& r, int& i) {  // t = R (R + 1) / 2 + I, I <= R
      r = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
      i = t - r * (r + 1) / 2;
    };
    // dV tile of this wave (waves 0..7): row tile w / 2, column tile w % 2 of the value tile
    const bool has_dv = w < 8;
    const int vrt = (w >> 1) & 3, vct = w & 1;
    f32x4 m1[2], m2[2], m3[2], pt[NPY], yt[NPY];
#pragma unroll
    for (int t = 0; t < 2; ++t) m1[t] = m2[t] = m3[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NPY; ++u) pt[u] = yt[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    // 512-thread workgroups (K = 64) keep two tiles in flight: tile t's loads
    // are issued two steps ahead of its products, into the register set of
    // its parity
    struct Tile { f32x4 s, l; float D[NR], d[NR], o[NR], v[NR]; };
    Tile ta, tb;
    float sdp = 0.f;
    auto fetch = [&](Tile& x, int j0) __attribute__((always_inline)) {
      const float4 s4 = *(const float4*)(S0 + (int64_t)sc * V + j0 + sj);
      const float4 l4 = *(const float4*)(dSL + (int64_t)sc * V + j0 + sj);
      x.s = f32x4{s4.x, s4.y, s4.z, s4.w};
      x.l = f32x4{l4.x, l4.y, l4.z, l4.w};
      const int64_t dr = (int64_t)rr * V + j0 + rj;
      if constexpr (NR == 2) {
        const float2 d2 = *(const float2*)(dDl + dr), D2 = *(const float2*)(Dl + dr);
        x.d[0] = d2.x; x.d[1] = d2.y;
        x.D[0] = D2.x; x.D[1] = D2.y;
      } else {
        const float4 d4 = *(const float4*)(dDl + dr), D4 = *(const float4*)(Dl + dr);
        x.d[0] = d4.x; x.d[1] = d4.y; x.d[2] = d4.z; x.d[3] = d4.w;
        x.D[0] = D4.x; x.D[1] = D4.y; x.D[2] = D4.z; x.D[3] = D4.w;
      }
      // rows past the chunk end read row 0 and are zeroed after the loads
      const bool in = rr < L;
      const int64_t rv = th(in ? rr : 0) * V + j0 + rj;
      float fo[NR], fv[NR];
      if (vec_ov) {
        uint32_t uo[NR / 2], uv[NR / 2];
        if constexpr (NR == 2) {
          uo[0] = *(const uint32_t*)(dO + rv);
          uv[0] = *(const uint32_t*)(v + rv);
        } else {
          const uint2 o2 = *(const uint2*)(dO + rv), v2 = *(const uint2*)(v + rv);
          uo[0] = o2.x; uo[1] = o2.y;
          uv[0] = v2.x; uv[1] = v2.y;
        }
#pragma unroll
        for (int q = 0; q < NR / 2; ++q) {
          fo[2 * q] = __uint_as_float(uo[q] << 16);
          fo[2 * q + 1] = __uint_as_float(uo[q] & 0xffff0000u);
          fv[2 * q] = __uint_as_float(uv[q] << 16);
          fv[2 * q + 1] = __uint_as_float(uv[q] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < NR; ++e) {
          fo[e] = load_f32(dO + rv + e);
          fv[e] = load_f32(v + rv + e);
        }
      }
#pragma unroll
      for (int e = 0; e < NR; ++e) {
        x.o[e] = in ? fo[e] : 0.f;
        x.v[e] = in ? fv[e] : 0.f;
      }
    };
    // NR values as bf16 in LDS, NR / 2 words
    auto put_bf16 = [&](bf16* dst, const float* f) __attribute__((always_inline)) {
      uint32_t wds[NR / 2];
#pragma unroll
      for (int q = 0; q < NR / 2; ++q)
        wds[q] = (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)f[2 * q]) |
                 ((uint32_t)__builtin_bit_cast(unsigned short, (__bf16)f[2 * q + 1]) << 16);
      if constexpr (NR == 2) *(uint32_t*)dst = wds[0];
      else *(uint2*)dst = make_uint2(wds[0], wds[1]);
    };
    // NR values as bf16 hi + lo parts (hi = bf16(x), lo = bf16(x - hi))
    auto put_split = [&](bf16* dhi, bf16* dlo, const float* f) __attribute__((always_inline)) {
      float hv_[NR], lv_[NR];
#pragma unroll
      for (int e = 0; e < NR; ++e) {
        hv_[e] = (float)(__bf16)f[e];
        lv_[e] = f[e] - hv_[e];
      }
      put_bf16(dhi, hv_);
      put_bf16(dlo, lv_);
    };
    auto stage = [&](const Tile& x) __attribute__((always_inline)) {
      uint2 hi, lo;
      split4_bf16(x.s, hi, lo);
      *(uint2*)&hS0[sc][sj] = hi;
      *(uint2*)&lS0[sc][sj] = lo;
      split4_bf16(x.l, hi, lo);
      *(uint2*)&hSL[sc][sj] = hi;
      *(uint2*)&lSL[sc][sj] = lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) sdp = fmaf(x.s[e], x.l[e], sdp);
      put_split(&hdD[rr][rj], &ldD[rr][rj], x.d);
      put_split(&hD[rr][rj], &lD[rr][rj], x.D);
      put_bf16(&hdO[rr][rj], x.o);
      put_bf16(&hv[rr][rj], x.v);
    };
    auto products = [&](const int j0) __attribute__((always_inline)) {
      {
        const int ar = 16 * rt + ln;
        const bf16x8 dh = frag8(&hdD[ar][8 * lg]), dl = frag8(&ldD[ar][8 * lg]);
        const bf16x8 o8 = frag8(&hdO[ar][8 * lg]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int cr = 16 * (ct0 + t) + ln;
          const bf16x8 sh = frag8(&hS0[cr][8 * lg]), sl = frag8(&lS0[cr][8 * lg]);
          m1[t] = mfma_bf16(dh, sh, m1[t]);
          m1[t] = mfma_bf16(dh, sl, m1[t]);
          m1[t] = mfma_bf16(dl, sh, m1[t]);
          m2[t] = mfma_bf16(o8, sh, m2[t]);
          m2[t] = mfma_bf16(o8, sl, m2[t]);
        }
      }
      {
        const int ar = 16 * rt + ln;
        const bf16x8 Dh = frag8(&hD[ar][8 * lg]), Dl8 = frag8(&lD[ar][8 * lg]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int cr = 16 * (ct0 + t) + ln;
          const bf16x8 Lh = frag8(&hSL[cr][8 * lg]), Ll = frag8(&lSL[cr][8 * lg]);
          m3[t] = mfma_bf16(Dh, Lh, m3[t]);
          m3[t] = mfma_bf16(Dh, Ll, m3[t]);
          m3[t] = mfma_bf16(Dl8, Lh, m3[t]);
        }
      }
#pragma unroll
      for (int u = 0; u < NPY; ++u) {
        const int t = w + NW * u;
        if (t < NTRI) {
          int R, I;
          tri_tile(t, R, I);
          const bf16x8 o8 = frag8(&hdO[16 * R + ln][8 * lg]);
          pt[u] = mfma_bf16(o8, frag8(&hD[16 * I + ln][8 * lg]), pt[u]);
          pt[u] = mfma_bf16(o8, frag8(&lD[16 * I + ln][8 * lg]), pt[u]);
          const bf16x8 v8 = frag8(&hv[16 * I + ln][8 * lg]);
          yt[u] = mfma_bf16(frag8(&hdD[16 * R + ln][8 * lg]), v8, yt[u]);
          yt[u] = mfma_bf16(frag8(&ldD[16 * R + ln][8 * lg]), v8, yt[u]);
        }
      }
      if (has_dv) {
        // dV rows 16 vrt .. + 15, value columns j0 + 16 vct .. + 15: the sum over
        // a >= r of Tm[a][r] dDelta[a][j] (Tm is lower triangular)
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int a0 = 16 * vrt; a0 < C; a0 += 4) {
          const int ar = a0 + lg, ac = 16 * vct + ln;
          acc = mfma_f32(sT[ar][16 * vrt + ln], bf16_to_f32(hdD[ar][ac]) + bf16_to_f32(ldD[ar][ac]), acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * vrt + 4 * lg + e;
          if (r < L) store_as(dv + th(r) * V + j0 + 16 * vct + ln, sB[r] * acc[e]);
        }
      }
    };
    if constexpr (NT <= 512) {
      static_assert(2 * VTL == 64, "V (64 or 128) is a whole number of tile pairs");
      fetch(ta, 0);
      fetch(tb, VTL);
      for (int j0 = 0; j0 < V; j0 += 2 * VTL) {
        __syncthreads();  // the previous tile's products are done
        stage(ta);
        if (j0 + 2 * VTL < V) fetch(ta, j0 + 2 * VTL);
        __syncthreads();
        products(j0);
        __syncthreads();
        stage(tb);
        if (j0 + 3 * VTL < V) fetch(tb, j0 + 3 * VTL);
        __syncthreads();
        products(j0 + VTL);
      }
    } else {
      // 1024 threads: 128 registers leave room for one tile in flight only
      fetch(ta, 0);
      for (int j0 = 0; j0 < V; j0 += VTL) {
        __syncthreads();
        stage(ta);
        if (j0 + VTL < V) fetch(ta, j0 + VTL);
        __syncthreads();
        products(j0);
      }
    }
    // rowsum(S0 . dS_L): each row's pieces sit in 8 consecutive lanes
    sdp += __shfl_xor(sdp, 1);
    sdp += __shfl_xor(sdp, 2);
    sdp += __shfl_xor(sdp, 4);
    if (sj == 0) sSd[sc] = sdp;
    __syncthreads();  // the tiles are dead: dW, then dQ~ and dKbar on their way to registers
    float (*sX)[K] = (float(*)[K])(sReg + C * DWS);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * lg + e, c = 16 * (ct0 + t) + ln;
        sDW[r][c] = -m1[t][e];
        sX[r][c] = scale * m2[t][e];
      }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NE1; ++m) dqs[m] = sX[rb1 + RSTEP1 * m][c1];
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) sX[16 * rt + 4 * lg + e][16 * (ct0 + t) + ln] = m3[t][e];
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NE1; ++m) dkb[m] = sX[rb1 + RSTEP1 * m][c1];
    __syncthreads();  // sX is dead: P, Y and K~^T take its place
#pragma unroll
    for (int m = 0; m < NE1; ++m) {
      const int r = rb1 + RSTEP1 * m;
      const float x = khat(r < L ? r : 0, c1);
      sKtT[c1][r] = r < L ? x * __expf(sGam[r][c1]) : 0.f;
    }
    // P (scaled) and the V half of Y, lower triangle i <= r < L; zero elsewhere
    for (int e = tid; e < C * C; e += NT) {
      const int r = e / C, i = e % C;
      if ((i >> 4) > (r >> 4)) sP[r][i] = sY[r][i] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < NPY; ++u) {
      const int t = w + NW * u;
      if (t < NTRI) {
        int R, I;
        tri_tile(t, R, I);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * R + 4 * lg + e, i = 16 * I + ln;
          const bool low = i <= r && r < L;
          sP[r][i] = low ? scale * pt[u][e] : 0.f;
          sY[r][i] = low ? yt[u][e] : 0.f;
        }
      }
    }
    __syncthreads();
  } else if constexpr (C == 64) {
    constexpr int NW = NT / 64;
    const int lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
    // dW, dQ~ and dKbar tiles: row tile rt, column tiles 2 (w / 4) + {0, 1}
    static_assert(2 * NW * 16 * 16 == C * K, "two output tiles per wave and product");
    const int rt = w & 3, ct0 = 2 * (w >> 2);
    // sweep 1: M1 = dDelta S0^T (-> -dW), M2 = dO S0^T (-> dQ~)
    f32x4 m1[2], m2[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) m1[t] = m2[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // each value tile is read into registers one tile ahead, so its loads are
    // in flight while the previous tile's products run
    constexpr int NS = K * VTL / NT, NR = C * VTL / NT;
    static_assert(NS * NT == K * VTL && NR * NT == C * VTL, "whole tiles per thread");
    float ps[NS], pd[NR], po[NR];
    auto fetch1 = [&](int j0) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int e = tid + NT * u, c = e / VTL, jj = e % VTL;
        ps[u] = S0[(int64_t)c * V + j0 + jj];
      }
#pragma unroll
      for (int u = 0; u < NR; ++u) {
        const int e = tid + NT * u, r = e / VTL, jj = e % VTL;
        pd[u] = dDl[(int64_t)r * V + j0 + jj];
        const float x = load_f32(dO + th(r < L ? r : 0) * V + j0 + jj);
        po[u] = r < L ? x : 0.f;
      }
    };
    fetch1(0);
    for (int j0 = 0; j0 < V; j0 += VTL) {
      __syncthreads();
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int e = tid + NT * u;
        tS0[e / VTL][e % VTL] = ps[u];
      }
#pragma unroll
      for (int u = 0; u < NR; ++u) {
        const int e = tid + NT * u;
        tdD[e / VTL][e % VTL] = pd[u];
        tdO[e / VTL][e % VTL] = po[u];
      }
      if (j0 + VTL < V) fetch1(j0 + VTL);
      __syncthreads();
#pragma unroll
      for (int jj = 0; jj < VTL; jj += 4) {
        const float ad = tdD[16 * rt + ln][jj + lg], ao = tdO[16 * rt + ln][jj + lg];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float bs = tS0[16 * (ct0 + t) + ln][jj + lg];
          m1[t] = mfma_f32(ad, bs, m1[t]);
          m2[t] = mfma_f32(ao, bs, m2[t]);
        }
      }
    }
    __syncthreads();  // the tiles are dead: dW, and dQ~ on its way to registers
    float (*sX)[K] = (float(*)[K])(sReg + C * DWS);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * lg + e, c = 16 * (ct0 + t) + ln;
        sDW[r][c] = -m1[t][e];
        sX[r][c] = scale * m2[t][e];
      }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NE1; ++m) dqs[m] = sX[rb1 + RSTEP1 * m][c1];
    // sweep 2: M3 = Delta dS_L^T (-> dKbar), P = dO Delta^T and Yv = dDelta V^T
    // (lower tiles only), dV = Diag(beta) Tm^T dDelta per value tile
    float* sReg2 = sReg + C * DWS;
    float (*tdSL2)[VTL + 1] = (float(*)[VTL + 1])sReg2;
    float (*tD2)[TS] = (float(*)[TS])(sReg2 + K * (VTL + 1));
    float (*tdO2)[TS] = (float(*)[TS])(sReg2 + K * (VTL + 1) + C * TS);
    float (*tdD2)[TS] = (float(*)[TS])(sReg2 + K * (VTL + 1) + 2 * C * TS);
    float (*tv2)[TS] = (float(*)[TS])(sReg2 + K * (VTL + 1) + 3 * C * TS);
    float (*tS02)[VTL + 1] = (float(*)[VTL + 1])(sReg2 + K * (VTL + 1) + 4 * C * TS);
    constexpr int NTRI = 10;                  // lower 16 x 16 tiles (rt >= it) of a 64 x 64 matrix
    constexpr int NPY = (NTRI + NW - 1) / NW;  // P and Yv tile pairs per wave
    f32x4 m3[2], pt[NPY], yt[NPY];
#pragma unroll
    for (int t = 0; t < 2; ++t) m3[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NPY; ++u) pt[u] = yt[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto tri_tile = [](int t, int& r, int& i) {  // t = R (R + 1) / 2 + I, I <= R
      r = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
      i = t - r * (r + 1) / 2;
    };
    // dV tile of this wave (waves 0..7): row tile w / 2, column tile w % 2 of the value tile
    const bool has_dv = w < 8;
    const int vrt = (w >> 1) & 3, vct = w & 1;
    float qs[NS], ql[NS], qd[NR], qD[NR], qo[NR], qv[NR];
    auto fetch2 = [&](int j0) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int e = tid + NT * u, c = e / VTL, jj = e % VTL;
        ql[u] = dSL[(int64_t)c * V + j0 + jj];
        qs[u] = S0[(int64_t)c * V + j0 + jj];
      }
#pragma unroll
      for (int u = 0; u < NR; ++u) {
        const int e = tid + NT * u, r = e / VTL, jj = e % VTL;
        const bool in = r < L;
        qd[u] = dDl[(int64_t)r * V + j0 + jj];
        qD[u] = Dl[(int64_t)r * V + j0 + jj];
        const int64_t rv = th(in ? r : 0) * V + j0 + jj;
        const float xo = load_f32(dO + rv), xv = load_f32(v + rv);
        qo[u] = in ? xo : 0.f;
        qv[u] = in ? xv : 0.f;
      }
    };
    fetch2(0);
    for (int j0 = 0; j0 < V; j0 += VTL) {
      __syncthreads();
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int e = tid + NT * u;
        tdSL2[e / VTL][e % VTL] = ql[u];
        tS02[e / VTL][e % VTL] = qs[u];
      }
#pragma unroll
      for (int u = 0; u < NR; ++u) {
        const int e = tid + NT * u;
        tdD2[e / VTL][e % VTL] = qd[u];
        tD2[e / VTL][e % VTL] = qD[u];
        tdO2[e / VTL][e % VTL] = qo[u];
        tv2[e / VTL][e % VTL] = qv[u];
      }
      if (j0 + VTL < V) fetch2(j0 + VTL);
      __syncthreads();
      if (tid < K) {
        const int c = tid;
#pragma unroll 8
        for (int jj = 0; jj < VTL; ++jj) sd = fmaf(tS02[c][jj], tdSL2[c][jj], sd);
      }
#pragma unroll
      for (int jj = 0; jj < VTL; jj += 4) {
        const float ad = tD2[16 * rt + ln][jj + lg];
#pragma unroll
        for (int t = 0; t < 2; ++t) m3[t] = mfma_f32(ad, tdSL2[16 * (ct0 + t) + ln][jj + lg], m3[t]);
#pragma unroll
        for (int u = 0; u < NPY; ++u) {
          const int t = w + NW * u;
          if (t < NTRI) {
            int R, I;
            tri_tile(t, R, I);
            pt[u] = mfma_f32(tdO2[16 * R + ln][jj + lg], tD2[16 * I + ln][jj + lg], pt[u]);
            yt[u] = mfma_f32(tdD2[16 * R + ln][jj + lg], tv2[16 * I + ln][jj + lg], yt[u]);
          }
        }
      }
      if (has_dv) {
        // dV rows 16 vrt .. + 15, value columns j0 + 16 vct .. + 15: the sum over
        // a >= r of Tm[a][r] dDelta[a][j] (Tm is lower triangular)
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int a0 = 16 * vrt; a0 < C; a0 += 4)
          acc = mfma_f32(sT[a0 + lg][16 * vrt + ln], tdD2[a0 + lg][16 * vct + ln], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * vrt + 4 * lg + e;
          if (r < L) store_as(dv + th(r) * V + j0 + 16 * vct + ln, sB[r] * acc[e]);
        }
      }
    }
    __syncthreads();  // the tiles are dead: dKbar on its way to registers
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) sX[16 * rt + 4 * lg + e][16 * (ct0 + t) + ln] = m3[t][e];
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NE1; ++m) dkb[m] = sX[rb1 + RSTEP1 * m][c1];
    __syncthreads();  // sX is dead: P, Y and K~^T take its place
#pragma unroll
  for (int m = 0; m < NE1; ++m) {
    const int r = rb1 + RSTEP1 * m;
    const float x = khat(r < L ? r : 0, c1);
    sKtT[c1][r] = r < L ? x * __expf(sGam[r][c1]) : 0.f;
  }
    // P (scaled) and the V half of Y, lower triangle i <= r < L; zero elsewhere
    for (int e = tid; e < C * C; e += NT) {
      const int r = e / C, i = e % C;
      if ((i >> 4) > (r >> 4)) sP[r][i] = sY[r][i] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < NPY; ++u) {
      const int t = w + NW * u;
      if (t < NTRI) {
        int R, I;
        tri_tile(t, R, I);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * R + 4 * lg + e, i = 16 * I + ln;
          const bool low = i <= r && r < L;
          sP[r][i] = low ? scale * pt[u][e] : 0.f;
          sY[r][i] = low ? yt[u][e] : 0.f;
        }
      }
    }
    if (tid < K) sSd[tid] = sd;
    __syncthreads();
  } else {
  {
    float dw[NE1], dqt[NE1];
#pragma unroll
    for (int m = 0; m < NE1; ++m) dw[m] = dqt[m] = 0.f;
    for (int j0 = 0; j0 < V; j0 += VTL) {
      __syncthreads();
      for (int e = tid; e < K * VTL; e += NT) {
        const int c = e / VTL, jj = e % VTL;
        tS0[c][jj] = S0[(int64_t)c * V + j0 + jj];
      }
      for (int e = tid; e < C * VTL; e += NT) {
        const int r = e / VTL, jj = e % VTL;
        tdD[r][jj] = dDl[(int64_t)r * V + j0 + jj];
        const float x = load_f32(dO + th(r < L ? r : 0) * V + j0 + jj);
        tdO[r][jj] = r < L ? x : 0.f;
      }
      __syncthreads();
      for (int jj = 0; jj < VTL; jj += 4) {
        const float s0[4] = {tS0[c1][jj], tS0[c1][jj + 1], tS0[c1][jj + 2], tS0[c1][jj + 3]};
#pragma unroll
        for (int m = 0; m < NE1; ++m) {
          const int r = rb1 + RSTEP1 * m;
          const float4 x = *(const float4*)&tdD[r][jj];
          const float4 y = *(const float4*)&tdO[r][jj];
          dw[m] += x.x * s0[0] + x.y * s0[1] + x.z * s0[2] + x.w * s0[3];
          dqt[m] += y.x * s0[0] + y.y * s0[1] + y.z * s0[2] + y.w * s0[3];
        }
      }
    }
    __syncthreads();  // the tiles are dead; dW goes where they were
#pragma unroll
    for (int m = 0; m < NE1; ++m) {
      const int r = rb1 + RSTEP1 * m;
      sDW[r][c1] = -dw[m];
      dqs[m] = scale * dqt[m];
    }
  }
  // second sweep: its tiles live in the part of the region above dW
  float* sReg2 = sReg + C * DWS;
  float (*tdSL2)[VTL + 1] = (float(*)[VTL + 1])sReg2;
  float (*tD2)[TS] = (float(*)[TS])(sReg2 + K * (VTL + 1));
  float (*tdO2)[TS] = (float(*)[TS])(sReg2 + K * (VTL + 1) + C * TS);
  float (*tdD2)[TS] = (float(*)[TS])(sReg2 + K * (VTL + 1) + 2 * C * TS);
  float (*tv2)[TS] = (float(*)[TS])(sReg2 + K * (VTL + 1) + 3 * C * TS);
  float (*tS02)[VTL + 1] = (float(*)[VTL + 1])(sReg2 + K * (VTL + 1) + 4 * C * TS);
  float pp[NE2], yv[NE2];
#pragma unroll
  for (int m = 0; m < NE1; ++m) dkb[m] = 0.f;
#pragma unroll
  for (int m = 0; m < NE2; ++m) pp[m] = yv[m] = 0.f;
  for (int j0 = 0; j0 < V; j0 += VTL) {
    __syncthreads();
    for (int e = tid; e < K * VTL; e += NT) {
      const int c = e / VTL, jj = e % VTL;
      tdSL2[c][jj] = dSL[(int64_t)c * V + j0 + jj];
      tS02[c][jj] = S0[(int64_t)c * V + j0 + jj];
    }
    for (int e = tid; e < C * VTL; e += NT) {
      const int r = e / VTL, jj = e % VTL;
      const bool in = r < L;
      tdD2[r][jj] = dDl[(int64_t)r * V + j0 + jj];
      tD2[r][jj] = Dl[(int64_t)r * V + j0 + jj];
      const int64_t rv = th(in ? r : 0) * V + j0 + jj;
      const float xo = load_f32(dO + rv), xv = load_f32(v + rv);
      tdO2[r][jj] = in ? xo : 0.f;
      tv2[r][jj] = in ? xv : 0.f;
    }
    __syncthreads();
    for (int jj = 0; jj < VTL; jj += 4) {
      const float l0[4] = {tdSL2[c1][jj], tdSL2[c1][jj + 1], tdSL2[c1][jj + 2], tdSL2[c1][jj + 3]};
      sd += tS02[c1][jj] * l0[0] + tS02[c1][jj + 1] * l0[1] + tS02[c1][jj + 2] * l0[2] +
            tS02[c1][jj + 3] * l0[3];
#pragma unroll
      for (int m = 0; m < NE1; ++m) {
        const int r = rb1 + RSTEP1 * m;
        const float4 z = *(const float4*)&tD2[r][jj];
        dkb[m] += z.x * l0[0] + z.y * l0[1] + z.z * l0[2] + z.w * l0[3];
      }
      const float4 di = *(const float4*)&tD2[i2][jj];
      const float4 vi = *(const float4*)&tv2[i2][jj];
#pragma unroll
      for (int m = 0; m < NE2; ++m) {
        const int r = rb2 + RSTEP2 * m;
        if (r < C) {
          const float4 o = *(const float4*)&tdO2[r][jj];
          const float4 x = *(const float4*)&tdD2[r][jj];
          pp[m] += o.x * di.x + o.y * di.y + o.z * di.z + o.w * di.w;
          yv[m] += x.x * vi.x + x.y * vi.y + x.z * vi.z + x.w * vi.w;
        }
      }
    }
    // dV = Diag(beta) Tm^T dDelta for this tile's columns
#pragma unroll
    for (int m = 0; m < NEV; ++m) {
      const int e = tid + NT * m, r = e / VTL, jj = e % VTL;
      if (e < C * VTL && r < L) {
        float acc = 0.f;
        for (int aa = r; aa < L; ++aa) acc = fmaf(sT[aa][r], tdD2[aa][jj], acc);
        store_as(dv + th(r) * V + j0 + jj, sB[r] * acc);
      }
    }
  }
  __syncthreads();  // the tiles are dead
#pragma unroll
  for (int m = 0; m < NE1; ++m) {
    const int r = rb1 + RSTEP1 * m;
    const float x = khat(r < L ? r : 0, c1);
    sKtT[c1][r] = r < L ? x * __expf(sGam[r][c1]) : 0.f;
  }
#pragma unroll
  for (int m = 0; m < NE2; ++m) {
    const int r = rb2 + RSTEP2 * m;
    if (r < C) {
      const bool low = i2 <= r && r < L;
      sP[r][i2] = low ? scale * pp[m] : 0.f;
      sY[r][i2] = low ? yv[m] : 0.f;
    }
  }
  if (tid < K) sSd[tid] = sd;
  __syncthreads();

  }

  // ---- phase C: Y += dW K~^T (i <= r) ----
  if constexpr (C == 64) {
    // the ten lower 16 x 16 tiles on fp32 matrix cores, each wave owning whole tiles
    const int lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
    for (int t = w; t < 10; t += NT / 64) {
      const int R = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0, I = t - R * (R + 1) / 2;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int c = 0; c < K; c += 4)
        acc = mfma_f32(sDW[16 * R + ln][c + lg], sKtT[c + lg][16 * I + ln], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * R + 4 * lg + e, i = 16 * I + ln;
        if (r < L && i <= r) sY[r][i] += acc[e];
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < NE2; ++m) {
      const int r = rb2 + RSTEP2 * m;
      if (r < L && i2 <= r) {
        float acc = 0.f;
        for (int c = 0; c < K; c += 4) {
          const float4 dwv = *(const float4*)&sDW[r][c];
          acc += dwv.x * sKtT[c][i2] + dwv.y * sKtT[c + 1][i2] + dwv.z * sKtT[c + 2][i2] +
                 dwv.w * sKtT[c + 3][i2];
        }
        sY[r][i2] += acc;
      }
    }
  }
  __syncthreads();

  // ---- phase D: dbeta (first part), Z = Tm^T dT (bb < r), and through dW the
  //      K~ term of k^ and gamma (kept in the element owner's registers) ----
  // (C = 64: dbeta's first part and Z come from one product on the matrix
  // cores below, once K~ and dW are dead)
  float zv[NE2];
  if constexpr (C != 64) {
    for (int r = tid; r < L; r += NT) {
      float acc = 0.f;
      for (int aa = r; aa < L; ++aa) acc = fmaf(sT[aa][r], sY[aa][r], acc);
      sDb[r] = acc;
    }
#pragma unroll
    for (int m = 0; m < NE2; ++m) {
      const int r = rb2 + RSTEP2 * m;
      float acc = 0.f;
      if (r < L && i2 < r)
        for (int aa = r; aa < L; ++aa) acc = fmaf(sT[aa][r], sY[aa][i2], acc);
      zv[m] = sB[i2] * acc;
    }
  }
  float ekt[NE1];  // e^gamma beta (Tm^T dW): the K~ term of dk^ (and, times k^, of dgamma)
  if constexpr (C == 64) {
    // Tm^T dW on fp32 matrix cores (Tm[aa][r] is zero for aa < r, so a row tile's
    // k-steps start at its own block), scaled and passed to the element owners
    // through the K~ region, which phase C has finished reading
    float (*sE)[K] = (float(*)[K])sR4;
    const int lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
    for (int t = w; t < (C / 16) * (K / 16); t += NT / 64) {
      const int rt = t / (K / 16), ct = t % (K / 16);
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int aa = 16 * rt; aa < C; aa += 4)
        acc = mfma_f32(sT[aa + lg][16 * rt + ln], sDW[aa + lg][16 * ct + ln], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * lg + e, c = 16 * ct + ln;
        sE[r][c] = r < L ? __expf(sGam[r][c]) * sB[r] * acc[e] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NE1; ++m) ekt[m] = sE[rb1 + RSTEP1 * m][c1];
  } else {
#pragma unroll
    for (int m = 0; m < NE1; ++m) {
      const int r = rb1 + RSTEP1 * m;
      float dxk = 0.f;
      if (r < L)
        for (int aa = r; aa < L; ++aa) dxk = fmaf(sT[aa][r], sDW[aa][c1], dxk);
      ekt[m] = r < L ? __expf(sGam[r][c1]) * sB[r] * dxk : 0.f;
    }
  }
  __syncthreads();  // K~ and dW are dead: Z and q^ take their places
  // q^ of the chunk (rebuilt from q and its norm scale) and below k^: loaded
  // ahead of the products of phases D and E and stored to LDS after them
  // where the registers allow it (not in the 1024-thread kernel, whose
  // spills grow with them)
  constexpr bool early_hat = NT < 1024;
  constexpr int NHAT = (C * K / 4 + NT - 1) / NT;
  float4 hat_pre[early_hat ? NHAT : 1];
  auto hat_load = [&](const Tin* x, const float* rs) {
#pragma unroll
    for (int u = 0; u < NHAT; ++u) {
      const int e = tid + u * NT, r = e / (K / 4), c4 = e % (K / 4);
      hat_pre[u] = hat4(x, rs, e < C * K / 4 && r < L ? r : 0, c4);
    }
  };
  auto hat_store = [&](float (*dst)[K]) {
#pragma unroll
    for (int u = 0; u < NHAT; ++u) {
      const int e = tid + u * NT, r = e / (K / 4), c4 = e % (K / 4);
      if (e < C * K / 4) ((float4*)&dst[r][0])[c4] = r < L ? hat_pre[u] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto hat_direct = [&](const Tin* x, const float* rs, float (*dst)[K]) {
#pragma unroll
    for (int e = tid; e < C * K / 4; e += NT) {
      const int r = e / (K / 4), c4 = e % (K / 4);
      const float4 v = hat4(x, rs, r < L ? r : 0, c4);
      ((float4*)&dst[r][0])[c4] = r < L ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  if constexpr (early_hat) hat_load((const Tin*)a.q, a.rq);
  if constexpr (C == 64) {
    // (Tm^T Y) on fp32 matrix cores, one 16 x 16 tile per wave and step:
    // Tm[aa][r] is zero for aa < r, so a row tile's k-steps start at its own
    // block; rows aa past the chunk end are masked.  Z = (Tm^T Y)[r][i] beta_i
    // for i < r (zero elsewhere), dbeta's first part is the diagonal.
    const int lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
    for (int t = w; t < 16; t += NT / 64) {
      const int rt = t / 4, it = t % 4;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (it <= rt)
        for (int aa = 16 * rt; aa < C; aa += 4) {
          const int ak = aa + lg;
          acc = mfma_f32(sT[ak][16 * rt + ln], ak < L ? sY[ak][16 * it + ln] : 0.f, acc);
        }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * lg + e, i = 16 * it + ln;
        sZ[r][i] = (i < r && r < L) ? sB[i] * acc[e] : 0.f;
        if (i == r && r < L) sDb[r] = acc[e];
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < NE2; ++m) {
      const int r = rb2 + RSTEP2 * m;
      if (r < C) sZ[r][i2] = zv[m];
    }
  }
  if constexpr (early_hat) hat_store(sQn);
  else hat_direct((const Tin*)a.q, a.rq, sQn);
  __syncthreads();

  // ---- phase E: dN = -Z Tm^T (i < r), dAkk = beta_r dN -> sY; dbeta (second part) ----
  // this thread's Akk elements for dbeta, issued ahead of the products below
  // (one uniform branch around each loop: a select between two loads per
  // element would branch and wait on every load)
  float akk[NE2];
  if constexpr (early_hat) hat_load((const Tin*)a.k, a.rk);
  if (a.ws_bf16) {
    const bf16* akb = (const bf16*)a.Akk_out + chb * C * C;
#pragma unroll
    for (int m = 0; m < NE2; ++m) {
      const int r = rb2 + RSTEP2 * m;
      akk[m] = bf16_to_f32(akb[(int64_t)(r < C ? r : 0) * C + i2]);
    }
  } else {
#pragma unroll
    for (int m = 0; m < NE2; ++m) {
      const int r = rb2 + RSTEP2 * m;
      akk[m] = Akk[(int64_t)(r < C ? r : 0) * C + i2];
    }
  }
  if constexpr (C == 64) {
    // (Z Tm^T)[r][i] on fp32 matrix cores (Tm[i][bb] is zero for bb > i, so a
    // column tile's k-steps end with its own block), into Y's place, which
    // nothing reads any more; each element's owner takes it from there
    const int lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
    for (int t = w; t < 16; t += NT / 64) {
      const int rt = t / 4, it = t % 4;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (it <= rt)
        for (int bb = 0; bb < 16 * (it + 1); bb += 4)
          acc = mfma_f32(sZ[16 * rt + ln][bb + lg], sT[16 * it + ln][bb + lg], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * lg + e, i = 16 * it + ln;
        sY[r][i] = (i < r && r < L) ? -acc[e] : 0.f;
      }
    }
    __syncthreads();
  }
  float dak[NE2];
#pragma unroll
  for (int m = 0; m < NE2; ++m) {
    const int r = rb2 + RSTEP2 * m;
    float dn = 0.f;
    if constexpr (C == 64) {
      if (r < C) dn = sY[r][i2];
    } else if (r < L && i2 < r) {
      for (int bb = 0; bb <= i2; ++bb) dn = fmaf(-sZ[r][bb], sT[i2][bb], dn);
    }
    float part = (r < L && i2 < r) ? dn * akk[m] : 0.f;
    if constexpr (C == 64) {
      part = wave_sum_dpp(part);  // a row's 64 columns are one wave
    } else {
#pragma unroll
      for (int off = C / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
    }
    if (r < C && i2 == 0) sDb[r] += part;
    dak[m] = (r < C) ? sB[r < C ? r : 0] * dn : 0.f;
  }
  __syncthreads();  // Z is dead: k^ takes its place; dAkk replaces Y
#pragma unroll
  for (int m = 0; m < NE2; ++m) {
    const int r = rb2 + RSTEP2 * m;
    if (r < C) sY[r][i2] = dak[m];
  }
  if constexpr (early_hat) hat_store(sKn);
  else hat_direct((const Tin*)a.k, a.rk, sKn);
  // C = 64: does any 16-row block decay by more than kBlockSafe in a channel?
  // Then the pairs inside the blocks keep their exact per-pair factor (below).
  bool exact_blocks = true;
  if constexpr (C == 64) {
    bool over = false;
    if (tid < 4 * K) {
      const int R = tid / K, c = tid % K;
      over = (R > 0 ? sGam[16 * R - 1][c] : 0.f) - sGam[16 * R + 15][c] > kBlockSafe;
    }
    exact_blocks = __syncthreads_or(over) != 0;
  } else {
    __syncthreads();
  }

  // ---- phase F: per element (r, c), the gradients of q^, k^ and gamma ----
  // The pairwise sums over the chunk:
  //   r1 = sum_{i<=r} P[r][i] k^_ic e^{g_rc - g_ic},  r2 likewise with Y,
  //   c12 = sum_{rr>=r} (P[rr][r] q^_rr,c + Y[rr][r] k^_rr,c) e^{g_rr,c - g_rc}.
  // C = 64: the blocks before and after run on the fp32 matrix cores with every
  // factor referenced to a block boundary (G_R = g at row 16R-1 for the blocks
  // before row block R, G'_R = g at its last row for the blocks after), so
  // that all are <= 1:
  //   r1 += e^{g_r - G_R} (P[R rows, <16R] (k^ e^{G_R - g}))
  //   c12 += e^{G'_R - g_r} (P[>R, R cols]^T (q^ e^{g - G'_R}) + Y^T (k^ e^{g - G'_R})).
  // The pairs inside a block join those products (k-steps 16R..16R+15, P and
  // Y being zero above the diagonal) while no block decays by more than
  // kBlockSafe: their inner factors e^{G_R - g_i} and e^{g_rr - G'_R} then stay
  // below e^kBlockSafe.  Otherwise (exact_blocks) each in-block pair takes its
  // exact factor e^{g_r - g_i} in the per-element loops.
  // Their tiles reach the element owners through the LDS that Tm used.
  // The blocks' terms are summed first (per owner: x1 = r1, x2 = r2 + c12,
  // x3 = q^ r1 + k^ (r2 - c12) of the off-diagonal blocks), then the in-block
  // pairs, and each element's outputs
  //   dq^ = e^g dq~ + r1,  dk^ = ekt + e^{g_L - g} dkb + r2 + c12,
  //   dg = k^ ekt + q^ e^g dq~ - tkb + q^ r1 + k^ (r2 - c12).
  float ox1[NE1], ox2[NE1], ox3[NE1];
#pragma unroll
  for (int m = 0; m < NE1; ++m) ox1[m] = ox2[m] = ox3[m] = 0.f;
  if constexpr (C == 64) {
    static_assert(RSTEP1 == 8 && NE1 == 8, "rows rb1 + 8m: two rows of each 16-row block per owner");
    constexpr int NW = NT / 64, CG = K < 64 ? K : 64, NGRP = K / CG, CTG = CG / 16;
    float (*stg)[16][CG + 1] = (float(*)[16][CG + 1])&sT[0][0];  // Tm is dead
    static_assert(3 * 16 * (CG + 1) <= C * (C + 1), "the staged tiles fit where Tm was");
    const int lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
#pragma unroll 1
    for (int R = 0; R < 4; ++R) {
#pragma unroll 1
      for (int grp = 0; grp < NGRP; ++grp) {
        // jobs 0..CTG-1: r1 tiles, then r2, then c12, of this row block and column group
        for (int job = w; job < 3 * CTG; job += NW) {
          const int kind = job / CTG, ctl = job % CTG, col = 16 * (grp * CTG + ctl) + ln;
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
          float rowf[4] = {0.f, 0.f, 0.f, 0.f};
          if (kind < 2) {
            const int kend = exact_blocks ? 16 * R : 16 * R + 16;
            if (kend > 0 && 16 * R < L) {  // rows before 16R are all inside the chunk
              const float gR = R > 0 ? sGam[16 * R - 1][col] : 0.f;
              for (int kk = 0; kk < kend; kk += 4) {
                const int i = kk + lg;
                const float bk = sKn[i][col] * __expf(gR - sGam[i][col]);
                acc = mfma_f32(kind == 0 ? sP[16 * R + ln][i] : sY[16 * R + ln][i], bk, acc);
              }
#pragma unroll
              for (int e = 0; e < 4; ++e) rowf[e] = __expf(sGam[16 * R + 4 * lg + e][col] - gR);
            }
          } else if (const int kbeg = exact_blocks ? 16 * (R + 1) : 16 * R; kbeg < C && kbeg < L) {
            // g is constant past the chunk end, and q^, k^ are zero there
            const float gE = sGam[16 * R + 15][col];
            for (int kk = kbeg; kk < C; kk += 4) {
              const int rr = kk + lg;
              const float f = __expf(sGam[rr][col] - gE);
              acc = mfma_f32(sP[rr][16 * R + ln], sQn[rr][col] * f, acc);
              acc = mfma_f32(sY[rr][16 * R + ln], sKn[rr][col] * f, acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) rowf[e] = __expf(gE - sGam[16 * R + 4 * lg + e][col]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) stg[kind][4 * lg + e][16 * ctl + ln] = rowf[e] * acc[e];
        }
        __syncthreads();
        // the owners of this block's rows (m = 2R, 2R+1) in this column group
        // (both conditions wave-uniform; m stays a compile-time index)
        if (c1 / CG == grp) {
#pragma unroll
          for (int m = 0; m < NE1; ++m) {
            if ((m >> 1) != R) continue;
            const int rl = rb1 + 8 * (m & 1), cl = c1 - grp * CG, r = 16 * R + rl;
            const float x1 = stg[0][rl][cl], x2 = stg[1][rl][cl], x3 = stg[2][rl][cl];
            ox1[m] = x1;
            ox2[m] = x2 + x3;
            ox3[m] = sQn[r][c1] * x1 + sKn[r][c1] * (x2 - x3);
          }
        }
        __syncthreads();
      }
    }
  }
  // One key head per value head: the L2 norm's Jacobian is applied here,
  // dq = rq (dq^ - q^ (q^ . dq^)) and likewise dk, the dot over the row's K
  // channels as a wave sum per row and the K/64 waves of the row added through
  // LDS (the dead Tm's place).  Grouped value heads leave dq^ and dk^ in the
  // workspace for k_bwd_qk, which sums the group first.
  const bool fuse_qk = a.H == a.HK;
  constexpr int NWV = NT / 64, WPR = (K + 63) / 64;  // waves; waves per row
  float* sPart = &sT[0][0];                          // [NWV][NE1][2]
  static_assert(NWV * NE1 * 2 <= C * (C + 1), "the partial dots fit where Tm was");
  float dqv[NE1], dkv[NE1];
  float dgm[NE1], tkm[NE1];
#pragma unroll
  for (int m = 0; m < NE1; ++m) {
    // rb1 = tid / K is the same for every lane of a wave, so the row and the
    // loop bounds below are wave-uniform (scalar loop control)
    const int r = __builtin_amdgcn_readfirstlane(rb1 + RSTEP1 * m), c = c1;
    dgm[m] = tkm[m] = 0.f;
    if (r >= L) continue;
    // (the in-block pairs ran on the matrix cores unless exact_blocks)
    const int i0 = C == 64 ? (exact_blocks ? (r & ~15) : r + 1) : 0;   // first column summed here
    const int rr1 = C == 64 ? (exact_blocks ? min((r | 15) + 1, L) : r) : L;  // past the last row summed here
    const float q = sQn[r][c], kk = sKn[r][c];
    const float gm = sGam[r][c], egm = __expf(gm), ekb = __expf(sGam[L - 1][c] - gm);
    float r1 = 0.f, r2 = 0.f;
#pragma unroll 4
    for (int i = i0; i <= r; ++i) {
      const float ke = sKn[i][c] * __expf(gm - sGam[i][c]);
      r1 = fmaf(sP[r][i], ke, r1);
      r2 = fmaf(sY[r][i], ke, r2);
    }
    float c12 = 0.f;
#pragma unroll 4
    for (int rr = r; rr < rr1; ++rr) {
      const float e = __expf(sGam[rr][c] - gm);
      c12 = fmaf(sP[rr][r] * sQn[rr][c] + sY[rr][r] * sKn[rr][c], e, c12);
    }
    const float tkb = kk * ekb * dkb[m];
    const float dqh = egm * dqs[m] + r1 + ox1[m];
    const float dkh = ekt[m] + ekb * dkb[m] + r2 + c12 + ox2[m];
    if (fuse_qk) {
      dqv[m] = dqh;
      dkv[m] = dkh;
      const float pq = wave_sum_dpp(q * dqh), pk = wave_sum_dpp(kk * dkh);
      if ((tid & 63) == 0) {
        sPart[((tid >> 6) * NE1 + m) * 2] = pq;
        sPart[((tid >> 6) * NE1 + m) * 2 + 1] = pk;
      }
    } else {
      b.dqh[th(r) * K + c] = dqh;
      b.dkh[th(r) * K + c] = dkh;
    }
    dgm[m] = kk * ekt[m] + q * egm * dqs[m] - tkb + q * r1 + kk * r2 - kk * c12 + ox3[m];
    tkm[m] = tkb;
  }
  if (fuse_qk) {
    // the rows' norm scales (a row is one wave's: scalar loads), all issued
    // before the barrier
    float rqm[NE1], rkm[NE1];
#pragma unroll
    for (int m = 0; m < NE1; ++m) {
      const int r = __builtin_amdgcn_readfirstlane(rb1 + RSTEP1 * m);
      rqm[m] = a.rq[th(r < L ? r : 0)];
      rkm[m] = a.rk[th(r < L ? r : 0)];
    }
    __syncthreads();  // the partial dots are in LDS
    Tin* dqo = (Tin*)b.dq;
    Tin* dko = (Tin*)b.dk;
#pragma unroll
    for (int m = 0; m < NE1; ++m) {
      const int r = __builtin_amdgcn_readfirstlane(rb1 + RSTEP1 * m);
      if (r >= L) continue;
      float dq_dot = 0.f, dk_dot = 0.f;
#pragma unroll
      for (int u = 0; u < WPR; ++u) {
        const int wv = WPR * rb1 + u;
        dq_dot += sPart[(wv * NE1 + m) * 2];
        dk_dot += sPart[(wv * NE1 + m) * 2 + 1];
      }
      const int64_t o = th(r) * K + c1;  // one key head per value head: thk(r) = th(r)
      store_as(dqo + o, rqm[m] * (dqv[m] - sQn[r][c1] * dq_dot));
      store_as(dko + o, rkm[m] * (dkv[m] - sKn[r][c1] * dk_dot));
    }
  }
  __syncthreads();  // q^, k^ are dead
#pragma unroll
  for (int m = 0; m < NE1; ++m) {
    const int r = rb1 + RSTEP1 * m;
    sDg[r][c1] = dgm[m];
    sTk[r][c1] = tkm[m];
  }
  __syncthreads();

  // gamma -> g (a reverse cumulative sum over rows, segmented: thread (c, s)
  // takes rows [s RSEG, (s+1) RSEG); gamma_L also collects the Kbar terms and
  // the state decay), then through the gate
  constexpr int NSEG = NT / K, RSEG = C / NSEG > 0 ? C / NSEG : 1;
  __shared__ float sSeg[NSEG][K], sSeg2[NSEG][K];
  const int cS = tid % K, sS_ = tid / K;
  Tin* dgate = (Tin*)b.dgate;
  const Tin* gate = (const Tin*)a.gate;
  const bool segok = sS_ * RSEG < C;
  // the raw gate of this thread's segment rows, issued before the barriers
  // below (the loop that uses them walks its rows one after another)
  float gin[RSEG];
#pragma unroll
  for (int u = 0; u < RSEG; ++u) {
    const int r = sS_ * RSEG + u;
    gin[u] = load_f32(gate + th(segok && r < L ? r : 0) * K + cS);
  }
  if (segok) {
    float sdg = 0.f, stk = 0.f;
#pragma unroll
    for (int u = 0; u < RSEG; ++u) {
      const int r = sS_ * RSEG + u;
      sdg += sDg[r][cS];
      stk += sTk[r][cS];
    }
    sSeg[sS_][cS] = sdg;
    sSeg2[sS_][cS] = stk;
  }
  __syncthreads();
  float ddt = 0.f, da = 0.f;
  if (segok) {
    float run = __expf(sGam[L - 1][cS]) * sSd[cS];
    for (int s2 = 0; s2 < NSEG; ++s2) {
      if (s2 * RSEG >= C) break;
      run += sSeg2[s2][cS];
      if (s2 > sS_) run += sSeg[s2][cS];
    }
    const float Aexp = expf(a.a_log[h]), db = a.dt_bias[(int64_t)h * K + cS];
#pragma unroll
    for (int u = RSEG - 1; u >= 0; --u) {
      const int r = sS_ * RSEG + u;
      if (r >= L) continue;
      run += sDg[r][cS];
      float gx, ga;
      gate_grad(gin[u] + db, Aexp, a.gate_form, a.lb, &gx, &ga);
      const float dg = run * gx;
      store_as(dgate + th(r) * K + cS, dg);
      ddt += dg;
      da = fmaf(run, ga, da);
    }
  }
  __syncthreads();  // segment sums are read; reuse them for the partials
  if (segok) {
    sSeg[sS_][cS] = ddt;
    sSeg2[sS_][cS] = da;
  }
  __syncthreads();
  for (int c = tid; c < K; c += NT) {
    float sddt = 0.f, sda = 0.f;
    for (int s2 = 0; s2 < NSEG && s2 * RSEG < C; ++s2) {
      sddt += sSeg[s2][c];
      sda += sSeg2[s2][c];
    }
    b.ddt_part[chb * K + c] = sddt;
    sRed[c] = sda;
  }
  // beta logit
  Tin* dbeta = (Tin*)b.dbeta;
  for (int r = tid; r < L; r += NT) store_as(dbeta + th(r), sDb[r] * sB[r] * (1.f - sB[r]));
  __syncthreads();
  if (tid < 64) {
    // wave 0 sums the K channel partials (a fixed order: deterministic)
    float acc = 0.f;
    for (int c = tid; c < K; c += 64) acc += sRed[c];
    acc = wave_sum_dpp(acc);
    if (tid == 0) b.da_part[chb] = acc;
  }
}

// dq, dk: sum over the value heads of a group, then the L2 norm's Jacobian.
// One wave per TPW (token, key head) pairs; lane l holds channels
// CPL l .. CPL l + CPL - 1 (one 8-byte or 4-byte piece per row), and every load
// of the wave's pairs is issued before the first reduction.
template <typename Tin, int K>
__global__ __launch_bounds__(kThreads) void k_bwd_qk(BwdArgs b) {
  constexpr int CPL = K / 64, TPW = 4;
  static_assert(CPL == 1 || CPL == 2, "head dims 64 and 128");
  const FwdArgs& a = b.f;
  const int H = a.H, HK = a.HK, G = H / HK;
  const int lane = threadIdx.x & 63, c0 = CPL * lane;
  const int64_t n_tk = (int64_t)a.B * a.T * HK;
  const int64_t tk0 = ((int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * TPW;
  if (tk0 >= n_tk) return;
  float dq[TPW][CPL], dk[TPW][CPL], vq[TPW][CPL], vk[TPW][CPL];
  auto ld = [&](const float* p, float* out) __attribute__((always_inline)) {
    if constexpr (CPL == 2) {
      const float2 x = *(const float2*)p;
      out[0] = x.x;
      out[1] = x.y;
    } else {
      out[0] = *p;
    }
  };
  // q and k need only their element alignment: one load per element
  auto ldt = [&](const Tin* p, float* out) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < CPL; ++e) out[e] = load_f32(p + e);
  };
  // past the last pair, the last one is read again and nothing is stored
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int64_t tk = tk0 + t < n_tk ? tk0 + t : n_tk - 1;
    const int64_t tok = tk / HK;
    const int hk = (int)(tk % HK);
    const int64_t row0 = (tok * H + (int64_t)hk * G) * K + c0;
    ld(b.dqh + row0, dq[t]);
    ld(b.dkh + row0, dk[t]);
    for (int gi = 1; gi < G; ++gi) {
      float xq[CPL], xk[CPL];
      ld(b.dqh + row0 + (int64_t)gi * K, xq);
      ld(b.dkh + row0 + (int64_t)gi * K, xk);
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        dq[t][e] += xq[e];
        dk[t][e] += xk[e];
      }
    }
    ldt((const Tin*)a.q + tk * K + c0, vq[t]);
    ldt((const Tin*)a.k + tk * K + c0, vk[t]);
  }
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int64_t tk = tk0 + t;
    if (tk >= n_tk) break;
    float ssq = 0.f, dotq = 0.f, ssk = 0.f, dotk = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      ssq = fmaf(vq[t][e], vq[t][e], ssq);
      dotq = fmaf(vq[t][e], dq[t][e], dotq);
      ssk = fmaf(vk[t][e], vk[t][e], ssk);
      dotk = fmaf(vk[t][e], dk[t][e], dotk);
    }
    ssq = wave_sum_dpp(ssq);
    dotq = wave_sum_dpp(dotq);
    ssk = wave_sum_dpp(ssk);
    dotk = wave_sum_dpp(dotk);
    const float rq = 1.f / sqrtf(ssq + 1e-6f), rk = 1.f / sqrtf(ssk + 1e-6f);
    const float r3q = rq * rq * rq, r3k = rk * rk * rk;
    Tin* oq = (Tin*)b.dq + tk * K + c0;
    Tin* ok = (Tin*)b.dk + tk * K + c0;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      store_as(oq + e, dq[t][e] * rq - vq[t][e] * dotq * r3q);
      store_as(ok + e, dk[t][e] * rk - vk[t][e] * dotk * r3k);
    }
  }
}

// da_log, ddt_bias: sums over chunks in chunk order (the additions stay in that
// order; the loads are issued 16 at a time).
__global__ __launch_bounds__(kThreads) void k_bwd_params(BwdArgs b) {
  const FwdArgs& a = b.f;
  const int H = a.H, K = a.K;
  const int nt = *a.nt_dev;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t < (int64_t)H * K) {
    const int h = (int)(t / K), c = (int)(t % K);
    float s = 0.f;
    int j = 0;
    for (; j + 16 <= nt; j += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = b.ddt_part[((int64_t)(j + u) * H + h) * K + c];
#pragma unroll
      for (int u = 0; u < 16; ++u) s += v[u];
    }
    for (; j < nt; ++j) s += b.ddt_part[((int64_t)j * H + h) * K + c];
    b.ddt_bias[t] = s;
  }
  if (t < H) {
    float s = 0.f;
    int j = 0;
    for (; j + 16 <= nt; j += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = b.da_part[(int64_t)(j + u) * H + t];
#pragma unroll
      for (int u = 0; u < 16; ++u) s += v[u];
    }
    for (; j < nt; ++j) s += b.da_part[(int64_t)j * H + t];
    b.da_log[t] = s;
  }
}

template <typename Tin, int C>
hipError_t run(const BwdArgs& b, hipStream_t s) {
  const FwdArgs& a = b.f;
  bmark(b, kBwdRecompute, 0, s);
  // bf16 inputs: the matrix-core chunk kernel when its fix-up list is given
  const bool mfma = std::is_same<Tin, bf16>::value && a.exact_list != nullptr;
  hipError_t e = mfma ? launch_mfma_recompute(a, s) : launch_valu_prep(a, s);
  if (e != hipSuccess) return e;
  bmark(b, kBwdRecompute, 1, s);
  const int64_t wgs = (int64_t)a.N * a.H * (a.V / 64);
  bmark(b, kBwdFState, 0, s);
  if (wgs > 0 && a.NT > 0) {
    constexpr int NTS = 64 * state_waves(C);
    if constexpr (C == 64) {
      const dim3 g((unsigned)wgs), t(1024);
      if (a.ws_bf16) {
        if (a.K == 64) hipLaunchKernelGGL((k_bwd_fstate_bf<64>), g, t, 0, s, b);
        else hipLaunchKernelGGL((k_bwd_fstate_bf<128>), g, t, 0, s, b);
      } else {
        if (a.K == 64) hipLaunchKernelGGL((k_bwd_fstate_mfma<64>), g, t, 0, s, b);
        else hipLaunchKernelGGL((k_bwd_fstate_mfma<128>), g, t, 0, s, b);
      }
    } else {
      if (a.K == 64) hipLaunchKernelGGL((k_bwd_fstate<C, 64>), dim3((unsigned)wgs), dim3(NTS), 0, s, b);
      else hipLaunchKernelGGL((k_bwd_fstate<C, 128>), dim3((unsigned)wgs), dim3(NTS), 0, s, b);
    }
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  bmark(b, kBwdFState, 1, s);
  bmark(b, kBwdDState, 0, s);
  if (wgs > 0) {
    constexpr int NTS = 64 * state_waves(C);
    if constexpr (C == 64) {
      const dim3 g((unsigned)wgs), t(1024);
      if (a.ws_bf16) {
        if (a.K == 64) hipLaunchKernelGGL((k_bwd_dstate_bf<64>), g, t, 0, s, b);
        else hipLaunchKernelGGL((k_bwd_dstate_bf<128>), g, t, 0, s, b);
      } else {
        if (a.K == 64) hipLaunchKernelGGL((k_bwd_dstate_mfma<Tin, 64>), g, t, 0, s, b);
        else hipLaunchKernelGGL((k_bwd_dstate_mfma<Tin, 128>), g, t, 0, s, b);
      }
    } else {
      if (a.K == 64) hipLaunchKernelGGL((k_bwd_dstate<Tin, C, 64>), dim3((unsigned)wgs), dim3(NTS), 0, s, b);
      else hipLaunchKernelGGL((k_bwd_dstate<Tin, C, 128>), dim3((unsigned)wgs), dim3(NTS), 0, s, b);
    }
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  bmark(b, kBwdDState, 1, s);
  bmark(b, kBwdChunk, 0, s);
  if (a.NT > 0) {
    const dim3 grid((unsigned)((int64_t)a.NT * a.H));
    constexpr int T64 = chunk_threads(C, 64), T128 = chunk_threads(C, 128);
    if (a.K == 64) hipLaunchKernelGGL((k_bwd_chunk<Tin, C, 64, T64>), grid, dim3(T64), 0, s, b);
    else hipLaunchKernelGGL((k_bwd_chunk<Tin, C, 128, T128>), grid, dim3(T128), 0, s, b);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  bmark(b, kBwdChunk, 1, s);
  const int64_t tk = (int64_t)a.B * a.T * a.HK;
  bmark(b, kBwdQK, 0, s);
  // (one key head per value head: done inside k_bwd_chunk)
  if (tk > 0 && a.H != a.HK) {
    const dim3 grid((unsigned)((tk + 15) / 16));  // 4 waves of 4 pairs
    if (a.K == 64) hipLaunchKernelGGL((k_bwd_qk<Tin, 64>), grid, dim3(kThreads), 0, s, b);
    else hipLaunchKernelGGL((k_bwd_qk<Tin, 128>), grid, dim3(kThreads), 0, s, b);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  bmark(b, kBwdQK, 1, s);
  const int64_t hk = (int64_t)a.H * a.K;
  bmark(b, kBwdParams, 0, s);
  hipLaunchKernelGGL(k_bwd_params, dim3((unsigned)((hk + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, b);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  bmark(b, kBwdParams, 1, s);
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
  bmark(b, kBwdTable, 0, s);
  hipError_t e = launch_chunk_table(b.f, s);
  if (e != hipSuccess) return e;
  bmark(b, kBwdTable, 1, s);
  return b.f.dtype == 0 ? run_c<float>(b, s) : run_c<bf16>(b, s);
}

}  // namespace kda
