// MFMA path of the KDA chunked forward (bf16 inputs, chunk 64, K,V in {64,128}).
//
// Two kernels:
//   k_chunk_mfma  one workgroup (4 waves) per chunk-head, all chunks in
//                 parallel.  Fuses the prologue (q/k L2 norm, in-kernel gate,
//                 beta sigmoid, chunk-local cumulative log-decay) with the
//                 chunk-local WY/UT factors, and writes one "chunk record" per
//                 chunk-head whose operands are already laid out as MFMA
//                 fragments for the state pass.
//   k_state_mfma  one workgroup per (sequence, head, column tile), sequential
//                 over the sequence's chunks.  The fp32 state lives in MFMA
//                 accumulators; per chunk
//                     X = W S,  Y = Qt S,  Delta = U - X,
//                     O = Y + Aqk Delta,  S <- Diag(gL) S + Kbar^T Delta.
//                 S and Delta enter W S and Kbar^T Delta as bf16 hi + lo pairs
//                 (about 16 significant bits), so the carried state, the final
//                 state and the slice summaries keep fp32-level accuracy.
//
// Chunk algebra (derived from the token recurrence, see kda_valu.hip):
//   Akk[r,i] = sum_c k^_rc k^_ic e^{gamma_rc-gamma_ic} (i<r), Aqk likewise with
//   q^ (i<=r), Tm = (I + Diag(beta) Akk)^-1, W = Tm Diag(beta)(K^ e^gamma),
//   U = Tm Diag(beta) V, Qt = scale Q^ e^gamma, Kbar = K^ e^{gamma_L-gamma},
//   gL = e^{gamma_L}, Aqk scaled by `scale` and masked to i <= r.
//
// Decay factors.  Rows of a chunk form four 16-row blocks b.  With lambda the
// cumulative log-decay from the start of a row's own block, Lam_b the block
// total and Gam_b the sum of the totals of the blocks before b:
//   e^{gamma_r - gamma_i} = e^{lambda_r} * e^{Gam_R - Gam_{I+1}} * e^{Lam_I - lambda_i}
// for rows r in block R and i in an earlier block I: three factors <= 1, so
// nothing overflows.  Inside one block (I = R) the split is
//   e^{lambda_r} * (e^{Lam_R - lambda_i} e^{-Lam_R}),
// whose second factor is >= 1; it is used while the block's total decay stays
// below 80 in every channel (e^80 fits bf16/fp32), and an exact per-pair path
// takes over otherwise.
//
// MFMA: v_mfma_f32_16x16x32_bf16.  Lane l = 16 g + n (g = l/16, n = l%16):
//   A operand  lane holds A[n][8g + e], e = 0..7      (m = n, k = 8g+e)
//   B operand  lane holds B[8g + e][n]
//   C/D        lane holds D[4g + e][n], e = 0..3
// A k-step of 32 uses the k order sigma(g, e) = e<4 ? 4g+e : 16+4g+(e-4): two
// accumulator tiles (rows 0-15 and 16-31) then give a B operand, and a matrix
// product with a 0/1 selection matrix turns "one row, 8 columns per lane"
// registers into accumulator layout (a transpose on the matrix cores).
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kC = 64;
constexpr int kThreads = 256;
constexpr int kXcds = 8;  // accelerator complex dies of an MI355X, each with its own L2
constexpr float kDiagSafe = 80.f;  // largest in-block decay the factorised diagonal accepts
constexpr float kGateFloor = -110.f;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ int sig(int g, int e) { return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4); }

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
  return r;
}
__device__ __forceinline__ bf16x8 pair_frag(f32x4 lo, f32x4 hi) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (__bf16)lo[e];
    r[e + 4] = (__bf16)hi[e];
  }
  return r;
}
// four fp32 -> four bf16 in 8 bytes, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint2 pk4(float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const bf16x4 r = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
  const u32x2 u = __builtin_bit_cast(u32x2, r);
  return make_uint2(u.x, u.y);
}
__device__ __forceinline__ uint2 pk4(f32x4 v) { return pk4(v[0], v[1], v[2], v[3]); }
// x = hi + lo with hi = bf16(x) and lo = x - hi (exact in fp32), both returned
// as fp32 values that are exactly representable in bf16 (hi) or rounded once (lo)
__device__ __forceinline__ void split4(f32x4 x, f32x4& hi, f32x4& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = (float)(__bf16)x[e];
    lo[e] = x[e] - hi[e];
  }
}
// Two accumulator tiles as one B operand in bf16 hi + lo parts: hi = bf16(x),
// lo = bf16(x - hi), so hi + lo carries about 16 significant bits of x.
__device__ __forceinline__ void split_frag(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
  f32x4 ah, al, bh, bl;
  split4(a, ah, al);
  split4(b, bh, bl);
  hi = pair_frag(ah, bh);
  lo = pair_frag(al, bl);
}
__device__ __forceinline__ void unpack4(uint2 u, float* out) {
  out[0] = bf16_to_f32((bf16)(u.x & 0xffff));
  out[1] = bf16_to_f32((bf16)(u.x >> 16));
  out[2] = bf16_to_f32((bf16)(u.y & 0xffff));
  out[3] = bf16_to_f32((bf16)(u.y >> 16));
}
// four consecutive bf16 (8 bytes) -> float
__device__ __forceinline__ void load4_bf16(const bf16* p, float* out) {
  uint2 u = *(const uint2*)p;
  out[0] = bf16_to_f32((bf16)(u.x & 0xffff));
  out[1] = bf16_to_f32((bf16)(u.x >> 16));
  out[2] = bf16_to_f32((bf16)(u.y & 0xffff));
  out[3] = bf16_to_f32((bf16)(u.y >> 16));
}
// Hardware transcendentals (v_exp_f32 / v_log_f32 are base 2, ~1 ulp): the
// bf16 path's tolerance is far above their error.
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float fsigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + fexp(-x)); }
// In-kernel gate, GATE as in FwdArgs::gate_form (see kda_valu.hip for the floor
// at -110), computed in base-2 units.  x2 = x log2(e) and lb2 = lb log2(e) in,
// the log-decay times log2(e) out, so that the decays are plain exp2 (no
// scaling multiply per element): softplus(x) log2(e) = max(x2, 0) +
// log2(1 + 2^-|x2|) and sigmoid(A x) = 1 / (1 + 2^(-A x2)).  A = 0 (GATE 0, 2)
// or lb2 = 0 (GATE 1) gives a zero gate, which masks rows past the chunk end.
constexpr float kLog2e = 1.4426950408889634f;
template <int GATE>
__device__ __forceinline__ float fgate2(float x2, float A, float lb2) {
  float g;
  if (GATE == 1) {
    g = lb2 * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-A * x2));
  } else {
    g = -A * (fmaxf(x2, 0.f) + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(x2))));
    if (GATE == 2) g = fmaxf(g, lb2);
  }
  return fmaxf(g, kGateFloor * kLog2e);
}
// Sum over the four 16-lane rows of the wave, in every lane.
__device__ __forceinline__ float rows_sum4(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}
// Row shift right by N inside each 16-lane row (DPP row_shr), zero fill.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, true));
}

// 0/1 selection fragment: as a B operand it picks logical column 16*half + n
// of a 32-wide k-step laid out in sigma order.
__device__ __forceinline__ bf16x8 select_frag(int g, int n, int half) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)((sig(g, e) == 16 * half + n) ? 1.f : 0.f);
  return r;
}

// ---------------------------------------------------------------------------
// Short convolution of width 4 + SiLU applied as q, k and v are loaded
// (FwdArgs::conv).  The lanes 16g + n of a 16-lane row group hold the same
// channels of token rows r0 + n; the inputs of rows r - 1, r - 2 and r - 3
// come from the lanes below (DPP row shifts) and, for the group's first three
// rows, from hx: each lane's copy of row r0 + n - 3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void window3(uint32_t x, uint32_t hx, uint32_t& r1, uint32_t& r2,
                                        uint32_t& r3) {
  const int xi = (int)x, hi = (int)hx;
  // lane n < s takes row r0 + n - s from the halo copy of lane n - s + 3
  const int h2 = __builtin_amdgcn_update_dpp(0, hi, 0x102, 0xF, 0xF, false);  // row_shl:2
  const int h1 = __builtin_amdgcn_update_dpp(0, hi, 0x101, 0xF, 0xF, false);  // row_shl:1
  // lane n >= s takes lane n - s (row_shr:s); the others keep the halo value
  r1 = (uint32_t)__builtin_amdgcn_update_dpp(h2, xi, 0x111, 0xF, 0xF, false);
  r2 = (uint32_t)__builtin_amdgcn_update_dpp(h1, xi, 0x112, 0xF, 0xF, false);
  r3 = (uint32_t)__builtin_amdgcn_update_dpp(hi, xi, 0x113, 0xF, 0xF, false);
}
// row r0 + n - 3 from the previous 16-row block of the same lanes (row_shl:13)
__device__ __forceinline__ uint2 halo_from_block(uint2 prev) {
  return make_uint2((uint32_t)__builtin_amdgcn_update_dpp(0, (int)prev.x, 0x10D, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_update_dpp(0, (int)prev.y, 0x10D, 0xF, 0xF, false));
}
// Four channels of one row (x: 4 bf16; hx its halo as above):
//   y = silu(b + w3 x_r + w2 x_{r-1} + w1 x_{r-2} + w0 x_{r-3}),
// with w = wt[4 e .. 4 e + 3] the taps of channel e and b = bias[e] (0 without
// a bias), in the standalone convolution's order of operations and with its
// SiLU (z times the hardware reciprocal of 1 + e^-z), rounded to bf16 as it
// stores it (f32_to_bf16).  Returns the four results as 4 bf16.
__device__ __forceinline__ uint2 conv4_silu_bf16(uint2 x, uint2 hx, const float* wt, const float* bias) {
  uint32_t a1, a2, a3, c1, c2, c3;
  window3(x.x, hx.x, a1, a2, a3);
  window3(x.y, hx.y, c1, c2, c3);
  const uint32_t back[4][2] = {{x.x, x.y}, {a1, c1}, {a2, c2}, {a3, c3}};  // rows r - s
  uint32_t outw[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float4 w4 = *(const float4*)(wt + 4 * e);
    auto xs = [&](int sb) {
      const uint32_t u = back[sb][e >> 1];
      return __uint_as_float((e & 1) ? (u & 0xffff0000u) : (u << 16));
    };
    float acc = fmaf(w4.w, xs(0), bias ? bias[e] : 0.f);
    acc = fmaf(w4.z, xs(1), acc);
    acc = fmaf(w4.y, xs(2), acc);
    acc = fmaf(w4.x, xs(3), acc);
    const float yy = acc * __builtin_amdgcn_rcpf(1.f + __expf(-acc));
    outw[e >> 1] |= (uint32_t)f32_to_bf16(yy) << (16 * (e & 1));
  }
  return make_uint2(outw[0], outw[1]);
}

// ---------------------------------------------------------------------------
// Chunk record layout (bytes, per chunk-head), shared by both kernels.
// ---------------------------------------------------------------------------
template <int K, int V>
struct Rec {
  static constexpr int NKJ = K / 32, NKT = K / 16, NVT = V / 16;
  static constexpr int kFrag = 1024;                        // 64 lanes x 16 B
  static constexpr int oQt = 0;                             // [4][NKJ] frags
  static constexpr int oW = oQt + 4 * NKJ * kFrag;          // [4][NKJ] frags
  static constexpr int oKbar = oW + 4 * NKJ * kFrag;        // [NKT][2] frags
  static constexpr int oGL = oKbar + NKT * 2 * kFrag;       // [K] fp32
  static constexpr int kStage = oGL + K * 4;                // staged into LDS by the state pass
  static constexpr int oAqk = kStage;                       // [4][2] frags (read straight to registers)
  static constexpr int oU = oAqk + 8 * kFrag;               // [4][NVT] tiles of 64 lanes x 8 B
  static constexpr int kBytes = oU + 4 * NVT * 512;
  // the state pass copies the stage in whole 1 KiB copies (64 lanes x 16 B);
  // the rounded stage still ends inside the record
  static constexpr int kStageCopies = (kStage + 1023) / 1024;
  static_assert(kStage % 16 == 0 && kBytes % 256 == 0, "record alignment");
  static_assert(kStageCopies * 1024 <= kBytes, "rounded stage must stay inside the record");
};

// ---------------------------------------------------------------------------
// Kernel A: prologue + chunk-local factors.
// ---------------------------------------------------------------------------
// Per-channel factor table rows (fp32, [kNF][K]) built once per workgroup from
// the block totals Lam_b (b = 0..3), with Gam_b = sum_{b'<b} Lam_b':
enum {
  kF_LAM = 0,    // 4 rows: Lam_b
  kF_EG = 4,     // 4 rows: e^{Gam_b}
  kF_EL = 8,     // 4 rows: e^{gamma_L - Gam_{b+1}}
  kF_EML = 12,   // 4 rows: e^{-Lam_b} (diagonal blocks; used while Lam_b >= -80)
  kF_M20 = 16,   // e^{Gam_2 - Gam_1} = e^{Lam_1}
  kF_M30 = 17,   // e^{Gam_3 - Gam_1} = e^{Lam_1 + Lam_2}
  kF_M31 = 18,   // e^{Gam_3 - Gam_2} = e^{Lam_2}
  kF_GL = 19,    // e^{gamma_L}
  kNF = 20
};

// One chunk-head.  EXACT = false: the common kernel; a 16-row block whose
// decay exceeds the factorised range makes the workgroup append the chunk-head
// to a fix-up list instead.  EXACT = true: the fix-up, with the exact per-pair
// path on such blocks.  GATE: the gate form (FwdArgs::gate_form).  CONV: q, k
// and v are the raw projections, convolved on load (FwdArgs::conv).  OUT32:
// the backward's recomputation; instead of a record, the factors go to the
// fp32 row-major arrays the backward reads (rq, rk, bt per token-head; Qt,
// Kb, W, U, Aqk, Akk_out, Tm_out, gL per chunk-head with C = FwdArgs::C rows;
// Qt, Kb, W, U, Aqk and Akk_out as bf16 when FwdArgs::ws_bf16 is set, U then
// as 16 x 16 accumulator tiles).
template <int K, int V, bool EXACT, int GATE, bool CONV, bool OUT32 = false>
__device__ __forceinline__ void chunk_body(const FwdArgs& a, const int jchunk, const int h,
                                           const int tok0, const int L, char* const rec,
                                           const bool keep_ok = false) {
  using R = Rec<K, V>;
  constexpr int NKJ = K / 32, NVJ = V / 32, NVT = V / 16, KL = K / 4;
  const int H = a.H;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = 16 * w + n;
  const bool valid = row < L;
  const int64_t th = (int64_t)(tok0 + (valid ? row : 0)) * H + h;  // token-head index
  // the same token at the key head this value head reads (grouped value heads)
  const int64_t thk = (int64_t)(tok0 + (valid ? row : 0)) * a.HK + h / (H / a.HK);
  // beta and a_log are issued with the row loads so that their latency is not
  // paid again after them
  const bf16 braw = ((const bf16*)a.beta)[th];
  const float alog = a.a_log[h];
  // the convolution's window reaches back into the previous chunk unless this
  // chunk starts its sequence (then the inputs before it count as zero)
  const bool first = CONV && (jchunk == 0 || a.chunk_seq[jchunk - 1] != a.chunk_seq[jchunk]);
  const int hk = h / (H / a.HK);  // the key head of q and k

  // the factor table (steps 3-5) and the diagonal Akk blocks (step 6) share storage
  __shared__ __attribute__((aligned(16))) float sFacMem[kNF * K];
  float (*sFac)[K] = (float(*)[K])sFacMem;
  float (*sDg)[16][16] = (float(*)[16][16])sFacMem;  // fp32 diagonal Akk blocks (step 6)
  static_assert(4 * 16 * 16 <= kNF * K, "sDg must fit in the factor table");
  __shared__ __attribute__((aligned(16))) float sBeta[kC];
  __shared__ bf16x8 sX[4][NKJ][64];
  __shared__ __attribute__((aligned(16))) bf16 sA[kC][72];  // Akk (bf16), rows padded
  // sKb (fragments, steps 4-5) and sT (triangular inverse, steps 6-7) share storage
  __shared__ __attribute__((aligned(16))) char sU1[(kC * 68 * 4 > 4 * NKJ * 64 * 16) ? kC * 68 * 4 : 4 * NKJ * 64 * 16];
  bf16x8 (*sKb)[NKJ][64] = (bf16x8(*)[NKJ][64])sU1;
  float (*sT)[68] = (float(*)[68])sU1;

  // ---- 1-3. own row: q^, k^ (L2 norm), gate, cumulative log-decay in the block ----
  constexpr int NJOBS = NKJ + NVJ;  // W channel pairs, then U value pairs
  int upair = -1;
  for (int job = w; job < NJOBS; job += 4)
    if (job >= NKJ) upair = job - NKJ;
  // Loads q, k, gate of the lane's row at channels 32j + sig(g, e), normalises
  // q and k, applies the gate and scans it over the 16 rows of the block.
  // Used once up front and again by the exact diagonal path.
  auto row_prologue = [&](float* qv, float* kv, float* lam, bool emit) __attribute__((always_inline)) {
    const bf16* q = (const bf16*)a.q + thk * K;
    const bf16* k = (const bf16*)a.k + thk * K;
    const bf16* gt = (const bf16*)a.gate + th * K;
    const float* db = a.dt_bias + (int64_t)h * K;
    // CONV: the halo row 16w + n - 3 (used by lanes n < 3): zero before the
    // sequence start; rows past the chunk end read row 0 (they only feed rows
    // past the chunk end)
    const int hr = row - 3;
    const bool hok = hr < 0 ? !first : hr < L;
    const int64_t thh = (int64_t)(tok0 + (hok ? hr : 0)) * a.HK + hk;
    auto conv_piece = [&](const bf16* xrow, const bf16* xhalo, const float* w, const float* b, int c,
                          float* out) __attribute__((always_inline)) {
      uint2 hx = *(const uint2*)(xhalo + c);
      if (!hok) hx = make_uint2(0u, 0u);
      const uint2 y = conv4_silu_bf16(*(const uint2*)(xrow + c), hx, w + ((int64_t)hk * K + c) * 4,
                                      b ? b + (int64_t)hk * K + c : nullptr);
      unpack4(y, out);
    };
    // rows past the chunk end read the chunk's first row (th is clamped) and
    // are zeroed below through the norm scale and the gate select
#pragma unroll
    for (int j = 0; j < NKJ; ++j) {
      const int c0 = 32 * j + 4 * g, c1 = c0 + 16;
      if (CONV) {
        const bf16* qh = (const bf16*)a.q + thh * K;
        const bf16* kh = (const bf16*)a.k + thh * K;
        conv_piece(q, qh, a.conv_wq, a.conv_bq, c0, qv + 8 * j);
        conv_piece(q, qh, a.conv_wq, a.conv_bq, c1, qv + 8 * j + 4);
        conv_piece(k, kh, a.conv_wk, a.conv_bk, c0, kv + 8 * j);
        conv_piece(k, kh, a.conv_wk, a.conv_bk, c1, kv + 8 * j + 4);
      } else {
        load4_bf16(q + c0, qv + 8 * j);
        load4_bf16(q + c1, qv + 8 * j + 4);
        load4_bf16(k + c0, kv + 8 * j);
        load4_bf16(k + c1, kv + 8 * j + 4);
      }
      load4_bf16(gt + c0, lam + 8 * j);
      load4_bf16(gt + c1, lam + 8 * j + 4);
      const float4 d0 = *(const float4*)(db + c0), d1 = *(const float4*)(db + c1);
      lam[8 * j + 0] += d0.x; lam[8 * j + 1] += d0.y; lam[8 * j + 2] += d0.z; lam[8 * j + 3] += d0.w;
      lam[8 * j + 4] += d1.x; lam[8 * j + 5] += d1.y; lam[8 * j + 6] += d1.z; lam[8 * j + 7] += d1.w;
#pragma unroll
      for (int e = 0; e < 8; ++e) lam[8 * j + e] *= kLog2e;
    }
    float ssq = 0.f, ssk = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < KL; ++s2) {
      ssq = fmaf(qv[s2], qv[s2], ssq);
      ssk = fmaf(kv[s2], kv[s2], ssk);
    }
    ssq = rows_sum4(ssq);
    ssk = rows_sum4(ssk);
    const float rq = valid ? __builtin_amdgcn_rsqf(ssq + 1e-6f) : 0.f;
    const float rk = valid ? __builtin_amdgcn_rsqf(ssk + 1e-6f) : 0.f;
    // q^ carries the attention scale from here on (Qt and Aqk are scaled)
    const float rqs = rq * a.scale;
    // a zero coefficient zeroes the gate of a row past the chunk end
    const float A = valid ? fexp(alog) : 0.f;
    const float lb2 = valid ? a.lb * kLog2e : 0.f;
#pragma unroll
    for (int s2 = 0; s2 < KL; ++s2) {
      qv[s2] *= rqs;
      kv[s2] *= rk;
    }
#pragma unroll
    for (int s2 = 0; s2 < KL; ++s2) lam[s2] = fgate2<GATE>(lam[s2], A, GATE == 1 ? lb2 : a.lb * kLog2e);
    if constexpr (OUT32) {
      // the norm scales of a valid row; q^ = q rq is rebuilt from them
      if (emit && valid && g == 0) {
        a.rq[th] = rq;
        a.rk[th] = rk;
      }
    }
    // the block scan, one shift step over all channels at a time (no DPP
    // read waits on the add just before it)
#pragma unroll
    for (int s2 = 0; s2 < KL; ++s2) lam[s2] += row_shr<1>(lam[s2]);
#pragma unroll
    for (int s2 = 0; s2 < KL; ++s2) lam[s2] += row_shr<2>(lam[s2]);
#pragma unroll
    for (int s2 = 0; s2 < KL; ++s2) lam[s2] += row_shr<4>(lam[s2]);
#pragma unroll
    for (int s2 = 0; s2 < KL; ++s2) lam[s2] += row_shr<8>(lam[s2]);
  };
  float qv[KL], kv[KL], lam[KL];
  row_prologue(qv, kv, lam, true);
  const float beta_r = valid ? fsigmoid(bf16_to_f32(braw)) : 0.f;
  // OUT32: rows and columns of the chunk-head's C x C, C x K and C x V arrays
  const int C = a.C;
  const int64_t chb = (int64_t)jchunk * H + h;
  if (OUT32 && g == 0 && valid) a.bt[th] = beta_r;
  if (n == 15) {
#pragma unroll
    for (int j = 0; j < NKJ; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) sFac[kF_LAM + w][32 * j + sig(g, e)] = lam[8 * j + e];
  }
  if (g == 0) sBeta[row] = beta_r;
  __syncthreads();
  // per-channel factor table, on waves 2 and 3 (wave 0 carries the longest
  // part of the triangular inverse below)
  static_assert(K <= kThreads - 128, "one factor-table channel per thread of waves 2 and 3");
  if (const int c = tid - 128; c >= 0 && c < K) {
    const float l0 = sFac[kF_LAM + 0][c], l1 = sFac[kF_LAM + 1][c];
    const float l2 = sFac[kF_LAM + 2][c], l3 = sFac[kF_LAM + 3][c];
    const float gam[5] = {0.f, l0, l0 + l1, l0 + l1 + l2, l0 + l1 + l2 + l3};
    const float lamb[4] = {l0, l1, l2, l3};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      sFac[kF_EG + b][c] = __builtin_amdgcn_exp2f(gam[b]);
      sFac[kF_EL + b][c] = __builtin_amdgcn_exp2f(gam[4] - gam[b + 1]);
      sFac[kF_EML + b][c] = __builtin_amdgcn_exp2f(-lamb[b]);
    }
    sFac[kF_M20][c] = __builtin_amdgcn_exp2f(l1);
    sFac[kF_M30][c] = __builtin_amdgcn_exp2f(l1 + l2);
    sFac[kF_M31][c] = __builtin_amdgcn_exp2f(l2);
    sFac[kF_GL][c] = __builtin_amdgcn_exp2f(gam[4]);
  }
  __syncthreads();

  // factor of table row `rowf` for the lane's 8 channels of k-step j
  auto fac8 = [&](int rowf, int j, float* out) {
    const float4 lo = *(const float4*)&sFac[rowf][32 * j + 4 * g];
    const float4 hi = *(const float4*)&sFac[rowf][32 * j + 16 + 4 * g];
    out[0] = lo.x; out[1] = lo.y; out[2] = lo.z; out[3] = lo.w;
    out[4] = hi.x; out[5] = hi.y; out[6] = hi.z; out[7] = hi.w;
  };

  // ---- the block totals decide the exact diagonal path ----
  float negmax = 0.f;
#pragma unroll
  for (int j = 0; j < NKJ; ++j) {
    float lt[8];
    fac8(kF_LAM + w, j, lt);
#pragma unroll
    for (int e = 0; e < 8; ++e) negmax = fmaxf(negmax, -lt[e]);
  }
  // (log-decays are in base-2 units here)
  const bool over = __builtin_amdgcn_ballot_w64(negmax > kDiagSafe * kLog2e) != 0;  // wave-uniform
  const bool exact_diag = EXACT && over;
  // keep: a sequence of this one chunk, starting from a zero state, is
  // finished here (keep_ok), unless the chunk-head needs the exact fix-up.
  // Then nothing goes to the record: Kbar^T fragments go to sX (whose W
  // operands are not needed), U to sU1, the Aqk fragments stay in registers.
  // The workgroup's decision takes two barriers; it is made here only when
  // the chunk may be kept, else after step 4, where its first barrier is the
  // one step 4 needs anyway.
  __shared__ int sNeedExact;
  auto decide_exact = [&]() {
    if (tid == 0) sNeedExact = 0;
    __syncthreads();
    if (over && lane == 0) sNeedExact = 1;
    __syncthreads();
    const bool need = sNeedExact != 0;
    if (tid == 0 && need) {
      // each chunk-head appends once after the chunk table cleared the count,
      // so slot < NT*H; the test keeps a stale count from writing past the list
      const int slot = atomicAdd(a.exact_count, 1);
      if (slot < a.NT * H) a.exact_list[slot] = jchunk * H + h;
    }
    return need;
  };
  bool keep = false;
  if (!EXACT && keep_ok) keep = !decide_exact();

  // ---- 4. per-element factors; fragments to LDS and to the record ----
  const bf16x8 sel0 = select_frag(g, n, 0), sel1 = select_frag(g, n, 1);
  bf16x8 qrow[NKJ], krow[NKJ], kdiag[NKJ];
  {
#pragma unroll
    for (int j = 0; j < NKJ; ++j) {
      float lt[8], eg[8], el[8], eml[8];
      fac8(kF_LAM + w, j, lt);
      fac8(kF_EG + w, j, eg);
      fac8(kF_EL + w, j, el);
      fac8(kF_EML + w, j, eml);
      float fq[8], fk[8], fx[8], fkb[8], fkbar[8], fqr[8], fkd[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float l = lam[8 * j + e];
        const float ef = __builtin_amdgcn_exp2f(l);          // e^{gamma_r - Gam_w}
        const float F = __builtin_amdgcn_exp2f(lt[e] - l);   // e^{Gam_{w+1} - gamma_r}
        fqr[e] = qv[8 * j + e] * ef;
        fk[e] = kv[8 * j + e] * ef;
        fq[e] = fqr[e] * eg[e];
        fx[e] = beta_r * fk[e] * eg[e];
        fkb[e] = kv[8 * j + e] * F;
        fkbar[e] = fkb[e] * el[e];
        fkd[e] = fkb[e] * eml[e];            // e^{-gamma_r + Gam_w}: diagonal block
      }
      qrow[j] = pack8(fqr);
      krow[j] = pack8(fk);
      kdiag[j] = pack8(fkd);
      // keep the packed fragments (not their fp32 sources) live into step 5
      asm volatile("" : "+v"(qrow[j]), "+v"(krow[j]), "+v"(kdiag[j]));
      if (OUT32) {
        // Qt and Kbar rows in fp32 (zero past the chunk end: q^ = k^ = 0 there)
        sX[w][j][lane] = pack8(fx);
        if (row < C) {
          const int64_t o = (chb * C + row) * K + 32 * j + 4 * g;
          if (a.ws_bf16) {
            *(uint2*)((bf16*)a.Qt + o) = pk4(fq[0], fq[1], fq[2], fq[3]);
            *(uint2*)((bf16*)a.Qt + o + 16) = pk4(fq[4], fq[5], fq[6], fq[7]);
            *(uint2*)((bf16*)a.Kb + o) = pk4(fkbar[0], fkbar[1], fkbar[2], fkbar[3]);
            *(uint2*)((bf16*)a.Kb + o + 16) = pk4(fkbar[4], fkbar[5], fkbar[6], fkbar[7]);
          } else {
            *(float4*)(((float*)a.Qt) + o) = make_float4(fq[0], fq[1], fq[2], fq[3]);
            *(float4*)(((float*)a.Qt) + o + 16) = make_float4(fq[4], fq[5], fq[6], fq[7]);
            *(float4*)(((float*)a.Kb) + o) = make_float4(fkbar[0], fkbar[1], fkbar[2], fkbar[3]);
            *(float4*)(((float*)a.Kb) + o + 16) = make_float4(fkbar[4], fkbar[5], fkbar[6], fkbar[7]);
          }
        }
      } else if (!keep) {
        ((bf16x8*)(rec + R::oQt))[(w * NKJ + j) * 64 + lane] = pack8(fq);
        sX[w][j][lane] = pack8(fx);
      }
      sKb[w][j][lane] = pack8(fkb);
      // Kbar^T fragments (a, w/2): this block's rows transposed on the matrix
      // cores, written as the (w%2) half of each lane's 16 bytes
      if (!OUT32) {
        const bf16x8 kb8 = pack8(fkbar);
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2) {
          const f32x4 d = mfma(kb8, a2 ? sel1 : sel0, zero4());
          const uint2 u = pk4(d);
          const int at = 2 * j + a2;
          const int off = ((at * 2 + (w >> 1)) * 64 + lane) * 16 + 8 * (w & 1);
          if (keep) *(uint2*)((char*)&sX[0][0][0] + off) = u;
          else *(uint2*)(rec + R::oKbar + off) = u;
        }
      }
    }
  }
  if (OUT32)
    for (int c = tid; c < K; c += kThreads) a.gL[chb * K + c] = sFac[kF_GL][c];
  else if (!keep)
    for (int c = tid; c < K; c += kThreads) ((float*)(rec + R::oGL))[c] = sFac[kF_GL][c];
  if (!EXACT && !keep_ok) decide_exact();
  else __syncthreads();

  // ---- 5. decayed key/query products, blocks (I <= R = w), transposed tiles ----
  f32x4 dq[4], dk[4];
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    dq[I] = zero4();
    dk[I] = zero4();
    if (I > w) continue;
    if (16 * w >= L) continue;  // rows past the chunk end: q^ = k^ = 0, so the products are zero
    if (I == w && exact_diag) continue;  // filled by the exact path below
    // factor row e^{Gam_w - Gam_{I+1}} below the diagonal (the diagonal
    // operand already carries e^{-Lam_w})
    int frow = -1;
    if (w == 2 && I == 0) frow = kF_M20;
    else if (w == 3 && I == 0) frow = kF_M30;
    else if (w == 3 && I == 1) frow = kF_M31;
#pragma unroll
    for (int j = 0; j < NKJ; ++j) {
      bf16x8 kc = (I == w) ? kdiag[j] : sKb[I][j][lane];
      if (frow >= 0) {
        float m[8], f[8];
        fac8(frow, j, m);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (float)kc[e] * m[e];
        kc = pack8(f);
      }
      dq[I] = mfma(kc, qrow[j], dq[I]);
      dk[I] = mfma(kc, krow[j], dk[I]);
    }
  }
  if (EXACT && exact_diag) {
    // exact per-pair path for the diagonal block (the block's decay exceeds the
    // factorised range).  Lane (g, n) is row n; for every row i of the block the
    // four g-lanes sum their channels and lane g keeps the sums for i = 4g..4g+3,
    // which are its entries of the transposed tile.  q^, k^ and lambda are
    // recomputed so that they need not stay live until here.
    row_prologue(qv, kv, lam, false);
    f32x4 eq = zero4(), ek = zero4();
#pragma unroll 1
    for (int i = 0; i < 16; ++i) {
      float pq = 0.f, pk = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < KL; ++s2) {
        const float ki = __shfl(kv[s2], 16 * g + i);
        const float li = __shfl(lam[s2], 16 * g + i);
        const float d = (i <= n) ? __builtin_amdgcn_exp2f(lam[s2] - li) : 0.f;
        pq = fmaf(qv[s2] * ki, d, pq);
        pk = fmaf(kv[s2] * ki, d, pk);
      }
      pq = rows_sum4(pq);
      pk = rows_sum4(pk);
      const bool mine = (i >> 2) == g;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool sel = mine && ((i & 3) == e);
        eq[e] = sel ? pq : eq[e];
        ek[e] = sel ? pk : ek[e];
      }
    }
    dq[w] = eq;
    dk[w] = ek;
  }
  // masks: Akk strictly lower -> LDS (bf16, row r = 16w+n; the diagonal block
  // also in fp32 after the barrier), Aqk lower incl. diagonal -> record
  float4 dgv;
  bf16x8 fA0, fA1;  // this row block's Aqk fragments (kept for a finished sequence)
  {
    const int r = 16 * w + n;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      float vv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * I + 4 * g + e;
        vv[e] = (i < r) ? dk[I][e] : 0.f;
        dq[I][e] = (i <= r) ? dq[I][e] : 0.f;
      }
      *(uint2*)&sA[r][16 * I + 4 * g] = pk4(vv[0], vv[1], vv[2], vv[3]);
      if (I == w) dgv = make_float4(vv[0], vv[1], vv[2], vv[3]);
      if (OUT32 && r < C && 16 * I < C) {
        // Akk strictly lower, Aqk (scaled) lower with the diagonal
        const int64_t o = (chb * C + r) * C + 16 * I + 4 * g;
        // (bf16 Akk with ws_bf16: the operand Tm was solved from, as in sA)
        if (a.ws_bf16) {
          *(uint2*)((bf16*)a.Akk_out + o) = pk4(vv[0], vv[1], vv[2], vv[3]);
          *(uint2*)((bf16*)a.Aqk + o) = pk4(dq[I]);
        } else {
          *(float4*)(a.Akk_out + o) = make_float4(vv[0], vv[1], vv[2], vv[3]);
          *(float4*)(((float*)a.Aqk) + o) = make_float4(dq[I][0], dq[I][1], dq[I][2], dq[I][3]);
        }
      }
    }
    fA0 = pair_frag(dq[0], dq[1]);
    fA1 = pair_frag(dq[2], dq[3]);
    if (!keep && !OUT32) {
      bf16x8* aq = (bf16x8*)(rec + R::oAqk);
      aq[(w * 2 + 0) * 64 + lane] = fA0;
      aq[(w * 2 + 1) * 64 + lane] = fA1;
    }
  }
  __syncthreads();

  // this wave's value-pair job (at most one): its V rows are fetched now, so
  // that the triangular solve hides their latency
  // (rows past the chunk end read row 0 and are zeroed by their beta = 0)
  uint2 vraw[4][2], vhalo[2];
  if (upair >= 0) {
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const int ri = 16 * I + n < L ? 16 * I + n : 0;
      const bf16* vp = (const bf16*)a.v + ((int64_t)(tok0 + ri) * H + h) * V + 32 * upair + 4 * g;
      vraw[I][0] = *(const uint2*)vp;
      vraw[I][1] = *(const uint2*)(vp + 16);
    }
    if (CONV) {
      // the rows before the chunk (lanes n < 3), zero before the sequence start
      const int hr = n - 3;
      const bool hok = hr < 0 ? !first : hr < L;
      const bf16* vp = (const bf16*)a.v + ((int64_t)(tok0 + (hok ? hr : 0)) * H + h) * V + 32 * upair + 4 * g;
      vhalo[0] = hok ? *(const uint2*)vp : make_uint2(0u, 0u);
      vhalo[1] = hok ? *(const uint2*)(vp + 16) : make_uint2(0u, 0u);
    }
  }

  // ---- 6. Tm = (I + Diag(beta) Akk)^-1 ----
  // (a) zero Tm's strictly-upper blocks and invert the diagonal blocks in fp32
  //     by forward substitution.  Every lane (g, n) builds column n of block w
  //     in full (the 4 g-lanes redundantly), reading each row of the fp32
  //     diagonal block as float4 broadcasts; the g = 0 lanes write the column.
  *(float4*)&sDg[w][n][4 * g] = dgv;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  {
    const int b0 = 16 * w;
#pragma unroll
    for (int I = 0; I < 4; ++I)
      if (I > w) *(float4*)&sT[b0 + n][16 * I + 4 * g] = make_float4(0.f, 0.f, 0.f, 0.f);
    float bw[16];
#pragma unroll
    for (int i4 = 0; i4 < 16; i4 += 4) {
      const float4 b4 = *(const float4*)&sBeta[b0 + i4];
      bw[i4] = b4.x; bw[i4 + 1] = b4.y; bw[i4 + 2] = b4.z; bw[i4 + 3] = b4.w;
    }
    float tc[16];
    if (b0 >= L) {
      // a block past the chunk end (beta = 0): its inverse is the identity
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) tc[rr] = (n == rr) ? 1.f : 0.f;
    } else {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i4 = 0; i4 < rr; i4 += 4) {
          const float4 a4 = *(const float4*)&sDg[w][rr][i4];
          const float ar[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (i4 + e < rr) acc[e] = fmaf(ar[e], tc[i4 + e], acc[e]);
        }
        const float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        // 1 on the diagonal, -beta * sum below it, 0 above (sum is finite)
        tc[rr] = fmaf((n < rr) ? -bw[rr] : 0.f, sum, (n == rr) ? 1.f : 0.f);
      }
    }
    if (g == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sT[b0 + i][b0 + n] = tc[i];
    }
  }
  __syncthreads();
  // (b) column block Ib = w, block rows R = w+1..3 in order, inside one wave,
  //     on the matrix cores: Tm_{R,Ib} = -Tm_RR Diag(beta_R) sum_{J=Ib}^{R-1}
  //     Akk_RJ Tm_{J,Ib}.  Tm enters the products as bf16 hi + lo parts (about
  //     16 significant bits); Akk is bf16 already.  Tiles are kept in the
  //     accumulator layout (lane (g, n): rows 4g..4g+3, column n), two of which
  //     form one B operand in sigma order.
  {
    auto colblock = [&](auto ibc) {
      constexpr int Ib = decltype(ibc)::value;
      f32x4 tcol[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) tcol[Ib][e] = sT[16 * Ib + 4 * g + e][16 * Ib + n];
#pragma unroll
      for (int Rb = Ib + 1; Rb < 4; ++Rb) {
        if (16 * Rb >= L) {
          // block rows past the chunk end (beta = 0): Tm_{R,Ib} = 0
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            tcol[Rb][e] = 0.f;
            sT[16 * Rb + 4 * g + e][16 * Ib + n] = 0.f;
          }
          continue;
        }
        f32x4 p = zero4();
#pragma unroll
        for (int J0 = Ib; J0 < Rb; J0 += 2) {
          const bool two = J0 + 1 < Rb;
          float av[8];
          unpack4(*(const uint2*)&sA[16 * Rb + n][16 * J0 + 4 * g], av);
          if (two) unpack4(*(const uint2*)&sA[16 * Rb + n][16 * J0 + 16 + 4 * g], av + 4);
          else av[4] = av[5] = av[6] = av[7] = 0.f;
          const bf16x8 af = pack8(av);
          const f32x4 t1 = two ? tcol[J0 + 1] : zero4();
          f32x4 h0, h1, l0, l1;
          split4(tcol[J0], h0, l0);
          split4(t1, h1, l1);
          p = mfma(af, pair_frag(h0, h1), p);
          p = mfma(af, pair_frag(l0, l1), p);
        }
        const float4 bt = *(const float4*)&sBeta[16 * Rb + 4 * g];
        const f32x4 y = {bt.x * p[0], bt.y * p[1], bt.z * p[2], bt.w * p[3]};
        f32x4 yh, yl;
        split4(y, yh, yl);
        const float4 td = *(const float4*)&sT[16 * Rb + n][16 * Rb + 4 * g];
        f32x4 th, tl;
        split4(f32x4{td.x, td.y, td.z, td.w}, th, tl);
        const bf16x8 tf = pair_frag(th, tl);  // [Tm_RR hi | Tm_RR lo] along k
        f32x4 d = mfma(tf, pair_frag(yh, yh), zero4());
        d = mfma(tf, pair_frag(yl, yl), d);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tcol[Rb][e] = -d[e];
          sT[16 * Rb + 4 * g + e][16 * Ib + n] = -d[e];
        }
      }
    };
    if (w == 0) colblock(std::integral_constant<int, 0>{});
    else if (w == 1) colblock(std::integral_constant<int, 1>{});
    else if (w == 2) colblock(std::integral_constant<int, 2>{});
  }
  __syncthreads();
  if (OUT32)
    for (int p = 4 * tid; p < C * C; p += 4 * kThreads) {
      const int r = p / C, i = p % C;
      *(float4*)(a.Tm_out + chb * C * C + p) = *(const float4*)&sT[r][i];
    }

  // ---- 7. jobs: W (channel pairs), U (value pairs) ----
  bf16x8 tfrag[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float4 lo = *(const float4*)&sT[16 * t + n][32 * j + 4 * g];
      const float4 hi = *(const float4*)&sT[16 * t + n][32 * j + 16 + 4 * g];
      float f[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      tfrag[t][j] = pack8(f);
    }
  // a finished sequence puts U where Tm was (sU1): every wave has read Tm first
  if (keep) __syncthreads();
  for (int job = w; job < NJOBS; job += 4) {
    if (job < NKJ) {
      if (keep) continue;  // W multiplies the state, which is zero here
      const int p = job;
      f32x4 did[4][2];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const bf16x8 src = sX[I][p][lane];
        did[I][0] = mfma(src, sel0, zero4());
        did[I][1] = mfma(src, sel1, zero4());
      }
      {
        // W^T = X^T Tm^T; X^T fragments from the transposed tiles
        bf16x8 xt[2][2];
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
          for (int j = 0; j < 2; ++j) xt[a2][j] = pair_frag(did[2 * j][a2], did[2 * j + 1][a2]);
        bf16x8* wout = (bf16x8*)(rec + R::oW);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          f32x4 acc[2];
#pragma unroll
          for (int a2 = 0; a2 < 2; ++a2) {
            acc[a2] = mfma(xt[a2][0], tfrag[t][0], zero4());
            if (t >= 2) acc[a2] = mfma(xt[a2][1], tfrag[t][1], acc[a2]);
          }
          if (OUT32) {
            // lane (g, n): W[16t + n][32p + 16a2 + 4g + e]
            const int r = 16 * t + n;
            if (r < C)
#pragma unroll
              for (int a2 = 0; a2 < 2; ++a2) {
                const int64_t o = (chb * C + r) * K + 32 * p + 16 * a2 + 4 * g;
                if (a.ws_bf16) *(uint2*)((bf16*)a.W + o) = pk4(acc[a2]);
                else *(f32x4*)(((float*)a.W) + o) = acc[a2];
              }
          } else {
            wout[(t * NKJ + p) * 64 + lane] = pair_frag(acc[0], acc[1]);
          }
        }
      }
    } else {
      const int p = job - NKJ;
      if (CONV) {
        // convolve the V rows in place, last block first: block I's halo is
        // block I - 1's raw rows
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const int64_t c = (int64_t)h * V + 32 * p + 16 * q2 + 4 * g;
          const float* wv = a.conv_wv + c * 4;
          const float* bv = a.conv_bv ? a.conv_bv + c : nullptr;
#pragma unroll
          for (int I = 3; I >= 0; --I) {
            const uint2 hx = I > 0 ? halo_from_block(vraw[I - 1][q2]) : vhalo[q2];
            vraw[I][q2] = conv4_silu_bf16(vraw[I][q2], hx, wv, bv);
          }
        }
      }
      f32x4 did[4][2];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const float bt = sBeta[16 * I + n];  // 0 on rows past the chunk end
        float f[8];
        unpack4(vraw[I][0], f);
        unpack4(vraw[I][1], f + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] *= bt;
        const bf16x8 src = pack8(f);
        did[I][0] = mfma(src, sel0, zero4());
        did[I][1] = mfma(src, sel1, zero4());
      }
      bf16x8 vb[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2) vb[j][a2] = pair_frag(did[2 * j][a2], did[2 * j + 1][a2]);
      uint2* uout = (uint2*)(rec + R::oU);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2) {
          f32x4 acc = mfma(tfrag[t][0], vb[0][a2], zero4());
          if (t >= 2) acc = mfma(tfrag[t][1], vb[1][a2], acc);
          const int at = (t * NVT + 2 * p + a2) * 64 + lane;
          if (OUT32) {
            // lane (g, n): U[16t + 4g + e][32p + 16a2 + n].  bf16 (64-row
            // chunks): as 16 x 16 accumulator tiles, [row tile][column tile]
            // [lane][4], the layout the backward's state pass reads; fp32: row-major
            if (a.ws_bf16) {
              ((uint2*)a.U)[((chb * 4 + t) * NVT + 2 * p + a2) * 64 + lane] = pk4(acc);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 16 * t + 4 * g + e;
                if (r < C) ((float*)a.U)[(chb * C + r) * V + 32 * p + 16 * a2 + n] = acc[e];
              }
            }
          } else if (keep) {
            ((uint2*)sU1)[at] = pk4(acc);
          } else {
            uout[at] = pk4(acc);
          }
        }
    }
  }

  // ---- 8. a one-chunk sequence from a zero state, finished here ----
  // Delta = U, O = Aqk U (wave w: output row tile w of every column tile),
  // final state S = Kbar^T U (wave w: key row tiles w, w+4, ...).  The same
  // products, in the same order, as the state pass for such a chunk.
  if (!EXACT && !OUT32) {
    if (keep) {
      __syncthreads();
      const int seq = a.chunk_seq[jchunk];
      const int64_t sbase = ((int64_t)seq * H + h) * K * V;
      const uint2* sUk = (const uint2*)sU1;
      const bf16x8* sKk = (const bf16x8*)&sX[0][0][0];
      bf16* const o = (bf16*)a.o;
#pragma unroll
      for (int ct = 0; ct < NVT; ++ct) {
        f32x4 D[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float u[4];
          unpack4(sUk[(t * NVT + ct) * 64 + lane], u);
          D[t] = f32x4{u[0], u[1], u[2], u[3]};
        }
        const bf16x8 db0 = pair_frag(D[0], D[1]), db1 = pair_frag(D[2], D[3]);
        f32x4 Y = mfma(db0, fA0, zero4());
        if (w >= 2) Y = mfma(db1, fA1, Y);
        const int r = 16 * w + n;
        if (r < L) *(uint2*)(o + ((int64_t)(tok0 + r) * H + h) * V + 16 * ct + 4 * g) = pk4(Y);
        if (a.fin) {
#pragma unroll
          for (int at = w; at < K / 16; at += 4) {
            const bf16x8 fk0 = sKk[(at * 2 + 0) * 64 + lane], fk1 = sKk[(at * 2 + 1) * 64 + lane];
            f32x4 acc = mfma(fk0, db0, zero4());
            acc = mfma(fk1, db1, acc);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              a.fin[sbase + (int64_t)(16 * at + 4 * g + e) * V + 16 * ct + n] = acc[e];
          }
        }
      }
    }
    if (tid == 0) a.done[jchunk * H + h] = keep ? 1 : 0;
  }
}

template <int K, int V, int GATE, bool CONV>
__global__ __launch_bounds__(kThreads, 3) void k_chunk_mfma(FwdArgs a) {
  const unsigned wid = blockIdx.x, H = (unsigned)a.H;
  const int jchunk = (int)(wid / H), h = (int)(wid % H);
  // the table holds at least gridDim.x / H entries, so the reads below stay in
  // bounds; they are issued together with the count, ahead of its test
  const int nt = *a.nt_dev;
  const int tok0 = a.chunk_tok[jchunk], L = a.chunk_len[jchunk];
  // the sequences of this chunk and of its neighbours in the table, read with
  // the entries above so that one memory latency covers them all (a chain
  // through seq_chunk0 would cost a second one before the first barrier)
  const int sq = a.chunk_seq[jchunk];
  const int sq_prev = jchunk > 0 ? a.chunk_seq[jchunk - 1] : -1;
  const int sq_next = a.chunk_seq[jchunk + 1 < a.NT ? jchunk + 1 : jchunk];
  asm volatile("" ::"s"(tok0), "s"(L));
  if (jchunk >= nt) return;
  // a sequence of this one chunk that starts from a zero state is finished
  // here (chunks of a sequence are consecutive in the table)
  const bool single = sq_prev != sq && (jchunk + 1 >= nt || sq_next != sq);
  const bool keep_ok = !a.summary && !a.norm && a.init == nullptr && single;
  chunk_body<K, V, false, GATE, CONV>(a, jchunk, h, tok0, L,
                                (char*)a.rec + ((int64_t)jchunk * a.H + h) * Rec<K, V>::kBytes,
                                keep_ok);
}

// Fix-up pass: recomputes the listed chunk-heads with the exact diagonal path.
template <int K, int V, int GATE, bool CONV>
__global__ __launch_bounds__(kThreads) void k_chunk_mfma_exact(FwdArgs a) {
  const int count = min(*a.exact_count, a.NT * a.H);
  for (int i = blockIdx.x; i < count; i += gridDim.x) {
    const int ch = a.exact_list[i];
    const int jchunk = ch / a.H;
    chunk_body<K, V, true, GATE, CONV>(a, jchunk, ch % a.H, a.chunk_tok[jchunk], a.chunk_len[jchunk],
                                 (char*)a.rec + (int64_t)ch * Rec<K, V>::kBytes);
    __syncthreads();
  }
}

// The backward's recomputation for bf16 inputs: every chunk-head's factors in
// the fp32 row-major arrays the backward reads (chunk_body's OUT32 mode), the
// chunk-heads that need the exact diagonal path listed for the fix-up pass.
// The products take bf16 operands with fp32 accumulation, as in the forward.
template <int K, int V, int GATE>
__global__ __launch_bounds__(kThreads, 3) void k_chunk_recompute(FwdArgs a) {
  const unsigned wid = blockIdx.x, H = (unsigned)a.H;
  const int jchunk = (int)(wid / H), h = (int)(wid % H);
  // the table holds at least gridDim.x / H entries
  const int nt = *a.nt_dev;
  const int tok0 = a.chunk_tok[jchunk], L = a.chunk_len[jchunk];
  asm volatile("" ::"s"(tok0), "s"(L));
  if (jchunk >= nt) return;
  chunk_body<K, V, false, GATE, false, true>(a, jchunk, h, tok0, L, nullptr);
}

template <int K, int V, int GATE>
__global__ __launch_bounds__(kThreads) void k_chunk_recompute_exact(FwdArgs a) {
  const int count = min(*a.exact_count, a.NT * a.H);
  for (int i = blockIdx.x; i < count; i += gridDim.x) {
    const int ch = a.exact_list[i];
    const int jchunk = ch / a.H;
    chunk_body<K, V, true, GATE, false, true>(a, jchunk, ch % a.H, a.chunk_tok[jchunk],
                                              a.chunk_len[jchunk], nullptr);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Kernel F: the whole forward of one (sequence, head) in one workgroup.
// ---------------------------------------------------------------------------
// For each of the sequence's chunks in order, the four waves first compute the
// chunk's factors exactly as k_chunk_mfma does, but into a record that stays
// in LDS, and then consume it: wave w owns V/64 16-column tiles of the fp32
// state (MFMA accumulators) and forms
//   X = W S,  Delta = U - X,  O = Qt S + Aqk Delta,  S <- Diag(gL) S + Kbar^T Delta
// with S and Delta as bf16 hi + lo pairs in the state's own products.  Nothing
// but q, k, v, gate, beta, the states and o touches HBM.  Blocks whose decay
// leaves the factorised range take the exact per-pair path in place.
template <int K, int V, int GATE, bool CONV>
__global__ __launch_bounds__(kThreads, 1) void k_fused(FwdArgs a) {
  using R = Rec<K, V>;
  constexpr int NKJ = K / 32, NKT = K / 16, NVT = V / 16;
  constexpr int NCT = NVT / 4;  // column tiles per wave
  static_assert(NCT >= 1 && NVT % 4 == 0, "four waves share the value columns");
  const int H = a.H;
  const int64_t nh = blockIdx.x;
  if (nh >= (int64_t)a.N * H) return;
  const int h = (int)(nh % H), seq = (int)(nh / H);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  __shared__ __attribute__((aligned(16))) char sRec[R::kBytes];
  const int jc0 = a.seq_chunk0[seq], jc1 = a.seq_chunk0[seq + 1];
  const int64_t sbase = ((int64_t)seq * H + h) * K * V;

  f32x4 S[NKT][NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = 16 * (w * NCT + ct) + n;
#pragma unroll
    for (int at = 0; at < NKT; ++at)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S[at][ct][e] = a.init ? a.init[sbase + (int64_t)(16 * at + 4 * g + e) * V + col] : 0.f;
  }

  const bf16x8* rQt = (const bf16x8*)(sRec + R::oQt);
  const bf16x8* rW = (const bf16x8*)(sRec + R::oW);
  const bf16x8* rKb = (const bf16x8*)(sRec + R::oKbar);
  const float* rGL = (const float*)(sRec + R::oGL);
  const bf16x8* rA = (const bf16x8*)(sRec + R::oAqk);
  const uint2* rU = (const uint2*)(sRec + R::oU);
  bf16* const o = (bf16*)a.o;

  for (int jc = jc0; jc < jc1; ++jc) {
    const int tok0 = a.chunk_tok[jc], L = a.chunk_len[jc];
    chunk_body<K, V, true, GATE, CONV>(a, jc, h, tok0, L, sRec);
    __syncthreads();
    bf16x8 fA[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      fA[t][0] = rA[(t * 2 + 0) * 64 + lane];
      fA[t][1] = t >= 2 ? rA[(t * 2 + 1) * 64 + lane] : fA[t][0];
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int ctg = w * NCT + ct;
      bf16x8 sb[NKJ], sl[NKJ];
#pragma unroll
      for (int j = 0; j < NKJ; ++j) split_frag(S[2 * j][ct], S[2 * j + 1][ct], sb[j], sl[j]);
      f32x4 X[4], Y[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        X[t] = zero4();
        Y[t] = zero4();
#pragma unroll
        for (int j = 0; j < NKJ; ++j) {
          const bf16x8 fw = rW[(t * NKJ + j) * 64 + lane];
          X[t] = mfma(fw, sb[j], X[t]);
          X[t] = mfma(fw, sl[j], X[t]);
          Y[t] = mfma(sb[j], rQt[(t * NKJ + j) * 64 + lane], Y[t]);
        }
      }
      f32x4 D[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float u[4];
        unpack4(rU[(t * NVT + ctg) * 64 + lane], u);
        D[t] = f32x4{u[0], u[1], u[2], u[3]} - X[t];
      }
      bf16x8 db[2], dl[2];
      split_frag(D[0], D[1], db[0], dl[0]);
      split_frag(D[2], D[3], db[1], dl[1]);
      // output rows 16t+n, columns 16ctg+4g..+3 (transposed tiles), rows
      // past the chunk end are not stored
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        Y[t] = mfma(db[0], fA[t][0], Y[t]);
        if (t >= 2) Y[t] = mfma(db[1], fA[t][1], Y[t]);
        const int r = 16 * t + n;
        if (r < L) *(uint2*)(o + ((int64_t)(tok0 + r) * H + h) * V + 16 * ctg + 4 * g) = pk4(Y[t]);
      }
#pragma unroll
      for (int at = 0; at < NKT; ++at) {
        const float4 gl = *(const float4*)&rGL[16 * at + 4 * g];
        const bf16x8 fk0 = rKb[(at * 2 + 0) * 64 + lane], fk1 = rKb[(at * 2 + 1) * 64 + lane];
        f32x4 acc = {gl.x * S[at][ct][0], gl.y * S[at][ct][1], gl.z * S[at][ct][2], gl.w * S[at][ct][3]};
        acc = mfma(fk0, db[0], acc);
        acc = mfma(fk1, db[1], acc);
        acc = mfma(fk0, dl[0], acc);
        acc = mfma(fk1, dl[1], acc);
        S[at][ct] = acc;
      }
    }
    // every wave is done with this chunk's record before the next overwrites it
    __syncthreads();
  }

  if (a.fin) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int col = 16 * (w * NCT + ct) + n;
#pragma unroll
      for (int at = 0; at < NKT; ++at)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a.fin[sbase + (int64_t)(16 * at + 4 * g + e) * V + col] = S[at][ct][e];
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel B: state pass and output.  SUM = summary mode (state columns only,
// with the transition columns [V, V+K) that start as I and carry no values).
// ---------------------------------------------------------------------------
// CW compute waves (1, 2 or 4) each own one 16-column tile of the state; one
// more wave only streams the records into LDS, so that the compute waves never
// stall on those loads.  Fewer compute waves per workgroup spread a problem
// with few (sequence, head) pairs over more CUs.
// (the bound is the five-wave workgroup for every CW: it keeps the register
// allocation of all variants within 256 without accumulator-register copies)
template <int K, int V, int CW, bool SUM>
__global__ __launch_bounds__(320) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_state_mfma(FwdArgs a) {
  static_assert(64 * (CW + 1) <= 320, "workgroup size");
  using R = Rec<K, V>;
  constexpr int NCT = 1;  // column tiles per compute wave
  constexpr int NKJ = K / 32, NKT = K / 16, NVT = V / 16;
  constexpr int ncols = SUM ? V + K : V;
  constexpr int nct_total = ncols / 16;
  constexpr int tiles_wg = CW * NCT;
  static_assert(nct_total % tiles_wg == 0, "every wave owns whole column tiles");
  constexpr int ntile_wg = nct_total / tiles_wg;
  const int H = a.H;
  // Workgroups are dealt to the 8 XCDs round-robin; the column tiles of one
  // (sequence, head) get consecutive slots of one XCD so that they share its L2.
  const int64_t bid = blockIdx.x;
  const int xcd = (int)(bid % kXcds);
  const int64_t q8 = bid / kXcds;
  const int tileg = (int)(q8 % ntile_wg);
  const int64_t nh = (q8 / ntile_wg) * kXcds + xcd;
  if (nh >= (int64_t)a.N * H) return;
  const int h = (int)(nh % H), seq = (int)(nh / H);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform

  // three stage buffers: chunk c is consumed while c+1 has landed or is landing
  // and c+2 streams in (global -> LDS, no registers), which gives each copy two
  // chunks' time to arrive from HBM
  constexpr int kStageBytes = R::kStageCopies * 1024;
  __shared__ __attribute__((aligned(16))) char sStage0[kStageBytes];
  __shared__ __attribute__((aligned(16))) char sStage1[kStageBytes];
  __shared__ __attribute__((aligned(16))) char sStage2[kStageBytes];
  const int jc0 = a.seq_chunk0[seq], jc1 = a.seq_chunk0[seq + 1];
  // a one-chunk sequence the chunk-factor kernel finished itself
  if (!SUM && jc1 - jc0 == 1 && a.done[(int64_t)jc0 * H + h]) return;
  const char* recbase = (const char*)a.rec;

  if (w == CW) {
    // The loader wave: at the start of chunk c it issues the copy of chunk c+2
    // and then waits only for chunk c+1's copy (vector-memory loads complete
    // in issue order) before the barrier that ends chunk c.  The barrier is
    // written out because a workgroup fence would also wait for the newer
    // copy; this wave reads nothing, and the memory clobber keeps each copy
    // below the barrier that frees its buffer.
    constexpr int kCopies = R::kStageCopies;  // copy instructions per record
    static_assert(kCopies < 64, "wait count field");
    // (the LDS side of a copy is a compile-time buffer: its address goes to M0)
    auto stage = [&](int jc, auto bufc) {
      constexpr int B = decltype(bufc)::value;
      char* const dst = B == 0 ? sStage0 : (B == 1 ? sStage1 : sStage2);
      const char* rec = recbase + ((int64_t)jc * H + h) * R::kBytes;
#pragma unroll
      for (int i = 0; i < kCopies; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(rec + (lane + 64 * i) * 16),
                                         (lds_void*)(&dst[(64 * i) * 16]), 16, 0, 0);
    };
    auto barrier_one_pending = [&]() { asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kCopies) : "memory"); };
    auto barrier_none_pending = [&]() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); };
    // chunk c+2 goes into buffer (c+2) % 3, freed by the barrier ending chunk c-1
    auto step = [&](int jc, auto nbufc) {
      if (jc + 2 < jc1) {
        // let the compute waves' own loads for the next chunk enter the memory
        // queue ahead of this copy
        __builtin_amdgcn_s_sleep(2);
        stage(jc + 2, nbufc);
        barrier_one_pending();
      } else {
        barrier_none_pending();
      }
    };
    if (jc0 < jc1) stage(jc0, std::integral_constant<int, 0>{});
    if (jc0 + 1 < jc1) {
      stage(jc0 + 1, std::integral_constant<int, 1>{});
      barrier_one_pending();
    } else {
      barrier_none_pending();
    }
    for (int jc = jc0; jc < jc1; jc += 3) {
      step(jc, std::integral_constant<int, 2>{});
      if (jc + 1 < jc1) step(jc + 1, std::integral_constant<int, 0>{});
      if (jc + 2 < jc1) step(jc + 2, std::integral_constant<int, 1>{});
    }
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }

  int ctg[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) ctg[ct] = tileg * tiles_wg + w * NCT + ct;
  const int64_t sbase = ((int64_t)seq * H + h) * K * V;

  // state S: K/16 accumulator tiles per column tile
  f32x4 S[NKT][NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = 16 * ctg[ct] + n;
    const bool vcol = col < V;
    const float* init = (!SUM && a.init && vcol) ? a.init + sbase + col : nullptr;
#pragma unroll
    for (int at = 0; at < NKT; ++at)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * at + 4 * g + e;
        float sv = 0.f;
        if (init) sv = init[(int64_t)c * V];
        if (SUM && !vcol) sv = (c == col - V) ? 1.f : 0.f;
        S[at][ct][e] = sv;
      }
  }

  // U tiles of this wave's column tiles for one chunk (zero for transition
  // columns) and the Aqk fragments: read straight to registers, one chunk ahead
  uint2 ucur[NCT][4], unext[NCT][4];
  bf16x8 fA[4][2], fAn[4][2];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int t = 0; t < 4; ++t) ucur[ct][t] = unext[ct][t] = make_uint2(0u, 0u);
  auto load_aqk = [&](const char* rec, bf16x8 (&dst)[4][2]) {
    const bf16x8* ga = (const bf16x8*)(rec + R::oAqk);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      dst[t][0] = ga[(t * 2 + 0) * 64 + lane];
      if (t >= 2) dst[t][1] = ga[(t * 2 + 1) * 64 + lane];
    }
  };
  int tok_cur = 0, len_cur = 0, tok_nxt = 0, len_nxt = 0;
  if (jc0 < jc1) {
    const char* rec = recbase + ((int64_t)jc0 * H + h) * R::kBytes;
    if (!SUM) load_aqk(rec, fA);
    const uint2* ug = (const uint2*)(rec + R::oU);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const bool vt = !SUM || 16 * ctg[ct] < V;  // transition columns carry no values
      const int ut = vt ? ctg[ct] : 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint2 u = ug[(t * NVT + ut) * 64 + lane];
        ucur[ct][t] = vt ? u : make_uint2(0u, 0u);
      }
    }
    tok_cur = a.chunk_tok[jc0];
    len_cur = a.chunk_len[jc0];
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // output of the previous chunk, stored one iteration late so that the
  // stores never hold up the wait for the next record
  uint2 opend[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int t = 0; t < 4; ++t) opend[ct][t] = make_uint2(0u, 0u);
  int otok = 0, olen = 0;
  bf16* const o = (bf16*)a.o;
  // opend[ct][t]: row 16t+n, columns 16*ctg+4g..+3 (the transposed output tile).
  // Rows past the chunk end (and the pass before the first chunk) are written
  // to a small sink in the workspace instead, which keeps the loop branch-free.
  uint2* const sink = (uint2*)a.sink + tid * NCT;
  auto store_out = [&]() {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = 16 * t + n;
      const bool ok = r < olen;
      bf16* orow = o + ((int64_t)(otok + (ok ? r : 0)) * H + h) * V + 4 * g;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        uint2* dst = ok ? (uint2*)(orow + 16 * ctg[ct]) : sink + ct;
        *dst = opend[ct][t];
      }
    }
  };

  // one chunk; BUF (compile-time) is the stage buffer holding it while the
  // loader wave fills the other one.
  auto chunk_step = [&](int jc, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    char* const cur = BUF == 0 ? sStage0 : (BUF == 1 ? sStage1 : sStage2);
    // the next chunk's U tiles, Aqk fragments and table entries (the current
    // chunk's again on the last chunk: harmless, and it keeps the body free of
    // branches)
    const int jn = (jc + 1 < jc1) ? jc + 1 : jc;
    {
      const char* rec = recbase + ((int64_t)jn * H + h) * R::kBytes;
      if (!SUM) load_aqk(rec, fAn);
      const uint2* ug = (const uint2*)(rec + R::oU);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const bool vt = !SUM || 16 * ctg[ct] < V;
        const int ut = vt ? ctg[ct] : 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint2 u = ug[(t * NVT + ut) * 64 + lane];
          unext[ct][t] = vt ? u : make_uint2(0u, 0u);
        }
      }
      tok_nxt = a.chunk_tok[jn];
      len_nxt = a.chunk_len[jn];
    }
    if (!SUM) store_out();
    const bf16x8* sQt = (const bf16x8*)(cur + R::oQt);
    const bf16x8* sW = (const bf16x8*)(cur + R::oW);
    const bf16x8* sKbar = (const bf16x8*)(cur + R::oKbar);
    const float* sGL = (const float*)(cur + R::oGL);
    // the staged A-operand fragments are read from LDS where each product
    // needs them (W, then Qt, then Kbar^T), so that one set is live at a time
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 Ut[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint2 u = ucur[ct][t];
        Ut[t][0] = bf16_to_f32((bf16)(u.x & 0xffff));
        Ut[t][1] = bf16_to_f32((bf16)(u.x >> 16));
        Ut[t][2] = bf16_to_f32((bf16)(u.y & 0xffff));
        Ut[t][3] = bf16_to_f32((bf16)(u.y >> 16));
      }
      // S as B operand (k = key channel in sigma order), as bf16 hi + lo parts:
      // the state's own products (W S here, Kbar^T Delta below) see about 16
      // significant bits of it, so the carried state keeps fp32-level accuracy
      // over long sequences; the output product Qt S uses the hi part alone
      bf16x8 sb[NKJ], sl[NKJ];
#pragma unroll
      for (int j = 0; j < NKJ; ++j) split_frag(S[2 * j][ct], S[2 * j + 1][ct], sb[j], sl[j]);
      // X = W S (rows r, column n); Yt = (Qt S)^T = S^T Qt^T: the same fragments
      // with the operands swapped, giving lane (g, n) row 16t+n, columns 4g..4g+3
      f32x4 X[4], Y[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        X[t] = zero4();
#pragma unroll
        for (int j = 0; j < NKJ; ++j) {
          const bf16x8 fw = sW[(t * NKJ + j) * 64 + lane];
          X[t] = mfma(fw, sb[j], X[t]);
          X[t] = mfma(fw, sl[j], X[t]);
        }
      }
      if (!SUM) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          Y[t] = zero4();
#pragma unroll
          for (int j = 0; j < NKJ; ++j) Y[t] = mfma(sb[j], sQt[(t * NKJ + j) * 64 + lane], Y[t]);
        }
      }
      f32x4 D[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) D[t] = Ut[t] - X[t];
      bf16x8 db[2], dl[2];
      split_frag(D[0], D[1], db[0], dl[0]);
      split_frag(D[2], D[3], db[1], dl[1]);
      if (!SUM) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          Y[t] = mfma(db[0], fA[t][0], Y[t]);
          if (t >= 2) Y[t] = mfma(db[1], fA[t][1], Y[t]);
          opend[ct][t] = pk4(Y[t]);
        }
      }
#pragma unroll
      for (int at = 0; at < NKT; ++at) {
        const float4 gl = *(const float4*)&sGL[16 * at + 4 * g];
        const bf16x8 fk0 = sKbar[(at * 2 + 0) * 64 + lane], fk1 = sKbar[(at * 2 + 1) * 64 + lane];
        f32x4 acc = {gl.x * S[at][ct][0], gl.y * S[at][ct][1], gl.z * S[at][ct][2], gl.w * S[at][ct][3]};
        acc = mfma(fk0, db[0], acc);
        acc = mfma(fk1, db[1], acc);
        acc = mfma(fk0, dl[0], acc);
        acc = mfma(fk1, dl[1], acc);
        S[at][ct] = acc;
      }
    }
    otok = tok_cur;
    olen = len_cur;
    // the next record has landed (the loader waited for it), and every wave is
    // done with this buffer.  The U and Aqk loads for the next chunk are not
    // waited for here: they share the memory queue with the loader's copies and
    // are waited for where they are first used.
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int t = 0; t < 4; ++t) ucur[ct][t] = unext[ct][t];
    if (!SUM) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        fA[t][0] = fAn[t][0];
        if (t >= 2) fA[t][1] = fAn[t][1];
      }
    }
    tok_cur = tok_nxt;
    len_cur = len_nxt;
  };
  for (int jc = jc0; jc < jc1; jc += 3) {
    chunk_step(jc, std::integral_constant<int, 0>{});
    if (jc + 1 < jc1) chunk_step(jc + 1, std::integral_constant<int, 1>{});
    if (jc + 2 < jc1) chunk_step(jc + 2, std::integral_constant<int, 2>{});
  }

  if (!SUM) store_out();

#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = 16 * ctg[ct] + n;
#pragma unroll
    for (int at = 0; at < NKT; ++at)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * at + 4 * g + e;
        const float sv = S[at][ct][e];
        if (!SUM) {
          if (a.fin) a.fin[sbase + (int64_t)c * V + col] = sv;
        } else if (col < V) {
          a.state_ext[sbase + (int64_t)c * V + col] = sv;
        } else {
          a.transition[((int64_t)seq * H + h) * K * K + (int64_t)c * K + (col - V)] = sv;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Kernel B2: state pass with the key dimension split across waves.
// ---------------------------------------------------------------------------
// CT column tiles per workgroup, each shared by KS compute waves: wave
// (tile, kq) holds rows [kq K/KS, (kq+1) K/KS) of that 16-column tile of the
// fp32 state, so a chunk's dependent chain of matrix products per wave is KS
// times shorter than with one wave per tile.  Per chunk:
//   1. each wave forms its partial X_kq = W[:, rows] S[rows] (S as bf16 hi + lo)
//      and puts it, and its rows of S (hi part), in LDS; barrier;
//   2. every wave of the tile sums the KS partials in the same order (so all
//      hold the same X), forms Delta = U - X (bf16 hi + lo), updates its rows
//      S[rows] <- Diag(gL) S[rows] + Kbar[:, rows]^T Delta, and computes the
//      output row tiles t = kq, kq + KS, ... as Qt S_hi + Aqk Delta_hi from
//      the exchanged S rows.
// One more wave streams W, Kbar^T and gL of each chunk into one of three LDS
// stage buffers two chunks ahead; the compute waves read U, the Aqk and the
// Qt fragments of their output rows straight into registers one chunk ahead.
template <int K, int V, int CT, int KS, bool SUM>
__global__ __launch_bounds__(64 * (CT * KS + 1)) void k_state_ks(FwdArgs a) {
  using R = Rec<K, V>;
  constexpr int CW = CT * KS;  // compute waves
  constexpr int NKJ = K / 32, NKT = K / 16, NVT = V / 16;
  constexpr int JW = NKJ / KS;  // k-steps (32 rows) per wave
  constexpr int TW = NKT / KS;  // accumulator tiles (16 rows) per wave
  constexpr int NTO = 4 / KS;   // output row tiles per wave
  static_assert(JW >= 1 && NKJ % KS == 0 && 4 % KS == 0, "key split");
  constexpr int ncols = SUM ? V + K : V;
  constexpr int nct_total = ncols / 16;
  static_assert(nct_total % CT == 0, "every workgroup owns whole column tiles");
  constexpr int ntile_wg = nct_total / CT;
  // the stage: W, Kbar^T and gL, contiguous in the record
  constexpr int kStageOff = R::oW;
  constexpr int kStageCopies = (R::kStage - kStageOff + 1023) / 1024;
  static_assert(kStageOff + kStageCopies * 1024 <= R::kBytes, "stage inside the record");
  constexpr int sW = R::oW - kStageOff, sKb = R::oKbar - kStageOff, sGLo = R::oGL - kStageOff;
  const int H = a.H;
  const int64_t bid = blockIdx.x;
  const int xcd = (int)(bid % kXcds);
  const int64_t q8 = bid / kXcds;
  const int tileg = (int)(q8 % ntile_wg);
  const int64_t nh = (q8 / ntile_wg) * kXcds + xcd;
  if (nh >= (int64_t)a.N * H) return;
  const int h = (int)(nh % H), seq = (int)(nh / H);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  constexpr int kStageBytes = kStageCopies * 1024;
  __shared__ __attribute__((aligned(16))) char sStage0[kStageBytes];
  __shared__ __attribute__((aligned(16))) char sStage1[kStageBytes];
  __shared__ __attribute__((aligned(16))) char sStage2[kStageBytes];
  // exchange: each compute wave's partial X (4 row tiles) and its S rows (hi)
  __shared__ f32x4 xX[CW][4][64];
  __shared__ bf16x8 xS[CW][JW][64];
  const int jc0 = a.seq_chunk0[seq], jc1 = a.seq_chunk0[seq + 1];
  if (!SUM && jc1 - jc0 == 1 && a.done[(int64_t)jc0 * H + h]) return;
  const char* recbase = (const char*)a.rec;

  if (w == CW) {
    // loader wave: as in k_state_mfma, but every chunk has two barriers
    static_assert(kStageCopies < 64, "wait count field");
    auto stage = [&](int jc, auto bufc) {
      constexpr int B = decltype(bufc)::value;
      char* const dst = B == 0 ? sStage0 : (B == 1 ? sStage1 : sStage2);
      const char* rec = recbase + ((int64_t)jc * H + h) * R::kBytes + kStageOff;
#pragma unroll
      for (int i = 0; i < kStageCopies; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(rec + (lane + 64 * i) * 16),
                                         (lds_void*)(&dst[(64 * i) * 16]), 16, 0, 0);
    };
    auto barrier_one_pending = [&]() { asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kStageCopies) : "memory"); };
    auto barrier_none_pending = [&]() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); };
    auto mid_barrier = [&]() { asm volatile("s_barrier" ::: "memory"); };
    auto step = [&](int jc, auto nbufc) {
      mid_barrier();
      if (jc + 2 < jc1) {
        __builtin_amdgcn_s_sleep(2);
        stage(jc + 2, nbufc);
        barrier_one_pending();
      } else {
        barrier_none_pending();
      }
    };
    if (jc0 < jc1) stage(jc0, std::integral_constant<int, 0>{});
    if (jc0 + 1 < jc1) {
      stage(jc0 + 1, std::integral_constant<int, 1>{});
      barrier_one_pending();
    } else {
      barrier_none_pending();
    }
    for (int jc = jc0; jc < jc1; jc += 3) {
      step(jc, std::integral_constant<int, 2>{});
      if (jc + 1 < jc1) step(jc + 1, std::integral_constant<int, 0>{});
      if (jc + 2 < jc1) step(jc + 2, std::integral_constant<int, 1>{});
    }
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }

  const int ct = w / KS, kq = w % KS;
  const int ctg = tileg * CT + ct;
  const int col = 16 * ctg + n;
  const bool vcol = col < V;
  const bool vt = !SUM || 16 * ctg < V;  // transition columns carry no values
  const int ut = vt ? ctg : 0;
  const int64_t sbase = ((int64_t)seq * H + h) * K * V;

  // this wave's rows of S: accumulator tiles a = kq*TW .. kq*TW+TW-1
  f32x4 S[TW];
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 16 * (kq * TW + i) + 4 * g + e;
      float sv = 0.f;
      if (!SUM && a.init && vcol) sv = a.init[sbase + (int64_t)c * V + col];
      if (SUM && !vcol) sv = (c == col - V) ? 1.f : 0.f;
      S[i][e] = sv;
    }

  // operands read straight to registers one chunk ahead: U tile, and (output
  // only) the Aqk and Qt fragments of this wave's output row tiles
  uint2 ucur[4], unext[4];
  bf16x8 aC[NTO][2], aN[NTO][2], qC[NTO][NKJ], qN[NTO][NKJ];
  auto load_ops = [&](int jc, uint2 (&u)[4], bf16x8 (&aq)[NTO][2], bf16x8 (&qt)[NTO][NKJ]) {
    const char* rec = recbase + ((int64_t)jc * H + h) * R::kBytes;
    const uint2* ug = (const uint2*)(rec + R::oU);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint2 uu = ug[(t * NVT + ut) * 64 + lane];
      u[t] = vt ? uu : make_uint2(0u, 0u);
    }
    if (!SUM) {
      const bf16x8* ga = (const bf16x8*)(rec + R::oAqk);
      const bf16x8* gq = (const bf16x8*)(rec + R::oQt);
#pragma unroll
      for (int i = 0; i < NTO; ++i) {
        const int t = kq + KS * i;
        aq[i][0] = ga[(t * 2 + 0) * 64 + lane];
        aq[i][1] = ga[(t * 2 + 1) * 64 + lane];
#pragma unroll
        for (int j = 0; j < NKJ; ++j) qt[i][j] = gq[(t * NKJ + j) * 64 + lane];
      }
    }
  };
  int tok_cur = 0, len_cur = 0, tok_nxt = 0, len_nxt = 0;
  if (jc0 < jc1) {
    load_ops(jc0, ucur, aC, qC);
    tok_cur = a.chunk_tok[jc0];
    len_cur = a.chunk_len[jc0];
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  bf16* const o = (bf16*)a.o;

  auto chunk_step = [&](int jc, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const char* const cur = BUF == 0 ? sStage0 : (BUF == 1 ? sStage1 : sStage2);
    const int jn = (jc + 1 < jc1) ? jc + 1 : jc;
    load_ops(jn, unext, aN, qN);
    tok_nxt = a.chunk_tok[jn];
    len_nxt = a.chunk_len[jn];
    const bf16x8* rW = (const bf16x8*)(cur + sW);
    const bf16x8* rKb = (const bf16x8*)(cur + sKb);
    const float* rGL = (const float*)(cur + sGLo);
    // 1. partial X over this wave's rows; S rows (hi) to the exchange
    bf16x8 sb[JW], sl[JW];
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      split_frag(S[2 * jj], S[2 * jj + 1], sb[jj], sl[jj]);
      if (!SUM) xS[w][jj][lane] = sb[jj];
    }
    f32x4 Xp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      Xp[t] = zero4();
#pragma unroll
      for (int jj = 0; jj < JW; ++jj) {
        const bf16x8 fw = rW[(t * NKJ + kq * JW + jj) * 64 + lane];
        Xp[t] = mfma(fw, sb[jj], Xp[t]);
        Xp[t] = mfma(fw, sl[jj], Xp[t]);
      }
      if (KS > 1) xX[w][t][lane] = Xp[t];
    }
    __syncthreads();
    // 2. X summed over the tile's KS waves in rank order (the same in each)
    f32x4 D[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 X = KS > 1 ? xX[ct * KS][t][lane] : Xp[t];
#pragma unroll
      for (int r = 1; r < KS; ++r) X += xX[ct * KS + r][t][lane];
      float u[4];
      unpack4(ucur[t], u);
      D[t] = f32x4{u[0], u[1], u[2], u[3]} - X;
    }
    bf16x8 db[2], dl[2];
    split_frag(D[0], D[1], db[0], dl[0]);
    split_frag(D[2], D[3], db[1], dl[1]);
    // this wave's rows of S
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      const int at = kq * TW + i;
      const float4 gl = *(const float4*)&rGL[16 * at + 4 * g];
      const bf16x8 fk0 = rKb[(at * 2 + 0) * 64 + lane], fk1 = rKb[(at * 2 + 1) * 64 + lane];
      f32x4 acc = {gl.x * S[i][0], gl.y * S[i][1], gl.z * S[i][2], gl.w * S[i][3]};
      acc = mfma(fk0, db[0], acc);
      acc = mfma(fk1, db[1], acc);
      acc = mfma(fk0, dl[0], acc);
      acc = mfma(fk1, dl[1], acc);
      S[i] = acc;
    }
    // output row tiles t = kq + KS i: Yt = (Qt S_hi)^T + (Aqk Delta_hi)^T,
    // lane (g, n) row 16t+n, columns 4g..4g+3; rows past the chunk end are
    // not stored
    if (!SUM) {
#pragma unroll
      for (int i = 0; i < NTO; ++i) {
        const int t = kq + KS * i;
        f32x4 Y = zero4();
#pragma unroll
        for (int j = 0; j < NKJ; ++j) {
          const int src = ct * KS + j / JW;  // the wave holding k-step j
          const bf16x8 sj = (j / JW == kq) ? sb[j % JW] : xS[src][j % JW][lane];
          Y = mfma(sj, qC[i][j], Y);
        }
        Y = mfma(db[0], aC[i][0], Y);
        if (t >= 2) Y = mfma(db[1], aC[i][1], Y);
        const int r = 16 * t + n;
        if (r < len_cur)
          *(uint2*)(o + ((int64_t)(tok_cur + r) * H + h) * V + 16 * ctg + 4 * g) = pk4(Y);
      }
    }
    // the next record's stage has landed and every wave is done with this
    // chunk's stage and exchange
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t) ucur[t] = unext[t];
    if (!SUM) {
#pragma unroll
      for (int i = 0; i < NTO; ++i) {
        aC[i][0] = aN[i][0];
        aC[i][1] = aN[i][1];
#pragma unroll
        for (int j = 0; j < NKJ; ++j) qC[i][j] = qN[i][j];
      }
    }
    tok_cur = tok_nxt;
    len_cur = len_nxt;
  };
  for (int jc = jc0; jc < jc1; jc += 3) {
    chunk_step(jc, std::integral_constant<int, 0>{});
    if (jc + 1 < jc1) chunk_step(jc + 1, std::integral_constant<int, 1>{});
    if (jc + 2 < jc1) chunk_step(jc + 2, std::integral_constant<int, 2>{});
  }

#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 16 * (kq * TW + i) + 4 * g + e;
      const float sv = S[i][e];
      if (!SUM) {
        if (a.fin) a.fin[sbase + (int64_t)c * V + col] = sv;
      } else if (col < V) {
        a.state_ext[sbase + (int64_t)c * V + col] = sv;
      } else {
        a.transition[((int64_t)seq * H + h) * K * K + (int64_t)c * K + (col - V)] = sv;
      }
    }
}

// ---------------------------------------------------------------------------
// Kernel B3: state pass for short sequences.
// ---------------------------------------------------------------------------
// With many sequences of a few chunks each (documents shorter than a few
// chunks), the staged pass above spends most of a workgroup's life filling its
// pipeline.  Here one workgroup of four waves takes one (sequence, head); wave
// w owns V/64 16-column tiles of the state and reads each chunk's fragments
// straight from the record into registers (no LDS, no loader wave), so many
// workgroups share a CU and hide each other's memory latency.  While the
// state is still zero (the sequence's first chunk without an initial state)
// the products with S are skipped: Delta = U, O = Aqk U, S = Kbar^T U.
template <int K, int V>
__global__ __launch_bounds__(256) void k_state_light(FwdArgs a) {
  using R = Rec<K, V>;
  constexpr int NKJ = K / 32, NKT = K / 16, NVT = V / 16;
  constexpr int NCT = NVT / 4;
  static_assert(NCT >= 1 && NVT % 4 == 0, "four waves share the value columns");
  const int H = a.H;
  const int64_t nh = blockIdx.x;
  if (nh >= (int64_t)a.N * H) return;
  const int h = (int)(nh % H), seq = (int)(nh / H);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jc0 = a.seq_chunk0[seq], jc1 = a.seq_chunk0[seq + 1];
  if (jc1 - jc0 == 1 && a.done[(int64_t)jc0 * H + h]) return;
  const int64_t sbase = ((int64_t)seq * H + h) * K * V;
  const char* recbase = (const char*)a.rec;
  bf16* const o = (bf16*)a.o;

  f32x4 S[NKT][NCT];
  bool zero = a.init == nullptr;  // S is exactly zero (wave-uniform)
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = 16 * (w * NCT + ct) + n;
#pragma unroll
    for (int at = 0; at < NKT; ++at)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S[at][ct][e] = zero ? 0.f : a.init[sbase + (int64_t)(16 * at + 4 * g + e) * V + col];
  }

  for (int jc = jc0; jc < jc1; ++jc) {
    const int tok0 = a.chunk_tok[jc], L = a.chunk_len[jc];
    const char* rec = recbase + ((int64_t)jc * H + h) * R::kBytes;
    const bf16x8* gW = (const bf16x8*)(rec + R::oW);
    const bf16x8* gQ = (const bf16x8*)(rec + R::oQt);
    const bf16x8* gK = (const bf16x8*)(rec + R::oKbar);
    const float* gG = (const float*)(rec + R::oGL);
    const bf16x8* gA = (const bf16x8*)(rec + R::oAqk);
    const uint2* gU = (const uint2*)(rec + R::oU);
    bf16x8 fA[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      fA[t][0] = gA[(t * 2 + 0) * 64 + lane];
      fA[t][1] = gA[(t * 2 + 1) * 64 + lane];
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int ctg = w * NCT + ct;
      f32x4 D[4], Y[4];
      uint2 uraw[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) uraw[t] = gU[(t * NVT + ctg) * 64 + lane];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float u[4];
        unpack4(uraw[t], u);
        D[t] = f32x4{u[0], u[1], u[2], u[3]};
        Y[t] = zero4();
      }
      if (!zero) {
        bf16x8 sb[NKJ], sl[NKJ];
#pragma unroll
        for (int j = 0; j < NKJ; ++j) split_frag(S[2 * j][ct], S[2 * j + 1][ct], sb[j], sl[j]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          f32x4 X = zero4();
#pragma unroll
          for (int j = 0; j < NKJ; ++j) {
            const bf16x8 fw = gW[(t * NKJ + j) * 64 + lane];
            X = mfma(fw, sb[j], X);
            X = mfma(fw, sl[j], X);
            Y[t] = mfma(sb[j], gQ[(t * NKJ + j) * 64 + lane], Y[t]);
          }
          D[t] -= X;
        }
      }
      bf16x8 db[2], dl[2];
      split_frag(D[0], D[1], db[0], dl[0]);
      split_frag(D[2], D[3], db[1], dl[1]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        Y[t] = mfma(db[0], fA[t][0], Y[t]);
        if (t >= 2) Y[t] = mfma(db[1], fA[t][1], Y[t]);
        const int r = 16 * t + n;
        if (r < L) *(uint2*)(o + ((int64_t)(tok0 + r) * H + h) * V + 16 * ctg + 4 * g) = pk4(Y[t]);
      }
#pragma unroll
      for (int at = 0; at < NKT; ++at) {
        const float4 gl = *(const float4*)&gG[16 * at + 4 * g];
        const bf16x8 fk0 = gK[(at * 2 + 0) * 64 + lane], fk1 = gK[(at * 2 + 1) * 64 + lane];
        f32x4 acc = zero4();
        if (!zero) acc = f32x4{gl.x * S[at][ct][0], gl.y * S[at][ct][1], gl.z * S[at][ct][2], gl.w * S[at][ct][3]};
        acc = mfma(fk0, db[0], acc);
        acc = mfma(fk1, db[1], acc);
        acc = mfma(fk0, dl[0], acc);
        acc = mfma(fk1, dl[1], acc);
        S[at][ct] = acc;
      }
    }
    zero = false;
  }

  if (a.fin) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int col = 16 * (w * NCT + ct) + n;
#pragma unroll
      for (int at = 0; at < NKT; ++at)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a.fin[sbase + (int64_t)(16 * at + 4 * g + e) * V + col] = S[at][ct][e];
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel B4: state pass with one workgroup per (sequence, head).
// ---------------------------------------------------------------------------
// V/16 waves each own one 16-column tile, so a workgroup holds whole output
// rows and can apply the gated output norm before storing them (NORM).  There
// is no separate loader wave: every wave issues its share of the next-but-one
// chunk's stage copy (Qt, W, Kbar^T, gL into one of three LDS buffers) at the
// start of a chunk and waits for its own copies at the end, so each copy has
// one chunk's time to land.  The output of chunk c is stored at the start of
// chunk c+1, after the barrier that makes every wave's per-row sum of squares
// of chunk c visible (two LDS slots, by chunk parity).
template <int K, int V, bool NORM, int ACT>
__global__ __launch_bounds__(64 * (V / 16)) void k_state_row(FwdArgs a) {
  using R = Rec<K, V>;
  constexpr int NW = V / 16;  // waves = column tiles
  constexpr int NKJ = K / 32, NKT = K / 16, NVT = V / 16;
  constexpr int kStageBytes = R::kStageCopies * 1024;
  const int H = a.H;
  const int64_t nh = blockIdx.x;
  if (nh >= (int64_t)a.N * H) return;
  const int h = (int)(nh % H), seq = (int)(nh / H);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jc0 = a.seq_chunk0[seq], jc1 = a.seq_chunk0[seq + 1];
  if (!NORM && jc1 - jc0 == 1 && a.done[(int64_t)jc0 * H + h]) return;
  __shared__ __attribute__((aligned(16))) char sStage0[kStageBytes];
  __shared__ __attribute__((aligned(16))) char sStage1[kStageBytes];
  __shared__ __attribute__((aligned(16))) char sStage2[kStageBytes];
  __shared__ float sSS[2][NW][4][16];  // per-row sums of squares, by chunk parity
  const char* recbase = (const char*)a.rec;
  const int ctg = w, col = 16 * w + n;
  const int64_t sbase = ((int64_t)seq * H + h) * K * V;

  auto stage = [&](int jc, auto bufc) {
    constexpr int B = decltype(bufc)::value;
    char* const dst = B == 0 ? sStage0 : (B == 1 ? sStage1 : sStage2);
    const char* rec = recbase + ((int64_t)jc * H + h) * R::kBytes;
    for (int i = w; i < R::kStageCopies; i += NW)
      __builtin_amdgcn_global_load_lds((const void*)(rec + (lane + 64 * i) * 16),
                                       (lds_void*)(&dst[(64 * i) * 16]), 16, 0, 0);
  };

  f32x4 S[NKT];
#pragma unroll
  for (int at = 0; at < NKT; ++at)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[at][e] = a.init ? a.init[sbase + (int64_t)(16 * at + 4 * g + e) * V + col] : 0.f;

  uint2 ucur[4], unext[4], gcur[4], gnext[4];
  bf16x8 fA[4][2], fAn[4][2];
  auto load_ops = [&](int jc, uint2 (&u)[4], bf16x8 (&aq)[4][2]) {
    const char* rec = recbase + ((int64_t)jc * H + h) * R::kBytes;
    const uint2* ug = (const uint2*)(rec + R::oU);
    const bf16x8* ga = (const bf16x8*)(rec + R::oAqk);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u[t] = ug[(t * NVT + ctg) * 64 + lane];
      aq[t][0] = ga[(t * 2 + 0) * 64 + lane];
      aq[t][1] = ga[(t * 2 + 1) * 64 + lane];
    }
  };
  // the output gate of rows 16t+n, columns 16w+4g..+3 (rows past the chunk
  // end read the chunk's first row; their results are not stored)
  auto load_gate = [&](int tok, int len, uint2 (&gg)[4]) {
    if (NORM) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 16 * t + n < len ? 16 * t + n : 0;
        gg[t] = *(const uint2*)((const bf16*)a.norm_gate + ((int64_t)(tok + r) * H + h) * V + 16 * w + 4 * g);
      }
    }
  };
  float wn[4] = {1.f, 1.f, 1.f, 1.f};
  if (NORM && a.norm_w) {
    const float4 w4 = *(const float4*)&a.norm_w[16 * w + 4 * g];
    wn[0] = w4.x; wn[1] = w4.y; wn[2] = w4.z; wn[3] = w4.w;
  }
  int tok_cur = 0, len_cur = 0;
  if (jc0 < jc1) {
    stage(jc0, std::integral_constant<int, 0>{});
    if (jc0 + 1 < jc1) stage(jc0 + 1, std::integral_constant<int, 1>{});
    load_ops(jc0, ucur, fA);
    tok_cur = a.chunk_tok[jc0];
    len_cur = a.chunk_len[jc0];
    load_gate(tok_cur, len_cur, gnext);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  uint2 opend[4];
  int otok = 0, olen = 0;
  bf16* const o = (bf16*)a.o;
  // stores chunk (otok, olen)'s output rows, normalised with the sums of
  // squares in slot par
  auto store_out = [&](int par) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = 16 * t + n;
      uint2 val = opend[t];
      if (NORM) {
        float ss = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) ss += sSS[par][ww][t][n];
        const float inv = 1.f / sqrtf(ss / V + a.norm_eps);
        float x[4], gt[4], y[4];
        unpack4(val, x);
        unpack4(gcur[t], gt);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-gt[e]));
          const float act = ACT == 0 ? sg : gt[e] * sg;
          y[e] = x[e] * inv * wn[e] * act;
        }
        val = pk4(y[0], y[1], y[2], y[3]);
      }
      if (r < olen) *(uint2*)(o + ((int64_t)(otok + r) * H + h) * V + 16 * w + 4 * g) = val;
    }
  };

  auto chunk_step = [&](int jc, auto bufc, auto nbufc) {
    constexpr int BUF = decltype(bufc)::value;
    const char* const cur = BUF == 0 ? sStage0 : (BUF == 1 ? sStage1 : sStage2);
    if (jc + 2 < jc1) stage(jc + 2, nbufc);
    const int jn = (jc + 1 < jc1) ? jc + 1 : jc;
    load_ops(jn, unext, fAn);
    const int tok_n = a.chunk_tok[jn], len_n = a.chunk_len[jn];
    // the previous chunk's output (its gate values are in gcur); then gcur
    // takes this chunk's gate values and gnext starts loading the next's
    if (jc > jc0) store_out((jc - 1 - jc0) & 1);
    if (NORM) {
#pragma unroll
      for (int t = 0; t < 4; ++t) gcur[t] = gnext[t];
    }
    load_gate(tok_n, len_n, gnext);
    const bf16x8* sQt = (const bf16x8*)(cur + R::oQt);
    const bf16x8* sW = (const bf16x8*)(cur + R::oW);
    const bf16x8* sKbar = (const bf16x8*)(cur + R::oKbar);
    const float* sGL = (const float*)(cur + R::oGL);
    f32x4 Ut[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float u[4];
      unpack4(ucur[t], u);
      Ut[t] = f32x4{u[0], u[1], u[2], u[3]};
    }
    bf16x8 sb[NKJ], sl[NKJ];
#pragma unroll
    for (int j = 0; j < NKJ; ++j) split_frag(S[2 * j], S[2 * j + 1], sb[j], sl[j]);
    f32x4 X[4], Y[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      X[t] = zero4();
#pragma unroll
      for (int j = 0; j < NKJ; ++j) {
        const bf16x8 fw = sW[(t * NKJ + j) * 64 + lane];
        X[t] = mfma(fw, sb[j], X[t]);
        X[t] = mfma(fw, sl[j], X[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      Y[t] = zero4();
#pragma unroll
      for (int j = 0; j < NKJ; ++j) Y[t] = mfma(sb[j], sQt[(t * NKJ + j) * 64 + lane], Y[t]);
    }
    f32x4 D[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) D[t] = Ut[t] - X[t];
    bf16x8 db[2], dl[2];
    split_frag(D[0], D[1], db[0], dl[0]);
    split_frag(D[2], D[3], db[1], dl[1]);
    const int par = (jc - jc0) & 1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      Y[t] = mfma(db[0], fA[t][0], Y[t]);
      if (t >= 2) Y[t] = mfma(db[1], fA[t][1], Y[t]);
      opend[t] = pk4(Y[t]);
      if (NORM) {
        // this wave's 16 columns of row 16t+n, as the stored (rounded) values
        float x[4];
        unpack4(opend[t], x);
        float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        if (g == 0) sSS[par][w][t][n] = ss;
      }
    }
#pragma unroll
    for (int at = 0; at < NKT; ++at) {
      const float4 gl = *(const float4*)&sGL[16 * at + 4 * g];
      const bf16x8 fk0 = sKbar[(at * 2 + 0) * 64 + lane], fk1 = sKbar[(at * 2 + 1) * 64 + lane];
      f32x4 acc = {gl.x * S[at][0], gl.y * S[at][1], gl.z * S[at][2], gl.w * S[at][3]};
      acc = mfma(fk0, db[0], acc);
      acc = mfma(fk1, db[1], acc);
      acc = mfma(fk0, dl[0], acc);
      acc = mfma(fk1, dl[1], acc);
      S[at] = acc;
    }
    otok = tok_cur;
    olen = len_cur;
    // this wave's stage copies for chunk c+1 (issued a chunk ago) and its
    // prefetched operands have landed; after the barrier every wave's copies
    // have, and every wave is done with this chunk's buffer
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      ucur[t] = unext[t];
      fA[t][0] = fAn[t][0];
      fA[t][1] = fAn[t][1];
    }
    tok_cur = tok_n;
    len_cur = len_n;
  };
  for (int jc = jc0; jc < jc1; jc += 3) {
    chunk_step(jc, std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{});
    if (jc + 1 < jc1) chunk_step(jc + 1, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
    if (jc + 2 < jc1) chunk_step(jc + 2, std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{});
  }
  if (jc1 > jc0) store_out((jc1 - 1 - jc0) & 1);
  if (a.fin) {
#pragma unroll
    for (int at = 0; at < NKT; ++at)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        a.fin[sbase + (int64_t)(16 * at + 4 * g + e) * V + col] = S[at][e];
  }
}

// compute units of the current device (cached per device)
inline int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

template <int K, int V>
hipError_t run(const FwdArgs& a, hipStream_t s) {
  mark(a, kStagePrologue, 0, s);
  mark(a, kStagePrologue, 1, s);
  mark(a, kStageChunk, 0, s);
  if (a.NT > 0) {
    const dim3 grid((unsigned)((int64_t)a.NT * a.H)), block(kThreads);
    // chunk-heads whose in-block decay left the factorised range go to a fix-up
    // pass (rare; its grid is fixed and exits at once when the list is empty)
    const dim3 fix_grid((unsigned)std::min<int64_t>((int64_t)a.NT * a.H, 256));
    auto launch_gate = [&](auto gc, auto cc) {
      constexpr int GATE = decltype(gc)::value;
      constexpr bool CONV = decltype(cc)::value;
      hipLaunchKernelGGL((k_chunk_mfma<K, V, GATE, CONV>), grid, block, 0, s, a);
      hipLaunchKernelGGL((k_chunk_mfma_exact<K, V, GATE, CONV>), fix_grid, block, 0, s, a);
    };
    auto launch_conv = [&](auto gc) {
      if (a.conv) launch_gate(gc, std::true_type{});
      else launch_gate(gc, std::false_type{});
    };
    if (a.gate_form == 1) launch_conv(std::integral_constant<int, 1>{});
    else if (a.gate_form == 2) launch_conv(std::integral_constant<int, 2>{});
    else launch_conv(std::integral_constant<int, 0>{});
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  mark(a, kStageChunk, 1, s);
  mark(a, kStageState, 0, s);
  // one 16-column tile per compute wave; the widest workgroup (most compute
  // waves) that still gives every CU a workgroup
  const int ncols = a.summary ? V + K : V;
  const int64_t heads = ((int64_t)a.N * a.H + kXcds - 1) / kXcds * kXcds;
  const int cus = device_cus();
  int cw = 4;
  while (cw > 1 && heads * (ncols / 16 / cw) < cus) cw /= 2;
  int64_t wgs = heads * (ncols / 16 / cw);
  // whole output rows per workgroup: needed by the fused output norm
  bool rowk = a.norm != 0;
  if (const char* env = std::getenv("KDA_STATE_ROW")) rowk = rowk || std::atoi(env) != 0;
  if (rowk && !a.summary) {
    const int64_t nwg = (int64_t)a.N * a.H;
    if (nwg > 0) {
      const dim3 grid((unsigned)nwg), block(64 * (V / 16));
      if (!a.norm) hipLaunchKernelGGL((k_state_row<K, V, false, 0>), grid, block, 0, s, a);
      else if (a.norm_act == 0) hipLaunchKernelGGL((k_state_row<K, V, true, 0>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_state_row<K, V, true, 1>), grid, block, 0, s, a);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    mark(a, kStageState, 1, s);
    return hipSuccess;
  }
  // many short sequences (at most four chunks each on average): the light pass
  bool light = !a.summary && (int64_t)a.NT <= 4 * (int64_t)a.N;
  if (const char* env = std::getenv("KDA_STATE_LIGHT")) light = !a.summary && std::atoi(env) != 0;
  if (light) {
    const int64_t nwg = (int64_t)a.N * a.H;
    if (nwg > 0) {
      hipLaunchKernelGGL((k_state_light<K, V>), dim3((unsigned)nwg), dim3(256), 0, s, a);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    mark(a, kStageState, 1, s);
    return hipSuccess;
  }
  // key split: when even one 16-column tile per workgroup leaves CUs idle,
  // the chains are few and long and each chunk's latency bounds the pass;
  // then KS waves share each tile's rows
  int ks = (cw == 1 && heads * (ncols / 16) <= cus && K == 128) ? 4 : 1;
  if (const char* env = std::getenv("KDA_STATE_KS")) ks = std::atoi(env);
  if (ks != 1 && ks != 2 && ks != 4) ks = 1;
  if (K == 64 && ks == 4) ks = 2;
  if (ks > 1 && wgs > 0 && (a.summary || a.fin || a.NT > 0)) {
    wgs = heads * (ncols / 16);
    const dim3 grid((unsigned)wgs), block(64 * (ks + 1));
    auto launch_ks = [&](auto ksc) {
      constexpr int KSc = decltype(ksc)::value;
      if (a.summary) hipLaunchKernelGGL((k_state_ks<K, V, 1, KSc, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_state_ks<K, V, 1, KSc, false>), grid, block, 0, s, a);
    };
    if (ks == 4) launch_ks(std::integral_constant<int, (K == 128 ? 4 : 2)>{});
    else launch_ks(std::integral_constant<int, 2>{});
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  } else if (wgs > 0 && (a.summary || a.fin || a.NT > 0)) {
    const dim3 grid((unsigned)wgs), block(64 * (cw + 1));
    auto launch_cw = [&](auto cwc) {
      constexpr int CW = decltype(cwc)::value;
      if (a.summary) hipLaunchKernelGGL((k_state_mfma<K, V, CW, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_state_mfma<K, V, CW, false>), grid, block, 0, s, a);
    };
    if (cw == 4) launch_cw(std::integral_constant<int, 4>{});
    else if (cw == 2) launch_cw(std::integral_constant<int, 2>{});
    else launch_cw(std::integral_constant<int, 1>{});
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  mark(a, kStageState, 1, s);
  return hipSuccess;
}

template <int K, int V>
hipError_t run_fused(const FwdArgs& a, hipStream_t s) {
  // the chunk factors are folded into the fused kernel: their stage's events
  // are recorded back to back
  mark(a, kStagePrologue, 0, s);
  mark(a, kStagePrologue, 1, s);
  mark(a, kStageChunk, 0, s);
  mark(a, kStageChunk, 1, s);
  mark(a, kStageState, 0, s);
  const int64_t wgs = (int64_t)a.N * a.H;
  if (wgs > 0) {
    const dim3 grid((unsigned)wgs), block(kThreads);
    auto launch_gate = [&](auto gc) {
      constexpr int GATE = decltype(gc)::value;
      if (a.conv) hipLaunchKernelGGL((k_fused<K, V, GATE, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_fused<K, V, GATE, false>), grid, block, 0, s, a);
    };
    if (a.gate_form == 1) launch_gate(std::integral_constant<int, 1>{});
    else if (a.gate_form == 2) launch_gate(std::integral_constant<int, 2>{});
    else launch_gate(std::integral_constant<int, 0>{});
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  mark(a, kStageState, 1, s);
  return hipSuccess;
}

}  // namespace

hipError_t launch_fused_path(const FwdArgs& a, hipStream_t s) {
  if (a.K == 128 && a.V == 128) return run_fused<128, 128>(a, s);
  if (a.K == 128 && a.V == 64) return run_fused<128, 64>(a, s);
  if (a.K == 64 && a.V == 128) return run_fused<64, 128>(a, s);
  return run_fused<64, 64>(a, s);
}

namespace {
template <int K, int V>
hipError_t run_recompute(const FwdArgs& a, hipStream_t s) {
  if (a.NT == 0) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)a.NT * a.H)), block(kThreads);
  const dim3 fix_grid((unsigned)std::min<int64_t>((int64_t)a.NT * a.H, 256));
  auto launch_gate = [&](auto gc) {
    constexpr int GATE = decltype(gc)::value;
    hipLaunchKernelGGL((k_chunk_recompute<K, V, GATE>), grid, block, 0, s, a);
    hipLaunchKernelGGL((k_chunk_recompute_exact<K, V, GATE>), fix_grid, block, 0, s, a);
  };
  if (a.gate_form == 1) launch_gate(std::integral_constant<int, 1>{});
  else if (a.gate_form == 2) launch_gate(std::integral_constant<int, 2>{});
  else launch_gate(std::integral_constant<int, 0>{});
  return hipGetLastError() == hipSuccess ? hipSuccess : hipErrorLaunchFailure;
}
}  // namespace

hipError_t launch_mfma_recompute(const FwdArgs& a, hipStream_t s) {
  if (a.K == 128 && a.V == 128) return run_recompute<128, 128>(a, s);
  if (a.K == 128 && a.V == 64) return run_recompute<128, 64>(a, s);
  if (a.K == 64 && a.V == 128) return run_recompute<64, 128>(a, s);
  return run_recompute<64, 64>(a, s);
}

size_t mfma_record_bytes(int K, int V) {
  if (K == 128 && V == 128) return Rec<128, 128>::kBytes;
  if (K == 128 && V == 64) return Rec<128, 64>::kBytes;
  if (K == 64 && V == 128) return Rec<64, 128>::kBytes;
  return Rec<64, 64>::kBytes;
}

hipError_t launch_mfma_path(const FwdArgs& a, hipStream_t s) {
  if (a.K == 128 && a.V == 128) return run<128, 128>(a, s);
  if (a.K == 128 && a.V == 64) return run<128, 64>(a, s);
  if (a.K == 64 && a.V == 128) return run<64, 128>(a, s);
  return run<64, 64>(a, s);
}

}  // namespace kda
