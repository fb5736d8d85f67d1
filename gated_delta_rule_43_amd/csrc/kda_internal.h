// Internal declarations shared by the host orchestration (kda_api.cpp) and the
// HIP kernels of libkda.so.  Not part of the public ABI (include/kda.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// ---------------------------------------------------------------------------
// bf16 stored as raw 16-bit patterns; conversions round to nearest even.
// ---------------------------------------------------------------------------
typedef uint16_t bf16;

__host__ __device__ inline float bf16_to_f32(bf16 x) {
  union { uint32_t u; float f; } c;
  c.u = ((uint32_t)x) << 16;
  return c.f;
}

__host__ __device__ inline bf16 f32_to_bf16(float f) {
  union { uint32_t u; float f; } c;
  c.f = f;
  if ((c.u & 0x7f800000u) == 0x7f800000u && (c.u & 0x007fffffu)) return (bf16)((c.u >> 16) | 0x40);
  uint32_t r = c.u + 0x7fffu + ((c.u >> 16) & 1u);
  return (bf16)(r >> 16);
}

__device__ inline float load_f32(const float* p) { return *p; }
__device__ inline float load_f32(const bf16* p) { return bf16_to_f32(*p); }
__device__ inline void store_as(float* p, float x) { *p = x; }
__device__ inline void store_as(bf16* p, float x) { *p = f32_to_bf16(x); }

// ---------------------------------------------------------------------------
// Everything one forward / summary call needs, resolved on the host.
// ---------------------------------------------------------------------------
struct FwdArgs {
  // shapes: H value heads (every per-head tensor but q, k), HK key heads of
  // q and k; value head h reads key head h / (H / HK)
  int B, T, H, K, V, C, N;
  int HK;
  int NT;          // chunk count: exact, or an upper bound when exact_nt == 0
  int exact_nt;
  int dtype;       // 0 fp32, 1 bf16
  float scale;
  int gate_form;   // 0: -A softplus(x); 1: lb sigmoid(A x); 2: max(lb, -A softplus(x))
  float lb;
  // inputs
  const int32_t* cu;  // device cu_seqlens or nullptr
  const void *q, *k, *v, *gate, *beta;
  const float *a_log, *dt_bias, *init;
  // outputs
  void* o;
  float* fin;
  float* state_ext;   // summary mode
  float* transition;  // summary mode
  int summary;
  // workspace: chunk table
  int32_t* chunk_tok;  // [NT] flat token index b*T + t of the chunk's first token
  int32_t* chunk_len;  // [NT] tokens in the chunk (1..C)
  int32_t* seq_chunk0; // [N+1] first chunk of each sequence
  int32_t* nt_dev;     // [1] actual number of chunks
  int32_t* chunk_seq;  // [NT] sequence (row or document) of each chunk
  // workspace: per-token prologue results (VALU path)
  float *qn, *kn, *g, *bt;
  // backward: the L2 norm's scales 1/||q||, 1/||k|| of each value-head
  // token-head (q^ = q rq), written by the recomputation
  float *rq, *rk;
  // workspace: per chunk-head factors, fp32; with ws_bf16 set, W, U, Qt, Kb,
  // Aqk and Akk_out are bf16 (the backward's matrix-core recomputation,
  // 64-token chunks), U then as 16 x 16 accumulator tiles
  // ([C/16][V/16][64 lanes][4]: lane l holds rows 4 (l / 16) .. + 3 of column
  // l % 16 of its tile)
  int ws_bf16;
  void *W, *U, *Qt, *Kb, *Aqk;
  float* gL;
  // backward only: Akk (strictly lower) and Tm per chunk-head, [C*C] each
  float* Akk_out;
  float* Tm_out;
  // workspace: per chunk-head records of the MFMA path, and a small sink for
  // the state pass's masked-off output stores
  void* rec;
  void* sink;
  int32_t* exact_count;  // [1] chunk-heads listed for the exact fix-up pass
  int32_t* exact_list;   // [NT*H]
  // [NT*H] written by the chunk-factor kernel for every chunk-head: 1 when it
  // finished the chunk's sequence itself (a one-chunk sequence), 0 otherwise
  int32_t* done;
  // optional gated output norm fused into the output store (norm != 0): o then
  // receives y = o / sqrt(mean_V(o^2) + eps) * weight * act(gate_o) per
  // (token, value head) row, o rounded to the input dtype first
  int norm;
  int norm_act;          // 0 sigmoid, 1 SiLU
  float norm_eps;
  const void* norm_gate; // [B,T,H,V], dtype as q
  const float* norm_w;   // [V] or null for ones
  // optional short convolution of width 4 + SiLU of q, k and v applied as the
  // matrix-core kernels load them (conv != 0; q, k, v are then the raw
  // projections): weights [C, 4] fp32 (tap 3 weights the current token),
  // biases [C] fp32 or null; C = HK*K for q and k, H*V for v.  Each convolved
  // value is rounded to the input dtype, as the standalone convolution stores it.
  int conv;
  const float *conv_wq, *conv_wk, *conv_wv, *conv_bq, *conv_bk, *conv_bv;
  // optional stage timing: hipEvent_t handles, [2 * kNumStages], entries may be null
  void* const* events;
};

// One short-convolution launch over up to three tensors x -> y ([B*T, C],
// dtype as FwdArgs::dtype); weights [C, width] fp32, bias [C] fp32 or null.
struct ConvTensor {
  const void* x;
  const float* w;
  const float* bias;
  void* y;
  int C;
};
struct ConvArgs {
  int B, T, N;
  int dtype;   // 0 fp32, 1 bf16
  int width;   // taps, 0..4 (0: SiLU alone)
  int count;   // tensors in t[]
  const int32_t* cu;  // device cu_seqlens or nullptr
  ConvTensor t[3];
};

// The backward: the forward's VALU workspace (FwdArgs, with Akk_out/Tm_out
// set) plus per-chunk states and their gradients, and the gradient outputs.
struct BwdArgs {
  FwdArgs f;
  // inputs
  const void* d_o;       // [B,T,H,V], dtype as f.dtype
  const float* d_fin;    // [N,H,K,V] or nullptr
  // workspace
  float *hc, *dhc;       // [NT*H][K*V] state entering each chunk, gradient of the state leaving it
  float *Dc, *dDc;       // [NT*H][C*V] Delta and its gradient
  float *dqh, *dkh;      // [B*T*H][K] gradient of q^, k^ per value head
  float *da_part;        // [NT*H]
  float *ddt_part;       // [NT*H][K]
  // outputs
  void *dq, *dk, *dv, *dgate, *dbeta;  // dtype as f.dtype
  float *da_log, *ddt_bias, *dinit;    // fp32; dinit may be nullptr
  void* const* events;  // 2 * kNumBwdStages hipEvent_t or nullptr (kda_bwd_profiled)
};

// The gated output norm over rows of V values (o, gate, y: dtype; w: fp32 [V] or null).
struct NormArgs {
  int64_t rows;
  int V;
  int dtype;   // 0 fp32, 1 bf16
  int act;     // 0 sigmoid, 1 SiLU
  float eps;
  const void* o;
  const void* gate;
  const float* w;
  void* y;
};

// Stages of one forward, in launch order (timing hooks of kda_fwd_profiled).
enum Stage { kStageTable = 0, kStagePrologue = 1, kStageChunk = 2, kStageState = 3, kNumStages = 4 };

inline void mark(const FwdArgs& a, int stage, int end, hipStream_t s) {
  if (a.events && a.events[2 * stage + end]) hipEventRecord((hipEvent_t)a.events[2 * stage + end], s);
}

// Stages of one backward, in launch order (timing hooks of kda_bwd_profiled).
enum BwdStage {
  kBwdTable = 0, kBwdRecompute = 1, kBwdFState = 2, kBwdDState = 3, kBwdChunk = 4,
  kBwdQK = 5, kBwdParams = 6, kNumBwdStages = 7
};

inline void bmark(const BwdArgs& b, int stage, int end, hipStream_t s) {
  if (b.events && b.events[2 * stage + end]) hipEventRecord((hipEvent_t)b.events[2 * stage + end], s);
}

// Kernel launchers (return the first HIP error, hipSuccess otherwise).
hipError_t launch_chunk_table(const FwdArgs& a, hipStream_t s);
hipError_t launch_valu_path(const FwdArgs& a, hipStream_t s);
hipError_t launch_valu_prep(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s);
hipError_t launch_mfma_path(const FwdArgs& a, hipStream_t s);
// The backward's recomputation of the chunk factors for bf16 inputs on the
// matrix-core chunk kernel, into the fp32 arrays that launch_valu_prep fills
// (needs exact_count and exact_list for its fix-up pass).
hipError_t launch_mfma_recompute(const FwdArgs& a, hipStream_t s);
hipError_t launch_fused_path(const FwdArgs& a, hipStream_t s);
hipError_t launch_short_conv(const ConvArgs& a, hipStream_t s);
hipError_t launch_gated_rms_norm(const NormArgs& a, hipStream_t s);
size_t mfma_record_bytes(int K, int V);
hipError_t launch_apply_summary(int B, int H, int K, int V, const float* E, const float* P,
                                const float* S0, float* F, hipStream_t s);

}  // namespace kda
