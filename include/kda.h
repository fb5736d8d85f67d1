/*
 * kda.h -- C ABI of the KDA (Kimi Delta Attention) chunked forward for AMD
 * MI355X (gfx950).  Library: libkda.so.
 *
 * KDA is a gated delta-rule linear attention with a per-key-channel decay.
 * Per sequence n and value head h the recurrent state S is a K x V fp32 matrix
 * (row = key channel, column = value channel) and, token by token,
 *
 *     q^ = q / sqrt(sum q^2 + 1e-6),     k^ likewise            (in-kernel L2 norm)
 *     x_c = gate_c + dt_bias[h,c],       A = exp(a_log[h])
 *     g_c = -A * softplus(x_c)                 when lower_bound is unset
 *     g_c = lower_bound * sigmoid(A * x_c)     when lower_bound < 0 (safe gate)
 *     g_c = max(lower_bound, -A * softplus(x_c))   the same, with lower_bound_form
 *                                                  = KDA_LB_CLAMP
 *     beta = sigmoid(beta_logit)                                  (in-kernel sigmoid)
 *     S_t = (I - beta k^ k^T) Diag(exp g) S_{t-1} + beta k^ v^T
 *     o_t = scale * S_t^T q^
 *
 * The entry points mirror the chunk_kda call and the affine state-summary pair
 * on the hyper_parallel coverage page for
 * context_parallel/kimi_delta_attention.py (`_run_local_kda`,
 * `_eager_kda_state_p2p`, `_validate_projected_inputs`), and take document
 * boundaries as cu_seqlens like the NeMo AutoModel page
 * "nemo_automodel.components.models.kimi_k3.cp" (module introduction,
 * `doc_ids_from_cu_seqlens`).  The gate formula is not printed on the pages;
 * the forms above are this library's reading of the in-kernel gate and of the
 * lower-bounded gate parameterisation (sigmoid by default; the hard clamp is
 * the alternative reading, selected per call).
 *
 * Conventions for every entry point
 *  - All tensors are dense, contiguous, token-major ("token-first"), with H key
 *    heads and HV value heads (HV a multiple of H; HV = H without grouping):
 *      q, k   : [B, T, H, K]       gate : [B, T, HV, K]     beta : [B, T, HV]
 *      v, o   : [B, T, HV, V]      a_log : [HV] fp32        dt_bias : [HV, K] fp32
 *      states : [N, HV, K, V] fp32      transitions : [B, HV, K, K] fp32
 *    Value head h reads key head h / (HV / H) (grouped value heads, the shape
 *    contract of `_validate_projected_inputs`).  q, k, v, gate, beta and o
 *    share one dtype (kda_dtype).
 *  - Every tensor pointer is a device pointer unless its name ends in _host.
 *  - The caller owns and allocates all memory, including the workspace.  The
 *    library allocates nothing, keeps no state between calls, never frees and
 *    never synchronises the stream.  Kernels are enqueued on `stream`
 *    (a hipStream_t; NULL = the default stream) and may still be running when
 *    the call returns.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    non-OK status nothing was launched and kda_last_error() describes why.
 *  - Not thread-safe across concurrent calls that share a workspace.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Form of the lower-bounded gate (used only when lower_bound is set). */
typedef enum { KDA_LB_SIGMOID = 0, KDA_LB_CLAMP = 1 } kda_lower_bound_form;

typedef enum {
  KDA_OK = 0,
  KDA_EINVAL = 1,        /* malformed argument (null pointer, bad shape, bad cu_seqlens, ...) */
  KDA_EUNSUPPORTED = 2,  /* well-formed but outside what this build implements          */
  KDA_EWORKSPACE = 3,    /* workspace missing or smaller than *_workspace_size()        */
  KDA_EHIP = 4           /* a HIP launch failed                                          */
} kda_status;

/*
 * One problem description, shared by kda_fwd and kda_state_summary.
 *
 *  B, T, H, K, V  shapes above.  T >= 0, B >= 1, H >= 1; K and V in {64, 128}.
 *  dtype          element type of q, k, v, gate, beta and o.
 *  scale          output scale; any value that is not > 0 (0, negative, NaN)
 *                 selects the default 1/sqrt(K) ("scale=None" of chunk_kda).
 *  lower_bound    NaN = unset (softplus gate); otherwise it must be < 0
 *                 ("lower_bound must be negative", KimiDeltaAttentionUlyssesCP
 *                 constructor on the hyper_parallel page).
 *  chunk_size     tokens per chunk: 16, 32 or 64 (default of the pages: 64).
 *                 <= 0 is KDA_EINVAL ("chunk_size must be positive"); other
 *                 positive values are KDA_EUNSUPPORTED.  The result does not
 *                 depend on it beyond rounding.
 *  cu_seqlens     NULL: every row b is one sequence (N = B).  Otherwise B must
 *                 be 1 and it holds N+1 int32 offsets into the row with
 *                 cu[0] = 0, cu[N] = T, non-decreasing (empty documents are
 *                 allowed); the state restarts at every document start.
 *                 Device pointer.
 *  cu_seqlens_host  optional host copy of the same N+1 offsets.  When given,
 *                 the offsets are validated (KDA_EINVAL on a violation,
 *                 including the negative padding sentinels some packers use)
 *                 and the launch is sized exactly.  When NULL the caller
 *                 guarantees validity; malformed device offsets are clamped
 *                 into range on the device so that no access leaves the
 *                 buffers, and the results are then unspecified.
 *  N              number of sequences: B without cu_seqlens, else len-1.
 *  lower_bound_form  KDA_LB_SIGMOID (0, default) or KDA_LB_CLAMP (1); with
 *                 KDA_LB_CLAMP lower_bound must be set.  Other values and a
 *                 clamp without a bound are KDA_EINVAL.
 *  HV             value heads; 0 means HV = H.  Otherwise a positive multiple
 *                 of H (KDA_EINVAL if not).
 * Fields are appended at the end only: a zero-initialised problem with the
 * first ten fields set describes the ungrouped, sigmoid-form problem.
 */
typedef struct kda_problem {
  int32_t B, T, H, K, V;
  int32_t dtype;
  float scale;
  float lower_bound;
  int32_t chunk_size;
  int32_t N;
  const int32_t* cu_seqlens;
  const int32_t* cu_seqlens_host;
  int32_t lower_bound_form;
  int32_t HV;
} kda_problem;

/* Host-only validation of a problem; launches nothing, touches no device. */
kda_status kda_validate(const kda_problem* p);

/* Bytes of device workspace kda_fwd needs for this problem (0 on a bad problem,
 * with the status in *status when status is not NULL).  The size depends only
 * on the shapes, dtype, chunk_size and, without a host copy of cu_seqlens, on
 * N through an upper bound of the chunk count. */
size_t kda_fwd_workspace_size(const kda_problem* p, kda_status* status);

/*
 * Chunked KDA forward (the chunk_kda call of `_run_local_kda` /
 * `_eager_kda_state_p2p` with use_qk_l2norm_in_kernel, use_gate_in_kernel and
 * use_beta_sigmoid_in_kernel all on).
 *
 *  q, k, v, gate, beta   inputs, dtype p->dtype, layouts above.
 *  a_log [HV], dt_bias [HV,K]   fp32 gate parameters.
 *  initial_state         [N,HV,K,V] fp32, or NULL for zeros.
 *  o                     [B,T,HV,V] output, dtype p->dtype (required).
 *  final_state           [N,HV,K,V] fp32 output, or NULL to not produce it
 *                        (output_final_state=False).  With cu_seqlens, entry n
 *                        is document n's state after its last token; an empty
 *                        document returns its initial state.
 *  workspace             device buffer of at least kda_fwd_workspace_size()
 *                        bytes, 256-byte aligned; contents need not be cleared.
 * Returns KDA_OK once every kernel is enqueued on `stream`.
 */
kda_status kda_fwd(const kda_problem* p, const void* q, const void* k, const void* v,
                   const void* gate, const void* beta, const float* a_log,
                   const float* dt_bias, const float* initial_state, void* o,
                   float* final_state, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Which kernels kda_fwd runs for this problem (host only, launches nothing):
 *   KDA_PATH_VALU   fp32 inputs: vector-ALU kernels;
 *   KDA_PATH_MFMA   bf16: all chunk-heads' factors in parallel into
 *                   workspace records, then the sequential state pass;
 *   KDA_PATH_FUSED  bf16: one workgroup per (sequence, head) that
 *                   computes and consumes each chunk's factors in on-chip
 *                   memory (no records in the workspace).
 * Both matrix-core paths compute the same algebra; their results agree to
 * rounding.  Their tiles hold 64 rows: a chunk of 16 or 32 tokens fills the
 * first rows and the rest is masked as past a sequence's end, so the tile
 * computes that chunk size's algebra (with the masked rows' products wasted).  Returns -1 (message in kda_last_error) for an invalid problem.
 */
#define KDA_PATH_VALU 0
#define KDA_PATH_MFMA 1
#define KDA_PATH_FUSED 2
int32_t kda_fwd_path(const kda_problem* p);

/*
 * kda_fwd with per-stage timing hooks, for measurement.  It does exactly the
 * work of kda_fwd; in addition, when stage_events is not NULL it must hold
 * 2 * KDA_NUM_STAGES hipEvent_t handles created by the caller (entries may be
 * NULL), and the library records stage_events[2*i] on `stream` just before
 * stage i is enqueued and stage_events[2*i+1] just after.  Stages, in order:
 *   0 chunk table, 1 per-token prologue, 2 chunk-local factors,
 *   3 state pass and output.
 * A stage that the chosen kernels fold into another records both events back
 * to back.
 */
#define KDA_NUM_STAGES 4
kda_status kda_fwd_profiled(const kda_problem* p, const void* q, const void* k, const void* v,
                            const void* gate, const void* beta, const float* a_log,
                            const float* dt_bias, const float* initial_state, void* o,
                            float* final_state, void* workspace, size_t workspace_bytes,
                            void* stream, void* const* stage_events);

/*
 * kda_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results as kda_fwd, without the workspace: the library uses a
 * device array of kda_fwd_noalloc_scratch_bytes() (64 MiB) that it holds on
 * every GPU it runs on until the process ends.  The entry point calls no
 * hipMalloc, hipFree or other allocating routine.
 *  - It runs kda_fwd's kernels: the path kda_fwd_path reports when that path's
 *    workspace fits the array, otherwise the fused path (which needs only the
 *    chunk table, about 8 bytes per chunk).  Problems whose workspace still
 *    exceeds the array return KDA_EWORKSPACE.
 *  - The stream must belong to the current device (KDA_EINVAL otherwise).
 *  - Every call on one GPU shares that GPU's array: calls that overlap on one
 *    GPU (concurrent streams, or threads) race and give undefined results.
 *    Calls in one stream order are safe; each call rewrites what it reads.
 */
size_t kda_fwd_noalloc_scratch_bytes(void);
kda_status kda_fwd_noalloc(const kda_problem* p, const void* q, const void* k, const void* v,
                           const void* gate, const void* beta, const float* a_log,
                           const float* dt_bias, const float* initial_state, void* o,
                           float* final_state, void* stream);

/* Workspace bytes for kda_state_summary. */
size_t kda_state_summary_workspace_size(const kda_problem* p, kda_status* status);

/*
 * Affine summary of each row as a contiguous slice (torch_kda_state_summary in
 * `_eager_kda_state_p2p` on the hyper_parallel page): the row's effect on the
 * state is  final = transition . initial + state_ext,  with
 *  state_ext  [B,HV,K,V] fp32 = the row's final state from a zero initial state,
 *  transition [B,HV,K,K] fp32 = the ordered product over the row's tokens of
 *             (I - beta k^ k^T) Diag(exp g), later tokens on the left.
 * p->cu_seqlens must be NULL (a slice summary has no document resets; the
 * pages' state-CP adapters reject cu_seqlens as well).  No output o is made.
 */
kda_status kda_state_summary(const kda_problem* p, const void* q, const void* k, const void* v,
                             const void* gate, const void* beta, const float* a_log,
                             const float* dt_bias, float* state_ext, float* transition,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * final_state = transition . initial_state + state_ext for each of the B*H
 * (row, head) pairs (H = the value heads of the summary) (torch_apply_kda_state_summary on the hyper_parallel
 * page); initial_state may be NULL (rank 0 of a state-parallel chain), then
 * final_state = state_ext.  All fp32, shapes [B,H,K,V] and [B,H,K,K].
 * final_state may alias state_ext (in-place update); it may not alias
 * transition or initial_state.
 */
kda_status kda_apply_state_summary(int32_t B, int32_t H, int32_t K, int32_t V,
                                   const float* state_ext, const float* transition,
                                   const float* initial_state, float* final_state, void* stream);

/*
 * The chunk table kda_fwd builds on the device, written into caller buffers so
 * that it can be inspected.  Every sequence is cut into chunks of chunk_size
 * tokens starting at the sequence's own first token (so the last chunk of a
 * document may be partial and the next document starts a new chunk):
 *  tok        [cap] flat token index (b*T + t) of each chunk's first token
 *  len        [cap] tokens in each chunk (1..chunk_size)
 *  seq_chunk0 [N+1] index of each sequence's first chunk; seq_chunk0[N] = count
 *  count      [1]   number of chunks
 * cap must be at least kda_chunk_capacity(p).  Device pointers.
 */
int32_t kda_chunk_capacity(const kda_problem* p, kda_status* status);
kda_status kda_chunk_table(const kda_problem* p, int32_t* tok, int32_t* len, int32_t* seq_chunk0,
                           int32_t* count, int32_t cap, void* stream);

/*
 * Gradients of the forward: for L = sum(d_o * o) + sum(d_final_state *
 * final_state), with o and final_state what kda_fwd returns for the same
 * problem and inputs, the gradient of L with respect to every input, through
 * the in-kernel L2 norm, gate and beta sigmoid (the chunk_kda call that the
 * torchtitan PR #4025 commit note tests forward and backward together; the
 * hyper_parallel page routes the state gradient between slices in the
 * backward of `_RecvKDAInitialState`).
 *
 *  q .. dt_bias, initial_state   the forward's inputs (initial_state NULL = zeros).
 *  d_o              [B,T,HV,V], p->dtype: gradient of o (required).
 *  d_final_state    [N,HV,K,V] fp32, or NULL for zeros.
 *  dq, dk           [B,T,H,K], p->dtype: with grouped value heads, summed over
 *                   the value heads that read the key head.
 *  dv [B,T,HV,V], dgate [B,T,HV,K], dbeta [B,T,HV]   p->dtype (dbeta is the
 *                   gradient of the beta logits).
 *  da_log [HV], ddt_bias [HV,K]   fp32, summed over all tokens (required).
 *  d_initial_state  [N,HV,K,V] fp32, or NULL to not produce it; for an empty
 *                   document it equals that document's d_final_state.
 *  workspace        at least kda_bwd_workspace_size() bytes, 256-byte aligned.
 * Where the forward floors the log-decay at -110 or clamps it at the bound,
 * the gate's gradient is zero.  The forward's chunk factors are recomputed,
 * not read from a forward call: in fp32 for fp32 inputs; for bf16 inputs on
 * the forward's matrix-core chunk kernel (bf16 operands, fp32 accumulation,
 * as in the forward), or in fp32 when the environment sets
 * KDA_BWD_RECOMPUTE=valu (slower; fp32 parameter and state gradients then
 * about 1e-6 instead of 1e-3 relative).  Everything after the recomputation
 * accumulates in fp32; for bf16 inputs with 64-token chunks the fp32 states
 * and Delta enter the matrix-core products as bf16 hi + lo pairs (about 16
 * significant bits).  Results are deterministic (fixed summation orders; the
 * one atomic counter only lists chunk-heads for a fix-up pass, each
 * recomputed whole).
 */
size_t kda_bwd_workspace_size(const kda_problem* p, kda_status* status);
kda_status kda_bwd(const kda_problem* p, const void* q, const void* k, const void* v,
                   const void* gate, const void* beta, const float* a_log, const float* dt_bias,
                   const float* initial_state, const void* d_o, const float* d_final_state,
                   void* dq, void* dk, void* dv, void* dgate, void* dbeta, float* da_log,
                   float* ddt_bias, float* d_initial_state, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * kda_bwd with per-stage timing hooks, for measurement.  It does exactly the
 * work of kda_bwd; in addition, when stage_events is not NULL it must hold
 * 2 * KDA_BWD_NUM_STAGES hipEvent_t handles created by the caller (entries may
 * be NULL), and the library records stage_events[2*i] on `stream` just before
 * stage i is enqueued and stage_events[2*i+1] just after.  Stages, in order:
 *   0 chunk table, 1 recomputation of the forward's chunk factors,
 *   2 forward state pass (state entering each chunk), 3 reverse state pass,
 *   4 chunk-local gradients, 5 dq/dk (with grouped value heads: the sums over
 *   a key head's value heads and the L2 norm's Jacobian; with one key head per
 *   value head nothing runs here, stage 4 applies the Jacobian),
 *   6 da_log and ddt_bias sums.
 * A stage with nothing to launch records both events back to back.
 */
#define KDA_BWD_NUM_STAGES 7
kda_status kda_bwd_profiled(const kda_problem* p, const void* q, const void* k, const void* v,
                            const void* gate, const void* beta, const float* a_log,
                            const float* dt_bias, const float* initial_state, const void* d_o,
                            const float* d_final_state, void* dq, void* dk, void* dv,
                            void* dgate, void* dbeta, float* da_log, float* ddt_bias,
                            float* d_initial_state, void* workspace, size_t workspace_bytes,
                            void* stream, void* const* stage_events);

/*
 * The layer's short convolution before the forward: SiLU of a causal
 * depthwise convolution over time, applied per channel to q, k and v
 * (hyper_parallel coverage page: `_run_causal_short_conv`,
 * `_local_short_conv` and the channel constraints of
 * `_validate_layer_short_conv` -- depthwise, stride 1, dilation 1, zero
 * padding of width-1 tokens on the left, output cut to the sequence length,
 * SiLU activation; without the convolution the layer applies SiLU alone, as
 * in the forward of KimiDeltaAttentionUlyssesCP).  For channel c of a tensor
 * x [B,T,C] (C = H*K for q and k, HV*V for v; channel h*D + d of head h):
 *
 *     y[t,c] = silu(bias[c] + sum_{j<W} weight[c,j] * x[t-(W-1)+j, c]),
 *     silu(z) = z * sigmoid(z)
 *
 * where x of a token before the first token of t's sequence counts as zero:
 * every row is padded on its own, and with cu_seqlens every document of the
 * packed row is (the NeMo AutoModel page "nemo_automodel.components.models.
 * kimi_k3.cp" hands the conv kernel size to the per-row context that carries
 * the document layout, `build_fla_cp_context`).
 *
 *  width      W, taps per channel: 0 = no convolution (y = silu(x), weights
 *             and biases ignored), 1..4.  Larger widths are KDA_EUNSUPPORTED,
 *             negative ones KDA_EINVAL.
 *  *_weight   fp32 [C, W] (the depthwise Conv1d weight [C, 1, W]); tap W-1
 *             weights the current token.  Required when width > 0.
 *  *_bias     fp32 [C], or NULL for no bias.
 * Device pointers, 4-byte aligned.
 */
typedef struct kda_short_conv {
  int32_t width;
  const float* q_weight;
  const float* k_weight;
  const float* v_weight;
  const float* q_bias;
  const float* k_bias;
  const float* v_bias;
} kda_short_conv;

/*
 * One tensor through the short convolution: y = SiLU(conv(x)) as above.
 * x, y [B,T,channels] with p->dtype elements, 16-byte aligned, channels a
 * multiple of 8 (bf16) or 4 (fp32); y may not overlap x.  Only B, T, dtype
 * and the document layout (N, cu_seqlens, cu_seqlens_host, validated as for
 * kda_fwd) are read from p.  Computes in fp32, rounds once to p->dtype.
 */
kda_status kda_short_conv_silu(const kda_problem* p, int32_t channels, int32_t width,
                               const void* x, const float* weight, const float* bias, void* y,
                               void* stream);

/* Workspace bytes for kda_fwd_short_conv: kda_fwd's plus the convolved q, k, v. */
size_t kda_fwd_short_conv_workspace_size(const kda_problem* p, kda_status* status);

/*
 * kda_fwd after the short convolution and SiLU of `conv` on q, k and v (the
 * layer order of the pages: projections, ShortConv + SiLU, then chunk_kda).
 * q, k, v are the raw projections; the convolved tensors live in the
 * workspace (p->dtype, rounded once), and the forward then runs on them
 * exactly as kda_fwd.  All other arguments are those of kda_fwd; q, k and v
 * must be 16-byte aligned.  (With the environment variable KDA_CONV_FUSED=1, a
 * bf16 matrix-core forward with width 4 and 16-byte aligned weights convolves
 * q, k and v as it loads them instead, with identical results; measured
 * slower, so not the default.)
 */
kda_status kda_fwd_short_conv(const kda_problem* p, const kda_short_conv* conv, const void* q,
                              const void* k, const void* v, const void* gate, const void* beta,
                              const float* a_log, const float* dt_bias,
                              const float* initial_state, void* o, float* final_state,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The gated output norm after the forward: o_norm(o, output_gate) of the
 * layer (hyper_parallel coverage page, the forward of
 * KimiDeltaAttentionUlyssesCP: the output gate projection reshaped to
 * [B, T, HV, V] and o_norm(output, output_gate) applied per value head; the
 * torchtitan PR #4025 review names the model's RMSNorm with an fp32
 * reduction).  The pages print neither the norm nor the gate's activation;
 * this library's reading, per (token, value head) row of V values:
 *
 *     y[v] = o[v] / sqrt(mean_v(o^2) + eps) * weight[v] * act(gate[v])
 *
 *  o, gate, y   [B, T, HV, V], p->dtype, 16-byte aligned; y may equal o.
 *  weight       fp32 [V] shared by all heads, or NULL for ones.
 *  eps          finite, >= 0.
 *  activation   KDA_NORM_SIGMOID (0) or KDA_NORM_SILU (1, x * sigmoid(x)).
 * Only B, T, H, HV, V, dtype and the row layout are read from p.  Computes in
 * fp32 (the mean over V in fp32), rounds once to p->dtype.
 */
#define KDA_NORM_SIGMOID 0
#define KDA_NORM_SILU 1
kda_status kda_gated_rms_norm(const kda_problem* p, const void* o, const void* gate,
                              const float* weight, float eps, int32_t activation, void* y,
                              void* stream);

/*
 * The forward followed by the gated output norm in one call (the layer's
 * chunk_kda then o_norm(o, output_gate), as above): writes
 *     y = o / sqrt(mean_V(o^2) + eps) * weight * act(norm->gate)
 * per (token, value head) row, where o is kda_fwd's output rounded to
 * p->dtype.  The forward writes o into y and kda_gated_rms_norm's kernel
 * normalises it in place on the same stream.  (The matrix-core state pass can
 * also apply the norm before storing the rows, with one workgroup holding
 * whole rows; that is slower on every measured shape and is used only when
 * the environment sets KDA_NORM_IN_PASS=1.)
 *  norm->gate     [B,T,HV,V], p->dtype, 16-byte aligned (not NULL).
 *  norm->weight   fp32 [V] or NULL for ones.
 *  norm->eps      finite, >= 0.   norm->activation  KDA_NORM_SIGMOID / _SILU.
 *  y              [B,T,HV,V], p->dtype (takes kda_fwd's o argument's place).
 * Everything else as kda_fwd; the workspace is
 * kda_fwd_gated_norm_workspace_size(p) bytes.
 */
typedef struct kda_output_norm {
  const void* gate;
  const float* weight;
  float eps;
  int32_t activation;
} kda_output_norm;
size_t kda_fwd_gated_norm_workspace_size(const kda_problem* p, kda_status* status);
kda_status kda_fwd_gated_norm(const kda_problem* p, const kda_output_norm* norm, const void* q,
                              const void* k, const void* v, const void* gate, const void* beta,
                              const float* a_log, const float* dt_bias,
                              const float* initial_state, void* y, float* final_state,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* kda_last_error(void);

/* Library version, (major << 16) | minor. */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
