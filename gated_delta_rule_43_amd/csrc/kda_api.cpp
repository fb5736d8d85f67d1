// Host side of libkda.so: argument validation, workspace layout, launch plan.
// Every check runs before anything is enqueued; see include/kda.h for the
// contract each entry point keeps.
#include "../../include/kda.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

constexpr size_t kAlign = 256;
constexpr size_t kSinkBytes = 16384;  // 256 threads x 2 column tiles x 8 B, with room
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }
bool wide(const kda_problem* p) { return p->K == 256 || p->V == 256; }

// value heads (HV, 0 meaning H)
int value_heads(const kda_problem* p) { return p->HV > 0 ? p->HV : p->H; }

// Rows, dtype and document layout (B, T, dtype, N, cu_seqlens, cu_seqlens_host).
kda_status validate_rows(const kda_problem* p, bool summary) {
  if (!p) return fail(KDA_EINVAL, "problem is NULL");
  if (p->B < 1 || p->T < 0) return fail(KDA_EINVAL, "bad shape B=%d T=%d (need B >= 1, T >= 0)", p->B, p->T);
  if (p->dtype != KDA_F32 && p->dtype != KDA_BF16)
    return fail(KDA_EINVAL, "dtype must be KDA_F32 or KDA_BF16, got %d", p->dtype);
  if ((long long)p->B * p->T >= (1LL << 31))
    return fail(KDA_EUNSUPPORTED, "B*T = %lld tokens exceeds 2^31", (long long)p->B * p->T);
  if (p->cu_seqlens == nullptr) {
    if (p->cu_seqlens_host != nullptr)
      return fail(KDA_EINVAL, "cu_seqlens_host given without cu_seqlens");
    if (p->N != p->B)
      return fail(KDA_EINVAL, "N must equal B (%d) without cu_seqlens, got %d", p->B, p->N);
  } else {
    if (summary) return fail(KDA_EINVAL, "a state summary takes no cu_seqlens (one slice per row)");
    if (p->B != 1) return fail(KDA_EINVAL, "cu_seqlens requires B == 1 (one packed row), got B=%d", p->B);
    if (p->N < 0 || (p->N == 0 && p->T != 0))
      return fail(KDA_EINVAL, "cu_seqlens must describe at least one sequence (N=%d, T=%d)", p->N, p->T);
    if (const int32_t* cu = p->cu_seqlens_host) {
      if (cu[0] != 0) return fail(KDA_EINVAL, "cu_seqlens[0] must be 0, got %d", cu[0]);
      for (int n = 0; n < p->N; ++n) {
        if (cu[n + 1] < 0)
          return fail(KDA_EINVAL, "cu_seqlens[%d] = %d is negative (padding sentinels are not accepted)",
                      n + 1, cu[n + 1]);
        if (cu[n + 1] < cu[n])
          return fail(KDA_EINVAL, "cu_seqlens must be non-decreasing: cu[%d]=%d < cu[%d]=%d", n + 1,
                      cu[n + 1], n, cu[n]);
      }
      if (cu[p->N] != p->T)
        return fail(KDA_EINVAL, "cu_seqlens[N] must equal T=%d, got %d", p->T, cu[p->N]);
    }
  }
  return KDA_OK;
}

// Shape/flag validation shared by every entry point (no pointers checked here).
kda_status validate_problem(const kda_problem* p, bool summary) {
  if (!p) return fail(KDA_EINVAL, "problem is NULL");
  if (p->B < 1 || p->T < 0 || p->H < 1 || p->K < 1 || p->V < 1)
    return fail(KDA_EINVAL, "bad shape B=%d T=%d H=%d K=%d V=%d (need B,H,K,V >= 1, T >= 0)", p->B,
                p->T, p->H, p->K, p->V);
  if (p->dtype != KDA_F32 && p->dtype != KDA_BF16)
    return fail(KDA_EINVAL, "dtype must be KDA_F32 or KDA_BF16, got %d", p->dtype);
  if (p->chunk_size <= 0) return fail(KDA_EINVAL, "chunk_size must be positive, got %d", p->chunk_size);
  if (p->chunk_size != 16 && p->chunk_size != 32 && p->chunk_size != 64)
    return fail(KDA_EUNSUPPORTED, "chunk_size %d is not supported (16, 32 or 64)", p->chunk_size);
  if (!std::isnan(p->lower_bound) && !(p->lower_bound < 0.f && std::isfinite(p->lower_bound)))
    return fail(KDA_EINVAL, "lower_bound must be negative, got %g", (double)p->lower_bound);
  if (p->lower_bound_form != KDA_LB_SIGMOID && p->lower_bound_form != KDA_LB_CLAMP)
    return fail(KDA_EINVAL, "lower_bound_form must be KDA_LB_SIGMOID or KDA_LB_CLAMP, got %d",
                p->lower_bound_form);
  if (p->lower_bound_form == KDA_LB_CLAMP && std::isnan(p->lower_bound))
    return fail(KDA_EINVAL, "the clamped gate needs a lower_bound");
  if (p->HV < 0 || (p->HV > 0 && p->HV % p->H != 0))
    return fail(KDA_EINVAL, "value heads HV=%d must be a positive multiple of the key heads H=%d (or 0)",
                p->HV, p->H);
  if (!head_dim_ok(p->K) || !head_dim_ok(p->V))
    return fail(KDA_EUNSUPPORTED, "head dims K=%d V=%d are not supported (64, 128 or 256)", p->K, p->V);
  if (wide(p) && p->chunk_size == 64)
    return fail(KDA_EUNSUPPORTED, "head dim 256 runs with chunk_size 16 or 32, got 64");
  const long long BT = (long long)p->B * p->T;
  if (BT >= (1LL << 31) || BT * value_heads(p) >= (1LL << 31))
    return fail(KDA_EUNSUPPORTED, "B*T*HV = %lld token-heads exceeds 2^31", BT * value_heads(p));
  return validate_rows(p, summary);
}

// Which kernels run.  fp32 inputs: the VALU path.  bf16: the matrix-core
// kernels, whose tiles hold 64 rows; chunks of 16 or 32 tokens fill the first
// rows of a tile and the rest is masked exactly as past a sequence's end (zero
// beta, q^, k^ and log-decay), so the tile computes those chunks' algebra.
// The matrix-core kernels run either fused (one
// workgroup per (sequence, head) computes and consumes each chunk's factors
// in LDS) or in two passes (all chunk-heads' factors in parallel as records in
// the workspace, then the sequential state pass over them).  Summaries take
// the two-pass kernels.  KDA_PATH=valu|mfma|fused forces a path where it
// applies (for comparisons).
enum Path { kPathValu = 0, kPathMfma = 1, kPathFused = 2 };

int choose_path(const kda_problem* p, bool summary) {
  const bool mfma_ok = p->dtype == KDA_BF16 && !wide(p) &&
                       (p->chunk_size == 64 || p->chunk_size == 32 || p->chunk_size == 16);
  const char* env = std::getenv("KDA_PATH");
  if (env && std::strcmp(env, "valu") == 0) return kPathValu;
  if (!mfma_ok) return kPathValu;
  if (env && std::strcmp(env, "mfma") == 0) return kPathMfma;
  if (summary) return kPathMfma;
  if (env && std::strcmp(env, "fused") == 0) return kPathFused;
  return kPathMfma;
}

struct Layout {
  int NT = 0;
  int exact = 1;
  int path = kPathValu;
  bool mfma = false;  // chunk records in the workspace (two-pass matrix-core path)
  size_t off_tok = 0, off_len = 0, off_seq0 = 0, off_nt = 0, off_cseq = 0, off_done = 0;
  size_t off_qn = 0, off_kn = 0, off_g = 0, off_bt = 0;
  size_t off_W = 0, off_U = 0, off_Qt = 0, off_Kb = 0, off_Aqk = 0, off_gL = 0;
  size_t off_rec = 0, off_sink = 0, off_xcount = 0, off_xlist = 0;
  size_t total = 0;
};

int chunk_count(const kda_problem* p, int* exact) {
  const int C = p->chunk_size;
  if (!p->cu_seqlens) {
    *exact = 1;
    return p->B * ((p->T + C - 1) / C);
  }
  if (p->cu_seqlens_host) {
    long long nt = 0;
    for (int n = 0; n < p->N; ++n) nt += (p->cu_seqlens_host[n + 1] - p->cu_seqlens_host[n] + C - 1) / C;
    *exact = 1;
    return (int)nt;
  }
  *exact = 0;  // sum_n ceil(L_n / C) <= floor(T / C) + N
  return p->T / C + p->N;
}

Layout layout_for(const kda_problem* p, int path) {
  Layout L;
  L.NT = chunk_count(p, &L.exact);
  L.path = path;
  L.mfma = path == kPathMfma;
  const size_t NT = (size_t)L.NT, H = value_heads(p), K = p->K, V = p->V, C = p->chunk_size, N = p->N;
  const size_t tokh = (size_t)p->B * p->T * H;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.off_tok = take(NT * 4);
  L.off_len = take(NT * 4);
  L.off_seq0 = take((N + 1) * 4);
  L.off_nt = take(4);
  L.off_cseq = take(NT * 4);
  if (L.mfma) {
    // one record of MFMA-ready chunk factors per chunk-head
    L.off_rec = take(NT * H * kda::mfma_record_bytes(p->K, p->V));
    L.off_sink = take(kSinkBytes);
    L.off_xcount = take(4);
    L.off_xlist = take(NT * H * 4);
    L.off_done = take(NT * H * 4);
  } else if (path == kPathValu) {
    L.off_qn = take(tokh * K * 4);
    L.off_kn = take(tokh * K * 4);
    L.off_g = take(tokh * K * 4);
    L.off_bt = take(tokh * 4);
    const size_t elt = 4;
    L.off_W = take(NT * H * C * K * elt);
    L.off_U = take(NT * H * C * V * elt);
    L.off_Qt = take(NT * H * C * K * elt);
    L.off_Kb = take(NT * H * C * K * elt);
    L.off_Aqk = take(NT * H * C * C * elt);
    L.off_gL = take(NT * H * K * 4);
  }
  L.total = o;
  return L;
}

Layout layout(const kda_problem* p, bool summary) { return layout_for(p, choose_path(p, summary)); }

// The backward's workspace: the VALU forward's (recomputed factors) followed by
// Akk and Tm, per-chunk states and their gradients, the per-value-head
// gradients of q^ and k^, per-chunk partial sums of the gate-parameter
// gradients, the L2 norm's scales per token-head and (bf16) the fix-up list
// of the matrix-core recomputation.
struct BwdLayout {
  Layout f;
  size_t off_akk = 0, off_tm = 0, off_hc = 0, off_dhc = 0, off_dc = 0, off_ddc = 0;
  size_t off_dqh = 0, off_dkh = 0, off_da = 0, off_ddt = 0;
  size_t off_xcount = 0, off_xlist = 0;  // bf16: the recomputation's fix-up list
  size_t off_rq = 0, off_rk = 0;         // the L2 norm's scales per token-head
  size_t total = 0;
};

BwdLayout bwd_layout(const kda_problem* p) {
  BwdLayout B;
  B.f = layout_for(p, kPathValu);
  const size_t NT = (size_t)B.f.NT, H = value_heads(p), K = p->K, V = p->V, C = p->chunk_size;
  const size_t tokh = (size_t)p->B * p->T * H;
  size_t o = B.f.total;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  B.off_akk = take(NT * H * C * C * 4);
  B.off_tm = take(NT * H * C * C * 4);
  B.off_hc = take(NT * H * K * V * 4);
  B.off_dhc = take(NT * H * K * V * 4);
  B.off_dc = take(NT * H * C * V * 4);
  B.off_ddc = take(NT * H * C * V * 4);
  B.off_dqh = take(tokh * K * 4);
  B.off_dkh = take(tokh * K * 4);
  B.off_da = take(NT * H * 4);
  B.off_ddt = take(NT * H * K * 4);
  B.off_rq = take(tokh * 4);
  B.off_rk = take(tokh * 4);
  if (p->dtype == KDA_BF16) {
    B.off_xcount = take(4);
    B.off_xlist = take(NT * H * 4);
  }
  B.total = o;
  return B;
}

kda::FwdArgs make_args(const kda_problem* p, const Layout& L, void* ws) {
  kda::FwdArgs a{};
  a.B = p->B; a.T = p->T; a.H = value_heads(p); a.HK = p->H; a.K = p->K; a.V = p->V;
  a.C = p->chunk_size; a.N = p->N;
  a.NT = L.NT;
  a.exact_nt = L.exact;
  a.dtype = p->dtype;
  a.scale = (p->scale > 0.f) ? p->scale : 1.0f / std::sqrt((float)p->K);
  a.gate_form = std::isnan(p->lower_bound) ? 0 : (p->lower_bound_form == KDA_LB_CLAMP ? 2 : 1);
  a.lb = a.gate_form ? p->lower_bound : 0.f;
  a.cu = p->cu_seqlens;
  char* w = (char*)ws;
  a.chunk_tok = (int32_t*)(w + L.off_tok);
  a.chunk_len = (int32_t*)(w + L.off_len);
  a.seq_chunk0 = (int32_t*)(w + L.off_seq0);
  a.nt_dev = (int32_t*)(w + L.off_nt);
  a.chunk_seq = (int32_t*)(w + L.off_cseq);
  if (L.path == kPathFused) {
    // the fused kernel needs the chunk table only
  } else if (L.mfma) {
    a.rec = w + L.off_rec;
    a.sink = w + L.off_sink;
    a.exact_count = (int32_t*)(w + L.off_xcount);
    a.exact_list = (int32_t*)(w + L.off_xlist);
    a.done = (int32_t*)(w + L.off_done);
  } else {
    a.qn = (float*)(w + L.off_qn);
    a.kn = (float*)(w + L.off_kn);
    a.g = (float*)(w + L.off_g);
    a.bt = (float*)(w + L.off_bt);
    a.W = w + L.off_W;
    a.U = w + L.off_U;
    a.Qt = w + L.off_Qt;
    a.Kb = w + L.off_Kb;
    a.Aqk = w + L.off_Aqk;
    a.gL = (float*)(w + L.off_gL);
  }
  return a;
}

hipError_t launch(const kda::FwdArgs& a, const Layout& L, hipStream_t s) {
  hipError_t e = kda::launch_chunk_table(a, s);
  if (e != hipSuccess) return e;
  if (L.path == kPathFused) return kda::launch_fused_path(a, s);
  return L.mfma ? kda::launch_mfma_path(a, s) : kda::launch_valu_path(a, s);
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

kda_status check_inputs(const kda_problem* p, const void* q, const void* k, const void* v,
                        const void* gate, const void* beta, const float* a_log,
                        const float* dt_bias) {
  const bool any_tokens = (long long)p->B * p->T > 0;
  if (any_tokens && (!q || !k || !v || !gate || !beta))
    return fail(KDA_EINVAL, "q, k, v, gate and beta must be non-NULL");
  if (!a_log || !dt_bias) return fail(KDA_EINVAL, "a_log and dt_bias must be non-NULL (fp32 [H] and [H,K])");
  const size_t elt = p->dtype == KDA_BF16 ? 2 : 4;
  const void* ptrs[] = {q, k, v, gate, beta};
  for (const void* ptr : ptrs)
    if (ptr && !aligned(ptr, elt)) return fail(KDA_EINVAL, "input tensor is not %zu-byte aligned", elt);
  if (!aligned(a_log, 4) || !aligned(dt_bias, 4)) return fail(KDA_EINVAL, "a_log/dt_bias misaligned");
  return KDA_OK;
}

kda_status check_ws(size_t need, void* ws, size_t bytes) {
  if (need == 0) return KDA_OK;
  if (!ws) return fail(KDA_EWORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (bytes < need) return fail(KDA_EWORKSPACE, "workspace has %zu bytes, %zu needed", bytes, need);
  if (!aligned(ws, kAlign)) return fail(KDA_EINVAL, "workspace must be 256-byte aligned");
  return KDA_OK;
}

// Widths of the short convolution this build instantiates.
kda_status check_width(int width) {
  if (width < 0) return fail(KDA_EINVAL, "short convolution width must be >= 0, got %d", width);
  if (width > 4) return fail(KDA_EUNSUPPORTED, "short convolution width %d is not supported (0..4)", width);
  return KDA_OK;
}

// The convolved q, k, v of kda_fwd_short_conv, placed after the forward's own
// workspace (which starts at offset 0 and is laid out as for kda_fwd).
struct ConvBuffers {
  size_t off_q = 0, off_k = 0, off_v = 0, total = 0;
};

ConvBuffers conv_buffers(const kda_problem* p, size_t base) {
  ConvBuffers c;
  const size_t elt = p->dtype == KDA_BF16 ? 2 : 4;
  const size_t tokens = (size_t)p->B * p->T;
  c.off_q = align_up(base);
  c.off_k = align_up(c.off_q + tokens * p->H * p->K * elt);
  c.off_v = align_up(c.off_k + tokens * p->H * p->K * elt);
  c.total = align_up(c.off_v + tokens * value_heads(p) * p->V * elt);
  return c;
}

kda_status check_conv(const kda_problem* p, const kda_short_conv* conv, const void* q,
                      const void* k, const void* v) {
  kda_status st = check_width(conv->width);
  if (st != KDA_OK) return st;
  if (conv->width > 0 && (!conv->q_weight || !conv->k_weight || !conv->v_weight))
    return fail(KDA_EINVAL, "a convolution of width %d needs q, k and v weights", conv->width);
  const float* fp[] = {conv->q_weight, conv->k_weight, conv->v_weight,
                       conv->q_bias, conv->k_bias, conv->v_bias};
  for (const float* f : fp)
    if (f && !aligned(f, 4)) return fail(KDA_EINVAL, "short convolution weights and biases must be 4-byte aligned");
  const void* in[] = {q, k, v};
  for (const void* ptr : in)
    if (ptr && !aligned(ptr, 16))
      return fail(KDA_EINVAL, "q, k and v must be 16-byte aligned for the short convolution");
  return KDA_OK;
}

// By default the standalone pass convolves q, k and v into the workspace and
// the forward reads the results.  KDA_CONV_FUSED=1 makes the matrix-core
// kernels apply a width-4 convolution as they load q, k and v instead (bf16,
// weights and biases 16-byte aligned); both round each convolved value to the
// input dtype in the same order of operations, so the results are identical.
// Measured slower: on the throughput shape (B=4, T=16384, H=32, d=128) the
// forward with the convolution takes 3.04 ms on load against 2.24 ms with the
// standalone pass (1.65 ms without any convolution), on short documents (d=64)
// 2.45 against 1.51 ms: in the chunk kernel's row layout every lane reloads its
// channels' weights and the convolution adds about 17 VALU operations per
// element to a kernel that is already mostly VALU-busy, while the standalone pass
// streams at HBM speed.
bool conv_on_load(const kda_problem* p, const kda_short_conv* conv, int path) {
  if (!conv || conv->width != 4 || path == kPathValu || p->dtype != KDA_BF16) return false;
  const float* fp[] = {conv->q_weight, conv->k_weight, conv->v_weight,
                       conv->q_bias, conv->k_bias, conv->v_bias};
  for (const float* f : fp)
    if (f && !aligned(f, 16)) return false;
  const char* env = std::getenv("KDA_CONV_FUSED");
  return env && std::atoi(env) != 0;
}

// kda_fwd, optionally after the short convolution of q, k and v.  path < 0:
// the library's choice; otherwise the path whose workspace the caller sized.
// The gated output norm needs whole output rows: the fused kernel's consumer
// waves split them, so a normed forward takes the two-pass kernels instead.
int norm_path(const kda_problem* p) {
  const int path = choose_path(p, false);
  return path == kPathFused ? kPathMfma : path;
}

kda_status check_norm(const kda_problem* p, const kda_output_norm* nrm) {
  if (!nrm->gate) return fail(KDA_EINVAL, "the output norm's gate must be non-NULL");
  if (!aligned(nrm->gate, 16)) return fail(KDA_EINVAL, "the output norm's gate must be 16-byte aligned");
  if (nrm->weight && !aligned(nrm->weight, 16)) return fail(KDA_EINVAL, "the output norm's weight must be 16-byte aligned");
  if (!std::isfinite(nrm->eps) || nrm->eps < 0.f) return fail(KDA_EINVAL, "eps must be finite and >= 0");
  if (nrm->activation != KDA_NORM_SIGMOID && nrm->activation != KDA_NORM_SILU)
    return fail(KDA_EINVAL, "activation must be KDA_NORM_SIGMOID or KDA_NORM_SILU");
  (void)p;
  return KDA_OK;
}

kda_status fwd_impl(const kda_problem* p, const kda_short_conv* conv, const void* q, const void* k,
                    const void* v, const void* gate, const void* beta, const float* a_log,
                    const float* dt_bias, const float* initial_state, void* o,
                    float* final_state, void* workspace, size_t workspace_bytes, void* stream,
                    void* const* stage_events, int path = -1,
                    const kda_output_norm* nrm = nullptr) {
  kda_status st = validate_problem(p, false);
  if (st != KDA_OK) return st;
  st = check_inputs(p, q, k, v, gate, beta, a_log, dt_bias);
  if (st != KDA_OK) return st;
  if (!o && (long long)p->B * p->T > 0) return fail(KDA_EINVAL, "output o must be non-NULL");
  if (initial_state && !aligned(initial_state, 4)) return fail(KDA_EINVAL, "initial_state misaligned");
  if (final_state && !aligned(final_state, 4)) return fail(KDA_EINVAL, "final_state misaligned");
  if (o && !aligned(o, p->dtype == KDA_BF16 ? 2 : 4)) return fail(KDA_EINVAL, "o misaligned");
  if (nrm) {
    st = check_norm(p, nrm);
    if (st != KDA_OK) return st;
    if (path < 0) path = norm_path(p);
  }
  const Layout L = path < 0 ? layout(p, false) : layout_for(p, path);
  ConvBuffers cb;
  bool on_load = false;
  if (conv) {
    st = check_conv(p, conv, q, k, v);
    if (st != KDA_OK) return st;
    on_load = conv_on_load(p, conv, L.path);
    if (!on_load) cb = conv_buffers(p, L.total);
  }
  st = check_ws(conv && !on_load ? cb.total : L.total, workspace, workspace_bytes);
  if (st != KDA_OK) return st;
  if (L.path != kPathValu) {
    const void* vec[] = {q, k, v, gate, o};
    for (const void* ptr : vec)
      if (ptr && !aligned(ptr, 16))
        return fail(KDA_EINVAL, "bf16 q, k, v, gate and o must be 16-byte aligned");
  }
  hipStream_t s = (hipStream_t)stream;
  if (conv && !on_load && (long long)p->B * p->T > 0) {
    char* w = (char*)workspace;
    kda::ConvArgs c{};
    c.B = p->B; c.T = p->T; c.N = p->N; c.dtype = p->dtype; c.width = conv->width;
    c.cu = p->cu_seqlens;
    c.count = 3;
    c.t[0] = kda::ConvTensor{q, conv->q_weight, conv->q_bias, w + cb.off_q, p->H * p->K};
    c.t[1] = kda::ConvTensor{k, conv->k_weight, conv->k_bias, w + cb.off_k, p->H * p->K};
    c.t[2] = kda::ConvTensor{v, conv->v_weight, conv->v_bias, w + cb.off_v, value_heads(p) * p->V};
    hipError_t e = kda::launch_short_conv(c, s);
    if (e != hipSuccess) return fail(KDA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    q = w + cb.off_q;
    k = w + cb.off_k;
    v = w + cb.off_v;
  }

  kda::FwdArgs a = make_args(p, L, workspace);
  a.q = q; a.k = k; a.v = v; a.gate = gate; a.beta = beta;
  a.a_log = a_log; a.dt_bias = dt_bias; a.init = initial_state;
  a.o = o; a.fin = final_state; a.summary = 0;
  a.events = stage_events;
  if (on_load) {
    a.conv = 1;
    a.conv_wq = conv->q_weight; a.conv_wk = conv->k_weight; a.conv_wv = conv->v_weight;
    a.conv_bq = conv->q_bias; a.conv_bk = conv->k_bias; a.conv_bv = conv->v_bias;
  }
  // The norm applied inside the state pass needs one workgroup per (sequence,
  // head) holding whole rows; on every measured shape that costs the pass
  // more than a separate pass over o costs (throughput shape 2.52 vs 1.97 ms,
  // packed varlen 0.36 vs 0.22, short documents 1.57 vs 1.20), so by default
  // the output is normalised in place right after the forward.
  // KDA_NORM_IN_PASS=1 selects the in-pass form.
  bool in_pass = false;
  if (nrm && L.path != kPathValu) {
    if (const char* env = std::getenv("KDA_NORM_IN_PASS")) in_pass = std::atoi(env) != 0;
  }
  if (in_pass) {
    a.norm = 1;
    a.norm_act = nrm->activation;
    a.norm_eps = nrm->eps;
    a.norm_gate = nrm->gate;
    a.norm_w = nrm->weight;
  }
  hipError_t e = launch(a, L, s);
  if (e == hipSuccess && nrm && !in_pass && (long long)p->B * p->T > 0) {
    kda::NormArgs na{};
    na.rows = (int64_t)p->B * p->T * value_heads(p);
    na.V = p->V;
    na.dtype = p->dtype == KDA_BF16 ? 1 : 0;
    na.act = nrm->activation;
    na.eps = nrm->eps;
    na.o = o;
    na.gate = nrm->gate;
    na.w = nrm->weight;
    na.y = o;
    e = kda::launch_gated_rms_norm(na, s);
  }
  if (e != hipSuccess) return fail(KDA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return KDA_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Allocation-free forward.  Its workspace is `scratch`, a device array of
// kNoAllocScratchBytes that every GPU the library runs on holds until the
// process ends.  In host code the array's name is only a stand-in: its device
// address comes from hipGetSymbolAddress, once per device (with that device
// current), and only that address is handed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The scratch array's device address on the current device (looked up once).
kda_status scratch_address(void* stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(KDA_EHIP, "no current HIP device (%s)", hipGetErrorString(e));
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess) return fail(KDA_EHIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(KDA_EINVAL, "the stream belongs to device %d but device %d is current", sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(KDA_EHIP, "hipGetSymbolAddress of the scratch array failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" {

size_t kda_fwd_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

size_t kda_fwd_gated_norm_workspace_size(const kda_problem* p, kda_status* status) {
  kda_status st = validate_problem(p, false);
  if (status) *status = st;
  return st == KDA_OK ? layout_for(p, norm_path(p)).total : 0;
}

kda_status kda_fwd_gated_norm(const kda_problem* p, const kda_output_norm* norm, const void* q,
                              const void* k, const void* v, const void* gate, const void* beta,
                              const float* a_log, const float* dt_bias,
                              const float* initial_state, void* y, float* final_state,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!norm) return fail(KDA_EINVAL, "output norm description is NULL");
  return fwd_impl(p, nullptr, q, k, v, gate, beta, a_log, dt_bias, initial_state, y, final_state,
                  workspace, workspace_bytes, stream, nullptr, -1, norm);
}

kda_status kda_fwd_noalloc(const kda_problem* p, const void* q, const void* k, const void* v,
                           const void* gate, const void* beta, const float* a_log,
                           const float* dt_bias, const float* initial_state, void* o,
                           float* final_state, void* stream) {
  kda_status st = validate_problem(p, false);
  if (st != KDA_OK) return st;
  // the library's path when its workspace fits the scratch array, else the
  // fused path, whose workspace is only the chunk table
  int path = choose_path(p, false);
  size_t need = layout_for(p, path).total;
  if (need > kNoAllocScratchBytes && path == kPathMfma) {
    path = kPathFused;
    need = layout_for(p, path).total;
  }
  if (need > kNoAllocScratchBytes)
    return fail(KDA_EWORKSPACE,
                "this problem needs %zu bytes of workspace; the allocation-free entry point has "
                "%zu (use kda_fwd with a caller-provided workspace)",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  st = scratch_address(stream, &ws);
  if (st != KDA_OK) return st;
  return fwd_impl(p, nullptr, q, k, v, gate, beta, a_log, dt_bias, initial_state, o, final_state,
                  ws, kNoAllocScratchBytes, stream, nullptr, path);
}

}  // extern "C"

extern "C" {

kda_status kda_validate(const kda_problem* p) {
  kda_status st = validate_problem(p, false);
  if (st == KDA_OK) g_last_error.clear();
  return st;
}

size_t kda_fwd_workspace_size(const kda_problem* p, kda_status* status) {
  kda_status st = validate_problem(p, false);
  if (status) *status = st;
  return st == KDA_OK ? layout(p, false).total : 0;
}

size_t kda_state_summary_workspace_size(const kda_problem* p, kda_status* status) {
  kda_status st = validate_problem(p, true);
  if (status) *status = st;
  return st == KDA_OK ? layout(p, true).total : 0;
}

int32_t kda_fwd_path(const kda_problem* p) {
  if (validate_problem(p, false) != KDA_OK) return -1;
  g_last_error.clear();
  return choose_path(p, false);
}

kda_status kda_fwd_profiled(const kda_problem* p, const void* q, const void* k, const void* v,
                            const void* gate, const void* beta, const float* a_log,
                            const float* dt_bias, const float* initial_state, void* o,
                            float* final_state, void* workspace, size_t workspace_bytes,
                            void* stream, void* const* stage_events) {
  return fwd_impl(p, nullptr, q, k, v, gate, beta, a_log, dt_bias, initial_state, o, final_state,
                  workspace, workspace_bytes, stream, stage_events);
}

kda_status kda_fwd(const kda_problem* p, const void* q, const void* k, const void* v,
                   const void* gate, const void* beta, const float* a_log, const float* dt_bias,
                   const float* initial_state, void* o, float* final_state, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return fwd_impl(p, nullptr, q, k, v, gate, beta, a_log, dt_bias, initial_state, o, final_state,
                  workspace, workspace_bytes, stream, nullptr);
}

size_t kda_fwd_short_conv_workspace_size(const kda_problem* p, kda_status* status) {
  kda_status st = validate_problem(p, false);
  if (status) *status = st;
  return st == KDA_OK ? conv_buffers(p, layout(p, false).total).total : 0;
}

kda_status kda_fwd_short_conv(const kda_problem* p, const kda_short_conv* conv, const void* q,
                              const void* k, const void* v, const void* gate, const void* beta,
                              const float* a_log, const float* dt_bias,
                              const float* initial_state, void* o, float* final_state,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!conv) return fail(KDA_EINVAL, "short convolution description is NULL");
  return fwd_impl(p, conv, q, k, v, gate, beta, a_log, dt_bias, initial_state, o, final_state,
                  workspace, workspace_bytes, stream, nullptr);
}

kda_status kda_short_conv_silu(const kda_problem* p, int32_t channels, int32_t width,
                               const void* x, const float* weight, const float* bias, void* y,
                               void* stream) {
  kda_status st = validate_rows(p, false);
  if (st != KDA_OK) return st;
  st = check_width(width);
  if (st != KDA_OK) return st;
  const int nv = p->dtype == KDA_BF16 ? 8 : 4;
  if (channels < 1 || channels % nv)
    return fail(KDA_EINVAL, "channels must be a positive multiple of %d, got %d", nv, channels);
  const long long tokens = (long long)p->B * p->T;
  if (tokens == 0) {
    g_last_error.clear();
    return KDA_OK;
  }
  if (!x || !y) return fail(KDA_EINVAL, "x and y must be non-NULL");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(KDA_EINVAL, "x and y must be 16-byte aligned");
  if (width > 0 && !weight) return fail(KDA_EINVAL, "a convolution of width %d needs its weight", width);
  if ((weight && !aligned(weight, 4)) || (bias && !aligned(bias, 4)))
    return fail(KDA_EINVAL, "weight and bias must be 4-byte aligned");
  const size_t bytes = (size_t)tokens * channels * (p->dtype == KDA_BF16 ? 2 : 4);
  const uintptr_t xb = (uintptr_t)x, yb = (uintptr_t)y;
  if (xb < yb + bytes && yb < xb + bytes) return fail(KDA_EINVAL, "y may not overlap x");
  kda::ConvArgs c{};
  c.B = p->B; c.T = p->T; c.N = p->N; c.dtype = p->dtype; c.width = width; c.cu = p->cu_seqlens;
  c.count = 1;
  c.t[0] = kda::ConvTensor{x, weight, bias, y, channels};
  hipError_t e = kda::launch_short_conv(c, (hipStream_t)stream);
  if (e != hipSuccess) return fail(KDA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return KDA_OK;
}

kda_status kda_state_summary(const kda_problem* p, const void* q, const void* k, const void* v,
                             const void* gate, const void* beta, const float* a_log,
                             const float* dt_bias, float* state_ext, float* transition,
                             void* workspace, size_t workspace_bytes, void* stream) {
  kda_status st = validate_problem(p, true);
  if (st != KDA_OK) return st;
  st = check_inputs(p, q, k, v, gate, beta, a_log, dt_bias);
  if (st != KDA_OK) return st;
  if (!state_ext || !transition) return fail(KDA_EINVAL, "state_ext and transition must be non-NULL");
  if (!aligned(state_ext, 4) || !aligned(transition, 4)) return fail(KDA_EINVAL, "summary outputs misaligned");
  const Layout L = layout(p, true);
  st = check_ws(L.total, workspace, workspace_bytes);
  if (st != KDA_OK) return st;
  if (L.mfma) {
    const void* vec[] = {q, k, v, gate};
    for (const void* ptr : vec)
      if (ptr && !aligned(ptr, 16))
        return fail(KDA_EINVAL, "bf16 q, k, v and gate must be 16-byte aligned");
  }
  kda::FwdArgs a = make_args(p, L, workspace);
  a.q = q; a.k = k; a.v = v; a.gate = gate; a.beta = beta;
  a.a_log = a_log; a.dt_bias = dt_bias; a.init = nullptr;
  a.o = nullptr; a.fin = nullptr; a.summary = 1;
  a.state_ext = state_ext; a.transition = transition;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch(a, L, s);
  if (e != hipSuccess) return fail(KDA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return KDA_OK;
}

kda_status kda_apply_state_summary(int32_t B, int32_t H, int32_t K, int32_t V,
                                   const float* state_ext, const float* transition,
                                   const float* initial_state, float* final_state, void* stream) {
  if (B < 1 || H < 1 || !head_dim_ok(K) || !head_dim_ok(V))
    return fail(B < 1 || H < 1 ? KDA_EINVAL : KDA_EUNSUPPORTED,
                "bad summary shape B=%d H=%d K=%d V=%d", B, H, K, V);
  if (!state_ext || !final_state || (initial_state && !transition))
    return fail(KDA_EINVAL, "state_ext, final_state (and transition when initial_state is given) must be non-NULL");
  if (initial_state && (final_state == initial_state || (const float*)final_state == transition))
    return fail(KDA_EINVAL, "final_state may not alias initial_state or transition");
  hipError_t e = kda::launch_apply_summary(B, H, K, V, state_ext, transition, initial_state,
                                           final_state, (hipStream_t)stream);
  if (e != hipSuccess) return fail(KDA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return KDA_OK;
}

int32_t kda_chunk_capacity(const kda_problem* p, kda_status* status) {
  kda_status st = validate_problem(p, false);
  if (status) *status = st;
  if (st != KDA_OK) return 0;
  int exact = 0;
  return chunk_count(p, &exact);
}

kda_status kda_chunk_table(const kda_problem* p, int32_t* tok, int32_t* len, int32_t* seq_chunk0,
                           int32_t* count, int32_t cap, void* stream) {
  kda_status st = validate_problem(p, false);
  if (st != KDA_OK) return st;
  int exact = 0;
  const int need = chunk_count(p, &exact);
  if (cap < need) return fail(KDA_EINVAL, "chunk table capacity %d < %d", cap, need);
  if ((need > 0 && (!tok || !len)) || !seq_chunk0 || !count)
    return fail(KDA_EINVAL, "chunk table buffers must be non-NULL");
  kda::FwdArgs a{};
  a.B = p->B; a.T = p->T; a.C = p->chunk_size; a.N = p->N; a.NT = need; a.cu = p->cu_seqlens;
  a.chunk_tok = tok; a.chunk_len = len; a.seq_chunk0 = seq_chunk0; a.nt_dev = count;
  hipError_t e = kda::launch_chunk_table(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(KDA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return KDA_OK;
}

// The backward keeps head dims 64 and 128 (its chunk kernel's LDS is sized for 128).
kda_status validate_bwd(const kda_problem* p) {
  kda_status st = validate_problem(p, false);
  if (st == KDA_OK && wide(p))
    return fail(KDA_EUNSUPPORTED, "the backward supports head dims 64 and 128, got K=%d V=%d", p->K, p->V);
  return st;
}

size_t kda_bwd_workspace_size(const kda_problem* p, kda_status* status) {
  kda_status st = validate_bwd(p);
  if (status) *status = st;
  return st == KDA_OK ? bwd_layout(p).total : 0;
}

kda_status kda_bwd(const kda_problem* p, const void* q, const void* k, const void* v,
                   const void* gate, const void* beta, const float* a_log, const float* dt_bias,
                   const float* initial_state, const void* d_o, const float* d_final_state,
                   void* dq, void* dk, void* dv, void* dgate, void* dbeta, float* da_log,
                   float* ddt_bias, float* d_initial_state, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return kda_bwd_profiled(p, q, k, v, gate, beta, a_log, dt_bias, initial_state, d_o,
                          d_final_state, dq, dk, dv, dgate, dbeta, da_log, ddt_bias,
                          d_initial_state, workspace, workspace_bytes, stream, nullptr);
}

kda_status kda_bwd_profiled(const kda_problem* p, const void* q, const void* k, const void* v,
                            const void* gate, const void* beta, const float* a_log,
                            const float* dt_bias, const float* initial_state, const void* d_o,
                            const float* d_final_state, void* dq, void* dk, void* dv,
                            void* dgate, void* dbeta, float* da_log, float* ddt_bias,
                            float* d_initial_state, void* workspace, size_t workspace_bytes,
                            void* stream, void* const* stage_events) {
  kda_status st = validate_bwd(p);
  if (st != KDA_OK) return st;
  st = check_inputs(p, q, k, v, gate, beta, a_log, dt_bias);
  if (st != KDA_OK) return st;
  const bool any_tokens = (long long)p->B * p->T > 0;
  if (any_tokens && (!d_o || !dq || !dk || !dv || !dgate || !dbeta))
    return fail(KDA_EINVAL, "d_o, dq, dk, dv, dgate and dbeta must be non-NULL");
  if (!da_log || !ddt_bias) return fail(KDA_EINVAL, "da_log and ddt_bias must be non-NULL");
  const size_t elt = p->dtype == KDA_BF16 ? 2 : 4;
  const void* typed[] = {d_o, dq, dk, dv, dgate, dbeta};
  for (const void* ptr : typed)
    if (ptr && !aligned(ptr, elt)) return fail(KDA_EINVAL, "gradient tensor is not %zu-byte aligned", elt);
  const void* f32[] = {initial_state, d_final_state, da_log, ddt_bias, d_initial_state};
  for (const void* ptr : f32)
    if (ptr && !aligned(ptr, 4)) return fail(KDA_EINVAL, "fp32 state or parameter gradient misaligned");
  const BwdLayout L = bwd_layout(p);
  st = check_ws(L.total, workspace, workspace_bytes);
  if (st != KDA_OK) return st;
  char* w = (char*)workspace;
  kda::BwdArgs b{};
  b.f = make_args(p, L.f, workspace);
  b.f.q = q; b.f.k = k; b.f.v = v; b.f.gate = gate; b.f.beta = beta;
  b.f.a_log = a_log; b.f.dt_bias = dt_bias; b.f.init = initial_state;
  b.f.Akk_out = (float*)(w + L.off_akk);
  b.f.Tm_out = (float*)(w + L.off_tm);
  b.f.rq = (float*)(w + L.off_rq);
  b.f.rk = (float*)(w + L.off_rk);
  // bf16: the chunk factors are recomputed on the matrix-core chunk kernel
  // (for comparisons, KDA_BWD_RECOMPUTE=valu keeps the fp32 vector-ALU kernels
  // and =mfma32 keeps every recomputed array in fp32)
  // (it reads q, k, v and gate in 8-byte pieces: they must be 16-byte aligned,
  // else the vector-ALU kernels run)
  const char* rc = std::getenv("KDA_BWD_RECOMPUTE");
  bool vec_ok = true;
  for (const void* ptr : {q, k, v, gate})
    if (ptr && !aligned(ptr, 16)) vec_ok = false;
  if (p->dtype == KDA_BF16 && vec_ok && !(rc && std::strcmp(rc, "valu") == 0)) {
    b.f.exact_count = (int32_t*)(w + L.off_xcount);
    b.f.exact_list = (int32_t*)(w + L.off_xlist);
    // the matrix-core state passes (64-token chunks) read W, U, Qt, Kbar and
    // Aqk as bf16, like the forward's records
    b.f.ws_bf16 = p->chunk_size == 64 && !(rc && std::strcmp(rc, "mfma32") == 0) ? 1 : 0;
  }
  b.d_o = d_o; b.d_fin = d_final_state;
  b.hc = (float*)(w + L.off_hc); b.dhc = (float*)(w + L.off_dhc);
  b.Dc = (float*)(w + L.off_dc); b.dDc = (float*)(w + L.off_ddc);
  b.dqh = (float*)(w + L.off_dqh); b.dkh = (float*)(w + L.off_dkh);
  b.da_part = (float*)(w + L.off_da); b.ddt_part = (float*)(w + L.off_ddt);
  b.dq = dq; b.dk = dk; b.dv = dv; b.dgate = dgate; b.dbeta = dbeta;
  b.da_log = da_log; b.ddt_bias = ddt_bias; b.dinit = d_initial_state;
  b.events = stage_events;
  hipError_t e = kda::launch_bwd(b, (hipStream_t)stream);
  if (e != hipSuccess) return fail(KDA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return KDA_OK;
}

kda_status kda_gated_rms_norm(const kda_problem* p, const void* o, const void* gate,
                              const float* weight, float eps, int32_t activation, void* y,
                              void* stream) {
  kda_status st = validate_rows(p, false);
  if (st != KDA_OK) return st;
  if (p->H < 1 || p->HV < 0 || (p->HV > 0 && p->HV % p->H != 0))
    return fail(KDA_EINVAL, "bad heads H=%d HV=%d", p->H, p->HV);
  if (!head_dim_ok(p->V)) return fail(KDA_EUNSUPPORTED, "value head dim V=%d is not supported (64, 128 or 256)", p->V);
  if (activation != KDA_NORM_SIGMOID && activation != KDA_NORM_SILU)
    return fail(KDA_EINVAL, "activation must be KDA_NORM_SIGMOID or KDA_NORM_SILU, got %d", activation);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(KDA_EINVAL, "eps must be finite and >= 0, got %g", (double)eps);
  const long long rows = (long long)p->B * p->T * value_heads(p);
  if (rows == 0) {
    g_last_error.clear();
    return KDA_OK;
  }
  if (!o || !gate || !y) return fail(KDA_EINVAL, "o, gate and y must be non-NULL");
  if (!aligned(o, 16) || !aligned(gate, 16) || !aligned(y, 16))
    return fail(KDA_EINVAL, "o, gate and y must be 16-byte aligned");
  if (weight && !aligned(weight, 4)) return fail(KDA_EINVAL, "weight must be 4-byte aligned");
  kda::NormArgs a{};
  a.rows = rows; a.V = p->V; a.dtype = p->dtype; a.act = activation; a.eps = eps;
  a.o = o; a.gate = gate; a.w = weight; a.y = y;
  hipError_t e = kda::launch_gated_rms_norm(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(KDA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return KDA_OK;
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

int32_t kda_version(void) { return (0 << 16) | 1; }

}  // extern "C"
