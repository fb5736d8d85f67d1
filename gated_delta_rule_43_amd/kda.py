"""Python binding of libkda.so (C ABI in include/kda.h).

Argument marshalling only: shapes, dtypes and devices are checked, outputs and
the workspace are allocated with torch, and every step of the forward runs in
the HIP kernels of libkda.so on the current HIP stream.  There is no other
implementation behind these functions: if the library is missing they raise.

Keywords mirror the chunk_kda call on the hyper_parallel coverage page for
context_parallel/kimi_delta_attention.py (`_run_local_kda`): scale,
lower_bound, chunk_size, initial_state, output_final_state; document boundaries
come as cu_seqlens (NeMo AutoModel page "nemo_automodel.components.models.
kimi_k3.cp").  Errors map as the pages raise them: malformed arguments ->
ValueError, unsupported shapes -> NotImplementedError, launch failures ->
RuntimeError.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
NUM_STAGES = 4
STAGE_NAMES = ("chunk_table", "prologue", "chunk_factors", "state_pass")
# stages of kda_bwd_profiled, in launch order (KDA_BWD_NUM_STAGES)
BWD_NUM_STAGES = 7
BWD_STAGE_NAMES = ("chunk_table", "recompute", "forward_states", "reverse_states",
                   "chunk_gradients", "dq_dk", "param_sums")
EXPORTED = ("kda_validate", "kda_fwd_workspace_size", "kda_fwd", "kda_fwd_profiled",
            "kda_state_summary_workspace_size", "kda_state_summary",
            "kda_apply_state_summary", "kda_chunk_capacity", "kda_chunk_table",
            "kda_short_conv_silu", "kda_fwd_short_conv_workspace_size", "kda_fwd_short_conv",
            "kda_bwd_workspace_size", "kda_bwd", "kda_bwd_profiled", "kda_gated_rms_norm",
            "kda_last_error", "kda_version", "kda_fwd_path", "kda_fwd_noalloc",
            "kda_fwd_noalloc_scratch_bytes", "kda_fwd_gated_norm",
            "kda_fwd_gated_norm_workspace_size")
MAX_CONV_WIDTH = 4


class KdaProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("lower_bound", ctypes.c_float),
                ("chunk_size", ctypes.c_int32), ("N", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
                ("lower_bound_form", ctypes.c_int32), ("HV", ctypes.c_int32)]

class KdaShortConv(ctypes.Structure):
    _fields_ = [("width", ctypes.c_int32),
                ("q_weight", ctypes.c_void_p), ("k_weight", ctypes.c_void_p),
                ("v_weight", ctypes.c_void_p), ("q_bias", ctypes.c_void_p),
                ("k_bias", ctypes.c_void_p), ("v_bias", ctypes.c_void_p)]


class KdaOutputNorm(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("activation", ctypes.c_int32)]


# form of the lower-bounded gate (kda_lower_bound_form)
LOWER_BOUND_FORMS = {"sigmoid": 0, "clamp": 1}


_lib = None


def load_library(path: Optional[str] = None):
    """Load libkda.so (once).  Raises ImportError when it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError("libkda.so is not built (expected at %s); run "
                          "`python -c 'import __graft_entry__ as g; g.build()'`" % path)
    lib = ctypes.CDLL(path)
    P, S, I32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    PP = ctypes.POINTER(KdaProblem)
    PI = ctypes.POINTER(ctypes.c_int)
    lib.kda_validate.argtypes = [PP]
    lib.kda_validate.restype = ctypes.c_int
    lib.kda_fwd_workspace_size.argtypes = [PP, PI]
    lib.kda_fwd_workspace_size.restype = S
    lib.kda_state_summary_workspace_size.argtypes = [PP, PI]
    lib.kda_state_summary_workspace_size.restype = S
    lib.kda_fwd.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.kda_fwd.restype = ctypes.c_int
    lib.kda_fwd_profiled.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, S, P, P]
    lib.kda_fwd_profiled.restype = ctypes.c_int
    lib.kda_state_summary.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.kda_state_summary.restype = ctypes.c_int
    lib.kda_apply_state_summary.argtypes = [I32, I32, I32, I32, P, P, P, P, P]
    lib.kda_apply_state_summary.restype = ctypes.c_int
    lib.kda_chunk_capacity.argtypes = [PP, PI]
    lib.kda_chunk_capacity.restype = I32
    lib.kda_chunk_table.argtypes = [PP, P, P, P, P, I32, P]
    lib.kda_chunk_table.restype = ctypes.c_int
    lib.kda_short_conv_silu.argtypes = [PP, I32, I32, P, P, P, P, P]
    lib.kda_short_conv_silu.restype = ctypes.c_int
    lib.kda_fwd_short_conv_workspace_size.argtypes = [PP, PI]
    lib.kda_fwd_short_conv_workspace_size.restype = S
    lib.kda_fwd_short_conv.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.kda_fwd_short_conv.restype = ctypes.c_int
    lib.kda_bwd_workspace_size.argtypes = [PP, PI]
    lib.kda_bwd_workspace_size.restype = S
    lib.kda_bwd.argtypes = [PP] + [P] * 18 + [P, S, P]
    lib.kda_bwd.restype = ctypes.c_int
    lib.kda_bwd_profiled.argtypes = [PP] + [P] * 18 + [P, S, P, P]
    lib.kda_bwd_profiled.restype = ctypes.c_int
    lib.kda_gated_rms_norm.argtypes = [PP, P, P, P, ctypes.c_float, I32, P, P]
    lib.kda_gated_rms_norm.restype = ctypes.c_int
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_fwd_gated_norm.argtypes = [PP, ctypes.POINTER(KdaOutputNorm)] + [P] * 11 + [S, P]
    lib.kda_fwd_gated_norm.restype = ctypes.c_int
    lib.kda_fwd_gated_norm_workspace_size.argtypes = [PP, PI]
    lib.kda_fwd_gated_norm_workspace_size.restype = S
    lib.kda_fwd_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P]
    lib.kda_fwd_noalloc.restype = ctypes.c_int
    lib.kda_fwd_noalloc_scratch_bytes.argtypes = []
    lib.kda_fwd_noalloc_scratch_bytes.restype = S
    lib.kda_fwd_path.argtypes = [PP]
    lib.kda_fwd_path.restype = I32
    lib.kda_version.argtypes = []
    lib.kda_version.restype = I32
    if path == LIB_PATH:
        _lib = lib
    return lib


def _raise(st: int, what: str):
    msg = "%s: %s" % (what, load_library().kda_last_error().decode())
    if st == EUNSUPPORTED:
        raise NotImplementedError(msg)
    if st == EHIP:
        raise RuntimeError(msg)
    raise ValueError(msg)


def _nan() -> float:
    return float("nan")


def make_problem(B, T, H, K, V, dtype, scale=None, lower_bound=None, chunk_size=64, N=None,
                 cu_seqlens_ptr=None, cu_seqlens_host_ptr=None, lower_bound_form="sigmoid",
                 HV=0) -> KdaProblem:
    if lower_bound_form not in LOWER_BOUND_FORMS:
        raise ValueError("lower_bound_form must be one of %s, got %r"
                         % (sorted(LOWER_BOUND_FORMS), lower_bound_form))
    p = KdaProblem()
    p.B, p.T, p.H, p.K, p.V = B, T, H, K, V
    p.dtype = dtype
    p.scale = 0.0 if scale is None else float(scale)
    p.lower_bound = _nan() if lower_bound is None else float(lower_bound)
    p.chunk_size = chunk_size
    p.N = B if N is None else N
    p.cu_seqlens = cu_seqlens_ptr
    p.cu_seqlens_host = cu_seqlens_host_ptr
    p.lower_bound_form = LOWER_BOUND_FORMS[lower_bound_form]
    p.HV = HV
    return p


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KDA_F32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    raise NotImplementedError("KDA inputs must be float32 or bfloat16, got %s" % t.dtype)


def _dev(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor, got device %s" % (name, t.device))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device):
    if nbytes == 0:
        return None, 0
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nbytes], nbytes


def _check_inputs(q, k, v, gate, beta, a_log, dt_bias):
    """Shapes of the projected inputs, against one table derived from q and v.

    The contract is the one the hyper_parallel coverage page checks in
    `_validate_projected_inputs`: q and k [B, T, H, K], v [B, T, HV, V],
    gate [B, T, HV, K], beta [B, T, HV], a_log HV values and dt_bias HV*K
    values, with HV a multiple of H.  Returns (B, T, H, K, V, HV)."""
    for name, t, rank in (("q", q, 4), ("k", k, 4), ("v", v, 4), ("gate", gate, 4),
                          ("beta", beta, 3)):
        if not isinstance(t, torch.Tensor) or t.dim() != rank:
            got = tuple(t.shape) if isinstance(t, torch.Tensor) else type(t).__name__
            raise ValueError("%s: expected a rank-%d tensor, got %s" % (name, rank, got))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    expected = (("k", k.shape, (B, T, H, K)),
                ("v (rows, tokens)", v.shape[:2], (B, T)),
                ("gate", gate.shape, (B, T, HV, K)),
                ("beta", beta.shape, (B, T, HV)))
    for name, got, want in expected:
        if tuple(got) != want:
            raise ValueError("%s: shape %s does not fit q %s and v %s (expected %s)"
                             % (name, tuple(got), tuple(q.shape), tuple(v.shape), want))
    if HV % H != 0:
        raise ValueError("v has %d value heads, not a multiple of the %d key heads of q and k"
                         % (HV, H))
    for name, t, count in (("a_log", a_log, HV), ("dt_bias", dt_bias, HV * K)):
        if not isinstance(t, torch.Tensor) or t.numel() != count:
            got = t.numel() if isinstance(t, torch.Tensor) else type(t).__name__
            raise ValueError("%s: expected %d values (%d value heads), got %s" % (name, count, HV, got))
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("beta", beta)):
        _dev(t, name, dtype=dt)
    _dtype_code(q)
    _dev(a_log, "a_log", dtype=torch.float32)
    _dev(dt_bias, "dt_bias", dtype=torch.float32)
    return B, T, H, K, V, HV


def _cu_args(cu_seqlens, cu_seqlens_host, T):
    if cu_seqlens is None:
        if cu_seqlens_host is not None:
            raise ValueError("cu_seqlens_host given without cu_seqlens")
        return None, None, None, None
    _dev(cu_seqlens, "cu_seqlens", dtype=torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of N+1 offsets")
    N = cu_seqlens.numel() - 1
    if cu_seqlens_host is None or cu_seqlens_host is False:
        # device offsets only: nothing waits for the GPU; the library sizes the
        # launch from an upper bound of the chunk count and clamps the offsets
        return cu_seqlens, None, N, None
    host = torch.as_tensor(cu_seqlens_host, dtype=torch.int32, device="cpu").contiguous()
    if host.numel() != N + 1:
        raise ValueError("cu_seqlens_host must hold the same N+1 offsets as cu_seqlens")
    return cu_seqlens, host, N, host.data_ptr()


PATH_NAMES = {0: "valu", 1: "mfma", 2: "fused"}


def fwd_path(q_shape, V, dtype=torch.bfloat16, chunk_size=64, N=None, HV=0, cu_seqlens=False) -> str:
    """Name of the kernel path kda_fwd takes for this problem: "valu",
    "mfma" (two passes with workspace records) or "fused"."""
    B, T, H, K = q_shape
    p = make_problem(B, T, H, K, V, KDA_F32 if dtype == torch.float32 else KDA_BF16,
                     chunk_size=chunk_size, N=N, cu_seqlens_ptr=1 if cu_seqlens else None, HV=HV)
    r = load_library().kda_fwd_path(ctypes.byref(p))
    if r < 0:
        _raise(EINVAL, "kda_fwd_path")
    return PATH_NAMES[r]


def fwd_workspace_size(q_shape, V, dtype=torch.bfloat16, chunk_size=64, lower_bound=None,
                       N=None, cu_seqlens_host=None, HV=0) -> int:
    B, T, H, K = q_shape
    host = None if cu_seqlens_host is None else torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    p = make_problem(B, T, H, K, V, KDA_F32 if dtype == torch.float32 else KDA_BF16,
                     lower_bound=lower_bound, chunk_size=chunk_size,
                     N=(host.numel() - 1) if host is not None else N,
                     cu_seqlens_ptr=1 if host is not None else None,
                     cu_seqlens_host_ptr=host.data_ptr() if host is not None else None, HV=HV)
    st = ctypes.c_int(0)
    n = load_library().kda_fwd_workspace_size(ctypes.byref(p), ctypes.byref(st))
    if st.value:
        _raise(st.value, "kda_fwd_workspace_size")
    return int(n)


def kda_fwd(q, k, v, gate, beta, a_log, dt_bias, *, scale=None, lower_bound=None,
            chunk_size=64, cu_seqlens=None, cu_seqlens_host=None, initial_state=None,
            output_final_state=False, out=None, workspace=None, stage_events=None,
            lower_bound_form="sigmoid"):
    """Chunked KDA forward; returns (o, final_state or None).

    q, k [B,T,H,K]; gate [B,T,HV,K]; v [B,T,HV,V]; beta [B,T,HV] (float32 or
    bfloat16, one dtype; HV a multiple of H, value head j reading key head
    j // (HV/H)); a_log [HV] and dt_bias [HV,K] float32; cu_seqlens int32 [N+1]
    on the GPU with B == 1; initial_state float32 [N,HV,K,V].
    ``lower_bound_form`` ("sigmoid" or "clamp") picks the form of the
    lower-bounded gate when lower_bound is given.  ``cu_seqlens_host`` may
    carry a CPU copy of the offsets: they are then validated on the host and
    the launch is sized exactly.  Without it (None, or False) nothing waits
    for the GPU: the launch is sized from an upper bound of the chunk count
    and the library clamps malformed device offsets into range (results are
    then unspecified).  ``stage_events`` is an
    optional ctypes array of 2*NUM_STAGES hipEvent_t handles recorded around
    each stage (see kda_fwd_profiled in include/kda.h).
    """
    return _fwd(q, k, v, gate, beta, a_log, dt_bias, None, scale, lower_bound, chunk_size,
                cu_seqlens, cu_seqlens_host, initial_state, output_final_state, out, workspace,
                stage_events, lower_bound_form)


def kda_fwd_gated_norm(q, k, v, gate, beta, a_log, dt_bias, norm_gate, norm_weight=None, *,
                       eps=1e-5, activation="sigmoid", scale=None, lower_bound=None,
                       chunk_size=64, cu_seqlens=None, cu_seqlens_host=None, initial_state=None,
                       output_final_state=False, out=None, workspace=None,
                       lower_bound_form="sigmoid"):
    """The forward followed by the gated output norm, in one call
    (kda_fwd_gated_norm): returns (y, final_state or None) with
    y = o / sqrt(mean_V(o^2) + eps) * norm_weight * act(norm_gate) per
    (token, value head) row, o being kda_fwd's output (never stored).
    norm_gate [B,T,HV,V] in the inputs' dtype; norm_weight float32 [V] or None;
    activation "sigmoid" or "silu".  Other arguments as kda_fwd."""
    if activation not in NORM_ACTIVATIONS:
        raise ValueError("activation must be one of %s, got %r" % (sorted(NORM_ACTIVATIONS), activation))
    B, T, H, K, V, HV = _check_inputs(q, k, v, gate, beta, a_log, dt_bias)
    _dev(norm_gate, "norm_gate", dtype=q.dtype, shape=(B, T, HV, V))
    if norm_weight is not None:
        _dev(norm_weight, "norm_weight", dtype=torch.float32, shape=(V,))
    nrm = KdaOutputNorm()
    nrm.gate = norm_gate.data_ptr()
    nrm.weight = None if norm_weight is None else norm_weight.data_ptr()
    nrm.eps = float(eps)
    nrm.activation = NORM_ACTIVATIONS[activation]
    lib = load_library()
    device = q.device
    cu, host, N, host_ptr = _cu_args(cu_seqlens, cu_seqlens_host, T)
    if N is None:
        N = B
    if initial_state is not None:
        _dev(initial_state, "initial_state", dtype=torch.float32, shape=(N, HV, K, V))
    if scale is not None and not scale > 0:
        raise ValueError("scale must be positive, got %r" % (scale,))
    p = make_problem(B, T, H, K, V, _dtype_code(q), scale, lower_bound, chunk_size, N,
                     None if cu is None else cu.data_ptr(), host_ptr, lower_bound_form, HV)
    st = ctypes.c_int(0)
    need = lib.kda_fwd_gated_norm_workspace_size(ctypes.byref(p), ctypes.byref(st))
    if st.value:
        _raise(st.value, "kda_fwd_gated_norm")
    y = out if out is not None else torch.empty((B, T, HV, V), dtype=q.dtype, device=device)
    _dev(y, "out", dtype=q.dtype, shape=(B, T, HV, V))
    fin = torch.empty((N, HV, K, V), dtype=torch.float32, device=device) if output_final_state else None
    if workspace is None:
        ws, nbytes = _workspace(need, device)
    else:
        _dev(workspace, "workspace", dtype=torch.uint8)
        ws, nbytes = workspace, workspace.numel()
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.kda_fwd_gated_norm(ctypes.byref(p), ctypes.byref(nrm), ptr(q), ptr(k), ptr(v),
                                ptr(gate), ptr(beta), ptr(a_log), ptr(dt_bias),
                                ptr(initial_state), ptr(y), ptr(fin), ptr(ws), nbytes,
                                _stream_ptr(device))
    if st:
        _raise(st, "kda_fwd_gated_norm")
    return y, fin


def kda_fwd_noalloc(q, k, v, gate, beta, a_log, dt_bias, *, scale=None, lower_bound=None,
                    chunk_size=64, cu_seqlens=None, cu_seqlens_host=None, initial_state=None,
                    out=None, final_state_out=None, lower_bound_form="sigmoid"):
    """kda_fwd through the allocation-free entry point (kda_fwd_noalloc).

    The library allocates nothing; the caller passes the outputs: ``out``
    (o, [B,T,HV,V], required) and ``final_state_out`` (float32 [N,HV,K,V] or
    None).  Returns (out, final_state_out).  The library's device scratch
    array is shared by every call on one GPU: calls that overlap on one GPU race."""
    B, T, H, K, V, HV = _check_inputs(q, k, v, gate, beta, a_log, dt_bias)
    cu, host, N, host_ptr = _cu_args(cu_seqlens, cu_seqlens_host, T)
    if N is None:
        N = B
    if initial_state is not None:
        _dev(initial_state, "initial_state", dtype=torch.float32, shape=(N, HV, K, V))
    if scale is not None and not scale > 0:
        raise ValueError("scale must be positive, got %r" % (scale,))
    if out is None:
        raise ValueError("kda_fwd_noalloc needs the output tensor `out` (it allocates nothing)")
    _dev(out, "out", dtype=q.dtype, shape=(B, T, HV, V))
    if final_state_out is not None:
        _dev(final_state_out, "final_state_out", dtype=torch.float32, shape=(N, HV, K, V))
    p = make_problem(B, T, H, K, V, _dtype_code(q), scale, lower_bound, chunk_size, N,
                     None if cu is None else cu.data_ptr(), host_ptr, lower_bound_form, HV)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = load_library().kda_fwd_noalloc(ctypes.byref(p), ptr(q), ptr(k), ptr(v), ptr(gate),
                                        ptr(beta), ptr(a_log), ptr(dt_bias), ptr(initial_state),
                                        ptr(out), ptr(final_state_out), _stream_ptr(q.device))
    if st:
        _raise(st, "kda_fwd_noalloc")
    return out, final_state_out


def kda_fwd_short_conv(q, k, v, gate, beta, a_log, dt_bias, conv_weights=None, conv_biases=None,
                       *, scale=None, lower_bound=None, chunk_size=64, cu_seqlens=None,
                       cu_seqlens_host=None, initial_state=None, output_final_state=False,
                       out=None, workspace=None, lower_bound_form="sigmoid"):
    """kda_fwd after the layer's short convolution and SiLU on q, k and v.

    q, k, v are the raw projections.  conv_weights: None (SiLU alone) or
    (w_q, w_k, w_v), float32 GPU tensors [channels, W] or [channels, 1, W]
    (channels H*K for q and k, HV*V for v; 1 <= W <= MAX_CONV_WIDTH);
    conv_biases: None or (b_q, b_k, b_v), each [channels] or None.  The other
    arguments are those of kda_fwd."""
    B, T, H, K, V, HV = _check_inputs(q, k, v, gate, beta, a_log, dt_bias)
    conv = _conv_spec(conv_weights, conv_biases, (H * K, H * K, HV * V))
    return _fwd(q, k, v, gate, beta, a_log, dt_bias, conv, scale, lower_bound, chunk_size,
                cu_seqlens, cu_seqlens_host, initial_state, output_final_state, out, workspace,
                None, lower_bound_form)


def _conv_weight(w, C, name):
    _dev(w, name, dtype=torch.float32)
    if w.dim() == 3 and w.shape[1] == 1:
        w = w.reshape(w.shape[0], w.shape[2])
    if w.dim() != 2 or w.shape[0] != C:
        raise ValueError("%s must be [%d, W] or [%d, 1, W], got %s" % (name, C, C, tuple(w.shape)))
    return w


def _conv_spec(conv_weights, conv_biases, channels):
    """A KdaShortConv (plus the tensors it points to, kept alive with it)."""
    spec = KdaShortConv()
    keep = []
    if conv_weights is None:
        if conv_biases is not None:
            raise ValueError("conv_biases given without conv_weights")
        spec.width = 0
        return spec, keep
    if len(conv_weights) != 3:
        raise ValueError("conv_weights must be (w_q, w_k, w_v)")
    ws = [_conv_weight(w, C, n) for w, C, n in zip(conv_weights, channels, ("w_q", "w_k", "w_v"))]
    widths = {w.shape[1] for w in ws}
    if len(widths) != 1:
        raise ValueError("q, k and v convolutions must have one width, got %s" % sorted(widths))
    spec.width = widths.pop()
    spec.q_weight, spec.k_weight, spec.v_weight = (w.data_ptr() for w in ws)
    keep += ws
    if conv_biases is not None:
        if len(conv_biases) != 3:
            raise ValueError("conv_biases must be (b_q, b_k, b_v)")
        ptrs = []
        for b, C, n in zip(conv_biases, channels, ("b_q", "b_k", "b_v")):
            if b is None:
                ptrs.append(None)
                continue
            _dev(b, n, dtype=torch.float32, shape=(C,))
            keep.append(b)
            ptrs.append(b.data_ptr())
        spec.q_bias, spec.k_bias, spec.v_bias = ptrs
    return spec, keep


def short_conv_silu(x, weight=None, bias=None, *, cu_seqlens=None, cu_seqlens_host=None, out=None):
    """SiLU of the causal depthwise convolution of x over time (one tensor).

    x [B,T,C] or [B,T,H,D] (channel h*D + d), float32 or bfloat16 on the GPU;
    weight float32 [C, W] or [C, 1, W] (None: SiLU alone); bias float32 [C] or
    None.  With cu_seqlens (B == 1) every document is padded on its own."""
    if not isinstance(x, torch.Tensor) or x.dim() < 3:
        raise ValueError("x must be a [B, T, ...] tensor")
    _dev(x, "x")
    B, T = x.shape[0], x.shape[1]
    C = 1
    for d in x.shape[2:]:
        C *= d
    width = 0
    if weight is not None:
        weight = _conv_weight(weight, C, "weight")
        width = weight.shape[1]
    elif bias is not None:
        raise ValueError("bias given without weight")
    if bias is not None:
        _dev(bias, "bias", dtype=torch.float32, shape=(C,))
    cu, host, N, host_ptr = _cu_args(cu_seqlens, cu_seqlens_host, T)
    if N is None:
        N = B
    p = make_problem(B, T, 0, 0, 0, _dtype_code(x), N=N,
                     cu_seqlens_ptr=None if cu is None else cu.data_ptr(),
                     cu_seqlens_host_ptr=host_ptr)
    y = torch.empty_like(x) if out is None else out
    _dev(y, "out", dtype=x.dtype, shape=tuple(x.shape))
    ptr = lambda t: None if t is None else t.data_ptr()
    st = load_library().kda_short_conv_silu(ctypes.byref(p), C, width, ptr(x), ptr(weight),
                                            ptr(bias), ptr(y), _stream_ptr(x.device))
    if st:
        _raise(st, "kda_short_conv_silu")
    return y


def _fwd(q, k, v, gate, beta, a_log, dt_bias, conv, scale, lower_bound, chunk_size, cu_seqlens,
         cu_seqlens_host, initial_state, output_final_state, out, workspace, stage_events,
         lower_bound_form):
    B, T, H, K, V, HV = _check_inputs(q, k, v, gate, beta, a_log, dt_bias)
    lib = load_library()
    device = q.device
    cu, host, N, host_ptr = _cu_args(cu_seqlens, cu_seqlens_host, T)
    if N is None:
        N = B
    if initial_state is not None:
        _dev(initial_state, "initial_state", dtype=torch.float32, shape=(N, HV, K, V))
    if scale is not None and not scale > 0:
        raise ValueError("scale must be positive, got %r" % (scale,))
    p = make_problem(B, T, H, K, V, _dtype_code(q), scale, lower_bound, chunk_size, N,
                     None if cu is None else cu.data_ptr(), host_ptr, lower_bound_form, HV)
    st = ctypes.c_int(0)
    size_fn = lib.kda_fwd_workspace_size if conv is None else lib.kda_fwd_short_conv_workspace_size
    need = size_fn(ctypes.byref(p), ctypes.byref(st))
    if st.value:
        _raise(st.value, "kda_fwd")
    o = out if out is not None else torch.empty((B, T, HV, V), dtype=q.dtype, device=device)
    _dev(o, "out", dtype=q.dtype, shape=(B, T, HV, V))
    fin = torch.empty((N, HV, K, V), dtype=torch.float32, device=device) if output_final_state else None
    if workspace is None:
        ws, nbytes = _workspace(need, device)
    else:
        _dev(workspace, "workspace", dtype=torch.uint8)
        ws, nbytes = workspace, workspace.numel()
    ptr = lambda t: None if t is None else t.data_ptr()
    if conv is None:
        st = lib.kda_fwd_profiled(ctypes.byref(p), ptr(q), ptr(k), ptr(v), ptr(gate), ptr(beta),
                                  ptr(a_log), ptr(dt_bias), ptr(initial_state), ptr(o), ptr(fin),
                                  ptr(ws), nbytes, _stream_ptr(device), stage_events)
    else:
        spec, _keep = conv
        st = lib.kda_fwd_short_conv(ctypes.byref(p), ctypes.byref(spec), ptr(q), ptr(k), ptr(v),
                                    ptr(gate), ptr(beta), ptr(a_log), ptr(dt_bias),
                                    ptr(initial_state), ptr(o), ptr(fin), ptr(ws), nbytes,
                                    _stream_ptr(device))
    if st:
        _raise(st, "kda_fwd_short_conv" if conv is not None else "kda_fwd")
    return o, fin


def kda_bwd(q, k, v, gate, beta, a_log, dt_bias, d_o, d_final_state=None, *, scale=None,
            lower_bound=None, chunk_size=64, cu_seqlens=None, cu_seqlens_host=None,
            initial_state=None, lower_bound_form="sigmoid", workspace=None, stage_events=None):
    """Gradients of L = sum(d_o * o) + sum(d_final_state * final_state) of kda_fwd
    with the same arguments.  Returns a dict: dq, dk [B,T,H,K], dv [B,T,HV,V],
    dgate [B,T,HV,K], dbeta [B,T,HV] (of the logits; q's dtype), da_log [HV],
    ddt_bias [HV,K] and dinit [N,HV,K,V] (float32).  `stage_events`: optional
    ctypes array of 2*BWD_NUM_STAGES hipEvent_t handles recorded around each
    stage (kda_bwd_profiled)."""
    B, T, H, K, V, HV = _check_inputs(q, k, v, gate, beta, a_log, dt_bias)
    lib = load_library()
    device = q.device
    _dev(d_o, "d_o", dtype=q.dtype, shape=(B, T, HV, V))
    cu, host, N, host_ptr = _cu_args(cu_seqlens, cu_seqlens_host, T)
    if N is None:
        N = B
    if initial_state is not None:
        _dev(initial_state, "initial_state", dtype=torch.float32, shape=(N, HV, K, V))
    if d_final_state is not None:
        _dev(d_final_state, "d_final_state", dtype=torch.float32, shape=(N, HV, K, V))
    if scale is not None and not scale > 0:
        raise ValueError("scale must be positive, got %r" % (scale,))
    p = make_problem(B, T, H, K, V, _dtype_code(q), scale, lower_bound, chunk_size, N,
                     None if cu is None else cu.data_ptr(), host_ptr, lower_bound_form, HV)
    st = ctypes.c_int(0)
    need = lib.kda_bwd_workspace_size(ctypes.byref(p), ctypes.byref(st))
    if st.value:
        _raise(st.value, "kda_bwd")
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dgate=torch.empty_like(gate), dbeta=torch.empty_like(beta),
               da_log=torch.empty(HV, dtype=torch.float32, device=device),
               ddt_bias=torch.empty(HV, K, dtype=torch.float32, device=device),
               dinit=torch.empty(N, HV, K, V, dtype=torch.float32, device=device))
    if workspace is None:
        ws, nbytes = _workspace(need, device)
    else:
        _dev(workspace, "workspace", dtype=torch.uint8)
        ws, nbytes = workspace, workspace.numel()
    ptr = lambda t: None if t is None else t.data_ptr()
    args = (ctypes.byref(p), ptr(q), ptr(k), ptr(v), ptr(gate), ptr(beta), ptr(a_log),
            ptr(dt_bias), ptr(initial_state), ptr(d_o), ptr(d_final_state),
            ptr(out["dq"]), ptr(out["dk"]), ptr(out["dv"]), ptr(out["dgate"]),
            ptr(out["dbeta"]), ptr(out["da_log"]), ptr(out["ddt_bias"]), ptr(out["dinit"]),
            ptr(ws), nbytes, _stream_ptr(device))
    if stage_events is None:
        st = lib.kda_bwd(*args)
    else:
        st = lib.kda_bwd_profiled(*args, stage_events)
    if st:
        _raise(st, "kda_bwd")
    return out


NORM_ACTIVATIONS = {"sigmoid": 0, "silu": 1}


def gated_rms_norm(o, gate, weight=None, *, eps=1e-5, activation="sigmoid", out=None):
    """The gated output norm after the forward: per [..., V] row,
    o / sqrt(mean(o^2) + eps) * weight * act(gate), act = sigmoid or SiLU.
    o, gate [B, T, HV, V] (float32 or bfloat16, GPU); weight float32 [V] or None."""
    if activation not in NORM_ACTIVATIONS:
        raise ValueError("activation must be one of %s, got %r" % (sorted(NORM_ACTIVATIONS), activation))
    if not isinstance(o, torch.Tensor) or o.dim() != 4:
        raise ValueError("o must be a [B, T, HV, V] tensor")
    _dev(o, "o")
    _dev(gate, "gate", dtype=o.dtype, shape=tuple(o.shape))
    B, T, HV, V = o.shape
    if weight is not None:
        _dev(weight, "weight", dtype=torch.float32, shape=(V,))
    p = make_problem(B, T, HV, 0, V, _dtype_code(o))
    y = torch.empty_like(o) if out is None else out
    _dev(y, "out", dtype=o.dtype, shape=tuple(o.shape))
    ptr = lambda t: None if t is None else t.data_ptr()
    st = load_library().kda_gated_rms_norm(ctypes.byref(p), ptr(o), ptr(gate), ptr(weight),
                                           float(eps), NORM_ACTIVATIONS[activation], ptr(y),
                                           _stream_ptr(o.device))
    if st:
        _raise(st, "kda_gated_rms_norm")
    return y


def kda_state_summary(q, k, v, gate, beta, a_log, dt_bias, *, lower_bound=None, chunk_size=64,
                      workspace=None, lower_bound_form="sigmoid"):
    """Affine summary of each row: (state_ext [B,HV,K,V], transition [B,HV,K,K]), float32."""
    B, T, H, K, V, HV = _check_inputs(q, k, v, gate, beta, a_log, dt_bias)
    lib = load_library()
    device = q.device
    p = make_problem(B, T, H, K, V, _dtype_code(q), None, lower_bound, chunk_size, B,
                     lower_bound_form=lower_bound_form, HV=HV)
    st = ctypes.c_int(0)
    need = lib.kda_state_summary_workspace_size(ctypes.byref(p), ctypes.byref(st))
    if st.value:
        _raise(st.value, "kda_state_summary")
    E = torch.empty((B, HV, K, V), dtype=torch.float32, device=device)
    P = torch.empty((B, HV, K, K), dtype=torch.float32, device=device)
    if workspace is None:
        ws, nbytes = _workspace(need, device)
    else:
        ws, nbytes = workspace, workspace.numel()
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.kda_state_summary(ctypes.byref(p), ptr(q), ptr(k), ptr(v), ptr(gate), ptr(beta),
                               ptr(a_log), ptr(dt_bias), ptr(E), ptr(P), ptr(ws), nbytes,
                               _stream_ptr(device))
    if st:
        _raise(st, "kda_state_summary")
    return E, P


def kda_apply_state_summary(state_ext, transition, initial_state=None, out=None):
    """final = transition . initial_state + state_ext (state_ext when initial_state is None)."""
    _dev(state_ext, "state_ext", dtype=torch.float32)
    if state_ext.dim() != 4:
        raise ValueError("state_ext must be [B,H,K,V]")
    B, H, K, V = state_ext.shape
    _dev(transition, "transition", dtype=torch.float32, shape=(B, H, K, K))
    if initial_state is not None:
        _dev(initial_state, "initial_state", dtype=torch.float32, shape=(B, H, K, V))
    out = torch.empty_like(state_ext) if out is None else out
    _dev(out, "out", dtype=torch.float32, shape=(B, H, K, V))
    ptr = lambda t: None if t is None else t.data_ptr()
    st = load_library().kda_apply_state_summary(B, H, K, V, ptr(state_ext), ptr(transition),
                                                ptr(initial_state), ptr(out),
                                                _stream_ptr(state_ext.device))
    if st:
        _raise(st, "kda_apply_state_summary")
    return out


def chunk_table(T, chunk_size=64, cu_seqlens=None, B=1, cu_seqlens_host=None, device="cuda"):
    """The device chunk table: (tok, len, seq_chunk0) as CPU int32 tensors."""
    lib = load_library()
    cu, host, N, host_ptr = _cu_args(cu_seqlens, cu_seqlens_host, T)
    if N is None:
        N = B
    p = make_problem(B, T, 1, 64, 64, KDA_BF16, None, None, chunk_size, N,
                     None if cu is None else cu.data_ptr(), host_ptr)
    st = ctypes.c_int(0)
    cap = lib.kda_chunk_capacity(ctypes.byref(p), ctypes.byref(st))
    if st.value:
        _raise(st.value, "kda_chunk_capacity")
    dev = torch.device(device) if cu is None else cu.device
    tok = torch.full((max(cap, 1),), -1, dtype=torch.int32, device=dev)
    ln = torch.full((max(cap, 1),), -1, dtype=torch.int32, device=dev)
    seq0 = torch.full((N + 1,), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros((1,), dtype=torch.int32, device=dev)
    st = lib.kda_chunk_table(ctypes.byref(p), tok.data_ptr(), ln.data_ptr(), seq0.data_ptr(),
                             cnt.data_ptr(), cap, _stream_ptr(dev))
    if st:
        _raise(st, "kda_chunk_table")
    n = int(cnt.item())
    return tok[:n].cpu(), ln[:n].cpu(), seq0.cpu()
