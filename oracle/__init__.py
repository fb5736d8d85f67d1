"""Plain CPU oracle for the KDA forward (fp64 token-by-token recurrence).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers.  The product path (the
HIP library and its Python binding) never imports this package, and this
package imports nothing from the product.

The arithmetic lives in ``kda_oracle.c`` (compiled with gcc, loaded through
ctypes).  Every input is taken as a float64 array (bf16 and fp32 values upcast
exactly; the short convolution's fp64 output passes through unrounded, and
finite differences can perturb any input); outputs are float64.  See ``kda_oracle.c`` for the definition and the
passages of the pages each part follows.  ``chunked.py`` holds a second,
chunk-parallel fp64 form used only to cross-check the chunk algebra.

Pins: every public function here is checked by ``tests/test_oracle_*.py``
against brute-force matrix products, closed forms and invariants; the
alternative gate reading (``gate_mode="clamp"``) is pinned by closed forms of
its own gate values only.  ``short_conv_silu`` (the layer's causal depthwise
convolution and SiLU before the forward) is pinned by
``tests/test_oracle_short_conv.py`` against the library conv1d called the way
the pages call it, closed-form taps and SiLU special values.  ``kda_bwd`` (the
reverse mode of the token recurrence) is pinned by
``tests/test_oracle_bwd.py`` against central finite differences of the forward,
entry by entry, for every input, plus closed forms.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liboracle_kda.so")

GATE_MODES = {"softplus": 0, "sigmoid": 1, "clamp": 2}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        os.makedirs(os.path.dirname(_LIB), exist_ok=True)
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        lib.oracle_prologue.argtypes = [I, I, I, I, P, P, P, P, P, P, I, D, P, P, P, P]
        lib.oracle_kda_fwd.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, D, I, D, I, P, P, P, P, I]
        lib.oracle_recurrence.argtypes = [I, I, I, I, I, P, P, P, P, P, D, I, P, P, P, P, I]
        lib.oracle_state_summary.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, I, D, P, P, I]
        lib.oracle_apply_state_summary.argtypes = [I, I, I, I, P, P, P, P]
        lib.oracle_short_conv_silu.argtypes = [I, I, I, I, P, P, P, I, P, P]
        lib.oracle_kda_bwd.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, D, I, D, I, P, P, P, P,
                                       P, P, P, P, P, P, P, P, I]
        lib.oracle_gated_rms_norm.argtypes = [ctypes.c_long, I, P, P, P, D, I, P]
        for f in (lib.oracle_prologue, lib.oracle_kda_fwd, lib.oracle_recurrence,
                  lib.oracle_state_summary, lib.oracle_apply_state_summary,
                  lib.oracle_short_conv_silu, lib.oracle_kda_bwd, lib.oracle_gated_rms_norm):
            f.restype = I
        _lib = lib
    return _lib


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _gate(lower_bound, gate_mode):
    if gate_mode is None:
        gate_mode = "softplus" if lower_bound is None else "sigmoid"
    mode = GATE_MODES[gate_mode]
    if mode != 0 and (lower_bound is None or not lower_bound < 0):
        raise ValueError("lower_bound must be negative when a bounded gate is used")
    return mode, (0.0 if lower_bound is None else float(lower_bound))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def prologue(q, k, gate, beta, a_log, dt_bias, lower_bound=None, gate_mode=None):
    """q^, k^ (L2-normalised), log-decay g and beta = sigmoid(logit), all fp64."""
    q, k, gate, beta, a_log, dt_bias = map(_f64, (q, k, gate, beta, a_log, dt_bias))
    B, T, H, K = q.shape
    mode, lb = _gate(lower_bound, gate_mode)
    qn = np.empty(q.shape, np.float64)
    kn = np.empty(q.shape, np.float64)
    g = np.empty(q.shape, np.float64)
    b = np.empty(beta.shape, np.float64)
    rc = _load().oracle_prologue(B, T, H, K, _ptr(q), _ptr(k), _ptr(gate), _ptr(beta),
                                 _ptr(a_log), _ptr(dt_bias), mode, lb,
                                 _ptr(qn), _ptr(kn), _ptr(g), _ptr(b))
    if rc:
        raise ValueError("oracle_prologue rejected its arguments (%d)" % rc)
    return qn, kn, g, b


def _cu(cu_seqlens, B, T):
    if cu_seqlens is None:
        return None, B
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    return cu, cu.shape[0] - 1


def kda_fwd(q, k, v, gate, beta, a_log, dt_bias, scale=None, lower_bound=None,
            cu_seqlens=None, initial_state=None, output_final_state=True,
            gate_mode=None, threads=None, want_output=True):
    """Full KDA forward.  Returns (o [B,T,H,V] fp64 or None, final [N,H,K,V] fp64 or None).

    H is the number of value heads (v, gate, beta, a_log, dt_bias, o, states);
    q and k may have fewer key heads HK dividing H, value head h then reading
    key head h // (H // HK) (grouped value heads)."""
    q, k, v, gate, beta, a_log, dt_bias = map(_f64, (q, k, v, gate, beta, a_log, dt_bias))
    B, T, HK, K = q.shape
    H, V = v.shape[2], v.shape[-1]
    if H % HK:
        raise ValueError("value heads %d must be a multiple of key heads %d" % (H, HK))
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    mode, lb = _gate(lower_bound, gate_mode)
    cu, N = _cu(cu_seqlens, B, T)
    init = None if initial_state is None else _f64(initial_state)
    o = np.zeros((B, T, H, V), np.float64) if want_output else None
    fin = np.zeros((N, H, K, V), np.float64) if output_final_state else None
    rc = _load().oracle_kda_fwd(B, T, H, HK, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
                                _ptr(a_log), _ptr(dt_bias), float(scale), mode, lb, N, _ptr(cu),
                                _ptr(init), _ptr(o), _ptr(fin), threads or default_threads())
    if rc:
        raise ValueError("oracle_kda_fwd rejected its arguments (%d)" % rc)
    return o, fin


def recurrence(qn, kn, v, g, b, scale, cu_seqlens=None, initial_state=None, threads=None):
    """Token recurrence from already normalised inputs.  Returns (o, final_state)."""
    qn, kn, g, b, v = map(_f64, (qn, kn, g, b, v))
    B, T, H, K = qn.shape
    V = v.shape[-1]
    cu, N = _cu(cu_seqlens, B, T)
    init = None if initial_state is None else _f64(initial_state)
    o = np.zeros((B, T, H, V), np.float64)
    fin = np.zeros((N, H, K, V), np.float64)
    rc = _load().oracle_recurrence(B, T, H, K, V, _ptr(qn), _ptr(kn), _ptr(v), _ptr(g), _ptr(b),
                                   float(scale), N, _ptr(cu), _ptr(init), _ptr(o), _ptr(fin),
                                   threads or default_threads())
    if rc:
        raise ValueError("oracle_recurrence rejected its arguments (%d)" % rc)
    return o, fin


def state_summary(q, k, v, gate, beta, a_log, dt_bias, lower_bound=None, gate_mode=None,
                  threads=None):
    """Affine summary of each row: (state_ext [B,H,K,V], transition [B,H,K,K]), fp64.
    Heads as in kda_fwd (q, k may carry fewer key heads)."""
    q, k, v, gate, beta, a_log, dt_bias = map(_f64, (q, k, v, gate, beta, a_log, dt_bias))
    B, T, HK, K = q.shape
    H, V = v.shape[2], v.shape[-1]
    if H % HK:
        raise ValueError("value heads %d must be a multiple of key heads %d" % (H, HK))
    mode, lb = _gate(lower_bound, gate_mode)
    E = np.zeros((B, H, K, V), np.float64)
    P = np.zeros((B, H, K, K), np.float64)
    rc = _load().oracle_state_summary(B, T, H, HK, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                                      _ptr(beta), _ptr(a_log), _ptr(dt_bias), mode, lb,
                                      _ptr(E), _ptr(P), threads or default_threads())
    if rc:
        raise ValueError("oracle_state_summary rejected its arguments (%d)" % rc)
    return E, P


def apply_state_summary(state_ext, transition, initial_state=None):
    """final = transition . initial + state_ext (state_ext alone when initial is None)."""
    E = _f64(state_ext)
    P = _f64(transition)
    B, H, K, V = E.shape
    init = None if initial_state is None else _f64(initial_state)
    out = np.zeros_like(E)
    _load().oracle_apply_state_summary(B, H, K, V, _ptr(E), _ptr(P), _ptr(init), _ptr(out))
    return out


def short_conv_silu(x, weight=None, bias=None, cu_seqlens=None):
    """SiLU of the causal depthwise convolution of x over time, fp64.

    x [B,T,C] or [B,T,H,D] (channels h*D + d); weight [C,W] (or [C,1,W], the
    depthwise Conv1d weight) with tap W-1 on the current token; bias [C] or
    None.  weight None: SiLU alone.  Tokens before a sequence's first token
    (row start, or document start with cu_seqlens) count as zero."""
    x = _f64(x)
    shape = x.shape
    B, T = shape[0], shape[1]
    C = int(np.prod(shape[2:]))
    if weight is None:
        W, w = 0, None
    else:
        w = _f64(weight).reshape(C, -1)
        W = w.shape[1]
    b = None if bias is None else _f64(bias).reshape(C)
    cu, N = _cu(cu_seqlens, B, T)
    y = np.empty(shape, np.float64)
    rc = _load().oracle_short_conv_silu(B, T, C, W, _ptr(x), _ptr(w), _ptr(b), N, _ptr(cu), _ptr(y))
    if rc:
        raise ValueError("oracle_short_conv_silu rejected its arguments (%d)" % rc)
    return y


def kda_fwd_short_conv(q, k, v, gate, beta, a_log, dt_bias, conv_weights=None, conv_biases=None,
                       cu_seqlens=None, **kwargs):
    """kda_fwd after the layer's short convolution and SiLU on q, k and v.

    conv_weights: None (SiLU alone) or (w_q, w_k, w_v), each [channels, W];
    conv_biases: None or (b_q, b_k, b_v), entries may be None.  The remaining
    keyword arguments are those of kda_fwd."""
    wq, wk, wv = conv_weights if conv_weights is not None else (None, None, None)
    bq, bk, bv = conv_biases if conv_biases is not None else (None, None, None)
    q2 = short_conv_silu(q, wq, bq, cu_seqlens)
    k2 = short_conv_silu(k, wk, bk, cu_seqlens)
    v2 = short_conv_silu(v, wv, bv, cu_seqlens)
    return kda_fwd(q2, k2, v2, gate, beta, a_log, dt_bias, cu_seqlens=cu_seqlens, **kwargs)


def kda_bwd(q, k, v, gate, beta, a_log, dt_bias, d_o, d_final=None, scale=None, lower_bound=None,
            cu_seqlens=None, initial_state=None, gate_mode=None, threads=None):
    """Gradients of L = sum(d_o * o) + sum(d_final * final_state) for kda_fwd's
    inputs (reverse mode of the token recurrence, fp64).  Returns a dict with
    dq, dk ([B,T,HK,K], summed over the value heads that share a key head), dv,
    dgate, dbeta (of the logit), da_log, ddt_bias and dinit (the initial state's
    gradient, [N,H,K,V]; returned also when no initial state is given)."""
    q, k, v, gate, beta, a_log, dt_bias, d_o = map(_f64, (q, k, v, gate, beta, a_log, dt_bias, d_o))
    B, T, HK, K = q.shape
    H, V = v.shape[2], v.shape[-1]
    if H % HK:
        raise ValueError("value heads %d must be a multiple of key heads %d" % (H, HK))
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    mode, lb = _gate(lower_bound, gate_mode)
    cu, N = _cu(cu_seqlens, B, T)
    init = None if initial_state is None else _f64(initial_state)
    dfin = None if d_final is None else _f64(d_final)
    out = dict(dq=np.zeros(q.shape), dk=np.zeros(q.shape), dv=np.zeros(v.shape),
               dgate=np.zeros(gate.shape), dbeta=np.zeros(beta.shape), da_log=np.zeros(H),
               ddt_bias=np.zeros((H, K)), dinit=np.zeros((N, H, K, V)))
    rc = _load().oracle_kda_bwd(B, T, H, HK, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
                                _ptr(a_log), _ptr(dt_bias), float(scale), mode, lb, N, _ptr(cu),
                                _ptr(init), _ptr(d_o), _ptr(dfin), _ptr(out["dq"]), _ptr(out["dk"]),
                                _ptr(out["dv"]), _ptr(out["dgate"]), _ptr(out["dbeta"]),
                                _ptr(out["da_log"]), _ptr(out["ddt_bias"]), _ptr(out["dinit"]),
                                threads or default_threads())
    if rc:
        raise ValueError("oracle_kda_bwd rejected its arguments (%d)" % rc)
    return out


NORM_ACTIVATIONS = {"sigmoid": 0, "silu": 1}


def gated_rms_norm(o, gate, weight=None, eps=1e-5, activation="sigmoid"):
    """The gated output norm (fp64): per row of the last dimension V,
    o / sqrt(mean(o^2) + eps) * weight * act(gate), act = sigmoid or SiLU."""
    o, gate = _f64(o), _f64(gate)
    if o.shape != gate.shape:
        raise ValueError("o and gate must have one shape")
    V = o.shape[-1]
    R = o.size // V if V else 0
    w = None if weight is None else _f64(weight).reshape(V)
    y = np.empty(o.shape, np.float64)
    rc = _load().oracle_gated_rms_norm(R, V, _ptr(o), _ptr(gate), _ptr(w), float(eps),
                                       NORM_ACTIVATIONS[activation], _ptr(y))
    if rc:
        raise ValueError("oracle_gated_rms_norm rejected its arguments (%d)" % rc)
    return y
