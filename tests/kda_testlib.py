"""Shared helpers for the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare them to the stated tolerances.

Tolerances: fp32 inputs -> max-abs error <= 1e-4; bf16 inputs -> max-abs error
<= 2e-2 and relative Frobenius error <= 1e-2 (fp32 state in both cases)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from gated_delta_rule_43_amd import kda

FP32_ATOL = 1e-4
BF16_ATOL = 2e-2
BF16_RELF = 1e-2


def to_np(t):
    return None if t is None else t.detach().float().cpu().numpy()


def gpu_fwd(inp, output_final_state=True, **kw):
    args = dict(scale=inp.get("scale"), lower_bound=inp.get("lower_bound"),
                chunk_size=inp.get("chunk_size", 64), cu_seqlens=inp.get("cu_seqlens"),
                initial_state=inp.get("initial_state"), output_final_state=output_final_state,
                lower_bound_form=inp.get("lower_bound_form", "sigmoid"))
    args.update(kw)
    o, fin = kda.kda_fwd(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["a_log"],
                         inp["dt_bias"], **args)
    torch.cuda.synchronize()
    return o, fin


def oracle_fwd(inp, heads=None, rows=None, threads=None):
    """Oracle on (a head/row subset of) the same inputs; returns fp64 numpy arrays.
    A head subset needs q and k with as many heads as v (no grouping)."""
    sel_h = slice(None) if heads is None else list(heads)
    sel_b = slice(None) if rows is None else list(rows)

    def cut(name, kind):
        t = inp[name]
        if t is None:
            return None
        if kind == "bthx":
            t = t[sel_b][:, :, sel_h]
        elif kind == "bth":
            t = t[sel_b][:, :, sel_h]
        elif kind == "h":
            t = t[sel_h]
        elif kind == "nh":
            t = t[sel_b][:, sel_h] if inp.get("cu_seqlens") is None else t[:, sel_h]
        return to_np(t)

    cu = inp.get("cu_seqlens")
    return oracle.kda_fwd(cut("q", "bthx"), cut("k", "bthx"), cut("v", "bthx"), cut("gate", "bthx"),
                          cut("beta", "bth"), cut("a_log", "h"), cut("dt_bias", "h"),
                          scale=inp.get("scale"), lower_bound=inp.get("lower_bound"),
                          gate_mode="clamp" if inp.get("lower_bound_form") == "clamp" else None,
                          cu_seqlens=None if cu is None else cu.cpu().numpy(),
                          initial_state=cut("initial_state", "nh"), threads=threads)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    maxabs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    relf = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    return maxabs, relf


def assert_close(got, ref, dtype, what=""):
    maxabs, relf = errors(got, ref)
    if dtype == torch.float32:
        assert maxabs <= FP32_ATOL, "%s: max-abs %.3g > %.1g (fp32)" % (what, maxabs, FP32_ATOL)
    else:
        assert maxabs <= BF16_ATOL and relf <= BF16_RELF, \
            "%s: max-abs %.3g (<= %.0g), rel-Frobenius %.3g (<= %.0g)" % (what, maxabs, BF16_ATOL, relf, BF16_RELF)
    return maxabs, relf


def to_device(inp, device="cuda"):
    out = {}
    for key, val in inp.items():
        out[key] = val.to(device) if isinstance(val, torch.Tensor) else val
    return out
