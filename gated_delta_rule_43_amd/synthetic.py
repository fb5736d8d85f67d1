"""Seeded synthetic inputs for the KDA forward.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic, and both the oracle-side tests and the GPU path take their
inputs from it.

Recipe (no public dataset stands behind these workloads; the shapes and value
distributions are the ones the five workload descriptions state):

* a config with seed ``s`` draws, in this order and as float32 from
  ``torch.Generator(device).manual_seed(s)``: q, k, v, gate, beta, a_log,
  dt_bias, initial_state (the last only when the config carries one);
* the float32 draws are then cast to the config's dtype (bf16 or fp32);
  a_log, dt_bias and initial_state stay float32;
* document lengths come from ``numpy.random.default_rng(s)``.

``device`` may be "cpu" or a CUDA/HIP device; the draws differ between the
two generators but both sides of every comparison read the same tensors.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    K: int
    V: int
    dtype: str                 # "f32" or "bf16"
    seed: int
    chunk_size: int = 64
    scale: Optional[float] = None
    lower_bound: Optional[float] = None
    gate_std: float = 1.0
    beta_std: float = 1.0
    init_std: Optional[float] = None   # None: no initial state
    lengths: str = "rows"              # "rows" | "composition7" | "short1to100"
    output_final_state: bool = True

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


# The five workloads: tiny fp32, packed varlen, throughput, long carried slice,
# gating/boundary stress.
WORKLOADS = {
    1: Workload("tiny_fp32_T256_H2_d64", B=1, T=256, H=2, K=64, V=64, dtype="f32", seed=1001,
                scale=1.0 / 8.0),
    2: Workload("packed_varlen_bf16_T8192_7docs_H16_d128", B=1, T=8192, H=16, K=128, V=128,
                dtype="bf16", seed=1002, lengths="composition7"),
    3: Workload("throughput_bf16_B4_T16384_H32_d128", B=4, T=16384, H=32, K=128, V=128,
                dtype="bf16", seed=1003),
    4: Workload("long_slice_bf16_T131072_H32_d128_carried_state", B=1, T=131072, H=32, K=128,
                V=128, dtype="bf16", seed=1004, init_std=0.02),
    5: Workload("short_docs_bf16_T32768_H64_d64_lb-5", B=1, T=32768, H=64, K=64, V=64,
                dtype="bf16", seed=1005, lower_bound=-5.0, gate_std=3.0, beta_std=2.0,
                lengths="short1to100"),
}


def lengths_composition(seed: int, T: int, n_docs: int, min_len: int) -> np.ndarray:
    """n_docs lengths, each >= min_len, summing to T: min_len plus a uniform
    composition of the remainder (n_docs-1 sorted uniform integer cut points)."""
    rng = np.random.default_rng(seed)
    rest = T - n_docs * min_len
    cuts = np.sort(rng.integers(0, rest + 1, size=n_docs - 1))
    parts = np.diff(np.concatenate([[0], cuts, [rest]]))
    return (parts + min_len).astype(np.int64)


def lengths_uniform_until(seed: int, T: int, lo: int, hi: int) -> np.ndarray:
    """Draw U{lo..hi} lengths until they reach T, truncating the last one."""
    rng = np.random.default_rng(seed)
    out, total = [], 0
    while total < T:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, T - total)
        out.append(n)
        total += n
    return np.asarray(out, np.int64)


def cu_from_lengths(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))]).astype(np.int32)


def doc_lengths(w: Workload) -> Optional[np.ndarray]:
    if w.lengths == "rows":
        return None
    if w.lengths == "composition7":
        return lengths_composition(w.seed, w.T, 7, 64)
    if w.lengths == "short1to100":
        return lengths_uniform_until(w.seed, w.T, 1, 100)
    raise ValueError(w.lengths)


def make_inputs(w: Workload, device="cpu", T: Optional[int] = None, H: Optional[int] = None,
                B: Optional[int] = None, lengths=None):
    """Draw one workload's tensors.  T/H/B/lengths may shrink it (same recipe)."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    H = w.H if H is None else H
    K, V = w.K, w.V
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)

    def randn(*shape, std=1.0):
        x = torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)
        return x * std if std != 1.0 else x

    q = randn(B, T, H, K)
    k = randn(B, T, H, K)
    v = randn(B, T, H, V)
    gate = randn(B, T, H, K, std=w.gate_std)
    beta = randn(B, T, H, std=w.beta_std)
    a_log = torch.rand(H, generator=gen, device=dev, dtype=torch.float32) * 2.0 - 1.0
    dt_bias = randn(H, K, std=0.1)
    cu = None
    if lengths is None and w.lengths != "rows" and T == w.T:
        lengths = doc_lengths(w)
    if lengths is not None:
        cu = torch.from_numpy(cu_from_lengths(lengths)).to(dev)
        N = len(lengths)
    else:
        N = B
    init = randn(N, H, K, V, std=w.init_std) if w.init_std is not None else None
    dt = w.torch_dtype
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), gate=gate.to(dt), beta=beta.to(dt),
                a_log=a_log, dt_bias=dt_bias, initial_state=init, cu_seqlens=cu,
                scale=w.scale, lower_bound=w.lower_bound, chunk_size=w.chunk_size)


def random_problem(seed, B, T, H, K, V, dtype=torch.float32, device="cpu", gate_std=1.0,
                   beta_std=1.0, init_std=None, lengths=None, a_log_range=1.0, HV=None):
    """Free-form draw with the same recipe, for edge-case tests.  HV (a multiple
    of H) gives v, gate, beta, a_log, dt_bias and the states HV value heads while
    q and k keep H key heads; None means HV = H."""
    HV = H if HV is None else HV
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)

    def randn(*shape, std=1.0):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32) * std

    q = randn(B, T, H, K)
    k = randn(B, T, H, K)
    v = randn(B, T, HV, V)
    gate = randn(B, T, HV, K, std=gate_std)
    beta = randn(B, T, HV, std=beta_std)
    a_log = (torch.rand(HV, generator=gen, device=dev) * 2.0 - 1.0) * a_log_range
    dt_bias = randn(HV, K, std=0.1)
    cu = None
    N = B
    if lengths is not None:
        cu = torch.from_numpy(cu_from_lengths(lengths)).to(dev)
        N = len(lengths)
    init = randn(N, HV, K, V, std=init_std) if init_std is not None else None
    return dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype), gate=gate.to(dtype),
                beta=beta.to(dtype), a_log=a_log, dt_bias=dt_bias, initial_state=init,
                cu_seqlens=cu)


def short_conv_params(seed, channels, width, bias=True, device="cpu"):
    """Seeded weights of the three short convolutions (q, k, v).

    ``channels`` = (C_q, C_k, C_v).  The draw follows the default
    initialisation of a depthwise torch Conv1d (fan-in = width): weights and
    biases uniform in [-1/sqrt(width), 1/sqrt(width)], float32, drawn in the
    order w_q, w_k, w_v, b_q, b_k, b_v from ``torch.Generator(device)``.
    Returns (weights [C, width] each, biases [C] each or None)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    bound = 1.0 / float(np.sqrt(width))

    def uni(n, shape):
        return (torch.rand(shape, generator=gen, device=dev) * 2.0 - 1.0) * bound

    ws = tuple(uni(C, (C, width)) for C in channels)
    bs = tuple(uni(C, (C,)) for C in channels) if bias else None
    return ws, bs
