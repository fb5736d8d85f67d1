"""The fused matrix-core path (one workgroup per (sequence, head), each chunk's
factors kept in LDS) against the oracle, and against the two-pass path.

Both paths run the same chunk-factor code and the same state products in the
same order, so their outputs and final states must agree bit for bit; the
oracle comparison holds them to the bf16 tolerance.  KDA_PATH selects the path
per call (it is read by the library at every call)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_43_amd import kda, synthetic
from kda_testlib import assert_close, gpu_fwd, oracle_fwd, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # (name, K, V, T, H, lengths, lower_bound, form, init_std, HV)
    ("rows_d128", 128, 128, 300, 2, None, None, "sigmoid", None, None),
    ("docs_d64_lb", 64, 64, 0, 3, [1, 64, 0, 65, 130, 7], -5.0, "sigmoid", 0.5, None),
    ("docs_k128_v64_clamp", 128, 64, 0, 2, [100, 28, 200], -3.0, "clamp", 0.2, None),
    ("rows_k64_v128_init", 64, 128, 193, 2, None, None, "sigmoid", 0.3, None),
    ("grouped_heads", 128, 128, 150, 2, None, None, "sigmoid", 0.1, 4),
    # one-chunk documents from a zero state: the two-pass path finishes them
    # inside the chunk-factor kernel
    ("short_docs_d128_no_init", 128, 128, 0, 3, [5, 64, 1, 70, 0, 33, 128, 64], None, "sigmoid", None, None),
    ("short_docs_d64_no_init_lb", 64, 64, 0, 2, [64, 17, 1, 2, 100, 63], -5.0, "sigmoid", None, None),
]


def _problem(case, seed):
    name, K, V, T, H, lengths, lb, form, init_std, HV = case
    if lengths is not None:
        T = sum(lengths)
    inp = synthetic.random_problem(seed, 1 if lengths else 2, T, H, K, V, dtype=torch.bfloat16,
                                   device=DEV, init_std=init_std, lengths=lengths, HV=HV)
    inp.update(scale=None, lower_bound=lb, chunk_size=64, lower_bound_form=form)
    return inp


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_matches_two_pass_bitwise_and_oracle(case, monkeypatch):
    print("[gpu-test] fused path " + case[0], flush=True)
    inp = _problem(case, 500 + CASES.index(case))
    monkeypatch.setenv("KDA_PATH", "mfma")
    o3, f3 = gpu_fwd(inp)           # the launcher's own choice of state pass
    monkeypatch.setenv("KDA_STATE_KS", "1")
    o2, f2 = gpu_fwd(inp)           # one wave per column tile, as the fused kernel
    monkeypatch.delenv("KDA_STATE_KS")
    monkeypatch.setenv("KDA_PATH", "fused")
    B, T, H, K = inp["q"].shape
    assert kda.fwd_path((B, T, H, K), inp["v"].shape[-1]) == "fused"
    o1, f1 = gpu_fwd(inp)
    assert torch.equal(o1, o2), "fused vs two-pass output differs"
    assert torch.equal(f1, f2), "fused vs two-pass final state differs"
    # a key-split state pass sums the partial products in another order
    assert_close(to_np(o3), to_np(o1), torch.bfloat16, "o, two-pass state pass of the launcher's choice")
    assert float((f3 - f1).abs().max()) <= 1e-4
    if case[-1] is None:
        o_ref, f_ref = oracle_fwd(inp)
        assert_close(to_np(o1), o_ref, torch.bfloat16, "o")
        assert_close(to_np(f1), f_ref, torch.bfloat16, "final_state")


def test_fused_extreme_gates(monkeypatch):
    """Single steps decaying by tens of nats: blocks leave the factorised range
    and the fused kernel takes the exact per-pair path in place."""
    inp = synthetic.random_problem(77, 1, 256, 2, 128, 128, dtype=torch.bfloat16, device=DEV,
                                   gate_std=1.0, init_std=0.1)
    g = inp["gate"].float()
    g[:, ::7] += 40.0   # softplus(x) ~ x: about -40 * e^{a_log} per marked token
    inp["gate"] = g.to(torch.bfloat16)
    inp["a_log"] = torch.full_like(inp["a_log"], 0.5)
    inp.update(scale=None, lower_bound=None, chunk_size=64)
    monkeypatch.setenv("KDA_PATH", "fused")
    o1, f1 = gpu_fwd(inp)
    o_ref, f_ref = oracle_fwd(inp)
    assert_close(to_np(o1), o_ref, torch.bfloat16, "o")
    assert_close(to_np(f1), f_ref, torch.bfloat16, "final_state")
    monkeypatch.setenv("KDA_PATH", "mfma")
    monkeypatch.setenv("KDA_STATE_KS", "1")
    o2, f2 = gpu_fwd(inp)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("C", [16, 32])
def test_short_chunks_on_matrix_cores(C, monkeypatch):
    """bf16 with 16- and 32-token chunks runs on the matrix-core kernels (the
    chunk fills the first rows of a 64-row tile); documents of every length
    class against the oracle, on both matrix-core paths (equal bit for bit)."""
    print("[gpu-test] chunk %d on matrix cores" % C, flush=True)
    lengths = [1, C - 1, C, C + 1, 3 * C + 5, 0, 64, 2 * C]
    inp = synthetic.random_problem(600 + C, 1, sum(lengths), 2, 128, 64, dtype=torch.bfloat16,
                                   device=DEV, init_std=0.2, lengths=lengths)
    inp.update(scale=None, lower_bound=None, chunk_size=C)
    assert kda.fwd_path((1, sum(lengths), 2, 128), 64, chunk_size=C, cu_seqlens=True) == "mfma"
    monkeypatch.setenv("KDA_STATE_KS", "1")
    o2, f2 = gpu_fwd(inp)
    monkeypatch.setenv("KDA_PATH", "fused")
    o1, f1 = gpu_fwd(inp)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    o_ref, f_ref = oracle_fwd(inp)
    assert_close(to_np(o1), o_ref, torch.bfloat16, "o")
    assert_close(to_np(f1), f_ref, torch.bfloat16, "final_state")
