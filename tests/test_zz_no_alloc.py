"""kda_fwd_noalloc (workspace in the library's static device scratch array)
against kda_fwd (caller-provided workspace), through the C ABI.

Both run the same kernels, so their outputs and final states must agree bit
for bit; two calls in a row, the second smaller, check that a call does not
depend on what the previous one left in the shared scratch array."""
import pytest
import torch

from gated_delta_rule_43_amd import kda, synthetic
from kda_testlib import assert_close, oracle_fwd, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(seed, T, H, K, V, lengths=None, init_std=None, dtype=torch.bfloat16):
    inp = synthetic.random_problem(seed, 1, T if lengths is None else sum(lengths), H, K, V,
                                   dtype=dtype, device=DEV, init_std=init_std, lengths=lengths)
    return inp


def _both(inp, lower_bound=None, ref_path=None, monkeypatch=None):
    """(kda_fwd_noalloc's outputs, kda_fwd's outputs); kda_fwd runs under
    KDA_PATH=ref_path when given (the path the allocation-free call takes)."""
    args = (inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["a_log"], inp["dt_bias"])
    cu = inp["cu_seqlens"]
    N = 1 if cu is None else cu.numel() - 1
    B, T, H, K = inp["q"].shape
    V = inp["v"].shape[-1]
    if ref_path is not None:
        monkeypatch.setenv("KDA_PATH", ref_path)
    o_ref, f_ref = kda.kda_fwd(*args, lower_bound=lower_bound, cu_seqlens=cu,
                               initial_state=inp["initial_state"], output_final_state=True)
    if ref_path is not None:
        monkeypatch.delenv("KDA_PATH")
    o = torch.full((B, T, H, V), float("nan"), dtype=inp["q"].dtype, device=DEV)
    f = torch.full((N, H, K, V), float("nan"), dtype=torch.float32, device=DEV)
    kda.kda_fwd_noalloc(*args, lower_bound=lower_bound, cu_seqlens=cu,
                        initial_state=inp["initial_state"], out=o, final_state_out=f)
    torch.cuda.synchronize()
    return (o, f), (o_ref, f_ref)


def test_noalloc_two_calls_second_smaller():
    print("[gpu-test] noalloc: two calls, second smaller", flush=True)
    assert kda.load_library().kda_fwd_noalloc_scratch_bytes() == 64 << 20
    big = _inputs(71, 640, 4, 128, 128, init_std=0.1)
    small = _inputs(72, 0, 2, 64, 64, lengths=[37, 0, 100, 64], init_std=0.3)
    for inp, lb in ((big, None), (small, -5.0)):
        (o, f), (o_ref, f_ref) = _both(inp, lb)
        assert torch.equal(o, o_ref), "output differs from kda_fwd"
        assert torch.equal(f, f_ref), "final state differs from kda_fwd"
        inp.update(scale=None, lower_bound=lb, chunk_size=64)
        oo, ff = oracle_fwd(inp)
        assert_close(to_np(o), oo, torch.bfloat16, "o vs oracle")
        assert_close(to_np(f), ff, torch.bfloat16, "final state vs oracle")


def test_noalloc_falls_back_to_fused_when_records_exceed_scratch(monkeypatch):
    """T=8192, 16 heads, d=128: the two-pass records (152 MB) exceed the 64 MiB
    array, so the fused path runs; it equals kda_fwd on the fused path bit for
    bit, and kda_fwd's own choice within the tolerances."""
    print("[gpu-test] noalloc: fused fallback", flush=True)
    inp = _inputs(73, 0, 16, 128, 128, lengths=[3000, 5192], init_std=0.05)
    (o, f), (o_ref, f_ref) = _both(inp, ref_path="fused", monkeypatch=monkeypatch)
    assert torch.equal(o, o_ref) and torch.equal(f, f_ref)
    (o, f), (o_ref, f_ref) = _both(inp)
    assert_close(to_np(o), to_np(o_ref), torch.bfloat16, "o vs kda_fwd")
    assert float((f - f_ref).abs().max()) <= 1e-4


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    """fp32 inputs run the vector-ALU path, whose workspace holds per-token
    and per-chunk factors; at T=8192, 4 heads, d=128 it exceeds 64 MiB."""
    inp = _inputs(74, 8192, 4, 128, 128, dtype=torch.float32)
    o = torch.empty(1, 8192, 4, 128, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError, match="allocation-free entry point has 67108864"):
        kda.kda_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"],
                            inp["a_log"], inp["dt_bias"], out=o)
