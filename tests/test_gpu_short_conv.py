"""GPU parity of the short convolution + SiLU before the forward: the HIP
kernels (through the C ABI) against the oracle on the same seeded inputs.

- kda_short_conv_silu alone: each output within one bf16 rounding of the
  oracle's fp64 value (bf16), or within 1e-5 (fp32), for every width 0..4,
  with and without bias, over rows and packed documents shorter than the
  window, empty documents and boundaries inside a thread's token run;
- kda_fwd_short_conv: output and final state against the oracle's forward on
  the oracle's convolved inputs, at the forward's tolerances (fp32 max-abs
  1e-4; bf16 max-abs 2e-2 and relative Frobenius 1e-2), on both kernel paths.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_43_amd import kda, synthetic
from kda_testlib import assert_close, to_device, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _banner(msg):
    print("[gpu-test] " + msg, flush=True)


def _conv_check(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    if dtype == torch.bfloat16:
        # computed in fp32 and rounded once: at most one bf16 unit in the last place
        bound = 2.0 ** -8 * np.abs(ref) + 1e-6
    else:
        bound = np.full_like(ref, 1e-5)
    worst = np.argmax(err - bound)
    assert np.all(err <= bound), "%s: |err| %.3g > bound %.3g at flat index %d" % (
        what, err.flat[worst], bound.flat[worst], worst)


def _params(seed, channels, width, bias):
    if width == 0:
        return None, None
    ws, bs = synthetic.short_conv_params(seed, channels, width, bias)
    return ws, bs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("width", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("bias", [False, True])
def test_short_conv_rows(dtype, width, bias):
    if width == 0 and bias:
        pytest.skip("SiLU alone takes no bias")
    _banner("short conv rows %s W=%d bias=%s" % (dtype, width, bias))
    B, T, H, D = 3, 77, 2, 64     # 77 tokens: two full 32-token runs and a ragged one
    gen = torch.Generator().manual_seed(40 + width)
    x = torch.randn(B, T, H, D, generator=gen).to(dtype)
    ws, bs = _params(7, (H * D,), width, bias)
    w = None if ws is None else ws[0]
    b = None if bs is None else bs[0]
    y = kda.short_conv_silu(x.to(DEV), None if w is None else w.to(DEV),
                            None if b is None else b.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.short_conv_silu(x.float().numpy(), None if w is None else w.numpy(),
                                 None if b is None else b.numpy())
    _conv_check(to_np(y), ref, dtype, "y")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("width", [2, 4])
def test_short_conv_packed_documents(dtype, width):
    _banner("short conv packed %s W=%d" % (dtype, width))
    lengths = [100, 0, 1, 2, 37, 33, 3, 64, 0, 5]
    T = sum(lengths)
    cu = synthetic.cu_from_lengths(lengths)
    C = 24  # a channel count that is not a power of two
    gen = torch.Generator().manual_seed(3)
    x = torch.randn(1, T, C, generator=gen).to(dtype)
    ws, bs = synthetic.short_conv_params(9, (C,), width, True)
    for host in (None, False):  # validated offsets, and the device-only search
        y = kda.short_conv_silu(x.to(DEV), ws[0].to(DEV), bs[0].to(DEV),
                                cu_seqlens=torch.from_numpy(cu).to(DEV), cu_seqlens_host=host)
        torch.cuda.synchronize()
        ref = oracle.short_conv_silu(x.float().numpy(), ws[0].numpy(), bs[0].numpy(), cu_seqlens=cu)
        _conv_check(to_np(y), ref, dtype, "y (host offsets %s)" % (host is None))


def test_short_conv_rows_shorter_than_the_window():
    """T = 2 < W - 1: every token's window reaches before the row start."""
    _banner("short conv T=2 rows")
    x = torch.randn(5, 2, 16, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    ws, bs = synthetic.short_conv_params(2, (16,), 4, True)
    y = kda.short_conv_silu(x.to(DEV), ws[0].to(DEV), bs[0].to(DEV))
    torch.cuda.synchronize()
    ref = oracle.short_conv_silu(x.float().numpy(), ws[0].numpy(), bs[0].numpy())
    _conv_check(to_np(y), ref, torch.bfloat16, "y")


def test_short_conv_empty_input():
    x = torch.empty(2, 0, 64, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(64, 4, device=DEV)
    y = kda.short_conv_silu(x, w)
    assert y.shape == x.shape


def _fwd_inputs(dtype, K, V, H, HV, lengths=None, B=1, T=None, seed=0):
    T = sum(lengths) if lengths is not None else T
    inp = synthetic.random_problem(seed, B, T, H, K, V, dtype=dtype, lengths=lengths, HV=HV,
                                   init_std=0.5)
    return to_device(inp)


def _fwd_compare(inp, width, bias, dtype, what, seed=11):
    H, K = inp["q"].shape[2], inp["q"].shape[3]
    HV, V = inp["v"].shape[2], inp["v"].shape[3]
    ws, bs = (None, None) if width == 0 else synthetic.short_conv_params(
        seed, (H * K, H * K, HV * V), width, bias)
    cu = inp["cu_seqlens"]
    o, fin = kda.kda_fwd_short_conv(
        inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["a_log"], inp["dt_bias"],
        None if ws is None else tuple(w.to(DEV) for w in ws),
        None if bs is None else tuple(b.to(DEV) for b in bs),
        cu_seqlens=cu, initial_state=inp["initial_state"], output_final_state=True)
    torch.cuda.synchronize()
    npy = lambda t: None if t is None else to_np(t)
    o_ref, f_ref = oracle.kda_fwd_short_conv(
        npy(inp["q"]), npy(inp["k"]), npy(inp["v"]), npy(inp["gate"]), npy(inp["beta"]),
        npy(inp["a_log"]), npy(inp["dt_bias"]),
        None if ws is None else tuple(w.numpy() for w in ws),
        None if bs is None else tuple(b.numpy() for b in bs),
        cu_seqlens=None if cu is None else to_np(cu).astype(np.int32),
        initial_state=npy(inp["initial_state"]))
    assert_close(to_np(o), o_ref, dtype, what + " o")
    assert_close(to_np(fin), f_ref, dtype, what + " final_state")


@pytest.mark.parametrize("dtype,K,V", [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 64),
                                       (torch.float32, 64, 64)])
@pytest.mark.parametrize("width,bias", [(4, True), (0, False)])
def test_fwd_short_conv_packed(dtype, K, V, width, bias):
    _banner("fwd short conv packed %s K=%d V=%d W=%d" % (dtype, K, V, width))
    inp = _fwd_inputs(dtype, K, V, H=2, HV=2, lengths=[100, 37, 0, 170, 2])
    _fwd_compare(inp, width, bias, dtype, "packed")


def test_fwd_short_conv_rows_grouped_heads():
    _banner("fwd short conv rows, grouped value heads")
    inp = _fwd_inputs(torch.bfloat16, 128, 128, H=2, HV=4, B=2, T=150)
    _fwd_compare(inp, 3, False, torch.bfloat16, "rows GVA")


def test_fwd_short_conv_matches_conv_then_fwd():
    """The fused entry point is the standalone convolution followed by kda_fwd,
    bit for bit (same kernels, same roundings)."""
    _banner("fwd short conv == conv then fwd")
    inp = _fwd_inputs(torch.bfloat16, 128, 128, H=2, HV=2, lengths=[90, 200, 7])
    H, K, HV, V = 2, 128, 2, 128
    ws, bs = synthetic.short_conv_params(5, (H * K, H * K, HV * V), 4, True)
    ws = tuple(w.to(DEV) for w in ws)
    bs = tuple(b.to(DEV) for b in bs)
    cu = inp["cu_seqlens"]
    o1, f1 = kda.kda_fwd_short_conv(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"],
                                    inp["a_log"], inp["dt_bias"], ws, bs, cu_seqlens=cu,
                                    output_final_state=True)
    qc = kda.short_conv_silu(inp["q"], ws[0], bs[0], cu_seqlens=cu)
    kc = kda.short_conv_silu(inp["k"], ws[1], bs[1], cu_seqlens=cu)
    vc = kda.short_conv_silu(inp["v"], ws[2], bs[2], cu_seqlens=cu)
    o2, f2 = kda.kda_fwd(qc, kc, vc, inp["gate"], inp["beta"], inp["a_log"], inp["dt_bias"],
                         cu_seqlens=cu, output_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


# KDA_CONV_FUSED=1: the matrix-core kernels apply a width-4 convolution as they
# load q, k and v (by default, and with =0, the standalone pass runs first).
# Both round each convolved value to bf16 in the same order of operations, so
# the outputs must agree bit for bit.
ON_LOAD_CASES = [
    # (name, K, V, H, HV, B, T, lengths, chunk, lower_bound, init_std, bias, gate_shift)
    ("rows_d128_init", 128, 128, 2, 2, 2, 300, None, 64, None, 0.3, True, 0.0),
    ("short_docs_d64_zero_state", 64, 64, 2, 2, 1, 0, [1, 2, 3, 64, 65, 0, 130, 17], 64, None, None, False, 0.0),
    ("k128_v64_grouped_chunk32", 128, 64, 2, 4, 2, 150, None, 32, None, 0.2, True, 0.0),
    ("docs_d128_chunk16_lb", 128, 128, 2, 2, 1, 0, [40, 3, 77, 16, 15], 16, -5.0, None, True, 0.0),
    ("k64_v128_rows", 64, 128, 3, 3, 1, 200, None, 64, None, 0.1, False, 0.0),
    ("extreme_gates_exact_path", 128, 128, 2, 2, 1, 256, None, 64, None, 0.1, True, 40.0),
]


def _on_load_problem(case, seed):
    name, K, V, H, HV, B, T, lengths, C, lb, init_std, bias, shift = case
    if lengths is not None:
        T = sum(lengths)
    inp = _to_dev_problem(seed, B, T, H, K, V, HV, lengths, init_std)
    if shift:
        g = inp["gate"].float()
        g[:, ::7] += shift      # single steps decaying by tens of nats
        inp["gate"] = g.to(torch.bfloat16)
        inp["a_log"] = torch.full_like(inp["a_log"], 0.5)
    ws, bs = synthetic.short_conv_params(seed + 1, (H * K, H * K, HV * V), 4, bias)
    ws = tuple(w.to(DEV) for w in ws)
    bs = None if bs is None else tuple(None if b is None else b.to(DEV) for b in bs)
    return inp, ws, bs, C, lb


def _to_dev_problem(seed, B, T, H, K, V, HV, lengths, init_std):
    inp = synthetic.random_problem(seed, B, T, H, K, V, dtype=torch.bfloat16, lengths=lengths,
                                   HV=HV, init_std=init_std)
    return to_device(inp)


def _conv_fwd(inp, ws, bs, C, lb, workspace=None):
    o, fin = kda.kda_fwd_short_conv(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"],
                                    inp["a_log"], inp["dt_bias"], ws, bs, chunk_size=C,
                                    lower_bound=lb, cu_seqlens=inp["cu_seqlens"],
                                    initial_state=inp["initial_state"], output_final_state=True,
                                    workspace=workspace)
    torch.cuda.synchronize()
    return o, fin


@pytest.mark.parametrize("case", ON_LOAD_CASES, ids=[c[0] for c in ON_LOAD_CASES])
def test_fwd_short_conv_on_load_matches_standalone(case, monkeypatch):
    _banner("conv on load " + case[0])
    inp, ws, bs, C, lb = _on_load_problem(case, 300 + ON_LOAD_CASES.index(case))
    monkeypatch.setenv("KDA_CONV_FUSED", "0")
    o0, f0 = _conv_fwd(inp, ws, bs, C, lb)
    monkeypatch.setenv("KDA_CONV_FUSED", "1")
    o1, f1 = _conv_fwd(inp, ws, bs, C, lb)
    assert torch.equal(o1, o0), "output differs: max %.3g" % float((o1.float() - o0.float()).abs().max())
    assert torch.equal(f1, f0), "final state differs: max %.3g" % float((f1 - f0).abs().max())
    # the fused kernel (one workgroup per sequence and head) convolves on load too
    monkeypatch.setenv("KDA_PATH", "fused")
    o2, f2 = _conv_fwd(inp, ws, bs, C, lb)
    monkeypatch.setenv("KDA_STATE_KS", "1")
    monkeypatch.setenv("KDA_PATH", "mfma")
    o3, f3 = _conv_fwd(inp, ws, bs, C, lb)
    assert torch.equal(o2, o3) and torch.equal(f2, f3)


def test_fwd_short_conv_on_load_needs_no_conv_buffers(monkeypatch):
    """With the convolution applied on load the forward's own workspace is
    enough; the standalone pass needs room for the convolved tensors."""
    case = ON_LOAD_CASES[0]
    inp, ws, bs, C, lb = _on_load_problem(case, 399)
    monkeypatch.setenv("KDA_CONV_FUSED", "1")
    B, T, H, K = inp["q"].shape
    HV, V = inp["v"].shape[2], inp["v"].shape[3]
    n = kda.fwd_workspace_size((B, T, H, K), V, chunk_size=C, HV=HV)
    small = torch.empty(n, dtype=torch.uint8, device=DEV)
    o1, f1 = _conv_fwd(inp, ws, bs, C, lb, workspace=small)
    monkeypatch.setenv("KDA_CONV_FUSED", "0")
    with pytest.raises(ValueError, match="workspace"):
        _conv_fwd(inp, ws, bs, C, lb, workspace=small)
    o0, f0 = _conv_fwd(inp, ws, bs, C, lb)
    assert torch.equal(o1, o0) and torch.equal(f1, f0)


def test_fwd_short_conv_on_load_throughput_shape_sampled(monkeypatch):
    """Workload 3's shape at full size, width 4 with bias, convolved on load,
    against the standalone convolution then kda_fwd (bit for bit)."""
    monkeypatch.setenv("KDA_CONV_FUSED", "1")
    w3 = synthetic.WORKLOADS[3]
    _banner("conv on load, " + w3.name)
    inp = synthetic.make_inputs(w3, DEV)
    ws, bs = synthetic.short_conv_params(33, (w3.H * w3.K, w3.H * w3.K, w3.H * w3.V), 4, True)
    ws = tuple(w.to(DEV) for w in ws)
    bs = tuple(b.to(DEV) for b in bs)
    args = (inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["a_log"], inp["dt_bias"], ws, bs)
    o1, _ = kda.kda_fwd_short_conv(*args)
    qc = kda.short_conv_silu(inp["q"], ws[0], bs[0])
    kc = kda.short_conv_silu(inp["k"], ws[1], bs[1])
    vc = kda.short_conv_silu(inp["v"], ws[2], bs[2])
    o2, _ = kda.kda_fwd(qc, kc, vc, inp["gate"], inp["beta"], inp["a_log"], inp["dt_bias"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
