"""GPU parity of the backward (kda_bwd through the C ABI) against the oracle's
reverse-mode gradients on the same seeded inputs.

Tolerances, per gradient tensor g with oracle value r (scaled by the tensor's
largest magnitude, since gradients of different inputs differ in size):
  fp32 inputs: max|g - r| <= 1e-4 * max(1, max|r|)   (fp32 sums of at most
               a few thousand terms, each within a few ulp);
  bf16 inputs: max|g - r| <= 2e-2 * max(1, max|r|) and ||g - r||_F <= 1e-2 ||r||_F
               (the gradients are rounded once to bf16 on output, 2^-9 relative,
               and the forward's bf16 tolerance carries over).
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_43_amd import kda, synthetic
from kda_testlib import to_device, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"
NAMES = ("dq", "dk", "dv", "dgate", "dbeta", "da_log", "ddt_bias", "dinit")


def _banner(msg):
    print("[gpu-test] " + msg, flush=True)


def _check(got, ref, dtype, what):
    for n in NAMES:
        g = to_np(got[n]).astype(np.float64)
        r = ref[n]
        assert g.shape == r.shape, (what, n, g.shape, r.shape)
        scale = max(1.0, float(np.abs(r).max()) if r.size else 1.0)
        err = np.abs(g - r).max() if r.size else 0.0
        if dtype == torch.float32:
            assert err <= 1e-4 * scale, "%s %s: max-abs %.3g > %.3g" % (what, n, err, 1e-4 * scale)
        else:
            rf = np.linalg.norm(g - r) / max(1e-30, np.linalg.norm(r))
            assert err <= 2e-2 * scale and (rf <= 1e-2 or np.linalg.norm(r) == 0), \
                "%s %s: max-abs %.3g (<= %.3g), rel-F %.3g" % (what, n, err, 2e-2 * scale, rf)


def _run(inp, d_o, d_fin, dtype, what, **kw):
    got = kda.kda_bwd(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["a_log"],
                      inp["dt_bias"], d_o, d_fin, cu_seqlens=inp["cu_seqlens"],
                      initial_state=inp["initial_state"], **kw)
    torch.cuda.synchronize()
    npy = lambda t: None if t is None else to_np(t)
    gm = {"sigmoid": "sigmoid", "clamp": "clamp"}.get(kw.get("lower_bound_form", "sigmoid"))
    ref = oracle.kda_bwd(npy(inp["q"]), npy(inp["k"]), npy(inp["v"]), npy(inp["gate"]),
                         npy(inp["beta"]), npy(inp["a_log"]), npy(inp["dt_bias"]), npy(d_o),
                         npy(d_fin), scale=kw.get("scale"), lower_bound=kw.get("lower_bound"),
                         cu_seqlens=None if inp["cu_seqlens"] is None
                         else to_np(inp["cu_seqlens"]).astype(np.int32),
                         initial_state=npy(inp["initial_state"]),
                         gate_mode=None if kw.get("lower_bound") is None else gm)
    _check(got, ref, dtype, what)
    return got, ref


def _upstream(inp, seed, with_final=True):
    g = torch.Generator().manual_seed(seed)
    B, T, HV, V = inp["v"].shape
    N = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    K = inp["q"].shape[-1]
    d_o = torch.randn(B, T, HV, V, generator=g).to(inp["v"].dtype).to(DEV)
    d_fin = torch.randn(N, HV, K, V, generator=g).to(DEV) if with_final else None
    return d_o, d_fin


@pytest.mark.parametrize("C", [64, 32, 16])
def test_bwd_fp32_rows(C):
    _banner("bwd fp32 rows C=%d" % C)
    inp = to_device(synthetic.random_problem(31, 2, 150, 2, 64, 64, dtype=torch.float32,
                                             init_std=0.5))
    d_o, d_fin = _upstream(inp, 1)
    _run(inp, d_o, d_fin, torch.float32, "fp32 rows C=%d" % C, chunk_size=C, scale=0.3)


def test_bwd_fp32_k128_v64_rows():
    """K=128 with V=64: the chunk-64 matrix-core paths with two state tiles per
    wave and a single 64-column state tile."""
    _banner("bwd fp32 rows K=128 V=64")
    inp = to_device(synthetic.random_problem(41, 2, 200, 2, 128, 64, dtype=torch.float32,
                                             init_std=0.5))
    d_o, d_fin = _upstream(inp, 11)
    _run(inp, d_o, d_fin, torch.float32, "fp32 rows K=128 V=64")


def test_bwd_fp32_packed_grouped_sigmoid_gate():
    _banner("bwd fp32 packed GVA sigmoid gate")
    inp = to_device(synthetic.random_problem(32, 1, 265, 1, 64, 64, dtype=torch.float32,
                                             lengths=[70, 0, 1, 130, 64], HV=2, init_std=0.5))
    d_o, d_fin = _upstream(inp, 2)
    _run(inp, d_o, d_fin, torch.float32, "fp32 packed GVA", lower_bound=-3.0)


def test_bwd_fp32_clamped_gate_no_final_gradient():
    _banner("bwd fp32 clamp gate, no d_final")
    inp = to_device(synthetic.random_problem(33, 1, 100, 2, 64, 128, dtype=torch.float32,
                                             gate_std=3.0))
    d_o, _ = _upstream(inp, 3, with_final=False)
    _run(inp, d_o, None, torch.float32, "fp32 clamp", lower_bound=-0.5, lower_bound_form="clamp")


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64)])
def test_bwd_bf16_packed(K, V):
    _banner("bwd bf16 packed K=%d V=%d" % (K, V))
    inp = to_device(synthetic.random_problem(34, 1, 309, 2, K, V, dtype=torch.bfloat16,
                                             lengths=[100, 37, 0, 170, 2], init_std=0.5))
    d_o, d_fin = _upstream(inp, 4)
    _run(inp, d_o, d_fin, torch.bfloat16, "bf16 packed K=%d" % K)


def test_bwd_bf16_rows_grouped_heads_lower_bound():
    _banner("bwd bf16 rows GVA lb")
    inp = to_device(synthetic.random_problem(35, 2, 130, 2, 128, 128, dtype=torch.bfloat16,
                                             HV=4))
    d_o, d_fin = _upstream(inp, 5)
    _run(inp, d_o, d_fin, torch.bfloat16, "bf16 rows GVA", lower_bound=-5.0)


def test_bwd_is_deterministic_and_matches_across_chunk_sizes():
    """Two calls give identical bits; chunk sizes 64 and 16 agree to fp32
    rounding (the result does not depend on the chunking)."""
    _banner("bwd determinism")
    inp = to_device(synthetic.random_problem(36, 1, 200, 2, 64, 64, dtype=torch.float32,
                                             init_std=0.5))
    d_o, d_fin = _upstream(inp, 6)
    args = (inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["a_log"], inp["dt_bias"],
            d_o, d_fin)
    a = kda.kda_bwd(*args, initial_state=inp["initial_state"])
    b = kda.kda_bwd(*args, initial_state=inp["initial_state"])
    c = kda.kda_bwd(*args, initial_state=inp["initial_state"], chunk_size=16)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n
        scale = max(1.0, a[n].abs().max().item())
        assert (a[n] - c[n]).abs().max().item() <= 1e-4 * scale, n


def test_bwd_empty_and_zero_upstream():
    _banner("bwd empty rows / zero upstream")
    inp = to_device(synthetic.random_problem(37, 1, 0, 2, 64, 64, dtype=torch.float32,
                                             lengths=[0, 0], init_std=0.5))
    d_o, d_fin = _upstream(inp, 7)
    got = kda.kda_bwd(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["a_log"],
                      inp["dt_bias"], d_o, d_fin, cu_seqlens=inp["cu_seqlens"],
                      initial_state=inp["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(got["dinit"], d_fin)   # empty documents pass the gradient through
    assert torch.all(got["da_log"] == 0) and torch.all(got["ddt_bias"] == 0)
    inp = to_device(synthetic.random_problem(38, 1, 90, 2, 64, 64, dtype=torch.float32))
    zero = torch.zeros(1, 90, 2, 64, device=DEV)
    got = kda.kda_bwd(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["a_log"],
                      inp["dt_bias"], zero)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.all(got[n] == 0), n


def test_bwd_device_only_offsets_match_host_checked():
    """cu_seqlens without a host copy (sized from the upper bound of the chunk
    count) gives the same bits as with the host-checked exact sizing."""
    _banner("bwd device-only offsets")
    inp = to_device(synthetic.random_problem(39, 1, 300, 2, 64, 64, dtype=torch.bfloat16,
                                             lengths=[1, 63, 64, 65, 0, 107], init_std=0.5))
    d_o, d_fin = _upstream(inp, 9)
    args = (inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["a_log"], inp["dt_bias"],
            d_o, d_fin)
    a = kda.kda_bwd(*args, cu_seqlens=inp["cu_seqlens"], initial_state=inp["initial_state"])
    b = kda.kda_bwd(*args, cu_seqlens=inp["cu_seqlens"], cu_seqlens_host=False,
                    initial_state=inp["initial_state"])
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


def test_bwd_profiled_same_bits_and_stage_times():
    """kda_bwd_profiled does exactly kda_bwd's work: identical bits, and every
    stage's pair of events is recorded in order on the launch stream."""
    from gated_delta_rule_43_amd.timing import StageEvents
    _banner("bwd profiled")
    inp = to_device(synthetic.random_problem(40, 1, 300, 2, 128, 128, dtype=torch.bfloat16,
                                             lengths=[100, 200], init_std=0.5))
    d_o, d_fin = _upstream(inp, 10)
    args = (inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["a_log"], inp["dt_bias"],
            d_o, d_fin)
    kw = dict(cu_seqlens=inp["cu_seqlens"], initial_state=inp["initial_state"])
    a = kda.kda_bwd(*args, **kw)
    ev = StageEvents(1, kda.BWD_NUM_STAGES)
    b = kda.kda_bwd(*args, stage_events=ev.arrays[0], **kw)
    torch.cuda.synchronize()
    ms = ev.stage_ms()
    ev.close()
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n
    assert ms.shape == (kda.BWD_NUM_STAGES,) and np.all(ms >= 0), ms
    assert ms[kda.BWD_STAGE_NAMES.index("chunk_gradients")] > 0, ms


def test_bwd_fp32_extreme_gates():
    """Single steps that decay by ~50 nats on ~10% of (token, channel) entries:
    the recomputation's block-split decay factors and the state passes stay
    finite and match the oracle's gradients."""
    _banner("bwd fp32 extreme gates")
    inp = to_device(synthetic.random_problem(42, 1, 260, 2, 128, 128, dtype=torch.float32,
                                             init_std=0.5, lengths=[150, 110]))
    gen = torch.Generator(device="cpu").manual_seed(8)
    spikes = torch.rand(inp["gate"].shape, generator=gen) < 0.1
    gate = inp["gate"].cpu()
    gate[spikes] = 30.0
    inp["gate"] = gate.to(DEV)
    inp["a_log"] = torch.full_like(inp["a_log"], 0.5)
    d_o, d_fin = _upstream(inp, 12)
    _run(inp, d_o, d_fin, torch.float32, "fp32 extreme gates")


def _max_block_decay(inp, head):
    """Largest decay of a 16-row block of 64-token chunks, over channels, for one
    head (plain in-kernel gate, documents from position 0 of each sequence)."""
    x = inp["gate"].float().cpu()[0, :, head] + inp["dt_bias"].float().cpu()[head]
    g = -torch.exp(inp["a_log"].float().cpu()[head]) * torch.nn.functional.softplus(x)
    g = torch.clamp(g, min=-110.0)
    cu = to_np(inp["cu_seqlens"]).astype(np.int64)
    worst = 0.0
    for s0, s1 in zip(cu[:-1], cu[1:]):
        for b in range(s0, s1, 16):
            worst = max(worst, float(-g[b:min(b + 16, s1)].sum(0).min()))
    return worst


@pytest.mark.parametrize("K", [128, 64])
def test_bwd_fp32_mixed_in_block_paths(K):
    """One call in which some chunk-heads keep the exact per-pair factors for
    the pairs inside 16-row blocks (a block decays by more than 60 nats in a
    channel: head 0) and the others take them on the matrix cores through the
    block boundary (head 1), at fp32 tolerance."""
    _banner("bwd fp32 mixed in-block paths K=%d" % K)
    inp = to_device(synthetic.random_problem(47, 1, 300, 2, K, 128, dtype=torch.float32,
                                             init_std=0.5, lengths=[170, 93, 37]))
    gen = torch.Generator(device="cpu").manual_seed(9)
    gate = inp["gate"].cpu()
    spikes = torch.rand(gate[:, :, 0].shape, generator=gen) < 0.15
    g0 = gate[:, :, 0]
    g0[spikes] = 30.0
    gate[:, :, 0] = g0
    inp["gate"] = gate.to(DEV)
    inp["a_log"] = torch.tensor([0.5, -1.0], device=DEV)
    assert _max_block_decay(inp, 0) > 60.0 and _max_block_decay(inp, 1) < 60.0
    d_o, d_fin = _upstream(inp, 19)
    _run(inp, d_o, d_fin, torch.float32, "fp32 mixed in-block paths")


# bf16 inputs recompute the chunk factors on the matrix-core chunk kernel
# (bf16 operands, fp32 accumulation); KDA_BWD_RECOMPUTE=valu keeps the fp32
# vector-ALU kernels.  Both are held to the bf16 tolerance above.
@pytest.mark.parametrize("C", [32, 16])
def test_bwd_bf16_short_chunks(C):
    _banner("bwd bf16 chunk %d" % C)
    inp = to_device(synthetic.random_problem(43, 1, 200, 2, 128, 128, dtype=torch.bfloat16,
                                             lengths=[77, 123], init_std=0.5))
    d_o, d_fin = _upstream(inp, 13)
    _run(inp, d_o, d_fin, torch.bfloat16, "bf16 chunk %d" % C, chunk_size=C)


def test_bwd_bf16_extreme_gates_exact_path():
    """The fp32 test's gate spikes in bf16: chunk-heads whose in-block decay
    leaves the factorised range go through the recomputation's exact fix-up."""
    _banner("bwd bf16 extreme gates")
    inp = to_device(synthetic.random_problem(42, 1, 260, 2, 128, 128, dtype=torch.bfloat16,
                                             init_std=0.5, lengths=[150, 110]))
    gen = torch.Generator(device="cpu").manual_seed(8)
    spikes = torch.rand(inp["gate"].shape, generator=gen) < 0.1
    gate = inp["gate"].float().cpu()
    gate[spikes] = 30.0
    inp["gate"] = gate.to(torch.bfloat16).to(DEV)
    inp["a_log"] = torch.full_like(inp["a_log"], 0.5)
    d_o, d_fin = _upstream(inp, 14)
    _run(inp, d_o, d_fin, torch.bfloat16, "bf16 extreme gates")


def test_bwd_bf16_clamped_gate():
    """The hard-clamp gate form in bf16 (the matrix-core recomputation's clamp
    instantiation), packed documents, no final-state gradient."""
    _banner("bwd bf16 clamp gate")
    inp = to_device(synthetic.random_problem(46, 1, 220, 2, 128, 128, dtype=torch.bfloat16,
                                             gate_std=3.0, lengths=[90, 130], init_std=0.5))
    d_o, _ = _upstream(inp, 17, with_final=False)
    _run(inp, d_o, None, torch.bfloat16, "bf16 clamp", lower_bound=-0.5, lower_bound_form="clamp")


@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (128, 64)])
def test_bwd_bf16_both_recomputations(monkeypatch, K, V):
    _banner("bwd bf16 recomputation kernels K=%d V=%d" % (K, V))
    inp = to_device(synthetic.random_problem(44, 1, 300, 2, K, V, dtype=torch.bfloat16,
                                             lengths=[64, 1, 129, 106], init_std=0.5))
    d_o, d_fin = _upstream(inp, 15)
    monkeypatch.delenv("KDA_BWD_RECOMPUTE", raising=False)
    _run(inp, d_o, d_fin, torch.bfloat16, "bf16 matrix-core recomputation", lower_bound=-4.0)
    monkeypatch.setenv("KDA_BWD_RECOMPUTE", "mfma32")
    _run(inp, d_o, d_fin, torch.bfloat16, "bf16 matrix-core recomputation, fp32 arrays",
         lower_bound=-4.0)
    monkeypatch.setenv("KDA_BWD_RECOMPUTE", "valu")
    _run(inp, d_o, d_fin, torch.bfloat16, "bf16 vector-ALU recomputation", lower_bound=-4.0)


def test_bwd_bf16_element_aligned_inputs(monkeypatch):
    """bf16 inputs that are 2-byte but not 16-byte aligned: the recomputation
    falls back to the vector-ALU kernels (the matrix-core one reads 8-byte
    pieces), bit for bit what KDA_BWD_RECOMPUTE=valu gives on aligned copies."""
    _banner("bwd bf16 element-aligned inputs")
    inp = to_device(synthetic.random_problem(45, 1, 150, 2, 128, 128, dtype=torch.bfloat16,
                                             lengths=[70, 80], init_std=0.5))
    d_o, d_fin = _upstream(inp, 16)

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        out = buf[1:].view(t.shape)
        out.copy_(t)
        assert out.data_ptr() % 16 != 0
        return out

    mis = dict(inp)
    for n in ("q", "k", "v", "gate", "beta"):
        mis[n] = shifted(inp[n])
    got, _ = _run(mis, shifted(d_o), d_fin, torch.bfloat16, "bf16 element-aligned")
    monkeypatch.setenv("KDA_BWD_RECOMPUTE", "valu")
    ref, _ = _run(inp, d_o, d_fin, torch.bfloat16, "bf16 aligned, vector-ALU recomputation")
    for n in NAMES:
        assert torch.equal(got[n], ref[n]), n
