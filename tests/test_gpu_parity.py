"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, element by element, plus the bit-exact properties
(chunk table, per-document independence, run-to-run repeatability)."""
import math

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_43_amd import kda, synthetic
from kda_testlib import assert_close, errors, gpu_fwd, oracle_fwd, to_device, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _banner(msg):
    print("[gpu-test] " + msg, flush=True)


# --------------------------------------------------------------------------
# workload 1: tiny fp32, whole output and final state
# --------------------------------------------------------------------------
def test_workload1_tiny_fp32():
    w = synthetic.WORKLOADS[1]
    _banner("workload 1 " + w.name)
    inp = to_device(synthetic.make_inputs(w, "cpu"))
    o, fin = gpu_fwd(inp)
    o_ref, f_ref = oracle_fwd(inp)
    assert_close(to_np(o), o_ref, torch.float32, "o")
    assert_close(to_np(fin), f_ref, torch.float32, "final_state")


# --------------------------------------------------------------------------
# workload 2: packed varlen bf16, checked per document
# --------------------------------------------------------------------------
def test_workload2_packed_varlen_per_document():
    w = synthetic.WORKLOADS[2]
    _banner("workload 2 " + w.name)
    inp = to_device(synthetic.make_inputs(w, "cpu"))
    cu = inp["cu_seqlens"].cpu().numpy()
    assert len(cu) == 8 and cu[-1] == 8192 and np.all(np.diff(cu) >= 64)
    o, fin = gpu_fwd(inp)
    o_ref, f_ref = oracle_fwd(inp)
    o = to_np(o)
    for n in range(len(cu) - 1):
        s = slice(cu[n], cu[n + 1])
        assert_close(o[:, s], o_ref[:, s], torch.bfloat16, "o doc %d" % n)
    assert_close(to_np(fin), f_ref, torch.bfloat16, "final_state")


# --------------------------------------------------------------------------
# small grid spanning several chunks and a ragged tail
# --------------------------------------------------------------------------
GRID = []
for dt in (torch.float32, torch.bfloat16):
    for (K, V) in ((64, 64), (128, 128), (64, 128), (128, 64)):
        for C in (16, 32, 64):
            for lb in (None, -5.0):
                GRID.append((dt, K, V, C, lb))


@pytest.mark.parametrize("dt,K,V,C,lb", GRID,
                         ids=lambda x: str(x).replace("torch.", ""))
def test_small_grid(dt, K, V, C, lb):
    seed = 100 + K + V + C + (7 if lb else 0) + (1 if dt == torch.float32 else 0)
    inp = synthetic.random_problem(seed, 2, 200, 3, K, V, dtype=dt, device=DEV, init_std=0.3,
                                   gate_std=2.0 if lb else 1.0)
    inp.update(scale=None, lower_bound=lb, chunk_size=C)
    o, fin = gpu_fwd(inp)
    o_ref, f_ref = oracle_fwd(inp)
    assert_close(to_np(o), o_ref, dt, "o")
    assert_close(to_np(fin), f_ref, dt, "final_state")


def test_scale_argument_is_used():
    inp = synthetic.random_problem(5, 1, 70, 2, 64, 64, dtype=torch.float32, device=DEV)
    inp.update(scale=0.37, lower_bound=None, chunk_size=64)
    o, _ = gpu_fwd(inp)
    o_ref, _ = oracle_fwd(inp)
    assert_close(to_np(o), o_ref, torch.float32, "o")


# --------------------------------------------------------------------------
# varlen edge cases: empty, 1-token, exactly-one-chunk and ragged documents
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("C", [16, 64])
def test_varlen_edge_documents(dt, C):
    lengths = [0, 1, 63, 64, 65, 0, 130, 7, 0]
    inp = synthetic.random_problem(11, 1, sum(lengths), 2, 64, 128, dtype=dt, device=DEV,
                                   init_std=0.5, lengths=lengths)
    inp.update(scale=None, lower_bound=-5.0, chunk_size=C)
    o, fin = gpu_fwd(inp)
    o_ref, f_ref = oracle_fwd(inp)
    assert_close(to_np(o), o_ref, dt, "o")
    assert_close(to_np(fin), f_ref, dt, "final_state")
    init = to_np(inp["initial_state"])
    for n, L in enumerate(lengths):
        if L == 0:
            assert np.array_equal(to_np(fin)[n], init[n]), "empty document must keep its state"


def test_varlen_without_host_copy_matches():
    lengths = [3, 70, 0, 128, 1, 40]
    inp = synthetic.random_problem(13, 1, sum(lengths), 2, 128, 128, dtype=torch.bfloat16,
                                   device=DEV, lengths=lengths)
    inp.update(scale=None, lower_bound=None, chunk_size=64)
    o1, f1 = gpu_fwd(inp, cu_seqlens_host=inp["cu_seqlens"].cpu())
    o2, f2 = gpu_fwd(inp)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_zero_length_sequence():
    inp = synthetic.random_problem(17, 2, 0, 2, 64, 64, dtype=torch.bfloat16, device=DEV,
                                   init_std=1.0)
    inp.update(scale=None, lower_bound=None, chunk_size=64)
    o, fin = gpu_fwd(inp)
    assert o.shape == (2, 0, 2, 64)
    assert torch.equal(fin, inp["initial_state"])
    o, fin = gpu_fwd(inp, initial_state=None)
    assert torch.count_nonzero(fin) == 0


def test_no_final_state_requested():
    inp = synthetic.random_problem(19, 1, 100, 2, 64, 64, dtype=torch.bfloat16, device=DEV)
    inp.update(scale=None, lower_bound=None, chunk_size=64)
    o, fin = gpu_fwd(inp, output_final_state=False)
    assert fin is None
    o_ref, _ = oracle_fwd(inp)
    assert_close(to_np(o), o_ref, torch.bfloat16, "o")


# --------------------------------------------------------------------------
# bit-exact: chunk table, document independence, repeatability
# --------------------------------------------------------------------------
def _expected_table(cu, C):
    tok, ln, seq0 = [], [], []
    for a, b in zip(cu[:-1], cu[1:]):
        seq0.append(len(tok))
        for t in range(a, b, C):
            tok.append(t)
            ln.append(min(C, b - t))
    seq0.append(len(tok))
    return tok, ln, seq0


@pytest.mark.parametrize("lengths,C", [
    ([5, 0, 64, 65, 1, 200], 64), ([1] * 50, 16), ([0, 0, 0], 32), ([4096], 64),
    (list(synthetic.lengths_uniform_until(1005, 32768, 1, 100)), 64),
])
@pytest.mark.parametrize("host", [True, False])
def test_chunk_table_bit_exact(lengths, C, host):
    cu = synthetic.cu_from_lengths(lengths)
    cu_dev = torch.from_numpy(cu).to(DEV)
    tok, ln, seq0 = kda.chunk_table(int(cu[-1]), C, cu_dev, cu_seqlens_host=cu if host else None)
    et, el, es = _expected_table(list(cu), C)
    assert tok.tolist() == et and ln.tolist() == el and seq0.tolist() == es


def test_chunk_table_rows():
    tok, ln, seq0 = kda.chunk_table(200, 64, None, B=3)
    et, el, es = [], [], [0]
    for b in range(3):
        for t in range(0, 200, 64):
            et.append(b * 200 + t)
            el.append(min(64, 200 - t))
        es.append(len(et))
    assert tok.tolist() == et and ln.tolist() == el and seq0.tolist() == es


def test_chunk_table_malformed_device_offsets_stay_in_range():
    """Without a host copy, malformed offsets are clamped: every chunk stays in the row."""
    cu = torch.tensor([0, 50, 20, 9999, -5, 100], dtype=torch.int32, device=DEV)
    tok, ln, seq0 = kda.chunk_table(100, 16, cu, cu_seqlens_host=False)
    assert len(tok) <= 100 // 16 + 5
    assert bool(((tok >= 0) & (tok + ln <= 100) & (ln >= 1) & (ln <= 16)).all())


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_document_independence_bitwise(dt):
    lengths = [37, 64, 1, 150, 90]
    inp = synthetic.random_problem(23, 1, sum(lengths), 2, 128, 64, dtype=dt, device=DEV,
                                   init_std=0.2, lengths=lengths)
    inp.update(scale=None, lower_bound=None, chunk_size=64)
    o, fin = gpu_fwd(inp)
    cu = inp["cu_seqlens"].cpu().tolist()
    for n in range(len(lengths)):
        s = slice(cu[n], cu[n + 1])
        sub = dict(inp)
        for key in ("q", "k", "v", "gate", "beta"):
            sub[key] = inp[key][:, s].contiguous()
        sub["cu_seqlens"] = None
        sub["initial_state"] = inp["initial_state"][n:n + 1].contiguous()
        on, fn = gpu_fwd(sub)
        assert torch.equal(o[:, s], on), "doc %d output differs from the document run alone" % n
        assert torch.equal(fin[n], fn[0])
    # perturbing document 1 leaves the others bit-identical
    pert = dict(inp)
    pert["v"] = inp["v"].clone()
    pert["v"][:, cu[1]:cu[2]] += 1
    o2, f2 = gpu_fwd(pert)
    assert torch.equal(o2[:, :cu[1]], o[:, :cu[1]]) and torch.equal(o2[:, cu[2]:], o[:, cu[2]:])


def test_repeatable_bitwise():
    inp = synthetic.random_problem(29, 2, 333, 4, 128, 128, dtype=torch.bfloat16, device=DEV,
                                   init_std=0.1)
    inp.update(scale=None, lower_bound=None, chunk_size=64)
    a = gpu_fwd(inp)
    b = gpu_fwd(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# --------------------------------------------------------------------------
# state summary / apply
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_state_summary_matches_oracle(dt):
    import oracle
    inp = synthetic.random_problem(31, 2, 150, 2, 64, 128, dtype=dt, device=DEV)
    E, P = kda.kda_state_summary(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"],
                                 inp["a_log"], inp["dt_bias"], chunk_size=64)
    torch.cuda.synchronize()
    Er, Pr = oracle.state_summary(*(to_np(inp[x]) for x in ("q", "k", "v", "gate", "beta", "a_log", "dt_bias")))
    assert_close(to_np(E), Er, dt, "state_ext")
    assert_close(to_np(P), Pr, dt, "transition")


def test_summary_composition_equals_whole_run():
    """Slices' summaries composed with apply equal the whole-row final state (fp32 tolerance)."""
    T, H, K, V = 640, 2, 128, 128
    inp = synthetic.random_problem(37, 1, T, H, K, V, dtype=torch.bfloat16, device=DEV,
                                   init_std=0.02)
    inp.update(scale=None, lower_bound=None, chunk_size=64)
    _, f_whole = gpu_fwd(inp)
    S = inp["initial_state"]
    for a in range(0, T, 128):
        sl = {key: inp[key][:, a:a + 128].contiguous() for key in ("q", "k", "v", "gate", "beta")}
        E, P = kda.kda_state_summary(sl["q"], sl["k"], sl["v"], sl["gate"], sl["beta"],
                                     inp["a_log"], inp["dt_bias"])
        S = kda.kda_apply_state_summary(E, P, S)
    torch.cuda.synchronize()
    maxabs, _ = errors(to_np(S), to_np(f_whole))
    assert maxabs <= 1e-4, maxabs


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_summary_composition_slow_decay(dt):
    """Composition where the slice transitions stay far from zero: a_log = -4
    makes A = e^-4, so a 128-token slice decays by about e^-1.5 per channel and
    the state entering each slice still shapes its end.  Each slice's summary
    is checked against the oracle's, and the chained composition against the
    oracle's whole-row final state and against the forward's."""
    T, H, K, V, S = 512, 2, 128, 128, 128
    inp = synthetic.random_problem(41, 1, T, H, K, V, dtype=dt, device=DEV, init_std=0.05)
    inp["a_log"] = torch.full_like(inp["a_log"], -4.0)
    inp.update(scale=None, lower_bound=None, chunk_size=64)
    _, f_whole = gpu_fwd(inp)
    np_in = {x: to_np(inp[x]) for x in ("q", "k", "v", "gate", "beta", "a_log", "dt_bias",
                                         "initial_state")}
    _, f_ref = oracle.kda_fwd(*(np_in[x] for x in ("q", "k", "v", "gate", "beta", "a_log",
                                                    "dt_bias")),
                              initial_state=np_in["initial_state"], want_output=False)
    St = inp["initial_state"]
    for a in range(0, T, S):
        sl = {x: inp[x][:, a:a + S].contiguous() for x in ("q", "k", "v", "gate", "beta")}
        E, P = kda.kda_state_summary(sl["q"], sl["k"], sl["v"], sl["gate"], sl["beta"],
                                     inp["a_log"], inp["dt_bias"])
        torch.cuda.synchronize()
        Er, Pr = oracle.state_summary(*(to_np(sl[x]) for x in ("q", "k", "v", "gate", "beta")),
                                      np_in["a_log"], np_in["dt_bias"])
        # the transition really is far from zero (its diagonal carries e^{gamma_L})
        assert np.abs(np.diagonal(Pr, axis1=-2, axis2=-1)).max() > 0.05
        assert_close(to_np(E), Er, dt, "state_ext, slice at %d" % a)
        assert_close(to_np(P), Pr, dt, "transition, slice at %d" % a)
        St = kda.kda_apply_state_summary(E, P, St)
    torch.cuda.synchronize()
    assert_close(to_np(St), f_ref, dt, "composed final state vs oracle")
    assert_close(to_np(St), to_np(f_whole), dt, "composed final state vs forward")


def test_apply_without_initial_state_is_state_ext():
    E = torch.randn(2, 3, 64, 128, device=DEV)
    P = torch.randn(2, 3, 64, 64, device=DEV)
    F = kda.kda_apply_state_summary(E, P, None)
    torch.cuda.synchronize()
    assert torch.equal(F, E)
    S0 = torch.randn(2, 3, 64, 128, device=DEV)
    F = kda.kda_apply_state_summary(E, P, S0)
    ref = (P.double() @ S0.double() + E.double()).cpu().numpy()
    assert errors(to_np(F), ref)[0] <= 1e-4


# --------------------------------------------------------------------------
# extreme decays: 16-row blocks whose decay leaves the factorised range
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dt,K,V", [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 64),
                                    (torch.float32, 128, 128), (torch.float32, 64, 64)],
                         ids=["bf16-128", "bf16-64", "f32-128", "f32-64"])
def test_extreme_gates_exact_diagonal(dt, K, V):
    """Gate logits of +30 on ~10% of (token, channel) entries make single steps
    decay by ~50 nats: in bf16 such blocks must take the exact in-block path;
    in fp32 the block-split decay factors of the off-diagonal products
    underflow to zero exactly where the true decay does."""
    inp = synthetic.random_problem(41, 1, 300, 2, K, V, dtype=dt, device=DEV,
                                   init_std=0.5, lengths=[170, 130])
    gen = torch.Generator(device="cpu").manual_seed(7)
    spikes = torch.rand(inp["gate"].shape, generator=gen) < 0.1
    gate = inp["gate"].float().cpu()
    gate[spikes] = 30.0
    inp["gate"] = gate.to(dt).to(DEV)
    inp["a_log"] = torch.full_like(inp["a_log"], 0.5)
    inp.update(scale=None, lower_bound=None, chunk_size=64)
    o, fin = gpu_fwd(inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(fin).all()
    o_ref, f_ref = oracle_fwd(inp)
    assert_close(to_np(o), o_ref, dt, "o")
    assert_close(to_np(fin), f_ref, dt, "final_state")


# ---------------------------------------------------------------------------
# Grouped value heads: q, k with H key heads, v/gate/beta/states with HV value
# heads, value head j reading key head j // (HV/H) (the shape contract of
# `_validate_projected_inputs` on the hyper_parallel page).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,K,V,chunk", [(torch.bfloat16, 128, 128, 64), (torch.bfloat16, 64, 64, 64),
                                             (torch.float32, 64, 64, 32)])
def test_grouped_value_heads_packed_documents(dtype, K, V, chunk):
    print("[gpu-test] grouped value heads %s K=%d V=%d chunk=%d" % (dtype, K, V, chunk), flush=True)
    lengths = [100, 37, 0, 170]
    inp = synthetic.random_problem(2101, 1, sum(lengths), 2, K, V, dtype=dtype, device=DEV,
                                   init_std=0.05, lengths=lengths, HV=6)
    inp["chunk_size"] = chunk
    o, fin = gpu_fwd(inp)
    assert o.shape == (1, sum(lengths), 6, V) and fin.shape == (4, 6, K, V)
    o_ref, f_ref = oracle_fwd(inp)
    assert_close(to_np(o), o_ref, dtype, "o")
    assert_close(to_np(fin), f_ref, dtype, "final_state")


def test_grouped_value_heads_rows_and_summary():
    print("[gpu-test] grouped value heads, rows + summary", flush=True)
    inp = synthetic.random_problem(2102, 2, 150, 2, 128, 128, dtype=torch.bfloat16, device=DEV, HV=4)
    o, fin = gpu_fwd(inp)
    o_ref, f_ref = oracle_fwd(inp)
    assert_close(to_np(o), o_ref, torch.bfloat16, "o")
    assert_close(to_np(fin), f_ref, torch.bfloat16, "final_state")
    E, P = kda.kda_state_summary(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"],
                                 inp["a_log"], inp["dt_bias"])
    torch.cuda.synchronize()
    E_ref, P_ref = oracle.state_summary(*(to_np(inp[x]) for x in ("q", "k", "v", "gate", "beta", "a_log", "dt_bias")))
    assert E.shape == (2, 4, 128, 128) and P.shape == (2, 4, 128, 128)
    assert_close(to_np(E), E_ref, torch.bfloat16, "state_ext")
    assert_close(to_np(P), P_ref, torch.bfloat16, "transition")


# ---------------------------------------------------------------------------
# The clamped lower-bounded gate, g = max(lb, -exp(a_log) softplus(x + b)), the
# alternative reading of the bounded gate.  Heavy-tailed gate logits and a
# tight bound make the clamp bind on a large share of the channels.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,chunk", [(torch.bfloat16, 64), (torch.float32, 64), (torch.float32, 16)])
def test_clamped_gate(dtype, chunk):
    print("[gpu-test] clamped gate %s chunk=%d" % (dtype, chunk), flush=True)
    lengths = [90, 1, 64, 129]
    inp = synthetic.random_problem(2103, 1, sum(lengths), 3, 64, 64, dtype=dtype, device=DEV,
                                   gate_std=3.0, beta_std=2.0, init_std=0.05, lengths=lengths)
    inp.update(lower_bound=-0.5, lower_bound_form="clamp", chunk_size=chunk)
    x = inp["gate"].float() + inp["dt_bias"][None, None]
    A = torch.exp(inp["a_log"])[None, None, :, None]
    g_free = -A * torch.nn.functional.softplus(x)
    frac = float((g_free < -0.5).float().mean())
    assert 0.2 < frac < 0.9, frac  # the clamp binds on a real share of the channels
    o, fin = gpu_fwd(inp)
    o_ref, f_ref = oracle_fwd(inp)
    assert_close(to_np(o), o_ref, dtype, "o")
    assert_close(to_np(fin), f_ref, dtype, "final_state")
    # and it is the clamp, not the sigmoid form: the result is several times
    # closer to the clamp oracle than to the sigmoid one
    o_sig, _ = oracle_fwd(dict(inp, lower_bound_form="sigmoid"))
    d_ref, _ = errors(to_np(o), o_ref)
    d_sig, _ = errors(to_np(o), o_sig)
    assert d_sig > 5e-3 and d_sig > 5 * d_ref, (d_sig, d_ref)


# --------------------------------------------------------------------------
# long rows with few (row, head) chains: every chain carries its state over
# 64 to 131 chunks (several record-staging rounds of the state pass, a ragged
# last chunk, grouped value heads)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("B,T,H,HV,K,V,init", [
    (2, 64 * 130 + 29, 2, 2, 128, 128, True),   # 131 chunks, ragged tail
    (1, 64 * 64, 1, 2, 64, 64, False),          # 64 chunks, grouped value heads
])
def test_long_rows_few_chains(B, T, H, HV, K, V, init):
    _banner("long rows B=%d T=%d HV=%d K=%d" % (B, T, HV, K))
    inp = to_device(synthetic.random_problem(61, B, T, H, K, V, dtype=torch.bfloat16, HV=HV,
                                             init_std=0.5 if init else None))
    o, fin = gpu_fwd(inp)
    o_ref, f_ref = oracle_fwd(inp)
    assert_close(to_np(o), o_ref, torch.bfloat16, "o")
    assert_close(to_np(fin), f_ref, torch.bfloat16, "final_state")
    # the output alone (no final state) is the same bits
    o2, _ = gpu_fwd(inp, output_final_state=False)
    assert torch.equal(o, o2)
