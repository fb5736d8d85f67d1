"""Pins for the CPU oracle: it is checked here against things other than itself.

* hand-derived worked examples (tests/golden/*.json, each with its citation);
* brute force: explicit K x K transition matrices and their products;
* closed forms and invariants of the recurrence (no decay/no update, orthogonal
  overwrite, full decay, document resets, slice composition, contractivity);
* the chunk-parallel fp64 form (oracle/chunked.py) against the token loop.

A plausible mistake in the oracle (decay after the update, output read before
the update, a transposed state, a dropped beta, a wrong gate form, state not
reset at a document start, a transposed transition) fails at least one test.
"""
import glob
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, B, T, H, K, V, gate_std=1.0, beta_std=1.0):
    r = np.random.default_rng(seed)
    return dict(
        q=r.standard_normal((B, T, H, K)).astype(np.float32),
        k=r.standard_normal((B, T, H, K)).astype(np.float32),
        v=r.standard_normal((B, T, H, V)).astype(np.float32),
        gate=(r.standard_normal((B, T, H, K)) * gate_std).astype(np.float32),
        beta=(r.standard_normal((B, T, H)) * beta_std).astype(np.float32),
        a_log=r.uniform(-1, 1, H).astype(np.float32),
        dt_bias=(r.standard_normal((H, K)) * 0.1).astype(np.float32),
    )


# --------------------------------------------------------------------------
# worked examples
# --------------------------------------------------------------------------
def _golden_files():
    return sorted(glob.glob(os.path.join(GOLDEN, "*.json")))


@pytest.mark.parametrize("path", _golden_files(), ids=os.path.basename)
def test_golden_worked_example(path):
    d = json.load(open(path))
    B, T, H, K, V = d["B"], d["T"], d["H"], d["K"], d["V"]
    if "k_slots" in d:  # one-hot construction
        q = np.zeros((B, T, H, K), np.float32)
        k = np.zeros((B, T, H, K), np.float32)
        for t, s in enumerate(d["k_slots"]):
            k[0, t, 0, s] = 1e6
        for t, s in enumerate(d["q_slots"]):
            q[0, t, 0, s] = 1e6
        v = np.asarray(d["v"], np.float32).reshape(B, T, H, V)
        gate = np.zeros((B, T, H, K), np.float32)
        beta = np.full((B, T, H), np.inf, np.float32)
        a_log = np.full((H,), -np.inf, np.float32)
        dt_bias = np.zeros((H, K), np.float32)
        init = np.asarray(d["initial_state"], np.float32).reshape(1, H, K, V)
        o, fin = oracle.kda_fwd(q, k, v, gate, beta, a_log, dt_bias, scale=1.0,
                                initial_state=init, threads=1)
    else:
        arr = lambda name, shape: np.asarray(d[name], np.float32).reshape(shape)
        init = None if d["initial_state"] is None else arr("initial_state", (B, H, K, V))
        o, fin = oracle.kda_fwd(arr("q", (B, T, H, K)), arr("k", (B, T, H, K)),
                                arr("v", (B, T, H, V)), arr("gate", (B, T, H, K)),
                                arr("beta", (B, T, H)), arr("a_log", (H,)),
                                arr("dt_bias", (H, K)), scale=d["scale"],
                                lower_bound=d["lower_bound"], gate_mode=d["gate_mode"],
                                initial_state=init, threads=1)
    exp_o = np.asarray(d["expected_o"], np.float64).reshape(o.shape)
    exp_f = np.asarray(d["expected_final"], np.float64).reshape(fin.shape)
    tol = d["tol"]
    assert np.max(np.abs(o - exp_o)) <= tol, (o.ravel(), exp_o.ravel())
    assert np.max(np.abs(fin - exp_f)) <= tol, (fin.ravel(), exp_f.ravel())


# --------------------------------------------------------------------------
# prologue closed forms
# --------------------------------------------------------------------------
def test_prologue_closed_forms():
    # gate logits x with a_log = 0 (A = 1), dt_bias = 0
    xs = np.array([0.0, math.log(3.0), 50.0, -50.0, -1.0], np.float32)
    K = len(xs)
    q = np.array([3.0, 4.0, 0.0, 0.0, 0.0], np.float32).reshape(1, 1, 1, K)
    k = np.zeros((1, 1, 1, K), np.float32)            # zero vector -> zero, not NaN
    gate = xs.reshape(1, 1, 1, K)
    beta = np.array([0.0], np.float32).reshape(1, 1, 1)
    a0 = np.zeros(1, np.float32)
    db = np.zeros((1, K), np.float32)
    qn, kn, g, b = oracle.prologue(q, k, gate, beta, a0, db)
    # q^ = q / sqrt(25 + 1e-6)
    np.testing.assert_allclose(qn.ravel()[:2], [3 / math.sqrt(25 + 1e-6), 4 / math.sqrt(25 + 1e-6)],
                               rtol=1e-15)
    assert np.all(kn == 0.0) and np.all(np.isfinite(kn))
    assert b.ravel()[0] == 0.5
    xs64 = xs.astype(np.float64)
    # softplus: ln2, ln4, ~50, ~e^-50, ln(1+e^-1)
    want = -np.array([math.log(2), math.log(1 + math.exp(xs64[1])), 50 + math.log1p(math.exp(-50)),
                      math.log1p(math.exp(-50)), math.log1p(math.exp(-1))])
    np.testing.assert_allclose(g.ravel(), want, rtol=1e-14)
    # a_log shifts the slope: A = e^{a_log}; dt_bias shifts the argument
    a1 = np.array([math.log(2.0)], np.float32)
    db1 = np.full((1, K), 1.0, np.float32)
    _, _, g1, _ = oracle.prologue(q, k, gate, beta, a1, db1)
    want1 = -math.exp(float(a1[0])) * np.array([math.log1p(math.exp(x + 1.0)) for x in xs64])
    np.testing.assert_allclose(g1.ravel(), want1, rtol=1e-13)
    # sigmoid bound: g = lb * sigmoid(A (x + dt_bias))
    lb = -5.0
    _, _, g2, _ = oracle.prologue(q, k, gate, beta, a1, db1, lower_bound=lb)
    A = math.exp(float(a1[0]))
    want2 = np.array([lb / (1 + math.exp(-A * (x + 1.0))) for x in xs64])
    np.testing.assert_allclose(g2.ravel(), want2, rtol=1e-14)
    # clamp reading
    _, _, g3, _ = oracle.prologue(q, k, gate, beta, a1, db1, lower_bound=lb, gate_mode="clamp")
    np.testing.assert_allclose(g3.ravel(), np.maximum(lb, want1), rtol=1e-14)


def test_prologue_ranges():
    d = _rand(1, 2, 64, 3, 16, 8, gate_std=3.0, beta_std=3.0)
    qn, kn, g, b = oracle.prologue(d["q"], d["k"], d["gate"], d["beta"], d["a_log"], d["dt_bias"])
    np.testing.assert_allclose(np.linalg.norm(qn, axis=-1), 1.0, atol=1e-6)
    np.testing.assert_allclose(np.linalg.norm(kn, axis=-1), 1.0, atol=1e-6)
    assert np.all(g < 0) and np.all((b > 0) & (b < 1))
    _, _, g2, _ = oracle.prologue(d["q"], d["k"], d["gate"], d["beta"], d["a_log"], d["dt_bias"],
                                  lower_bound=-5.0)
    assert np.all((g2 > -5.0) & (g2 < 0))
    with pytest.raises(ValueError):
        oracle.prologue(d["q"], d["k"], d["gate"], d["beta"], d["a_log"], d["dt_bias"],
                        lower_bound=0.5, gate_mode="sigmoid")


# --------------------------------------------------------------------------
# brute force: explicit transition matrices
# --------------------------------------------------------------------------
def _brute(qn, kn, v, g, b, scale, S0):
    """o_t and S_T from explicit products of A_t = (I - b k k^T) Diag(e^g)."""
    T, K = qn.shape
    A = [(np.eye(K) - b[t] * np.outer(kn[t], kn[t])) @ np.diag(np.exp(g[t])) for t in range(T)]
    o = []
    for t in range(T):
        # S_t = (A_t..A_0) S0 + sum_{s<=t} (A_t..A_{s+1}) b_s k_s v_s^T
        prod = np.eye(K)
        for s in range(t, -1, -1):
            prod = prod @ A[s]
        S = prod @ S0
        for s in range(t + 1):
            after = np.eye(K)
            for r in range(t, s, -1):
                after = after @ A[r]
            S = S + after @ (b[s] * np.outer(kn[s], v[s]))
        o.append(scale * S.T @ qn[t])
    return np.array(o), S


@pytest.mark.parametrize("mode", ["softplus", "sigmoid"])
def test_brute_force_matrix_products(mode):
    B, T, H, K, V = 1, 7, 2, 4, 3
    d = _rand(7, B, T, H, K, V)
    lb = -5.0 if mode == "sigmoid" else None
    r = np.random.default_rng(3)
    S0 = r.standard_normal((B, H, K, V)).astype(np.float32)
    qn, kn, g, b = oracle.prologue(d["q"], d["k"], d["gate"], d["beta"], d["a_log"], d["dt_bias"],
                                   lower_bound=lb)
    o_raw, f_raw = oracle.kda_fwd(**d, scale=0.7, lower_bound=lb, initial_state=S0, threads=2)
    o_rec, f_rec = oracle.recurrence(qn, kn, d["v"], g, b, 0.7, initial_state=S0)
    for h in range(H):
        ob, Sb = _brute(qn[0, :, h], kn[0, :, h], d["v"][0, :, h].astype(np.float64),
                        g[0, :, h], b[0, :, h], 0.7, S0[0, h].astype(np.float64))
        np.testing.assert_allclose(o_raw[0, :, h], ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(o_rec[0, :, h], ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(f_raw[0, h], Sb, rtol=0, atol=1e-12)
        np.testing.assert_allclose(f_rec[0, h], Sb, rtol=0, atol=1e-12)


def test_brute_force_transition_summary():
    B, T, H, K, V = 2, 6, 2, 3, 2
    d = _rand(11, B, T, H, K, V)
    qn, kn, g, b = oracle.prologue(d["q"], d["k"], d["gate"], d["beta"], d["a_log"], d["dt_bias"])
    E, P = oracle.state_summary(**d)
    for bb in range(B):
        for h in range(H):
            prod = np.eye(K)
            for t in range(T):   # later tokens on the left
                A = (np.eye(K) - b[bb, t, h] * np.outer(kn[bb, t, h], kn[bb, t, h])) @ np.diag(np.exp(g[bb, t, h]))
                prod = A @ prod
            np.testing.assert_allclose(P[bb, h], prod, atol=1e-13)
            _, Sb = _brute(qn[bb, :, h], kn[bb, :, h], d["v"][bb, :, h].astype(np.float64),
                           g[bb, :, h], b[bb, :, h], 1.0, np.zeros((K, V)))
            np.testing.assert_allclose(E[bb, h], Sb, atol=1e-13)


# --------------------------------------------------------------------------
# invariants and closed forms
# --------------------------------------------------------------------------
def test_no_decay_no_update_keeps_state():
    """g = 0 and beta = 0 leave S unchanged, so o_t = scale * S0^T q^_t."""
    B, T, H, K, V = 1, 20, 2, 8, 5
    d = _rand(5, B, T, H, K, V)
    d["a_log"][:] = -np.inf          # A = 0  ->  g = -0
    d["beta"][:] = -np.inf           # beta = 0
    S0 = np.random.default_rng(1).standard_normal((1, H, K, V)).astype(np.float32)
    o, fin = oracle.kda_fwd(**d, scale=0.3, initial_state=S0)
    qn, _, g, b = oracle.prologue(d["q"], d["k"], d["gate"], d["beta"], d["a_log"], d["dt_bias"])
    assert np.all(g == 0) and np.all(b == 0)
    want = 0.3 * np.einsum("thk,hkv->thv", qn[0], S0[0].astype(np.float64))
    np.testing.assert_allclose(o[0], want, atol=1e-14)
    assert np.array_equal(fin, S0.astype(np.float64))


def test_orthogonal_overwrite():
    """beta = 1, unit keys, no decay: S_t^T k_t = v_t and S_t^T x = S_{t-1}^T x for x orthogonal to k_t."""
    K, V, T = 6, 4, 12
    r = np.random.default_rng(9)
    Q, _ = np.linalg.qr(r.standard_normal((K, K)))
    slots = r.integers(0, K, T)
    kn = Q[:, slots].T.copy()                    # orthonormal key directions
    qn = Q[:, r.integers(0, K, T)].T.copy()
    v = r.standard_normal((T, V)).astype(np.float32)
    g = np.zeros((T, K))
    b = np.ones(T)
    S0 = r.standard_normal((K, V)).astype(np.float32)
    o, fin = oracle.recurrence(qn[None, :, None], kn[None, :, None], v[None, :, None], g[None, :, None],
                               b[None, :, None], 1.0, initial_state=S0[None, None])
    # closed form: reading direction j returns the last value written along it, else S0^T e_j
    mem = {j: Q[:, j] @ S0.astype(np.float64) for j in range(K)}
    for t in range(T):
        mem[slots[t]] = v[t].astype(np.float64)
        qs = int(np.argmax(np.abs(Q.T @ qn[t])))
        np.testing.assert_allclose(o[0, t, 0], mem[qs], atol=1e-12)
    want_fin = sum(np.outer(Q[:, j], mem[j]) for j in range(K))
    np.testing.assert_allclose(fin[0, 0], want_fin, atol=1e-12)


def test_full_decay_makes_state_rank_one():
    """g = -inf (softplus of +inf) with beta = 1: S_t = k^_t v_t^T, o_t = scale (k^_t . q^_t) v_t."""
    B, T, H, K, V = 1, 9, 2, 5, 3
    d = _rand(13, B, T, H, K, V)
    d["gate"][:] = np.inf
    d["beta"][:] = np.inf
    S0 = np.ones((1, H, K, V), np.float32)
    o, fin = oracle.kda_fwd(**d, scale=0.5, initial_state=S0)
    qn, kn, _, _ = oracle.prologue(d["q"], d["k"], d["gate"], d["beta"], d["a_log"], d["dt_bias"])
    dots = np.einsum("bthk,bthk->bth", qn, kn)
    np.testing.assert_allclose(o, 0.5 * dots[..., None] * d["v"].astype(np.float64), atol=1e-14)
    np.testing.assert_allclose(fin[0], np.einsum("hk,hv->hkv", kn[0, -1], d["v"][0, -1]), atol=1e-14)


def test_default_scale_and_linearity():
    d = _rand(17, 1, 10, 2, 16, 4)
    o1, _ = oracle.kda_fwd(**d)
    o2, _ = oracle.kda_fwd(**d, scale=1.0 / 4.0)
    o3, _ = oracle.kda_fwd(**d, scale=0.5)
    assert np.array_equal(o1, o2)
    np.testing.assert_allclose(o3, 2.0 * o2, rtol=1e-15, atol=0)


def test_document_resets_bitwise():
    """Each document of a pack equals the same document run alone, bit for bit,
    and perturbing one document leaves its neighbours untouched."""
    H, K, V = 2, 8, 6
    lengths = [5, 0, 13, 1, 9]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    d = _rand(21, 1, T, H, K, V)
    r = np.random.default_rng(4)
    init = r.standard_normal((len(lengths), H, K, V)).astype(np.float32)
    o, fin = oracle.kda_fwd(**d, cu_seqlens=cu, initial_state=init)
    for n, L in enumerate(lengths):
        s = slice(cu[n], cu[n + 1])
        dn = {key: (val[:, s] if val.ndim >= 3 else val) for key, val in d.items()}
        on, fn = oracle.kda_fwd(**dn, initial_state=init[n:n + 1])
        assert np.array_equal(o[:, s], on)
        assert np.array_equal(fin[n], fn[0])
    assert np.array_equal(fin[1], init[1].astype(np.float64))  # empty document
    d2 = {key: val.copy() for key, val in d.items()}
    d2["v"][:, cu[2]:cu[3]] += 1.0
    o2, fin2 = oracle.kda_fwd(**d2, cu_seqlens=cu, initial_state=init)
    assert np.array_equal(o2[:, cu[3]:], o[:, cu[3]:]) and np.array_equal(o2[:, :cu[2]], o[:, :cu[2]])
    assert not np.array_equal(o2[:, cu[2]:cu[3]], o[:, cu[2]:cu[3]])
    assert np.array_equal(fin2[3:], fin[3:])


@pytest.mark.parametrize("lb", [None, -5.0])
def test_slice_summaries_compose(lb):
    """apply(summary(slice)) chained over contiguous slices equals the whole run,
    and carrying final_state into initial_state equals the whole run."""
    B, T, H, K, V = 1, 96, 2, 8, 6
    d = _rand(23, B, T, H, K, V)
    S0 = np.random.default_rng(5).standard_normal((1, H, K, V)).astype(np.float32) * 0.1
    o_all, f_all = oracle.kda_fwd(**d, lower_bound=lb, initial_state=S0)
    cuts = [0, 17, 40, 41, 96]
    S = S0.astype(np.float64)
    Sc = S0
    outs = []
    for a, bnd in zip(cuts[:-1], cuts[1:]):
        ds = {key: (val[:, a:bnd] if val.ndim >= 3 else val) for key, val in d.items()}
        E, P = oracle.state_summary(**ds, lower_bound=lb)
        S = oracle.apply_state_summary(E, P, S)
        o_s, f_s = oracle.kda_fwd(**ds, lower_bound=lb, initial_state=Sc)
        outs.append(o_s)
        Sc = f_s.astype(np.float32)  # carried through fp32 like the state tensor
    np.testing.assert_allclose(S, f_all, atol=1e-10)
    np.testing.assert_allclose(np.concatenate(outs, axis=1), o_all, atol=1e-5)
    E, P = oracle.state_summary(**d, lower_bound=lb)
    assert np.array_equal(oracle.apply_state_summary(E, P, None), E)


def test_contractivity_bound():
    """Every factor (I - b k k^T) Diag(e^g) has spectral norm <= 1, so the state
    norm is bounded by ||S0|| + sum_t b_t ||k^_t|| ||v_t||."""
    B, T, H, K, V = 1, 200, 3, 16, 16
    d = _rand(29, B, T, H, K, V, gate_std=0.1)
    d["a_log"][:] = -4.0          # weak decay: the bound is nearly tight in places
    S0 = np.random.default_rng(6).standard_normal((1, H, K, V)).astype(np.float32)
    _, fin = oracle.kda_fwd(**d, initial_state=S0)
    _, kn, _, b = oracle.prologue(d["q"], d["k"], d["gate"], d["beta"], d["a_log"], d["dt_bias"])
    for h in range(H):
        bound = np.linalg.norm(S0[0, h]) + np.sum(
            b[0, :, h] * np.linalg.norm(kn[0, :, h], axis=-1) * np.linalg.norm(d["v"][0, :, h], axis=-1))
        assert np.linalg.norm(fin[0, h]) <= bound * (1 + 1e-12)


def test_threads_do_not_change_results():
    d = _rand(31, 2, 40, 5, 8, 8)
    a = oracle.kda_fwd(**d, threads=1)
    b = oracle.kda_fwd(**d, threads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# --------------------------------------------------------------------------
# the chunk algebra the kernels follow equals the token recurrence
# --------------------------------------------------------------------------
@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("lb", [None, -5.0])
def test_chunked_form_matches_recurrence(C, lb):
    H, K, V = 2, 8, 6
    lengths = [70, 1, 33, 64, 0, 17]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    d = _rand(37 + C, 1, T, H, K, V, gate_std=2.0)
    init = np.random.default_rng(8).standard_normal((len(lengths), H, K, V)).astype(np.float32)
    qn, kn, g, b = oracle.prologue(d["q"], d["k"], d["gate"], d["beta"], d["a_log"], d["dt_bias"],
                                   lower_bound=lb)
    o_ref, f_ref = oracle.recurrence(qn, kn, d["v"], g, b, 0.35, cu_seqlens=cu, initial_state=init)
    o_chk, f_chk = chunked.kda_fwd_chunked(qn, kn, d["v"], g, b, 0.35, C, cu_seqlens=cu,
                                           initial_state=init)
    np.testing.assert_allclose(o_chk, o_ref, atol=1e-10)
    np.testing.assert_allclose(f_chk, f_ref, atol=1e-10)


def test_grouped_value_heads_equal_repeated_key_heads():
    """Grouped value heads (hyper_parallel page, `_validate_projected_inputs`:
    v/gate/beta carry HV heads, a multiple of the H heads of q and k).  Under the
    reading that value head j uses key head j // (HV/H), a grouped run must equal
    the ungrouped run on q and k repeated along the head axis, bit for bit (the
    same fp64 operations), for the forward and for the state summary.  A modulo
    mapping (j % H) or a swapped group order fails this for G, H > 1."""
    rng = np.random.default_rng(7)
    B, T, HK, G, K, V = 2, 29, 2, 3, 8, 5
    H = HK * G
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    q, k = f(B, T, HK, K), f(B, T, HK, K)
    v, gate, beta = f(B, T, H, V), f(B, T, H, K), f(B, T, H)
    a_log = rng.uniform(-1, 1, H).astype(np.float32)
    dt_bias = (0.1 * f(H, K)).astype(np.float32)
    init = f(B, H, K, V)
    qr, kr = np.repeat(q, G, axis=2), np.repeat(k, G, axis=2)
    for lb, mode in ((None, None), (-3.0, "sigmoid"), (-3.0, "clamp")):
        o1, f1 = oracle.kda_fwd(q, k, v, gate, beta, a_log, dt_bias, lower_bound=lb, gate_mode=mode,
                                initial_state=init, threads=2)
        o2, f2 = oracle.kda_fwd(qr, kr, v, gate, beta, a_log, dt_bias, lower_bound=lb, gate_mode=mode,
                                initial_state=init, threads=2)
        assert np.array_equal(o1, o2) and np.array_equal(f1, f2)
        E1, P1 = oracle.state_summary(q, k, v, gate, beta, a_log, dt_bias, lower_bound=lb, gate_mode=mode)
        E2, P2 = oracle.state_summary(qr, kr, v, gate, beta, a_log, dt_bias, lower_bound=lb, gate_mode=mode)
        assert np.array_equal(E1, E2) and np.array_equal(P1, P2)
    # the key heads matter: changing key head 1 changes exactly value heads G..2G-1
    q2 = q.copy()
    q2[:, :, 1] += 1.0
    o3, _ = oracle.kda_fwd(q2, k, v, gate, beta, a_log, dt_bias, threads=2)
    o1, _ = oracle.kda_fwd(q, k, v, gate, beta, a_log, dt_bias, threads=2)
    changed = [j for j in range(H) if not np.array_equal(o1[:, :, j], o3[:, :, j])]
    assert changed == list(range(G, 2 * G))
