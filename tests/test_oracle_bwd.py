"""Pins of the oracle's backward (reverse mode of the token recurrence).

The gradients are checked against central finite differences of the oracle's
own forward in fp64, entry by entry, for every input (q, k, v, gate, beta
logit, a_log, dt_bias, initial state), under each gate form, with grouped
value heads, packed documents (one empty) and rows.  A finite difference is
independent of the reverse-mode code: a dropped term, a wrong sign or a
transposed operand anywhere in it moves some entry far outside the
difference's O(h^2) error.  Plus closed forms: zero upstream gradients give
zero gradients; with beta -> 0 and no decay the state never changes, so dv
vanishes and dq is the norm's Jacobian applied to scale * S0 d_o.
"""
import numpy as np
import pytest

import oracle

NAMES = ("q", "k", "v", "gate", "beta", "a_log", "dt_bias", "initial_state")
GRAD = {"q": "dq", "k": "dk", "v": "dv", "gate": "dgate", "beta": "dbeta", "a_log": "da_log",
        "dt_bias": "ddt_bias", "initial_state": "dinit"}


def _problem(seed, B, T, HK, H, K, V, lengths=None):
    rng = np.random.default_rng(seed)
    p = dict(q=rng.standard_normal((B, T, HK, K)), k=rng.standard_normal((B, T, HK, K)),
             v=rng.standard_normal((B, T, H, V)), gate=rng.standard_normal((B, T, H, K)),
             beta=rng.standard_normal((B, T, H)), a_log=rng.uniform(-1, 1, H),
             dt_bias=0.3 * rng.standard_normal((H, K)))
    cu = None
    N = B
    if lengths is not None:
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        N = len(lengths)
    p["initial_state"] = 0.5 * rng.standard_normal((N, H, K, V))
    d_o = rng.standard_normal((B, T, H, V))
    d_fin = rng.standard_normal((N, H, K, V))
    return p, cu, d_o, d_fin


def _loss(p, cu, d_o, d_fin, kw):
    o, fin = oracle.kda_fwd(p["q"], p["k"], p["v"], p["gate"], p["beta"], p["a_log"], p["dt_bias"],
                            cu_seqlens=cu, initial_state=p["initial_state"], threads=1, **kw)
    return float(np.sum(o * d_o) + np.sum(fin * d_fin))


def _check_fd(p, cu, d_o, d_fin, kw, h=1e-6, rtol=1e-6, atol=1e-7):
    g = oracle.kda_bwd(p["q"], p["k"], p["v"], p["gate"], p["beta"], p["a_log"], p["dt_bias"], d_o,
                       d_fin, cu_seqlens=cu, initial_state=p["initial_state"], threads=1, **kw)
    for name in NAMES:
        x = p[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = _loss(p, cu, d_o, d_fin, kw)
            x[idx] = keep - h
            lm = _loss(p, cu, d_o, d_fin, kw)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        got = g[GRAD[name]]
        assert got.shape == fd.shape, name
        err = np.abs(got - fd)
        assert np.all(err <= atol + rtol * np.abs(fd)), "%s: max err %.3g (at %s), |fd| max %.3g" % (
            name, err.max(), np.unravel_index(np.argmax(err), err.shape), np.abs(fd).max())


@pytest.mark.parametrize("gate_mode,lb", [("softplus", None), ("sigmoid", -2.0), ("clamp", -0.7)])
def test_bwd_matches_finite_differences_rows(gate_mode, lb):
    p, cu, d_o, d_fin = _problem(1, B=2, T=6, HK=2, H=2, K=3, V=2)
    _check_fd(p, cu, d_o, d_fin, dict(gate_mode=gate_mode, lower_bound=lb, scale=0.7))


def test_bwd_matches_finite_differences_grouped_packed():
    p, cu, d_o, d_fin = _problem(2, B=1, T=9, HK=1, H=3, K=3, V=2, lengths=[4, 0, 5])
    _check_fd(p, cu, d_o, d_fin, dict(gate_mode="sigmoid", lower_bound=-1.5))


def test_clamped_entries_have_no_gate_gradient():
    p, cu, d_o, d_fin = _problem(3, B=1, T=5, HK=1, H=1, K=4, V=2)
    p["gate"][0, :, 0, :2] = 3.0   # -exp(a_log) softplus(3 + b) < -0.4: clamped
    p["a_log"][:] = 0.5
    p["dt_bias"][:] = 0.0
    g = oracle.kda_bwd(p["q"], p["k"], p["v"], p["gate"], p["beta"], p["a_log"], p["dt_bias"], d_o,
                       d_fin, initial_state=p["initial_state"], gate_mode="clamp", lower_bound=-0.4)
    assert np.all(g["dgate"][0, :, 0, :2] == 0.0)
    assert np.any(g["dgate"][0, :, 0, 2:] != 0.0)
    _check_fd(p, cu, d_o, d_fin, dict(gate_mode="clamp", lower_bound=-0.4))


def test_zero_upstream_gives_zero_gradients():
    p, cu, d_o, d_fin = _problem(4, B=1, T=7, HK=2, H=2, K=4, V=3)
    g = oracle.kda_bwd(p["q"], p["k"], p["v"], p["gate"], p["beta"], p["a_log"], p["dt_bias"],
                       np.zeros_like(d_o), None, initial_state=p["initial_state"])
    for name, arr in g.items():
        assert np.all(arr == 0.0), name


def test_no_update_no_decay_closed_form():
    """beta -> 0 and a decay of exactly 1 (sigmoid gate with a bound so small that
    g underflows to -0 is not available, so take the softplus gate with
    a_log -> -inf): S_t = S0 for all t, o_t = scale S0^T q^_t.  Then dv = 0,
    d(initial) = scale sum_t q^_t d_o_t^T + d_final, and dq is the L2 norm's
    Jacobian applied to scale S0 d_o_t."""
    rng = np.random.default_rng(5)
    B, T, H, K, V = 1, 4, 1, 3, 2
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    gate = rng.standard_normal((B, T, H, K))
    beta = np.full((B, T, H), -800.0)          # sigmoid(-800) = 0 in fp64
    a_log = np.full(H, -800.0)                 # exp(-800) = 0: g = -0
    dt_bias = np.zeros((H, K))
    S0 = rng.standard_normal((1, H, K, V))
    d_o = rng.standard_normal((B, T, H, V))
    d_fin = rng.standard_normal((1, H, K, V))
    scale = 0.6
    g = oracle.kda_bwd(q, k, v, gate, beta, a_log, dt_bias, d_o, d_fin, scale=scale, initial_state=S0)
    assert np.all(g["dv"] == 0.0)
    qn = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + 1e-6)
    dinit = scale * np.einsum("tk,tv->kv", qn[0, :, 0], d_o[0, :, 0]) + d_fin[0, 0]
    np.testing.assert_allclose(g["dinit"][0, 0], dinit, rtol=1e-12, atol=1e-12)
    for t in range(T):
        x = q[0, t, 0]
        nr = np.sqrt(x @ x + 1e-6)
        jac = np.eye(K) / nr - np.outer(x, x) / nr ** 3
        dqn = scale * S0[0, 0] @ d_o[0, t, 0]
        np.testing.assert_allclose(g["dq"][0, t, 0], jac @ dqn, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("C,lengths", [(4, None), (3, [5, 0, 1, 6])])
def test_chunked_backward_matches_finite_differences_of_the_recurrence(C, lengths):
    """The chunked reverse mode (the decomposition of the GPU backward) against
    central differences of the token recurrence, for the normalised inputs,
    the log-decay, beta and the initial state."""
    from oracle import chunked
    rng = np.random.default_rng(8)
    B, H, K, V = (2, 2, 3, 2) if lengths is None else (1, 1, 3, 2)
    T = 9 if lengths is None else sum(lengths)
    cu = None if lengths is None else np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = B if cu is None else len(lengths)
    x = dict(qn=rng.standard_normal((B, T, H, K)), kn=rng.standard_normal((B, T, H, K)) * 0.6,
             v=rng.standard_normal((B, T, H, V)), g=-np.log1p(np.exp(rng.standard_normal((B, T, H, K)))),
             b=1 / (1 + np.exp(-rng.standard_normal((B, T, H)))),
             init=rng.standard_normal((N, H, K, V)))
    d_o = rng.standard_normal((B, T, H, V))
    d_fin = rng.standard_normal((N, H, K, V))
    scale = 0.8

    def loss():
        o, fin = oracle.recurrence(x["qn"], x["kn"], x["v"], x["g"], x["b"], scale, cu_seqlens=cu,
                                   initial_state=x["init"], threads=1)
        return float(np.sum(o * d_o) + np.sum(fin * d_fin))

    got = chunked.kda_bwd_chunked(x["qn"], x["kn"], x["v"], x["g"], x["b"], d_o, d_fin, scale, C,
                                  cu_seqlens=cu, initial_state=x["init"])
    names = {"qn": "dqn", "kn": "dkn", "v": "dv", "g": "dg", "b": "db", "init": "dinit"}
    h = 1e-6
    for name, key in names.items():
        arr = x[name]
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            lp = loss()
            arr[idx] = keep - h
            lm = loss()
            arr[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(got[key], fd, rtol=1e-6, atol=1e-7, err_msg=name)
