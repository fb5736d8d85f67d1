"""Pins of the oracle's short convolution + SiLU (the step before the forward).

The layer's ShortConv, as the hyper_parallel coverage page runs it
(`_run_causal_short_conv`, `_local_short_conv`) and constrains it
(`_validate_layer_short_conv`): a depthwise conv1d with stride 1, dilation 1,
zero padding of W-1 on the left, output cut to the sequence length, then SiLU;
without the convolution, SiLU alone.  The oracle computes it with plain loops;
these tests pin it to
  - the library convolution called exactly the way the page calls it (fp64),
  - closed forms: an identity tap gives SiLU(x), a tap s steps back gives
    SiLU(x shifted by s) with zeros before the sequence start,
  - SiLU's own special values (silu(0) = 0, silu(+-ln 3) = +-ln 3 * 3/4 or 1/4),
  - the packed reading: each document of a packed row equals the same tokens
    run as a row of their own.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _page_conv_silu(x, w, b):
    """The page's call, on one row set [B,T,C], in fp64 with torch CPU ops."""
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    C, W = w.shape
    wt = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float64)).reshape(C, 1, W)
    bt = None if b is None else torch.from_numpy(np.ascontiguousarray(b, dtype=np.float64))
    out = F.conv1d(xt.transpose(1, 2), wt, bt, stride=1, padding=W - 1, dilation=1, groups=C)
    out = out[:, :, : x.shape[1]]
    return F.silu(out).transpose(1, 2).numpy()


@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("with_bias", [False, True])
def test_rows_match_library_conv(W, with_bias):
    rng = np.random.default_rng(100 + W)
    B, T, C = 3, 23, 10
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal((C, W))
    b = rng.standard_normal(C) if with_bias else None
    got = oracle.short_conv_silu(x, w, b)
    ref = _page_conv_silu(x, w, b)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_head_shaped_input_uses_channel_h_times_d_plus_d():
    rng = np.random.default_rng(7)
    B, T, H, D, W = 2, 9, 3, 4, 3
    x = rng.standard_normal((B, T, H, D))
    w = rng.standard_normal((H * D, W))
    got = oracle.short_conv_silu(x, w)
    ref = _page_conv_silu(x.reshape(B, T, H * D), w, None).reshape(B, T, H, D)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_silu_special_values():
    ln3 = math.log(3.0)
    x = np.array([[[0.0, ln3, -ln3, 40.0, -800.0]]])
    y = oracle.short_conv_silu(x)  # no convolution: SiLU alone
    expect = [0.0, ln3 * 0.75, -ln3 * 0.25, 40.0, 0.0]
    np.testing.assert_allclose(y[0, 0], expect, rtol=1e-15, atol=1e-300)


def test_silu_alone_matches_expit():
    from scipy.special import expit
    x = np.random.default_rng(3).standard_normal((2, 11, 5)) * 4
    np.testing.assert_allclose(oracle.short_conv_silu(x), x * expit(x), rtol=1e-15, atol=0)


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_identity_and_shift_taps(W):
    rng = np.random.default_rng(11)
    B, T, C = 2, 12, 6
    x = rng.standard_normal((B, T, C))
    from scipy.special import expit

    def silu(z):
        return z * expit(z)

    for s in range(W):  # tap W-1-s looks s tokens back
        w = np.zeros((C, W))
        w[:, W - 1 - s] = 1.0
        shifted = np.zeros_like(x)
        shifted[:, s:] = x[:, : T - s]
        np.testing.assert_allclose(oracle.short_conv_silu(x, w), silu(shifted), rtol=1e-15, atol=0)


def test_bias_alone_on_zero_input():
    from scipy.special import expit
    C, W = 5, 4
    b = np.linspace(-2, 2, C)
    y = oracle.short_conv_silu(np.zeros((1, 7, C)), np.ones((C, W)), b)
    np.testing.assert_allclose(y, np.broadcast_to(b * expit(b), y.shape), rtol=1e-15, atol=0)


@pytest.mark.parametrize("W", [2, 4])
def test_packed_documents_restart_the_padding(W):
    rng = np.random.default_rng(21)
    lengths = [5, 0, 1, 9, 3]
    T, C = sum(lengths), 7
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = rng.standard_normal((1, T, C))
    w = rng.standard_normal((C, W))
    b = rng.standard_normal(C)
    got = oracle.short_conv_silu(x, w, b, cu_seqlens=cu)
    for n in range(len(lengths)):
        t0, t1 = cu[n], cu[n + 1]
        if t1 == t0:
            continue
        alone = _page_conv_silu(x[:, t0:t1], w, b)
        np.testing.assert_allclose(got[:, t0:t1], alone, rtol=1e-13, atol=1e-13)
    # and a packed row differs from treating it as one sequence (the reset matters)
    whole = _page_conv_silu(x, w, b)
    assert np.abs(got - whole).max() > 1e-3


def test_forward_with_short_conv_composes():
    """kda_fwd_short_conv equals kda_fwd applied to the convolved inputs, and a
    zero-weight convolution with no bias feeds zeros (SiLU(0) = 0): with a zero
    initial state the output and the final state are then exactly zero."""
    from gated_delta_rule_43_amd.synthetic import random_problem
    inp = random_problem(5, 1, 20, 2, 8, 4)
    q, k, v = (inp[n].numpy() for n in ("q", "k", "v"))
    rng = np.random.default_rng(1)
    ws = tuple(rng.standard_normal((8 * 2 if n != "v" else 4 * 2, 3)) for n in "qkv")
    args = [inp[n].numpy() for n in ("gate", "beta", "a_log", "dt_bias")]
    o1, f1 = oracle.kda_fwd_short_conv(q, k, v, *args, conv_weights=ws)
    o2, f2 = oracle.kda_fwd(oracle.short_conv_silu(q, ws[0]), oracle.short_conv_silu(k, ws[1]),
                            oracle.short_conv_silu(v, ws[2]), *args)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)
    zeros = tuple(np.zeros_like(wi) for wi in ws)
    o3, f3 = oracle.kda_fwd_short_conv(q, k, v, *args, conv_weights=zeros)
    assert np.all(o3 == 0) and np.all(f3 == 0)
