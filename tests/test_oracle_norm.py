"""Pins of the oracle's gated output norm (the step after the forward).

The reading (the pages name o_norm(output, output_gate) and an RMSNorm with an
fp32 reduction but print neither the norm nor the gate's activation): per row
of V values, y = o / sqrt(mean(o^2) + eps) * weight * act(gate), act = sigmoid
or SiLU.  Pinned against torch's rms_norm (a library routine, fp64), closed
forms and invariances."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


@pytest.mark.parametrize("activation", ["sigmoid", "silu"])
def test_matches_library_rms_norm_times_gate(activation):
    rng = np.random.default_rng(1)
    o = rng.standard_normal((3, 5, 2, 16)) * 3
    g = rng.standard_normal(o.shape) * 2
    w = rng.standard_normal(16)
    eps = 1e-5
    got = oracle.gated_rms_norm(o, g, w, eps, activation)
    t = F.rms_norm(torch.from_numpy(o), (16,), torch.from_numpy(w), eps)
    gt = torch.from_numpy(g)
    act = torch.sigmoid(gt) if activation == "sigmoid" else gt * torch.sigmoid(gt)
    np.testing.assert_allclose(got, (t * act).numpy(), rtol=1e-13, atol=1e-13)


def test_closed_forms():
    V = 8
    # a constant row c normalises to sign(c) (up to eps), the gate 0 gives sigmoid 1/2
    o = np.full((1, V), -3.0)
    y = oracle.gated_rms_norm(o, np.zeros((1, V)), None, eps=0.0)
    np.testing.assert_allclose(y, np.full((1, V), -0.5), rtol=1e-15)
    # SiLU(ln 3) = 3/4 ln 3
    y = oracle.gated_rms_norm(np.ones((1, V)), np.full((1, V), math.log(3.0)), None, eps=0.0,
                              activation="silu")
    np.testing.assert_allclose(y, np.full((1, V), 0.75 * math.log(3.0)), rtol=1e-15)
    # one non-zero entry a in V: rms = |a| / sqrt(V)
    o = np.zeros((1, V))
    o[0, 3] = 2.0
    y = oracle.gated_rms_norm(o, np.full((1, V), 50.0), None, eps=0.0)
    assert abs(y[0, 3] - math.sqrt(V)) < 1e-12 and np.all(y[0, [0, 1, 2, 4, 5, 6, 7]] == 0)


def test_scale_invariance_and_weight():
    rng = np.random.default_rng(2)
    o = rng.standard_normal((4, 32))
    g = rng.standard_normal((4, 32))
    w = rng.standard_normal(32)
    a = oracle.gated_rms_norm(o, g, w, eps=0.0)
    b = oracle.gated_rms_norm(7.5 * o, g, w, eps=0.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    np.testing.assert_allclose(oracle.gated_rms_norm(o, g, 2 * w, eps=0.0), 2 * a, rtol=1e-15)
