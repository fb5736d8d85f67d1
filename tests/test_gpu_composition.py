"""Slice-summary composition with live transitions, at the fp32 tolerance.

The pages' sequence sharding composes per-slice affine summaries of the state
(hyper_parallel coverage page, context_parallel/kimi_delta_attention.py,
`_eager_kda_state_p2p`: torch_kda_state_summary, then
torch_apply_kda_state_summary).  Composing the summaries of contiguous slices
must give the whole row's final state; the carried-state workload states this
at the fp32 tolerance (max-abs 1e-4) even for bf16 inputs.

At the carried-state workload's own gates every 16,384-token slice forgets its
entering state (the transition underflows to zero), so a check there cannot
see a wrong transition.  Here the decay is slow (a_log = -7, beta logits
shifted down by 1) so that every slice's transition keeps entries above 0.05
and the state entering each slice still shapes its end: a transition computed
with too little precision moves the composed state."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_43_amd import kda, synthetic
from kda_testlib import assert_close, errors, gpu_fwd, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _live_problem(T, H, seed=4242):
    inp = synthetic.random_problem(seed, 1, T, H, 128, 128, dtype=torch.bfloat16, device=DEV,
                                   init_std=0.02)
    inp["a_log"] = torch.full_like(inp["a_log"], -7.0)
    inp["beta"] = (inp["beta"].float() - 1.0).to(torch.bfloat16)
    inp.update(scale=None, lower_bound=None, chunk_size=64)
    return inp


def test_live_transition_composition_fp32_tolerance():
    T, H, NS = 8192, 4, 8
    S = T // NS
    print("[gpu-test] live-transition composition T=%d H=%d slices=%d" % (T, H, NS), flush=True)
    inp = _live_problem(T, H)
    _, f_whole = gpu_fwd(inp)
    a_log, dt_bias = to_np(inp["a_log"]), to_np(inp["dt_bias"])
    St = inp["initial_state"]
    worst = [0.0, 0.0]
    for s in range(NS):
        sl = {x: inp[x][:, s * S:(s + 1) * S].contiguous() for x in ("q", "k", "v", "gate", "beta")}
        E, P = kda.kda_state_summary(sl["q"], sl["k"], sl["v"], sl["gate"], sl["beta"],
                                     inp["a_log"], inp["dt_bias"])
        torch.cuda.synchronize()
        Er, Pr = oracle.state_summary(*(to_np(sl[x]) for x in ("q", "k", "v", "gate", "beta")),
                                      a_log, dt_bias)
        # every head's transition is live in this slice
        assert np.abs(Pr).max(axis=(-2, -1)).min() > 0.05
        worst[0] = max(worst[0], assert_close(to_np(E), Er, torch.bfloat16, "state_ext, slice %d" % s)[0])
        worst[1] = max(worst[1], assert_close(to_np(P), Pr, torch.bfloat16, "transition, slice %d" % s)[0])
        St = kda.kda_apply_state_summary(E, P, St)
    torch.cuda.synchronize()
    maxabs, relf = errors(to_np(St), to_np(f_whole))
    print("live composition vs whole-row forward: max-abs %.3g rel-F %.3g; "
          "summaries vs oracle max-abs E %.3g P %.3g" % (maxabs, relf, worst[0], worst[1]), flush=True)
    _, f_ref = oracle.kda_fwd(*(to_np(inp[x]) for x in ("q", "k", "v", "gate", "beta")), a_log,
                              dt_bias, initial_state=to_np(inp["initial_state"]), want_output=False)
    assert_close(to_np(f_whole), f_ref, torch.bfloat16, "whole-row final state vs oracle")
    assert maxabs <= 1e-4, "composed vs whole-row final state: max-abs %.3g > 1e-4" % maxabs


def test_live_transition_carried_state_split():
    """Carrying final_state -> initial_state slice by slice equals the whole run
    at the fp32 tolerance (the pages' p2p hand-over of the state)."""
    T, H, NS = 4096, 2, 4
    S = T // NS
    inp = _live_problem(T, H, seed=4343)
    _, f_whole = gpu_fwd(inp)
    St = inp["initial_state"]
    for s in range(NS):
        sl = dict(inp)
        for x in ("q", "k", "v", "gate", "beta"):
            sl[x] = inp[x][:, s * S:(s + 1) * S].contiguous()
        sl["initial_state"] = St
        _, St = gpu_fwd(sl)
    maxabs, _ = errors(to_np(St), to_np(f_whole))
    print("live carried split vs whole-row forward: max-abs %.3g" % maxabs, flush=True)
    assert maxabs <= 1e-4, maxabs
