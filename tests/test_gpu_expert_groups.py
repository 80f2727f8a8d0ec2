"""Experts holding more than 8 pooled rows on the GPU: a 64-row batch whose every row picks
the same four experts, so each of them is 8 groups of 8 rows (one MFMA column tile each),
through sd_moe_experts and through the layer step (routing in the W13 kernel), against the
oracle.  Plus a mixed batch: one expert chosen by every row, the other choices natural."""

import numpy as np
import pytest
import torch

import oracle
from speculative_verify_decode_amd import binding as B
from tests.gpu_util import DEV, runner, say, workload
from tests.helpers import assert_close, np64, oracle_layer_inputs

pytestmark = pytest.mark.gpu

NAME = "h4096_b64_ragged"


def biased_workload(forced):
    """The 64-row workload with +50 on the logits of `forced` experts in every row."""
    wk = workload(NAME)
    b, E = wk["workload"].b, wk["dims"]["n_experts"]
    bias = torch.zeros(b, E, dtype=torch.float32)
    bias[:, list(forced)] = 50.0
    return dict(wk, act=dict(wk["act"], logit_bias=bias))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("forced", [(0, 1, 2, 3), (5,)])
def test_experts_of_64_rows(forced):
    wk = biased_workload(forced)
    r = runner(wk)
    lay, d, b = wk["layers"][0], wk["dims"], r.b
    k, I, H = d["top_k"], d["inter"], d["hidden"]
    x = wk["act"]["front_embed"]
    B.moe_route(r.dims, b, x.to(DEV), r.layers[0].t["w_router"], r.act["logit_bias"], r.route, r.ws)
    y = torch.empty(b * k, H, dtype=torch.float32, device=DEV)
    h = torch.empty(b * k, I, dtype=torch.bfloat16, device=DEV)
    B.moe_experts(r.dims, b, x.to(DEV), r.layers[0].moe_w, r.route, y, h, r.ws)
    m = torch.empty(b, H, dtype=torch.float32, device=DEV)
    B.moe_unpool(r.dims, b, y, r.route, m)
    torch.cuda.synchronize()
    rt = {kk: np64(v) for kk, v in r.route_t.items()}
    counts, offsets, tos = rt["expert_counts"], rt["expert_offsets"], rt["token_of_slot"]
    assert all(counts[e] == b for e in forced), counts[list(forced)]
    check = sorted(set(forced) | set(np.nonzero(counts)[0][-2:].tolist()))
    say(f"[gpu-test] groups {forced}: counts of the checked experts {counts[check].tolist()}")
    h_ref, y_ref = oracle.moe_experts(np64(x), counts, offsets, tos, np64(lay["w13_codes"]),
                                      np64(lay["w13_scales"]), np64(lay["w13_gscale"]),
                                      np64(lay["w2_codes"]), np64(lay["w2_scales"]),
                                      np64(lay["w2_gscale"]), I, experts=set(check))
    rows = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in check])
    assert_close(np64(h)[rows], h_ref[rows], "SwiGLU output h")
    w = assert_close(np64(y)[rows], y_ref[rows], "expert output y")
    say(f"[gpu-test] groups {forced}: worst scaled err {w:.2e}")
    if len(forced) == k:  # every row's output comes from the checked experts
        m_ref = oracle.unpool(y_ref, rt["topk_w"], rt["slot_of"])
        assert_close(np64(m), m_ref, "unpooled output")


@pytest.mark.timeout(900)
def test_layer_step_with_experts_of_64_rows():
    wk = biased_workload((0, 1, 2, 3))
    r = runner(wk)
    d, act, lay = wk["dims"], wk["act"], wk["layers"][0]
    s = r.act["stream"].clone()
    out = r.layer_step(0, s, r.act["branch_in"])
    torch.cuda.synchronize()
    ids = np64(r.route_t["topk_ids"])
    assert (np.sort(ids, axis=1) == np.array([0, 1, 2, 3])).all()
    ref = oracle.layer_step(oracle_layer_inputs(lay, act), d, branch_in=np64(act["branch_in"]),
                            route_override=ids)
    w1 = assert_close(np64(s), ref["stream"], "stream")
    w2 = assert_close(np64(out), ref["m"], "branch out")
    say(f"[gpu-test] layer step, 4 experts x 64 rows: worst scaled err stream {w1:.2e} branch {w2:.2e}")
