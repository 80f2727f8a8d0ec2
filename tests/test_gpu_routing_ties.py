"""Exact router ties on the GPU: the top-k must take the lower expert index, bit-exactly,
with no near-tie relaxation, through both routing paths (sd_moe_route, and the layer step's
fused router + in-kernel routing), and the pooler maps must follow.

Ties are made exact by construction: router rows that are bit-identical copies give
bit-identical logits (both kernels compute every expert's logit with the same arithmetic
in the same order), and equal per-row biases keep them tied after the bias.  Row patterns:
  0: +40 on a tied pair {3, 17} and +30 on a tied triple {6, 11, 29}: the pair first (3
     then 17), then the two lower members of the triple; 29 loses its tie at the k-th place;
  1: +35 on the triple: 6, 11, 29 in index order, then the best unbiased expert;
  2: no bias: the natural top-k, where the duplicated experts tie wherever they rank.
"""

import numpy as np
import pytest
import torch

import oracle
from speculative_verify_decode_amd import binding as B
from tests.gpu_util import DEV, runner, say, workload
from tests.helpers import assert_close, np64, oracle_layer_inputs

pytestmark = pytest.mark.gpu

PAIR, TRIPLE = (3, 17), (6, 11, 29)


def tied_workload(name):
    wk = workload(name)
    lay = dict(wk["layers"][0])
    w = lay["w_router"].clone()
    for e in PAIR[1:]:
        w[e] = w[PAIR[0]]
    for e in TRIPLE[1:]:
        w[e] = w[TRIPLE[0]]
    lay["w_router"] = w
    b, E = wk["workload"].b, wk["dims"]["n_experts"]
    bias = torch.zeros(b, E, dtype=torch.float32)
    for t in range(b):
        if t % 3 == 0:
            bias[t, list(PAIR)] = 40.0
            bias[t, list(TRIPLE)] = 30.0
        elif t % 3 == 1:
            bias[t, list(TRIPLE)] = 35.0
    act = dict(wk["act"], logit_bias=bias)
    return dict(wk, layers=[lay], act=act)


def check_ties(z, ids, k, what):
    """z: the GPU's logits [b, E]; ids: its top-k.  The duplicates are exactly tied, the ids
    are exactly the (-z, index) top-k of z, and the crafted rows take the expected ids."""
    assert np.array_equal(z[:, PAIR[0]], z[:, PAIR[1]]), f"{what}: pair not tied"
    for e in TRIPLE[1:]:
        assert np.array_equal(z[:, TRIPLE[0]], z[:, e]), f"{what}: triple not tied"
    assert np.array_equal(ids, oracle.topk_route(z, k)[0]), what
    for t in range(ids.shape[0]):
        if t % 3 == 0:
            assert ids[t].tolist() == [3, 17, 6, 11], (what, t, ids[t])
        elif t % 3 == 1:
            assert ids[t, :3].tolist() == [6, 11, 29], (what, t, ids[t])
            assert ids[t, 3] != PAIR[1], (what, t, ids[t])   # 17 never precedes its twin 3
        else:
            row = ids[t].tolist()
            if PAIR[1] in row:          # a tied pair ranks together, the lower index first
                assert PAIR[0] in row and row.index(PAIR[0]) < row.index(PAIR[1]), (what, t, row)


def check_pooler(route_t, ids, E, what):
    counts, offsets, slot_of, tos = oracle.pooler(ids, E)
    assert np.array_equal(np64(route_t["expert_counts"]), counts), what
    assert np.array_equal(np64(route_t["expert_offsets"]), offsets), what
    assert np.array_equal(np64(route_t["slot_of"]), slot_of), what
    assert np.array_equal(np64(route_t["token_of_slot"]), tos), what


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["h4096_b8_ctx8k", "h4096_b64_ragged"])
def test_moe_route_exact_ties_take_the_lower_index(name):
    wk = tied_workload(name)
    r = runner(wk)
    d, b = wk["dims"], r.b
    x = wk["act"]["front_embed"]
    B.moe_route(r.dims, b, x.to(DEV), r.layers[0].t["w_router"], r.act["logit_bias"], r.route, r.ws)
    torch.cuda.synchronize()
    z, ids = np64(r.route_t["logits"]), np64(r.route_t["topk_ids"])
    check_ties(z, ids, d["top_k"], f"sd_moe_route {name}")
    check_pooler(r.route_t, ids, d["n_experts"], f"sd_moe_route {name}")
    z_ref = oracle.router_logits(np64(x), np64(wk["layers"][0]["w_router"]),
                                 np64(wk["act"]["logit_bias"]))
    assert_close(z, z_ref, "router logits", tol=1e-3)
    say(f"[gpu-test] ties {name} (sd_moe_route): rows by pattern "
        f"{[int((np.arange(b) % 3 == p).sum()) for p in range(3)]}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["h4096_b8_ctx8k", "h4096_b64_ragged"])
def test_layer_step_exact_ties_take_the_lower_index(name):
    wk = tied_workload(name)
    r = runner(wk)
    d, b = wk["dims"], r.b
    act, lay = wk["act"], wk["layers"][0]
    s = r.act["stream"].clone()
    out = r.layer_step(0, s, r.act["branch_in"])
    torch.cuda.synchronize()
    z, ids = np64(r.route_t["logits"]), np64(r.route_t["topk_ids"])
    check_ties(z, ids, d["top_k"], f"sd_layer_step {name}")
    check_pooler(r.route_t, ids, d["n_experts"], f"sd_layer_step {name}")
    # the rest of the step against the oracle routed the same way
    ref = oracle.layer_step(oracle_layer_inputs(lay, act), d, branch_in=np64(act["branch_in"]),
                            route_override=ids)
    assert_close(z, ref["z"], "router logits", tol=1e-3)
    assert_close(np64(r.route_t["topk_w"]), ref["w"], "route weights", tol=1e-4)
    w1 = assert_close(np64(s), ref["stream"], "stream")
    w2 = assert_close(np64(out), ref["m"], "branch out")
    say(f"[gpu-test] ties {name} (sd_layer_step): worst scaled err stream {w1:.2e} branch {w2:.2e}")
