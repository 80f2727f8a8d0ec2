"""The pooled layer step (the unpooler moved into the next layer's input boundary) against
the plain layer step: the same sequence of layer steps from the front, run both ways on
fresh copies of a workload, gives the same stream, the same routing and, after the final
gather (sd_moe_unpool), the same branch."""

import numpy as np
import pytest
import torch

from speculative_verify_decode_amd import binding as B
from tests.gpu_util import DEV, runner, say, workload
from tests.helpers import assert_close, close, np64

pytestmark = pytest.mark.gpu


def layer_sequence(wk):
    n = len(wk["layers"])
    return list(range(n)) if n > 1 else [0, 0, 0]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_b8_ctx128", "h4096_b8_ctx8k", "h4096_b64_ragged",
                                  "h4096_chain4_head"])
def test_pooled_steps_match_plain_steps(name):
    say(f"[gpu-test] pooled layer steps {name}")
    wk = workload(name)
    seq = layer_sequence(wk)
    H = wk["dims"]["hidden"]

    r1 = runner(wk)
    s1 = r1.act["stream"].clone()
    bufs = [torch.empty(r1.b, H, dtype=torch.float32, device=DEV) for _ in seq]
    ids1 = []
    u = None
    for n, i in enumerate(seq):
        if u is None:
            u = r1.layer_step(i, s1, None, front_embed=r1.act["front_embed"], branch_out=bufs[n])
        else:
            u = r1.layer_step(i, s1, u, branch_out=bufs[n])
        torch.cuda.synchronize()
        ids1.append(np64(r1.route_t["topk_ids"]).copy())

    r2 = runner(wk)
    s2 = r2.act["stream"].clone()
    pb = [r2.pooled_buf(), r2.pooled_buf()]
    ids2 = []
    p_in = None
    for n, i in enumerate(seq):
        p_out = pb[n % 2]
        r2.layer_step_pooled(i, s2, p_in, p_out, front_embed=r2.act["front_embed"])
        torch.cuda.synchronize()
        ids2.append(np64(p_out["route_t"]["topk_ids"]).copy())
        p_in = p_out
    m2 = torch.empty(r2.b, H, dtype=torch.float32, device=DEV)
    B.moe_unpool(r2.dims, r2.b, p_in["y"], p_in["route"], m2)
    torch.cuda.synchronize()

    for n in range(len(seq)):
        assert np.array_equal(ids1[n], ids2[n]), n
    d_s = float((s1 - s2).abs().max())
    d_m = float((u - m2).abs().max())
    _, w_s, _ = close(np64(s2), np64(s1), 0.0)
    _, w_m, _ = close(np64(m2), np64(u), 0.0)
    say(f"[gpu-test] {name}: max |diff| stream {d_s:.3e} branch {d_m:.3e}; "
        f"scaled {w_s:.3e} {w_m:.3e}")
    assert_close(np64(s2), np64(s1).astype(np.float64), "stream", tol=1e-5)
    assert_close(np64(m2), np64(u).astype(np.float64), "branch", tol=1e-5)


def test_pooled_step_rejects_missing_output():
    wk = workload("tiny_b8_ctx128")
    r = runner(wk)
    s = r.act["stream"].clone()
    with pytest.raises(B.SdError):
        B._check(B.lib().sd_layer_step_pooled(
            B.ctypes.byref(r.dims), r.b, B.ptr(s), None, B.ptr(r.act["front_embed"]),
            B.ctypes.byref(r.layers[0].weights), B.ctypes.byref(r.layers[0].kv), None, None,
            None, B.ptr(r.ws), r.ws.numel() * r.ws.element_size(), None))


def test_pooled_step_graph_replays_match_eager():
    """The pooled step reading and writing the same pooled buffer, captured once and replayed
    from restored inputs with eager work in between, equals the eager step every time."""
    wk = workload("tiny_b8_ctx128")
    r = runner(wk)
    pool = r.pooled_buf()
    s = r.act["stream"].clone()
    r.layer_step_pooled(0, s, None, pool, front_embed=r.act["front_embed"])  # a real pooled input
    torch.cuda.synchronize()
    s0 = r.act["stream"].clone()
    k0, v0 = r.layers[0].t["k_cache"].clone(), r.layers[0].t["v_cache"].clone()
    y0 = pool["y"].clone()
    rt0 = {k: v.clone() for k, v in pool["route_t"].items()}

    def restore():
        s.copy_(s0)
        r.layers[0].t["k_cache"].copy_(k0)
        r.layers[0].t["v_cache"].copy_(v0)
        pool["y"].copy_(y0)
        for k, v in pool["route_t"].items():
            v.copy_(rt0[k])

    restore()
    r.layer_step_pooled(0, s, pool, pool)
    torch.cuda.synchronize()
    eager_s, eager_y = s.clone(), pool["y"].clone()
    eager_ids = pool["route_t"]["topk_ids"].clone()
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=st):
        r.layer_step_pooled(0, s, pool, pool, stream=st)
    for rep in range(4):
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _ = (torch.randn(1000, device=DEV) * 2).sum().item()     # eager work between replays
        assert torch.equal(s.view(torch.int32), eager_s.view(torch.int32)), rep
        assert torch.equal(pool["y"].view(torch.int32), eager_y.view(torch.int32)), rep
        assert torch.equal(pool["route_t"]["topk_ids"], eager_ids), rep
