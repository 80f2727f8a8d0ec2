"""sd_layer_step_noalloc: the layer step on the library's static scratch, for callers that
cannot allocate.  Its results must equal sd_layer_step's (same kernels, workspace given),
here bit for bit, on two calls in a row where the second is smaller than the first (so the
second runs on scratch the first left behind)."""

import pytest
import torch

from speculative_verify_decode_amd import binding as B
from speculative_verify_decode_amd.runner import alloc_route
from tests.gpu_util import DEV, runner, say, workload

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _step(r, noalloc):
    d = r.d
    s = r.act["stream"].clone()
    out = torch.full_like(s, float("nan"))
    aux = torch.full_like(s, float("nan"))
    rt, route = alloc_route(r.b, d["top_k"], d["n_experts"], DEV)
    L = r.layers[0]
    if noalloc:
        B.layer_step_noalloc(r.dims, r.b, s, r.act["branch_in"], None, L.weights, L.kv,
                             r.act["logit_bias"], out, route, aux=aux)
    else:
        B.layer_step(r.dims, r.b, s, r.act["branch_in"], None, L.weights, L.kv,
                     r.act["logit_bias"], out, route, r.ws, aux=aux)
    return dict(stream=s, out=out, aux=aux, **rt)


@pytest.mark.timeout(600)
def test_noalloc_step_equals_the_workspace_step_on_two_calls_in_a_row():
    assert B.lib().sd_noalloc_scratch_bytes() == 32 << 20
    big, small = runner(workload("h4096_b64_ragged")), runner(workload("h4096_b8_ctx8k"))
    assert big.ws_bytes > small.ws_bytes
    refs = [_step(r, noalloc=False) for r in (big, small)]
    torch.cuda.synchronize()
    got = [_step(r, noalloc=True) for r in (big, small)]     # back to back, big then small
    torch.cuda.synchronize()
    for name, ref, g in zip(("b64 ragged", "b8 8k"), refs, got):
        for key in ref:
            assert torch.equal(_bits(g[key]), _bits(ref[key])), (name, key)
        say(f"[gpu-test] noalloc {name}: bit-identical to sd_layer_step")


def test_noalloc_rejects_a_step_larger_than_its_scratch():
    r = runner(workload("tiny_b8_ctx128"))
    kv = B.SdKv.from_buffer_copy(r.layers[0].kv)
    kv.max_seq_len = 1 << 28                 # attention partials beyond 32 MiB
    kv.max_blocks = 1 << 24
    assert B.workspace_bytes(r.dims, r.b, 1, kv.max_seq_len) > B.lib().sd_noalloc_scratch_bytes()
    with pytest.raises(B.SdError) as e:
        B._check(B.lib().sd_layer_step_noalloc(
            B.ctypes.byref(r.dims), r.b, B.ptr(r.act["stream"]), B.ptr(r.act["branch_in"]), None,
            B.ctypes.byref(r.layers[0].weights), B.ctypes.byref(kv), None, B.ptr(r.branch_out),
            None, None, None))
    assert e.value.code == -4 and "scratch" in str(e.value)
