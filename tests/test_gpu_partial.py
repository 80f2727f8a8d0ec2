"""GPU parity of partial drafts: steps whose requests verify 1..q_rows tokens each, described
by query_start (row starts per request), against the fp64 oracle on the same seeded inputs."""

import numpy as np
import pytest
import torch

import oracle
from speculative_verify_decode_amd import binding as B
from speculative_verify_decode_amd import synth
from tests.gpu_util import DEV, runner, say, workload
from tests.helpers import assert_close, np64
from tests.test_gpu_layer import run_and_compare

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_partial", "h4096_partial_drafts"])
def test_attn_verify_partial_drafts_match_oracle(name):
    wk = workload(name)
    r = runner(wk)
    lay, d, b = wk["layers"][0], wk["dims"], r.b
    qs = np64(lay["query_start"]).astype(np.int64)
    say(f"[gpu-test] attn_verify {name}: rows per request {np.diff(qs).tolist()}")
    x = wk["act"]["front_embed"]
    out = torch.empty(b, d["hidden"], dtype=torch.float32, device=DEV)
    L = r.layers[0]
    B.attn_verify(r.dims, b, x.to(DEV), L.attn_w, L.kv, out, r.ws)
    torch.cuda.synchronize()
    q, k, v, gate = oracle.qkv_front(np64(x), np64(lay["w_qkv"]), np64(lay["positions"]),
                                     d["n_q_heads"], d["n_kv_heads"], d["head_dim"], d["eps"],
                                     d["rope_theta"], bool(d["qk_norm"]))
    kc, vc = oracle.kv_write(np64(lay["k_cache"]), np64(lay["v_cache"]), k, v,
                             np64(lay["slot_mapping"]))
    o = oracle.paged_attention(q, kc, vc, np64(lay["block_table"]), np64(lay["positions"]),
                               d["q_rows"], query_start=qs)
    a = oracle.gate_oproj(o, gate, np64(lay["w_o"]))
    w = assert_close(np64(out), a, "attention output")
    say(f"[gpu-test] attn {name}: worst scaled err {w:.2e}")
    # only the step's slots changed
    slots = np64(lay["slot_mapping"]).astype(np.int64)
    for key in ("k_cache", "v_cache"):
        new, before = L.t[key], lay[key].to(DEV)
        same = (new == before) | (torch.isnan(new) & torch.isnan(before))
        changed = (~same).reshape(new.shape[0], -1).any(dim=1).nonzero().flatten().cpu().numpy()
        assert set(changed.tolist()) <= set((slots // 16).tolist()), key


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_partial", "h4096_partial_drafts"])
def test_layer_step_partial_drafts_end_to_end(name):
    say(f"[gpu-test] layer step {name}")
    run_and_compare(workload(name))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("q_lens,ctx", [((1,), (1,)), ((1,), (128,)), ((5,), (128,)),
                                        ((1, 8), (1, 45)), ((2, 1, 7), (9, 200, 31))])
def test_layer_step_partial_drafts_tiny_edges(q_lens, ctx):
    # one row at position 0 (a request holding only its one verify token), one row (plain
    # decode), a single partial request, the one-token request next to a full one, three
    # requests of mixed counts
    w = synth.with_overrides(synth.WORKLOADS["tiny_partial"], n_req=len(q_lens), ctx=ctx,
                             q_lens=q_lens, name=f"tiny_q{'_'.join(map(str, q_lens))}")
    run_and_compare(synth.make_workload(w))


@pytest.mark.timeout(900)
def test_layer_step_single_partial_request_config_shape():
    # the 8k single-request shape verifying 5 of its 8 draft tokens
    w = synth.with_overrides(synth.WORKLOADS["h4096_b8_ctx8k"], q_lens=(5,),
                             name="h4096_q5_ctx8k")
    run_and_compare(synth.make_workload(w))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("window", [1, 20])
def test_layer_step_partial_drafts_with_window_tiny(window):
    w = synth.with_overrides(synth.WORKLOADS["tiny_partial"], window=window,
                             name=f"tiny_partial_win{window}")
    run_and_compare(synth.make_workload(w))


@pytest.mark.timeout(900)
def test_partial_drafts_uniform_query_start_matches_default():
    # query_start describing q_rows rows per request gives the default split bit for bit
    wk = workload("tiny_b8_ctx128")
    r = runner(wk)
    d, b = wk["dims"], r.b
    x = wk["act"]["front_embed"].to(DEV)
    L = r.layers[0]
    outs = []
    for qs in (None, torch.arange(0, b + 1, d["q_rows"], dtype=torch.int32, device=DEV)):
        kv = B.SdKv.from_buffer_copy(L.kv)
        kv.query_start = None if qs is None else qs.data_ptr()
        out = torch.empty(b, d["hidden"], dtype=torch.float32, device=DEV)
        B.attn_verify(r.dims, b, x, L.attn_w, kv, out, r.ws)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
