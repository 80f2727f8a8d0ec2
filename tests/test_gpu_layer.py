"""End-to-end GPU parity of the layer step and the 4-layer chain with the draft head.

Routing is checked twice.  Stage A, on every row: the layer step's own router logits
(route.logits) are compared with the oracle's, and the expert ids must be exactly the
oracle's top-k of those same logits (ties to the lower index), with the pooler maps
exactly the oracle's pooler of those ids.  Stage B: the oracle runs its own fp64 chain;
where its routing gap is below 2e-3 * (1 + max|z|) it is teacher-forced to the GPU's ids
(those rows are reported, and at least half the rows must be left to check).  Plus the
aux taps, determinism, HIP-graph replay, block-table permutation and edge shapes."""

import numpy as np
import pytest
import torch

import oracle
from speculative_verify_decode_amd import binding as B
from speculative_verify_decode_amd import synth
from speculative_verify_decode_amd.runner import StepRunner, alloc_route
from oracle.head import output_multiplier
from tests.gpu_util import (DEV, check_route_stage_a, head_flags, require_lib, runner, say,
                            teacher_forcer, workload)
from tests.helpers import assert_close, np64, oracle_layer_inputs

pytestmark = pytest.mark.gpu

STAGE_B_GAP = 2e-3


def check_fused_routing(route_t, z_ref, k, n_experts, what):
    """Stage A of the layer step's routing on its own logits (every row, no near-tie
    relaxation): ids = oracle top-k of the GPU logits, pooler maps = oracle pooler of the
    ids, weights = softmax over the selected GPU logits; the logits themselves close to the
    oracle's."""
    z = np64(route_t["logits"])
    assert_close(z, z_ref, f"{what}: router logits", tol=1e-3)
    gid = np64(route_t["topk_ids"])
    ids_a, w_a = oracle.topk_route(z, k)
    assert np.array_equal(gid, ids_a), what
    assert_close(np64(route_t["topk_w"]), w_a, f"{what}: route weights", tol=1e-5)
    counts, offsets, slot_of, tos = oracle.pooler(gid, n_experts)
    assert np.array_equal(np64(route_t["expert_counts"]), counts), what
    assert np.array_equal(np64(route_t["expert_offsets"]), offsets), what
    assert np.array_equal(np64(route_t["slot_of"]), slot_of), what
    assert np.array_equal(np64(route_t["token_of_slot"]), tos), what
    act = np64(route_t["active_experts"])
    assert act[-1] == (counts > 0).sum() and np.array_equal(act[:act[-1]], np.nonzero(counts)[0])


def run_and_compare(wk, front=False):
    r = runner(wk)
    d, b = wk["dims"], r.b
    act, lay = wk["act"], wk["layers"][0]
    s = r.act["stream"].clone()
    aux = torch.full_like(s, float("nan"))
    if front:
        out = r.layer_step(0, s, None, front_embed=r.act["front_embed"], aux=aux)
    else:
        out = r.layer_step(0, s, r.act["branch_in"], aux=aux)
    torch.cuda.synchronize()
    gid = np64(r.route_t["topk_ids"])
    forced = []
    inp = oracle_layer_inputs(lay, act)
    ref = oracle.layer_step(inp, d, branch_in=None if front else np64(act["branch_in"]),
                            front_embed=np64(act["front_embed"]) if front else None,
                            route_override=teacher_forcer(gid, STAGE_B_GAP, forced))
    say(f"[gpu-test] {wk['workload'].name}: teacher-forced rows {forced[0].tolist()}")
    check_fused_routing(r.route_t, ref["z"], d["top_k"], d["n_experts"], wk["workload"].name)
    free = np.setdiff1d(np.arange(b), forced[0])
    assert len(free) >= b // 2, f"only {len(free)} of {b} rows left unforced"
    assert np.array_equal(gid[free], ref["ids"][free])
    assert np.array_equal(np64(r.route_t["slot_of"]), ref["slot_of"])
    assert np.array_equal(np64(r.route_t["token_of_slot"]), ref["token_of_slot"])
    if front:
        assert np.array_equal(np64(aux), ref["aux"])   # the tap is the embedding itself
    else:
        assert_close(np64(aux), ref["aux"], "aux tap")
    w1 = assert_close(np64(s), ref["stream"], "stream")
    w2 = assert_close(np64(out), ref["m"], "branch out")
    say(f"[gpu-test] {wk['workload'].name}: worst scaled err stream {w1:.2e} branch {w2:.2e}")
    slots = np64(lay["slot_mapping"])
    kc = np64(r.layers[0].t["k_cache"][torch.from_numpy(slots // 16).to(DEV)])
    assert_close(kc[np.arange(b), :, slots % 16, :], ref["k_cache"][slots // 16, :, slots % 16, :],
                 "written K")
    return r, ref


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_b8_ctx128", "h4096_b8_ctx8k", "h4096_b64_ragged",
                                  "h4096_b8_ctx131k", "h4096_b8_ctx131k_win8k"])
def test_layer_step_end_to_end(name):
    say(f"[gpu-test] layer step {name}")
    run_and_compare(workload(name))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n_experts", [12, 20])
def test_layer_step_expert_counts_off_the_grid(n_experts):
    # expert counts that leave part of the router's 8-expert groups, and of the routing's
    # 32-key rows, as padding
    w = synth.with_overrides(synth.WORKLOADS["h4096_b8_ctx8k"], n_experts=n_experts,
                             ctx=(1000,), pool_blocks=128, name=f"h4096_e{n_experts}")
    say(f"[gpu-test] layer step {w.name}")
    run_and_compare(synth.make_workload(w))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("base,top_k", [("tiny_b8_ctx128", 1), ("tiny_b8_ctx128", 8),
                                        ("h4096_b8_ctx8k", 1)])
def test_layer_step_top_k_extremes(base, top_k):
    # one choice per row (weight 1), and every expert of the tiny shape chosen by every row
    over = dict(top_k=top_k, name=f"{base}_k{top_k}")
    if base.startswith("h4096"):
        over.update(ctx=(1000,), pool_blocks=128)
    w = synth.with_overrides(synth.WORKLOADS[base], **over)
    say(f"[gpu-test] layer step {w.name}")
    run_and_compare(synth.make_workload(w))


def test_layer_step_front_mode_tiny():
    run_and_compare(workload("tiny_b8_ctx128"), front=True)


@pytest.mark.parametrize("ctx", [(45, 8), (17, 200), (16, 31)])
def test_layer_step_ragged_and_minimal_contexts(ctx):
    # partial last blocks, a request holding only its 8 verify tokens, two requests
    w = synth.with_overrides(synth.WORKLOADS["tiny_b8_ctx128"], n_req=2, ctx=ctx, name=f"tiny_{ctx}")
    run_and_compare(synth.make_workload(w))


def test_layer_step_max_rows_tiny():
    w = synth.with_overrides(synth.WORKLOADS["tiny_b8_ctx128"], n_req=8,
                             ctx=(128, 9, 64, 300, 33, 16, 250, 100), name="tiny_b64")
    run_and_compare(synth.make_workload(w))


@pytest.mark.parametrize("window", [1, 20, 64])
def test_layer_step_sliding_window_ragged_tiny(window):
    # two requests of different lengths: the first visible block differs per request
    w = synth.with_overrides(synth.WORKLOADS["tiny_b8_ctx128"], n_req=2, ctx=(45, 200),
                             window=window, name=f"tiny_win{window}")
    run_and_compare(synth.make_workload(w))


def test_layer_step_qk_norm_off_tiny():
    w = synth.with_overrides(synth.WORKLOADS["tiny_b8_ctx128"], qk_norm=0, name="tiny_noqk")
    run_and_compare(synth.make_workload(w))


@pytest.mark.parametrize("name", ["tiny_b8_ctx128", "h4096_b8_ctx8k"])
def test_layer_step_is_deterministic(name):
    wk = workload(name)
    outs = []
    for _ in range(2):
        r = runner(wk)
        s = r.act["stream"].clone()
        o = r.layer_step(0, s, r.act["branch_in"]).clone()
        torch.cuda.synchronize()
        outs.append((s.cpu(), o.cpu(), r.layers[0].t["k_cache"].cpu(), r.route_t["slot_of"].cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                           b.view(torch.uint8) if b.dtype != torch.int32 else b)


def test_block_table_permutation_gives_identical_output():
    wk = workload("tiny_b8_ctx128")
    lay = wk["layers"][0]
    r1 = runner(wk)
    s1 = r1.act["stream"].clone()
    o1 = r1.layer_step(0, s1, r1.act["branch_in"]).clone()
    nb = lay["num_blocks"]
    perm = torch.from_numpy(np.random.default_rng(11).permutation(nb))
    inv = torch.argsort(perm)
    lay2 = dict(lay, k_cache=lay["k_cache"][perm].contiguous(), v_cache=lay["v_cache"][perm].contiguous(),
                block_table=inv[lay["block_table"].long()].int(),
                slot_mapping=inv[lay["slot_mapping"] // 16] * 16 + lay["slot_mapping"] % 16)
    wk2 = dict(wk, layers=[lay2])
    r2 = runner(wk2)
    s2 = r2.act["stream"].clone()
    o2 = r2.layer_step(0, s2, r2.act["branch_in"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))


def test_hip_graph_replays_match_eager():
    wk = workload("tiny_b8_ctx128")
    r = runner(wk)
    s0 = r.act["stream"].clone()
    k0, v0 = r.layers[0].t["k_cache"].clone(), r.layers[0].t["v_cache"].clone()
    s = s0.clone()
    eager = r.layer_step(0, s, r.act["branch_in"]).clone()
    eager_s = s.clone()
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s.copy_(s0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=st):
        r.layer_step(0, s, r.act["branch_in"], stream=st)
    for rep in range(4):
        s.copy_(s0)
        r.layers[0].t["k_cache"].copy_(k0)
        r.layers[0].t["v_cache"].copy_(v0)
        r.branch_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _ = (torch.randn(1000, device=DEV) * 2).sum().item()     # eager work between replays
        assert torch.equal(s, eager_s), rep
        assert torch.equal(r.branch_out.view(torch.int32), eager.view(torch.int32)), rep


@pytest.mark.timeout(1200)
def test_chain_of_four_layers_with_draft_head():
    wk = workload("h4096_chain4_head")
    require_lib()
    r = StepRunner(wk, DEV)
    d, b, H = wk["dims"], r.b, wk["dims"]["hidden"]
    routes = [alloc_route(b, d["top_k"], d["n_experts"], DEV) for _ in r.layers]
    bufs = [torch.empty(b, H, dtype=torch.float32, device=DEV) for _ in r.layers]
    auxs = [torch.full((b, H), float("nan"), dtype=torch.float32, device=DEV)
            for _ in range(len(r.layers) + 1)]
    mult = output_multiplier(H, wk["head"]["base_width"], wk["head"]["mult_mode"])
    s = r.act["stream"].clone()
    u = r.act["branch_in"]
    for i in range(len(r.layers)):
        r.route_t, r.route = routes[i]
        u = r.layer_step(i, s, u, branch_out=bufs[i], aux=auxs[i])
    hd = r.head
    B.boundary_dualnorm(r.dims, b, s, u, None, r.layers[-1].t["g_post_ffn"], hd["g_final"], r.head_h,
                        aux=auxs[-1])
    V = hd["w_lm"].shape[0]
    B.draft_head(H, V, b, r.head_h, hd["w_lm"], mult, hd["soft_cap"], hd["d2t"], r.tau,
                 r.draft_ids, r.target_ids, r.head_ws)
    torch.cuda.synchronize()
    say("[gpu-test] chain: GPU done, running the oracle chain")
    forced = []
    gids = [np64(rt[0]["topk_ids"]) for rt in routes]
    act = wk["act"]
    layers = [oracle_layer_inputs(l, act) for l in wk["layers"]]
    ref = oracle.chain_step(layers, d, np64(act["stream"]), np64(act["branch_in"]),
                            np64(wk["head"]["g_final"]), np64(wk["head"]["w_lm"]),
                            mult, wk["head"]["soft_cap"], np64(wk["head"]["d2t"]),
                            route_overrides=[teacher_forcer(g, STAGE_B_GAP, forced) for g in gids],
                            on_layer=lambda i: say(f"[gpu-test] chain oracle: layer {i} done"))
    for i in range(4):
        say(f"[gpu-test] chain layer {i}: teacher-forced rows {forced[i].tolist()}")
        check_fused_routing(routes[i][0], ref["layers"][i]["z"], d["top_k"], d["n_experts"],
                            f"chain layer {i}")
        free = np.setdiff1d(np.arange(b), forced[i])
        assert len(free) >= b // 2, f"layer {i}: only {len(free)} of {b} rows left unforced"
        assert np.array_equal(gids[i][free], ref["layers"][i]["ids"][free]), i
        assert_close(np64(bufs[i]), ref["layers"][i]["m"], f"layer {i} branch")
    for i, a in enumerate(auxs):
        assert_close(np64(a), ref["aux"][i], f"aux tap {i}")
    assert torch.equal(auxs[-1], s)                   # the final tap is the final stream
    assert_close(np64(s), ref["stream"], "final stream")
    assert_close(np64(r.head_h), ref["h"], "final hidden")
    # stage A on the head: the oracle head on the GPU's own bf16 hidden, ids bit-exact
    ra = oracle.draft_head(np64(r.head_h), np64(wk["head"]["w_lm"]), mult,
                           wk["head"]["soft_cap"], np64(wk["head"]["d2t"]))
    exact = np64(r.head_h) @ np64(wk["head"]["w_lm"]).T
    flagged = head_flags(exact)
    gid = np64(r.draft_ids)
    for t in range(b):
        if not flagged[t]:
            assert gid[t] == ra["ids"][t], (t, gid[t], ra["ids"][t])
    assert np.array_equal(np64(r.target_ids), np64(wk["head"]["d2t"])[gid])
    assert_close(np64(r.tau), ra["tau"], "transformed logits", tol=1e-2)
    # stage B on the head: rows whose exact top-2 gap is clear must agree end to end
    lg = ref["head"]["logits"]
    top2 = -np.sort(-lg, axis=1)[:, :2]
    clear = (top2[:, 0] - top2[:, 1]) > STAGE_B_GAP * (1 + np.abs(lg).max(axis=1))
    say(f"[gpu-test] head stage B: {clear.sum()} of {b} rows with a clear top-2 gap")
    assert np.array_equal(gid[clear], ref["head"]["ids"][clear])
