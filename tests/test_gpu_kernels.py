"""Per-call GPU parity (stage A: the oracle takes the same inputs the GPU call took).

Floats: |gpu - ref| <= 2e-2 * (1 + |ref|) elementwise.  Discrete outputs: bit-exact
(expert ids except near ties, which must still be a valid top-k; pooler maps always).
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import dequant_nvfp4
from speculative_verify_decode_amd import binding as B
from speculative_verify_decode_amd import synth
from speculative_verify_decode_amd.runner import alloc_route
from oracle.head import output_multiplier
from tests.gpu_util import (DEV, check_route_stage_a, head_flags, require_lib, runner, say,
                            workload)
from tests.helpers import assert_close, np64

pytestmark = pytest.mark.gpu

ALL = ["tiny_b8_ctx128", "h4096_b8_ctx8k", "h4096_b64_ragged", "h4096_b8_ctx131k"]


# ------------------------------------------------------------------------ cross-lane helpers
def test_cross_lane_exchanges_are_exact():
    """The kernels' lane exchanges (DPP and permlane swaps) against their definition on the
    lane index, bit for bit: partner values, the butterflies' float32 sums and maxima in
    their stated partner order, and the integer prefix sum."""
    require_lib()
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(64) * 10.0).astype(np.float32)
    x[5] = x[9]  # a repeated value
    xi = rng.integers(-50, 50, 64).astype(np.int32)
    xd = torch.from_numpy(x).to(DEV)
    xid = torch.from_numpy(xi).to(DEV)
    out = torch.empty(10, 64, dtype=torch.float32, device=DEV)
    out_i = torch.empty(2, 64, dtype=torch.int32, device=DEV)
    B.debug_lanes(xd, xid, out, out_i)
    torch.cuda.synchronize()
    got, got_i = out.cpu().numpy(), out_i.cpu().numpy()
    lane = np.arange(64)
    for row, o in enumerate([1, 2, 4, 8, 16, 32]):
        assert np.array_equal(got[row], x[lane ^ o]), f"lane ^ {o}"

    def butterfly(v, offsets, op):
        v = v.copy()
        for o in offsets:
            v = op(v, v[lane ^ o]).astype(np.float32)
        return v

    add = lambda a, b: np.float32(a) + np.float32(b)
    assert np.array_equal(got[6], butterfly(x, [32, 16, 8, 4, 2, 1], add)), "wave sum"
    assert np.array_equal(got[7], np.full(64, x.max(), dtype=np.float32)), "wave max"
    assert np.array_equal(got[8], butterfly(x, [1, 2, 4], add)), "sum over groups of 8"
    assert np.array_equal(got[9], butterfly(x, [1, 2, 4, 8, 16], add)), "sum over groups of 32"
    assert np.array_equal(got_i[0], np.cumsum(xi).astype(np.int32)), "inclusive prefix sum"
    assert np.array_equal(got_i[1], xi[lane ^ 4]), "int lane ^ 4"


# ------------------------------------------------------------------------ dequant
def test_debug_dequant_is_bit_exact():
    require_lib()
    rng = np.random.default_rng(3)
    n, k = 48, 4096
    codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    valid = [c for c in range(256) if c not in (0x7F, 0xFF)]
    scales = rng.choice(valid, (n, k // 16)).astype(np.uint8)      # every finite E4M3 code
    out = torch.empty(n, k, dtype=torch.float32, device=DEV)
    for gscale in (1.0, 0.5, 4.0):
        B.debug_dequant(n, k, torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                        gscale, out)
        torch.cuda.synchronize()
        ref = dequant_nvfp4(codes, scales, gscale)
        assert np.array_equal(out.cpu().numpy().astype(np.float64), ref), gscale


# ------------------------------------------------------------------------ weight packing
# Expected layouts are the header's tile definitions, written as numpy reshapes.
def packed_dense_ref(w):
    n, k = w.shape
    npad = -(-n // 16) * 16
    full = np.zeros((npad, k), dtype=w.dtype)
    full[:n] = w
    # tile (nt, kt), lane l = 16 g + i, element j  <-  W[16 nt + i, 32 kt + 8 g + j]
    return full.reshape(npad // 16, 16, k // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)


def packed_fp4_ref(codes, scales):
    e, n, kh = codes.shape
    nt, kt = n // 16, (2 * kh) // 128
    # lane l = 16 g + i of tile (e, nt, kt): code bytes 64 kt + 16 g .., scale bytes 8 kt + 2 g ..
    c = codes.reshape(e, nt, 16, kt, 4, 16).transpose(0, 1, 3, 4, 2, 5).reshape(-1)
    s = scales.reshape(e, nt, 16, kt, 4, 2).transpose(0, 1, 3, 4, 2, 5).reshape(-1)
    return c, s


@pytest.mark.parametrize("n,k", [(40, 96), (48, 4096), (10240, 4096)])
def test_pack_dense_layout_is_exact(n, k):
    require_lib()
    rng = np.random.default_rng(n + k)
    w = rng.integers(0, 1 << 16, (n, k), dtype=np.uint16)
    dev = torch.from_numpy(w.view(np.int16)).to(DEV).view(torch.bfloat16)
    out = B.pack_dense(dev)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    assert np.array_equal(got, packed_dense_ref(w))


@pytest.mark.parametrize("e,n,k", [(3, 32, 128), (2, 3072, 4096), (4, 4096, 1536)])
def test_pack_fp4_layout_is_exact(e, n, k):
    require_lib()
    rng = np.random.default_rng(e * n + k)
    codes = rng.integers(0, 256, (e, n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (e, n, k // 16), dtype=np.uint8)
    co, so = B.pack_fp4(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV))
    torch.cuda.synchronize()
    c_ref, s_ref = packed_fp4_ref(codes, scales)
    assert np.array_equal(co.cpu().numpy().reshape(-1), c_ref)
    assert np.array_equal(so.cpu().numpy().reshape(-1), s_ref)


# ------------------------------------------------------------------------ dual norm
@pytest.mark.parametrize("name", ["tiny_b8_ctx128", "h4096_b8_ctx8k"])
def test_boundary_dualnorm_modes(name):
    require_lib()
    wk = workload(name)
    act, lay, d = wk["act"], wk["layers"][0], wk["dims"]
    dims, b, H = B.make_dims(d), wk["workload"].b, d["hidden"]
    s = act["stream"].to(DEV).clone()
    out = torch.empty(b, H, dtype=torch.bfloat16, device=DEV)
    out16 = torch.empty(2, b, H, dtype=torch.float16, device=DEV)
    gp, gq = lay["g_post_prev"].to(DEV), lay["g_pre_attn"].to(DEV)
    aux = torch.full((b, H), float("nan"), dtype=torch.float32, device=DEV)
    B.boundary_dualnorm(dims, b, s, act["branch_in"].float().to(DEV), None, gp, gq, out,
                        out16=out16, aux=aux)
    torch.cuda.synchronize()
    s_ref, x_ref = oracle.dual_norm(np64(act["stream"]), np64(act["branch_in"]), np64(lay["g_post_prev"]),
                                    np64(lay["g_pre_attn"]), d["eps"])
    assert_close(np64(s), s_ref, "stream")
    assert torch.equal(aux, s)                       # the tap is the stream it hands on
    assert_close(np64(aux), s_ref, "aux tap")
    assert_close(np64(out), x_ref, "pre-norm output")
    # the expert-input form: hi + lo = y * 2^-8 to fp32 accuracy
    terms = np64(out16)
    assert_close((terms[0] + terms[1]) * 256.0, x_ref, "expert-input terms", tol=1e-4)
    # front mode: the stream becomes the embedding
    B.boundary_dualnorm(dims, b, s, None, act["front_embed"].to(DEV), None, gq, out, aux=aux)
    torch.cuda.synchronize()
    s_ref, x_ref = oracle.front_norm(np64(act["front_embed"]), np64(lay["g_pre_attn"]), d["eps"])
    assert np.array_equal(np64(s), s_ref)
    assert np.array_equal(np64(aux), s_ref)
    assert_close(np64(out), x_ref, "front pre-norm output")


# ------------------------------------------------------------------------ attention
def check_attn_verify(wk, name):
    r = runner(wk)
    lay, d, b = wk["layers"][0], wk["dims"], r.b
    say(f"[gpu-test] attn_verify {name}")
    x = wk["act"]["front_embed"]
    out = torch.empty(b, d["hidden"], dtype=torch.float32, device=DEV)
    L = r.layers[0]
    B.attn_verify(r.dims, b, x.to(DEV), L.attn_w, L.kv, out, r.ws)
    torch.cuda.synchronize()
    q, k, v, gate = oracle.qkv_front(np64(x), np64(lay["w_qkv"]), np64(lay["positions"]),
                                     d["n_q_heads"], d["n_kv_heads"], d["head_dim"], d["eps"],
                                     d["rope_theta"], bool(d["qk_norm"]))
    kc, vc = oracle.kv_write(np64(lay["k_cache"]), np64(lay["v_cache"]), k, v, np64(lay["slot_mapping"]))
    o = oracle.paged_attention(q, kc, vc, np64(lay["block_table"]), np64(lay["positions"]), d["q_rows"])
    a = oracle.gate_oproj(o, gate, np64(lay["w_o"]))
    w = assert_close(np64(out), a, "attention output")
    say(f"[gpu-test] attn {name}: worst scaled err {w:.2e}")
    # the cache changed exactly at the step's slots, to the bf16 K/V of the oracle
    slots = np64(lay["slot_mapping"])
    for key, ref_cache, new in (("k_cache", kc, L.t["k_cache"]), ("v_cache", vc, L.t["v_cache"])):
        before = lay[key].to(DEV)
        same = (new == before) | (torch.isnan(new) & torch.isnan(before))
        changed = (~same).reshape(new.shape[0], -1).any(dim=1).nonzero().flatten().cpu().numpy()
        assert set(changed.tolist()) <= set((slots // 16).tolist()), key
        blocks = np.unique(slots // 16)
        got = np64(new[torch.from_numpy(blocks).to(DEV)])
        want = ref_cache[blocks]
        mask = ~np.isnan(want)
        assert np.array_equal(np.isnan(got), ~mask), key
        assert_close(got[mask], want[mask], key)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ALL)
def test_attn_verify_matches_oracle(name):
    check_attn_verify(workload(name), name)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ctx", [
    (30000, 8, 16, 17, 4096, 9, 1000, 12000),  # one long request among minimal ones
    (8, 8, 8, 8, 8, 8, 8, 24576),              # nearly all blocks in the last request
    (2048,) * 8,                               # equal lengths
])
def test_attn_verify_skewed_request_lengths(ctx):
    """Several requests share each KV head's chunk slots in proportion to their lengths, so
    the chunk size differs from the host's (sized for every request at max_seq_len) and
    requests own different slot counts, down to a single chunk of one block."""
    w = synth.with_overrides(synth.WORKLOADS["h4096_b64_ragged"], ctx=ctx,
                             name=f"h4096_skew_{ctx[0]}_{ctx[-1]}")
    check_attn_verify(synth.make_workload(w), w.name)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,windows", [
    ("tiny_b8_ctx128", (1, 9, 40, 300)),
    ("h4096_b8_ctx8k", (1, 100, 4096, 8184, 9000)),
    ("h4096_b64_ragged", (2048,)),
    ("h4096_b8_ctx131k", (8192,)),
])
def test_attn_sliding_window_matches_oracle(name, windows):
    """Sliding windows from one visible token (the row's own) past the whole context."""
    wk = workload(name)
    r = runner(wk)
    lay, d, b = wk["layers"][0], wk["dims"], r.b
    x = wk["act"]["front_embed"]
    L = r.layers[0]
    q, k, v, gate = oracle.qkv_front(np64(x), np64(lay["w_qkv"]), np64(lay["positions"]),
                                     d["n_q_heads"], d["n_kv_heads"], d["head_dim"], d["eps"],
                                     d["rope_theta"], bool(d["qk_norm"]))
    kc, vc = oracle.kv_write(np64(lay["k_cache"]), np64(lay["v_cache"]), k, v, np64(lay["slot_mapping"]))
    for window in windows:
        say(f"[gpu-test] attn_verify {name} window {window}")
        kv = B.SdKv.from_buffer_copy(L.kv)
        kv.window = window
        out = torch.empty(b, d["hidden"], dtype=torch.float32, device=DEV)
        B.attn_verify(r.dims, b, x.to(DEV), L.attn_w, kv, out, r.ws)
        torch.cuda.synchronize()
        o = oracle.paged_attention(q, kc, vc, np64(lay["block_table"]), np64(lay["positions"]),
                                   d["q_rows"], window=window)
        a = oracle.gate_oproj(o, gate, np64(lay["w_o"]))
        w = assert_close(np64(out), a, f"attention output, window {window}")
        say(f"[gpu-test] attn {name} window {window}: worst scaled err {w:.2e}")


# ------------------------------------------------------------------------ routing
@pytest.mark.parametrize("name", ["tiny_b8_ctx128", "h4096_b8_ctx8k", "h4096_b64_ragged"])
def test_moe_route_matches_oracle(name):
    wk = workload(name)
    r = runner(wk)
    lay, d, b = wk["layers"][0], wk["dims"], r.b
    x = wk["act"]["front_embed"]
    z = r.route_t["logits"]
    B.moe_route(r.dims, b, x.to(DEV), r.layers[0].t["w_router"], r.act["logit_bias"], r.route, r.ws)
    torch.cuda.synchronize()
    z_ref = oracle.router_logits(np64(x), np64(lay["w_router"]), np64(wk["act"].get("logit_bias")))
    assert_close(np64(z), z_ref, "router logits", tol=1e-3)
    gid = np64(r.route_t["topk_ids"])
    flagged = check_route_stage_a(z_ref, gid, d["top_k"])
    say(f"[gpu-test] route {name}: {len(flagged)} near-tie rows")
    # the ids are exactly the (-z, index) top-k of the logits the routing ranked, every row
    assert np.array_equal(gid, oracle.topk_route(np64(z), d["top_k"])[0])
    # weights: softmax over the GPU's own selection of the exact logits
    sel = np.take_along_axis(z_ref, gid.astype(np.int64), 1)
    ex = np.exp(sel - sel.max(1, keepdims=True))
    assert_close(np64(r.route_t["topk_w"]), ex / ex.sum(1, keepdims=True), "route weights", tol=1e-3)
    counts, offsets, slot_of, tos = oracle.pooler(gid, d["n_experts"])
    assert np.array_equal(np64(r.route_t["expert_counts"]), counts)
    assert np.array_equal(np64(r.route_t["expert_offsets"]), offsets)
    assert np.array_equal(np64(r.route_t["slot_of"]), slot_of)
    assert np.array_equal(np64(r.route_t["token_of_slot"]), tos)
    act_list = np64(r.route_t["active_experts"])
    assert act_list[-1] == (counts > 0).sum()
    assert np.array_equal(act_list[:act_list[-1]], np.nonzero(counts)[0])
    if "skew_rows" in wk["act"]:
        assert np.all(gid[wk["act"]["skew_rows"], 0] == 0)


# ------------------------------------------------------------------------ experts + unpool
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_b8_ctx128", "h4096_b8_ctx8k", "h4096_b64_ragged"])
def test_moe_experts_and_unpool_match_oracle(name):
    wk = workload(name)
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
    touched = np.nonzero(counts)[0]
    subset = touched if len(touched) <= 24 else np.concatenate([touched[:1], touched[-5:]])
    say(f"[gpu-test] experts {name}: checking {len(subset)} of {len(touched)} touched experts")
    h_ref, y_ref = oracle.moe_experts(np64(x), counts, offsets, tos, np64(lay["w13_codes"]),
                                      np64(lay["w13_scales"]), np64(lay["w13_gscale"]),
                                      np64(lay["w2_codes"]), np64(lay["w2_scales"]),
                                      np64(lay["w2_gscale"]), I, experts=set(subset.tolist()))
    rows = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in subset])
    assert_close(np64(h)[rows], h_ref[rows], "SwiGLU output h")
    assert_close(np64(y)[rows], y_ref[rows], "expert output y")
    m_ref = oracle.unpool(np64(y), rt["topk_w"], rt["slot_of"])
    assert_close(np64(m), m_ref, "unpooled output")


@pytest.mark.timeout(600)
def test_moe_experts_x16_on_the_boundary_output():
    """The split-form entry point on the expert input a boundary writes (front mode: the
    pre-norm of the embedding), against the oracle's experts on the oracle's norm output."""
    wk = workload("h4096_b8_ctx8k")
    r = runner(wk)
    lay, act, d, b = wk["layers"][0], wk["act"], wk["dims"], r.b
    k, H = d["top_k"], d["hidden"]
    x = act["front_embed"]
    B.moe_route(r.dims, b, x.to(DEV), r.layers[0].t["w_router"], None, r.route, r.ws)
    s = torch.empty(b, H, dtype=torch.float32, device=DEV)
    hb = torch.empty(b, H, dtype=torch.bfloat16, device=DEV)
    x16 = torch.empty(2, b, H, dtype=torch.float16, device=DEV)
    B.boundary_dualnorm(r.dims, b, s, None, x.to(DEV), None, r.layers[0].t["g_pre_ffn"], hb,
                        out16=x16)
    y = torch.empty(b * k, H, dtype=torch.float32, device=DEV)
    B.moe_experts_x16(r.dims, b, x16, r.layers[0].moe_w, r.route, y, None, r.ws)
    torch.cuda.synchronize()
    _, x_ref = oracle.front_norm(np64(x), np64(lay["g_pre_ffn"]), d["eps"])
    rt = {kk: np64(v) for kk, v in r.route_t.items()}
    touched = np.nonzero(rt["expert_counts"])[0][:6]
    _, y_ref = oracle.moe_experts(x_ref, rt["expert_counts"], rt["expert_offsets"],
                                  rt["token_of_slot"], np64(lay["w13_codes"]),
                                  np64(lay["w13_scales"]), np64(lay["w13_gscale"]),
                                  np64(lay["w2_codes"]), np64(lay["w2_scales"]),
                                  np64(lay["w2_gscale"]), d["inter"], experts=set(touched.tolist()))
    off = rt["expert_offsets"]
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in touched])
    w = assert_close(np64(y)[rows], y_ref[rows], "expert output y (split form)")
    say(f"[gpu-test] experts x16: worst scaled err {w:.2e}")


# ------------------------------------------------------------------------ draft head
@pytest.mark.timeout(600)
def test_draft_head_full_size_matches_oracle():
    require_lib()
    w = synth.WORKLOADS["h4096_chain4_head"]
    hd = synth.make_head(w, 0)
    H, V, b = w.hidden, w.draft_vocab, w.b
    h = synth._bf16(synth._normal(0, "head_probe_h", (b, H)))
    w_lm, d2t = B.pack_dense(hd["w_lm"].to(DEV)), hd["d2t"].to(DEV)
    mult = output_multiplier(H, hd["base_width"], hd["mult_mode"])
    ws = torch.empty(B.draft_head_workspace_bytes(H, V, b), dtype=torch.uint8, device=DEV)
    tau = torch.empty(b, V, dtype=torch.float32, device=DEV)
    ids = torch.empty(b, dtype=torch.int32, device=DEV)
    tgt = torch.empty(b, dtype=torch.int64, device=DEV)
    B.draft_head(H, V, b, h.to(DEV), w_lm, mult, hd["soft_cap"], d2t, tau, ids, tgt, ws)
    torch.cuda.synchronize()
    ref = oracle.draft_head(np64(h), np64(hd["w_lm"]), mult, hd["soft_cap"], np64(hd["d2t"]))
    exact = np64(h) @ np64(hd["w_lm"]).T
    flagged = head_flags(exact)
    say(f"[gpu-test] head: {flagged.sum()} near-midpoint rows")
    gid = np64(ids)
    for t in range(b):
        if flagged[t]:
            assert exact[t, gid[t]] >= exact[t].max() - 2 * 2.0 ** -6
        else:
            assert gid[t] == ref["ids"][t], (t, gid[t], ref["ids"][t])
    assert np.array_equal(np64(tgt), np64(hd["d2t"])[gid])
    assert_close(np64(tau), ref["tau"], "transformed logits", tol=1e-2)


def test_draft_head_ties_take_the_lower_index():
    require_lib()
    H, V, b = 128, 64, 8
    w = torch.zeros(V, H, dtype=torch.bfloat16)
    w[[5, 17, 40], 0] = 1.0                  # three identical best rows
    h = torch.zeros(b, H, dtype=torch.bfloat16)
    h[:, 0] = 2.0
    d2t = torch.arange(V, dtype=torch.int64) * 7 + 3
    ws = torch.empty(B.draft_head_workspace_bytes(H, V, b), dtype=torch.uint8, device=DEV)
    ids = torch.empty(b, dtype=torch.int32, device=DEV)
    tgt = torch.empty(b, dtype=torch.int64, device=DEV)
    B.draft_head(H, V, b, h.to(DEV), B.pack_dense(w.to(DEV)), 0.25, 30.0, d2t.to(DEV), None, ids,
                 tgt, ws)
    torch.cuda.synchronize()
    assert ids.cpu().tolist() == [5] * b and tgt.cpu().tolist() == [38] * b


def test_attn_negative_slots_store_nothing_and_read_the_cache():
    """Rows with a negative slot: their new K/V are not stored, and attention reads whatever
    the cache holds at their positions (here finite values planted there)."""
    wk = workload("tiny_b8_ctx128")
    lay, d = wk["layers"][0], wk["dims"]
    rows = [2, 5]
    sm = lay["slot_mapping"].clone()
    kc0, vc0 = lay["k_cache"].clone(), lay["v_cache"].clone()
    g = torch.Generator().manual_seed(7)
    for j in rows:
        blk, off = int(sm[j]) // 16, int(sm[j]) % 16
        kc0[blk, :, off, :] = torch.randn(kc0.shape[1], kc0.shape[3], generator=g).to(kc0.dtype)
        vc0[blk, :, :, off] = torch.randn(vc0.shape[1], vc0.shape[2], generator=g).to(vc0.dtype)
        sm[j] = -1
    lay2 = dict(lay, slot_mapping=sm, k_cache=kc0, v_cache=vc0)
    wk2 = dict(wk, layers=[lay2])
    r = runner(wk2)
    b = r.b
    x = wk["act"]["front_embed"]
    out = torch.empty(b, d["hidden"], dtype=torch.float32, device=DEV)
    L = r.layers[0]
    B.attn_verify(r.dims, b, x.to(DEV), L.attn_w, L.kv, out, r.ws)
    torch.cuda.synchronize()
    q, k, v, gate = oracle.qkv_front(np64(x), np64(lay["w_qkv"]), np64(lay["positions"]),
                                     d["n_q_heads"], d["n_kv_heads"], d["head_dim"], d["eps"],
                                     d["rope_theta"], bool(d["qk_norm"]))
    kc, vc = oracle.kv_write(np64(kc0), np64(vc0), k, v, np64(sm))
    o = oracle.paged_attention(q, kc, vc, np64(lay["block_table"]), np64(lay["positions"]), d["q_rows"])
    a = oracle.gate_oproj(o, gate, np64(lay["w_o"]))
    assert_close(np64(out), a, "attention output with negative slots")
    for j in rows:  # the planted values are still there
        blk, off = int(lay["slot_mapping"][j]) // 16, int(lay["slot_mapping"][j]) % 16
        assert torch.equal(L.t["k_cache"][blk, :, off, :].cpu(), kc0[blk, :, off, :])
        assert torch.equal(L.t["v_cache"][blk, :, :, off].cpu(), vc0[blk, :, :, off])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("L", [7684, 7937])
def test_attn_new_tokens_across_chunks_and_blocks(L):
    """A request whose verify tokens straddle an attention chunk (256 tokens of 16 blocks at
    this shape; L = 7684) or a 2-block window and a block (L = 7937): each chunk's workgroup
    stores its own new tokens and reads the others from the cache."""
    wk = workload("h4096_b8_ctx8k")
    lay, d = wk["layers"][0], wk["dims"]
    q = d["q_rows"]
    pos = torch.arange(L - q, L, dtype=torch.int32)
    bt = lay["block_table"][0].long()
    sm = (bt[pos.long() // 16] * 16 + pos.long() % 16).to(torch.int64)
    lay2 = dict(lay, seq_lens=torch.tensor([L], dtype=torch.int32), positions=pos, slot_mapping=sm)
    r = runner(dict(wk, layers=[lay2]))
    b = r.b
    say(f"[gpu-test] attention with new tokens at {L - q}..{L - 1}")
    x = wk["act"]["front_embed"]
    out = torch.empty(b, d["hidden"], dtype=torch.float32, device=DEV)
    Ld = r.layers[0]
    B.attn_verify(r.dims, b, x.to(DEV), Ld.attn_w, Ld.kv, out, r.ws)
    torch.cuda.synchronize()
    qq, k, v, gate = oracle.qkv_front(np64(x), np64(lay["w_qkv"]), np64(pos),
                                      d["n_q_heads"], d["n_kv_heads"], d["head_dim"], d["eps"],
                                      d["rope_theta"], bool(d["qk_norm"]))
    kc, vc = oracle.kv_write(np64(lay["k_cache"]), np64(lay["v_cache"]), k, v, np64(sm))
    o = oracle.paged_attention(qq, kc, vc, np64(lay["block_table"]), np64(pos), q)
    a = oracle.gate_oproj(o, gate, np64(lay["w_o"]))
    assert_close(np64(out), a, "attention output")
    slots = np64(sm)
    got = np64(Ld.t["k_cache"][torch.from_numpy(slots // 16).to(DEV)])
    assert_close(got[np.arange(b), :, slots % 16, :], kc[slots // 16, :, slots % 16, :], "written K")
