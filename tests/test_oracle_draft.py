"""Pins of the draft-side oracle (dense decoder layer, context-K/V store): an independent
torch fp64 composition (``tests/torch_ref.py``), closed forms and invariants, and planted
mistakes that the pins must catch."""

import numpy as np
import pytest
import torch

import oracle
from oracle import draft as OD
from speculative_verify_decode_amd import synth
from tests import torch_ref as TR
from tests.helpers import np64

WK = synth.make_workload("tiny_dense")
D = WK["dims"]


def _dense_inputs(lay, stream):
    inp = {k: np64(lay[k]) for k in ("g_pre_attn", "g_post_attn", "g_pre_ffn", "g_post_ffn",
                                     "w_qkv", "w_o", "w_gate_up", "w_down", "k_cache",
                                     "v_cache", "block_table", "positions", "slot_mapping")}
    inp["stream"] = np64(stream)
    inp["window"] = int(lay.get("window", 0))
    return inp


def _ctx_inputs():
    ctx, lays = WK["context"], WK["layers"]
    hkv, d = D["n_kv_heads"], D["head_dim"]
    qs = D["n_q_heads"] * d
    w_kv = np.stack([np64(l["w_qkv"])[qs:qs + 2 * hkv * d] for l in lays])
    g_pre = np.stack([np64(l["g_pre_attn"]) for l in lays])
    return ctx, w_kv, g_pre


@pytest.mark.parametrize("window", [0, 20])
def test_dense_layer_matches_torch_composition(window):
    lay = dict(WK["layers"][0], window=window)
    ref = TR.dense_layer(lay, WK["act"]["stream"], D)
    got = OD.dense_layer_step(_dense_inputs(lay, WK["act"]["stream"]), D)
    for key in ("x_a", "a", "x_f", "h", "y", "stream"):
        r = ref[key].numpy()
        assert np.allclose(got[key], r, rtol=1e-9, atol=1e-9 * np.abs(r).max()), key


def test_dense_ffn_closed_form():
    # one hidden unit: gate and up rows pick single coordinates of x
    x = np.array([[1.5, -2.0, 0.25]])
    w_gu = np.array([[1.0, 0.0, 0.0],    # gate = x0
                     [0.0, 0.0, 4.0]])   # up = 4 x2
    w_down = np.array([[2.0], [-1.0], [0.0]])
    h, y = OD.dense_ffn(x, w_gu, w_down, 1)
    g, u = 1.5, 1.0
    want_h = g / (1.0 + np.exp(-g)) * u
    assert np.isclose(h[0, 0], want_h, rtol=1e-15)
    assert np.allclose(y[0], [2.0 * want_h, -want_h, 0.0], rtol=1e-15)
    # a zero gate gives silu(0) = 0: no output whatever the up projection
    h0, y0 = OD.dense_ffn(np.array([[0.0, 3.0, 7.0]]), w_gu, w_down, 1)
    assert h0[0, 0] == 0.0 and not y0.any()


def test_dense_layer_input_norms_see_the_bf16_stream():
    # a stream already on the bf16 grid and the same stream nudged below half a bf16 ulp
    # give the same attention and FFN inputs: both pre-norms read bf16(stream)
    lay = WK["layers"][0]
    s = np64(TR.bf16(WK["act"]["stream"]))
    nudged = s * (1.0 + 2.0 ** -12)
    a = OD.dense_layer_step(_dense_inputs(lay, s), D)
    b = OD.dense_layer_step(_dense_inputs(lay, nudged), D)
    assert np.array_equal(a["x_a"], b["x_a"])
    assert not np.array_equal(a["stream"], b["stream"])   # the fp32 stream itself is kept


def test_context_kv_matches_torch_composition():
    ctx, w_kv, g_pre = _ctx_inputs()
    hkv, d = D["n_kv_heads"], D["head_dim"]
    k, v = OD.context_kv(np64(ctx["states"]), np64(ctx["g_hidden"]), g_pre, w_kv,
                         np64(ctx["positions"]), hkv, d, D["eps"], D["rope_theta"])
    kr, vr = TR.context_kv(ctx["states"], ctx["g_hidden"], torch.from_numpy(g_pre),
                           torch.from_numpy(w_kv), ctx["positions"], hkv, d, D["eps"],
                           D["rope_theta"])
    assert np.array_equal(v, vr.numpy())
    # K passes three bf16 roundings; a value that lands on a rounding midpoint in one
    # fp64 evaluation order and not the other moves by one bf16 step, so allow that
    diff = np.abs(k - kr.numpy())
    step = np.abs(kr.numpy()) * 2.0 ** -7 + 1e-30
    assert (diff <= step).all() and (diff > 0).mean() < 1e-3


def test_context_k_norm_and_rotation_invariants():
    ctx, w_kv, g_pre = _ctx_inputs()
    hkv, d = D["n_kv_heads"], D["head_dim"]
    k, _ = OD.context_kv(np64(ctx["states"]), np64(ctx["g_hidden"]), g_pre, w_kv,
                         np64(ctx["positions"]), hkv, d, D["eps"], D["rope_theta"])
    # weightless RMSNorm then a rotation: every head vector has mean square ~1
    ms = (k ** 2).mean(-1)
    assert np.allclose(ms, 1.0, atol=2e-2)
    # at position 0 the rotation is the identity: K is the norms, the matmul and the K norm
    # written out step by step, with the bf16 casts of the context chain
    eps = D["eps"]
    x0 = np64(ctx["states"])[:1]
    k0, _ = OD.context_kv(x0, np64(ctx["g_hidden"]), g_pre, w_kv, np.zeros(1), hkv, d, eps,
                          D["rope_theta"])
    bf = oracle.bf16_round
    fc = bf(x0 / np.sqrt((x0 ** 2).mean() + eps) * np64(ctx["g_hidden"]))
    for li in range(len(g_pre)):
        xl = bf(fc / np.sqrt((fc ** 2).mean() + eps) * g_pre[li])
        kk = bf(xl @ w_kv[li].T)[0, :hkv * d].reshape(hkv, d)
        kk = bf(kk / np.sqrt((kk ** 2).mean(-1, keepdims=True) + eps))
        assert np.array_equal(k0[li, 0], kk), li


def test_context_kv_store_writes_only_its_slots():
    ctx, w_kv, g_pre = _ctx_inputs()
    lays = WK["layers"]
    k, v = OD.context_kv(np64(ctx["states"]), np64(ctx["g_hidden"]), g_pre, w_kv,
                         np64(ctx["positions"]), D["n_kv_heads"], D["head_dim"], D["eps"],
                         D["rope_theta"])
    kcs = [np64(l["k_cache"]) for l in lays]
    vcs = [np64(l["v_cache"]) for l in lays]
    nk, nv = OD.context_kv_store(kcs, vcs, k, v, [np64(s) for s in ctx["slot_mappings"]])
    for li, sm in enumerate(ctx["slot_mappings"]):
        sm = np64(sm).astype(np.int64)
        blocks = set((sm // 16).tolist())
        for blk in range(kcs[li].shape[0]):
            if blk not in blocks:
                assert np.array_equal(nk[li][blk], kcs[li][blk], equal_nan=True)
        for j, slot in enumerate(sm):
            assert np.array_equal(nk[li][slot // 16, :, slot % 16, :], k[li, j])
            assert np.array_equal(nv[li][slot // 16, :, :, slot % 16], v[li, j])


# ---------------------------------------------------------------- planted mistakes
def _ffn_gate_up_swapped(x, w_gate_up, w_down, inter):
    w = np.asarray(w_gate_up, np.float64)
    return ORIG_FFN(x, np.concatenate([w[inter:], w[:inter]]), w_down, inter)


def _ffn_no_gate_activation(x, w_gate_up, w_down, inter):
    gu = np.asarray(x, np.float64) @ np.asarray(w_gate_up, np.float64).T
    h = gu[:, :inter] * gu[:, inter:]
    return h, h @ np.asarray(w_down, np.float64).T


ORIG_FFN = OD.dense_ffn


@pytest.mark.parametrize("mutant", [_ffn_gate_up_swapped, _ffn_no_gate_activation])
def test_dense_pin_catches_planted_mistake(monkeypatch, mutant):
    monkeypatch.setattr(OD, "dense_ffn", mutant)
    with pytest.raises(AssertionError):
        test_dense_layer_matches_torch_composition(0)


def test_context_pin_catches_missing_k_norm(monkeypatch):
    monkeypatch.setattr(OD, "head_rmsnorm", lambda x, eps: np.asarray(x, np.float64))
    with pytest.raises(AssertionError):
        test_context_kv_matches_torch_composition()
