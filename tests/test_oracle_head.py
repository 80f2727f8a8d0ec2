"""Pins of the oracle's final boundary, draft head and layer chain."""

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from oracle import head as OH
from speculative_verify_decode_amd import synth
from tests import torch_ref
from tests.helpers import np64, oracle_layer_inputs

RNG = np.random.default_rng(777)


def test_output_multiplier_closed_forms():
    # width_mult = hidden / base_width; mup -> 1/width_mult, sp -> width_mult**-0.5
    assert OH.output_multiplier(4096, 1024, "mup") == 0.25
    assert OH.output_multiplier(4096, 1024, "sp") == 0.5
    assert OH.output_multiplier(1024, 1024, "mup") == 1.0


def test_head_logits_are_bf16_and_transform_limits():
    h = RNG.standard_normal((4, 64))
    w = torch.from_numpy(RNG.standard_normal((300, 64)) / 8).to(torch.bfloat16).double().numpy()
    out = oracle.draft_head(h, w, 0.25, 30.0, np.arange(300) * 3)
    lg = out["logits"]
    assert np.array_equal(torch.from_numpy(lg).float().to(torch.bfloat16).double().numpy(), lg)
    # cap * tanh(x / cap): odd, monotone, below the cap, ~x for small x
    x = lg * 0.25
    assert np.all(np.abs(out["tau"]) < 30.0)
    assert np.allclose(out["tau"], x, atol=1e-3 * np.abs(x).max() ** 3 + 1e-12)
    big = oracle.draft_head(np.ones((1, 64)) * 50, np.ones((2, 64)), 1.0, 30.0, np.arange(2))
    assert np.allclose(big["tau"], 30.0, atol=1e-12)


def test_head_argmax_is_first_max_of_logits_and_d2t_gathers():
    h = RNG.standard_normal((6, 32))
    w = RNG.standard_normal((500, 32))
    d2t = RNG.choice(100000, 500, replace=False)
    out = oracle.draft_head(h, w, 0.25, 30.0, d2t)
    lg = torch.from_numpy(out["logits"])
    first = torch.argmax(lg, dim=1).numpy()     # monotone transform keeps the argmax
    assert np.array_equal(out["ids"], first)
    assert np.array_equal(out["target_ids"], d2t[out["ids"]])


def test_head_crafted_ties_go_to_lower_index():
    w = np.zeros((8, 4))
    w[2] = w[5] = w[7] = [1, 0, 0, 0]
    out = oracle.draft_head(np.array([[2.0, 0, 0, 0]]), w, 0.25, 30.0, np.arange(8) + 100)
    assert out["ids"].tolist() == [2] and out["target_ids"].tolist() == [102]


def test_head_rounds_hidden_to_bf16_first():
    # a hidden value that bf16 rounds away must not influence the logits
    h = np.array([[1.0 + 2.0 ** -10]])
    out = oracle.draft_head(h, np.array([[1.0]]), 1.0, None, np.array([0]))
    assert out["logits"][0, 0] == 1.0


def test_product_head_multiplier_follows_the_oracle():
    """The runner computes the head's multiplier from its config; it must be the oracle's."""
    from speculative_verify_decode_amd.runner import head_multiplier
    for hidden, base in ((4096, 1024), (256, 64), (1024, 1024), (6144, 256)):
        for mode in ("mup", "sp"):
            assert head_multiplier(hidden, base, mode) == OH.output_multiplier(hidden, base, mode)


def test_final_boundary_is_library_dual_norm():
    s, m = RNG.standard_normal((2, 48)), RNG.standard_normal((2, 48))
    gp, gf = 1 + 0.1 * RNG.standard_normal(48), 1 + 0.1 * RNG.standard_normal(48)
    s2, h = oracle.final_boundary(s, m, gp, gf, 1e-6)
    st = torch.from_numpy(s) + F.rms_norm(torch.from_numpy(m), (48,), torch.from_numpy(gp), 1e-6)
    assert np.allclose(s2, st.numpy(), atol=1e-13)
    assert np.allclose(h, F.rms_norm(st, (48,), torch.from_numpy(gf), 1e-6).numpy(), atol=1e-13)


def test_two_layer_chain_matches_torch_composition():
    w = synth.with_overrides(synth.WORKLOADS["tiny_b8_ctx128"], n_layers=2, draft_vocab=512,
                             target_vocab=4096, base_width=64)
    wk = synth.make_workload(w)
    act, dims, head = wk["act"], wk["dims"], wk["head"]
    layers = [oracle_layer_inputs(l, act) for l in wk["layers"]]
    out = oracle.chain_step(layers, dims, np64(act["stream"]), np64(act["branch_in"]),
                            np64(head["g_final"]), np64(head["w_lm"]),
                            OH.output_multiplier(w.hidden, head["base_width"], head["mult_mode"]),
                            head["soft_cap"], np64(head["d2t"]))
    # independent composition: torch layer twice, library rms_norm, torch argmax
    a = dict(act)
    u = act["branch_in"]
    for lay in wk["layers"]:
        r = torch_ref.layer(lay, a, dims, u)
        a = dict(a, stream=r["stream"])
        u = r["m"]
    s = r["stream"] + F.rms_norm(u, (w.hidden,), torch_ref.t64(wk["layers"][-1]["g_post_ffn"]), w.eps)
    hh = F.rms_norm(s, (w.hidden,), torch_ref.t64(head["g_final"]), w.eps)
    lg = torch_ref.bf16(torch_ref.bf16(hh) @ torch_ref.t64(head["w_lm"]).T)
    assert np.allclose(out["stream"], s.numpy(), rtol=1e-10, atol=1e-10)
    assert np.allclose(out["head"]["logits"], lg.numpy(), atol=0.02)   # bf16 ulp at most
    assert out["head"]["ids"].tolist() == torch.argmax(lg, 1).tolist()
    assert out["head"]["target_ids"].tolist() == head["d2t"][torch.argmax(lg, 1)].tolist()
    # aux taps: each layer's input-boundary stream, then the final boundary's stream
    assert len(out["aux"]) == 3
    assert np.array_equal(out["aux"][-1], out["stream"])
    for i in range(2):
        assert np.array_equal(out["aux"][i], out["layers"][i]["stream_in"])
