"""Plant plausible mistakes in the oracle (on the CPU, through monkeypatch) and check
that the pins catch each one: a dropped term, a wrong sign, an off-by-one, a wrong
tie rule, a transposed operand."""

import numpy as np
import pytest

import oracle
from oracle import formats as OF
from oracle import layer as OL
from tests import test_oracle_formats as TF
from tests import test_oracle_layer as TL

ORIG_ATTN, ORIG_E4M3, ORIG_POOLER = OL.paged_attention, OF.e4m3_decode, OL.pooler
ORIG_KV_WRITE = OL.kv_write


def _rope_wrong_sign(x, positions, theta):
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    f = theta ** (-2.0 * np.arange(half) / x.shape[-1])
    a = np.asarray(positions, np.float64)[:, None] * f
    c, s = np.cos(a)[:, None], np.sin(a)[:, None]
    return np.concatenate([x[..., :half] * c + x[..., half:] * s,
                           x[..., half:] * c - x[..., :half] * s], -1)


def _topk_high_index(z, k):
    z = np.asarray(z, np.float64)
    ids = np.stack([np.lexsort((-np.arange(z.shape[1]), -row))[:k] for row in z]).astype(np.int32)
    sel = np.take_along_axis(z, ids.astype(np.int64), 1)
    ex = np.exp(sel - sel.max(1, keepdims=True))
    return ids, ex / ex.sum(1, keepdims=True)


def _dual_norm_plain_add(stream, branch, g_post, g_pre, eps):
    s = np.asarray(stream, np.float64) + np.asarray(branch, np.float64)
    return s, OL.rmsnorm(s, g_pre, eps)


def _attn_off_by_one(q, kc, vc, bt, pos, q_rows, scale=None, window=0, query_start=None):
    return ORIG_ATTN(q, kc, vc, bt, np.asarray(pos) - 1, q_rows, scale, window, query_start)


def _window_one_too_wide(q, kc, vc, bt, pos, q_rows, scale=None, window=0, query_start=None):
    return ORIG_ATTN(q, kc, vc, bt, pos, q_rows, scale, window + 1 if window > 0 else 0,
                     query_start)


def _request_by_fixed_rows(t, q_rows, query_start=None):
    return t // q_rows          # ignores the partial drafts' row starts


def _gate_dropped(o, gate, w_o):
    return np.asarray(o, np.float64).reshape(gate.shape[0], -1) @ np.asarray(w_o, np.float64).T


def _e4m3_bias8(codes):
    return ORIG_E4M3(codes) * 0.5


def _pooler_reversed(ids, n_experts):
    c, off, slot_of, tos = ORIG_POOLER(ids, n_experts)
    b, k = slot_of.shape
    for e in range(n_experts):
        seg = slice(off[e], off[e + 1])
        tos[seg] = tos[seg][::-1]
    return c, off, slot_of, tos


def _kv_write_python_negative_index(k_cache, v_cache, k, v, slot_mapping):
    # forgets the negative-slot rule: slot -1 lands at offset 15 of the last block
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        blk, off = int(slot) // 16, int(slot) % 16
        kc[blk, :, off, :] = OF.bf16_round(k[t])
        vc[blk, :, :, off] = OF.bf16_round(v[t])
    return kc, vc


MUTANTS = [
    ("kv_write", _kv_write_python_negative_index, [TL.test_kv_write_negative_slot_writes_nothing]),
    ("rope", _rope_wrong_sign, [TL.test_rope_matches_complex_rotation]),
    ("topk_route", _topk_high_index, [TL.test_topk_ties_go_to_lower_index]),
    ("dual_norm", _dual_norm_plain_add, [TL.test_dual_norm_post_norm_on_branch_then_pre_norm]),
    ("paged_attention", _attn_off_by_one, [TL.test_paged_attention_matches_sdpa_on_gathered_kv]),
    ("paged_attention", _window_one_too_wide,
     [TL.test_window_of_one_returns_the_rows_own_value,
      lambda: TL.test_sliding_window_matches_sdpa_with_band_mask(7)]),
    ("request_of_row", _request_by_fixed_rows,
     [TL.test_partial_drafts_match_sdpa_per_request,
      TL.test_partial_drafts_equal_each_request_run_alone,
      TL.test_tiny_partial_drafts_layer_matches_independent_torch_composition]),
    ("gate_oproj", _gate_dropped, [TL.test_gate_limits]),
    ("pooler", _pooler_reversed, [TL.test_pooler_is_stable_counting_sort]),
]


@pytest.mark.parametrize("name,mutant,pins", MUTANTS, ids=[m[1].__name__.strip("_") for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(oracle, name, mutant)
    monkeypatch.setattr(OL, name, mutant)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()


def test_pins_catch_wrong_e4m3_bias(monkeypatch):
    monkeypatch.setattr(OF, "e4m3_decode", _e4m3_bias8)
    with pytest.raises(AssertionError):
        TF.test_e4m3_all_codes_match_torch()


def test_pins_catch_planted_mistake_in_whole_layer(monkeypatch):
    # a transposed-operand style slip deep inside the layer (router reads W_r^T rows in
    # the wrong order) must break the independent torch composition pin
    orig = OL.router_logits
    monkeypatch.setattr(OL, "router_logits", lambda x, w, b=None: orig(x, np.asarray(w)[::-1], b))
    with pytest.raises(AssertionError):
        TL.test_tiny_layer_matches_independent_torch_composition()
