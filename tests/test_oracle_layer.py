"""Pins of the oracle's layer step: library routines, closed forms, brute force and
invariants.  None of these re-types the oracle's own formula."""

import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import layer as OL
from speculative_verify_decode_amd import synth
from tests import torch_ref
from tests.helpers import np64, oracle_layer_inputs

RNG = np.random.default_rng(12345)


# ------------------------------------------------------------------ norms
def test_rmsnorm_matches_torch_rms_norm():
    x = RNG.standard_normal((5, 96)) * 3.0
    g = 1.0 + 0.1 * RNG.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(oracle.rmsnorm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-13)


def test_rmsnorm_scale_invariance_and_unit_rms():
    x = RNG.standard_normal((4, 64))
    assert np.allclose(oracle.rmsnorm(x, None, 0.0), oracle.rmsnorm(7.5 * x, None, 0.0), atol=1e-13)
    y = oracle.rmsnorm(x, None, 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-13)


def test_dual_norm_post_norm_on_branch_then_pre_norm():
    s = RNG.standard_normal((3, 32))
    u = RNG.standard_normal((3, 32))
    gp, gq = 1 + 0.1 * RNG.standard_normal(32), 1 + 0.1 * RNG.standard_normal(32)
    # the branch is normalised before the add: scaling it changes nothing (eps = 0)
    s0, x0 = oracle.dual_norm(s, u, gp, gq, 0.0)
    s2, x2 = oracle.dual_norm(s, 1000.0 * u, gp, gq, 0.0)
    assert np.allclose(s0, s2, atol=1e-12) and np.allclose(x0, x2, atol=1e-12)
    s1, x1 = oracle.dual_norm(s, u, gp, gq, 1e-6)
    # a zero branch leaves the stream as it was; x is then the pre-norm of the stream
    s3, x3 = oracle.dual_norm(s, np.zeros_like(u), gp, gq, 1e-6)
    assert np.array_equal(s3, s)
    ref = F.rms_norm(torch.from_numpy(s), (32,), weight=torch.from_numpy(gq), eps=1e-6).numpy()
    assert np.allclose(x3, ref, atol=1e-13)
    # the stream moves by exactly the post-normed branch (library rms_norm)
    post = F.rms_norm(torch.from_numpy(u), (32,), weight=torch.from_numpy(gp), eps=1e-6).numpy()
    assert np.allclose(s1 - s, post, atol=1e-13)


def test_front_norm_copies_embedding():
    e = RNG.standard_normal((2, 16))
    g = np.ones(16)
    s, x = oracle.front_norm(e, g, 1e-6)
    assert np.array_equal(s, e)
    assert np.allclose(x, F.rms_norm(torch.from_numpy(e), (16,), eps=1e-6).numpy(), atol=1e-14)


# ------------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    x = RNG.standard_normal((3, 4, 64))
    assert np.array_equal(oracle.rope(x, np.zeros(3, np.int64), 1e4), x)


def test_rope_matches_complex_rotation():
    x = RNG.standard_normal((5, 3, 128))
    pos = np.array([0, 1, 17, 8191, 131071])
    ref = torch_ref.rope_complex(torch.from_numpy(x), torch.from_numpy(pos), 1e4).numpy()
    assert np.allclose(oracle.rope(x, pos, 1e4), ref, atol=1e-9)


def test_rope_single_pair_closed_form():
    # D = 2: one pair, frequency theta**0 = 1, rotation by angle p
    out = oracle.rope(np.array([[[1.0, 0.0]]]), np.array([0.75]), 1e4)
    assert np.allclose(out[0, 0], [np.cos(0.75), np.sin(0.75)], atol=1e-15)


def test_rope_relative_and_norm_preserving():
    q = RNG.standard_normal((1, 1, 64))
    k = RNG.standard_normal((1, 1, 64))
    def dot(pq, pk):
        return float(np.sum(oracle.rope(q, np.array([pq]), 1e4) * oracle.rope(k, np.array([pk]), 1e4)))
    assert np.isclose(dot(100, 37), dot(100 + 999, 37 + 999), atol=1e-9)
    r = oracle.rope(q, np.array([12345]), 1e4)
    assert np.isclose(np.linalg.norm(r), np.linalg.norm(q), atol=1e-12)


def test_rope_does_not_touch_its_input():
    x = RNG.standard_normal((2, 2, 8))
    keep = x.copy()
    oracle.rope(x, np.array([3, 4]), 10.0)
    assert np.array_equal(x, keep)


# ------------------------------------------------------------------- QKV front
def test_qkv_split_order_q_k_v_gate():
    hq, hkv, d, hidden = 2, 1, 4, 3
    rows = (2 * hq + 2 * hkv) * d
    y = np.arange(rows, dtype=np.float64)[None, :]
    q, k, v, gate = oracle.qkv_split(y, hq, hkv, d)
    assert q.ravel().tolist() == list(range(0, 8))
    assert k.ravel().tolist() == list(range(8, 12))
    assert v.ravel().tolist() == list(range(12, 16))
    assert gate.ravel().tolist() == list(range(16, 24))


def test_qkv_front_without_rope_or_norm_is_the_projection():
    x = RNG.standard_normal((2, 16))
    w = RNG.standard_normal((24, 16))
    q, k, v, gate = oracle.qkv_front(x, w, np.zeros(2, np.int64), 2, 1, 4, 1e-6, 1e4, qk_norm=False)
    y = torch.from_numpy(x) @ torch.from_numpy(w).T
    assert np.allclose(np.concatenate([q.reshape(2, -1), k.reshape(2, -1), v.reshape(2, -1), gate], 1),
                       y.numpy(), atol=1e-12)


def test_head_rmsnorm_gives_unit_rms_per_head():
    x = RNG.standard_normal((3, 4, 32)) * 5
    y = oracle.head_rmsnorm(x, 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, atol=1e-12)


def test_kv_write_targets_slots_and_rounds_to_bf16():
    nb, hkv, d = 4, 2, 8
    kc = np.full((nb, hkv, 16, d), np.nan)
    vc = np.full((nb, hkv, d, 16), np.nan)
    k = RNG.standard_normal((2, hkv, d))
    v = RNG.standard_normal((2, hkv, d))
    slots = np.array([3 * 16 + 5, 0 * 16 + 15])
    k2, v2 = oracle.kv_write(kc, vc, k, v, slots)
    kb = torch.from_numpy(k).float().to(torch.bfloat16).double().numpy()
    vb = torch.from_numpy(v).float().to(torch.bfloat16).double().numpy()
    assert np.array_equal(k2[3, :, 5, :], kb[0]) and np.array_equal(k2[0, :, 15, :], kb[1])
    assert np.array_equal(v2[3, :, :, 5], vb[0]) and np.array_equal(v2[0, :, :, 15], vb[1])
    assert np.isnan(k2).sum() == kc.size - 2 * hkv * d
    assert np.isnan(kc).all()                     # input untouched


def test_kv_write_negative_slot_writes_nothing():
    """A negative slot marks a row whose K/V is not stored (vLLM's padding convention):
    the cache changes at the other rows' slots only, exactly as if the row were absent,
    and in particular the last block (where a negative index would land) is untouched."""
    nb, hkv, d = 5, 2, 8
    kc = RNG.standard_normal((nb, hkv, 16, d))
    vc = RNG.standard_normal((nb, hkv, d, 16))
    k = RNG.standard_normal((4, hkv, d))
    v = RNG.standard_normal((4, hkv, d))
    slots = np.array([2 * 16 + 3, -1, 0 * 16 + 9, -16])
    keep = slots >= 0
    k2, v2 = oracle.kv_write(kc, vc, k, v, slots)
    k3, v3 = oracle.kv_write(kc, vc, k[keep], v[keep], slots[keep])
    assert np.array_equal(k2, k3) and np.array_equal(v2, v3)
    assert np.array_equal(k2[nb - 1], kc[nb - 1]) and np.array_equal(v2[nb - 1], vc[nb - 1])
    changed = np.argwhere((k2 != kc).any(axis=(1, 3)))           # (block, offset) pairs
    assert sorted(map(tuple, changed.tolist())) == [(0, 9), (2, 3)]
    k4, v4 = oracle.kv_write(kc, vc, k, v, np.full(4, -5))
    assert np.array_equal(k4, kc) and np.array_equal(v4, vc)


# ------------------------------------------------------------------- attention
def _attn_case(n_req=2, q_rows=8, hq=4, hkv=2, d=16, lens=(45, 70), nb=16, seed=0):
    rng = np.random.default_rng(seed)
    need = [-(-L // 16) for L in lens]
    perm = rng.permutation(nb)
    bt = np.zeros((n_req, max(need)), np.int64)
    o = 0
    for r, n in enumerate(need):
        bt[r, :n] = perm[o:o + n]
        o += n
    kc = rng.standard_normal((nb, hkv, 16, d))
    vc = rng.standard_normal((nb, hkv, d, 16))
    pos = np.concatenate([np.arange(L - q_rows, L) for L in lens])
    q = rng.standard_normal((n_req * q_rows, hq, d))
    return q, kc, vc, bt, pos


def _ragged_case(q_lens=(8, 3, 1, 5), lens=(45, 70, 20, 33), hq=4, hkv=2, d=16, nb=24, seed=0):
    """Partial drafts: request r verifies q_lens[r] rows at positions L_r - q_r .. L_r - 1."""
    rng = np.random.default_rng(seed)
    need = [-(-L // 16) for L in lens]
    perm = rng.permutation(nb)
    bt = np.zeros((len(lens), max(need)), np.int64)
    o = 0
    for r, n in enumerate(need):
        bt[r, :n] = perm[o:o + n]
        o += n
    kc = rng.standard_normal((nb, hkv, 16, d))
    vc = rng.standard_normal((nb, hkv, d, 16))
    pos = np.concatenate([np.arange(L - qn, L) for L, qn in zip(lens, q_lens)])
    qs = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    q = rng.standard_normal((int(qs[-1]), hq, d))
    return q, kc, vc, bt, pos, qs


def _sdpa_reference(q, kc, vc, bt, pos, q_rows, window=0, starts=None):
    b, hq, d = q.shape
    hkv = kc.shape[1]
    out = np.zeros_like(q)
    starts = list(range(0, b + 1, q_rows)) if starts is None else [int(v) for v in starts]
    for r in range(len(starts) - 1):
        rows = slice(starts[r], starts[r + 1])
        L = int(pos[starts[r + 1] - 1]) + 1
        t = np.arange(L)
        k = torch.from_numpy(kc[bt[r, t // 16], :, t % 16, :]).permute(1, 0, 2)
        v = torch.from_numpy(vc[bt[r, t // 16], :, :, t % 16]).permute(1, 0, 2)
        k, v = k.repeat_interleave(hq // hkv, 0), v.repeat_interleave(hq // hkv, 0)
        mask = t[None, :] <= pos[rows][:, None]
        if window > 0:                                  # band of the w most recent positions
            mask &= t[None, :] > pos[rows][:, None] - window
        mask = torch.from_numpy(mask)
        qq = torch.from_numpy(q[rows]).permute(1, 0, 2)
        out[rows] = F.scaled_dot_product_attention(qq, k, v, attn_mask=mask).permute(1, 0, 2).numpy()
    return out


def test_paged_attention_matches_sdpa_on_gathered_kv():
    q, kc, vc, bt, pos = _attn_case()
    got = oracle.paged_attention(q, kc, vc, bt, pos, 8)
    assert np.allclose(got, _sdpa_reference(q, kc, vc, bt, pos, 8), atol=1e-12)


@pytest.mark.parametrize("window", [1, 2, 7, 16, 23, 40])
def test_sliding_window_matches_sdpa_with_band_mask(window):
    q, kc, vc, bt, pos = _attn_case(seed=11)
    got = oracle.paged_attention(q, kc, vc, bt, pos, 8, window=window)
    assert np.allclose(got, _sdpa_reference(q, kc, vc, bt, pos, 8, window=window), atol=1e-12)


def test_partial_drafts_match_sdpa_per_request():
    q, kc, vc, bt, pos, qs = _ragged_case(seed=21)
    got = oracle.paged_attention(q, kc, vc, bt, pos, 8, query_start=qs)
    assert np.allclose(got, _sdpa_reference(q, kc, vc, bt, pos, 8, starts=qs), atol=1e-12)


def test_partial_drafts_equal_each_request_run_alone():
    # requests are independent: each one's rows, run as a one-request step on its own block
    # table row, give exactly the rows of the ragged step
    q, kc, vc, bt, pos, qs = _ragged_case(seed=22)
    got = oracle.paged_attention(q, kc, vc, bt, pos, 8, query_start=qs)
    for r in range(len(qs) - 1):
        rows = slice(qs[r], qs[r + 1])
        alone = oracle.paged_attention(q[rows], kc, vc, bt[r:r + 1], pos[rows], 8)
        assert np.array_equal(got[rows], alone), r


def test_uniform_query_start_is_the_default_split():
    q, kc, vc, bt, pos = _attn_case(seed=23)
    qs = np.arange(0, q.shape[0] + 1, 8)
    assert np.array_equal(oracle.paged_attention(q, kc, vc, bt, pos, 8, query_start=qs),
                          oracle.paged_attention(q, kc, vc, bt, pos, 8))


def test_request_of_row_follows_query_start():
    qs = [0, 8, 11, 12, 17]
    want = [0] * 8 + [1] * 3 + [2] + [3] * 5
    assert [oracle.request_of_row(t, 8, qs) for t in range(17)] == want
    assert [oracle.request_of_row(t, 8) for t in range(17)] == [t // 8 for t in range(17)]
    with pytest.raises(ValueError):
        oracle.request_of_row(17, 8, qs)


def test_window_of_one_returns_the_rows_own_value():
    # one visible key: softmax weight 1, so the output is V at the row's own position
    q, kc, vc, bt, pos = _attn_case(hq=4, hkv=2, seed=12)
    got = oracle.paged_attention(q, kc, vc, bt, pos, 8, window=1)
    for t in range(q.shape[0]):
        p = int(pos[t])
        blk = bt[t // 8, p // 16]
        for h in range(4):
            assert np.array_equal(got[t, h], vc[blk, h // 2, :, p % 16])


def test_window_covering_the_context_equals_full_causal():
    q, kc, vc, bt, pos = _attn_case(seed=13)
    full = oracle.paged_attention(q, kc, vc, bt, pos, 8)
    for w in (int(pos.max()) + 1, 10 ** 6):
        assert np.array_equal(oracle.paged_attention(q, kc, vc, bt, pos, 8, window=w), full)


def test_paged_attention_block_table_permutation_invariant():
    q, kc, vc, bt, pos = _attn_case(seed=3)
    perm = np.random.default_rng(9).permutation(kc.shape[0])
    inv = np.argsort(perm)
    kc2, vc2 = kc[perm], vc[perm]          # block i of the new pool is old block perm[i]
    bt2 = inv[bt]
    got = oracle.paged_attention(q, kc2, vc2, bt2, pos, 8)
    assert np.allclose(got, oracle.paged_attention(q, kc, vc, bt, pos, 8), atol=1e-13)


def test_paged_attention_single_block_equals_unpaged():
    rng = np.random.default_rng(4)
    d, L = 8, 16
    q = rng.standard_normal((8, 1, d))
    kc = rng.standard_normal((1, 1, 16, d))
    vc = rng.standard_normal((1, 1, d, 16))
    pos = np.arange(L - 8, L)
    got = oracle.paged_attention(q, kc, vc, np.zeros((1, 1), np.int64), pos, 8)
    k, v = kc[0, 0], vc[0, 0].T
    for j in range(8):
        sc = k[:pos[j] + 1] @ q[j, 0] / np.sqrt(d)
        a = np.exp(sc - sc.max())
        want = (a / a.sum()) @ v[:pos[j] + 1]
        assert np.allclose(got[j, 0], want, atol=1e-13)


def test_verify_row_equals_single_token_decode():
    q, kc, vc, bt, pos = _attn_case(seed=5)
    full = oracle.paged_attention(q, kc, vc, bt, pos, 8)
    for t in (0, 5, 9, 15):
        r = t // 8
        one = oracle.paged_attention(q[t:t + 1], kc, vc, bt[r:r + 1], pos[t:t + 1], 1)
        assert np.allclose(one[0], full[t], atol=1e-13)


def test_gqa_uses_kv_head_h_div_group():
    q, kc, vc, bt, pos = _attn_case(hq=4, hkv=2, seed=6)
    got = oracle.paged_attention(q, kc, vc, bt, pos, 8)
    # heads 0,1 read KV head 0 and heads 2,3 read KV head 1: run each half as MHA-1
    lo = oracle.paged_attention(q[:, :2], kc[:, :1], vc[:, :1], bt, pos, 8)
    hi = oracle.paged_attention(q[:, 2:], kc[:, 1:], vc[:, 1:], bt, pos, 8)
    assert np.allclose(got, np.concatenate([lo, hi], 1), atol=1e-14)


def test_gate_limits():
    o = RNG.standard_normal((2, 8))
    w = RNG.standard_normal((5, 8))
    big = np.full((2, 8), 800.0)
    assert np.allclose(oracle.gate_oproj(o, big, w), o @ w.T, atol=1e-13)
    assert np.allclose(oracle.gate_oproj(o, np.zeros((2, 8)), w), 0.5 * (o @ w.T), atol=1e-13)
    assert np.allclose(oracle.gate_oproj(o, np.full((2, 8), -800.0), w), 0.0, atol=1e-300)


# ------------------------------------------------------------------- routing
def test_topk_matches_bruteforce_over_subsets():
    z = RNG.standard_normal((40, 8))
    z[3, 5] = z[3, 2]                               # crafted exact tie
    z[7] = 0.25                                     # all tied
    ids, w = oracle.topk_route(z, 2)
    for t in range(z.shape[0]):
        best = None
        for sub in itertools.combinations(range(8), 2):
            key = (-sum(z[t, list(sub)]), sub)     # lexicographically smallest set wins ties
            if best is None or key < best:
                best = key
        assert tuple(sorted(ids[t].tolist())) == best[1], t
        assert z[t, ids[t, 0]] >= z[t, ids[t, 1]]
    assert ids[7].tolist() == [0, 1]
    assert 2 in ids[3].tolist() or z[3].argsort()[-1] not in (2, 5)


def test_topk_ties_go_to_lower_index():
    z = np.array([[1.0, 3.0, 3.0, 3.0, 0.0]])
    ids, _ = oracle.topk_route(z, 2)
    assert ids.tolist() == [[1, 2]]


def test_topk_weights_are_renormalised_full_softmax():
    z = RNG.standard_normal((6, 32))
    ids, w = oracle.topk_route(z, 4)
    full = torch.softmax(torch.from_numpy(z), dim=1).numpy()
    sel = np.take_along_axis(full, ids.astype(np.int64), 1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), atol=1e-14)
    tv, ti = torch.topk(torch.from_numpy(z), 4, dim=1)
    assert np.array_equal(ids, ti.numpy())


def test_pooler_is_stable_counting_sort():
    ids = np.stack([RNG.permutation(32)[:4] for _ in range(64)]).astype(np.int32)
    counts, offsets, slot_of, token_of_slot = oracle.pooler(ids, 32)
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=32))
    flat = ids.ravel()
    order = np.argsort(flat, kind="stable")          # library stable sort by expert
    assert np.array_equal(token_of_slot, order // 4)
    assert np.array_equal(np.sort(slot_of.ravel()), np.arange(64 * 4))   # bijection
    assert np.array_equal(token_of_slot[slot_of], np.repeat(np.arange(64)[:, None], 4, 1))
    assert offsets[-1] == 256 and np.array_equal(np.diff(offsets), counts)


# ------------------------------------------------------------------- experts
def _fp4_expert(rng, e, i, h):
    w13c = rng.integers(0, 256, (e, 2 * i, h // 2), dtype=np.uint8)
    w13s = rng.integers(0x20, 0x40, (e, 2 * i, h // 16), dtype=np.uint8)
    w2c = rng.integers(0, 256, (e, h, i // 2), dtype=np.uint8)
    w2s = rng.integers(0x20, 0x40, (e, h, i // 16), dtype=np.uint8)
    return w13c, w13s, np.ones(e), w2c, w2s, np.ones(e)


def test_expert_ffn_matches_torch_silu():
    x = RNG.standard_normal((3, 32))
    w13 = RNG.standard_normal((32, 32))
    w2 = RNG.standard_normal((32, 16))
    h, y = oracle.expert_ffn(x, w13, w2, 16)
    gu = torch.from_numpy(x) @ torch.from_numpy(w13).T
    ht = F.silu(gu[:, :16]) * gu[:, 16:]
    assert np.allclose(h, ht.numpy(), atol=1e-12)
    assert np.allclose(y, (ht @ torch.from_numpy(w2).T).numpy(), atol=1e-11)


def test_moe_expert_permutation_invariance():
    rng = np.random.default_rng(7)
    E, I, H, b, k = 6, 32, 64, 5, 2
    ex = _fp4_expert(rng, E, I, H)
    x = rng.standard_normal((b, H))
    wr = rng.standard_normal((E, H))
    def run(perm):
        z = oracle.router_logits(x, wr[perm])
        ids, w = oracle.topk_route(z, k)
        c, off, slot_of, tos = oracle.pooler(ids, E)
        args = [a[perm] for a in ex]
        _, y = oracle.moe_experts(x, c, off, tos, *args, I)
        return oracle.unpool(y, w, slot_of)
    base = run(np.arange(E))
    assert np.allclose(run(rng.permutation(E)), base, atol=1e-10)


def test_moe_topk_all_with_identical_experts_is_dense_ffn():
    rng = np.random.default_rng(8)
    E, I, H, b = 4, 32, 64, 3
    one = _fp4_expert(rng, 1, I, H)
    ex = [np.repeat(a, E, axis=0) for a in one]
    x = rng.standard_normal((b, H))
    z = rng.standard_normal((b, E))
    ids, w = oracle.topk_route(z, E)
    c, off, slot_of, tos = oracle.pooler(ids, E)
    _, y = oracle.moe_experts(x, c, off, tos, *ex, I)
    m = oracle.unpool(y, w, slot_of)
    from oracle.formats import dequant_nvfp4
    _, dense = oracle.expert_ffn(x, dequant_nvfp4(one[0][0], one[1][0], 1.0),
                                 dequant_nvfp4(one[3][0], one[4][0], 1.0), I)
    assert np.allclose(m, dense, atol=1e-9 * (1 + np.abs(dense).max()))


def test_unpool_sums_in_choice_order():
    y = RNG.standard_normal((6, 4))
    slot_of = np.array([[4, 0], [1, 5], [2, 3]])
    w = np.array([[0.25, 0.75], [0.5, 0.5], [1.0, 0.0]])
    m = oracle.unpool(y, w, slot_of)
    for t in range(3):
        assert np.allclose(m[t], w[t, 0] * y[slot_of[t, 0]] + w[t, 1] * y[slot_of[t, 1]], atol=0)


# ------------------------------------------------------------------- whole layer
def test_tiny_layer_matches_independent_torch_composition():
    wk = synth.make_workload("tiny_b8_ctx128")
    lay, act, dims = wk["layers"][0], wk["act"], wk["dims"]
    ref = torch_ref.layer(lay, act, dims, act["branch_in"])
    out = oracle.layer_step(oracle_layer_inputs(lay, act), dims, branch_in=np64(act["branch_in"]))
    for key in ("aux", "x_a", "gate", "o", "a", "stream", "x_m", "z", "w", "m"):
        r = ref[key].numpy().reshape(out[key].shape)
        assert np.allclose(out[key], r, rtol=1e-10, atol=1e-10), key
    for key in ("q", "k", "v"):
        assert np.allclose(out[key], ref[key].numpy(), atol=1e-10), key
    assert np.array_equal(out["ids"], ref["ids"].numpy())
    assert np.isfinite(out["m"]).all() and np.isfinite(out["stream"]).all()


def test_aux_tap_is_the_stream_entering_the_attention_block():
    """The aux tap is the stream the input boundary hands on: its pre-norm is the attention
    input, and at the front it is the embedding itself (a copy, not a view)."""
    wk = synth.make_workload("tiny_b8_ctx128")
    lay, act, dims = wk["layers"][0], wk["act"], wk["dims"]
    out = oracle.layer_step(oracle_layer_inputs(lay, act), dims, branch_in=np64(act["branch_in"]))
    g = torch.from_numpy(np64(lay["g_pre_attn"]))
    x_ref = F.rms_norm(torch.from_numpy(out["aux"]), (dims["hidden"],), g, dims["eps"]).numpy()
    assert np.allclose(out["x_a"], x_ref, rtol=1e-12, atol=1e-12)
    assert not np.allclose(out["aux"], out["stream"])       # the attention boundary moved on
    front = oracle.layer_step(oracle_layer_inputs(lay, act), dims,
                              front_embed=np64(act["front_embed"]))
    assert np.array_equal(front["aux"], np64(act["front_embed"]))


def test_tiny_partial_drafts_layer_matches_independent_torch_composition():
    wk = synth.make_workload("tiny_partial")
    lay, act, dims = wk["layers"][0], wk["act"], wk["dims"]
    assert lay["query_start"].tolist() == [0, 8, 11, 12, 17] and act["stream"].shape[0] == 17
    ref = torch_ref.layer(lay, act, dims, act["branch_in"])
    out = oracle.layer_step(oracle_layer_inputs(lay, act), dims, branch_in=np64(act["branch_in"]))
    for key in ("o", "a", "stream", "m"):
        r = ref[key].numpy().reshape(out[key].shape)
        assert np.allclose(out[key], r, rtol=1e-10, atol=1e-10), key
    assert np.array_equal(out["ids"], ref["ids"].numpy())
    assert np.isfinite(out["m"]).all()


def test_tiny_layer_slot_mapping_matches_block_table():
    kv = synth.make_kv(synth.WORKLOADS["tiny_b8_ctx128"], 0)
    bt, pos, sm = kv["block_table"].numpy(), kv["positions"].numpy(), kv["slot_mapping"].numpy()
    for t, p in enumerate(pos):
        assert sm[t] == bt[t // 8, p // 16] * 16 + p % 16


def test_tiny_layer_qk_norm_off_still_matches_torch():
    w = synth.with_overrides(synth.WORKLOADS["tiny_b8_ctx128"], qk_norm=0)
    wk = synth.make_workload(w)
    lay, act, dims = wk["layers"][0], wk["act"], wk["dims"]
    ref = torch_ref.layer(lay, act, dims, act["branch_in"])
    out = oracle.layer_step(oracle_layer_inputs(lay, act), dims, branch_in=np64(act["branch_in"]))
    assert np.allclose(out["m"], ref["m"].numpy(), rtol=1e-10, atol=1e-10)
