"""Seeded synthetic inputs for the verify-decode layer step.

This module draws random numbers and lays them out in the library's boundary layouts.
It holds none of the step's arithmetic: bf16 and E4M3 encodings are torch's own
dtype conversions, and the only computed metadata are the step's positions and slot
mapping, which the serving runtime would hand to the step.  Both the GPU harness and
the CPU oracle tests take their inputs from here, and from nowhere else.

Each tensor draws from its own PCG64 stream keyed by (seed, tensor name), so the order
of generation does not change any value.
"""

from dataclasses import dataclass, replace
import zlib

import numpy as np
import torch

BLOCK = 16


@dataclass(frozen=True)
class Workload:
    """Shapes and input recipe of one workload."""
    name: str
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    inter: int
    n_req: int
    ctx: tuple = ()                   # fixed per-request context lengths (incl. 8 verify)
    ctx_range: tuple = ()             # (lo, hi) inclusive, uniform, when ctx is empty
    pool_blocks: int = 0              # minimum KV pool size in blocks
    q_rows: int = 8                   # 1 + 7 speculative tokens per request
    eps: float = 1e-6
    rope_theta: float = 1e4
    qk_norm: int = 1
    skew_rows: float = 0.0            # fraction of rows biased toward expert 0
    skew_bias: float = 8.0
    n_layers: int = 1
    draft_vocab: int = 0              # > 0: a draft head follows the last layer
    target_vocab: int = 0
    base_width: int = 1024            # the draft head's base width (width_mult = hidden / it)
    mult_mode: str = "mup"            # the draft head's output-multiplier rule
    soft_cap: float = 30.0
    window: int = 0                   # sliding window of every layer (0: full causal)
    dense_inter: int = 0              # > 0: layers also carry a dense feed-forward (draft)
    n_ctx: int = 0                    # > 0: context rows for the context-K/V store
    q_lens: tuple = ()                # partial drafts: verify rows per request (1..q_rows)
    seed: int = 0

    @property
    def verify_rows(self):
        """Verify rows of each request: q_lens, or q_rows for every request."""
        if self.q_lens:
            assert len(self.q_lens) == self.n_req
            assert all(1 <= q <= self.q_rows for q in self.q_lens)
            return tuple(int(q) for q in self.q_lens)
        return (self.q_rows,) * self.n_req

    @property
    def b(self):
        return sum(self.verify_rows)

    @property
    def qkv_rows(self):
        return (2 * self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def dims(self):
        """The step's dimensions as a plain mapping (oracle and binding both read it)."""
        return dict(hidden=self.hidden, n_q_heads=self.n_q_heads, n_kv_heads=self.n_kv_heads,
                    head_dim=self.head_dim, q_rows=self.q_rows, block_size=BLOCK,
                    n_experts=self.n_experts, top_k=self.top_k, inter=self.inter,
                    qk_norm=self.qk_norm, eps=self.eps, rope_theta=self.rope_theta,
                    dense_inter=self.dense_inter)


_BIG = dict(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, n_experts=32, top_k=4,
            inter=1536)

WORKLOADS = {
    "tiny_b8_ctx128": Workload("tiny_b8_ctx128", hidden=256, n_q_heads=4, n_kv_heads=1,
                               head_dim=64, n_experts=8, top_k=2, inter=128, n_req=1,
                               ctx=(128,), pool_blocks=64),
    "h4096_b8_ctx8k": Workload("h4096_b8_ctx8k", n_req=1, ctx=(8192,), pool_blocks=4096, **_BIG),
    "h4096_b64_ragged": Workload("h4096_b64_ragged", n_req=8, ctx_range=(1024, 32768),
                                 pool_blocks=4096, skew_rows=0.25, **_BIG),
    "h4096_b8_ctx131k": Workload("h4096_b8_ctx131k", n_req=1, ctx=(131072,),
                                 pool_blocks=8192 + 64, **_BIG),
    "h4096_b8_ctx131k_win8k": Workload("h4096_b8_ctx131k_win8k", n_req=1, ctx=(131072,),
                                       pool_blocks=8192 + 64, window=8192, **_BIG),
    "tiny_dense": Workload("tiny_dense", hidden=256, n_q_heads=4, n_kv_heads=1, head_dim=64,
                           n_experts=8, top_k=2, inter=128, n_req=1, ctx=(128,), pool_blocks=64,
                           dense_inter=512, n_layers=2, n_ctx=8),
    "h4096_b8_ctx8k_dense": Workload("h4096_b8_ctx8k_dense", n_req=1, ctx=(8192,),
                                     pool_blocks=4096, dense_inter=8192, n_ctx=8, **_BIG),
    "tiny_partial": Workload("tiny_partial", hidden=256, n_q_heads=4, n_kv_heads=1, head_dim=64,
                             n_experts=8, top_k=2, inter=128, n_req=4, ctx=(128, 45, 20, 97),
                             q_lens=(8, 3, 1, 5), pool_blocks=64),
    "h4096_partial_drafts": Workload("h4096_partial_drafts", n_req=8, ctx_range=(1024, 32768),
                                     q_lens=(8, 3, 1, 6, 8, 2, 5, 7), pool_blocks=4096, **_BIG),
    "h4096_chain4_head": Workload("h4096_chain4_head", n_req=1, ctx=(8192,), pool_blocks=4096,
                                  n_layers=4, draft_vocab=32768, target_vocab=131072, **_BIG),
}


def rng_for(seed, name):
    return np.random.default_rng(np.random.SeedSequence([int(seed), zlib.crc32(name.encode())]))


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _normal(seed, name, shape, std=1.0):
    return rng_for(seed, name).standard_normal(shape, dtype=np.float32) * np.float32(std)


def _e4m3_codes(values):
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8)


def context_lengths(w: Workload, seed=None):
    seed = w.seed if seed is None else seed
    if w.ctx:
        assert len(w.ctx) == w.n_req
        return np.array(w.ctx, dtype=np.int64)
    lo, hi = w.ctx_range
    return rng_for(seed, "ctx_lens").integers(lo, hi, size=w.n_req, endpoint=True)


def make_kv(w: Workload, seed, tag=""):
    """Paged bf16 KV caches and the step metadata.

    K cache [num_blocks, Hkv, 16, D]; V cache [num_blocks, Hkv, D, 16].  Each request's
    blocks are a seeded random choice from the pool with no aliasing.  Context tokens
    (positions < L - q_r, q_r the request's verify rows) hold N(0,1); the verify slots,
    every unused block and the tail of each last partial block hold NaN, so a read before
    the write or past the end shows up as NaN.  With partial drafts (q_lens) the metadata
    also holds query_start, int32 [n_req + 1], the first row of each request.
    """
    lens = context_lengths(w, seed)
    need = [int(-(-L // BLOCK)) for L in lens]
    nb = max(w.pool_blocks, sum(need) + 64)
    max_blocks = max(need)
    perm = rng_for(seed, tag + "block_perm").permutation(nb)
    bt = np.zeros((w.n_req, max_blocks), dtype=np.int32)
    o = 0
    for r, n in enumerate(need):
        bt[r, :n] = perm[o:o + n]
        o += n
    hkv, d = w.n_kv_heads, w.head_dim
    k = np.full((nb, hkv, BLOCK, d), np.nan, dtype=np.float32)
    v = np.full((nb, hkv, d, BLOCK), np.nan, dtype=np.float32)
    qn = w.verify_rows
    for r, L in enumerate(lens):
        n_ctx = int(L) - qn[r]
        full, rem = n_ctx // BLOCK, n_ctx % BLOCK
        blocks = bt[r, :full]
        if full:
            k[blocks] = _normal(seed, f"{tag}k{r}", (full, hkv, BLOCK, d))
            v[blocks] = _normal(seed, f"{tag}v{r}", (full, hkv, d, BLOCK))
        if rem:
            k[bt[r, full], :, :rem, :] = _normal(seed, f"{tag}kt{r}", (hkv, rem, d))
            v[bt[r, full], :, :, :rem] = _normal(seed, f"{tag}vt{r}", (hkv, d, rem))
    starts = np.concatenate([[0], np.cumsum(qn)]).astype(np.int32)
    positions = np.zeros(w.b, dtype=np.int32)
    slots = np.zeros(w.b, dtype=np.int64)
    for r, L in enumerate(lens):
        for j in range(qn[r]):
            p = int(L) - qn[r] + j
            positions[starts[r] + j] = p
            slots[starts[r] + j] = int(bt[r, p // BLOCK]) * BLOCK + p % BLOCK
    return dict(k_cache=_bf16(k), v_cache=_bf16(v), block_table=torch.from_numpy(bt),
                seq_lens=torch.from_numpy(lens.astype(np.int32)),
                positions=torch.from_numpy(positions), slot_mapping=torch.from_numpy(slots),
                num_blocks=nb, max_blocks=max_blocks, max_seq_len=int(lens.max()),
                window=int(w.window),
                query_start=torch.from_numpy(starts) if w.q_lens else None)


def make_layer_weights(w: Workload, seed, tag=""):
    """One layer's weights: dense bf16 projections, fp32 gains, block-scaled FP4 experts.

    Dense weights ~ N(0, 1/fan_in), rounded to bf16.  Gains ~ 1 + N(0, 0.1).  Expert
    codes are uniform over the 16 E2M1 values (uniform bytes carry two independent
    uniform nibbles, the low one first); block scales are |N(0, 0.05)| rounded to
    E4M3FN; per-matrix fp32 scales are 1.
    """
    H, E, I = w.hidden, w.n_experts, w.inter
    hq_d = w.n_q_heads * w.head_dim
    out = {}
    for g in ("g_post_prev", "g_pre_attn", "g_post_attn", "g_pre_ffn", "g_post_ffn"):
        out[g] = torch.from_numpy(1.0 + _normal(seed, tag + g, (H,), 0.1))
    out["w_qkv"] = _bf16(_normal(seed, tag + "w_qkv", (w.qkv_rows, H), H ** -0.5))
    out["w_o"] = _bf16(_normal(seed, tag + "w_o", (H, hq_d), hq_d ** -0.5))
    out["w_router"] = _bf16(_normal(seed, tag + "w_router", (E, H), H ** -0.5))
    r = rng_for(seed, tag + "w13_codes")
    out["w13_codes"] = torch.from_numpy(r.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8))
    out["w13_scales"] = _e4m3_codes(np.abs(_normal(seed, tag + "w13_scales", (E, 2 * I, H // 16), 0.05)))
    out["w13_gscale"] = torch.ones(E, dtype=torch.float32)
    r = rng_for(seed, tag + "w2_codes")
    out["w2_codes"] = torch.from_numpy(r.integers(0, 256, (E, H, I // 2), dtype=np.uint8))
    out["w2_scales"] = _e4m3_codes(np.abs(_normal(seed, tag + "w2_scales", (E, H, I // 16), 0.05)))
    out["w2_gscale"] = torch.ones(E, dtype=torch.float32)
    if w.dense_inter:
        Id = w.dense_inter
        out["w_gate_up"] = _bf16(_normal(seed, tag + "w_gate_up", (2 * Id, H), H ** -0.5))
        out["w_down"] = _bf16(_normal(seed, tag + "w_down", (H, Id), Id ** -0.5))
    return out


def make_context(w: Workload, seed, layers):
    """Context rows for the context-K/V store: hidden taps ~ N(0,1) bf16 [n_ctx, H], the
    hidden-norm gain, and per layer the slots of the request's last n_ctx context
    positions before its verify rows (their prefilled K/V are overwritten)."""
    H, n = w.hidden, w.n_ctx
    L0 = int(layers[0]["seq_lens"][0])
    pos = np.arange(L0 - w.q_rows - n, L0 - w.q_rows, dtype=np.int32)
    slots = []
    for lay in layers:
        bt = lay["block_table"].numpy()
        slots.append(torch.from_numpy(np.array([int(bt[0, p // BLOCK]) * BLOCK + p % BLOCK
                                                for p in pos], dtype=np.int64)))
    return dict(states=_bf16(_normal(seed, "context_states", (n, H))),
                g_hidden=torch.from_numpy(1.0 + _normal(seed, "g_hidden", (H,), 0.1)),
                positions=torch.from_numpy(pos), slot_mappings=slots)


def make_activations(w: Workload, seed):
    b, H = w.b, w.hidden
    out = dict(stream=torch.from_numpy(_normal(seed, "stream", (b, H))),
               branch_in=_bf16(_normal(seed, "branch_in", (b, H))),
               front_embed=_bf16(_normal(seed, "front_embed", (b, H))))
    if w.skew_rows > 0:
        bias = np.zeros((b, w.n_experts), dtype=np.float32)
        rows = rng_for(seed, "skew_rows").choice(b, int(round(w.skew_rows * b)), replace=False)
        bias[rows, 0] = w.skew_bias
        out["logit_bias"] = torch.from_numpy(bias)
        out["skew_rows"] = np.sort(rows)
    else:
        out["logit_bias"] = None
    return out


def make_head(w: Workload, seed):
    """Draft head: lm_head bf16 [Vd, H] ~ N(0, 1/H), g_final ~ 1 + N(0, 0.1), and a d2t
    map of Vd distinct target ids drawn from [0, target_vocab).  The output multiplier is
    not computed here: the head's config (base_width, mult_mode) is passed on."""
    H, V = w.hidden, w.draft_vocab
    d2t = rng_for(seed, "d2t").choice(w.target_vocab, V, replace=False).astype(np.int64)
    return dict(w_lm=_bf16(_normal(seed, "w_lm", (V, H), H ** -0.5)),
                g_final=torch.from_numpy(1.0 + _normal(seed, "g_final", (H,), 0.1)),
                d2t=torch.from_numpy(d2t),
                base_width=int(w.base_width), mult_mode=w.mult_mode, soft_cap=float(w.soft_cap))


def make_workload(name_or_w, seed=None):
    """All inputs of a workload.  Returns dict(workload, dims, act, layers=[...], head).

    Each layer dict holds its weights and its own KV pool and step metadata.  In a
    chain, layer i's incoming-branch gain g_post_prev is layer i-1's g_post_ffn.
    """
    w = WORKLOADS[name_or_w] if isinstance(name_or_w, str) else name_or_w
    seed = w.seed if seed is None else seed
    layers = []
    for i in range(w.n_layers):
        tag = "" if w.n_layers == 1 else f"L{i}."
        lay = make_layer_weights(w, seed, tag)
        lay.update(make_kv(w, seed, tag))
        if i > 0:
            lay["g_post_prev"] = layers[i - 1]["g_post_ffn"]
        layers.append(lay)
    return dict(workload=w, dims=w.dims(), act=make_activations(w, seed), layers=layers,
                head=make_head(w, seed) if w.draft_vocab else None,
                context=make_context(w, seed, layers) if w.n_ctx else None)


def with_overrides(w: Workload, **kw):
    return replace(w, **kw)
