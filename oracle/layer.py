"""fp64 definition of one decoder layer's speculative-verification step.

Test infrastructure: see the package docstring for who may import this.

Shapes: ``b`` rows = ``n_req`` requests x ``q_rows`` (= 1 + 7) verify tokens, request
major ([DEC] module docstring: one request verifying 1 + 7 tokens; ``decode_metadata``:
the step's token count equals q); with ``query_start`` (partial drafts) request r owns
rows ``query_start[r] .. query_start[r+1] - 1``, 1..q_rows of them.  ``H`` hidden, ``Hq``/``Hkv`` query/KV heads, ``D``
head dim, ``E`` experts, ``k`` top-k, ``I`` expert intermediate size.

Cache layout (the library's boundary layout, read here as is):
K cache ``[num_blocks, Hkv, 16, D]`` (token-major inside a block),
V cache ``[num_blocks, Hkv, D, 16]`` (dim-major inside a block);
token ``p`` of request ``r`` lives in block ``block_table[r, p // 16]`` at offset ``p % 16``
([RT] ``unsupported``: block size 16).
"""

import numpy as np

from .formats import bf16_round, dequant_nvfp4

BLOCK = 16


# --------------------------------------------------------------------------- norms
def rmsnorm(v, g, eps):
    """Row RMSNorm over the last axis: v * (mean(v**2) + eps) ** -1/2 * g.

    The arithmetic is the one [DSP] ``precompute_and_store_context_kv`` spells out for
    its weightless K norm (mean of squares, plus eps, reciprocal square root); the gain
    ``g`` is the effective multiplier of the norm class the layers use.
    """
    v = np.asarray(v, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    out = v * r
    if g is not None:
        out = out * np.asarray(g, dtype=np.float64)
    return out


def front_norm(embed, g_pre, eps):
    """First layer: the embedded tokens become the fp32 stream and its pre-attention
    norm becomes the attention input ([DEC] module docstring, the first layer's front).
    Returns (stream, x)."""
    s = np.asarray(embed, dtype=np.float64).copy()
    return s, rmsnorm(s, g_pre, eps)


def dual_norm(stream, branch, g_post, g_pre, eps):
    """A sandwich-norm boundary: stream <- stream + RMSNorm(branch; g_post), then
    x = RMSNorm(stream; g_pre) feeds the next block.

    Order from [DSP] ``MuseSparkDSparkDecoderLayer.forward`` (post-norm of the branch
    added to the stream, then the next block's pre-norm of the stream) and [DEC] module
    docstring (input boundary, attention boundary and final boundary are each a dual
    norm into the stream and the next input).  The residual add is a plain sum: the
    pages name a gated residual without printing its constants, and this reads them
    as 1.  Returns (new stream, x).
    """
    s = np.asarray(stream, dtype=np.float64) + rmsnorm(branch, g_post, eps)
    return s, rmsnorm(s, g_pre, eps)


# ------------------------------------------------------------------------ QKV front
def qkv_split(y, n_q_heads, n_kv_heads, head_dim):
    """Split the stacked projection output into q | k | v | o_gate, in that order
    ([DSP] ``hf_to_vllm_mapper`` stacks q, k, v, o_gate into qkv_proj; the context
    chain takes K/V at rows [q_size, q_size + 2 * kv_size) of it)."""
    b = y.shape[0]
    qs, ks = n_q_heads * head_dim, n_kv_heads * head_dim
    q = y[:, :qs].reshape(b, n_q_heads, head_dim)
    k = y[:, qs:qs + ks].reshape(b, n_kv_heads, head_dim)
    v = y[:, qs + ks:qs + 2 * ks].reshape(b, n_kv_heads, head_dim)
    gate = y[:, qs + 2 * ks:qs + 2 * ks + qs]
    assert gate.shape[1] == qs
    return q, k, v, gate


def head_rmsnorm(x, eps):
    """Weightless RMSNorm over each head vector (last axis), as [DSP]
    ``precompute_and_store_context_kv`` applies to K before RoPE.  Applying the same
    norm to q is this implementation's reading of the layers' qk_norm."""
    return rmsnorm(x, None, eps)


def rope(x, positions, theta):
    """Rotary embedding, rotate-half form, over the full head dim D.

    For i < D/2 the pair (x_i, x_{i+D/2}) turns by angle p * theta**(-2i/D).
    [DSP] ``precompute_and_store_context_kv`` applies a rotary embedding to K at the
    context positions; the pairing and frequencies are this implementation's reading.
    x: [b, heads, D], positions: [b].  Returns a new array: q and k are rotated
    separately, never through a shared buffer ([DSP] notes that aliasing one tensor
    as both operands rotates it twice).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    freq = theta ** (-2.0 * i / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * freq[None, :]   # [b, half]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def qkv_front(x_a, w_qkv, positions, n_q_heads, n_kv_heads, head_dim, eps, theta,
              qk_norm=True):
    """QKV front of [DEC] module docstring: stacked projection, then q/k preparation.

    y = x_a @ W_qkv^T; q and k get the weightless per-head RMSNorm (if ``qk_norm``)
    and RoPE at their row's position; v and the output gate pass through.
    Returns (q [b,Hq,D], k [b,Hkv,D], v [b,Hkv,D], gate [b,Hq*D]) in fp64.
    """
    y = np.asarray(x_a, dtype=np.float64) @ np.asarray(w_qkv, dtype=np.float64).T
    q, k, v, gate = qkv_split(y, n_q_heads, n_kv_heads, head_dim)
    if qk_norm:
        q, k = head_rmsnorm(q, eps), head_rmsnorm(k, eps)
    return rope(q, positions, theta), rope(k, positions, theta), v, gate


def kv_write(k_cache, v_cache, k, v, slot_mapping):
    """Write this step's K/V into the paged cache at ``slot_mapping`` (slot =
    block * 16 + offset; the step carries its slot mapping, [DEC] ``plan``).  The cache
    holds bf16 ([RT] ``unsupported``), so values are rounded to bf16 here.
    Returns new fp64 caches (inputs are not modified)."""
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:                   # a negative slot marks a row whose K/V is not stored
            continue
        blk, off = int(slot) // BLOCK, int(slot) % BLOCK
        kc[blk, :, off, :] = bf16_round(k[t])
        vc[blk, :, :, off] = bf16_round(v[t])
    return kc, vc


# ----------------------------------------------------------------------- attention
def gather_request_kv(k_cache, v_cache, block_table_row, length):
    """Contiguous K, V [length, Hkv, D] of one request, read through its block table."""
    t = np.arange(length)
    blocks = np.asarray(block_table_row)[t // BLOCK]
    offs = t % BLOCK
    k = k_cache[blocks, :, offs, :]            # [length, Hkv, D]
    v = v_cache[blocks, :, :, offs]            # [length, Hkv, D]
    return k, v


def request_of_row(t, q_rows, query_start=None):
    """The request that row t belongs to.  Every request verifies q_rows tokens unless
    query_start is given: then request r owns rows query_start[r] .. query_start[r+1] - 1
    (partial drafts: requests verifying fewer tokens, which [DEC] ``plan`` hands to the
    stock forward and this library serves)."""
    if query_start is None:
        return t // q_rows
    for r in range(len(query_start) - 1):
        if query_start[r] <= t < query_start[r + 1]:
            return r
    raise ValueError(f"row {t} lies in no request of {list(query_start)}")


def paged_attention(q, k_cache, v_cache, block_table, positions, q_rows, scale=None, window=0,
                    query_start=None):
    """Causal GQA attention of each verify row over its request's paged KV.

    Row t belongs to request r (``request_of_row``) and sits at position p = positions[t];
    it attends to tokens 0..p of that request (the draft layers are causal, [DSP]
    ``MuseSparkDSparkDecoderLayer.__init__``; attn2 reads the paged cache through the
    block table, [DEC] ``plan``).  With a sliding window w > 0 (attn2 serves each layer's
    sliding window, [DEC] ``plan``; the pages give no size or convention) the row sees only
    the w most recent positions, max(0, p - w + 1)..p.  Query head h uses KV head
    h // (Hq / Hkv).  softmax(scale * q . K^T) . V with scale = D**-1/2 unless given.
    q: [b, Hq, D] -> o [b, Hq, D], fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    b, hq, d = q.shape
    hkv = k_cache.shape[1]
    group = hq // hkv
    if scale is None:
        scale = d ** -0.5
    o = np.zeros_like(q)
    for t in range(b):
        r, p = request_of_row(t, q_rows, query_start), int(positions[t])
        lo = max(0, p - window + 1) if window > 0 else 0
        k, v = gather_request_kv(k_cache, v_cache, block_table[r], p + 1)
        k, v = k[lo:], v[lo:]
        for h in range(hq):
            g = h // group
            sc = scale * (k[:, g, :] @ q[t, h])
            sc = sc - sc.max()
            a = np.exp(sc)
            a /= a.sum()
            o[t, h] = a @ v[:, g, :]
    return o


def gate_oproj(o, gate, w_o):
    """Output gate then o_proj: a = (o * sigmoid(gate)) @ W_o^T.

    The stacked projection's last shard is the output gate ([DSP] ``hf_to_vllm_mapper``:
    o_gate_proj stacked into qkv_proj); using it as an elementwise sigmoid gate on the
    attention output before o_proj is this implementation's reading.  o: [b, Hq, D] or
    [b, Hq*D]; gate: [b, Hq*D].
    """
    b = gate.shape[0]
    with np.errstate(over="ignore"):          # exp(-gate) -> inf gives the exact limit 0
        sig = 1.0 / (1.0 + np.exp(-np.asarray(gate, np.float64)))
    og = np.asarray(o, dtype=np.float64).reshape(b, -1) * sig
    return og @ np.asarray(w_o, dtype=np.float64).T


# ------------------------------------------------------------------------- routing
def router_logits(x_m, w_router, logit_bias=None):
    """Router logits z = x_m @ W_r^T (+ bias), W_r stored [E, H] ([DEC] module docstring:
    router -> routing -> pooler)."""
    z = np.asarray(x_m, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T
    if logit_bias is not None:
        z = z + np.asarray(logit_bias, dtype=np.float64)
    return z


def topk_route(z, k):
    """Top-k experts per row and their weights.

    ids: the k experts with the largest logits, ordered by (-z, expert index), so ties
    go to the lower index; w = softmax over the k selected logits (a softmax renormalised
    over the selection).  Routing follows the router in [DEC] module docstring; the tie
    rule and renormalisation are this implementation's stated reading.
    """
    z = np.asarray(z, dtype=np.float64)
    b, e = z.shape
    ids = np.empty((b, k), dtype=np.int32)
    w = np.empty((b, k), dtype=np.float64)
    for t in range(b):
        order = np.lexsort((np.arange(e), -z[t]))   # primary key -z, then index
        ids[t] = order[:k]
        sel = z[t, ids[t]]
        ex = np.exp(sel - sel.max())
        w[t] = ex / ex.sum()
    return ids, w


def pooler(ids, n_experts):
    """Group (row, choice) pairs by expert: a stable counting sort by (expert, row).

    counts[e]      number of pairs routed to e
    offsets[e]     exclusive prefix sum of counts (offsets[E] = b * k)
    slot_of[t, j]  offsets[e] + number of rows t' < t that also chose e (e = ids[t, j])
    token_of_slot  the inverse map, slot -> row
    The pooler groups token rows by expert ([DEC] module docstring and ``build``); the
    exact maps are this implementation's definition.
    """
    ids = np.asarray(ids, dtype=np.int64)
    b, k = ids.shape
    counts = np.zeros(n_experts, dtype=np.int32)
    for t in range(b):
        for j in range(k):
            counts[ids[t, j]] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    slot_of = np.empty((b, k), dtype=np.int32)
    token_of_slot = np.empty(b * k, dtype=np.int32)
    for t in range(b):                 # rows in order: stable within each expert
        for j in range(k):
            e = ids[t, j]
            slot_of[t, j] = fill[e]
            token_of_slot[fill[e]] = t
            fill[e] += 1
    return counts, offsets, slot_of, token_of_slot


# ------------------------------------------------------------------------- experts
def silu(x):
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def expert_ffn(x, w13, w2, inter):
    """SwiGLU expert on dense fp64 weights: g, u = x @ W13[:I]^T, x @ W13[I:]^T;
    h = silu(g) * u; y = h @ W2^T.  Gate rows come first in the stacked W13
    ([DSP] ``hf_to_vllm_mapper``: gate_proj is shard 0 of gate_up_proj, up_proj shard 1).
    Returns (h, y)."""
    x = np.asarray(x, dtype=np.float64)
    g = x @ w13[:inter].T
    u = x @ w13[inter:2 * inter].T
    h = silu(g) * u
    return h, h @ w2.T


def moe_experts(x_m, counts, offsets, token_of_slot, w13_codes, w13_scales, w13_gscale,
                w2_codes, w2_scales, w2_gscale, inter, experts=None):
    """Routed experts over pooled slots: for slot s = (row t, expert e),
    y[s] = SwiGLU_e(x_m[t]) with W13_e, W2_e dequantised exactly from block-scaled FP4.
    Only experts with counts > 0 are dequantised (one at a time, to bound memory).
    ``experts`` optionally restricts the computation to a subset (other slots stay 0).
    Returns (h [b*k, I], y [b*k, H])."""
    x_m = np.asarray(x_m, dtype=np.float64)
    n_slots = int(offsets[-1])
    hidden = x_m.shape[1]
    h = np.zeros((n_slots, inter))
    y = np.zeros((n_slots, hidden))
    for e in range(len(counts)):
        if counts[e] == 0 or (experts is not None and e not in experts):
            continue
        sl = slice(int(offsets[e]), int(offsets[e + 1]))
        w13 = dequant_nvfp4(w13_codes[e], w13_scales[e], w13_gscale[e])
        w2 = dequant_nvfp4(w2_codes[e], w2_scales[e], w2_gscale[e])
        h[sl], y[sl] = expert_ffn(x_m[token_of_slot[sl]], w13, w2, inter)
    return h, y


def unpool(y, w, slot_of):
    """Weighted combine back per row: m[t] = sum over j (in order) of w[t, j] *
    y[slot_of[t, j]] ([DEC] module docstring: the unpooler after the routed experts)."""
    b, k = slot_of.shape
    m = np.zeros((b, y.shape[1]))
    for j in range(k):
        m += np.asarray(w, np.float64)[:, j:j + 1] * y[slot_of[:, j]]
    return m


# ---------------------------------------------------------------------- layer step
def layer_step(inp, dims, branch_in=None, front_embed=None, route_override=None):
    """One layer's verify step, in the order of [DEC] ``SpecializedDecode.run``:
    input boundary (or the first layer's front) -> attention (QKV front, paged
    attention, gated o_proj) -> attention boundary -> MoE (router, routing, pooler,
    experts, unpooler).

    ``inp`` holds the layer's weights, caches and step metadata as arrays (fp64 values
    of the bf16/fp32 inputs, raw codes for FP4/E4M3).  ``dims`` is a mapping with
    hidden, n_q_heads, n_kv_heads, head_dim, q_rows, n_experts, top_k, inter, eps,
    rope_theta, qk_norm.  ``route_override`` (ids, or a function (z, ids) -> ids)
    replaces this step's own top-k, for teacher forcing at near ties; the weights are
    then the softmax over the replaced selection.
    Returns a dict with the new stream, the branch output m, the updated caches and
    every intermediate.  ``aux`` is the layer's aux hidden-state tap: the stream its
    input boundary (or front) hands on, after the residual add and before the pre-norm.
    [DEC] ``SpecializedDecode.run`` passes the layer's fp32 aux buffer to that boundary,
    which writes it for the drafter (``DecodeLayer.aux``: the drafter's input); which
    value is tapped is not printed, and this reads it as the stream entering the layer.
    """
    d = dims
    eps = d["eps"]
    if front_embed is not None:
        s, x_a = front_norm(front_embed, inp["g_pre_attn"], eps)
    else:
        s, x_a = dual_norm(inp["stream"], branch_in, inp["g_post_prev"], inp["g_pre_attn"], eps)
    s_after_in = s
    q, k, v, gate = qkv_front(x_a, inp["w_qkv"], inp["positions"], d["n_q_heads"],
                              d["n_kv_heads"], d["head_dim"], eps, d["rope_theta"],
                              bool(d.get("qk_norm", True)))
    kc, vc = kv_write(inp["k_cache"], inp["v_cache"], k, v, inp["slot_mapping"])
    o = paged_attention(q, kc, vc, inp["block_table"], inp["positions"], d["q_rows"],
                        window=int(inp.get("window", 0)), query_start=inp.get("query_start"))
    a = gate_oproj(o, gate, inp["w_o"])
    s, x_m = dual_norm(s, a, inp["g_post_attn"], inp["g_pre_ffn"], eps)
    z = router_logits(x_m, inp["w_router"], inp.get("logit_bias"))
    ids, w = topk_route(z, d["top_k"])
    if route_override is not None:
        ids = route_override(z, ids) if callable(route_override) else route_override
        ids = np.asarray(ids, dtype=np.int32)
        sel = np.take_along_axis(z, ids.astype(np.int64), axis=1)
        ex = np.exp(sel - sel.max(axis=1, keepdims=True))
        w = ex / ex.sum(axis=1, keepdims=True)
    counts, offsets, slot_of, token_of_slot = pooler(ids, d["n_experts"])
    h, y = moe_experts(x_m, counts, offsets, token_of_slot,
                       inp["w13_codes"], inp["w13_scales"], inp["w13_gscale"],
                       inp["w2_codes"], inp["w2_scales"], inp["w2_gscale"], d["inter"])
    m = unpool(y, w, slot_of)
    return dict(stream_in=s_after_in, aux=s_after_in, x_a=x_a, q=q, k=k, v=v, gate=gate, k_cache=kc,
                v_cache=vc, o=o, a=a, stream=s, x_m=x_m, z=z, ids=ids, w=w, counts=counts,
                offsets=offsets, slot_of=slot_of, token_of_slot=token_of_slot, h=h, y=y,
                m=m)
