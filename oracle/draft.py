"""fp64 definition of the draft side: the dense decoder layer and the context-K/V store.

Test infrastructure: see the package docstring for who may import this.

Sources, by page title and section:
  [DSP] "vllm.models.muse_spark.common.dspark": ``MuseSparkDSparkDecoderLayer.forward``
        (the dense layer's order and its bf16 casts), ``MuseSparkDSparkForCausalLM``
        (``hf_to_vllm_mapper``: gate_proj and up_proj stacked as shards 0 and 1 of
        gate_up_proj), ``MuseSparkDSparkModel._project_muse_context_kv`` and
        ``precompute_and_store_context_kv`` (the context-K/V store).

Readings (where the pages are silent):
  - The feed-forward is the stacked gate/up projection, silu(gate) * up, then down_proj:
    the mapper stacks gate_proj (shard 0) and up_proj (shard 1); the activation between
    them is not printed and is read as SiLU-and-multiply, as in the routed experts.
  - The residual adds are plain sums (the gated residual's constants are not printed).
  - The only 16-bit roundings are the ones the forward spells out: the stream is cast to
    the compute dtype (bf16) before each trained input norm, and those norms return bf16.
    Branches, the SwiGLU output and the stream stay at full precision.
"""

import numpy as np

from .formats import bf16_round
from .layer import (gate_oproj, head_rmsnorm, kv_write, paged_attention, qkv_front, rmsnorm,
                    rope)


def dense_ffn(x, w_gate_up, w_down, inter):
    """Dense SwiGLU feed-forward: [g | u] = x W_gu^T (gate rows first), h = silu(g) * u,
    y = h W_down^T.  x: [b, H]; w_gate_up: [2 inter, H]; w_down: [H, inter].
    Returns (h, y) in fp64."""
    x = np.asarray(x, dtype=np.float64)
    gu = x @ np.asarray(w_gate_up, dtype=np.float64).T
    g, u = gu[:, :inter], gu[:, inter:]
    h = g / (1.0 + np.exp(-g)) * u
    y = h @ np.asarray(w_down, dtype=np.float64).T
    return h, y


def dense_layer_step(inp, dims):
    """One dense draft layer on the fp32 stream, in the order of [DSP]
    ``MuseSparkDSparkDecoderLayer.forward``:

      x_a = bf16(RMSNorm(bf16(stream); g_pre_attn))      pre-QKV norm, bf16 in and out
      a   = attention(x_a)                               QKV front, paged attention, gate, o_proj
      stream += RMSNorm(a; g_post_attn)
      x_f = bf16(RMSNorm(bf16(stream); g_pre_ffn))       pre-FFN norm on the bf16 stream
      y   = dense_ffn(x_f)
      stream += RMSNorm(y; g_post_ffn)

    ``inp`` holds the layer's gains, attention weights, w_gate_up, w_down, KV and step
    metadata, and the stream.  ``dims`` as for ``layer_step`` plus ``dense_inter``.
    Returns a dict with the new stream, the caches and the intermediates."""
    d = dims
    eps = d["eps"]
    s = np.asarray(inp["stream"], dtype=np.float64)
    x_a = bf16_round(rmsnorm(bf16_round(s), inp["g_pre_attn"], eps))
    q, k, v, gate = qkv_front(x_a, inp["w_qkv"], inp["positions"], d["n_q_heads"],
                              d["n_kv_heads"], d["head_dim"], eps, d["rope_theta"],
                              bool(d.get("qk_norm", True)))
    kc, vc = kv_write(inp["k_cache"], inp["v_cache"], k, v, inp["slot_mapping"])
    o = paged_attention(q, kc, vc, inp["block_table"], inp["positions"], d["q_rows"],
                        window=int(inp.get("window", 0)), query_start=inp.get("query_start"))
    a = gate_oproj(o, gate, inp["w_o"])
    s = s + rmsnorm(a, inp["g_post_attn"], eps)
    s_mid = s
    x_f = bf16_round(rmsnorm(bf16_round(s), inp["g_pre_ffn"], eps))
    h, y = dense_ffn(x_f, inp["w_gate_up"], inp["w_down"], d["dense_inter"])
    s = s + rmsnorm(y, inp["g_post_ffn"], eps)
    return dict(x_a=x_a, q=q, k=k, v=v, gate=gate, k_cache=kc, v_cache=vc, o=o, a=a,
                stream_mid=s_mid, x_f=x_f, h=h, y=y, stream=s)


def context_rows(context_states, g_hidden, g_pre, eps):
    """The per-layer inputs of the context K/V product ([DSP] ``_project_muse_context_kv``):
    fc = bf16(RMSNorm(context; g_hidden)), x_l = bf16(RMSNorm(fc; g_pre[l])).
    context_states: [n, H]; g_pre: [L, H].  Returns x [L, n, H] (bf16 values in fp64)."""
    ctx = np.asarray(context_states, dtype=np.float64)
    fc = bf16_round(rmsnorm(ctx, g_hidden, eps))
    return np.stack([bf16_round(rmsnorm(fc, g, eps)) for g in np.asarray(g_pre)])


def context_project(x, w_kv, positions, n_kv_heads, head_dim, eps, theta, qk_norm=True):
    """K/V of the context rows x [L, n, H] ([DSP] ``precompute_and_store_context_kv``):
    kv = bf16(x_l W_kv[l]^T) (stacked k | v rows, one bmm); K through the weightless
    RMSNorm (fp32 arithmetic, cast back to bf16), then RoPE at the context positions,
    bf16; V as the product returns it.  Returns (k, v), each [L, n, Hkv, D]."""
    x = np.asarray(x, dtype=np.float64)
    w_kv = np.asarray(w_kv, dtype=np.float64)
    nl, n = x.shape[0], x.shape[1]
    ks, vs = [], []
    for li in range(nl):
        kv = bf16_round(x[li] @ w_kv[li].T)
        k = kv[:, :n_kv_heads * head_dim].reshape(n, n_kv_heads, head_dim)
        v = kv[:, n_kv_heads * head_dim:].reshape(n, n_kv_heads, head_dim)
        if qk_norm:
            k = bf16_round(head_rmsnorm(k, eps))
        k = bf16_round(rope(k, positions, theta))
        ks.append(k)
        vs.append(v)
    return np.stack(ks), np.stack(vs)


def context_kv(context_states, g_hidden, g_pre, w_kv, positions, n_kv_heads, head_dim, eps,
               theta, qk_norm=True):
    """K/V of context tokens for every draft layer ([DSP] ``_project_muse_context_kv`` and
    ``precompute_and_store_context_kv``): ``context_rows`` then ``context_project``.

    context_states: [n, H]; g_pre: [L, H]; w_kv: [L, 2 Hkv D, H] (k rows then v rows, the
    layer's qkv_proj rows after q).  Returns (k, v), each [L, n, Hkv, D] bf16 values in
    fp64."""
    x = context_rows(context_states, g_hidden, g_pre, eps)
    return context_project(x, w_kv, positions, n_kv_heads, head_dim, eps, theta, qk_norm)


def context_kv_store(k_caches, v_caches, k, v, slot_mappings):
    """Write each layer's context K/V at its slot mapping (negative slots write nothing),
    into copies of the caches; returns the new (k_caches, v_caches) lists."""
    outk, outv = [], []
    for li in range(len(k_caches)):
        kc, vc = kv_write(k_caches[li], v_caches[li], k[li], v[li], slot_mappings[li])
        outk.append(kc)
        outv.append(vc)
    return outk, outv
