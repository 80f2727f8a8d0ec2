"""A second CPU reference of the layer step, composed from torch library calls in fp64.

It shares no code with ``oracle/``: RMSNorm is ``F.rms_norm``, attention is
``F.scaled_dot_product_attention`` on K/V gathered through the block table, routing is
``torch.topk`` + ``torch.softmax``, RoPE is a complex multiplication, FP4/E4M3 decoding
goes through torch's float8 decoder and a lookup table.  It only exists to pin the
oracle (the two must agree to ~1e-10 on the tiny workload).
"""

import torch
import torch.nn.functional as F

D64 = torch.float64
E2M1_LUT = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                         -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=D64)


def t64(x):
    return x.to(D64) if isinstance(x, torch.Tensor) else torch.as_tensor(x, dtype=D64)


def rms(x, g, eps):
    return F.rms_norm(t64(x), (x.shape[-1],), weight=None if g is None else t64(g), eps=eps)


def rope_complex(x, pos, theta):
    d = x.shape[-1]
    half = d // 2
    freq = theta ** (-torch.arange(0, d, 2, dtype=D64) / d)                 # [half]
    rot = torch.polar(torch.ones(len(pos), half, dtype=D64), t64(pos)[:, None] * freq[None])
    z = torch.complex(x[..., :half], x[..., half:]) * rot[:, None, :]
    return torch.cat([z.real, z.imag], dim=-1)


def dequant(codes, scales, gscale):
    c = codes.to(torch.int64)
    lo, hi = c & 0xF, c >> 4
    vals = torch.stack([E2M1_LUT[lo], E2M1_LUT[hi]], dim=-1).reshape(*c.shape[:-1], -1)
    sc = scales.view(torch.float8_e4m3fn).to(D64).repeat_interleave(16, dim=-1)
    return vals * sc * float(gscale)


def bf16(x):
    return t64(x).to(torch.float32).to(torch.bfloat16).to(D64)


def attn_block(lay, x_a, dims):
    """QKV front, cache write, paged attention (causal, or a sliding window), gate, o_proj."""
    eps, theta = dims["eps"], dims["rope_theta"]
    hq, hkv, d, qr = dims["n_q_heads"], dims["n_kv_heads"], dims["head_dim"], dims["q_rows"]
    window = int(lay.get("window", 0))
    b = x_a.shape[0]
    y = t64(x_a) @ t64(lay["w_qkv"]).T
    q, k, v, gate = torch.split(y, [hq * d, hkv * d, hkv * d, hq * d], dim=1)
    q, k, v = q.reshape(b, hq, d), k.reshape(b, hkv, d), v.reshape(b, hkv, d)
    if dims.get("qk_norm", 1):
        q, k = rms(q, None, eps), rms(k, None, eps)
    pos = lay["positions"].to(torch.int64)
    q, k = rope_complex(q, pos, theta), rope_complex(k, pos, theta)
    kc = t64(lay["k_cache"]).clone()                 # [nb, hkv, 16, d]
    vc = t64(lay["v_cache"]).clone().transpose(2, 3)  # -> [nb, hkv, 16, d]
    slots = lay["slot_mapping"].to(torch.int64)
    kc[slots // 16, :, slots % 16, :] = bf16(k)
    vc[slots // 16, :, slots % 16, :] = bf16(v)
    o = torch.empty(b, hq, d, dtype=D64)
    bt = lay["block_table"].to(torch.int64)
    qs = lay.get("query_start")
    starts = list(range(0, b + 1, qr)) if qs is None else [int(v) for v in qs]
    for r in range(len(starts) - 1):
        rows = slice(starts[r], starts[r + 1])
        L = int(pos[starts[r + 1] - 1]) + 1
        tok = torch.arange(L)
        kk = kc[bt[r, tok // 16], :, tok % 16, :].permute(1, 0, 2)   # [hkv, L, d]
        vv = vc[bt[r, tok // 16], :, tok % 16, :].permute(1, 0, 2)
        kk = kk.repeat_interleave(hq // hkv, dim=0)
        vv = vv.repeat_interleave(hq // hkv, dim=0)
        mask = tok[None, :] <= pos[rows][:, None]                    # [qr, L]
        if window > 0:
            mask &= tok[None, :] > pos[rows][:, None] - window
        qq = q[rows].permute(1, 0, 2)                                # [hq, qr, d]
        o[rows] = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask).permute(1, 0, 2)
    a = (o.reshape(b, -1) * torch.sigmoid(gate)) @ t64(lay["w_o"]).T
    return dict(q=q, k=k, v=v, gate=gate, o=o, a=a)


def layer(lay, act, dims, branch_in):
    """The layer step of one workload; returns a dict of the main intermediates."""
    eps = dims["eps"]
    b = act["stream"].shape[0]
    s = t64(act["stream"]) + rms(branch_in, lay["g_post_prev"], eps)
    aux = s
    x_a = rms(s, lay["g_pre_attn"], eps)
    at = attn_block(lay, x_a, dims)
    s = s + rms(at["a"], lay["g_post_attn"], eps)
    x_m = rms(s, lay["g_pre_ffn"], eps)
    z = x_m @ t64(lay["w_router"]).T
    if act.get("logit_bias") is not None:
        z = z + t64(act["logit_bias"])
    top = torch.topk(z, dims["top_k"], dim=1)
    ids, w = top.indices, torch.softmax(top.values, dim=1)
    m = torch.zeros(b, dims["hidden"], dtype=D64)
    inter = dims["inter"]
    for e in torch.unique(ids).tolist():
        w13 = dequant(lay["w13_codes"][e], lay["w13_scales"][e], lay["w13_gscale"][e])
        w2 = dequant(lay["w2_codes"][e], lay["w2_scales"][e], lay["w2_gscale"][e])
        rows, js = (ids == e).nonzero(as_tuple=True)
        gu = x_m[rows] @ w13.T
        h = F.silu(gu[:, :inter]) * gu[:, inter:]
        m[rows] += w[rows, js][:, None] * (h @ w2.T)
    return dict(aux=aux, x_a=x_a, q=at["q"], k=at["k"], v=at["v"], gate=at["gate"], o=at["o"],
                a=at["a"], stream=s, x_m=x_m, z=z, ids=ids, w=w, m=m)


def dense_layer(lay, stream, dims):
    """The draft's dense layer: bf16 stream into each pre-norm, bf16 pre-norm outputs,
    F.silu(gate) * up between the stacked projection and down_proj."""
    eps, Id = dims["eps"], dims["dense_inter"]
    s = t64(stream)
    x_a = bf16(rms(bf16(s), lay["g_pre_attn"], eps))
    at = attn_block(lay, x_a, dims)
    s = s + rms(at["a"], lay["g_post_attn"], eps)
    x_f = bf16(rms(bf16(s), lay["g_pre_ffn"], eps))
    gu = x_f @ t64(lay["w_gate_up"]).T
    h = F.silu(gu[:, :Id]) * gu[:, Id:]
    y = h @ t64(lay["w_down"]).T
    s = s + rms(y, lay["g_post_ffn"], eps)
    return dict(x_a=x_a, a=at["a"], x_f=x_f, h=h, y=y, stream=s)


def context_kv(states, g_hidden, g_pre, w_kv, positions, hkv, d, eps, theta):
    """Context K/V of every layer: hidden norm, per-layer norms, one batched matmul over
    the stacked K/V rows, fp32-style K norm cast back to bf16, complex RoPE."""
    fc = bf16(rms(states, g_hidden, eps))
    per_layer = torch.stack([bf16(rms(fc, g, eps)) for g in t64(g_pre)])      # [L, n, H]
    kv = bf16(torch.bmm(per_layer, t64(w_kv).transpose(1, 2)))                  # [L, n, 2 hkv d]
    nl, n = kv.shape[0], kv.shape[1]
    k = kv[..., :hkv * d].reshape(nl, n, hkv, d)
    v = kv[..., hkv * d:].reshape(nl, n, hkv, d)
    k = bf16(k * torch.rsqrt(k.pow(2).mean(-1, keepdim=True) + eps))
    k = torch.stack([bf16(rope_complex(k[i], positions.to(torch.int64), theta)) for i in range(nl)])
    return k, v
