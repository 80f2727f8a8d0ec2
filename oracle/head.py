"""fp64 definition of the final boundary, the draft head and a chain of layer steps.

Test infrastructure: see the package docstring for who may import this.
"""

import numpy as np

from .formats import bf16_round
from .layer import dual_norm, layer_step


def final_boundary(stream, branch, g_post, g_final, eps):
    """The last gather + dual norm into the model's final norm ([DEC] module docstring,
    ``final``).  Returns (new stream, h) with h in fp64 (not yet cast).  The new stream is
    also the final boundary's aux tap ([DEC] ``SpecializedDecode.run``: the final boundary
    writes the last aux buffer), read like a layer's tap as the stream after the add."""
    return dual_norm(stream, branch, g_post, g_final, eps)


def output_multiplier(hidden, base_width, mode):
    """Output multiplier of the draft head ([DSP] ``MuseSparkDSparkForCausalLM.__init__``):
    width_mult = hidden / base_width; 'mup' -> width_mult**-1, 'sp' -> width_mult**-0.5."""
    width_mult = hidden / base_width
    if mode == "mup":
        return width_mult ** -1
    if mode == "sp":
        return width_mult ** -0.5
    raise ValueError(mode)


def draft_head(h, w_lm, multiplier, soft_cap, d2t):
    """Draft head on the final hidden rows.

    * the hidden is cast to the head's dtype, bf16 ([DSP] ``compute_draft_logits``);
    * logits are produced in bf16 ([RT] ``unsupported``: BF16 draft logits), so the exact
      product is rounded to bf16 once;
    * transform ([DSP] ``apply_output_logit_transform``): x = logits * multiplier, then
      soft_cap * tanh(x / soft_cap) when a cap is set;
    * id = the lowest index of the largest transformed logit (argmax with ties to the
      lower index, the stated tie rule);
    * target id = d2t[id] ([DSP] ``draft_id_to_target_id``, an int64 map of draft
      vocabulary size, read as absolute target ids).
    Returns dict(logits_bf16, tau, ids, target_ids).
    """
    hb = bf16_round(np.asarray(h, dtype=np.float64))
    logits = bf16_round(hb @ np.asarray(w_lm, dtype=np.float64).T)
    x = logits * multiplier
    tau = soft_cap * np.tanh(x / soft_cap) if soft_cap is not None and soft_cap > 0 else x
    ids = np.argmax(tau, axis=1).astype(np.int32)      # first occurrence of the max
    return dict(h_bf16=hb, logits=logits, tau=tau, ids=ids,
                target_ids=np.asarray(d2t, dtype=np.int64)[ids])


def chain_step(layers, dims, stream, branch_in, g_final, w_lm, multiplier, soft_cap, d2t,
               route_overrides=None, on_layer=None):
    """Several layers of [DEC] ``SpecializedDecode.run`` chained through their input
    boundaries, then the final boundary and the draft head.

    ``layers`` is a list of per-layer input dicts (weights, caches, step metadata; the
    stream comes from ``stream``).  The first layer takes ``branch_in`` through its
    input boundary, each later layer the previous layer's unpooled branch.
    Returns dict(layers=[per-layer outputs], stream, h, head=draft_head(...), aux=[each
    layer's aux tap, then the final boundary's]).
    """
    outs = []
    s, u = np.asarray(stream, dtype=np.float64), branch_in
    for i, inp in enumerate(layers):
        li = dict(inp)
        li["stream"] = s
        ro = None if route_overrides is None else route_overrides[i]
        out = layer_step(li, dims, branch_in=u, route_override=ro)
        outs.append(out)
        if on_layer is not None:          # progress report only
            on_layer(i)
        s, u = out["stream"], out["m"]
    s, h = final_boundary(s, u, layers[-1]["g_post_ffn"], g_final, dims["eps"])
    return dict(layers=outs, stream=s, h=h, aux=[o["aux"] for o in outs] + [s],
                head=draft_head(h, w_lm, multiplier, soft_cap, d2t))
