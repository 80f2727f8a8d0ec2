"""Device-side plumbing around the C ABI: upload a generated workload, allocate the
step's outputs and workspace, and call the entry points.  PyTorch is used here for device
memory and streams only; every step of the computation is a library call."""

import torch

from . import binding as B

LAYER_TENSORS = ("g_post_prev", "g_pre_attn", "g_post_attn", "g_pre_ffn", "g_post_ffn", "w_qkv",
                 "w_o", "w_router", "w13_codes", "w13_scales", "w13_gscale", "w2_codes",
                 "w2_scales", "w2_gscale", "k_cache", "v_cache", "block_table", "seq_lens",
                 "positions", "slot_mapping")


def to_dev(t, device):
    return None if t is None else t.to(device).contiguous()


DENSE_TENSORS = ("w_gate_up", "w_down")  # a dense (draft) layer's feed-forward, when present


def pack_layer(t):
    """Replace the row-major weights of a device layer dict by their packed copies."""
    for k in ("w_qkv", "w_o", "w_router") + DENSE_TENSORS:
        if t.get(k) is not None:
            t[k] = B.pack_dense(t[k])
    t["w13_codes"], t["w13_scales"] = B.pack_fp4(t["w13_codes"], t["w13_scales"])
    t["w2_codes"], t["w2_scales"] = B.pack_fp4(t["w2_codes"], t["w2_scales"])


class DeviceLayer:
    """One layer's weights (packed), KV pool and step metadata on the device, with its C
    structs."""

    def __init__(self, lay, device):
        self.t = {k: to_dev(lay[k], device) for k in LAYER_TENSORS}
        for k in DENSE_TENSORS:
            if lay.get(k) is not None:
                self.t[k] = to_dev(lay[k], device)
        pack_layer(self.t)
        for k in ("num_blocks", "max_blocks", "max_seq_len"):
            self.t[k] = lay[k]
        self.t["window"] = int(lay.get("window", 0))
        self.t["query_start"] = to_dev(lay.get("query_start"), device)  # partial drafts
        self.weights = B.make_layer_weights(self.t)
        self.kv = B.make_kv(self.t)
        self.attn_w = self.weights.attn
        self.moe_w = self.weights.moe
        self.dense_w = B.make_dense_layer_weights(self.t) if "w_down" in self.t else None


def alloc_route(b, k, E, device):
    i32 = dict(dtype=torch.int32, device=device)
    r = dict(topk_ids=torch.empty(b, k, **i32), topk_w=torch.empty(b, k, dtype=torch.float32, device=device),
             expert_counts=torch.empty(E, **i32), expert_offsets=torch.empty(E + 1, **i32),
             slot_of=torch.empty(b, k, **i32), token_of_slot=torch.empty(b * k, **i32),
             active_experts=torch.empty(E + 1, **i32),
             logits=torch.empty(b, E, dtype=torch.float32, device=device))
    return r, B.make_route(r)


def head_multiplier(hidden, base_width, mode):
    """The draft head's output multiplier from its config (page
    "vllm.models.muse_spark.common.dspark", MuseSparkDSparkForCausalLM.__init__): the width
    multiplier is hidden / base_width; the "mup" rule takes its reciprocal, "sp" its
    reciprocal square root.  A config constant handed to sd_draft_head."""
    width_mult = hidden / base_width
    if mode == "mup":
        return float(width_mult ** -1)
    if mode == "sp":
        return float(width_mult ** -0.5)
    raise ValueError(f"unknown output multiplier rule {mode!r}")


class StepRunner:
    """A whole workload (activations, layers, head) resident on one device."""

    def __init__(self, wk, device="cuda:0", head_mult=None):
        """head_mult: the draft head's output multiplier (None: from the head's config)."""
        self.device = torch.device(device)
        self.w = wk["workload"]
        self.d = wk["dims"]
        self.dims = B.make_dims(self.d)
        self.b = self.w.b
        self.act = {k: to_dev(v, device) for k, v in wk["act"].items()
                    if isinstance(v, torch.Tensor)}
        self.act["logit_bias"] = to_dev(wk["act"].get("logit_bias"), device)
        # the branches between blocks are fp32 at the boundary (values of the bf16 draw)
        self.act["branch_in"] = self.act["branch_in"].float()
        self.layers = [DeviceLayer(l, device) for l in wk["layers"]]
        max_seq = max(l.t["max_seq_len"] for l in self.layers)
        self.ws_bytes = B.workspace_bytes(self.dims, self.b, self.w.n_req, max_seq)
        if self.ws_bytes == 0:
            raise B.SdError(-1, B.lib().sd_last_error().decode())
        if self.w.dense_inter:
            self.ws_bytes = max(self.ws_bytes, B.dense_workspace_bytes(
                self.dims, self.b, self.w.n_req, max_seq, self.w.dense_inter))
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.route_t, self.route = alloc_route(self.b, self.d["top_k"], self.d["n_experts"], device)
        H = self.d["hidden"]
        self.branch_out = torch.empty(self.b, H, dtype=torch.float32, device=device)
        self.ctx = None
        if wk.get("context") is not None:
            c = wk["context"]
            self.ctx = dict(states=to_dev(c["states"], device), g_hidden=to_dev(c["g_hidden"], device),
                            positions=to_dev(c["positions"], device),
                            slots=[to_dev(sm, device) for sm in c["slot_mappings"]])
            self.ctx["layers"] = B.make_ctx_layers([l.t for l in self.layers], self.ctx["slots"])
            n = int(c["states"].shape[0])
            self.ctx["ws"] = torch.empty(B.context_kv_workspace_bytes(self.dims, n, len(self.layers)),
                                         dtype=torch.uint8, device=device)
        self.head = None
        if wk.get("head") is not None:
            h = wk["head"]
            mult = (head_multiplier(self.d["hidden"], h["base_width"], h["mult_mode"])
                    if head_mult is None else float(head_mult))
            self.head = dict(w_lm=B.pack_dense(to_dev(h["w_lm"], device)), g_final=to_dev(h["g_final"], device),
                             d2t=to_dev(h["d2t"], device), multiplier=mult,
                             soft_cap=h["soft_cap"])
            V = h["w_lm"].shape[0]
            self.head_ws = torch.empty(B.draft_head_workspace_bytes(H, V, self.b),
                                       dtype=torch.uint8, device=device)
            self.head_h = torch.empty(self.b, H, dtype=torch.bfloat16, device=device)
            self.draft_ids = torch.empty(self.b, dtype=torch.int32, device=device)
            self.target_ids = torch.empty(self.b, dtype=torch.int64, device=device)
            self.tau = torch.empty(self.b, V, dtype=torch.float32, device=device)

    def layer_step(self, i, stream_buf, branch_in, front_embed=None, branch_out=None,
                   with_route=True, stream=None, aux=None):
        L = self.layers[i]
        out = self.branch_out if branch_out is None else branch_out
        B.layer_step(self.dims, self.b, stream_buf, branch_in, front_embed, L.weights, L.kv,
                     self.act["logit_bias"], out, self.route if with_route else None, self.ws,
                     stream, aux=aux)
        return out

    def pooled_buf(self):
        """A pooled MoE branch: y_slots fp32 [b * k, H] (zeros) and its own routing maps."""
        k, H = self.d["top_k"], self.d["hidden"]
        y = torch.zeros(self.b * k, H, dtype=torch.float32, device=self.device)
        route_t, route = alloc_route(self.b, k, self.d["n_experts"], self.device)
        for t in route_t.values():  # a valid (all-zero) branch until a step writes it
            t.zero_()
        return dict(y=y, route_t=route_t, route=route, p=B.make_pooled(y, route))

    def layer_step_pooled(self, i, stream_buf, pooled_in, pooled_out, front_embed=None,
                          stream=None):
        """Layer i in pooled form: gathers pooled_in (None: the front) in its input boundary
        and leaves its own experts' output in pooled_out (no unpooler)."""
        L = self.layers[i]
        B.layer_step_pooled(self.dims, self.b, stream_buf,
                            None if pooled_in is None else pooled_in["p"], front_embed,
                            L.weights, L.kv, self.act["logit_bias"], pooled_out["p"], self.ws,
                            stream)
        return pooled_out

    def dense_step(self, i, stream_buf, stream=None):
        """Layer i as a dense draft layer on stream_buf (in place)."""
        L = self.layers[i]
        B.dense_layer_step(self.dims, self.b, stream_buf, L.dense_w, L.kv, self.ws, stream)

    def context_kv(self, stream=None):
        """The context-K/V store of every layer for the workload's context rows."""
        c = self.ctx
        B.context_kv(self.dims, int(c["states"].shape[0]), c["states"], c["g_hidden"],
                     c["layers"], c["positions"], c["ws"], stream)

    def chain(self, stream_buf, branch_in, branch_bufs, with_tau=True, stream=None,
              aux_bufs=None):
        """All layers through their input boundaries, the final boundary and the head.
        branch_bufs: one fp32 [b, H] buffer per layer for the layer outputs.  aux_bufs
        (optional): one fp32 [b, H] buffer per layer for its aux tap, then one for the final
        boundary's."""
        u = branch_in
        for i in range(len(self.layers)):
            u = self.layer_step(i, stream_buf, u, branch_out=branch_bufs[i], stream=stream,
                                aux=None if aux_bufs is None else aux_bufs[i])
        hd = self.head
        B.boundary_dualnorm(self.dims, self.b, stream_buf, u, None,
                            self.layers[-1].t["g_post_ffn"], hd["g_final"], self.head_h, stream,
                            aux=None if aux_bufs is None else aux_bufs[-1])
        V = hd["w_lm"].shape[0]
        B.draft_head(self.d["hidden"], V, self.b, self.head_h, hd["w_lm"], hd["multiplier"],
                     hd["soft_cap"], hd["d2t"], self.tau if with_tau else None, self.draft_ids,
                     self.target_ids, self.head_ws, stream)
        return self.draft_ids, self.target_ids
