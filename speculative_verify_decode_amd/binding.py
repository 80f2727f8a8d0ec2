"""ctypes binding of libsdverify.so: the same entry points as include/sdverify.h.

Argument marshalling only: tensors become device pointers, dims become the C struct, a
nonzero return code becomes a RuntimeError carrying sd_last_error().  Every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the library is
missing, loading raises.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsdverify.so")

c_int, c_float, c_size_t, c_void_p = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class SdDims(ctypes.Structure):
    _fields_ = [(n, c_int) for n in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "q_rows",
                                     "block_size", "n_experts", "top_k", "inter", "qk_norm")] + \
               [(n, c_float) for n in ("eps", "rope_theta", "attn_scale")]


class SdAttnWeights(ctypes.Structure):
    _fields_ = [("w_qkv", c_void_p), ("w_o", c_void_p)]


class SdMoeWeights(ctypes.Structure):
    _fields_ = [("w_router", c_void_p), ("w13_codes", c_void_p), ("w13_scales", c_void_p),
                ("w13_gscale", c_void_p), ("w2_codes", c_void_p), ("w2_scales", c_void_p),
                ("w2_gscale", c_void_p)]


class SdLayerWeights(ctypes.Structure):
    _fields_ = [("g_post_prev", c_void_p), ("g_pre_attn", c_void_p), ("g_post_attn", c_void_p),
                ("g_pre_ffn", c_void_p), ("attn", SdAttnWeights), ("moe", SdMoeWeights)]


class SdKv(ctypes.Structure):
    _fields_ = [("k_cache", c_void_p), ("v_cache", c_void_p), ("num_blocks", c_int),
                ("block_table", c_void_p), ("max_blocks", c_int), ("seq_lens", c_void_p),
                ("positions", c_void_p), ("slot_mapping", c_void_p), ("n_req", c_int),
                ("max_seq_len", c_int), ("window", c_int), ("query_start", c_void_p)]


ROUTE_FIELDS = ("topk_ids", "topk_w", "expert_counts", "expert_offsets", "slot_of",
                "token_of_slot", "active_experts", "logits")


class SdRoute(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ROUTE_FIELDS]


class SdDenseLayerWeights(ctypes.Structure):
    _fields_ = [("g_pre_attn", c_void_p), ("g_post_attn", c_void_p), ("g_pre_ffn", c_void_p),
                ("g_post_ffn", c_void_p), ("attn", SdAttnWeights), ("w_gate_up", c_void_p),
                ("w_down", c_void_p), ("inter", c_int)]


class SdCtxLayer(ctypes.Structure):
    _fields_ = [("g_pre_attn", c_void_p), ("w_qkv", c_void_p), ("k_cache", c_void_p),
                ("v_cache", c_void_p), ("num_blocks", c_int), ("slot_mapping", c_void_p)]


class SdPooled(ctypes.Structure):
    _fields_ = [("y_slots", c_void_p), ("route", ctypes.POINTER(SdRoute))]


SYMBOLS = {
    "sd_abi_version": (c_int, []),
    "sd_last_error": (ctypes.c_char_p, []),
    "sd_packed_dense_bytes": (c_size_t, [c_int, c_int]),
    "sd_pack_dense": (c_int, [c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "sd_pack_fp4": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_void_p]),
    "sd_workspace_bytes": (c_size_t, [ctypes.POINTER(SdDims), c_int, c_int, c_int]),
    "sd_boundary_dualnorm": (c_int, [ctypes.POINTER(SdDims), c_int, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p]),
    "sd_attn_verify": (c_int, [ctypes.POINTER(SdDims), c_int, c_void_p,
                               ctypes.POINTER(SdAttnWeights), ctypes.POINTER(SdKv), c_void_p,
                               c_void_p, c_size_t, c_void_p]),
    "sd_moe_route": (c_int, [ctypes.POINTER(SdDims), c_int, c_void_p, c_void_p, c_void_p,
                             ctypes.POINTER(SdRoute), c_void_p, c_size_t, c_void_p]),
    "sd_moe_experts": (c_int, [ctypes.POINTER(SdDims), c_int, c_void_p,
                               ctypes.POINTER(SdMoeWeights), ctypes.POINTER(SdRoute), c_void_p,
                               c_void_p, c_void_p, c_size_t, c_void_p]),
    "sd_moe_experts_x16": (c_int, [ctypes.POINTER(SdDims), c_int, c_void_p,
                                   ctypes.POINTER(SdMoeWeights), ctypes.POINTER(SdRoute),
                                   c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "sd_moe_unpool": (c_int, [ctypes.POINTER(SdDims), c_int, c_void_p, ctypes.POINTER(SdRoute),
                              c_void_p, c_void_p]),
    "sd_layer_step": (c_int, [ctypes.POINTER(SdDims), c_int, c_void_p, c_void_p, c_void_p,
                              ctypes.POINTER(SdLayerWeights), ctypes.POINTER(SdKv), c_void_p,
                              c_void_p, ctypes.POINTER(SdRoute), c_void_p, c_void_p, c_size_t,
                              c_void_p]),
    "sd_layer_step_pooled": (c_int, [ctypes.POINTER(SdDims), c_int, c_void_p,
                                     ctypes.POINTER(SdPooled), c_void_p,
                                     ctypes.POINTER(SdLayerWeights), ctypes.POINTER(SdKv),
                                     c_void_p, ctypes.POINTER(SdPooled), c_void_p, c_void_p,
                                     c_size_t, c_void_p]),
    "sd_layer_step_noalloc": (c_int, [ctypes.POINTER(SdDims), c_int, c_void_p, c_void_p,
                                      c_void_p, ctypes.POINTER(SdLayerWeights),
                                      ctypes.POINTER(SdKv), c_void_p, c_void_p,
                                      ctypes.POINTER(SdRoute), c_void_p, c_void_p]),
    "sd_noalloc_scratch_bytes": (c_size_t, []),
    "sd_draft_head": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p, c_float, c_float,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                              c_void_p]),
    "sd_draft_head_workspace_bytes": (c_size_t, [c_int, c_int, c_int]),
    "sd_debug_dequant": (c_int, [c_int, c_int, c_void_p, c_void_p, c_float, c_void_p, c_void_p]),
    "sd_debug_read_probe": (c_int, [c_void_p, c_size_t, c_void_p, c_void_p]),
    "sd_debug_lanes": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "sd_read_probe_sink_words": (c_int, []),
    "sd_dense_workspace_bytes": (c_size_t, [ctypes.POINTER(SdDims), c_int, c_int, c_int, c_int]),
    "sd_dense_layer_step": (c_int, [ctypes.POINTER(SdDims), c_int, c_void_p,
                                    ctypes.POINTER(SdDenseLayerWeights), ctypes.POINTER(SdKv),
                                    c_void_p, c_size_t, c_void_p]),
    "sd_context_kv_workspace_bytes": (c_size_t, [ctypes.POINTER(SdDims), c_int, c_int]),
    "sd_context_kv": (c_int, [ctypes.POINTER(SdDims), c_int, c_int, c_void_p, c_void_p,
                              ctypes.POINTER(SdCtxLayer), c_void_p, c_void_p, c_size_t,
                              c_void_p]),
}

_lib = None


def lib():
    """The loaded library (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing: build it with "
                          "`python -m speculative_verify_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SYMBOLS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


class SdError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"sdverify error {code}: {msg}")
        self.code = code


def _check(rc):
    if rc != 0:
        raise SdError(rc, lib().sd_last_error().decode())


def ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def cur_stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def make_dims(d):
    return SdDims(hidden=d["hidden"], n_q_heads=d["n_q_heads"], n_kv_heads=d["n_kv_heads"],
                  head_dim=d["head_dim"], q_rows=d["q_rows"], block_size=d.get("block_size", 16),
                  n_experts=d["n_experts"], top_k=d["top_k"], inter=d["inter"],
                  qk_norm=int(d.get("qk_norm", 1)), eps=d["eps"], rope_theta=d["rope_theta"],
                  attn_scale=d.get("attn_scale", 0.0))


def make_kv(kv):
    """kv: dict with device tensors k_cache, v_cache, block_table, seq_lens, positions,
    slot_mapping and ints num_blocks, max_blocks, max_seq_len (and window, default 0; and
    query_start, a device int32 [n_req + 1] tensor for partial drafts, default none)."""
    qs = kv.get("query_start")
    return SdKv(k_cache=ptr(kv["k_cache"]), v_cache=ptr(kv["v_cache"]),
                num_blocks=kv["num_blocks"], block_table=ptr(kv["block_table"]),
                max_blocks=kv["max_blocks"], seq_lens=ptr(kv["seq_lens"]),
                positions=ptr(kv["positions"]), slot_mapping=ptr(kv["slot_mapping"]),
                n_req=int(kv["seq_lens"].numel()), max_seq_len=kv["max_seq_len"],
                window=int(kv.get("window", 0)),
                query_start=ptr(qs) if qs is not None else None)


def make_attn_weights(lay):
    return SdAttnWeights(w_qkv=ptr(lay["w_qkv"]), w_o=ptr(lay["w_o"]))


def make_moe_weights(lay):
    return SdMoeWeights(w_router=ptr(lay["w_router"]), w13_codes=ptr(lay["w13_codes"]),
                        w13_scales=ptr(lay["w13_scales"]), w13_gscale=ptr(lay["w13_gscale"]),
                        w2_codes=ptr(lay["w2_codes"]), w2_scales=ptr(lay["w2_scales"]),
                        w2_gscale=ptr(lay["w2_gscale"]))


def make_layer_weights(lay):
    return SdLayerWeights(g_post_prev=ptr(lay["g_post_prev"]), g_pre_attn=ptr(lay["g_pre_attn"]),
                          g_post_attn=ptr(lay["g_post_attn"]), g_pre_ffn=ptr(lay["g_pre_ffn"]),
                          attn=make_attn_weights(lay), moe=make_moe_weights(lay))


def make_route(r):
    """SdRoute of a dict of device tensors (its "logits" entry is optional)."""
    return SdRoute(**{k: ptr(r.get(k)) for k in ROUTE_FIELDS})


# ------------------------------------------------------------------ entry points
def abi_version():
    return lib().sd_abi_version()


def pack_dense(w, stream=None):
    """Packed copy (sd_pack_dense) of a row-major bf16 device weight [n, k].  The result is
    shaped [ceil(n / 16) * 16, k] for size bookkeeping only: its elements are in the packed
    tile order, not row-major."""
    n, k = w.shape
    nbytes = lib().sd_packed_dense_bytes(n, k)
    if nbytes == 0:
        raise SdError(-1, f"dense weight [{n}, {k}] cannot be packed")
    out = torch.empty(nbytes // (2 * k), k, dtype=torch.bfloat16, device=w.device)
    _check(lib().sd_pack_dense(n, k, ptr(w), ptr(out), cur_stream(stream)))
    return out


def pack_fp4(codes, scales, stream=None):
    """Packed copies (sd_pack_fp4) of block-scaled FP4 device weights: codes uint8 [e, n, k/2],
    scales uint8 [e, n, k/16]."""
    e, n, kh = codes.shape
    co, so = torch.empty_like(codes), torch.empty_like(scales)
    _check(lib().sd_pack_fp4(e, n, 2 * kh, ptr(codes), ptr(scales), ptr(co), ptr(so),
                             cur_stream(stream)))
    return co, so


def workspace_bytes(dims, b, n_req, max_seq_len):
    return lib().sd_workspace_bytes(ctypes.byref(dims), b, n_req, max_seq_len)


def boundary_dualnorm(dims, b, stream_buf, branch, front_embed, g_post, g_pre, out, stream=None,
                      out16=None, aux=None):
    _check(lib().sd_boundary_dualnorm(ctypes.byref(dims), b, ptr(stream_buf), ptr(branch),
                                      ptr(front_embed), ptr(g_post), ptr(g_pre), ptr(out),
                                      ptr(out16), ptr(aux), cur_stream(stream)))


def attn_verify(dims, b, x, attn_w, kv, out, ws, stream=None):
    _check(lib().sd_attn_verify(ctypes.byref(dims), b, ptr(x), ctypes.byref(attn_w),
                                ctypes.byref(kv), ptr(out), ptr(ws), ws.numel() * ws.element_size(),
                                cur_stream(stream)))


def moe_route(dims, b, x, w_router, logit_bias, route, ws, stream=None):
    _check(lib().sd_moe_route(ctypes.byref(dims), b, ptr(x), ptr(w_router), ptr(logit_bias),
                              ctypes.byref(route), ptr(ws), ws.numel() * ws.element_size(),
                              cur_stream(stream)))


def moe_experts(dims, b, x, moe_w, route, y_slots, h_slots, ws, stream=None):
    _check(lib().sd_moe_experts(ctypes.byref(dims), b, ptr(x), ctypes.byref(moe_w),
                                ctypes.byref(route), ptr(y_slots), ptr(h_slots), ptr(ws),
                                ws.numel() * ws.element_size(), cur_stream(stream)))


def moe_experts_x16(dims, b, x16, moe_w, route, y_slots, h_slots, ws, stream=None):
    _check(lib().sd_moe_experts_x16(ctypes.byref(dims), b, ptr(x16), ctypes.byref(moe_w),
                                    ctypes.byref(route), ptr(y_slots), ptr(h_slots), ptr(ws),
                                    ws.numel() * ws.element_size(), cur_stream(stream)))


def moe_unpool(dims, b, y_slots, route, out, stream=None):
    _check(lib().sd_moe_unpool(ctypes.byref(dims), b, ptr(y_slots), ctypes.byref(route),
                               ptr(out), cur_stream(stream)))


def layer_step(dims, b, stream_buf, branch_in, front_embed, layer_w, kv, logit_bias, branch_out,
               route, ws, stream=None, aux=None):
    _check(lib().sd_layer_step(ctypes.byref(dims), b, ptr(stream_buf), ptr(branch_in),
                               ptr(front_embed), ctypes.byref(layer_w), ctypes.byref(kv),
                               ptr(logit_bias), ptr(branch_out),
                               ctypes.byref(route) if route is not None else None, ptr(aux),
                               ptr(ws), ws.numel() * ws.element_size(), cur_stream(stream)))


def layer_step_noalloc(dims, b, stream_buf, branch_in, front_embed, layer_w, kv, logit_bias,
                       branch_out, route, stream=None, aux=None):
    """sd_layer_step on the library's static scratch (no workspace argument)."""
    _check(lib().sd_layer_step_noalloc(ctypes.byref(dims), b, ptr(stream_buf), ptr(branch_in),
                                       ptr(front_embed), ctypes.byref(layer_w), ctypes.byref(kv),
                                       ptr(logit_bias), ptr(branch_out),
                                       ctypes.byref(route) if route is not None else None,
                                       ptr(aux), cur_stream(stream)))


def make_pooled(y_slots, route):
    """A pooled MoE branch: y_slots fp32 [b * k, H] and its SdRoute (kept alive by the
    returned struct's _keep)."""
    p = SdPooled(y_slots=ptr(y_slots), route=ctypes.pointer(route))
    p._keep = (y_slots, route)
    return p


def layer_step_pooled(dims, b, stream_buf, pooled_in, front_embed, layer_w, kv, logit_bias,
                      pooled_out, ws, stream=None, aux=None):
    _check(lib().sd_layer_step_pooled(ctypes.byref(dims), b, ptr(stream_buf),
                                      ctypes.byref(pooled_in) if pooled_in is not None else None,
                                      ptr(front_embed), ctypes.byref(layer_w), ctypes.byref(kv),
                                      ptr(logit_bias), ctypes.byref(pooled_out), ptr(aux),
                                      ptr(ws), ws.numel() * ws.element_size(),
                                      cur_stream(stream)))


def make_dense_layer_weights(lay):
    """Dense draft layer (gains, attention, packed w_gate_up and w_down); the intermediate
    size is read from w_down's shape."""
    return SdDenseLayerWeights(g_pre_attn=ptr(lay["g_pre_attn"]), g_post_attn=ptr(lay["g_post_attn"]),
                               g_pre_ffn=ptr(lay["g_pre_ffn"]), g_post_ffn=ptr(lay["g_post_ffn"]),
                               attn=make_attn_weights(lay), w_gate_up=ptr(lay["w_gate_up"]),
                               w_down=ptr(lay["w_down"]), inter=int(lay["w_down"].shape[1]))


def dense_workspace_bytes(dims, b, n_req, max_seq_len, inter):
    return lib().sd_dense_workspace_bytes(ctypes.byref(dims), b, n_req, max_seq_len, inter)


def dense_layer_step(dims, b, stream_buf, dense_w, kv, ws, stream=None):
    _check(lib().sd_dense_layer_step(ctypes.byref(dims), b, ptr(stream_buf), ctypes.byref(dense_w),
                                     ctypes.byref(kv), ptr(ws), ws.numel() * ws.element_size(),
                                     cur_stream(stream)))


def make_ctx_layers(layers, slot_mappings):
    """Host array of context-store layer descriptors (each layer dict holds g_pre_attn,
    the packed w_qkv, its caches and num_blocks)."""
    arr = (SdCtxLayer * len(layers))()
    for i, (lay, sm) in enumerate(zip(layers, slot_mappings)):
        arr[i] = SdCtxLayer(g_pre_attn=ptr(lay["g_pre_attn"]), w_qkv=ptr(lay["w_qkv"]),
                            k_cache=ptr(lay["k_cache"]), v_cache=ptr(lay["v_cache"]),
                            num_blocks=int(lay["num_blocks"]), slot_mapping=ptr(sm))
    return arr


def context_kv_workspace_bytes(dims, n_ctx, n_layers):
    return lib().sd_context_kv_workspace_bytes(ctypes.byref(dims), n_ctx, n_layers)


def context_kv(dims, n_ctx, states, g_hidden, ctx_layers, positions, ws, stream=None):
    _check(lib().sd_context_kv(ctypes.byref(dims), n_ctx, len(ctx_layers), ptr(states),
                               ptr(g_hidden), ctx_layers, ptr(positions), ptr(ws),
                               ws.numel() * ws.element_size(), cur_stream(stream)))


def draft_head_workspace_bytes(hidden, draft_vocab, b):
    return lib().sd_draft_head_workspace_bytes(hidden, draft_vocab, b)


def draft_head(hidden, draft_vocab, b, h, w_lm, multiplier, soft_cap, d2t, tau_out, draft_ids,
               target_ids, ws, stream=None):
    _check(lib().sd_draft_head(hidden, draft_vocab, b, ptr(h), ptr(w_lm), multiplier, soft_cap,
                               ptr(d2t), ptr(tau_out), ptr(draft_ids), ptr(target_ids), ptr(ws),
                               ws.numel() * ws.element_size(), cur_stream(stream)))


def debug_dequant(n, k, codes, scales, gscale, out, stream=None):
    _check(lib().sd_debug_dequant(n, k, ptr(codes), ptr(scales), gscale, ptr(out),
                                  cur_stream(stream)))


def debug_lanes(x, xi, out, out_i, stream=None):
    """One wave of the kernels' cross-lane exchanges (see sd_debug_lanes)."""
    _check(lib().sd_debug_lanes(ptr(x), ptr(xi), ptr(out), ptr(out_i), cur_stream(stream)))


def read_probe_sink(device):
    """Scratch words sd_debug_read_probe may write."""
    return torch.empty(lib().sd_read_probe_sink_words(), dtype=torch.int32, device=device)


def debug_read_probe(src, sink, stream=None):
    """One plain streaming read of the whole tensor src (the HBM read ceiling probe)."""
    _check(lib().sd_debug_read_probe(ptr(src), src.numel() * src.element_size(), ptr(sink),
                                     cur_stream(stream)))
