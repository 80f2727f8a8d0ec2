"""Test-side glue: converts generator tensors to the arrays the oracle reads, and the
comparison rules shared by the parity tests."""

import numpy as np
import torch


def np64(t):
    """fp64 values of a float tensor (bf16/fp32), or the raw array of an integer one."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t
    if t.dtype in (torch.bfloat16, torch.float16, torch.float32, torch.float64):
        return t.detach().cpu().to(torch.float64).numpy()
    return t.detach().cpu().numpy()


LAYER_KEYS = ("g_post_prev", "g_pre_attn", "g_post_attn", "g_pre_ffn", "g_post_ffn", "w_qkv",
              "w_o", "w_router", "w13_codes", "w13_scales", "w13_gscale", "w2_codes",
              "w2_scales", "w2_gscale", "k_cache", "v_cache", "block_table", "seq_lens",
              "positions", "slot_mapping")


def oracle_layer_inputs(lay, act, stream=None):
    inp = {k: np64(lay[k]) for k in LAYER_KEYS}
    inp["stream"] = np64(act["stream"]) if stream is None else stream
    inp["logit_bias"] = np64(act.get("logit_bias"))
    inp["window"] = int(lay.get("window", 0))
    qs = lay.get("query_start")
    inp["query_start"] = None if qs is None else np.asarray(qs).astype(np.int64)
    return inp


def close(gpu, ref, tol=2e-2):
    """The float bar: |gpu - ref| <= tol * (1 + |ref|) for every element."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bound = tol * (1.0 + np.abs(ref))
    bad = ~(err <= bound)
    return not bad.any(), float((err / (1.0 + np.abs(ref))).max(initial=0.0)), int(bad.sum())


def assert_close(gpu, ref, what, tol=2e-2):
    ok, worst, nbad = close(gpu, ref, tol)
    assert ok, f"{what}: {nbad} elements beyond {tol}*(1+|ref|); worst scaled error {worst:.3e}"
    return worst
