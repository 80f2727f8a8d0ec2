"""The C-ABI library loads, exports every symbol the header declares, and rejects bad
arguments on the host before any launch (no GPU needed: every call here fails validation,
so no kernel is ever enqueued)."""

import ctypes
import os
import re
import subprocess

import pytest

from speculative_verify_decode_amd import binding as B
from speculative_verify_decode_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdverify.h")
FAKE = 0x10000          # an aligned address that validation failures never dereference


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\**\s*(sd_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libsdverify.so not built")
    return B.lib()


def dims(**kw):
    d = synth.WORKLOADS["h4096_b8_ctx8k"].dims()
    d.update(kw)
    return B.make_dims(d)


def test_every_header_function_is_exported(lib):
    names = header_functions()
    assert len(names) >= 12, names
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (sd_\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert n in B.SYMBOLS, f"binding lacks {n}"
        getattr(lib, n)


def test_no_extra_exports_beyond_header(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (sd_\w+)$", out, flags=re.M))
    assert exported == set(header_functions())


def test_abi_version(lib):
    assert B.abi_version() == 7


def test_workspace_bytes_host_only(lib):
    d = dims()
    n = B.workspace_bytes(d, 8, 1, 8192)
    assert n > 0 and n % 256 == 0
    assert B.workspace_bytes(d, 64, 8, 32768) > n
    assert B.workspace_bytes(dims(block_size=32), 8, 1, 8192) == 0
    assert B.workspace_bytes(d, 7, 1, 8192) > 0            # a partial draft of 7 rows
    assert B.workspace_bytes(d, 65, 9, 8192) == 0


def _rc_dualnorm(d, b=8, stream=FAKE, branch=FAKE, front=None, g_post=FAKE, g_pre=FAKE, out=FAKE,
                 aux=None):
    L = B.lib()
    return L.sd_boundary_dualnorm(ctypes.byref(d) if d is not None else None, b, stream, branch,
                                  front, g_post, g_pre, out, None, aux, None)


@pytest.mark.parametrize("kw,code,text", [
    (dict(hidden=300), -2, "hidden"),
    (dict(head_dim=96), -2, "head_dim"),
    (dict(n_kv_heads=5), -1, "multiple"),
    (dict(q_rows=4), -2, "q_rows"),
    (dict(block_size=32), -2, "block size"),
    (dict(n_experts=0), -2, "n_experts"),
    (dict(top_k=9), -2, "top_k"),
    (dict(inter=100), -2, "inter"),
    (dict(eps=0.0), -1, "eps"),
    (dict(qk_norm=2), -1, "qk_norm"),
])
def test_bad_dims_rejected_with_reason(lib, kw, code, text):
    assert _rc_dualnorm(dims(**kw)) == code
    assert text in lib.sd_last_error().decode()


def test_null_dims_and_pointers(lib):
    assert _rc_dualnorm(None) == -1
    assert _rc_dualnorm(dims(), stream=None) == -1
    assert _rc_dualnorm(dims(), branch=None, front=None) == -1
    assert "front" in lib.sd_last_error().decode()
    assert _rc_dualnorm(dims(), aux=FAKE + 4) == -1                # a misaligned aux tap
    assert "aux" in lib.sd_last_error().decode()


def test_row_count_limits(lib):
    # entry points without a KV cache take any b in 1..64 (partial drafts give any count)
    assert _rc_dualnorm(dims(), b=0) == -2
    assert _rc_dualnorm(dims(), b=72) == -2
    d = dims()
    assert lib.sd_workspace_bytes(ctypes.byref(d), 12, 2, 8192) > 0
    assert lib.sd_workspace_bytes(ctypes.byref(d), 65, 9, 8192) == 0


def _kv(**kw):
    base = dict(k_cache=FAKE, v_cache=FAKE, num_blocks=4096, block_table=FAKE, max_blocks=512,
                seq_lens=FAKE, positions=FAKE, slot_mapping=FAKE, n_req=1, max_seq_len=8192)
    base.update(kw)
    return B.SdKv(**base)


def _rc_attn(d, kv, ws=None, ws_bytes=0, b=8):
    w = B.SdAttnWeights(w_qkv=FAKE, w_o=FAKE)
    return B.lib().sd_attn_verify(ctypes.byref(d), b, FAKE, ctypes.byref(w), ctypes.byref(kv),
                                  FAKE, ws, ws_bytes, None)


def test_attention_validation(lib):
    d = dims()
    assert _rc_attn(d, _kv(n_req=2)) == -2                        # b != n_req * q_rows
    assert _rc_attn(d, _kv(n_req=0)) == -1
    # partial drafts: 1..q_rows rows per request
    assert _rc_attn(d, _kv(n_req=2, query_start=FAKE), b=17) == -1  # more than 2 * 8 rows
    assert "1..8 verify rows" in lib.sd_last_error().decode()
    assert _rc_attn(d, _kv(n_req=3, query_start=FAKE), b=2) == -1   # fewer rows than requests
    assert _rc_attn(d, _kv(n_req=2, query_start=FAKE), b=9) == -4   # valid rows: workspace next
    assert _rc_attn(d, _kv(max_blocks=4)) == -1                   # table too short
    assert _rc_attn(d, _kv(k_cache=FAKE + 2)) == -1                # misaligned cache
    assert _rc_attn(d, _kv(seq_lens=None)) == -1
    assert _rc_attn(d, _kv(window=-1)) == -1                      # negative sliding window
    assert "window" in lib.sd_last_error().decode()
    assert _rc_attn(d, _kv()) == -4                               # no workspace
    assert _rc_attn(d, _kv(), ws=FAKE, ws_bytes=1024) == -4        # too small
    assert "need" in lib.sd_last_error().decode()


def test_layer_step_validation(lib):
    d = dims()
    lw = B.SdLayerWeights(g_post_prev=FAKE, g_pre_attn=FAKE, g_post_attn=FAKE, g_pre_ffn=FAKE,
                          attn=B.SdAttnWeights(FAKE, FAKE),
                          moe=B.SdMoeWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE))
    kv = _kv()
    L = B.lib()
    def rc(front=None, branch=FAKE, route=None, aux=None, ws=None, ws_bytes=0):
        return L.sd_layer_step(ctypes.byref(d), 8, FAKE, branch, front, ctypes.byref(lw),
                               ctypes.byref(kv), None, FAKE,
                               ctypes.byref(route) if route is not None else None, aux, ws,
                               ws_bytes, None)
    assert rc(branch=None) == -1 and "front" in L.sd_last_error().decode()
    assert rc() == -4
    assert rc(aux=FAKE + 4) == -1 and "aux" in L.sd_last_error().decode()
    route = B.SdRoute(*([FAKE] * 7), FAKE + 4)                     # misaligned logits
    assert rc(route=route) == -1 and "logits" in L.sd_last_error().decode()
    route = B.SdRoute(*([FAKE] * 7), None)                         # logits are optional
    assert rc(route=route) == -4
    lw.moe.w13_codes = FAKE + 8
    assert rc(ws=FAKE, ws_bytes=1 << 40) == -1 and "aligned" in L.sd_last_error().decode()


def test_expert_entry_points_validation(lib):
    d = dims()
    mw = B.SdMoeWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    route = B.SdRoute(*([FAKE] * 7), None)
    for fn, name in ((lib.sd_moe_experts, "x"), (lib.sd_moe_experts_x16, "x16")):
        def rc(x=FAKE, y=FAKE, ws=FAKE, ws_bytes=1 << 30, r=route):
            return fn(ctypes.byref(d), 8, x, ctypes.byref(mw), ctypes.byref(r), y, None, ws,
                      ws_bytes, None)
        assert rc(x=None) == -1 and name in lib.sd_last_error().decode()
        assert rc(x=FAKE + 2) == -1 and "aligned" in lib.sd_last_error().decode()
        assert rc(ws=None) == -4
        assert rc(r=B.SdRoute(None, *([FAKE] * 6), None)) == -1
    assert lib.sd_moe_route(ctypes.byref(d), 8, FAKE, FAKE, None,
                            ctypes.byref(B.SdRoute(*([FAKE] * 7), FAKE + 4)), FAKE, 1 << 30,
                            None) == -1
    assert "logits" in lib.sd_last_error().decode()


def test_dense_layer_validation(lib):
    d = dims()
    attn = B.SdAttnWeights(w_qkv=FAKE, w_o=FAKE)
    def rc(inter=8192, ws=FAKE, ws_bytes=1 << 40, g=FAKE, kv=None):
        w = B.SdDenseLayerWeights(g_pre_attn=g, g_post_attn=FAKE, g_pre_ffn=FAKE, g_post_ffn=FAKE,
                                  attn=attn, w_gate_up=FAKE, w_down=FAKE, inter=inter)
        return lib.sd_dense_layer_step(ctypes.byref(d), 8, FAKE, ctypes.byref(w),
                                       ctypes.byref(kv or _kv()), ws, ws_bytes, None)
    assert rc(g=None) == -1                                       # a gain is null
    assert rc(inter=1000) == -2 and "128" in lib.sd_last_error().decode()
    assert rc(kv=_kv(window=-3)) == -1
    assert rc(ws=None) == -4
    need = B.dense_workspace_bytes(d, 8, 1, 8192, 8192)
    assert need > B.workspace_bytes(d, 8, 1, 8192)                # the FFN regions on top
    assert rc(ws_bytes=need - 1) == -4 and "need" in lib.sd_last_error().decode()


def test_context_kv_validation(lib):
    d = dims()
    lay = (B.SdCtxLayer * 2)()
    for i in range(2):
        lay[i] = B.SdCtxLayer(g_pre_attn=FAKE, w_qkv=FAKE, k_cache=FAKE, v_cache=FAKE,
                              num_blocks=64, slot_mapping=FAKE)
    def rc(n=8, nl=2, ws=FAKE, ws_bytes=1 << 30, states=FAKE):
        return lib.sd_context_kv(ctypes.byref(d), n, nl, states, FAKE, lay, FAKE, ws, ws_bytes, None)
    assert rc(n=0) == -2 and rc(n=65) == -2
    assert rc(nl=17) == -2
    assert rc(states=None) == -1
    assert rc(states=FAKE + 2) == -1                               # misaligned
    assert rc(ws=None) == -4
    assert B.context_kv_workspace_bytes(d, 0, 2) == 0
    assert B.context_kv_workspace_bytes(d, 8, 2) > 0
    lay[1].v_cache = None
    assert rc() == -1 and "layer 1" in lib.sd_last_error().decode()


def test_draft_head_validation(lib):
    L = B.lib()
    args = lambda **kw: dict(dict(hidden=4096, vocab=32768, b=8, mult=0.25, ws=FAKE, nbytes=1 << 30), **kw)
    def rc(a):
        return L.sd_draft_head(a["hidden"], a["vocab"], a["b"], FAKE, FAKE, a["mult"], 30.0, FAKE,
                               None, FAKE, FAKE, a["ws"], a["nbytes"], None)
    assert rc(args(mult=-1.0)) == -1
    assert rc(args(mult=0.0)) == -1
    assert rc(args(vocab=1000)) == -2
    assert rc(args(hidden=100)) == -2
    assert rc(args(b=65)) == -2
    assert rc(args(ws=None)) == -4
    assert B.draft_head_workspace_bytes(4096, 32768, 8) > 0


def test_debug_dequant_validation(lib):
    L = B.lib()
    assert L.sd_debug_dequant(4, 48, FAKE, FAKE, 1.0, FAKE, None) == -1
    assert L.sd_debug_dequant(4, 64, FAKE + 1, FAKE, 1.0, FAKE, None) == -1


def test_packed_dense_bytes(lib):
    L = B.lib()
    assert L.sd_packed_dense_bytes(10240, 4096) == 10240 * 4096 * 2
    assert L.sd_packed_dense_bytes(40, 96) == 48 * 96 * 2      # rows padded to 16
    assert L.sd_packed_dense_bytes(16, 48) == 0                # k % 32 != 0
    assert L.sd_packed_dense_bytes(0, 64) == 0


def test_pack_validation(lib):
    L = B.lib()
    assert L.sd_pack_dense(16, 48, FAKE, FAKE + 4096, None) == -1
    assert L.sd_pack_dense(16, 64, FAKE + 8, FAKE + 4096, None) == -1   # misaligned
    assert L.sd_pack_dense(16, 64, FAKE, FAKE, None) == -1              # in place
    assert "in place" in L.sd_last_error().decode() or "out of place" in L.sd_last_error().decode()
    assert L.sd_pack_fp4(2, 24, 128, FAKE, FAKE, FAKE + 4096, FAKE + 8192, None) == -1  # n % 16
    assert L.sd_pack_fp4(2, 32, 96, FAKE, FAKE, FAKE + 4096, FAKE + 8192, None) == -1   # k % 128
    assert L.sd_pack_fp4(2, 32, 128, FAKE, FAKE + 1, FAKE + 4096, FAKE + 8192, None) == -1
    assert L.sd_pack_fp4(2, 32, 128, None, FAKE, FAKE + 4096, FAKE + 8192, None) == -1


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "speculative_verify_decode_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, flags=re.M), f
                assert "oracle/" not in text, f


def test_noalloc_step_validates_on_the_host(lib):
    """sd_layer_step_noalloc checks sizes before it touches the device: a step whose
    workspace exceeds the static scratch fails with SD_EWORKSPACE, and bad arguments fail as
    for sd_layer_step (no device is needed for either)."""
    d = dims()
    lw = B.SdLayerWeights(g_post_prev=FAKE, g_pre_attn=FAKE, g_post_attn=FAKE, g_pre_ffn=FAKE,
                          attn=B.SdAttnWeights(FAKE, FAKE),
                          moe=B.SdMoeWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE))
    assert lib.sd_noalloc_scratch_bytes() == 32 << 20
    def rc(b=8, **kw):
        kv = _kv(**kw)
        return lib.sd_layer_step_noalloc(ctypes.byref(d), b, FAKE, FAKE, None, ctypes.byref(lw),
                                         ctypes.byref(kv), None, FAKE, None, None, None)
    assert rc(max_seq_len=1 << 24, max_blocks=1 << 20) == -4
    assert "scratch" in lib.sd_last_error().decode()
    assert B.workspace_bytes(d, 8, 1, 1 << 24) > lib.sd_noalloc_scratch_bytes()
    assert rc(n_req=2) == -2                                       # b != n_req * q_rows
    assert rc(b=0) == -2
