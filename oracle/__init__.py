"""Plain fp64 CPU oracle of one speculative-verification decode layer step.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The GPU path (``speculative_verify_decode_amd``) never imports it, and this package
imports nothing from the GPU path: the two share no code.  Inputs come from the
seeded generator, which holds none of the method's arithmetic.

Sources, cited by page title and section (the pages have no numbered equations):

* [DEC]  page "vllm.models.muse_spark.nvidia.specialized_decode.runtime.decode":
  the module docstring's per-layer step list, ``SpecializedDecode.run``,
  ``SpecializedDecode.plan``, ``decode_metadata``.
* [RT]   page "vllm.models.muse_spark.nvidia.specialized_decode.runtime":
  ``unsupported`` (BF16 KV cache, block size 16, 7 speculative tokens, BF16 draft logits).
* [DSP]  page "vllm.models.muse_spark.common.dspark":
  ``MuseSparkDSparkDecoderLayer.forward`` (sandwich-norm order),
  ``MuseSparkDSparkForCausalLM`` (stacked-weight mapper, output multiplier,
  ``apply_output_logit_transform``, ``compute_draft_logits``, ``draft_id_to_target_id``),
  ``MuseSparkDSparkModel.precompute_and_store_context_kv`` (weightless K RMSNorm,
  RoPE, the aliasing pitfall).
* [OCP]  OCP Microscaling Formats (MX) Specification v1.0, sections on the FP4 (E2M1)
  and FP8 (E4M3) element encodings.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms, library
routines, brute force or invariants.  Readings where the pages are silent are listed
in each function's docstring; those readings are "parity unpinned" by the pages.
"""

from .formats import bf16_round, e2m1_decode, e4m3_decode, dequant_nvfp4  # noqa: F401
from .layer import (  # noqa: F401
    rmsnorm,
    dual_norm,
    front_norm,
    qkv_split,
    head_rmsnorm,
    rope,
    qkv_front,
    kv_write,
    paged_attention,
    request_of_row,
    gate_oproj,
    router_logits,
    topk_route,
    pooler,
    expert_ffn,
    moe_experts,
    unpool,
    layer_step,
)
from .head import final_boundary, draft_head, chain_step  # noqa: F401
from .draft import (dense_ffn, dense_layer_step, context_kv, context_kv_store,  # noqa: F401
                    context_rows, context_project)
