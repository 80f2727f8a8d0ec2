/*
 * sdverify.h -- C ABI of libsdverify.so: one speculative-verification decode layer step of
 * a Muse-Spark-style MoE decoder layer on one MI355X (gfx950) GPU.
 *
 * Sources, cited by page title and section:
 *   [DEC] "vllm.models.muse_spark.nvidia.specialized_decode.runtime.decode": module
 *         docstring (the per-layer step list), SpecializedDecode.run / .build / .plan,
 *         decode_metadata.
 *   [RT]  "vllm.models.muse_spark.nvidia.specialized_decode.runtime": unsupported
 *         (BF16 KV cache, block size 16, 7 speculative tokens, BF16 draft logits).
 *   [DSP] "vllm.models.muse_spark.common.dspark": MuseSparkDSparkDecoderLayer.forward
 *         (sandwich norms), MuseSparkDSparkForCausalLM (stacked weights, output transform,
 *         draft_id_to_target_id), MuseSparkDSparkModel.precompute_and_store_context_kv.
 *
 * Conventions (all entry points):
 *   - Every pointer is a DEVICE pointer unless stated otherwise; the caller owns all memory.
 *     The library never allocates, frees or synchronises; weights are read-only (the
 *     executor reads the backbone and never modifies it, [DEC] SpecializedDecode).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only enqueues
 *     kernels on it and may be captured into a HIP graph ([DEC] module docstring and
 *     SpecializedDecode.plan: the step runs inside a captured graph).
 *   - bf16 tensors are raw 16-bit bfloat16; fp32 are IEEE float; activations, caches and
 *     metadata are row-major and contiguous.  Weight matrices are in the packed layouts
 *     below, made once from row-major weights by sd_pack_dense / sd_pack_fp4.
 *   - b = rows of the step, request-major.  q_rows = 1 + 7 verify tokens ([RT]
 *     unsupported; [DEC] decode_metadata).  By default every request verifies q_rows tokens:
 *     b = n_req * q_rows and row t belongs to request t / q_rows.  With sd_kv.query_start a
 *     request verifies 1..q_rows tokens (partial drafts, below).  Entry points that take no
 *     KV cache accept any b in 1..64.
 *   - Return 0 on success, a negative SD_E* code otherwise; nothing is enqueued on an
 *     error.  sd_last_error() gives the first failing reason in words (thread-local).
 *   - Validation happens on the host, before any launch: dims, sizes, null pointers,
 *     16-byte alignment of vector-loaded tensors, workspace size.  Device-side contents
 *     (block-table entries, slot mapping, positions) are the caller's contract: they must
 *     address blocks < num_blocks, positions < seq_len, and be consistent with each other.
 *   - Calls that share a workspace on different streams must not overlap.
 */
#ifndef SDVERIFY_H
#define SDVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SD_ABI_VERSION 7

enum {
  SD_OK = 0,
  SD_EINVAL = -1,        /* a null pointer, a bad size or a misaligned tensor            */
  SD_EUNSUPPORTED = -2,  /* valid request outside what the kernels implement             */
  SD_EHIP = -3,          /* a HIP runtime call failed (launch error)                     */
  SD_EWORKSPACE = -4     /* workspace null or smaller than sd_workspace_bytes()          */
};

/* Layer dimensions.  Supported: hidden % 256 == 0 and <= 8192; head_dim in {64, 128};
 * n_q_heads % n_kv_heads == 0 with (n_q_heads / n_kv_heads) * q_rows in {16, 32, 64};
 * q_rows == 8; block_size == 16 ([RT] unsupported: KV block sizes other than 16);
 * n_experts in [1, 256]; 1 <= top_k <= min(8, n_experts); inter % 128 == 0;
 * qk_norm in {0, 1}; eps > 0; attn_scale 0 means head_dim ** -0.5. */
typedef struct sd_dims {
  int32_t hidden, n_q_heads, n_kv_heads, head_dim, q_rows, block_size;
  int32_t n_experts, top_k, inter, qk_norm;
  float eps, rope_theta, attn_scale;
} sd_dims;

/* Packed weight layouts.  The step streams every weight byte once per step; it reads them
 * in the order the matrix cores consume them, so that each load instruction of a wave is
 * one contiguous 1 KB piece.  Packing is a one-time preprocessing of loaded weights.
 *
 * Dense bf16 W [N, K] (w_qkv, w_o, w_router, w_lm), K % 32 == 0: ceil(N / 16) tiles of 16
 * rows by K / 32 tiles of 32 columns.  Tile (nt, kt) is 512 contiguous bf16 starting at
 * element (nt * (K / 32) + kt) * 512; its element 8 * l + j (l < 64, j < 8) is
 * W[16 nt + l % 16, 32 kt + 8 (l / 16) + j], and 0 for rows >= N.  Size:
 * sd_packed_dense_bytes(N, K) = ceil(N / 16) * 16 * K * 2 bytes.
 *
 * Block-scaled FP4 weights [E, N, K] (codes [E, N, K/2], scales [E, N, K/16] as described at
 * sd_moe_weights), N % 16 == 0, K % 128 == 0: tiles of 16 rows by 128 weights, indexed
 * t = (e * (N / 16) + nt) * (K / 128) + kt.  Codes tile t is 1024 bytes at t * 1024: bytes
 * 16 l .. 16 l + 15 are the code bytes 64 kt + 16 (l / 16) .. + 15 of row 16 nt + l % 16 of
 * expert e.  Scales tile t is 128 bytes at t * 128: bytes 2 l, 2 l + 1 are the scale bytes
 * 8 kt + 2 (l / 16), + 1 of that row.  Packed sizes equal the row-major sizes. */

/* Attention weights, packed bf16 (see above).  w_qkv [(2*Hq + 2*Hkv) * D, H]: rows are the
 * stacked q | k | v | o_gate projections in that order ([DSP] hf_to_vllm_mapper).
 * w_o [H, Hq * D]. */
typedef struct sd_attn_weights {
  const void *w_qkv;
  const void *w_o;
} sd_attn_weights;

/* Routed-MoE weights, packed (see above).  w_router bf16 [E, H].  Experts are block-scaled
 * FP4; in row-major terms, for matrix
 * [N, K] of expert e, codes uint8 [E, N, K/2] hold two E2M1 codes per byte (low nibble =
 * even k), scales uint8 [E, N, K/16] hold one E4M3FN scale per 16 consecutive k, gscale
 * fp32 [E] one scale per matrix: W[n, k] = e2m1 * e4m3 * gscale.  W13 is [2I, H] with the
 * gate rows first ([DSP] hf_to_vllm_mapper: gate_proj then up_proj); W2 is [H, I]. */
typedef struct sd_moe_weights {
  const void *w_router;
  const uint8_t *w13_codes, *w13_scales;
  const float *w13_gscale;
  const uint8_t *w2_codes, *w2_scales;
  const float *w2_gscale;
} sd_moe_weights;

/* One layer.  Gains are fp32 [H]: g_post_prev is the post-norm of the incoming branch (the
 * previous layer's post-FFN norm), g_pre_attn / g_post_attn / g_pre_ffn the layer's own
 * sandwich norms ([DSP] MuseSparkDSparkDecoderLayer.forward). */
typedef struct sd_layer_weights {
  const float *g_post_prev, *g_pre_attn, *g_post_attn, *g_pre_ffn;
  sd_attn_weights attn;
  sd_moe_weights moe;
} sd_layer_weights;

/* Paged KV cache and the step's metadata ([DEC] plan: block-table decode metadata and
 * the step's slot mapping).  k_cache bf16 [num_blocks, Hkv, 16, D] (token-major inside
 * a block); v_cache bf16 [num_blocks, Hkv, D, 16] (dim-major inside a block).
 * block_table int32 [n_req, max_blocks]; seq_lens int32 [n_req] count every token of the
 * request including its verify tokens; positions int32 [b] (row j of request r is at
 * seq_lens[r] - q_rows + j); slot_mapping int64 [b] = block * 16 + offset where that
 * row's K/V is written (a negative slot writes nothing, and attention then reads whatever
 * the cache holds at that row's position).  max_seq_len bounds seq_lens
 * (host value, sizes the launch; device seq_lens are clamped to max_blocks * 16).
 * window: the layer's sliding window ([DEC] SpecializedDecode.plan: attn2 serves each
 * layer's sliding window).  0 = full causal attention; w > 0 = a row at position p sees
 * positions max(0, p - w + 1) .. p only.  The blocks a request's rows cannot see are not
 * read; which blocks those are follows from seq_lens and the positions contract above.
 * query_start: NULL, or int32 [n_req + 1] for partial drafts (requests that verify fewer
 * than q_rows tokens; [DEC] SpecializedDecode.plan leaves them, and steps of several
 * requests, to the stock forward).  Request r's rows are query_start[r] ..
 * query_start[r + 1] - 1, q_r = their count in 1..q_rows, query_start[0] = 0 and
 * query_start[n_req] = b; row j of request r is at position seq_lens[r] - q_r + j.  The
 * host checks n_req <= b <= n_req * q_rows; the contents are the caller's contract, and
 * every row index the kernels derive from them is clamped into 0 .. b - 1, so a bad array
 * gives wrong rows, never an access out of range. */
typedef struct sd_kv {
  void *k_cache, *v_cache;
  int32_t num_blocks;
  const int32_t *block_table;
  int32_t max_blocks;
  const int32_t *seq_lens;
  const int32_t *positions;
  const int64_t *slot_mapping;
  int32_t n_req, max_seq_len;
  int32_t window;
  const int32_t *query_start;
} sd_kv;

/* Routing outputs.  topk_ids int32 [b, k] (descending logit, ties to the lower expert
 * index), topk_w fp32 [b, k] (softmax over the k selected logits), expert_counts int32
 * [E], expert_offsets int32 [E + 1] (exclusive prefix sum), slot_of int32 [b, k] (pooled
 * slot of each choice: a stable counting sort by (expert, row)), token_of_slot int32
 * [b * k] (its inverse), active_experts int32 [E + 1]: the ids of experts with a nonzero
 * count in ascending order, then at index E their number.  logits (may be NULL) fp32
 * [b, E] receives the router logits the routing ranked, bias included: the routing is
 * exactly the top-k of these values by (-z, index). */
typedef struct sd_route {
  int32_t *topk_ids;
  float *topk_w;
  int32_t *expert_counts, *expert_offsets, *slot_of, *token_of_slot, *active_experts;
  float *logits;
} sd_route;

int sd_abi_version(void);
const char *sd_last_error(void);

/* Bytes of the packed copy of a dense bf16 [n, k] weight (0 if k % 32 != 0 or n, k <= 0). */
size_t sd_packed_dense_bytes(int32_t n, int32_t k);

/* Pack a row-major bf16 weight src [n, k] into dst (sd_packed_dense_bytes(n, k) bytes).
 * k % 32 == 0; src and dst 16-byte aligned and not overlapping.  Enqueued on stream. */
int sd_pack_dense(int32_t n, int32_t k, const void *src, void *dst, void *stream_handle);

/* Pack row-major block-scaled FP4 weights of e matrices [n, k] (codes [e, n, k/2], scales
 * [e, n, k/16]) into codes_out / scales_out of the same sizes.  n % 16 == 0, k % 128 == 0;
 * codes 16-byte and scales 2-byte aligned; outputs do not overlap inputs. */
int sd_pack_fp4(int32_t e, int32_t n, int32_t k, const uint8_t *codes, const uint8_t *scales,
                uint8_t *codes_out, uint8_t *scales_out, void *stream_handle);

/* Bytes of workspace every call below needs for this shape (the largest of them). */
size_t sd_workspace_bytes(const sd_dims *dims, int32_t b, int32_t n_req, int32_t max_seq_len);

/* Input boundary / front / final boundary ([DEC] module docstring: the first layer's front,
 * the input boundary's dual norm, the final boundary; order from [DSP]
 * MuseSparkDSparkDecoderLayer.forward).  stream fp32 [b, H] in/out.
 *   branch != NULL: stream += RMSNorm(branch; g_post); y = RMSNorm(stream; g_pre).
 *   branch == NULL (front): stream = front_embed; y = RMSNorm(stream; g_pre).
 * branch fp32 [b, H] (the branches between blocks are fp32); front_embed bf16 [b, H];
 * gains fp32 [H]; out bf16 [b, H] = bf16(y) (e.g. the final hidden cast for the draft
 * head); out16 (may be NULL) fp16 [2, b, H] = the expert-input form of y: hi terms, then
 * lo terms, of y * 2^-8 (y * 2^-8 ~ hi + lo to about 2^-22 relative).
 * aux (may be NULL) fp32 [b, H]: the aux hidden-state tap, a copy of the stream this
 * boundary hands on (after its residual add, before the norm), as the boundary of an aux
 * layer and the final boundary write it for the drafter ([DEC] DecodeLayer.aux,
 * SpecializedDecode.build / .run). */
int sd_boundary_dualnorm(const sd_dims *dims, int32_t b, float *stream, const float *branch,
                         const void *front_embed, const float *g_post, const float *g_pre,
                         void *out, void *out16, float *aux, void *stream_handle);

/* Attention of one layer ([DEC] module docstring: QKV front -> attn2 -> o_proj):
 * stacked QKV projection of x (bf16 [b, H]); weightless per-head RMSNorm of q and k when
 * dims->qk_norm; RoPE at each row's position; bf16 K/V written to the cache at
 * slot_mapping (the cache is modified there and nowhere else); causal GQA attention of each
 * row over positions 0..p of its request (the last kv->window of them when window > 0);
 * output gate o * sigmoid(o_gate); o_proj.
 * out fp32 [b, H] (the attention branch). */
int sd_attn_verify(const sd_dims *dims, int32_t b, const void *x, const sd_attn_weights *w,
                   const sd_kv *kv, float *out, void *ws, size_t ws_bytes, void *stream_handle);

/* Router -> routing -> pooler ([DEC] module docstring).  z = x (bf16 [b, H]) * w_router^T
 * + logit_bias (fp32 [b, E], may be NULL); top-k, weights and pooler maps into *route
 * (every field required except route->logits, which receives z when not NULL). */
int sd_moe_route(const sd_dims *dims, int32_t b, const void *x, const void *w_router,
                 const float *logit_bias, const sd_route *route, void *ws, size_t ws_bytes,
                 void *stream_handle);

/* Routed experts over pooled slots ([DEC] module docstring: routed experts; [RT] module
 * list: NVFP4 routed experts): for slot s = (row t, expert e), y[s] = W2_e * h[s] with
 * h[s] = silu(g) * u and [g | u] = W13_e * x[t], weights dequantised exactly, fp32
 * accumulation, h kept at near-fp32 precision between the two GEMMs.  x bf16 [b, H] (the
 * MoE input); route as produced by sd_moe_route; y_slots fp32 [b * k, H]; h_slots (may be
 * NULL) receives bf16(h) [b * k, I].  The call first writes the expert GEMMs' input form
 * of x into the workspace (see sd_moe_experts_x16), then runs the two GEMMs. */
int sd_moe_experts(const sd_dims *dims, int32_t b, const void *x, const sd_moe_weights *w,
                   const sd_route *route, void *y_slots, void *h_slots, void *ws,
                   size_t ws_bytes, void *stream_handle);

/* sd_moe_experts on the expert GEMMs' own input form, as the layer step feeds them: x16
 * fp16 [2, b, H] holds the hi terms, then the lo terms, of x * 2^-8 (x * 2^-8 ~ hi + lo to
 * about 2^-22 relative), which sd_boundary_dualnorm's out16 writes from the fp32 norm
 * output.  Every other argument and result is as for sd_moe_experts. */
int sd_moe_experts_x16(const sd_dims *dims, int32_t b, const void *x16,
                       const sd_moe_weights *w, const sd_route *route, void *y_slots,
                       void *h_slots, void *ws, size_t ws_bytes, void *stream_handle);

/* Unpooler ([DEC] module docstring): out[t] = sum over j < k, in order, of
 * topk_w[t, j] * y_slots[slot_of[t, j]], in fp32.  y_slots fp32 [b * k, H];
 * out fp32 [b, H] (the MoE branch). */
int sd_moe_unpool(const sd_dims *dims, int32_t b, const float *y_slots, const sd_route *route,
                  float *out, void *stream_handle);

/* One whole layer step in the order of [DEC] SpecializedDecode.run: input boundary (or the
 * front when branch_in == NULL, taking front_embed) -> attention -> attention boundary ->
 * router -> routing -> pooler -> experts -> unpooler.  stream fp32 [b, H] in/out;
 * branch_in fp32 [b, H] (the previous layer's MoE output); front_embed bf16 [b, H];
 * branch_out fp32 [b, H] receives the unpooled MoE output (the next boundary's branch;
 * it may alias branch_in, which is read first).  route_out may be NULL (then routing lives
 * in the workspace; route_out->logits may be NULL); logit_bias may be NULL.  aux (may be
 * NULL) fp32 [b, H]: the layer's aux hidden-state tap, written by its input boundary as
 * sd_boundary_dualnorm's aux (the stream entering the layer's attention block). */
int sd_layer_step(const sd_dims *dims, int32_t b, float *stream, const float *branch_in,
                  const void *front_embed, const sd_layer_weights *w, const sd_kv *kv,
                  const float *logit_bias, float *branch_out, const sd_route *route_out,
                  float *aux, void *ws, size_t ws_bytes, void *stream_handle);

/* A pooled MoE branch: the routed experts' per-slot outputs y_slots fp32 [b * k, H] and the
 * routing that weighs them (route: topk_w and slot_of are read; every field is written by
 * the step that produces it). */
typedef struct sd_pooled {
  float *y_slots;
  const sd_route *route;
} sd_pooled;

/* The layer step of a stack, with the unpooler moved into the next layer's input boundary
 * ([DEC] SpecializedDecode.run: the input boundary gathers the previous layer's MoE output
 * before its dual norm).  branch_in: the previous layer's pooled output, gathered as
 * u[t] = sum over j < k, in order, of topk_w[t, j] * y_slots[slot_of[t, j]], then the same
 * boundary as sd_layer_step (NULL: the front, from front_embed).  branch_out: this layer's
 * experts write y_slots and the routing writes route (route->logits may be NULL), and no
 * unpooler runs; the final boundary of a stack gathers with sd_moe_unpool.  Every other
 * argument and result, aux included, is as for sd_layer_step.  branch_out may be
 * branch_in (it is read before it is written). */
int sd_layer_step_pooled(const sd_dims *dims, int32_t b, float *stream,
                         const sd_pooled *branch_in, const void *front_embed,
                         const sd_layer_weights *w, const sd_kv *kv, const float *logit_bias,
                         const sd_pooled *branch_out, float *aux, void *ws, size_t ws_bytes,
                         void *stream_handle);

/* sd_layer_step for callers that cannot allocate (code under HIP graph capture that may not
 * call hipMalloc, tight serving loops, harnesses that forbid allocation): the same step, the
 * same arguments and results, with no workspace argument.  Its scratch is a static device
 * array the library owns, sd_noalloc_scratch_bytes() (32 MiB) on each GPU it runs on, held
 * until the process ends; its address is looked up on the first call on each device (with
 * that device current).  A step whose workspace (sd_workspace_bytes) exceeds that size
 * returns SD_EWORKSPACE before anything is enqueued.  The call allocates and frees nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (different
 * streams, or graphs replayed concurrently) race and must be serialised by the caller. */
int sd_layer_step_noalloc(const sd_dims *dims, int32_t b, float *stream, const float *branch_in,
                          const void *front_embed, const sd_layer_weights *w, const sd_kv *kv,
                          const float *logit_bias, float *branch_out, const sd_route *route_out,
                          float *aux, void *stream_handle);

/* Bytes of the static scratch of sd_layer_step_noalloc (per GPU). */
size_t sd_noalloc_scratch_bytes(void);

/* Draft head on bf16 hidden rows h [b, hidden] ([DSP] compute_draft_logits,
 * apply_output_logit_transform, draft_id_to_target_id; [RT] unsupported: BF16 logits):
 * logits = bf16(h * w_lm^T) with w_lm packed bf16 [draft_vocab, hidden]; tau = soft_cap *
 * tanh(logits * multiplier / soft_cap) (soft_cap <= 0: tau = logits * multiplier);
 * draft_ids int32 [b] = lowest index of the largest logit; target_ids int64 [b] =
 * d2t[draft_ids] with d2t int64 [draft_vocab].  tau_out fp32 [b, draft_vocab] may be NULL.
 * multiplier must be > 0 (the transform is then monotone and keeps the argmax). */
int sd_draft_head(int32_t hidden, int32_t draft_vocab, int32_t b, const void *h,
                  const void *w_lm, float multiplier, float soft_cap, const int64_t *d2t,
                  float *tau_out, int32_t *draft_ids, int64_t *target_ids, void *ws,
                  size_t ws_bytes, void *stream_handle);

/* Bytes of workspace sd_draft_head needs. */
size_t sd_draft_head_workspace_bytes(int32_t hidden, int32_t draft_vocab, int32_t b);

/* ---- Draft side ([DSP] MuseSparkDSparkDecoderLayer, MuseSparkDSparkModel) ---- */

/* One dense draft layer.  Gains fp32 [H] (the layer's own sandwich norms); attention
 * weights as for sd_attn_verify; w_gate_up packed bf16 [2 * inter, H] with the gate rows
 * first ([DSP] hf_to_vllm_mapper: gate_proj and up_proj stacked as shards 0 and 1);
 * w_down packed bf16 [H, inter]; inter % 128 == 0. */
typedef struct sd_dense_layer_weights {
  const float *g_pre_attn, *g_post_attn, *g_pre_ffn, *g_post_ffn;
  sd_attn_weights attn;
  const void *w_gate_up, *w_down;
  int32_t inter;
} sd_dense_layer_weights;

/* Bytes of workspace sd_dense_layer_step needs. */
size_t sd_dense_workspace_bytes(const sd_dims *dims, int32_t b, int32_t n_req,
                                int32_t max_seq_len, int32_t inter);

/* One dense draft layer on the fp32 stream [b, H] (in/out), in the order of [DSP]
 * MuseSparkDSparkDecoderLayer.forward: x = bf16(RMSNorm(bf16(stream); g_pre_attn));
 * attention as sd_attn_verify (K/V written at kv->slot_mapping); stream +=
 * RMSNorm(attention; g_post_attn); x = bf16(RMSNorm(bf16(stream); g_pre_ffn));
 * stream += RMSNorm(down(silu(gate(x)) * up(x)); g_post_ffn).  The bf16 casts are the
 * ones the forward spells out; the branches and the SwiGLU output stay near fp32. */
int sd_dense_layer_step(const sd_dims *dims, int32_t b, float *stream,
                        const sd_dense_layer_weights *w, const sd_kv *kv, void *ws,
                        size_t ws_bytes, void *stream_handle);

/* One layer of the context-K/V store: its pre-QKV norm gain fp32 [H], its packed w_qkv
 * (the K/V rows [Hq D, Hq D + 2 Hkv D) are the ones read), its caches (as sd_kv) and
 * num_blocks, and slot_mapping int64 [n_ctx] (a negative slot writes nothing). */
typedef struct sd_ctx_layer {
  const float *g_pre_attn;
  const void *w_qkv;
  void *k_cache, *v_cache;
  int32_t num_blocks;
  const int64_t *slot_mapping;
} sd_ctx_layer;

/* Bytes of workspace sd_context_kv needs. */
size_t sd_context_kv_workspace_bytes(const sd_dims *dims, int32_t n_ctx, int32_t n_layers);

/* Context-K/V store of n_layers draft layers ([DSP] _project_muse_context_kv,
 * precompute_and_store_context_kv): fc = bf16(RMSNorm(states; g_hidden)); per layer
 * x = bf16(RMSNorm(fc; g_pre_attn)), kv = bf16(x W_kv^T), K = bf16(weightless RMSNorm(K))
 * (when dims->qk_norm) then RoPE at positions, bf16 K and V written at the layer's slots.
 * states bf16 [n_ctx, H] (1 <= n_ctx <= 64); g_hidden fp32 [H]; layers: HOST array of
 * n_layers (1 .. 16) descriptors; positions int32 [n_ctx]. */
int sd_context_kv(const sd_dims *dims, int32_t n_ctx, int32_t n_layers, const void *states,
                  const float *g_hidden, const sd_ctx_layer *layers, const int32_t *positions,
                  void *ws, size_t ws_bytes, void *stream_handle);

/* Test entry: dequantise row-major block-scaled FP4 rows [n, k] exactly as the expert
 * kernels do, into out fp32 [n, k] (codes [n, k/2], scales [n, k/16], one gscale).
 * k % 32 == 0. */
int sd_debug_dequant(int32_t n, int32_t k, const uint8_t *codes, const uint8_t *scales,
                     float gscale, float *out, void *stream_handle);

/* Test entry: one wave (64 lanes) of the kernels' cross-lane exchanges on device arrays
 * x fp32 [64] and xi int32 [64] (lane l holds x[l], xi[l]).  out fp32 [10, 64]: rows 0-5
 * the value of lane l ^ 1, 2, 4, 8, 16, 32; row 6 the wave sum (butterfly over partners
 * 32, 16, .., 1, each step adding the partner's value); row 7 the wave maximum (the same
 * butterfly); rows 8 and 9 the sums over aligned groups of 8 and 32 lanes (partners 1, 2,
 * .. in that order).  out_i int32 [2, 64]: row 0 the inclusive prefix sum of xi, row 1
 * xi of lane l ^ 4.  Asynchronous on the stream. */
int sd_debug_lanes(const float *x, const int32_t *xi, float *out, int32_t *out_i,
                   void *stream_handle);

/* Measurement entry: one plain streaming read of bytes (> 0, a multiple of 16) at src
 * (16-byte aligned), each 16-byte piece loaded once with the non-temporal policy of the
 * step's weight and KV streams, each workgroup reading one contiguous part: the practical
 * HBM read ceiling the step is measured against.  sink: uint32
 * [sd_read_probe_sink_words()] scratch the kernel may write. */
int sd_debug_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream_handle);

/* Words of sink that sd_debug_read_probe needs. */
int32_t sd_read_probe_sink_words(void);

#ifdef __cplusplus
}
#endif
#endif /* SDVERIFY_H */
