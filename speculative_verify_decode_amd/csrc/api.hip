// C ABI of libsdverify.so: host-side validation, workspace layout and the launch order of
// one layer step.  Nothing here allocates, frees or synchronises; every call enqueues its
// kernels on the caller's stream and returns.
//
// The per-layer order is the one of page
// "vllm.models.muse_spark.nvidia.specialized_decode.runtime.decode", SpecializedDecode.run:
// input boundary -> attention -> attention boundary -> MoE.  Validation mirrors that page's
// and page "vllm.models.muse_spark.nvidia.specialized_decode.runtime"'s host-only checks
// (`unsupported`: the first failing reason, in words), before any launch.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "sd_common.h"

// Scratch of sd_layer_step_noalloc: device memory the library owns, one copy per GPU the
// library runs on, held until the process ends.  In host code this name is a host-side
// stand-in, not a device address: host code reaches the array only through the pointer
// hipGetSymbolAddress gives for the current device (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[SD_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err = "no error";

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err = "no error";
  return SD_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SD_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define SD_LAUNCH(expr, what)                          \
  do {                                                 \
    hipError_t e_ = (expr);                            \
    if (e_ != hipSuccess) return hip_fail(e_, what);   \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int kMaxRows = 64;
// K slices of the QKV and o_proj GEMMs inside a layer step: each writes this many fp32
// partials, which their consumers (the QKV epilogue, the attention boundary) sum in order.
constexpr int kDenseSplit = 4;

bool norm_width_ok(int H) {
  if (H <= 0 || H % 256) return false;
  switch (H / 256) {
    case 1: case 2: case 4: case 8: case 12: case 16: case 20: case 24: case 32: return true;
    default: return false;
  }
}

int check_dims(const sd_dims* d) {
  if (d == nullptr) return fail(SD_EINVAL, "dims is null");
  if (!norm_width_ok(d->hidden))
    return fail(SD_EUNSUPPORTED, "hidden %d (need 256 * {1,2,4,8,12,16,20,24,32})", d->hidden);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(SD_EUNSUPPORTED, "head_dim %d (need 64 or 128)", d->head_dim);
  if (d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->n_q_heads % d->n_kv_heads)
    return fail(SD_EINVAL, "n_q_heads %d must be a positive multiple of n_kv_heads %d",
                d->n_q_heads, d->n_kv_heads);
  if (d->q_rows != 8)
    return fail(SD_EUNSUPPORTED, "q_rows %d (verify steps are 1 + 7 tokens)", d->q_rows);
  const int qg = (d->n_q_heads / d->n_kv_heads) * d->q_rows;
  if (!((d->head_dim == 128 && (qg == 16 || qg == 32)) ||
        (d->head_dim == 64 && (qg == 16 || qg == 32 || qg == 64))))
    return fail(SD_EUNSUPPORTED, "query group %d per KV head at head_dim %d", qg, d->head_dim);
  if ((d->n_q_heads * d->head_dim) % 128)
    return fail(SD_EUNSUPPORTED, "n_q_heads * head_dim = %d (o_proj needs a multiple of 128)",
                d->n_q_heads * d->head_dim);
  if (d->block_size != 16)
    return fail(SD_EUNSUPPORTED, "KV cache block size %d (only 16)", d->block_size);
  if (d->n_experts < 1 || d->n_experts > 256)
    return fail(SD_EUNSUPPORTED, "n_experts %d (1..256)", d->n_experts);
  if (d->top_k < 1 || d->top_k > 8 || d->top_k > d->n_experts)
    return fail(SD_EUNSUPPORTED, "top_k %d (1..min(8, n_experts))", d->top_k);
  if (d->inter <= 0 || d->inter % 128)
    return fail(SD_EUNSUPPORTED, "inter %d (need a multiple of 128)", d->inter);
  if (!moe_shape_supported(d->hidden, d->inter))
    return fail(SD_EUNSUPPORTED,
                "expert GEMM split of hidden %d / inter %d (each must be 128 * n * ks with "
                "n <= 4, ks in {1, 2, 4, 8})",
                d->hidden, d->inter);
  if (d->qk_norm != 0 && d->qk_norm != 1) return fail(SD_EINVAL, "qk_norm %d", d->qk_norm);
  if (!(d->eps > 0.f)) return fail(SD_EINVAL, "eps must be > 0");
  if (!(d->rope_theta > 0.f)) return fail(SD_EINVAL, "rope_theta must be > 0");
  if (d->attn_scale < 0.f) return fail(SD_EINVAL, "attn_scale must be >= 0");
  return SD_OK;
}

int check_rows(const sd_dims* d, int b) {
  (void)d;
  if (b <= 0 || b > kMaxRows) return fail(SD_EUNSUPPORTED, "b = %d rows (1..%d)", b, kMaxRows);
  return SD_OK;
}

// requests that b rows can belong to when no KV metadata says (sizes the unused attention
// part of a workspace for the entry points without a KV cache)
int requests_of(const sd_dims* d, int b) { return (b + d->q_rows - 1) / d->q_rows; }

struct Ws {
  size_t x_a, x_a_lo, s1, qkv, part_acc, part_ml, o, o_lo, a, x_m, x_m_lo, x16,
      x16_lo, zpart, counter, ids, w, counts, offsets, slot_of, tos, active, h16, h16_lo, y, total;
};

size_t up(size_t v) { return (v + 255) & ~(size_t)255; }

Ws ws_layout(const sd_dims& d, int b, int n_req, int max_seq_len) {
  const AttnPlan p = attn_plan(d, n_req, max_seq_len, 0);
  const size_t n_chunks = attn_chunk_bound(d, n_req, max_seq_len);  // any window fits
  const size_t H = d.hidden, D = d.head_dim, Hq = d.n_q_heads, Hkv = d.n_kv_heads;
  const size_t E = d.n_experts, k = d.top_k, I = d.inter, B = b;
  const size_t N = (2 * Hq + 2 * Hkv) * D;
  const size_t parts = (size_t)n_req * Hkv * n_chunks;
  Ws w;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += up(bytes); return at; };
  w.x_a = take(B * H * 2);
  w.x_a_lo = take(B * H * 2);
  w.s1 = take(B * H * 4);
  w.qkv = take(kDenseSplit * B * N * 4);
  w.part_acc = take(parts * p.qg * D * 4);
  w.part_ml = take(parts * p.qg * 2 * 4);
  w.o = take(B * Hq * D * 2);
  w.o_lo = take(B * Hq * D * 2);
  w.a = take(kDenseSplit * B * H * 4);
  w.x_m = take(B * H * 2);
  w.x_m_lo = take(B * H * 2);
  w.x16 = take(B * H * 2);
  w.x16_lo = take(B * H * 2);
  w.zpart = take((H / 256) * B * E * 4);
  w.counter = take(4);
  w.ids = take(B * k * 4);
  w.w = take(B * k * 4);
  w.counts = take(E * 4);
  w.offsets = take((E + 1) * 4);
  w.slot_of = take(B * k * 4);
  w.tos = take(B * k * 4);
  w.active = take((E + 1) * 4);
  w.h16 = take(B * k * I * 2);
  w.h16_lo = take(B * k * I * 2);
  w.y = take(B * k * H * 4);
  w.total = o;
  return w;
}

template <typename T>
T* at(void* ws, size_t off) { return (T*)((char*)ws + off); }

int check_kv(const sd_dims* d, int b, const sd_kv* kv) {
  if (kv == nullptr) return fail(SD_EINVAL, "kv is null");
  if (!kv->k_cache || !kv->v_cache || !kv->block_table || !kv->seq_lens || !kv->positions ||
      !kv->slot_mapping)
    return fail(SD_EINVAL, "a kv pointer is null");
  if (!aligned16(kv->k_cache) || !aligned16(kv->v_cache))
    return fail(SD_EINVAL, "KV caches must be 16-byte aligned");
  if (kv->n_req <= 0) return fail(SD_EINVAL, "n_req %d", kv->n_req);
  if (kv->query_start == nullptr && kv->n_req * d->q_rows != b)
    return fail(SD_EUNSUPPORTED,
                "b = %d but n_req = %d requests of %d verify rows (without query_start a step "
                "verifies q_rows tokens of every request)",
                b, kv->n_req, d->q_rows);
  if (kv->query_start != nullptr && (b < kv->n_req || b > kv->n_req * d->q_rows))
    return fail(SD_EINVAL, "b = %d rows for %d requests of 1..%d verify rows", b, kv->n_req,
                d->q_rows);
  const int min_len = kv->query_start ? 1 : d->q_rows;  // a partial draft may verify one
  if (kv->max_seq_len < min_len)
    return fail(SD_EINVAL, "max_seq_len %d shorter than the %d verify tokens", kv->max_seq_len,
                min_len);
  if (kv->num_blocks <= 0) return fail(SD_EINVAL, "num_blocks %d", kv->num_blocks);
  if (kv->max_blocks * 16 < kv->max_seq_len)
    return fail(SD_EINVAL, "block table of %d blocks per request cannot hold %d tokens",
                kv->max_blocks, kv->max_seq_len);
  if (kv->window < 0) return fail(SD_EINVAL, "sliding window %d is negative", kv->window);
  return SD_OK;
}

int check_ws(const sd_dims* d, int b, int n_req, int max_seq_len, const void* ws,
             size_t ws_bytes) {
  const size_t need = ws_layout(*d, b, n_req, max_seq_len).total;
  if (ws == nullptr || ws_bytes < need)
    return fail(SD_EWORKSPACE, "workspace of %zu bytes, need %zu", ws ? ws_bytes : 0, need);
  if (!aligned16(ws)) return fail(SD_EINVAL, "workspace must be 16-byte aligned");
  return SD_OK;
}

float scale_of(const sd_dims* d) {
  return d->attn_scale > 0.f ? d->attn_scale : 1.0f / sqrtf((float)d->head_dim);
}

#define SD_CHECK(expr)        \
  do {                        \
    int rc_ = (expr);         \
    if (rc_ != SD_OK) return rc_; \
  } while (0)

// ---- launch sequences (validated arguments only) ----
// x (bf16 hi terms) and x_lo (bf16 lo terms after x in one buffer, may be null) -> out fp32
// [out_parts, b, H]: out_parts = 1 gives the attention output itself; more leaves K-slice
// partials of o_proj for a consumer that sums them.  Returns the partial count used.
int run_attention(const sd_dims* d, int b, const uint16_t* x, const uint16_t* x_lo,
                  const sd_attn_weights* w, const sd_kv* kv, float* out, int out_parts,
                  void* ws, const Ws& L, hipStream_t st, int* parts_used) {
  const int H = d->hidden, D = d->head_dim, Hq = d->n_q_heads, Hkv = d->n_kv_heads;
  const int N = (2 * Hq + 2 * Hkv) * D;
  const bool lo = x_lo != nullptr;
  float* qkv = at<float>(ws, L.qkv);
  GemmArgs g{};
  g.M = b; g.N = N; g.K = H; g.x = x; g.x_lo = x_lo; g.w = (const uint16_t*)w->w_qkv;
  g.y = qkv;
  g.ksplit = gemm_split_ok(b, N, H, lo, kDenseSplit) ? kDenseSplit : 1;
  SD_LAUNCH(launch_gemm(GEMM_F32, g, st), "qkv projection");
  const AttnPlan p = attn_plan(*d, kv->n_req, kv->max_seq_len, kv->window);
  if (p.n_chunks > attn_chunk_bound(*d, kv->n_req, kv->max_seq_len))
    return fail(SD_EHIP, "internal: attention plan of %d chunks exceeds the workspace's",
                p.n_chunks);
  AttnArgs aa{};
  aa.qkv = qkv; aa.nparts = g.ksplit; aa.part_stride = (size_t)b * N;
  aa.qk_norm = d->qk_norm; aa.eps = d->eps;
  for (int i = 0; i < D / 2; ++i) aa.freq[i] = pow((double)d->rope_theta, -2.0 * i / D);
  aa.slot_mapping = kv->slot_mapping;
  aa.k_cache = (uint16_t*)kv->k_cache; aa.v_cache = (uint16_t*)kv->v_cache;
  aa.block_table = kv->block_table; aa.max_blocks = kv->max_blocks; aa.seq_lens = kv->seq_lens;
  aa.num_blocks = kv->num_blocks;
  aa.positions = kv->positions; aa.n_req = kv->n_req; aa.Hq = Hq; aa.Hkv = Hkv; aa.D = D;
  aa.q_rows = d->q_rows; aa.window = kv->window; aa.scale = scale_of(d);
  aa.query_start = kv->query_start; aa.b = b;
  aa.part_acc = at<float>(ws, L.part_acc); aa.part_ml = at<float>(ws, L.part_ml);
  aa.gate = qkv + (size_t)(Hq + 2 * Hkv) * D; aa.gate_stride = N;  // the o_gate columns
  uint16_t* o = at<uint16_t>(ws, L.o);
  uint16_t* o_lo = at<uint16_t>(ws, L.o_lo);
  aa.out = o; aa.out_lo = o_lo;
  SD_LAUNCH(launch_attention(aa, p, st), "paged attention");
  GemmArgs go{};
  go.M = b; go.N = H; go.K = Hq * D; go.x = o; go.x_lo = o_lo; go.w = (const uint16_t*)w->w_o;
  go.y = out;
  go.ksplit = (out_parts > 1 && gemm_split_ok(b, H, Hq * D, true, out_parts)) ? out_parts : 1;
  SD_LAUNCH(launch_gemm(GEMM_F32, go, st), "o_proj");
  if (parts_used) *parts_used = go.ksplit;
  return SD_OK;
}

// The router kernel's arrival counter must be 0 at launch: in a layer step the attention
// boundary's norm kernel zeroes it; a standalone call zeroes it first.
RouterArgs router_args(const sd_dims* d, int b, const uint16_t* x, const uint16_t* x_lo,
                       const void* w_router, const float* bias, const sd_route* r, void* ws,
                       const Ws& L) {
  RouterArgs ra{};
  ra.b = b; ra.H = d->hidden; ra.E = d->n_experts; ra.k = d->top_k;
  ra.x = x; ra.x_lo = x_lo; ra.w = (const uint16_t*)w_router; ra.bias = bias;
  ra.part = at<float>(ws, L.zpart); ra.counter = at<int>(ws, L.counter); ra.logits = r->logits;
  ra.ids = r->topk_ids; ra.w_out = r->topk_w; ra.counts = r->expert_counts;
  ra.offsets = r->expert_offsets; ra.slot_of = r->slot_of; ra.tos = r->token_of_slot;
  ra.active = r->active_experts;
  return ra;
}

int run_route(const sd_dims* d, int b, const uint16_t* x, const uint16_t* x_lo,
              const void* w_router, const float* bias, const sd_route* r, void* ws,
              const Ws& L, hipStream_t st) {
  const RouterArgs ra = router_args(d, b, x, x_lo, w_router, bias, r, ws, L);
  SD_LAUNCH(launch_router(ra, st), "router, routing and pooler");
  return SD_OK;
}

// route (may be null): the router's logits and map outputs, routed inside the W13 kernel
int run_experts(const sd_dims* d, int b, const _Float16* x16, const _Float16* x16_lo,
                const sd_moe_weights* w, const sd_route* r, float* y, uint16_t* h_bf16,
                _Float16* h16, _Float16* h16_lo, hipStream_t st,
                const RouterArgs* route = nullptr) {
  MoeArgs m{};
  m.b = b; m.H = d->hidden; m.I = d->inter; m.E = d->n_experts; m.k = d->top_k;
  m.x16 = x16; m.x16_lo = x16_lo; m.h16_lo = h16_lo;
  m.w13_codes = w->w13_codes; m.w13_scales = w->w13_scales; m.w13_gscale = w->w13_gscale;
  m.w2_codes = w->w2_codes; m.w2_scales = w->w2_scales; m.w2_gscale = w->w2_gscale;
  m.counts = r->expert_counts; m.offsets = r->expert_offsets; m.tos = r->token_of_slot;
  m.active = r->active_experts;
  m.h16 = h16; m.h_bf16 = h_bf16; m.y = y;
  if (route != nullptr) {
    m.route = 1;
    m.r = *route;
  }
  SD_LAUNCH(launch_moe_experts(m, st), "routed experts");
  return SD_OK;
}

int check_attn_weights(const sd_attn_weights* w) {
  if (w == nullptr || !w->w_qkv || !w->w_o) return fail(SD_EINVAL, "attention weight is null");
  if (!aligned16(w->w_qkv) || !aligned16(w->w_o))
    return fail(SD_EINVAL, "attention weights must be 16-byte aligned");
  return SD_OK;
}

int check_moe_weights(const sd_moe_weights* w, bool need_router, bool need_experts) {
  if (w == nullptr) return fail(SD_EINVAL, "moe weights are null");
  if (need_router && (!w->w_router || !aligned16(w->w_router)))
    return fail(SD_EINVAL, "router weight null or not 16-byte aligned");
  if (need_experts) {
    if (!w->w13_codes || !w->w13_scales || !w->w13_gscale || !w->w2_codes || !w->w2_scales ||
        !w->w2_gscale)
      return fail(SD_EINVAL, "an expert weight pointer is null");
    if (!aligned16(w->w13_codes) || !aligned16(w->w2_codes))
      return fail(SD_EINVAL, "expert codes must be 16-byte aligned");
    if (((uintptr_t)w->w13_scales & 1u) || ((uintptr_t)w->w2_scales & 1u))
      return fail(SD_EINVAL, "expert scales must be 2-byte aligned");
  }
  return SD_OK;
}

int check_route(const sd_route* r) {
  if (r == nullptr || !r->topk_ids || !r->topk_w || !r->expert_counts || !r->expert_offsets ||
      !r->slot_of || !r->token_of_slot || !r->active_experts)
    return fail(SD_EINVAL, "a route pointer is null");
  return SD_OK;  // r->logits is optional
}

sd_route ws_route(void* ws, const Ws& L) {
  sd_route r;
  r.topk_ids = at<int32_t>(ws, L.ids);
  r.topk_w = at<float>(ws, L.w);
  r.expert_counts = at<int32_t>(ws, L.counts);
  r.expert_offsets = at<int32_t>(ws, L.offsets);
  r.slot_of = at<int32_t>(ws, L.slot_of);
  r.token_of_slot = at<int32_t>(ws, L.tos);
  r.active_experts = at<int32_t>(ws, L.active);
  r.logits = nullptr;
  return r;
}

// The current device's address of `scratch`, looked up once per device (with that device
// current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SD_EUNSUPPORTED, "device %d (the scratch table holds %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(SD_EHIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SD_OK;
}

}  // namespace

extern "C" {

int sd_abi_version(void) { return SD_ABI_VERSION; }

const char* sd_last_error(void) { return g_err.c_str(); }

size_t sd_packed_dense_bytes(int32_t n, int32_t k) {
  if (n <= 0 || k <= 0 || k % 32) return 0;
  return (size_t)((n + 15) / 16) * 16 * (size_t)k * 2;
}

int sd_pack_dense(int32_t n, int32_t k, const void* src, void* dst, void* stream_handle) {
  if (sd_packed_dense_bytes(n, k) == 0)
    return fail(SD_EINVAL, "dense weight [%d, %d] (need n, k > 0 and k %% 32 == 0)", n, k);
  if (!src || !dst || !aligned16(src) || !aligned16(dst))
    return fail(SD_EINVAL, "src/dst null or not 16-byte aligned");
  if (src == dst) return fail(SD_EINVAL, "packing is out of place");
  SD_LAUNCH(launch_pack_dense(n, k, (const uint16_t*)src, (uint16_t*)dst,
                              (hipStream_t)stream_handle),
            "dense weight packing");
  return ok();
}

int sd_pack_fp4(int32_t e, int32_t n, int32_t k, const uint8_t* codes, const uint8_t* scales,
                uint8_t* codes_out, uint8_t* scales_out, void* stream_handle) {
  if (e <= 0 || n <= 0 || k <= 0 || n % 16 || k % 128)
    return fail(SD_EINVAL, "fp4 weights [%d, %d, %d] (need n %% 16 == 0, k %% 128 == 0)", e, n,
                k);
  if (!codes || !scales || !codes_out || !scales_out)
    return fail(SD_EINVAL, "a packing pointer is null");
  if (!aligned16(codes) || !aligned16(codes_out) || ((uintptr_t)scales & 1u) ||
      ((uintptr_t)scales_out & 1u))
    return fail(SD_EINVAL, "codes must be 16-byte and scales 2-byte aligned");
  if (codes == codes_out || scales == scales_out) return fail(SD_EINVAL, "packing is out of place");
  SD_LAUNCH(launch_pack_fp4(e, n, k, codes, scales, codes_out, scales_out,
                            (hipStream_t)stream_handle),
            "fp4 weight packing");
  return ok();
}

size_t sd_workspace_bytes(const sd_dims* dims, int32_t b, int32_t n_req, int32_t max_seq_len) {
  if (check_dims(dims) != SD_OK || check_rows(dims, b) != SD_OK || n_req <= 0 ||
      max_seq_len <= 0)
    return 0;
  return ws_layout(*dims, b, n_req, max_seq_len).total;
}

int sd_boundary_dualnorm(const sd_dims* dims, int32_t b, float* stream, const float* branch,
                         const void* front_embed, const float* g_post, const float* g_pre,
                         void* out, void* out16, float* aux, void* stream_handle) {
  SD_CHECK(check_dims(dims));
  SD_CHECK(check_rows(dims, b));
  if (!stream || !out || !g_pre) return fail(SD_EINVAL, "stream, out or g_pre is null");
  if (branch == nullptr && front_embed == nullptr)
    return fail(SD_EINVAL, "front mode needs front_embed");
  if (branch != nullptr && g_post == nullptr) return fail(SD_EINVAL, "g_post is null");
  if (!aligned16(stream) || !aligned16(out) || (branch != nullptr && !aligned16(branch)) || !aligned16(g_pre) ||
      (g_post != nullptr && !aligned16(g_post)) || (out16 != nullptr && !aligned16(out16)) ||
      (aux != nullptr && !aligned16(aux)))
    return fail(SD_EINVAL, "stream, branch, gains, out16 and aux must be 16-byte aligned");
  _Float16* x16 = (_Float16*)out16;
  SD_LAUNCH(launch_dualnorm(b, dims->hidden, stream, stream, (const float*)branch, 1,
                            (const uint16_t*)front_embed, g_post, g_pre, dims->eps,
                            (uint16_t*)out, nullptr, x16,
                            x16 ? x16 + (size_t)b * dims->hidden : nullptr, nullptr, aux,
                            (hipStream_t)stream_handle),
            "dual norm");
  return ok();
}

int sd_attn_verify(const sd_dims* dims, int32_t b, const void* x, const sd_attn_weights* w,
                   const sd_kv* kv, float* out, void* ws, size_t ws_bytes, void* stream_handle) {
  SD_CHECK(check_dims(dims));
  SD_CHECK(check_rows(dims, b));
  SD_CHECK(check_attn_weights(w));
  SD_CHECK(check_kv(dims, b, kv));
  if (!x || !out || !aligned16(x) || !aligned16(out))
    return fail(SD_EINVAL, "x or out null or misaligned");
  SD_CHECK(check_ws(dims, b, kv->n_req, kv->max_seq_len, ws, ws_bytes));
  const Ws L = ws_layout(*dims, b, kv->n_req, kv->max_seq_len);
  SD_CHECK(run_attention(dims, b, (const uint16_t*)x, nullptr, w, kv, (float*)out, 1, ws, L,
                         (hipStream_t)stream_handle, nullptr));
  return ok();
}

int sd_moe_route(const sd_dims* dims, int32_t b, const void* x, const void* w_router,
                 const float* logit_bias, const sd_route* route, void* ws, size_t ws_bytes,
                 void* stream_handle) {
  SD_CHECK(check_dims(dims));
  SD_CHECK(check_rows(dims, b));
  SD_CHECK(check_route(route));
  if (!x || !aligned16(x) || !w_router || !aligned16(w_router))
    return fail(SD_EINVAL, "x or w_router null or misaligned");
  if (route->logits && !aligned16(route->logits)) return fail(SD_EINVAL, "route logits misaligned");
  SD_CHECK(check_ws(dims, b, requests_of(dims, b), dims->q_rows, ws, ws_bytes));
  const Ws L = ws_layout(*dims, b, requests_of(dims, b), dims->q_rows);
  hipStream_t st = (hipStream_t)stream_handle;
  SD_LAUNCH(launch_zero_i32(at<int>(ws, L.counter), st), "router counter");
  SD_CHECK(run_route(dims, b, (const uint16_t*)x, nullptr, w_router, logit_bias, route, ws, L,
                     st));
  return ok();
}

namespace {

// Shared checks of the two expert entry points; x names the input in messages.
int check_experts(const sd_dims* dims, int32_t b, const void* x, const sd_moe_weights* w,
                  const sd_route* route, void* y_slots, void* h_slots, void* ws,
                  size_t ws_bytes, const char* xname) {
  SD_CHECK(check_dims(dims));
  SD_CHECK(check_rows(dims, b));
  SD_CHECK(check_moe_weights(w, false, true));
  SD_CHECK(check_route(route));
  if (!x || !y_slots) return fail(SD_EINVAL, "%s or y_slots is null", xname);
  if (!aligned16(x) || !aligned16(y_slots) || (h_slots && !aligned16(h_slots)))
    return fail(SD_EINVAL, "%s, y_slots and h_slots must be 16-byte aligned", xname);
  return check_ws(dims, b, requests_of(dims, b), dims->q_rows, ws, ws_bytes);
}

}  // namespace

int sd_moe_experts(const sd_dims* dims, int32_t b, const void* x, const sd_moe_weights* w,
                   const sd_route* route, void* y_slots, void* h_slots, void* ws,
                   size_t ws_bytes, void* stream_handle) {
  SD_CHECK(check_experts(dims, b, x, w, route, y_slots, h_slots, ws, ws_bytes, "x"));
  const Ws L = ws_layout(*dims, b, requests_of(dims, b), dims->q_rows);
  hipStream_t st = (hipStream_t)stream_handle;
  _Float16* x16 = at<_Float16>(ws, L.x16);
  _Float16* x16_lo = at<_Float16>(ws, L.x16_lo);
  SD_LAUNCH(launch_expert_input(b, dims->hidden, (const uint16_t*)x, x16, x16_lo, st),
            "expert input");
  SD_CHECK(run_experts(dims, b, x16, x16_lo, w, route, (float*)y_slots, (uint16_t*)h_slots,
                       at<_Float16>(ws, L.h16), at<_Float16>(ws, L.h16_lo), st));
  return ok();
}

int sd_moe_experts_x16(const sd_dims* dims, int32_t b, const void* x16,
                       const sd_moe_weights* w, const sd_route* route, void* y_slots,
                       void* h_slots, void* ws, size_t ws_bytes, void* stream_handle) {
  SD_CHECK(check_experts(dims, b, x16, w, route, y_slots, h_slots, ws, ws_bytes, "x16"));
  const Ws L = ws_layout(*dims, b, requests_of(dims, b), dims->q_rows);
  const _Float16* hi = (const _Float16*)x16;
  SD_CHECK(run_experts(dims, b, hi, hi + (size_t)b * dims->hidden, w, route, (float*)y_slots,
                       (uint16_t*)h_slots, at<_Float16>(ws, L.h16), at<_Float16>(ws, L.h16_lo),
                       (hipStream_t)stream_handle));
  return ok();
}

int sd_moe_unpool(const sd_dims* dims, int32_t b, const float* y_slots, const sd_route* route,
                  float* out, void* stream_handle) {
  SD_CHECK(check_dims(dims));
  SD_CHECK(check_rows(dims, b));
  SD_CHECK(check_route(route));
  if (!y_slots || !out || !aligned16(y_slots) || !aligned16(out))
    return fail(SD_EINVAL, "y_slots or out null or misaligned");
  SD_LAUNCH(launch_unpool(b, dims->hidden, dims->top_k, (const float*)y_slots, route->topk_w,
                          route->slot_of, (float*)out, (hipStream_t)stream_handle),
            "unpooler");
  return ok();
}

namespace {

// The layer step.  Input: branch_in (fp32 [b, H]), or pool_in (the previous layer's pooled
// MoE output, gathered by the input boundary), or neither (the front, from front_embed).
// Output: branch_out (the unpooled branch), or pool_out (y_slots and the route, no unpool).
int layer_step_impl(const sd_dims* dims, int32_t b, float* stream, const float* branch_in,
                    const sd_pooled* pool_in, const void* front_embed, const sd_layer_weights* w,
                    const sd_kv* kv, const float* logit_bias, float* branch_out,
                    const sd_route* route_out, const sd_pooled* pool_out, float* aux, void* ws,
                    size_t ws_bytes, void* stream_handle) {
  SD_CHECK(check_dims(dims));
  SD_CHECK(check_rows(dims, b));
  if (w == nullptr) return fail(SD_EINVAL, "layer weights are null");
  if (!w->g_pre_attn || !w->g_post_attn || !w->g_pre_ffn)
    return fail(SD_EINVAL, "a layer gain is null");
  const bool has_in = branch_in != nullptr || pool_in != nullptr;
  if (has_in && !w->g_post_prev) return fail(SD_EINVAL, "g_post_prev is null");
  if (!has_in && front_embed == nullptr)
    return fail(SD_EINVAL, "the first layer's front needs front_embed");
  SD_CHECK(check_attn_weights(&w->attn));
  SD_CHECK(check_moe_weights(&w->moe, true, true));
  SD_CHECK(check_kv(dims, b, kv));
  if (!stream || (branch_in != nullptr && !aligned16(branch_in)))
    return fail(SD_EINVAL, "stream null, or branch_in misaligned");
  if (pool_out == nullptr && (!branch_out || !aligned16(branch_out)))
    return fail(SD_EINVAL, "branch_out null or misaligned");
  for (const sd_pooled* pp : {pool_in, pool_out}) {
    if (pp == nullptr) continue;
    if (!pp->y_slots || !aligned16(pp->y_slots) || !pp->route)
      return fail(SD_EINVAL, "a pooled branch has a null or misaligned y_slots, or no route");
    SD_CHECK(check_route(pp->route));
  }
  if (route_out) SD_CHECK(check_route(route_out));
  if (aux != nullptr && !aligned16(aux)) return fail(SD_EINVAL, "aux misaligned");
  const sd_route* rl = pool_out ? pool_out->route : route_out;
  if (rl != nullptr && rl->logits != nullptr && !aligned16(rl->logits))
    return fail(SD_EINVAL, "route logits misaligned");
  SD_CHECK(check_ws(dims, b, kv->n_req, kv->max_seq_len, ws, ws_bytes));
  const Ws L = ws_layout(*dims, b, kv->n_req, kv->max_seq_len);
  hipStream_t st = (hipStream_t)stream_handle;
  const int H = dims->hidden;
  uint16_t* x_a = at<uint16_t>(ws, L.x_a);
  uint16_t* x_a_lo = at<uint16_t>(ws, L.x_a_lo);
  // the stream after the input boundary: the attention boundary reads it here and writes the
  // caller's stream, so no kernel of the step updates a row that another workgroup still reads
  float* s1 = at<float>(ws, L.s1);
  if (pool_in != nullptr) {
    SD_LAUNCH(launch_dualnorm(b, H, stream, s1, pool_in->y_slots, 1, nullptr, w->g_post_prev,
                              w->g_pre_attn, dims->eps, x_a, x_a_lo, nullptr, nullptr,
                              at<int>(ws, L.counter), aux, st, pool_in->route->topk_w,
                              pool_in->route->slot_of, dims->top_k),
              "input boundary (gathering the pooled branch)");
  } else {
    SD_LAUNCH(launch_dualnorm(b, H, stream, s1, (const float*)branch_in, 1,
                              (const uint16_t*)front_embed, w->g_post_prev, w->g_pre_attn,
                              dims->eps, x_a, x_a_lo, nullptr, nullptr, at<int>(ws, L.counter),
                              aux, st),
              "input boundary");
  }
  float* a = at<float>(ws, L.a);
  int a_parts = 1;
  SD_CHECK(run_attention(dims, b, x_a, x_a_lo, &w->attn, kv, a, kDenseSplit, ws, L, st,
                         &a_parts));
  uint16_t* x_m = at<uint16_t>(ws, L.x_m);
  uint16_t* x_m_lo = at<uint16_t>(ws, L.x_m_lo);
  _Float16* x16 = at<_Float16>(ws, L.x16);
  _Float16* x16_lo = at<_Float16>(ws, L.x16_lo);
  const sd_route r = pool_out ? *pool_out->route : route_out ? *route_out : ws_route(ws, L);
  NormRouterArgs nr{};
  const RouterArgs* route_in_experts = nullptr;  // the expert kernel routes from the logits
  if (norm_router_parts(H, dims->n_experts, b, dims->top_k) > 0 && (a_parts == 1 || a_parts == 4)) {
    // attention boundary and the router's product in one launch
    nr.H = H; nr.branch = a; nr.branch_stride = (size_t)b * H; nr.stream_in = s1;
    nr.stream = stream;
    nr.g_post = w->g_post_attn; nr.g_pre = w->g_pre_ffn; nr.eps = dims->eps;
    nr.out = nullptr; nr.out_lo = nullptr;  // the bf16 row feeds only the router
    nr.x16 = x16; nr.x16_lo = x16_lo;
    nr.r = router_args(dims, b, nullptr, nullptr, w->moe.w_router, logit_bias, &r, ws, L);
    nr.r.part = at<float>(ws, L.zpart);
    SD_LAUNCH(launch_norm_router(nr, a_parts, st), "attention boundary and router");
    route_in_experts = &nr.r;
  } else {
    SD_LAUNCH(launch_dualnorm(b, H, s1, stream, a, a_parts, nullptr, w->g_post_attn, w->g_pre_ffn,
                              dims->eps, x_m, x_m_lo, x16, x16_lo, at<int>(ws, L.counter),
                              nullptr, st),
              "attention boundary");
    SD_CHECK(run_route(dims, b, x_m, x_m_lo, w->moe.w_router, logit_bias, &r, ws, L, st));
  }
  float* y = pool_out ? pool_out->y_slots : at<float>(ws, L.y);
  SD_CHECK(run_experts(dims, b, x16, x16_lo, &w->moe, &r, y, nullptr, at<_Float16>(ws, L.h16),
                       at<_Float16>(ws, L.h16_lo), st, route_in_experts));
  if (pool_out == nullptr)
    SD_LAUNCH(launch_unpool(b, H, dims->top_k, y, r.topk_w, r.slot_of, (float*)branch_out, st),
              "unpooler");
  return ok();
}

}  // namespace

int sd_layer_step(const sd_dims* dims, int32_t b, float* stream, const float* branch_in,
                  const void* front_embed, const sd_layer_weights* w, const sd_kv* kv,
                  const float* logit_bias, float* branch_out, const sd_route* route_out,
                  float* aux, void* ws, size_t ws_bytes, void* stream_handle) {
  return layer_step_impl(dims, b, stream, branch_in, nullptr, front_embed, w, kv, logit_bias,
                         branch_out, route_out, nullptr, aux, ws, ws_bytes, stream_handle);
}

int sd_layer_step_pooled(const sd_dims* dims, int32_t b, float* stream,
                         const sd_pooled* branch_in, const void* front_embed,
                         const sd_layer_weights* w, const sd_kv* kv, const float* logit_bias,
                         const sd_pooled* branch_out, float* aux, void* ws, size_t ws_bytes,
                         void* stream_handle) {
  if (branch_out == nullptr) return fail(SD_EINVAL, "branch_out is null");
  return layer_step_impl(dims, b, stream, nullptr, branch_in, front_embed, w, kv, logit_bias,
                         nullptr, nullptr, branch_out, aux, ws, ws_bytes, stream_handle);
}

size_t sd_noalloc_scratch_bytes(void) { return SD_NOALLOC_SCRATCH_BYTES; }

int sd_layer_step_noalloc(const sd_dims* dims, int32_t b, float* stream, const float* branch_in,
                          const void* front_embed, const sd_layer_weights* w, const sd_kv* kv,
                          const float* logit_bias, float* branch_out, const sd_route* route_out,
                          float* aux, void* stream_handle) {
  // host-only checks first: nothing touches the device before the size is known to fit
  SD_CHECK(check_dims(dims));
  SD_CHECK(check_rows(dims, b));
  SD_CHECK(check_kv(dims, b, kv));
  const size_t need = ws_layout(*dims, b, kv->n_req, kv->max_seq_len).total;
  if (need > (size_t)SD_NOALLOC_SCRATCH_BYTES)
    return fail(SD_EWORKSPACE,
                "this step needs %zu bytes of scratch; the library's static scratch holds %zu "
                "(use sd_layer_step with a workspace)",
                need, (size_t)SD_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  SD_CHECK(scratch_ptr(&ws));
  // Every region the step reads is written earlier in the same call (the one counter a
  // kernel needs is zeroed by a preceding kernel), so the previous call's contents never
  // reach the result; nothing is cleared with a memset.
  return layer_step_impl(dims, b, stream, branch_in, nullptr, front_embed, w, kv, logit_bias,
                         branch_out, route_out, nullptr, aux, ws, need, stream_handle);
}

// ------------------------------------------------------------------------ draft side
namespace {

struct DenseWs {
  Ws L;  // the attention regions of the layer step
  size_t x_f, gu, h, h_lo, y, total;
};

DenseWs dense_layout(const sd_dims& d, int b, int n_req, int max_seq_len, int inter) {
  DenseWs w;
  w.L = ws_layout(d, b, n_req, max_seq_len);
  size_t o = w.L.total;
  auto take = [&](size_t bytes) { size_t at = o; o += up(bytes); return at; };
  const size_t B = b, H = d.hidden, I = inter;
  w.x_f = take(B * H * 2);
  w.gu = take(kDenseSplit * B * 2 * I * 4);
  w.h = take(B * I * 2);     // bf16 hi terms of h, then
  w.h_lo = take(B * I * 2);  // its lo terms, one buffer for the down projection
  w.y = take(kDenseSplit * B * H * 4);
  w.total = o;
  return w;
}

int ctx_parts(const sd_dims& d, int n) {
  const int N = 2 * d.n_kv_heads * d.head_dim;
  return gemm_split_ok(n, N, d.hidden, false, kDenseSplit) ? kDenseSplit : 1;
}

}  // namespace

size_t sd_dense_workspace_bytes(const sd_dims* dims, int32_t b, int32_t n_req,
                                int32_t max_seq_len, int32_t inter) {
  if (dims == nullptr || b <= 0 || n_req <= 0 || max_seq_len <= 0 || inter <= 0) return 0;
  return dense_layout(*dims, b, n_req, max_seq_len, inter).total;
}

int sd_dense_layer_step(const sd_dims* dims, int32_t b, float* stream,
                        const sd_dense_layer_weights* w, const sd_kv* kv, void* ws,
                        size_t ws_bytes, void* stream_handle) {
  SD_CHECK(check_dims(dims));
  SD_CHECK(check_rows(dims, b));
  if (w == nullptr) return fail(SD_EINVAL, "dense layer weights are null");
  if (!w->g_pre_attn || !w->g_post_attn || !w->g_pre_ffn || !w->g_post_ffn)
    return fail(SD_EINVAL, "a dense layer gain is null");
  SD_CHECK(check_attn_weights(&w->attn));
  if (!w->w_gate_up || !w->w_down || !aligned16(w->w_gate_up) || !aligned16(w->w_down))
    return fail(SD_EINVAL, "w_gate_up or w_down null or misaligned");
  if (w->inter <= 0 || w->inter % 128)
    return fail(SD_EUNSUPPORTED, "dense inter %d (need a positive multiple of 128)", w->inter);
  SD_CHECK(check_kv(dims, b, kv));
  if (!stream || !aligned16(stream)) return fail(SD_EINVAL, "stream null or misaligned");
  const size_t need = sd_dense_workspace_bytes(dims, b, kv->n_req, kv->max_seq_len, w->inter);
  if (ws == nullptr || ws_bytes < need)
    return fail(SD_EWORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
  if (!aligned16(ws)) return fail(SD_EINVAL, "workspace must be 16-byte aligned");
  const DenseWs D = dense_layout(*dims, b, kv->n_req, kv->max_seq_len, w->inter);
  hipStream_t st = (hipStream_t)stream_handle;
  const int H = dims->hidden, I = w->inter;
  const float eps = dims->eps;
  uint16_t* x_a = at<uint16_t>(ws, D.L.x_a);
  SD_LAUNCH(launch_draft_norm(0, b, H, stream, nullptr, 1, nullptr, w->g_pre_attn, eps, x_a, st),
            "dense layer input norm");
  float* a = at<float>(ws, D.L.a);
  int a_parts = 1;
  SD_CHECK(run_attention(dims, b, x_a, nullptr, &w->attn, kv, a, kDenseSplit, ws, D.L, st,
                         &a_parts));
  uint16_t* x_f = at<uint16_t>(ws, D.x_f);
  SD_LAUNCH(launch_draft_norm(1, b, H, stream, a, a_parts, w->g_post_attn, w->g_pre_ffn, eps,
                              x_f, st),
            "dense layer attention boundary");
  uint16_t* h = at<uint16_t>(ws, D.h);
  uint16_t* h_lo = at<uint16_t>(ws, D.h_lo);
  GemmArgs g{};
  g.M = b; g.N = 2 * I; g.K = H; g.x = x_f; g.x_lo = nullptr;
  g.w = (const uint16_t*)w->w_gate_up;
  if (gemm_swiglu_ok(b, 2 * I, H, false)) {
    // one K slice: each workgroup finishes a gate tile and then its up tile, and the SwiGLU
    // runs in the projection's epilogue
    g.y = h; g.y_lo = h_lo; g.ksplit = 1;
    SD_LAUNCH(launch_gemm(GEMM_SWIGLU, g, st), "gate_up projection with SwiGLU");
  } else {
    g.y = at<float>(ws, D.gu);
    g.ksplit = gemm_split_ok(b, 2 * I, H, false, kDenseSplit) ? kDenseSplit : 1;
    SD_LAUNCH(launch_gemm(GEMM_F32, g, st), "gate_up projection");
    SD_LAUNCH(launch_swiglu_dense(b, I, at<float>(ws, D.gu), g.ksplit, h, h_lo, st), "SwiGLU");
  }
  GemmArgs gd{};
  gd.M = b; gd.N = H; gd.K = I; gd.x = h; gd.x_lo = h_lo;
  gd.w = (const uint16_t*)w->w_down; gd.y = at<float>(ws, D.y);
  gd.ksplit = gemm_split_ok(b, H, I, true, kDenseSplit) ? kDenseSplit : 1;
  SD_LAUNCH(launch_gemm(GEMM_F32, gd, st), "down projection");
  SD_LAUNCH(launch_draft_norm(2, b, H, stream, at<float>(ws, D.y), gd.ksplit, w->g_post_ffn,
                              nullptr, eps, nullptr, st),
            "dense layer output add");
  return ok();
}

size_t sd_context_kv_workspace_bytes(const sd_dims* dims, int32_t n_ctx, int32_t n_layers) {
  if (dims == nullptr || n_ctx <= 0 || n_ctx > 64 || n_layers <= 0 || n_layers > kMaxCtxLayers)
    return 0;
  const size_t H = dims->hidden, N = 2 * (size_t)dims->n_kv_heads * dims->head_dim;
  const size_t parts = ctx_parts(*dims, n_ctx);
  return up((size_t)n_layers * n_ctx * H * 2) + up((size_t)n_layers * parts * n_ctx * N * 4);
}

int sd_context_kv(const sd_dims* dims, int32_t n_ctx, int32_t n_layers, const void* states,
                  const float* g_hidden, const sd_ctx_layer* layers, const int32_t* positions,
                  void* ws, size_t ws_bytes, void* stream_handle) {
  SD_CHECK(check_dims(dims));
  if (n_ctx < 1 || n_ctx > 64) return fail(SD_EUNSUPPORTED, "n_ctx %d (need 1 .. 64)", n_ctx);
  if (n_layers < 1 || n_layers > kMaxCtxLayers)
    return fail(SD_EUNSUPPORTED, "n_layers %d (need 1 .. %d)", n_layers, kMaxCtxLayers);
  if (!states || !g_hidden || !layers || !positions)
    return fail(SD_EINVAL, "states, g_hidden, layers or positions is null");
  if (!aligned16(states)) return fail(SD_EINVAL, "states must be 16-byte aligned");
  CtxPtrs P{};
  for (int l = 0; l < n_layers; ++l) {
    const sd_ctx_layer& c = layers[l];
    if (!c.g_pre_attn || !c.w_qkv || !c.k_cache || !c.v_cache || !c.slot_mapping)
      return fail(SD_EINVAL, "a pointer of context layer %d is null", l);
    if (!aligned16(c.w_qkv) || !aligned16(c.k_cache) || !aligned16(c.v_cache))
      return fail(SD_EINVAL, "context layer %d: weights or caches misaligned", l);
    if (c.num_blocks <= 0) return fail(SD_EINVAL, "context layer %d: num_blocks %d", l, c.num_blocks);
    P.g_pre[l] = c.g_pre_attn;
    P.k_cache[l] = (uint16_t*)c.k_cache;
    P.v_cache[l] = (uint16_t*)c.v_cache;
    P.slots[l] = c.slot_mapping;
  }
  const size_t need = sd_context_kv_workspace_bytes(dims, n_ctx, n_layers);
  if (ws == nullptr || ws_bytes < need)
    return fail(SD_EWORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
  if (!aligned16(ws)) return fail(SD_EINVAL, "workspace must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream_handle;
  const int H = dims->hidden, Hq = dims->n_q_heads, Hkv = dims->n_kv_heads, D = dims->head_dim;
  const int N = 2 * Hkv * D, parts = ctx_parts(*dims, n_ctx);
  uint16_t* x = (uint16_t*)ws;
  float* kv = at<float>(ws, up((size_t)n_layers * n_ctx * H * 2));
  const size_t layer_stride = (size_t)parts * n_ctx * N;
  SD_LAUNCH(launch_ctx_norm(n_ctx, n_layers, H, (const uint16_t*)states, g_hidden, P, dims->eps,
                            x, st),
            "context norms");
  for (int l = 0; l < n_layers; ++l) {
    GemmArgs g{};
    g.M = n_ctx; g.N = N; g.K = H; g.x = x + (size_t)l * n_ctx * H; g.x_lo = nullptr;
    // the packed K/V rows start at row Hq D: tiles of 16 rows keep them contiguous
    g.w = (const uint16_t*)layers[l].w_qkv + (size_t)Hq * D * H;
    g.y = kv + l * layer_stride;
    g.ksplit = parts;
    SD_LAUNCH(launch_gemm(GEMM_F32, g, st), "context K/V projection");
  }
  SD_LAUNCH(launch_ctx_kv_post(kv, layer_stride, parts, n_ctx, n_layers, Hkv, D, dims->qk_norm,
                               dims->eps, dims->rope_theta, positions, P, st),
            "context K/V norm, RoPE and store");
  return ok();
}

size_t sd_draft_head_workspace_bytes(int32_t hidden, int32_t draft_vocab, int32_t b) {
  if (hidden <= 0 || draft_vocab <= 0 || b <= 0) return 0;
  const size_t tiles = (size_t)draft_vocab / 16;
  return up((size_t)b * tiles * 4) * 2;
}

int sd_draft_head(int32_t hidden, int32_t draft_vocab, int32_t b, const void* h,
                  const void* w_lm, float multiplier, float soft_cap, const int64_t* d2t,
                  float* tau_out, int32_t* draft_ids, int64_t* target_ids, void* ws,
                  size_t ws_bytes, void* stream_handle) {
  if (hidden <= 0 || hidden % 128)
    return fail(SD_EUNSUPPORTED, "hidden %d (need a multiple of 128)", hidden);
  if (draft_vocab <= 0 || draft_vocab % 16)
    return fail(SD_EUNSUPPORTED, "draft_vocab %d (need a multiple of 16)", draft_vocab);
  if (b <= 0 || b > kMaxRows) return fail(SD_EUNSUPPORTED, "b = %d rows (1..%d)", b, kMaxRows);
  if (!(multiplier > 0.f))
    return fail(SD_EINVAL, "multiplier must be > 0 (the transform must keep the argmax)");
  if (!h || !w_lm || !d2t || !draft_ids || !target_ids)
    return fail(SD_EINVAL, "a draft head pointer is null");
  if (!aligned16(h) || !aligned16(w_lm) || (tau_out && !aligned16(tau_out)))
    return fail(SD_EINVAL, "h, w_lm and tau_out must be 16-byte aligned");
  const size_t need = sd_draft_head_workspace_bytes(hidden, draft_vocab, b);
  if (ws == nullptr || ws_bytes < need)
    return fail(SD_EWORKSPACE, "workspace of %zu bytes, need %zu", ws ? ws_bytes : 0, need);
  hipStream_t st = (hipStream_t)stream_handle;
  const int tiles = draft_vocab / 16;
  float* val = (float*)ws;
  int* idx = (int*)((char*)ws + up((size_t)b * tiles * 4));
  GemmArgs g{};
  g.M = b; g.N = draft_vocab; g.K = hidden; g.x = (const uint16_t*)h; g.ksplit = 1;
  g.w = (const uint16_t*)w_lm; g.y = tau_out; g.head_val = val; g.head_idx = idx;
  g.multiplier = multiplier; g.soft_cap = soft_cap;
  SD_LAUNCH(launch_gemm(GEMM_HEAD, g, st), "lm_head");
  SD_LAUNCH(launch_head_argmax(b, tiles, val, idx, d2t, draft_ids, target_ids, st),
            "draft argmax");
  return ok();
}

int sd_debug_dequant(int32_t n, int32_t k, const uint8_t* codes, const uint8_t* scales,
                     float gscale, float* out, void* stream_handle) {
  if (n <= 0 || k <= 0 || k % 32) return fail(SD_EINVAL, "n %d, k %d (k % 32 == 0)", n, k);
  if (!codes || !scales || !out || !aligned16(codes) || ((uintptr_t)scales & 1u))
    return fail(SD_EINVAL, "codes/scales/out null or misaligned");
  SD_LAUNCH(launch_debug_dequant(n, k, codes, scales, gscale, out, (hipStream_t)stream_handle),
            "debug dequant");
  return ok();
}

int sd_debug_lanes(const float* x, const int32_t* xi, float* out, int32_t* out_i,
                   void* stream_handle) {
  if (!x || !xi || !out || !out_i) return fail(SD_EINVAL, "debug lanes: null pointer");
  SD_LAUNCH(launch_debug_lanes(x, xi, out, out_i, (hipStream_t)stream_handle), "debug lanes");
  return ok();
}

namespace {
constexpr int kProbeGrid = 8192;  // 32 workgroups per CU of a 256-CU device
}  // namespace

int32_t sd_read_probe_sink_words(void) { return kProbeGrid; }

int sd_debug_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream_handle) {
  if (!src || !sink || !aligned16(src) || bytes == 0 || bytes % 16)
    return fail(SD_EINVAL, "read probe: src/sink null, src misaligned or bytes %zu not a "
                "positive multiple of 16", bytes);
  SD_LAUNCH(launch_read_probe(src, bytes, sink, kProbeGrid, (hipStream_t)stream_handle),
            "read probe");
  return ok();
}

}  // extern "C"
