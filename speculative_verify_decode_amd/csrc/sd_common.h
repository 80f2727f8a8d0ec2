// Internal declarations shared by the gfx950 kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdverify.h"

// Bytes of the static scratch array of sd_layer_step_noalloc (one per GPU).
#define SD_NOALLOC_SCRATCH_BYTES (32u << 20)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Precision.  The stream and the branches between blocks are fp32.  An activation that
// feeds a matrix-core reduction enters as two 16-bit terms, x ~ hi + lo: bf16 hi/lo
// (~2^-16 relative) against bf16 weights, and fp16 hi/lo of x * 2^-8 (~2^-22 relative, an
// absolute floor of 2^-16 below |x| = 2^-6) against the exactly dequantised fp16 expert
// weights.  With at most 8 rows per MFMA column tile, columns 0-7 carry the hi terms and
// columns 8-15 the lo terms of the same rows, and the epilogue adds the two columns (lanes
// l and l ^ 8); attention runs its hi and lo operands as separate MFMAs.  Expert results
// are multiplied back by 2^8 (exact in fp32).  Only the KV cache and the draft-head logits
// are rounded to 16 bits, as the format fixes them.
#define SD_X16_SCALE 0.00390625f
#define SD_X16_UNSCALE 256.0f

namespace sd {

// Buffer resource over [p, p + bytes): loads at offsets past `bytes` return 0 and touch no
// memory (the range check), so an out-of-range offset is a load with no traffic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
constexpr uint32_t kOob = 0x80000000u;  // a byte offset past every buffer the kernels read
// Weights and K/V are read once per step: non-temporal loads (cache policy bit 1) stream
// them without displacing reusable lines, which measurably raises the achieved HBM rate.
constexpr int kStream = 2;

// VW consecutive 16-bit values as one store (VW = 1, 2 or 4).
template <int VW>
__device__ __forceinline__ void store16(uint16_t* p, const uint16_t* v) {
  if constexpr (VW == 4) {
    *(u32x2_t*)p = u32x2_t{v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16)};
  } else if constexpr (VW == 2) {
    *(uint32_t*)p = v[0] | ((uint32_t)v[1] << 16);
  } else {
    *p = v[0];
  }
}

// fp32 vector of VW lanes (VW = 1, 2 or 4).
template <int VW>
struct VecF;
template <> struct VecF<1> { typedef float T; };
template <> struct VecF<2> { typedef f32x2_t T; };
template <> struct VecF<4> { typedef f32x4_t T; };

__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// fp32 -> (hi, lo) fp16 terms of x * 2^-8.
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  const float xs = x * SD_X16_SCALE;
  hi = (_Float16)xs;
  lo = (_Float16)(xs - (float)hi);
}

// fp32 -> (hi, lo) bf16 terms: x ~ hi + lo to ~2^-16 relative.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

// The 32-bit value of lane (lane ^ O) of the wave, O a power of two below 64, without a
// round trip through the LDS crossbar: DPP within rows of 16 lanes (quad permutes for 1
// and 2; for 4, row shifts by 4 into the banks of lanes 0-3 and 8-11 and out of the others;
// for 8, a row rotate by 8) and the gfx950 permlane swaps across rows (each returns the
// lower and the upper row of the pair).  Every lane of the wave must be active.
template <int O, class T>
__device__ __forceinline__ T lane_xor(T v) {
  static_assert(sizeof(T) == 4, "32-bit values");
  const int x = __builtin_bit_cast(int, v);
  int r;
  if constexpr (O == 1) {
    r = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
  } else if constexpr (O == 2) {
    r = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
  } else if constexpr (O == 4) {
    r = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xf, 0x5, false);  // row_shl:4, banks 0, 2
    r = __builtin_amdgcn_update_dpp(r, x, 0x114, 0xf, 0xa, false);  // row_shr:4, banks 1, 3
  } else if constexpr (O == 8) {
    r = __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false);  // row_ror:8
  } else if constexpr (O == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    r = (threadIdx.x & 16) ? p[0] : p[1];
  } else {
    static_assert(O == 32, "lane offsets 1 .. 32");
    const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    r = (threadIdx.x & 32) ? p[0] : p[1];
  }
  return __builtin_bit_cast(T, r);
}

// Butterfly over the wave, partners 32, 16, .., 1 in that order: every lane gets the same
// bits.
__device__ __forceinline__ float wave_sum(float v) {
  v += lane_xor<32>(v);
  v += lane_xor<16>(v);
  v += lane_xor<8>(v);
  v += lane_xor<4>(v);
  v += lane_xor<2>(v);
  v += lane_xor<1>(v);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, lane_xor<32>(v));
  v = fmaxf(v, lane_xor<16>(v));
  v = fmaxf(v, lane_xor<8>(v));
  v = fmaxf(v, lane_xor<4>(v));
  v = fmaxf(v, lane_xor<2>(v));
  v = fmaxf(v, lane_xor<1>(v));
  return v;
}

// Sum over aligned groups of N lanes (N = 2 .. 64), partners 1, 2, .., N / 2 in that order.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N > 1) v += lane_xor<1>(v);
  if constexpr (N > 2) v += lane_xor<2>(v);
  if constexpr (N > 4) v += lane_xor<4>(v);
  if constexpr (N > 8) v += lane_xor<8>(v);
  if constexpr (N > 16) v += lane_xor<16>(v);
  if constexpr (N > 32) v += lane_xor<32>(v);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within each row of 16 lanes
// (DPP row_shr 1, 2, 4, 8; a lane with no source adds 0), then each row adds the totals
// of the rows before it, read from lanes 15, 31 and 47.  Every lane of the wave must be
// active.
__device__ __forceinline__ int wave_scan_incl(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Sum over a block of NW waves; `red` holds NW floats of LDS.  All threads get the sum.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) s += red[i];
  __syncthreads();
  return s;
}

// Eight E2M1 codes (one dword, low nibble first) -> eight fp16 weights w = e2m1 * scale.
// The hardware convert applies only the exponent of its scale operand, so it runs at
// scale 1 (exact E2M1 values) and the E4M3 block scale is a packed fp16 multiply.  The
// product of an E2M1 value (<= 2 significant bits) and an E4M3 value (<= 4 significant
// bits, 2^-9 .. 448) is exact in fp16, so each weight is the exact dequantised value.
// `scale2` holds the block's scale in both halves; written as a broadcast of one half of
// a pair, the multiply reads it through the packed op's half selectors, at no cost.
__device__ __forceinline__ f16x8_t dequant8(uint32_t codes, f16x2_t scale2) {
  f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0);
  f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1);
  f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2);
  f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3);
  p0 *= scale2;
  p1 *= scale2;
  p2 *= scale2;
  p3 *= scale2;
  f16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// A 32-weight unit: 16 bytes of codes + 2 scale bytes -> four MFMA A/B operands of 8 fp16
// (operand m holds weights 8m .. 8m+7 of the unit).  Both E4M3 scales decode in one
// packed convert (exact: every finite E4M3 value is an fp16 value).
__device__ __forceinline__ void dequant_unit(u32x4_t codes, uint32_t scales2, f16x8_t out[4]) {
  const f16x2_t s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scales2, 1.0f, false);
  const f16x2_t s0 = __builtin_shufflevector(s, s, 0, 0);
  const f16x2_t s1 = __builtin_shufflevector(s, s, 1, 1);
  out[0] = dequant8(codes[0], s0);
  out[1] = dequant8(codes[1], s0);
  out[2] = dequant8(codes[2], s1);
  out[3] = dequant8(codes[3], s1);
}

}  // namespace sd

// Workgroups are dispatched round-robin over the chip's 8 XCDs (workgroup w on XCD w % 8),
// and each XCD has its own L2.  xcd_rank(w, G) renumbers the G workgroups XCD by XCD (the
// first XCD's workgroups first, in dispatch order), so that workgroups given neighbouring
// ranks share an L2 and data they both read is fetched into it once.
__device__ __forceinline__ int xcd_rank(int w, int G) {
  const int x = w & 7, l = w >> 3;
  // XCD x' holds (G - x' + 7) / 8 workgroups; those of XCDs below x come first
  return x * (G >> 3) + min(x, G & 7) + l;
}

// ---------------------------------------------------------------------------- launches
// Every launcher enqueues on `st` and returns the launch status (hipGetLastError).

// branch: fp32 [nbranch, b, H], nbranch partials summed in order (null: front mode, the
// stream becomes the bf16 `front` rows).
// out: bf16 pre-norm output (hi term); out_lo (optional): its bf16 lo term; x16 / x16_lo
// (optional): fp16 hi / lo terms of the pre-norm output * 2^-8 (the expert input).
// zero (optional): an int set to 0, for a later kernel's arrival counter.
// aux (optional): fp32 [b, H] copy of the updated stream (the aux hidden-state tap).
// stream_out: the updated stream (may be `stream` itself).
// pool_slot (optional): the branch is pooled, branch = y [b * pool_k, H], row t gathered
// as sum over j of pool_w[t, j] * y[pool_slot[t, j]] (nbranch must be 1).
hipError_t launch_dualnorm(int b, int H, const float* stream, float* stream_out,
                           const float* branch, int nbranch,
                           const uint16_t* front, const float* g_post, const float* g_pre,
                           float eps, uint16_t* out, uint16_t* out_lo, _Float16* x16,
                           _Float16* x16_lo, int* zero, float* aux, hipStream_t st,
                           const float* pool_w = nullptr, const int* pool_slot = nullptr,
                           int pool_k = 0);
// x16 / x16_lo = fp16 hi / lo terms of x * 2^-8 for bf16 x [b, H] (the expert GEMMs' input)
hipError_t launch_expert_input(int b, int H, const uint16_t* x, _Float16* x16, _Float16* x16_lo,
                               hipStream_t st);

// GEMM_SWIGLU: W = [gate (N/2 rows); up (N/2 rows)], one K slice; y receives the bf16 hi
// terms of silu(gate) * up [M, N/2] and y_lo their lo terms (N/2 a multiple of 16).
enum GemmMode { GEMM_F32 = 0, GEMM_F32_BIAS = 2, GEMM_HEAD = 3, GEMM_SWIGLU = 4 };

struct GemmArgs {
  int M, N, K;
  const uint16_t* x;   // bf16 [M, K]
  const uint16_t* x_lo; // optional bf16 lo terms of x [M, K], after x in one buffer
  int ksplit;          // K slices: y holds ksplit partials [ksplit, M, N] (1: one output)
  uint32_t x_lo_off;   // set by the launcher
  const uint16_t* w;   // bf16 [N, K] in packed 16 x 32 tiles
  void* y;             // fp32 [M, N] (GEMM_HEAD: optional fp32 tau)
  const float* bias;   // [M, N] for GEMM_F32_BIAS (may be null)
  float* head_val;     // GEMM_HEAD: per (m, tile) best logit
  int* head_idx;       // GEMM_HEAD: per (m, tile) its index
  float multiplier, soft_cap;
  uint16_t* y_lo;      // GEMM_SWIGLU: the lo terms
};
// ksplit > 1 is taken only by the persistent kernel (M <= 64, shapes whose resident
// activations fit: gemm_split_ok says which); otherwise the launch fails with
// hipErrorInvalidValue.
hipError_t launch_gemm(GemmMode mode, const GemmArgs& a, hipStream_t st);
bool gemm_split_ok(int M, int N, int K, bool lo, int ksplit);
bool gemm_swiglu_ok(int M, int N, int K, bool lo);  // GEMM_SWIGLU serves the shape


// Weight packing (layouts in sdverify.h).
hipError_t launch_pack_dense(int N, int K, const uint16_t* src, uint16_t* dst, hipStream_t st);
hipError_t launch_pack_fp4(int E, int N, int K, const uint8_t* codes, const uint8_t* scales,
                           uint8_t* codes_out, uint8_t* scales_out, hipStream_t st);

// ---- draft side (k_draft.hip)
// mode 0: out = bf16(RMSNorm(bf16(stream); g_pre)); 1: stream += RMSNorm(sum of nbranch
// branch partials; g_post), then as 0; 2: only the stream update.
hipError_t launch_draft_norm(int mode, int b, int H, float* stream, const float* branch,
                             int nbranch, const float* g_post, const float* g_pre, float eps,
                             uint16_t* out, hipStream_t st);
// h = silu(g) * u from nparts partials of [g | u] [nparts, b, 2I]; bf16 hi / lo terms out
hipError_t launch_swiglu_dense(int b, int I, const float* gu, int nparts, uint16_t* h,
                               uint16_t* h_lo, hipStream_t st);
constexpr int kMaxCtxLayers = 16;
struct CtxPtrs {  // per-layer pointers of the context-K/V store, passed by value
  const float* g_pre[kMaxCtxLayers];
  uint16_t* k_cache[kMaxCtxLayers];
  uint16_t* v_cache[kMaxCtxLayers];
  const int64_t* slots[kMaxCtxLayers];
};
// x [L, n, H] bf16 = each layer's pre-norm of the bf16 hidden norm of the context rows
hipError_t launch_ctx_norm(int n, int L, int H, const uint16_t* states, const float* g_hidden,
                           const CtxPtrs& P, float eps, uint16_t* x, hipStream_t st);
// kv: per layer (stride layer_stride floats) nparts partials [nparts, n, 2 Hkv D]
hipError_t launch_ctx_kv_post(const float* kv, size_t layer_stride, int nparts, int n, int L,
                              int Hkv, int D, int qk_norm, float eps, float theta,
                              const int* positions, const CtxPtrs& P, hipStream_t st);

struct AttnPlan {
  int chunk_blocks;   // blocks per workgroup (a multiple of 8)
  int n_chunks;       // chunks per (request, kv head) over the visible span
  int qg;             // queries per (request, kv head) = group * q_rows
};
// window 0: the span is every block up to max_seq_len; window w > 0: the blocks a request's
// rows can see, at most ceil((w + q_rows - 1) / 16) + 1 starting at the first visible one
AttnPlan attn_plan(const sd_dims& d, int n_req, int max_seq_len, int window);
// chunks per (request, kv head) that no window can exceed at this max_seq_len
int attn_chunk_bound(const sd_dims& d, int n_req, int max_seq_len);

struct AttnArgs {
  // the stacked projection [q | k | v | o_gate] of the step's rows as nparts K-slice
  // partials [nparts, b, (2Hq + 2Hkv) D], summed in slice order by the kernels
  const float* qkv;
  int nparts;                 // 1 .. 4
  size_t part_stride;         // floats between partials
  int qk_norm;                // weightless RMSNorm of q and k heads before RoPE
  float eps;
  double freq[64];            // RoPE frequencies theta^(-2d/D), d < D/2 (host, in double)
  const int64_t* slot_mapping;  // cache slot of each row's new K/V (negative: not stored)
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int* block_table;
  int max_blocks;             // entries per block-table row
  int num_blocks;             // blocks in the pool (block ids are clamped below it)
  const int* seq_lens;
  const int* positions;
  int n_req, Hq, Hkv, D, q_rows;
  int window;                 // 0: causal; w > 0: positions p - w + 1 .. p
  const int* query_start;     // null: q_rows rows per request; else [n_req + 1] row starts
  int b;                      // rows of the step (query_start indices are clamped below it)
  float scale;
  float* part_acc;            // [Hkv, nslot = n_req * n_chunks, qg, D] (slot-major per head)
  float* part_ml;             // [Hkv, nslot, qg, 2]
  const float* gate;          // row t of partial p at gate + p * part_stride + t * gate_stride
  int gate_stride;
  uint16_t* out;              // bf16 hi terms of the gated output [b, Hq * D]
  uint16_t* out_lo;           // bf16 lo terms
};
hipError_t launch_attention(const AttnArgs& a, const AttnPlan& p, hipStream_t st);

// Router GEMM + top-k + softmax + pooler in one launch: workgroups compute split-K
// partial logits; the last to arrive (counter) reduces them and routes.
struct RouterArgs {
  int b, H, E, k;
  const uint16_t* x;     // bf16 [b, H] hi terms
  const uint16_t* x_lo;  // bf16 [b, H] lo terms (may be null)
  const uint16_t* w;     // packed bf16 [E, H]
  const float* bias;     // fp32 [b, E] (may be null)
  float* part;           // fp32 [H / 256, b, E] scratch
  int* counter;          // 0 at launch; the kernel leaves it 0
  float* logits;         // fp32 [b, E] (may be null)
  int* ids;
  float* w_out;
  int *counts, *offsets, *slot_of, *tos, *active;
};
hipError_t launch_router(const RouterArgs& a, hipStream_t st);

// Attention boundary (dual norm over nbranch partials of the attention branch) fused with
// the router's product: r.part receives the [b, E] logits (no bias); r.x / r.x_lo are
// unused.  The routing itself runs in the expert kernel (MoeArgs::route).
struct NormRouterArgs {
  int H;
  const float* branch;     // fp32 [nbranch, b, H]
  size_t branch_stride;    // floats between partials
  const float* stream_in;  // the stream entering the boundary
  float* stream;           // the updated stream (not stream_in: parts of a row write it)
  const float *g_post, *g_pre;
  float eps;
  uint16_t *out, *out_lo;  // bf16 hi / lo terms of the pre-FFN norm output
  _Float16 *x16, *x16_lo;  // fp16 hi / lo terms of it * 2^-8 (the expert input)
  RouterArgs r;
};
int norm_router_parts(int H, int E, int b, int k);  // 0: shape not served by the fusion
hipError_t launch_norm_router(const NormRouterArgs& a, int nbranch, hipStream_t st);
hipError_t launch_zero_i32(int* p, hipStream_t st);

struct MoeArgs {
  int b, H, I, E, k;
  const _Float16* x16;        // [b, H] hi terms of the expert input * 2^-8
  const _Float16* x16_lo;     // [b, H] lo terms after x16 in one buffer (null: exact in fp16)
  const uint8_t *w13_codes, *w13_scales;
  const float* w13_gscale;
  const uint8_t *w2_codes, *w2_scales;
  const float* w2_gscale;
  const int *counts, *offsets, *tos;
  const int* active;          // [E + 1]: active expert ids ascending, then their number
  _Float16* h16;              // [b*k, I] scratch: hi terms of the SwiGLU output * 2^-8
  _Float16* h16_lo;           // [b*k, I] scratch: lo terms, after h16 in one buffer
  uint16_t* h_bf16;           // [b*k, I] optional bf16 copy of the SwiGLU output
  float* y;                   // fp32 [b*k, H]
  uint32_t x16_lo_off;        // set by the launcher: bytes from x16 to x16_lo (0: none)
  uint32_t h16_lo_off;        // set by the launcher: bytes from h16 to h16_lo
  // route != 0: the W13 kernel first routes from the logits r.part [b, E] (+ r.bias), E <=
  // 32, and writes r's maps, which counts / offsets / tos / active must point to
  int route;
  RouterArgs r;
};
hipError_t launch_moe_experts(const MoeArgs& a, hipStream_t st);
bool moe_shape_supported(int H, int I);  // the expert GEMMs' K splits exist for H and I

hipError_t launch_unpool(int b, int H, int k, const float* y, const float* w,
                         const int* slot_of, float* out, hipStream_t st);

hipError_t launch_head_argmax(int b, int n_tiles, const float* val, const int* idx,
                              const int64_t* d2t, int32_t* ids, int64_t* target,
                              hipStream_t st);

hipError_t launch_debug_dequant(int n, int k, const uint8_t* codes, const uint8_t* scales,
                                float gscale, float* out, hipStream_t st);

// plain streaming read of bytes (a multiple of 16) at src; sink holds grid words
hipError_t launch_debug_lanes(const float* x, const int* xi, float* out, int* out_i,
                              hipStream_t st);
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int grid,
                             hipStream_t st);
