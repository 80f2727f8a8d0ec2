// Draft side: the dense decoder layer's norms and feed-forward, and the context-K/V store.
//
// Page "vllm.models.muse_spark.common.dspark":
//   MuseSparkDSparkDecoderLayer.forward - the stream is cast to the compute dtype (bf16)
//     before each trained input norm and those norms return bf16; the post-norms of the
//     attention and feed-forward outputs are added to the fp32 stream.
//   MuseSparkDSparkForCausalLM.hf_to_vllm_mapper - gate_proj and up_proj stacked as shards
//     0 and 1 of gate_up_proj (gate rows first).
//   MuseSparkDSparkModel._project_muse_context_kv / precompute_and_store_context_kv - the
//     hidden norm, each layer's pre-QKV norm, one batched product with the stacked K/V
//     rows, a weightless fp32 K RMSNorm cast back to bf16, RoPE, the cache update.
#include "sd_common.h"

namespace {

using sd::store16;
using sd::VecF;


// bf16 value of an fp32 (round to nearest even), as fp32
__device__ __forceinline__ float rbf(float x) { return sd::bf2f(sd::f2bf(x)); }

// One workgroup per row, H = 256 * EPT, thread tid owning vectors v at (v * 256 + tid) * VW.
//   MODE kPre:      out = bf16(RMSNorm(bf16(stream); g_pre))
//   MODE kBoundary: stream += RMSNorm(sum of NB branch partials; g_post), then as kPre
//   MODE kPost:     stream += RMSNorm(sum of NB branch partials; g_post)
enum DraftNorm { kPre = 0, kBoundary = 1, kPost = 2 };

template <int EPT, int NB, int MODE>
__global__ __launch_bounds__(256) void k_draft_norm(int H, float* __restrict__ stream,
                                                    const float* __restrict__ branch,
                                                    size_t branch_stride,
                                                    const float* __restrict__ g_post,
                                                    const float* __restrict__ g_pre, float eps,
                                                    uint16_t* __restrict__ out) {
  constexpr int VW = EPT % 4 == 0 ? 4 : (EPT % 2 == 0 ? 2 : 1);
  constexpr int NV = EPT / VW;
  typedef typename VecF<VW>::T V;
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const size_t base = (size_t)row * H;
  const float inv_h = 1.0f / (float)H;
  float s[EPT], u[EPT], gp[EPT], gq[EPT];
  // every load before the first reduction
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int i0 = (v * 256 + tid) * VW;
    const V bs = *(const V*)(stream + base + i0);
#pragma unroll
    for (int j = 0; j < VW; ++j) s[v * VW + j] = ((const float*)&bs)[j];
    if constexpr (MODE != kPost) {
      const V q = *(const V*)(g_pre + i0);
#pragma unroll
      for (int j = 0; j < VW; ++j) gq[v * VW + j] = ((const float*)&q)[j];
    }
    if constexpr (MODE != kPre) {
      V bu = *(const V*)(branch + base + i0);
#pragma unroll
      for (int p = 1; p < NB; ++p) bu += *(const V*)(branch + p * branch_stride + base + i0);
      const V bg = *(const V*)(g_post + i0);
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        u[v * VW + j] = ((const float*)&bu)[j];
        gp[v * VW + j] = ((const float*)&bg)[j];
      }
    }
  }
  if constexpr (MODE != kPre) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) ss += u[e] * u[e];
    ss = sd::block_sum<4>(ss, red);
    const float r = rsqrtf(ss * inv_h + eps);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      V o;
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        s[v * VW + j] += u[v * VW + j] * r * gp[v * VW + j];
        ((float*)&o)[j] = s[v * VW + j];
      }
      *(V*)(stream + base + (v * 256 + tid) * VW) = o;
    }
  }
  if constexpr (MODE != kPost) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      s[e] = rbf(s[e]);  // the norm reads the stream in the compute dtype
      ss += s[e] * s[e];
    }
    ss = sd::block_sum<4>(ss, red);
    const float r = rsqrtf(ss * inv_h + eps);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      uint16_t o[VW];
#pragma unroll
      for (int j = 0; j < VW; ++j) o[j] = sd::f2bf(s[v * VW + j] * r * gq[v * VW + j]);
      store16<VW>(out + base + (v * 256 + tid) * VW, o);
    }
  }
}

// h = silu(g) * u from NP K-slice partials of [g | u] ([NP, b, 2I], gate columns first);
// h leaves as bf16 hi terms at h and lo terms at h_lo.  Four columns per thread.
template <int NP>
__global__ __launch_bounds__(256) void k_swiglu_dense(int b, int I, const float* __restrict__ gu,
                                                      size_t part_stride,
                                                      uint16_t* __restrict__ h,
                                                      uint16_t* __restrict__ h_lo) {
  const size_t n4 = (size_t)b * I / 4;
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n4) return;
  const size_t e = q * 4;
  const int t = (int)(e / I), i = (int)(e - (size_t)t * I);
  const float* g0 = gu + (size_t)t * 2 * I + i;
  f32x4_t g = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NP; ++p) {  // every partial's loads in flight together, summed in order
    g += *(const f32x4_t*)(g0 + p * part_stride);
    u += *(const f32x4_t*)(g0 + p * part_stride + I);
  }
  uint16_t hi[4], lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sd::split_bf16(g[j] / (1.0f + __expf(-g[j])) * u[j], hi[j], lo[j]);
  store16<4>(h + e, hi);
  store16<4>(h_lo + e, lo);
}

// Context rows: x[l, row] = bf16(RMSNorm(bf16(RMSNorm(states[row]; g_hidden)); g_pre[l])).
// Workgroup (row, layer); the hidden norm is recomputed per layer (one row, no traffic).
template <int EPT>
__global__ __launch_bounds__(256) void k_ctx_norm(int H, int n, const uint16_t* __restrict__ states,
                                                  const float* __restrict__ g_hidden,
                                                  CtxPtrs P, float eps, uint16_t* __restrict__ x) {
  __shared__ float red[4];
  const int row = blockIdx.x, l = blockIdx.y, tid = threadIdx.x;
  const float* g_pre = P.g_pre[l];
  const float inv_h = 1.0f / (float)H;
  float v[EPT], g1[EPT], g2[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = e * 256 + tid;
    v[e] = sd::bf2f(states[(size_t)row * H + i]);
    g1[e] = g_hidden[i];
    g2[e] = g_pre[i];
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) ss += v[e] * v[e];
  float r = rsqrtf(sd::block_sum<4>(ss, red) * inv_h + eps);
  ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    v[e] = rbf(v[e] * r * g1[e]);  // the hidden norm's bf16 output
    ss += v[e] * v[e];
  }
  r = rsqrtf(sd::block_sum<4>(ss, red) * inv_h + eps);
  uint16_t* xo = x + ((size_t)l * n + row) * H;
#pragma unroll
  for (int e = 0; e < EPT; ++e) xo[e * 256 + tid] = sd::f2bf(v[e] * r * g2[e]);
}

// Context K/V of one (kv head, row, layer): NP K-slice partials of the [n, 2 Hkv D] product
// summed and cast to bf16; K through the weightless RMSNorm (fp32, cast to bf16) and RoPE;
// both written into the layer's cache at its slot (a negative slot writes nothing).  One
// wave; lane d handles the rotation pair (d, d + D/2).
template <int NP>
__global__ __launch_bounds__(64) void k_ctx_kv_post(const float* __restrict__ kv, size_t layer_stride,
                                                    size_t part_stride, int n, int Hkv, int D,
                                                    int qk_norm, float eps, float theta,
                                                    const int* __restrict__ positions, CtxPtrs P) {
  const int h = blockIdx.x, t = blockIdx.y, l = blockIdx.z, d = threadIdx.x;
  const int half = D >> 1;
  const bool act = d < half;
  const float* row = kv + l * layer_stride + (size_t)t * 2 * Hkv * D;
  float k1 = 0.f, k2 = 0.f, v1 = 0.f, v2 = 0.f;
  if (act) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float* rp = row + p * part_stride;
      k1 += rp[h * D + d];
      k2 += rp[h * D + d + half];
      v1 += rp[(Hkv + h) * D + d];
      v2 += rp[(Hkv + h) * D + d + half];
    }
  }
  k1 = rbf(k1);  // the batched product returns bf16
  k2 = rbf(k2);
  if (qk_norm) {
    const float ss = sd::wave_sum(act ? k1 * k1 + k2 * k2 : 0.f);
    const float r = rsqrtf(ss / (float)D + eps);
    k1 = rbf(k1 * r);
    k2 = rbf(k2 * r);
  }
  const int64_t slot = P.slots[l][t];
  if (!act || slot < 0) return;
  // angle in double: positions reach 1e5 and fp32 would lose ~1e-2 rad
  const double freq = pow((double)theta, -2.0 * (double)d / (double)D);
  const double ang = (double)positions[t] * freq;
  const float c = (float)cos(ang), s = (float)sin(ang);
  const float y1 = k1 * c - k2 * s, y2 = k2 * c + k1 * s;
  const int64_t blk = slot >> 4;
  const int off = (int)(slot & 15);
  uint16_t* kp = P.k_cache[l] + ((size_t)(blk * Hkv + h) * 16 + off) * D;
  kp[d] = sd::f2bf(y1);
  kp[d + half] = sd::f2bf(y2);
  uint16_t* vp = P.v_cache[l] + (size_t)(blk * Hkv + h) * D * 16 + off;
  vp[(size_t)d * 16] = sd::f2bf(v1);
  vp[(size_t)(d + half) * 16] = sd::f2bf(v2);
}

}  // namespace

hipError_t launch_draft_norm(int mode, int b, int H, float* stream, const float* branch,
                             int nbranch, const float* g_post, const float* g_pre, float eps,
                             uint16_t* out, hipStream_t st) {
  if (H % 256 || (mode != kPost && (g_pre == nullptr || out == nullptr)) ||
      (mode != kPre && (branch == nullptr || g_post == nullptr)))
    return hipErrorInvalidValue;
  const int ept = H / 256;
  if (mode == kPre) nbranch = 1;
  const dim3 grid(b), block(256);
  const size_t bs = (size_t)b * H;
#define SD_DN(E, NBV, M)                                                                      \
  if (ept == E && nbranch == NBV && mode == M) {                                            \
    hipLaunchKernelGGL((k_draft_norm<E, NBV, M>), grid, block, 0, st, H, stream, branch, bs,  \
                       g_post, g_pre, eps, out);                                            \
    return hipGetLastError();                                                               \
  }
#define SD_DN_E(E) SD_DN(E, 1, kPre) SD_DN(E, 1, kBoundary) SD_DN(E, 4, kBoundary) \
                   SD_DN(E, 1, kPost) SD_DN(E, 4, kPost)
  SD_DN_E(1) SD_DN_E(2) SD_DN_E(4) SD_DN_E(8) SD_DN_E(16) SD_DN_E(32)
#undef SD_DN_E
#undef SD_DN
  return hipErrorInvalidValue;
}

hipError_t launch_swiglu_dense(int b, int I, const float* gu, int nparts, uint16_t* h,
                               uint16_t* h_lo, hipStream_t st) {
  if (I % 4) return hipErrorInvalidValue;
  const size_t n4 = (size_t)b * I / 4;
  const dim3 grid((unsigned)((n4 + 255) / 256)), block(256);
  const size_t ps = (size_t)b * 2 * I;
  if (nparts == 1) hipLaunchKernelGGL((k_swiglu_dense<1>), grid, block, 0, st, b, I, gu, ps, h, h_lo);
  else if (nparts == 4) hipLaunchKernelGGL((k_swiglu_dense<4>), grid, block, 0, st, b, I, gu, ps, h, h_lo);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_ctx_norm(int n, int L, int H, const uint16_t* states, const float* g_hidden,
                           const CtxPtrs& P, float eps, uint16_t* x, hipStream_t st) {
  const dim3 grid(n, L), block(256);
  switch (H / 256) {
#define SD_CN(E) case E: hipLaunchKernelGGL((k_ctx_norm<E>), grid, block, 0, st, H, n, states, g_hidden, P, eps, x); break;
    SD_CN(1) SD_CN(2) SD_CN(4) SD_CN(8) SD_CN(16) SD_CN(32)
#undef SD_CN
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_ctx_kv_post(const float* kv, size_t layer_stride, int nparts, int n, int L,
                              int Hkv, int D, int qk_norm, float eps, float theta,
                              const int* positions, const CtxPtrs& P, hipStream_t st) {
  if (D > 128 || D % 2) return hipErrorInvalidValue;
  const dim3 grid(Hkv, n, L), block(64);
  const size_t ps = (size_t)n * 2 * Hkv * D;
  if (nparts == 1)
    hipLaunchKernelGGL((k_ctx_kv_post<1>), grid, block, 0, st, kv, layer_stride, ps, n, Hkv, D,
                       qk_norm, eps, theta, positions, P);
  else if (nparts == 4)
    hipLaunchKernelGGL((k_ctx_kv_post<4>), grid, block, 0, st, kv, layer_stride, ps, n, Hkv, D,
                       qk_norm, eps, theta, positions, P);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
