// K-A: sandwich-norm boundary.  One workgroup per row; the row lives in registers.
//
// Page "vllm.models.muse_spark.nvidia.specialized_decode.runtime.decode", module
// docstring: the first layer's front puts the embedded tokens into the fp32 stream and
// its pre-attention norm into the attention input; each later boundary adds the
// post-norm of the incoming branch to the stream and writes the next block's pre-norm.
// Order of the two norms: page "vllm.models.muse_spark.common.dspark",
// MuseSparkDSparkDecoderLayer.forward.
#include "sd_common.h"

namespace {

using sd::store16;
using sd::VecF;


// H = 256 * EPT.  Thread tid owns NV vectors of VW consecutive elements, vector v at
// element (v * 256 + tid) * VW, so every load is coalesced and as wide as H allows.  All
// inputs (the NB branch partials, stream, both gains) are loaded before the first
// reduction, so the row costs one round trip to memory; outputs leave as packed stores.
// POOL: the branch is the previous layer's pooled MoE output, gathered here (the weighted
// unpooler): branch row t = sum over j < k, in order, of w[t, j] * y[slot_of[t, j]] (y fp32
// [b * k, H]); the row's k slot ids and weights are read first, then every slot row at once.
// The updated stream goes to stream_out, which may be the stream itself (a workgroup reads
// its whole row before it writes it).
template <int EPT, int NB, bool POOL>
__global__ __launch_bounds__(256) void k_dualnorm(int H, const float* stream,
                                                  float* stream_out,
                                                  const float* __restrict__ branch,
                                                  size_t branch_stride,
                                                  const float* __restrict__ pw,
                                                  const int* __restrict__ pslot, int pk,
                                                  const uint16_t* __restrict__ front,
                                                  const float* __restrict__ g_post,
                                                  const float* __restrict__ g_pre, float eps,
                                                  uint16_t* __restrict__ out,
                                                  uint16_t* __restrict__ out_lo,
                                                  _Float16* __restrict__ x16,
                                                  _Float16* __restrict__ x16_lo,
                                                  int* __restrict__ zero,
                                                  float* __restrict__ aux) {
  constexpr int VW = EPT % 4 == 0 ? 4 : (EPT % 2 == 0 ? 2 : 1);
  constexpr int NV = EPT / VW;
  typedef typename VecF<VW>::T V;
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  if (zero != nullptr && row == 0 && tid == 0) *zero = 0;
  const size_t base = (size_t)row * H;
  const float inv_h = 1.0f / (float)H;
  float s[EPT], gq[EPT];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int i0 = (v * 256 + tid) * VW;
    const V q = *(const V*)(g_pre + i0);
#pragma unroll
    for (int j = 0; j < VW; ++j) gq[v * VW + j] = ((const float*)&q)[j];
  }
  if (branch != nullptr) {
    float u[EPT], gp[EPT];
    int sl[POOL ? 8 : 1];
    float wj[POOL ? 8 : 1];
    if constexpr (POOL) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // clamped into the pooled rows, so a bad slot id reads a wrong row, never past y
        sl[j] = min(max(pslot[row * pk + min(j, pk - 1)], 0), (int)gridDim.x * pk - 1);
        wj[j] = j < pk ? pw[row * pk + j] : 0.f;
      }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int i0 = (v * 256 + tid) * VW;
      V bu;
      if constexpr (POOL) {
        // choices past k repeat the last slot with weight 0 (an exact +0 to the sum)
        V yv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) yv[j] = *(const V*)(branch + (size_t)sl[j] * H + i0);
        bu = V{};
#pragma unroll
        for (int j = 0; j < 8; ++j) bu += wj[j] * yv[j];
      } else {
        bu = *(const V*)(branch + base + i0);
#pragma unroll
        for (int p = 1; p < NB; ++p) bu += *(const V*)(branch + p * branch_stride + base + i0);
      }
      const V bs = *(const V*)(stream + base + i0);
      const V bg = *(const V*)(g_post + i0);
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        u[v * VW + j] = ((const float*)&bu)[j];
        s[v * VW + j] = ((const float*)&bs)[j];
        gp[v * VW + j] = ((const float*)&bg)[j];
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the first use
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) ss += u[e] * u[e];
    ss = sd::block_sum<4>(ss, red);
    const float r = rsqrtf(ss * inv_h + eps);
#pragma unroll
    for (int e = 0; e < EPT; ++e) s[e] += u[e] * r * gp[e];
  } else {
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int j = 0; j < VW; ++j) s[v * VW + j] = sd::bf2f(front[base + (v * 256 + tid) * VW + j]);
  }
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    V o;
#pragma unroll
    for (int j = 0; j < VW; ++j) {
      ((float*)&o)[j] = s[v * VW + j];
      ss += s[v * VW + j] * s[v * VW + j];
    }
    *(V*)(stream_out + base + (v * 256 + tid) * VW) = o;
    if (aux != nullptr) *(V*)(aux + base + (v * 256 + tid) * VW) = o;
  }
  ss = sd::block_sum<4>(ss, red);
  const float r = rsqrtf(ss * inv_h + eps);
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const size_t i0 = base + (size_t)(v * 256 + tid) * VW;
    uint16_t hi[VW], lo[VW];
    _Float16 h16[VW], l16[VW];
#pragma unroll
    for (int j = 0; j < VW; ++j) {
      const float x = s[v * VW + j] * r * gq[v * VW + j];
      sd::split_bf16(x, hi[j], lo[j]);
      sd::split_f16(x, h16[j], l16[j]);
    }
    store16<VW>(out + i0, hi);
    if (out_lo != nullptr) store16<VW>(out_lo + i0, lo);
    if (x16 != nullptr) {
      store16<VW>((uint16_t*)x16 + i0, (const uint16_t*)h16);
      store16<VW>((uint16_t*)x16_lo + i0, (const uint16_t*)l16);
    }
  }
}

// bf16 x -> fp16 hi / lo terms of x * 2^-8, four elements per thread (H % 4 == 0).
__global__ __launch_bounds__(256) void k_expert_input(int n4, const uint16_t* __restrict__ x,
                                                      _Float16* __restrict__ x16,
                                                      _Float16* __restrict__ x16_lo) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const u32x2_t v = *(const u32x2_t*)(x + 4 * (size_t)i);
  const float f[4] = {__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u),
                      __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xffff0000u)};
  _Float16 h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sd::split_f16(f[j], h[j], l[j]);
  store16<4>((uint16_t*)x16 + 4 * (size_t)i, (const uint16_t*)h);
  store16<4>((uint16_t*)x16_lo + 4 * (size_t)i, (const uint16_t*)l);
}

}  // namespace

hipError_t launch_expert_input(int b, int H, const uint16_t* x, _Float16* x16, _Float16* x16_lo,
                               hipStream_t st) {
  if (H % 4) return hipErrorInvalidValue;
  const int n4 = b * H / 4;
  hipLaunchKernelGGL(k_expert_input, dim3((n4 + 255) / 256), dim3(256), 0, st, n4, x, x16, x16_lo);
  return hipGetLastError();
}

hipError_t launch_dualnorm(int b, int H, const float* stream, float* stream_out,
                           const float* branch, int nbranch,
                           const uint16_t* front, const float* g_post, const float* g_pre,
                           float eps, uint16_t* out, uint16_t* out_lo, _Float16* x16,
                           _Float16* x16_lo, int* zero, float* aux, hipStream_t st,
                           const float* pool_w, const int* pool_slot, int pool_k) {
  if ((x16 == nullptr) != (x16_lo == nullptr)) return hipErrorInvalidValue;
  if (branch != nullptr && nbranch < 1) return hipErrorInvalidValue;
  const bool pool = pool_slot != nullptr;
  if (pool && (branch == nullptr || pool_w == nullptr || pool_k < 1 || pool_k > 8))
    return hipErrorInvalidValue;
  const dim3 grid(b), block(256);
  const size_t bs = (size_t)b * H;
  if (branch == nullptr) nbranch = 1;
  if (nbranch != 1 && nbranch != 2 && nbranch != 4) return hipErrorInvalidValue;
#define SD_NORM_NB(E, NBV, P)                                                              \
  hipLaunchKernelGGL((k_dualnorm<E, NBV, P>), grid, block, 0, st, H, stream, stream_out,     \
                     branch, bs,                                                          \
                     pool_w, pool_slot, pool_k, front, g_post, g_pre, eps, out, out_lo, x16,  \
                     x16_lo, zero, aux)
#define SD_NORM_CASE(E)                                                                   \
  case E:                                                                                 \
    if (pool) SD_NORM_NB(E, 1, true);                                                     \
    else if (nbranch == 1) SD_NORM_NB(E, 1, false);                                       \
    else if (nbranch == 2) SD_NORM_NB(E, 2, false);                                       \
    else SD_NORM_NB(E, 4, false);                                                         \
    break;
  switch (H / 256) {
    SD_NORM_CASE(1)
    SD_NORM_CASE(2)
    SD_NORM_CASE(4)
    SD_NORM_CASE(8)
    SD_NORM_CASE(12)
    SD_NORM_CASE(16)
    SD_NORM_CASE(20)
    SD_NORM_CASE(24)
    SD_NORM_CASE(32)
    default:
      return hipErrorInvalidValue;
  }
#undef SD_NORM_CASE
#undef SD_NORM_NB
  return hipGetLastError();
}
