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

template <int EPT>  // elements per thread: H = 256 * EPT
__global__ __launch_bounds__(256) void k_dualnorm(int H, float* __restrict__ stream,
                                                  const float* __restrict__ branch,
                                                  const uint16_t* __restrict__ front,
                                                  const float* __restrict__ g_post,
                                                  const float* __restrict__ g_pre, float eps,
                                                  uint16_t* __restrict__ out,
                                                  uint16_t* __restrict__ out_lo,
                                                  _Float16* __restrict__ x16,
                                                  _Float16* __restrict__ x16_lo) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const size_t base = (size_t)row * H;
  const float inv_h = 1.0f / (float)H;
  float s[EPT];
  if (branch != nullptr) {
    float u[EPT];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      u[e] = branch[base + e * 256 + tid];
      ss += u[e] * u[e];
    }
    ss = sd::block_sum<4>(ss, red);
    const float r = rsqrtf(ss * inv_h + eps);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = e * 256 + tid;
      s[e] = stream[base + i] + u[e] * r * g_post[i];
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) s[e] = sd::bf2f(front[base + e * 256 + tid]);
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    stream[base + e * 256 + tid] = s[e];
    ss += s[e] * s[e];
  }
  ss = sd::block_sum<4>(ss, red);
  const float r = rsqrtf(ss * inv_h + eps);
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = e * 256 + tid;
    const float x = s[e] * r * g_pre[i];
    uint16_t hi, lo;
    sd::split_bf16(x, hi, lo);
    out[base + i] = hi;
    if (out_lo != nullptr) out_lo[base + i] = lo;
    if (x16 != nullptr) {
      _Float16 h16, l16;
      sd::split_f16(x, h16, l16);
      x16[base + i] = h16;
      x16_lo[base + i] = l16;
    }
  }
}

// bf16 -> fp16 hi term of x * 2^-8 (exact for |x| >= 2^-6, so no lo term is kept).
__global__ __launch_bounds__(256) void k_to_f16(int n, const uint16_t* __restrict__ x,
                                                _Float16* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = (_Float16)(sd::bf2f(x[i]) * SD_X16_SCALE);
}

}  // namespace

hipError_t launch_dualnorm(int b, int H, float* stream, const float* branch,
                           const uint16_t* front, const float* g_post, const float* g_pre,
                           float eps, uint16_t* out, uint16_t* out_lo, _Float16* x16,
                           _Float16* x16_lo, hipStream_t st) {
  if ((x16 == nullptr) != (x16_lo == nullptr)) return hipErrorInvalidValue;
  const dim3 grid(b), block(256);
  switch (H / 256) {
#define SD_NORM_CASE(E)                                                                   \
  case E:                                                                                 \
    hipLaunchKernelGGL(k_dualnorm<E>, grid, block, 0, st, H, stream, branch, front, g_post, \
                       g_pre, eps, out, out_lo, x16, x16_lo);                              \
    break;
    SD_NORM_CASE(1)
    SD_NORM_CASE(2)
    SD_NORM_CASE(4)
    SD_NORM_CASE(8)
    SD_NORM_CASE(12)
    SD_NORM_CASE(16)
    SD_NORM_CASE(20)
    SD_NORM_CASE(24)
    SD_NORM_CASE(32)
#undef SD_NORM_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_to_f16(int n, const uint16_t* x, _Float16* out, hipStream_t st) {
  hipLaunchKernelGGL(k_to_f16, dim3((n + 255) / 256), dim3(256), 0, st, n, x, out);
  return hipGetLastError();
}
