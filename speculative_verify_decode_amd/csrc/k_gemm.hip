// K-B: skinny bf16 GEMM for the step's dense projections (QKV, o_proj, router, lm_head),
// y[m, n] = sum_k x[m, k] * W[n, k] with M <= 64 rows, on v_mfma_f32_16x16x32_bf16.
//
// A workgroup owns 16 output features (one MFMA row tile) and all M rows; its 4 waves
// split K and meet in LDS.  Weights are the A operand, streamed once from HBM with
// 16-byte loads (4 lanes cover 64 contiguous bytes of a row per step); the activation
// rows are the B operand, read from L2.  Only the weight bytes scale with the layer, so
// the kernel is HBM-bound at b <= 64.  SPLIT: x carries bf16 hi/lo terms, 8 rows per
// column tile (columns 0-7 hi, 8-15 lo), summed in the epilogue.
//
// Also here: the QKV front's per-head epilogue (weightless qk RMSNorm, RoPE, bf16 K/V
// cache write) and the draft head's argmax reduction.
#include "sd_common.h"

namespace {

// NW waves split K; each wave works in passes of S MFMA steps (32 k each) and issues every
// weight and activation load of a pass before the first MFMA of it.  Loads are
// unconditional (rows past M or N read a valid clamped row) so nothing serialises them;
// activation rows past M are zeroed after their loads.
template <int NCT, int NW, int S, int MODE, bool SPLIT>
__global__ __launch_bounds__(64 * NW) void k_gemm(GemmArgs a) {
  constexpr int RPC = SPLIT ? 8 : 16;  // activation rows per column tile
  __shared__ f32x4_t red[NW - 1][NCT][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int KW = a.K / NW;
  const int k0 = wave * KW + 8 * g;
  // rows past N (a ragged last tile) re-read row N-1; their results are never stored
  const uint16_t* wrow = a.w + (size_t)min(n0 + i, a.N - 1) * a.K + k0;
  const uint16_t* xrow[NCT];
  bool xv[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int m = RPC * c + (SPLIT ? (i & 7) : i);
    const uint16_t* src = (SPLIT && (i >> 3)) ? a.x_lo : a.x;
    xv[c] = m < a.M;
    xrow[c] = src + (size_t)(xv[c] ? m : 0) * a.K + k0;
  }
  f32x4_t acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bf16x8_t zero8 = {};
  const int passes = (KW >> 5) / S;
  for (int p = 0; p < passes; ++p) {
    const int s0 = p * S * 32;
    bf16x8_t av[S];
    bf16x8_t bv[S][NCT];
#pragma unroll
    for (int u = 0; u < S; ++u)
      av[u] = __builtin_nontemporal_load((const bf16x8_t*)(wrow + s0 + 32 * u));
#pragma unroll
    for (int u = 0; u < S; ++u)
#pragma unroll
      for (int c = 0; c < NCT; ++c) bv[u][c] = *(const bf16x8_t*)(xrow[c] + s0 + 32 * u);
#pragma unroll
    for (int u = 0; u < S; ++u)
#pragma unroll
      for (int c = 0; c < NCT; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], xv[c] ? bv[u][c] : zero8, acc[c],
                                                         0, 0, 0);
  }
  if (wave > 0) {
#pragma unroll
    for (int c = 0; c < NCT; ++c) red[wave - 1][c][lane] = acc[c];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) acc[c] += red[w][c][lane];
    if (SPLIT) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[c][r] += __shfl_xor(acc[c][r], 8, 64);
    }
  }
  if (SPLIT && i >= 8) return;

  // lane holds y[m = RPC*c + i][n = n0 + 4g + r], r = 0..3
  const int nb = n0 + 4 * g;
  const bool full = nb + 3 < a.N;
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int m = RPC * c + i;
    const bool mv = m < a.M;
    if (MODE == GEMM_F32 || MODE == GEMM_F32_BIAS) {
      f32x4_t v = acc[c];
      if (MODE == GEMM_F32_BIAS && a.bias != nullptr && mv) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nb + r < a.N) v[r] += a.bias[(size_t)m * a.N + nb + r];
      }
      if (mv && full) {
        *(f32x4_t*)((float*)a.y + (size_t)m * a.N + nb) = v;
      } else if (mv) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nb + r < a.N) ((float*)a.y)[(size_t)m * a.N + nb + r] = v[r];
      }
    } else if (MODE == GEMM_BF16) {
      if (mv && full) {
        uint32_t lo = sd::f2bf(acc[c][0]) | ((uint32_t)sd::f2bf(acc[c][1]) << 16);
        uint32_t hi = sd::f2bf(acc[c][2]) | ((uint32_t)sd::f2bf(acc[c][3]) << 16);
        *(u32x2_t*)((uint16_t*)a.y + (size_t)m * a.N + nb) = u32x2_t{lo, hi};
      } else if (mv) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nb + r < a.N) ((uint16_t*)a.y)[(size_t)m * a.N + nb + r] = sd::f2bf(acc[c][r]);
      }
    } else {  // GEMM_HEAD: bf16 logits, optional transform, per-tile argmax (ties: low index)
      float best = -INFINITY;
      int bidx = nb;  // always a valid index, even if every logit is NaN
      f32x4_t tau;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float lg = sd::bf2f(sd::f2bf(acc[c][r]));
        if (lg > best) { best = lg; bidx = nb + r; }
        const float x = lg * a.multiplier;
        tau[r] = a.soft_cap > 0.f ? a.soft_cap * tanhf(x / a.soft_cap) : x;
      }
      if (mv && a.y != nullptr) *(f32x4_t*)((float*)a.y + (size_t)m * a.N + nb) = tau;
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float ov = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bidx, o, 64);
        if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
      }
      if (mv && g == 0) {
        a.head_val[(size_t)m * gridDim.x + blockIdx.x] = best;
        a.head_idx[(size_t)m * gridDim.x + blockIdx.x] = bidx;
      }
    }
  }
}

template <int NCT, int NW, int MODE, bool SPLIT>
void launch_s(const GemmArgs& a, hipStream_t st) {
  // steps per wave; the pass size S divides it and keeps the in-flight registers bounded
  constexpr int SCAP = NCT >= 8 ? 2 : 16 / NCT;
  const int steps = a.K / NW / 32;
  const dim3 grid((a.N + 15) / 16), block(64 * NW);
  if (SCAP >= 16 && steps % 16 == 0)
    hipLaunchKernelGGL((k_gemm<NCT, NW, (SCAP >= 16 ? 16 : 1), MODE, SPLIT>), grid, block, 0, st, a);
  else if (SCAP >= 8 && steps % 8 == 0)
    hipLaunchKernelGGL((k_gemm<NCT, NW, (SCAP >= 8 ? 8 : 1), MODE, SPLIT>), grid, block, 0, st, a);
  else if (SCAP >= 4 && steps % 4 == 0)
    hipLaunchKernelGGL((k_gemm<NCT, NW, (SCAP >= 4 ? 4 : 1), MODE, SPLIT>), grid, block, 0, st, a);
  else if (steps % 2 == 0)
    hipLaunchKernelGGL((k_gemm<NCT, NW, 2, MODE, SPLIT>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm<NCT, NW, 1, MODE, SPLIT>), grid, block, 0, st, a);
}

template <int NCT, int MODE, bool SPLIT>
hipError_t launch_u(const GemmArgs& a, hipStream_t st) {
  if (a.K % 256 == 0) launch_s<NCT, 8, MODE, SPLIT>(a, st);
  else launch_s<NCT, 4, MODE, SPLIT>(a, st);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_m(const GemmArgs& a, hipStream_t st) {
  if (a.x_lo != nullptr) {
    if (MODE == GEMM_HEAD) return hipErrorInvalidValue;
    if (a.M <= 8) return launch_u<1, MODE, true>(a, st);
    if (a.M <= 16) return launch_u<2, MODE, true>(a, st);
    if (a.M <= 32) return launch_u<4, MODE, true>(a, st);
    return launch_u<8, MODE, true>(a, st);
  }
  if (a.M <= 16) return launch_u<1, MODE, false>(a, st);
  if (a.M <= 32) return launch_u<2, MODE, false>(a, st);
  return launch_u<4, MODE, false>(a, st);
}

// One wave per (row, head).  Lane d < D/2 owns the rotate-half pair (d, d + D/2).
__global__ __launch_bounds__(64) void k_qkv_post(const float* __restrict__ qkv, int Hq, int Hkv,
                                                 int D, int qk_norm, float eps, float theta,
                                                 const int* __restrict__ positions,
                                                 const int64_t* __restrict__ slots,
                                                 uint16_t* __restrict__ q_out,
                                                 uint16_t* __restrict__ q_lo,
                                                 uint16_t* __restrict__ k_cache,
                                                 uint16_t* __restrict__ v_cache) {
  const int h = blockIdx.x, t = blockIdx.y, d = threadIdx.x;
  const int half = D >> 1;
  const int N = (2 * Hq + 2 * Hkv) * D;
  const float* row = qkv + (size_t)t * N;
  const bool act = d < half;
  const bool is_q = h < Hq;
  const int kvh = h - Hq;
  const float* src = is_q ? row + h * D : row + Hq * D + kvh * D;
  float x1 = act ? src[d] : 0.f, x2 = act ? src[d + half] : 0.f;
  if (qk_norm) {
    const float ss = sd::wave_sum(x1 * x1 + x2 * x2);
    const float r = rsqrtf(ss / (float)D + eps);
    x1 *= r;
    x2 *= r;
  }
  if (act) {
    // angle in double: positions reach 1e5 and fp32 would lose ~1e-2 rad
    const double freq = pow((double)theta, -2.0 * (double)d / (double)D);
    const double ang = (double)positions[t] * freq;
    const float c = (float)cos(ang), s = (float)sin(ang);
    const float y1 = x1 * c - x2 * s, y2 = x2 * c + x1 * s;
    if (is_q) {  // q as bf16 hi/lo terms
      const size_t o = ((size_t)t * Hq + h) * D;
      uint16_t h1, l1, h2, l2;
      sd::split_bf16(y1, h1, l1);
      sd::split_bf16(y2, h2, l2);
      q_out[o + d] = h1;
      q_out[o + d + half] = h2;
      q_lo[o + d] = l1;
      q_lo[o + d + half] = l2;
    } else if (slots[t] >= 0) {  // a negative slot writes nothing
      const int64_t slot = slots[t];
      const int64_t blk = slot >> 4;
      const int off = (int)(slot & 15);
      uint16_t* kp = k_cache + ((size_t)(blk * Hkv + kvh) * 16 + off) * D;
      kp[d] = sd::f2bf(y1);
      kp[d + half] = sd::f2bf(y2);
      const float* vs = row + Hq * D + Hkv * D + kvh * D;
      uint16_t* vp = v_cache + (size_t)(blk * Hkv + kvh) * D * 16 + off;
      vp[(size_t)d * 16] = sd::f2bf(vs[d]);
      vp[(size_t)(d + half) * 16] = sd::f2bf(vs[d + half]);
    }
  }
}

// Argmax over the per-tile bests of one row (ties: lower index), then the d2t gather.
__global__ __launch_bounds__(256) void k_head_argmax(int n_tiles, int n_vocab,
                                                     const float* __restrict__ val,
                                                     const int* __restrict__ idx,
                                                     const int64_t* __restrict__ d2t,
                                                     int32_t* __restrict__ ids,
                                                     int64_t* __restrict__ target) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int m = blockIdx.x;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int t = threadIdx.x; t < n_tiles; t += 256) {
    const float v = val[(size_t)m * n_tiles + t];
    const int ii = idx[(size_t)m * n_tiles + t];
    if (v > best || (v == best && ii < bi)) { best = v; bi = ii; }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
  }
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = best; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (sv[w] > best || (sv[w] == best && si[w] < bi)) { best = sv[w]; bi = si[w]; }
    if (bi < 0 || bi >= n_vocab) bi = 0;
    ids[m] = bi;
    target[m] = d2t[bi];
  }
}

}  // namespace

hipError_t launch_gemm(GemmMode mode, const GemmArgs& a, hipStream_t st) {
  switch (mode) {
    case GEMM_F32: return launch_m<GEMM_F32>(a, st);
    case GEMM_BF16: return launch_m<GEMM_BF16>(a, st);
    case GEMM_F32_BIAS: return launch_m<GEMM_F32_BIAS>(a, st);
    case GEMM_HEAD: return launch_m<GEMM_HEAD>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_qkv_post(const float* qkv, int b, int Hq, int Hkv, int D, int qk_norm,
                           float eps, float theta, const int* positions, const int64_t* slots,
                           uint16_t* q_out, uint16_t* q_lo, uint16_t* k_cache,
                           uint16_t* v_cache, hipStream_t st) {
  hipLaunchKernelGGL(k_qkv_post, dim3(Hq + Hkv, b), dim3(64), 0, st, qkv, Hq, Hkv, D, qk_norm,
                     eps, theta, positions, slots, q_out, q_lo, k_cache, v_cache);
  return hipGetLastError();
}

hipError_t launch_head_argmax(int b, int n_tiles, const float* val, const int* idx,
                              const int64_t* d2t, int32_t* ids, int64_t* target,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_head_argmax, dim3(b), dim3(256), 0, st, n_tiles, n_tiles * 16, val, idx,
                     d2t, ids, target);
  return hipGetLastError();
}
