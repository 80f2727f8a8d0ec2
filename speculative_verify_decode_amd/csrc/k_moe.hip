// K-D .. K-G: routing, pooler, routed FP4 experts and the weighted unpooler.
//
// Page "vllm.models.muse_spark.nvidia.specialized_decode.runtime.decode", module
// docstring: the MoE block is router -> routing -> pooler -> routed experts -> tail ->
// unpooler (the tail is a cross-rank combine and is the identity on one GPU).  The
// routed experts are NVFP4 (page "vllm.models.muse_spark.nvidia.specialized_decode.
// runtime", module list: expert_tp).
//
// Expert GEMMs: workgroup (n-tile of 16 output features, expert e) with KS waves splitting
// K.  Weights are the A operand of v_mfma_f32_16x16x32_f16, dequantised exactly in
// registers (dequant_unit); each lane streams a contiguous run of K/(4*KS) codes of its
// row.  The pooled tokens of expert e are the B operand, 8 per column tile as hi/lo fp16
// terms (columns 0-7 / 8-15).  Workgroups of experts with no routed token exit at once.
#include "sd_common.h"

namespace {

// ---------------------------------------------------------------- routing + pooler
// One workgroup.  Top-k by (-z, index); weights = softmax over the selected logits;
// pooler = stable counting sort of (row, choice) pairs by expert.
__global__ __launch_bounds__(256) void k_route_pool(const float* __restrict__ z, int b, int E,
                                                    int k, int* __restrict__ ids,
                                                    float* __restrict__ w,
                                                    int* __restrict__ counts,
                                                    int* __restrict__ offsets,
                                                    int* __restrict__ slot_of,
                                                    int* __restrict__ tos,
                                                    int* __restrict__ active) {
  __shared__ int s_ids[64 * 8];
  __shared__ int s_cnt[256];
  __shared__ int s_off[257];
  const int tid = threadIdx.x;
  if (tid < b) {
    const float* zr = z + (size_t)tid * E;
    float prev_v = INFINITY;
    int prev_i = -1;
    float sel[8];
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = -1;
      for (int e = 0; e < E; ++e) {
        const float v = zr[e] != zr[e] ? -INFINITY : zr[e];  // NaN ranks last
        // eligible: after the previous pick in the order (-z, index)
        const bool after = v < prev_v || (v == prev_v && e > prev_i);
        if (after && (bi < 0 || v > bv)) { bv = v; bi = e; }
      }
      s_ids[tid * k + j] = bi;
      ids[tid * k + j] = bi;
      sel[j] = bv;
      prev_v = bv;
      prev_i = bi;
    }
    float den = 0.f;
    for (int j = 0; j < k; ++j) den += __expf(sel[j] - sel[0]);
    for (int j = 0; j < k; ++j) w[tid * k + j] = __expf(sel[j] - sel[0]) / den;
  }
  __syncthreads();
  const int nk = b * k;
  if (tid < E) {
    int c = 0;
    for (int p = 0; p < nk; ++p) c += s_ids[p] == tid;
    s_cnt[tid] = c;
  }
  __syncthreads();
  if (tid == 0) {
    int o = 0, na = 0;
    for (int e = 0; e < E; ++e) {
      s_off[e] = o;
      offsets[e] = o;
      counts[e] = s_cnt[e];
      if (s_cnt[e] > 0) active[na++] = e;
      o += s_cnt[e];
    }
    s_off[E] = o;
    offsets[E] = o;
    active[E] = na;
  }
  __syncthreads();
  if (tid < E) {
    int slot = s_off[tid];
    for (int p = 0; p < nk; ++p)
      if (s_ids[p] == tid) {
        slot_of[p] = slot;
        tos[slot] = p / k;
        ++slot;
      }
  }
}

// ---------------------------------------------------------------- expert GEMMs
// Load 16 bytes of codes + 2 scale bytes of one row at k offset kk (a 32-weight unit).
__device__ __forceinline__ void load_unit(const uint8_t* codes_row, const uint8_t* scale_row,
                                          int kk, u32x4_t& c, uint32_t& s) {
  c = __builtin_nontemporal_load((const u32x4_t*)(codes_row + (kk >> 1)));
  s = *(const uint16_t*)(scale_row + (kk >> 4));
}

// Column-tile rows of the B operand: lane column i holds token slot 8c + (i & 7), hi term
// for i < 8 and lo term for i >= 8.  Returns the row pointer at k offset kl0, or null.
__device__ __forceinline__ const _Float16* b_row(const _Float16* hi, const _Float16* lo,
                                                 size_t row, int K, int kl0, int i) {
  const _Float16* base = (i >> 3) ? lo : hi;
  return base == nullptr ? nullptr : base + row * K + kl0;
}

// W13 (gate rows [0, I), up rows [I, 2I)) + SwiGLU.
template <int NCT, int KS>
__global__ __launch_bounds__(64 * KS) void k_moe_w13(MoeArgs a) {
  __shared__ f32x4_t red[KS > 1 ? KS - 1 : 1][2][NCT][64];
  const int nt = blockIdx.x, e = blockIdx.y;
  const int Te = a.counts[e];
  if (Te == 0) return;
  const int off = a.offsets[e];
  const int nct = (Te + 7) >> 3;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = lane & 15, G = lane >> 4;
  const int K = a.H;
  const int KL = K / (4 * KS);
  const int kl0 = wave * (K / KS) + G * KL;
  const size_t rowg = (size_t)e * 2 * a.I + nt * 16 + i;
  const size_t rowu = rowg + a.I;
  const uint8_t* cg = a.w13_codes + rowg * (K >> 1);
  const uint8_t* cu = a.w13_codes + rowu * (K >> 1);
  const uint8_t* sg = a.w13_scales + rowg * (K >> 4);
  const uint8_t* su = a.w13_scales + rowu * (K >> 4);
  const _Float16* xr[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int slot = 8 * c + (i & 7);
    xr[c] = slot < Te ? b_row(a.x16, a.x16_lo, a.tos[off + slot], K, kl0, i) : nullptr;
  }
  f32x4_t ag[NCT], au[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) ag[c] = au[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const f16x8_t zero8 = {};
  for (int kk = 0; kk < KL; kk += 32) {
    u32x4_t c0, c1;
    uint32_t s0, s1;
    load_unit(cg, sg, kl0 + kk, c0, s0);
    load_unit(cu, su, kl0 + kk, c1, s1);
    f16x8_t wg[4], wu[4];
    sd::dequant_unit(c0, s0, wg);
    sd::dequant_unit(c1, s1, wu);
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      if (c >= nct) break;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f16x8_t bx = xr[c] != nullptr ? *(const f16x8_t*)(xr[c] + kk + 8 * m) : zero8;
        ag[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wg[m], bx, ag[c], 0, 0, 0);
        au[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wu[m], bx, au[c], 0, 0, 0);
      }
    }
  }
  if (KS > 1) {
    if (wave > 0) {
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        red[wave - 1][0][c][lane] = ag[c];
        red[wave - 1][1][c][lane] = au[c];
      }
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int w = 0; w < KS - 1; ++w) {
        ag[c] += red[w][0][c][lane];
        au[c] += red[w][1][c][lane];
      }
  }
  // hi + lo columns
#pragma unroll
  for (int c = 0; c < NCT; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ag[c][r] += __shfl_xor(ag[c][r], 8, 64);
      au[c][r] += __shfl_xor(au[c][r], 8, 64);
    }
  if (i >= 8) return;
  const float sc = SD_X16_UNSCALE * a.w13_gscale[e];
  const int n = nt * 16 + 4 * G;  // lane rows n .. n+3 of the gate (and up) block
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int slot = 8 * c + i;
    if (slot >= Te) continue;
    const size_t o = (size_t)(off + slot) * a.I + n;
    _Float16 hh[4], hl[4];
    uint16_t hb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float gv = ag[c][r] * sc, uv = au[c][r] * sc;
      const float h = gv / (1.0f + __expf(-gv)) * uv;
      sd::split_f16(h, hh[r], hl[r]);
      hb[r] = sd::f2bf(h);
    }
    *(u32x2_t*)(a.h16 + o) = u32x2_t{__builtin_bit_cast(uint32_t, f16x2_t{hh[0], hh[1]}),
                                     __builtin_bit_cast(uint32_t, f16x2_t{hh[2], hh[3]})};
    *(u32x2_t*)(a.h16_lo + o) = u32x2_t{__builtin_bit_cast(uint32_t, f16x2_t{hl[0], hl[1]}),
                                        __builtin_bit_cast(uint32_t, f16x2_t{hl[2], hl[3]})};
    if (a.h_bf16 != nullptr)
      *(u32x2_t*)(a.h_bf16 + o) = u32x2_t{hb[0] | ((uint32_t)hb[1] << 16),
                                          hb[2] | ((uint32_t)hb[3] << 16)};
  }
}

// W2: y[slot, n] = h[slot] . W2_e[n], fp32.
template <int NCT, int KS>
__global__ __launch_bounds__(64 * KS) void k_moe_w2(MoeArgs a) {
  __shared__ f32x4_t red[KS > 1 ? KS - 1 : 1][NCT][64];
  const int nt = blockIdx.x, e = blockIdx.y;
  const int Te = a.counts[e];
  if (Te == 0) return;
  const int off = a.offsets[e];
  const int nct = (Te + 7) >> 3;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = lane & 15, G = lane >> 4;
  const int K = a.I;
  const int KL = K / (4 * KS);
  const int kl0 = wave * (K / KS) + G * KL;
  const size_t row = (size_t)e * a.H + nt * 16 + i;
  const uint8_t* cw = a.w2_codes + row * (K >> 1);
  const uint8_t* sw = a.w2_scales + row * (K >> 4);
  const _Float16* xr[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int slot = 8 * c + (i & 7);
    xr[c] = slot < Te ? b_row(a.h16, a.h16_lo, off + slot, K, kl0, i) : nullptr;
  }
  f32x4_t acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const f16x8_t zero8 = {};
  for (int kk = 0; kk < KL; kk += 32) {
    u32x4_t c0;
    uint32_t s0;
    load_unit(cw, sw, kl0 + kk, c0, s0);
    f16x8_t wv[4];
    sd::dequant_unit(c0, s0, wv);
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      if (c >= nct) break;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f16x8_t bx = xr[c] != nullptr ? *(const f16x8_t*)(xr[c] + kk + 8 * m) : zero8;
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv[m], bx, acc[c], 0, 0, 0);
      }
    }
  }
  if (KS > 1) {
    if (wave > 0) {
#pragma unroll
      for (int c = 0; c < NCT; ++c) red[wave - 1][c][lane] = acc[c];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int w = 0; w < KS - 1; ++w) acc[c] += red[w][c][lane];
  }
#pragma unroll
  for (int c = 0; c < NCT; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[c][r] += __shfl_xor(acc[c][r], 8, 64);
  if (i >= 8) return;
  const float sc = SD_X16_UNSCALE * a.w2_gscale[e];
  const int n = nt * 16 + 4 * G;
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int slot = 8 * c + i;
    if (slot >= Te) continue;
    *(f32x4_t*)(a.y + (size_t)(off + slot) * a.H + n) = acc[c] * sc;
  }
}

// ---------------------------------------------------------------- unpooler
// out[t, n] = sum_j w[t, j] * y[slot_of[t, j], n], j in order, fp32.  4 features/thread.
__global__ __launch_bounds__(256) void k_unpool(int H, int k, const float* __restrict__ y,
                                                const float* __restrict__ w,
                                                const int* __restrict__ slot_of,
                                                float* __restrict__ out) {
  const int t = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const float wj = w[t * k + j];
    const f32x4_t v = *(const f32x4_t*)(y + (size_t)slot_of[t * k + j] * H + n);
    acc += wj * v;
  }
  *(f32x4_t*)(out + (size_t)t * H + n) = acc;
}

// ---------------------------------------------------------------- debug dequant
__global__ __launch_bounds__(256) void k_debug_dequant(int n, int k, const uint8_t* codes,
                                                       const uint8_t* scales, float gscale,
                                                       float* out) {
  const int units = k / 32;
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u >= n * units) return;
  const int row = u / units, kk = (u - row * units) * 32;
  u32x4_t c;
  uint32_t s;
  load_unit(codes + (size_t)row * (k >> 1), scales + (size_t)row * (k >> 4), kk, c, s);
  f16x8_t wv[4];
  sd::dequant_unit(c, s, wv);
  float* o = out + (size_t)row * k + kk;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[8 * m + e] = (float)wv[m][e] * gscale;
}

template <int NCT>
hipError_t launch_experts_nct(const MoeArgs& a, hipStream_t st) {
  auto ks_for = [](int K) { return K % 512 == 0 ? 4 : (K % 256 == 0 ? 2 : 1); };
  const int ks13 = ks_for(a.H), ks2 = ks_for(a.I);
  const dim3 g13(a.I / 16, a.E), g2(a.H / 16, a.E);
  if (ks13 == 4) hipLaunchKernelGGL((k_moe_w13<NCT, 4>), g13, dim3(256), 0, st, a);
  else if (ks13 == 2) hipLaunchKernelGGL((k_moe_w13<NCT, 2>), g13, dim3(128), 0, st, a);
  else hipLaunchKernelGGL((k_moe_w13<NCT, 1>), g13, dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ks2 == 4) hipLaunchKernelGGL((k_moe_w2<NCT, 4>), g2, dim3(256), 0, st, a);
  else if (ks2 == 2) hipLaunchKernelGGL((k_moe_w2<NCT, 2>), g2, dim3(128), 0, st, a);
  else hipLaunchKernelGGL((k_moe_w2<NCT, 1>), g2, dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_pool(const float* z, int b, int E, int k, int* ids, float* w,
                             int* counts, int* offsets, int* slot_of, int* tos, int* active,
                             hipStream_t st) {
  hipLaunchKernelGGL(k_route_pool, dim3(1), dim3(256), 0, st, z, b, E, k, ids, w, counts,
                     offsets, slot_of, tos, active);
  return hipGetLastError();
}

hipError_t launch_moe_experts(const MoeArgs& a, hipStream_t st) {
  // a token chooses an expert at most once, so an expert holds at most b pooled tokens
  if (a.b <= 8) return launch_experts_nct<1>(a, st);
  if (a.b <= 16) return launch_experts_nct<2>(a, st);
  if (a.b <= 32) return launch_experts_nct<4>(a, st);
  return launch_experts_nct<8>(a, st);
}

hipError_t launch_unpool(int b, int H, int k, const float* y, const float* w, const int* slot_of,
                         float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_unpool, dim3((H / 4 + 255) / 256, b), dim3(256), 0, st, H, k, y, w,
                     slot_of, out);
  return hipGetLastError();
}

hipError_t launch_debug_dequant(int n, int k, const uint8_t* codes, const uint8_t* scales,
                                float gscale, float* out, hipStream_t st) {
  const int units = n * (k / 32);
  hipLaunchKernelGGL(k_debug_dequant, dim3((units + 255) / 256), dim3(256), 0, st, n, k, codes,
                     scales, gscale, out);
  return hipGetLastError();
}
