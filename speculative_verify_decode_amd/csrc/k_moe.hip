// K-D .. K-G: routing, pooler, routed FP4 experts and the weighted unpooler.
//
// Page "vllm.models.muse_spark.nvidia.specialized_decode.runtime.decode", module
// docstring: the MoE block is router -> routing -> pooler -> routed experts -> tail ->
// unpooler (the tail is a cross-rank combine and is the identity on one GPU).  The
// routed experts are NVFP4 (page "vllm.models.muse_spark.nvidia.specialized_decode.
// runtime", module list: expert_tp).
//
// Expert GEMMs: workgroup (16-feature tile, active expert) with KS waves splitting K.
// Weights are the A operand of v_mfma_f32_16x16x32_f16, dequantised exactly in registers.
// Each load instruction covers 64 contiguous code bytes of each of 16 rows (4 lanes per
// row, 32 weights per lane) and a wave issues all of its weight loads before it waits on
// any, so the whole K slice of the tile is in flight at once.  The pooled tokens of the
// expert are the B operand, 8 per column tile as hi/lo fp16 terms (columns 0-7 / 8-15).
// Workgroups are indexed by the ascending active-expert list, so the grid's live part is
// dispatched first and the rest exits at once.
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
  __shared__ float s_z[64 * 256 + 1];
  __shared__ int s_ids[64 * 8];
  __shared__ int s_cnt[256];
  __shared__ int s_off[257];
  const int tid = threadIdx.x;
  for (int p = tid; p < b * E; p += 256) {
    const float v = z[p];
    s_z[p] = v != v ? -INFINITY : v;  // NaN ranks last
  }
  __syncthreads();
  if (tid < b) {
    const float* zr = s_z + tid * E;
    float prev_v = INFINITY;
    int prev_i = -1;
    float sel[8];
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = -1;
      for (int e = 0; e < E; ++e) {
        const float v = zr[e];
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
// One wave's share of a 16-row weight tile: NU groups of 128 weights per row.  Lane (i, G)
// holds weights kw0 + 128u + 32G + [0, 32) of row i: 16 code bytes and 2 scale bytes per
// group, so each load instruction covers 64 contiguous code bytes of each of the 16 rows.
template <int NU>
struct RowSlice {
  u32x4_t codes[NU];
  uint32_t scales[NU];
};

template <int NU>
__device__ __forceinline__ void load_slice(RowSlice<NU>& s, const uint8_t* codes_row,
                                           const uint8_t* scale_row, int kw0, int G) {
  const uint8_t* c = codes_row + (kw0 >> 1) + 16 * G;
  const uint8_t* sc = scale_row + (kw0 >> 4) + 2 * G;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    s.codes[u] = __builtin_nontemporal_load((const u32x4_t*)(c + 64 * u));
    s.scales[u] = *(const uint16_t*)(sc + 8 * u);
  }
}

// B operand of one column tile: lane column i holds a pooled token (hi term for i < 8, lo
// term for i >= 8); f16x8 m of group u covers k = kw0 + 128u + 32G + 8m.  `row` is always
// a valid row (invalid lanes read row 0) and `valid` zeroes the operand after the loads.
template <int NU>
__device__ __forceinline__ void load_b(f16x8_t (&bx)[NU][4], const _Float16* row, bool valid) {
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int m = 0; m < 4; ++m) bx[u][m] = *(const f16x8_t*)(row + 128 * u + 8 * m);
  if (!valid) {
    const f16x8_t zero8 = {};
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int m = 0; m < 4; ++m) bx[u][m] = zero8;
  }
}

// W13 (gate rows [0, I), up rows [I, 2I)) + SwiGLU.  KS waves split K = H, NU = H/(128 KS).
template <int NCT, int NU, int KS>
__global__ __launch_bounds__(64 * KS) void k_moe_w13(MoeArgs a) {
  __shared__ f32x4_t red[KS > 1 ? KS - 1 : 1][2][NCT][64];
  if ((int)blockIdx.y >= a.active[a.E]) return;
  const int e = a.active[blockIdx.y];
  const int nt = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = lane & 15, G = lane >> 4;
  const int K = a.H;
  const int kw0 = wave * (NU * 128);
  const size_t rowg = (size_t)e * 2 * a.I + nt * 16 + i;
  const size_t rowu = rowg + a.I;
  RowSlice<NU> wg, wu;
  load_slice<NU>(wg, a.w13_codes + rowg * (K >> 1), a.w13_scales + rowg * (K >> 4), kw0, G);
  load_slice<NU>(wu, a.w13_codes + rowu * (K >> 1), a.w13_scales + rowu * (K >> 4), kw0, G);
  const int Te = a.counts[e];
  const int off = a.offsets[e];
  const int nct = (Te + 7) >> 3;
  f32x4_t ag[NCT], au[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) ag[c] = au[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    if (c >= nct) break;
    const int slot = 8 * c + (i & 7);
    const bool lo = (i >> 3) != 0;
    const bool valid = slot < Te && (!lo || a.x16_lo != nullptr);
    const _Float16* base = (lo && a.x16_lo != nullptr) ? a.x16_lo : a.x16;
    // the tile's 8 token ids through uniform (scalar) loads, which do not queue behind the
    // weight loads; each lane then selects its own
    int tok = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = (8 * c + j < Te) ? a.tos[off + 8 * c + j] : 0;
      tok = ((i & 7) == j) ? t : tok;
    }
    tok = valid ? tok : 0;
    f16x8_t bx[NU][4];
    load_b<NU>(bx, base + (size_t)tok * K + kw0 + 32 * G, valid);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      f16x8_t dg[4], du[4];
      sd::dequant_unit(wg.codes[u], wg.scales[u], dg);
      sd::dequant_unit(wu.codes[u], wu.scales[u], du);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        ag[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dg[m], bx[u][m], ag[c], 0, 0, 0);
        au[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(du[m], bx[u][m], au[c], 0, 0, 0);
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

// W2: y[slot, n] = h[slot] . W2_e[n], fp32.  KS waves split K = I, NU = I/(128 KS).
template <int NCT, int NU, int KS>
__global__ __launch_bounds__(64 * KS) void k_moe_w2(MoeArgs a) {
  __shared__ f32x4_t red[KS > 1 ? KS - 1 : 1][NCT][64];
  if ((int)blockIdx.y >= a.active[a.E]) return;
  const int e = a.active[blockIdx.y];
  const int nt = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = lane & 15, G = lane >> 4;
  const int K = a.I;
  const int kw0 = wave * (NU * 128);
  const size_t row = (size_t)e * a.H + nt * 16 + i;
  RowSlice<NU> wv;
  load_slice<NU>(wv, a.w2_codes + row * (K >> 1), a.w2_scales + row * (K >> 4), kw0, G);
  const int Te = a.counts[e];
  const int off = a.offsets[e];
  const int nct = (Te + 7) >> 3;
  f32x4_t acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    if (c >= nct) break;
    const int slot = 8 * c + (i & 7);
    const bool valid = slot < Te;
    const _Float16* base = (i >> 3) ? a.h16_lo : a.h16;
    f16x8_t bx[NU][4];
    load_b<NU>(bx, base + (size_t)(off + (valid ? slot : 0)) * K + kw0 + 32 * G, valid);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      f16x8_t dw[4];
      sd::dequant_unit(wv.codes[u], wv.scales[u], dw);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dw[m], bx[u][m], acc[c], 0, 0, 0);
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
  const u32x4_t c = *(const u32x4_t*)(codes + (size_t)row * (k >> 1) + (kk >> 1));
  const uint32_t s = *(const uint16_t*)(scales + (size_t)row * (k >> 4) + (kk >> 4));
  f16x8_t wv[4];
  sd::dequant_unit(c, s, wv);
  float* o = out + (size_t)row * k + kk;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[8 * m + e] = (float)wv[m][e] * gscale;
}

// A K split of an expert GEMM: K = 128 * NU * KS with NU <= 4 groups per wave.
struct Split { int nu, ks; };
Split split_for(int K) {
  const int g = K / 128;
  for (int ks = 8; ks >= 1; ks >>= 1)
    if (K % 128 == 0 && g % ks == 0 && g / ks >= 1 && g / ks <= 4) return {g / ks, ks};
  return {0, 0};
}

#define SD_SPLITS(X) X(1, 1) X(1, 2) X(1, 4) X(1, 8) X(2, 1) X(2, 2) X(2, 4) X(2, 8) \
                     X(3, 1) X(3, 2) X(3, 4) X(3, 8) X(4, 1) X(4, 2) X(4, 4) X(4, 8)

template <int NCT>
hipError_t launch_experts_nct(const MoeArgs& a, hipStream_t st) {
  const Split s13 = split_for(a.H), s2 = split_for(a.I);
  const dim3 g13(a.I / 16, a.E), g2(a.H / 16, a.E);
  bool done = false;
#define SD_W13(NU, KS)                                                                     \
  if (!done && s13.nu == NU && s13.ks == KS) {                                             \
    hipLaunchKernelGGL((k_moe_w13<NCT, NU, KS>), g13, dim3(64 * KS), 0, st, a);            \
    done = true;                                                                          \
  }
  SD_SPLITS(SD_W13)
#undef SD_W13
  if (!done) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  done = false;
#define SD_W2(NU, KS)                                                                      \
  if (!done && s2.nu == NU && s2.ks == KS) {                                               \
    hipLaunchKernelGGL((k_moe_w2<NCT, NU, KS>), g2, dim3(64 * KS), 0, st, a);              \
    done = true;                                                                          \
  }
  SD_SPLITS(SD_W2)
#undef SD_W2
  if (!done) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

bool moe_shape_supported(int H, int I) { return split_for(H).nu > 0 && split_for(I).nu > 0; }

hipError_t launch_route_pool(const float* z, int b, int E, int k, int* ids, float* w,
                             int* counts, int* offsets, int* slot_of, int* tos, int* active,
                             hipStream_t st) {
  hipLaunchKernelGGL(k_route_pool, dim3(1), dim3(256), 0, st, z, b, E, k, ids, w, counts,
                     offsets, slot_of, tos, active);
  return hipGetLastError();
}

hipError_t launch_moe_experts(const MoeArgs& a, hipStream_t st) {
  // a token chooses an expert at most once, so an expert holds at most b pooled tokens;
  // b <= 8 fits one column tile, larger batches take up to 8 tiles (64 tokens)
  if (a.b <= 8) return launch_experts_nct<1>(a, st);
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
