// K-B: skinny bf16 GEMM for the step's dense projections (QKV, o_proj, router, lm_head),
// y[m, n] = sum_k x[m, k] * W[n, k] with M <= 64 rows, on v_mfma_f32_16x16x32_bf16.
//
// Weights are stored packed in the order the matrix cores consume them: the 16 x 32 tile
// (rows 16nt.., columns 32kt..) is 1 KB of contiguous bf16, lane l's A operand (row l%16,
// columns 8(l/16) .. +7) at bytes 16l .. 16l+15.  Every weight load instruction of a wave
// is therefore one contiguous 1 KB piece, which streams at close to the HBM rate.
//
// Persistent kernel (M <= 64): a grid of one workgroup per CU walks the 16-row tiles; its
// NW waves split K (and the grid splits K ksplit ways) and keep their slice of the
// activations, NCT column tiles of 8 rows (16 without lo terms), in registers for the whole
// launch; the next tile's weights are loaded while the current one is reduced, so the
// weight stream never drains and the activations are read once per workgroup.  Shapes it
// cannot hold: one workgroup per tile, activations re-read per tile from L2.  Activation rows past M are
// read through buffer loads whose range check returns zero without a memory access.
//
// SPLIT: x carries bf16 hi/lo terms, 8 rows per column tile (columns 0-7 hi, 8-15 lo),
// summed in the epilogue.
//
// Also here: the weight packing, the QKV front's per-head epilogue (weightless qk RMSNorm,
// RoPE, bf16 K/V cache write) and the draft head's argmax reduction.
#include "sd_common.h"

namespace {

using sd::kOob;
using sd::kStream;
using sd::rsrc;


__device__ __forceinline__ bf16x8_t buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ bf16x8_t buf_load8_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStream));
}


// Byte offset of the lane's activation row `m` at column k (kOob when m >= M).
__device__ __forceinline__ uint32_t x_off(int m, int M, int K, int k) {
  return m < M ? (uint32_t)(((size_t)m * K + k) * 2) : kOob;
}

// Epilogue of one 16-feature tile: lane (i, g) holds y[m = RPC*c + i][n = 16 t + 4g + r].
template <int MODE>
__device__ __forceinline__ void store_tile(const GemmArgs& a, int m, int tile, int ntiles,
                                           int g, f32x4_t v) {
  const int nb = tile * 16 + 4 * g;
  const bool mv = m < a.M;
  if (MODE == GEMM_F32 || MODE == GEMM_F32_BIAS) {
    if (!mv) return;
    if (MODE == GEMM_F32_BIAS && a.bias != nullptr) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (nb + r < a.N) v[r] += a.bias[(size_t)m * a.N + nb + r];
    }
    float* y = (float*)a.y + (size_t)m * a.N + nb;
    if (nb + 3 < a.N) {
      *(f32x4_t*)y = v;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (nb + r < a.N) y[r] = v[r];
    }
  } else {  // GEMM_HEAD: bf16 logits, optional transform, per-tile argmax (ties: low index)
    float best = -INFINITY;
    int bidx = nb;  // always a valid index, even if every logit is NaN
    f32x4_t tau;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lg = sd::bf2f(sd::f2bf(v[r]));
      if (lg > best) { best = lg; bidx = nb + r; }
      const float x = lg * a.multiplier;
      tau[r] = a.soft_cap > 0.f ? a.soft_cap * tanhf(x / a.soft_cap) : x;
    }
    if (mv && a.y != nullptr) *(f32x4_t*)((float*)a.y + (size_t)m * a.N + nb) = tau;
    auto take = [&](float ov, int oi) {
      if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
    };
    take(sd::lane_xor<16>(best), sd::lane_xor<16>(bidx));
    take(sd::lane_xor<32>(best), sd::lane_xor<32>(bidx));
    if (mv && g == 0) {
      a.head_val[(size_t)m * ntiles + tile] = best;
      a.head_idx[(size_t)m * ntiles + tile] = bidx;
    }
  }
}

// Persistent kernel, NCT column tiles: wave w owns K steps [w S, (w+1) S) of every tile.
// Workgroup w owns K slice ks = w % ksplit (wave v: steps ks * KT / ksplit + v S ..) of the
// tiles w / ksplit + j * (grid / ksplit); slice ks writes partial ks of the output, which
// the consumer sums in slice order.
template <int NCT, int NW, int S, int MODE, bool SPLIT>
__global__ __launch_bounds__(64 * NW) void k_gemm_res(GemmArgs a, int ntiles) {
  constexpr int RPC = SPLIT ? 8 : 16;  // activation rows per column tile
  __shared__ f32x4_t red[2][NW - 1][NCT][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const int KT = a.K >> 5;
  const int ks = blockIdx.x % a.ksplit, grp = blockIdx.x / a.ksplit;
  const int ngrp = gridDim.x / a.ksplit;
  const int kt0 = ks * (KT / a.ksplit) + wave * S;
  // activations: hi terms at x, lo terms x_lo_off bytes further in the same buffer
  const uint32_t xbytes = (uint32_t)(a.M * a.K * 2);
  const auto rx = rsrc(a.x, (SPLIT ? a.x_lo_off : 0u) + xbytes);
  const int m = SPLIT ? (i & 7) : i;  // the lane's row within a column tile
  const bool lo = SPLIT && (i >> 3);
  bf16x8_t bv[NCT][S];
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const uint32_t ob = x_off(RPC * c + m, a.M, a.K, kt0 * 32 + 8 * g);
    const uint32_t ox = ob == kOob ? kOob : ob + (lo ? a.x_lo_off : 0u);
#pragma unroll
    for (int u = 0; u < S; ++u) bv[c][u] = buf_load8(rx, ox + 64 * u);
  }
  GemmArgs ap = a;
  if (MODE != GEMM_HEAD && MODE != GEMM_SWIGLU) ap.y = (float*)a.y + (size_t)ks * a.M * a.N;
  f32x4_t gsave = f32x4_t{0.f, 0.f, 0.f, 0.f};  // GEMM_SWIGLU: the finishing wave's gate sums

  // weights through a buffer resource: a tile index past the last loads zeros without a
  // memory access, so the prefetch of a missing next tile needs no branch and every wait
  // before a tile's MFMAs covers exactly that tile
  const auto rw = rsrc(a.w, (uint32_t)((size_t)ntiles * KT * 1024));
  bf16x8_t A0[S], A1[S];
  auto load = [&](bf16x8_t (&A)[S], int tile) {
    const uint32_t o0 = tile < ntiles ? (uint32_t)(((size_t)tile * KT + kt0) * 1024 + lane * 16) : kOob;
#pragma unroll
    for (int u = 0; u < S; ++u) A[u] = buf_load8_nt(rw, o0 + 1024 * u);
  };
  auto finish = [&](bf16x8_t (&A)[S], int tile, int buf) {
    f32x4_t acc[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < S; ++u)
#pragma unroll
      for (int c = 0; c < NCT; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[u], bv[c][u], acc[c], 0, 0, 0);
    // column tile c is finished by wave c % NW: the other waves leave their partials of it
    // in LDS (in their wave order), so with several column tiles the sums and stores are
    // spread over the waves instead of all falling on one
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int o = c % NW;
      if (wave != o) red[buf][wave - (wave > o ? 1 : 0)][c][lane] = acc[c];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      if (wave != c % NW) continue;  // wave-uniform
      f32x4_t v = acc[c];
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) v += red[buf][w][c][lane];
      if (SPLIT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += sd::lane_xor<8>(v[r]);
      }
      if constexpr (MODE == GEMM_SWIGLU) {
        // buffer 0 finishes the gate tile, buffer 1 the up tile of the same columns
        if (buf == 0) {
          gsave = v;
        } else if ((!SPLIT || i < 8) && RPC * c + m < a.M) {
          uint16_t hh[4], hl[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sd::split_bf16(gsave[r] / (1.0f + __expf(-gsave[r])) * v[r], hh[r], hl[r]);
          const size_t o = (size_t)(RPC * c + m) * (a.N >> 1) + tile * 16 + 4 * g;
          *(u32x2_t*)((uint16_t*)a.y + o) = u32x2_t{hh[0] | ((uint32_t)hh[1] << 16), hh[2] | ((uint32_t)hh[3] << 16)};
          *(u32x2_t*)(a.y_lo + o) = u32x2_t{hl[0] | ((uint32_t)hl[1] << 16), hl[2] | ((uint32_t)hl[3] << 16)};
        }
      } else {
        if (!SPLIT || i < 8) store_tile<MODE>(ap, RPC * c + m, tile, ntiles, g, v);
      }
    }
  };
  if constexpr (MODE == GEMM_SWIGLU) {
    // column tile pairs p: gate tile p, then up tile p + NTG, into the two buffers in turn
    const int NTG = ntiles >> 1;
    int p = grp;
    if (p >= NTG) return;  // uniform per workgroup
    load(A0, p);
    while (true) {
      load(A1, p + NTG);
      finish(A0, p, 0);
      const int pn = p + ngrp;
      load(A0, pn < NTG ? pn : ntiles);  // past the last pair: zeros, no memory access
      finish(A1, p, 1);
      if (pn >= NTG) break;
      p = pn;
    }
    return;
  }
  int t = grp;
  if (t >= ntiles) return;  // uniform per workgroup
  load(A0, t);
  while (true) {
    const int t1 = t + ngrp;
    load(A1, t1);
    finish(A0, t, 0);
    if (t1 >= ntiles) break;
    const int t2 = t1 + ngrp;
    load(A0, t2);
    finish(A1, t1, 1);
    if (t2 >= ntiles) break;
    t = t2;
  }
}

// One workgroup per tile, NCT column tiles (M up to 64): NW waves split K, each in passes
// of S steps whose weight and activation loads are all issued before the first MFMA.
template <int NCT, int NW, int S, int MODE, bool SPLIT>
__global__ __launch_bounds__(64 * NW) void k_gemm_tile(GemmArgs a) {
  constexpr int RPC = SPLIT ? 8 : 16;  // activation rows per column tile
  __shared__ f32x4_t red[NW - 1][NCT][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x;
  const int KT = a.K >> 5;
  const int KTW = KT / NW;  // steps per wave
  const int kt0 = wave * KTW;
  const uint32_t xbytes = (uint32_t)(a.M * a.K * 2);
  const auto rx = rsrc(a.x, (SPLIT ? a.x_lo_off : 0u) + xbytes);
  const bool lo = SPLIT && (i >> 3);
  uint32_t ox[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const uint32_t ob = x_off(RPC * c + (SPLIT ? (i & 7) : i), a.M, a.K, kt0 * 32 + 8 * g);
    ox[c] = ob == kOob ? kOob : ob + (lo ? a.x_lo_off : 0u);
  }
  const uint16_t* wt = a.w + ((size_t)tile * KT + kt0) * 512 + lane * 8;
  f32x4_t acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int passes = KTW / S;
  for (int p = 0; p < passes; ++p) {
    bf16x8_t av[S];
    bf16x8_t bv[S][NCT];
#pragma unroll
    for (int u = 0; u < S; ++u)
      av[u] = __builtin_nontemporal_load((const bf16x8_t*)(wt + (size_t)(p * S + u) * 512));
#pragma unroll
    for (int u = 0; u < S; ++u)
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        bv[u][c] = buf_load8(rx, ox[c] + (uint32_t)(p * S + u) * 64);
      }
#pragma unroll
    for (int u = 0; u < S; ++u)
#pragma unroll
      for (int c = 0; c < NCT; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[u][c], acc[c], 0, 0, 0);
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
      for (int r = 0; r < 4; ++r) acc[c][r] += sd::lane_xor<8>(acc[c][r]);
    }
  }
  if (SPLIT && i >= 8) return;
#pragma unroll
  for (int c = 0; c < NCT; ++c) store_tile<MODE>(a, RPC * c + i, tile, gridDim.x, g, acc[c]);
}

int cu_count() {
  static int n[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (n[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    n[dev] = v;
  }
  return n[dev];
}

// Whether k_gemm_res<NCT, NW, S> fits one workgroup per CU: the resident activations
// (NCT x S operands a lane) within the registers, the cross-wave reduction within LDS.
// Registers a lane: activations 4 NCT S, two weight buffers 8 S, accumulators 4 NCT, and
// about 40 more; 512 threads allow 256, 1024 allow 128.
constexpr bool res_fits(int NCT, int NW, int S) {
  return (NCT == 1 ? (S <= 16 && !(NW > 8 && S == 16))
                   : 4 * NCT * S + 8 * S + 4 * NCT + 40 <= (NW > 8 ? 128 : 256)) &&
         2 * (NW - 1) * NCT <= 120;  // KB of reduction buffers
}

template <int NCT, int NW, int S, int MODE, bool SPLIT>
bool launch_res_s(const GemmArgs& a, int ntiles, int grid, hipStream_t st) {
  if constexpr (!res_fits(NCT, NW, S)) {
    return false;
  } else {
    hipLaunchKernelGGL((k_gemm_res<NCT, NW, S, MODE, SPLIT>), dim3(grid), dim3(64 * NW), 0, st,
                       a, ntiles);
    return true;
  }
}

template <int NCT, int NW, int MODE, bool SPLIT>
bool try_res(const GemmArgs& a, int ntiles, hipStream_t st) {
  const int KT = a.K / 32;
  if (KT % (NW * a.ksplit)) return false;
  if ((size_t)ntiles * KT * 1024 >= 0x80000000u) return false;  // buffer offsets are 32-bit
  const int grid = (min(ntiles * a.ksplit, cu_count()) / a.ksplit) * a.ksplit;
  if (grid < a.ksplit) return false;
  switch (KT / (NW * a.ksplit)) {
    case 16: return launch_res_s<NCT, NW, 16, MODE, SPLIT>(a, ntiles, grid, st);
    case 8: return launch_res_s<NCT, NW, 8, MODE, SPLIT>(a, ntiles, grid, st);
    case 4: return launch_res_s<NCT, NW, 4, MODE, SPLIT>(a, ntiles, grid, st);
    case 2: return launch_res_s<NCT, NW, 2, MODE, SPLIT>(a, ntiles, grid, st);
    case 1: return launch_res_s<NCT, NW, 1, MODE, SPLIT>(a, ntiles, grid, st);
    default: return false;
  }
}

template <int NCT, int MODE, bool SPLIT>
bool try_res_nw(const GemmArgs& a, int ntiles, hipStream_t st) {
  return try_res<NCT, 8, MODE, SPLIT>(a, ntiles, st) || try_res<NCT, 16, MODE, SPLIT>(a, ntiles, st) ||
         try_res<NCT, 4, MODE, SPLIT>(a, ntiles, st);
}

template <int NCT, int NW, int MODE, bool SPLIT>
void launch_tile_s(const GemmArgs& a, int ntiles, hipStream_t st) {
  // pass size: divides the steps per wave and bounds the in-flight registers
  constexpr int SCAP = NCT >= 8 ? 2 : 16 / NCT;
  const int steps = a.K / NW / 32;
  const dim3 grid(ntiles), block(64 * NW);
  if (SCAP >= 16 && steps % 16 == 0)
    hipLaunchKernelGGL((k_gemm_tile<NCT, NW, (SCAP >= 16 ? 16 : 1), MODE, SPLIT>), grid, block, 0, st, a);
  else if (SCAP >= 8 && steps % 8 == 0)
    hipLaunchKernelGGL((k_gemm_tile<NCT, NW, (SCAP >= 8 ? 8 : 1), MODE, SPLIT>), grid, block, 0, st, a);
  else if (SCAP >= 4 && steps % 4 == 0)
    hipLaunchKernelGGL((k_gemm_tile<NCT, NW, (SCAP >= 4 ? 4 : 1), MODE, SPLIT>), grid, block, 0, st, a);
  else if (steps % 2 == 0)
    hipLaunchKernelGGL((k_gemm_tile<NCT, NW, 2, MODE, SPLIT>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm_tile<NCT, NW, 1, MODE, SPLIT>), grid, block, 0, st, a);
}

template <int NCT, int MODE, bool SPLIT>
hipError_t launch_tile(const GemmArgs& a, int ntiles, hipStream_t st) {
  if (a.K % 256 == 0) launch_tile_s<NCT, 8, MODE, SPLIT>(a, ntiles, st);
  else launch_tile_s<NCT, 4, MODE, SPLIT>(a, ntiles, st);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_m(const GemmArgs& in, hipStream_t st) {
  GemmArgs a = in;
  const int ntiles = (a.N + 15) / 16;
  if (a.ksplit < 1 || (MODE == GEMM_HEAD && a.ksplit != 1)) return hipErrorInvalidValue;
  if (a.x_lo != nullptr) {
    // lo terms must follow the hi terms in one buffer (the workspace lays them out so)
    const ptrdiff_t off = (const char*)a.x_lo - (const char*)a.x;
    if (MODE == GEMM_HEAD || off < (ptrdiff_t)a.M * a.K * 2 || off + (ptrdiff_t)a.M * a.K * 2 >= 0x80000000LL)
      return hipErrorInvalidValue;
    a.x_lo_off = (uint32_t)off;
  } else {
    a.x_lo_off = 0;
  }
  if constexpr (MODE == GEMM_SWIGLU) {
    // one column tile of rows (the gate sums wait in the finishing wave's registers for the
    // up tile), one K slice, the persistent kernel only
    if (!gemm_swiglu_ok(a.M, a.N, a.K, a.x_lo != nullptr) || a.ksplit != 1 || a.y_lo == nullptr)
      return hipErrorInvalidValue;
    const bool res = a.x_lo != nullptr ? try_res_nw<1, MODE, true>(a, ntiles, st)
                                       : try_res_nw<1, MODE, false>(a, ntiles, st);
    return res ? hipGetLastError() : hipErrorInvalidValue;
  } else {
  // the persistent kernel takes any K slicing; the per-tile kernel only whole K
  if (a.x_lo != nullptr) {
    const bool res = a.M <= 8    ? try_res_nw<1, MODE, true>(a, ntiles, st)
                     : a.M <= 16 ? try_res_nw<2, MODE, true>(a, ntiles, st)
                     : a.M <= 32 ? try_res_nw<4, MODE, true>(a, ntiles, st)
                                 : try_res_nw<8, MODE, true>(a, ntiles, st);
    if (res) return hipGetLastError();
    if (a.ksplit != 1) return hipErrorInvalidValue;
    if (a.M <= 8) return launch_tile<1, MODE, true>(a, ntiles, st);
    if (a.M <= 16) return launch_tile<2, MODE, true>(a, ntiles, st);
    if (a.M <= 32) return launch_tile<4, MODE, true>(a, ntiles, st);
    return launch_tile<8, MODE, true>(a, ntiles, st);
  }
  const bool res = a.M <= 16   ? try_res_nw<1, MODE, false>(a, ntiles, st)
                   : a.M <= 32 ? try_res_nw<2, MODE, false>(a, ntiles, st)
                               : try_res_nw<4, MODE, false>(a, ntiles, st);
  if (res) return hipGetLastError();
  if (a.ksplit != 1) return hipErrorInvalidValue;
  if (a.M <= 16) return launch_tile<1, MODE, false>(a, ntiles, st);
  if (a.M <= 32) return launch_tile<2, MODE, false>(a, ntiles, st);
  return launch_tile<4, MODE, false>(a, ntiles, st);
  }
}

// Row-major bf16 [N, K] -> packed tiles (rows past N are zero).  One thread per 16 bytes.
__global__ __launch_bounds__(256) void k_pack_dense(int N, int K, const uint16_t* __restrict__ src,
                                                    uint16_t* __restrict__ dst, size_t nchunks) {
  const int KT = K >> 5;
  for (size_t c = (size_t)blockIdx.x * 256 + threadIdx.x; c < nchunks;
       c += (size_t)gridDim.x * 256) {
    const size_t tile = c >> 6;
    const int l = (int)(c & 63);
    const size_t row = (tile / KT) * 16 + (l & 15);
    const int k = (int)(tile % KT) * 32 + 8 * (l >> 4);
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (row < (size_t)N) v = *(const u32x4_t*)(src + row * K + k);
    *(u32x4_t*)(dst + c * 8) = v;
  }
}

// Row-major block-scaled FP4 [E, N, K] -> packed tiles of 16 rows x 128 weights: 1 KB of
// codes (lane l: 16 code bytes of row l%16 at weight 32(l/16)) and 128 B of scales (lane l:
// its 2 scale bytes).  One thread per (tile, lane).
__global__ __launch_bounds__(256) void k_pack_fp4(int N, int K, const uint8_t* __restrict__ codes,
                                                  const uint8_t* __restrict__ scales,
                                                  uint8_t* __restrict__ codes_out,
                                                  uint8_t* __restrict__ scales_out,
                                                  size_t nlanes) {
  const int KT = K >> 7;
  for (size_t c = (size_t)blockIdx.x * 256 + threadIdx.x; c < nlanes;
       c += (size_t)gridDim.x * 256) {
    const size_t tile = c >> 6;
    const int l = (int)(c & 63);
    const size_t row = (tile / KT) * 16 + (l & 15);  // rows of all matrices, expert-major
    const int kt = (int)(tile % KT);
    *(u32x4_t*)(codes_out + c * 16) =
        *(const u32x4_t*)(codes + row * (K >> 1) + 64 * kt + 16 * (l >> 4));
    *(uint16_t*)(scales_out + c * 2) =
        *(const uint16_t*)(scales + row * (K >> 4) + 8 * kt + 2 * (l >> 4));
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
  auto take = [&](float ov, int oi) {
    if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
  };
  take(sd::lane_xor<32>(best), sd::lane_xor<32>(bi));
  take(sd::lane_xor<16>(best), sd::lane_xor<16>(bi));
  take(sd::lane_xor<8>(best), sd::lane_xor<8>(bi));
  take(sd::lane_xor<4>(best), sd::lane_xor<4>(bi));
  take(sd::lane_xor<2>(best), sd::lane_xor<2>(bi));
  take(sd::lane_xor<1>(best), sd::lane_xor<1>(bi));
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
    case GEMM_F32_BIAS: return launch_m<GEMM_F32_BIAS>(a, st);
    case GEMM_HEAD: return launch_m<GEMM_HEAD>(a, st);
    case GEMM_SWIGLU: return launch_m<GEMM_SWIGLU>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_pack_dense(int N, int K, const uint16_t* src, uint16_t* dst, hipStream_t st) {
  const size_t nchunks = (size_t)((N + 15) / 16) * 16 * K / 8;
  const size_t blocks = (nchunks + 255) / 256;
  hipLaunchKernelGGL(k_pack_dense, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256),
                     0, st, N, K, src, dst, nchunks);
  return hipGetLastError();
}

hipError_t launch_pack_fp4(int E, int N, int K, const uint8_t* codes, const uint8_t* scales,
                           uint8_t* codes_out, uint8_t* scales_out, hipStream_t st) {
  const size_t nlanes = (size_t)E * N * K / 128 / 16 * 64;
  const size_t blocks = (nlanes + 255) / 256;
  hipLaunchKernelGGL(k_pack_fp4, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256),
                     0, st, N, K, codes, scales, codes_out, scales_out, nlanes);
  return hipGetLastError();
}

bool gemm_swiglu_ok(int M, int N, int K, bool lo) {
  if (M < 1 || M > (lo ? 8 : 16) || N % 32 != 0 || K % 32 != 0) return false;
  const int KT = K / 32, ntiles = N / 16;
  if ((size_t)ntiles * KT * 1024 >= 0x80000000u) return false;
  for (int nw : {8, 16, 4}) {
    if (KT % nw) continue;
    const int S = KT / nw;
    if ((S == 1 || S == 2 || S == 4 || S == 8 || S == 16) && res_fits(1, nw, S)) return true;
  }
  return false;
}

bool gemm_split_ok(int M, int N, int K, bool lo, int ksplit) {
  if (ksplit == 1) return true;
  const int rpc = lo ? 8 : 16;  // the persistent kernel's column tiles, as launch_m picks them
  const int nct = M <= rpc ? 1 : M <= 2 * rpc ? 2 : M <= 4 * rpc ? 4 : (lo && M <= 8 * rpc) ? 8 : 0;
  if (nct == 0 || M > 64 || K % 32) return false;
  const int KT = K / 32, ntiles = (N + 15) / 16;
  if ((size_t)ntiles * KT * 1024 >= 0x80000000u || ntiles * ksplit < ksplit) return false;
  for (int nw : {8, 16, 4}) {
    if (KT % (nw * ksplit)) continue;
    const int S = KT / (nw * ksplit);
    if ((S == 1 || S == 2 || S == 4 || S == 8 || S == 16) && res_fits(nct, nw, S)) return true;
  }
  return false;
}

hipError_t launch_head_argmax(int b, int n_tiles, const float* val, const int* idx,
                              const int64_t* d2t, int32_t* ids, int64_t* target,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_head_argmax, dim3(b), dim3(256), 0, st, n_tiles, n_tiles * 16, val, idx,
                     d2t, ids, target);
  return hipGetLastError();
}
