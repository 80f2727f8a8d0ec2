// K-D .. K-G: routing, pooler, routed FP4 experts and the weighted unpooler.
//
// Page "vllm.models.muse_spark.nvidia.specialized_decode.runtime.decode", module
// docstring: the MoE block is router -> routing -> pooler -> routed experts -> tail ->
// unpooler (the tail is a cross-rank combine and is the identity on one GPU).  The
// routed experts are NVFP4 (page "vllm.models.muse_spark.nvidia.specialized_decode.
// runtime", module list: expert_tp).
//
// Expert GEMMs: the weights are the A operand of v_mfma_f32_16x16x32_f16, dequantised
// exactly in registers from packed tiles, and the pooled tokens of the expert are the B
// operand.  Only the experts the router picked are walked: the work list is the ascending
// active-expert list the pooler writes.
#include <type_traits>

#include "sd_common.h"

namespace {

using sd::kOob;
using sd::kStream;
using sd::rsrc;
using sd::store16;

// ---------------------------------------------------------------- router + routing + pooler
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Phase 1, every workgroup: partial logits of one 16-expert tile over 256 columns of H
// (4 waves x 2 MFMA steps; rows as bf16 hi/lo terms in columns 0-7 / 8-15 of NCT tiles),
// written to part[ks, t, e].  Phase 2, the last workgroup to arrive: z = sum over ks in
// order + bias; top-k per row by (-z, index), each (row, expert) finding its own rank;
// weights = softmax over the selected logits; pooler = stable counting sort of (row,
// choice) by expert,
// through per-expert row bitmasks (a row picks an expert at most once, so an entry's
// rank within its expert is the number of earlier rows in the expert's mask).
// The routing of the last router workgroup: z = sum over ks < KS of part[ks] (in order) +
// bias; top-k per row by (-z, index) with each (row, expert) finding its own rank; weights
// = softmax over the selected logits; pooler = stable counting sort of (row, choice) by
// expert through per-expert row bitmasks (a row picks an expert at most once, so an
// entry's rank within its expert is the number of earlier rows in the expert's mask).
// 256 threads.
struct MoeMeta {
  int active[257];
  int cnt[256];
  int off[256];
  int tos[512];
  float g13[256], g2[256];  // per-expert global scales: an LDS read in the epilogue, not a
                            // global load queued behind the next unit's weights
};

// With expert groups (batches of more than 8 rows): expert e with c pooled rows is
// ceil(c / 8) groups of at most 8 rows (one MFMA column tile each), in active-list order;
// at most E + b k / 8 groups.  Kernels for b <= 8 use the plain MoeMeta (each expert is one
// group), so they carry none of this.
struct MoeMetaG : MoeMeta {
  int ng;
  int gexp[320], goff[320], gcnt[320];
  int wsum[16];
};
template <bool GRP>
using MoeMetaT = typename std::conditional<GRP, MoeMetaG, MoeMeta>::type;

// The expert groups of m's active list (block-wide: block scans over the active list, one
// pass per blockDim.x experts).
__device__ void build_groups(MoeMetaG& m, int E) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int n_act = m.active[E];
  int carry = 0;  // groups of the earlier passes
  for (int a0 = 0; a0 < n_act; a0 += blockDim.x) {  // uniform
    const int t = a0 + tid;
    int e = 0, ng = 0;
    if (t < n_act) {
      e = m.active[t];
      ng = (m.cnt[e] + 7) >> 3;
    }
    const int inc = sd::wave_scan_incl(ng);
    if (lane == 63) m.wsum[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
      if (w < wave) base += m.wsum[w];
      tot += m.wsum[w];
    }
    const int start = carry + base + inc - ng;
    for (int j = 0; j < ng; ++j) {
      m.gexp[start + j] = e;
      m.goff[start + j] = m.off[e] + 8 * j;
      m.gcnt[start + j] = min(8, m.cnt[e] - 8 * j);
    }
    carry += tot;
    __syncthreads();  // wsum is reused by the next pass
  }
  if (tid == 0) m.ng = carry;
  __syncthreads();
}

template <int KEYS>
struct RouteLdsT {
  uint32_t key[KEYS];      // order keys: larger = earlier in (-z, index) order, NaN last
  float sel[512 + 8];      // 8 spare: unrolled reads of a row's k values stay in the array
  int ids[512];
  uint32_t mlo[256], mhi[256];
  int off[257];
  int wc[16], wa[16];
};
using RouteLds = RouteLdsT<64 * 256>;  // b <= 64 rows, E <= 256 experts

// The softmax weight of choice p (row t = p / k) over its row's k selected logits, summed in
// rank order; the ids and weights go to memory.  EMAX > 0: k <= 8, unrolled LDS reads.
template <int EMAX, class RL>
__device__ __forceinline__ void route_weight(const RouterArgs& a, const RL& R, int p) {
  const int k = a.k, t = p / k;
  const float m = R.sel[t * k];
  float den = 0.f;
  if constexpr (EMAX > 0) {
    float sv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sv[j] = R.sel[t * k + j];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) den += expf(sv[j] - m);
  } else {
    for (int j = 0; j < k; ++j) den += expf(R.sel[t * k + j] - m);
  }
  a.ids[p] = R.ids[p];
  a.w_out[p] = expf(R.sel[p] - m) / den;
}

// EMAX > 0: E <= EMAX and k <= 8, ranks and weights from fully unrolled LDS reads.  NT
// threads (a multiple of 64, at least E).  out: write the maps (and the logits) to memory;
// meta (may be null): the expert GEMMs' copy of the maps in LDS (active list, counts,
// offsets, token of each slot).  SOFT false: the ids and softmax weights are left to the
// caller (route_weight over p < b k, after this returns; R keeps what it needs).
template <int EMAX, int NT, bool SOFT = true, class RL>
__device__ void route_phase2(const RouterArgs& a, int KS, RL& R, bool out = true,
                             MoeMeta* meta = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int NW = NT / 64;
  const int b = a.b, E = a.E, k = a.k;
  // z = sum over ks in order + bias, every (row, expert) at once: one round of loads.  The
  // LDS copy is an order key: larger key = earlier in (-z, index) order, NaN last.
  const size_t st = (size_t)b * E;
  // the bias is read unconditionally (the partials stand in when there is none), so its load
  // goes out with the partials' instead of after them
  const float* bias = a.bias != nullptr ? a.bias : a.part;
  auto key_of = [&](int idx) {
    const float bv = bias[idx];
    float z = 0.f;
#pragma unroll 16
    for (int j = 0; j < KS; ++j) z += a.part[j * st + idx];
    if (a.bias != nullptr) z += bv;
    if (out && a.logits != nullptr) a.logits[idx] = z;
    const uint32_t u = __float_as_uint(z == 0.f ? 0.f : z);  // -0 ties with +0
    return z != z ? 0u : (u & 0x80000000u ? ~u : u | 0x80000000u);
  };
  if constexpr (EMAX > 0) {
    // rows of EMAX keys, experts E .. EMAX - 1 padded with key 0
    static_assert((EMAX & (EMAX - 1)) == 0 && EMAX % 8 == 0, "EMAX: a power of two, at least 8");
    for (int p = tid; p < b * EMAX; p += NT) {
      const int t = p / EMAX, e = p & (EMAX - 1);
      R.key[p] = e < E ? key_of(t * E + e) : 0u;
    }
  } else {
    for (int idx = tid; idx < b * E; idx += NT) R.key[idx] = key_of(idx);
  }
  if (tid < E) R.mlo[tid] = R.mhi[tid] = 0u;
  __syncthreads();
  // top-k by rank: (t, e) is choice number rank(t, e) if that is < k, where rank counts the
  // experts of row t ordered before e (larger key, or equal key and lower index).  The
  // logit comes back from its key (key 0: NaN); the softmax sums in rank order.
  auto key_value = [](uint32_t ke) {
    return ke == 0u ? __uint_as_float(0x7fc00000u)
                    : __uint_as_float(ke & 0x80000000u ? ke & 0x7fffffffu : ~ke);
  };
  const int nk = b * k;
  if constexpr (EMAX > 0) {
    for (int p = tid; p < b * EMAX; p += NT) {
      const int t = p / EMAX, e = p & (EMAX - 1);
      if (e >= E) continue;
      const uint32_t* kr = R.key + t * EMAX;
      const uint32_t ke = kr[e];
      // (key, EMAX - 1 - index) as one 64-bit value orders the row as (-z, index) does; a
      // padding entry (key 0 at an index past every expert) orders after every expert
      const uint64_t ce = ((uint64_t)ke << 32) | (uint32_t)(EMAX - 1 - e);
      int rank = 0;
#pragma unroll
      for (int j0 = 0; j0 < EMAX; j0 += 8) {
        if (j0 >= E) break;  // uniform; a row's padding past E in this group counts nothing
#pragma unroll
        for (int j = j0; j < j0 + 8; ++j)
          rank += ((((uint64_t)kr[j]) << 32) | (uint32_t)(EMAX - 1 - j)) > ce ? 1 : 0;
      }
      if (rank < k) {
        R.ids[t * k + rank] = e;
        R.sel[t * k + rank] = key_value(ke);
      }
    }
    __syncthreads();
    for (int p = tid; p < nk; p += NT) {
      const int t = p / k, ex = R.ids[p];
      if (SOFT && out) route_weight<EMAX>(a, R, p);
      atomicOr(t < 32 ? &R.mlo[ex] : &R.mhi[ex], 1u << (t & 31));
    }
  } else {
    for (int p = tid; p < b * E; p += NT) {
      const int t = p / E, e = p - t * E;
      const uint32_t* kr = R.key + t * E;
      const uint32_t ke = kr[e];
      int rank = 0;
      for (int j = 0; j < E; ++j) {
        const uint32_t kj = kr[j];
        rank += (kj > ke || (kj == ke && j < e)) ? 1 : 0;
      }
      if (rank < k) {
        R.ids[t * k + rank] = e;
        R.sel[t * k + rank] = key_value(ke);
      }
    }
    __syncthreads();
    if (SOFT && out)
      for (int p = tid; p < nk; p += NT) route_weight<EMAX>(a, R, p);
    for (int p = tid; p < nk; p += NT) {
      const int t = p / k;
      atomicOr(t < 32 ? &R.mlo[R.ids[p]] : &R.mhi[R.ids[p]], 1u << (t & 31));
    }
  }
  __syncthreads();
  // counts, exclusive offsets and the active list: scans over experts (tid = e), within
  // wave 0 when it holds every expert, else across the block's waves
  const int e = tid;  // NT >= E
  const int cnt = e < E ? __popc(R.mlo[e]) + __popc(R.mhi[e]) : 0;
  const int act = cnt > 0 ? 1 : 0;
  int ic, ia, pc = 0, pa = 0, total, n_act;
  if constexpr (EMAX > 0 && EMAX <= 64) {
    ic = sd::wave_scan_incl(cnt);
    ia = sd::wave_scan_incl(act);
    total = __builtin_amdgcn_readlane(ic, 63);
    n_act = __builtin_amdgcn_readlane(ia, 63);
  } else {
    ic = sd::wave_scan_incl(cnt);
    ia = sd::wave_scan_incl(act);
    if (lane == 63) { R.wc[wave] = ic; R.wa[wave] = ia; }
    __syncthreads();
    total = 0;
    n_act = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) { pc += R.wc[w]; pa += R.wa[w]; }
      total += R.wc[w];
      n_act += R.wa[w];
    }
  }
  const int off = pc + ic - cnt;
  if (e < E) {
    if (out) {
      a.counts[e] = cnt;
      a.offsets[e] = off;
      if (act) a.active[pa + ia - 1] = e;
      if (e >= n_act) a.active[e] = -1;
    }
    if (meta != nullptr) {
      meta->cnt[e] = cnt;
      meta->off[e] = off;
      if (act) meta->active[pa + ia - 1] = e;
      if (e >= n_act) meta->active[e] = -1;
    }
    R.off[e] = off;
  }
  if (tid == 0) {
    if (out) {
      a.offsets[E] = total;
      a.active[E] = n_act;
    }
    if (meta != nullptr) meta->active[E] = n_act;
  }
  __syncthreads();
  for (int p = tid; p < nk; p += NT) {
    const int t = p / k, ex = R.ids[p];
    const int rank = t < 32 ? __popc(R.mlo[ex] & ((1u << t) - 1u))
                            : __popc(R.mlo[ex]) + __popc(R.mhi[ex] & ((1u << (t - 32)) - 1u));
    const int slot = R.off[ex] + rank;
    if (out) {
      a.slot_of[p] = slot;
      a.tos[slot] = t;
    }
    if (meta != nullptr) meta->tos[slot] = t;
  }
  if (out && tid == 0 && a.counter != nullptr) *a.counter = 0;  // ready for the next launch
  if (meta != nullptr) __syncthreads();
}

template <int NCT>
__global__ __launch_bounds__(256) void k_router(RouterArgs a) {
  __shared__ f32x4_t red[3][NCT][64];
  __shared__ RouteLds R;
  __shared__ int s_last;
  const int ntiles = (a.E + 15) >> 4;
  const int nt = blockIdx.x % ntiles, ks = blockIdx.x / ntiles;
  const int KS = gridDim.x / ntiles;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  const int i = lane & 15, g = lane >> 4;
  const int KT = a.H >> 5;
  const int kt0 = ks * 8 + wave * 2;
  {
    const uint32_t xbytes = (uint32_t)(a.b * a.H * 2);
    const auto rh = rsrc(a.x, xbytes);
    const auto rl = rsrc(a.x_lo != nullptr ? a.x_lo : a.x, a.x_lo != nullptr ? xbytes : 0);
    const bool lo = (i >> 3) != 0;
    const uint16_t* wt = a.w + ((size_t)nt * KT + kt0) * 512 + lane * 8;
    const bf16x8_t a0 = __builtin_nontemporal_load((const bf16x8_t*)wt);
    const bf16x8_t a1 = __builtin_nontemporal_load((const bf16x8_t*)(wt + 512));
    bf16x8_t b0[NCT], b1[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int row = 8 * c + (i & 7);
      const uint32_t ob = row < a.b ? (uint32_t)((row * a.H + kt0 * 32 + 8 * g) * 2) : kOob;
      const uint32_t oh = lo ? kOob : ob, ol = lo ? ob : kOob;
      b0[c] = __builtin_bit_cast(bf16x8_t, buf_load16(rh, oh) | buf_load16(rl, ol));
      b1[c] = __builtin_bit_cast(bf16x8_t, buf_load16(rh, oh + 64) | buf_load16(rl, ol + 64));
    }
    f32x4_t acc[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0[c], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1[c], acc[c], 0, 0, 0);
    }
    if (wave > 0) {
#pragma unroll
      for (int c = 0; c < NCT; ++c) red[wave - 1][c][lane] = acc[c];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        acc[c] += red[0][c][lane];
        acc[c] += red[1][c][lane];
        acc[c] += red[2][c][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[c][r] += sd::lane_xor<8>(acc[c][r]);
        const int row = 8 * c + i;
        if (i < 8 && row < a.b) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = nt * 16 + 4 * g + r;
            if (e < a.E) a.part[((size_t)ks * a.b + row) * a.E + e] = acc[c][r];
          }
        }
      }
    }
  }
  // arrival: wave 0 wrote the partials; thread 0 releases them before counting, and the
  // last arrival acquires every workgroup's partials before reading them
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    s_last = atomicAdd(a.counter, 1) == (int)gridDim.x - 1;
    if (s_last) __threadfence();
  }
  __syncthreads();
  if (!s_last) return;

  route_phase2<0, 256>(a, KS, R);
}

// Attention boundary fused with the router, for the layer step.  Workgroup (row t, part q)
// of RS per row redoes the row's dual norm (latency-bound, so the repeat costs nothing
// measurable), writes its RS-th of the boundary's outputs, and computes in fp32 the logits
// of experts e = q + RS j (j < EPW) as the normalised row times the packed router rows.
// The last of the b * RS workgroups to arrive routes (route_phase2 over one partial).
template <int VW>
__device__ __forceinline__ void load_bf16v(const uint16_t* p, float* out) {
  if constexpr (VW == 4) {
    const u32x2_t v = *(const u32x2_t*)p;
    out[0] = __uint_as_float(v[0] << 16); out[1] = __uint_as_float(v[0] & 0xffff0000u);
    out[2] = __uint_as_float(v[1] << 16); out[3] = __uint_as_float(v[1] & 0xffff0000u);
  } else if constexpr (VW == 2) {
    const uint32_t v = *(const uint32_t*)p;
    out[0] = __uint_as_float(v << 16); out[1] = __uint_as_float(v & 0xffff0000u);
  } else {
    out[0] = sd::bf2f(p[0]);
  }
}

template <int VW>
__device__ __forceinline__ void load_f32v(const float* p, float* out) {
  if constexpr (VW == 4) {
    const f32x4_t v = *(const f32x4_t*)p;
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  } else if constexpr (VW == 2) {
    const f32x2_t v = *(const f32x2_t*)p;
    out[0] = v[0]; out[1] = v[1];
  } else {
    out[0] = p[0];
  }
}


template <int EPT, int NB, int RS>
__global__ __launch_bounds__(256) void k_norm_router(NormRouterArgs A) {
  constexpr int VW = EPT % 4 == 0 ? 4 : (EPT % 2 == 0 ? 2 : 1);
  constexpr int NV = EPT / VW;
  static_assert(NV % RS == 0, "each part writes whole vectors");
  __shared__ float red[4];
  __shared__ float s_z[4][8];
  __shared__ float s_x[256 * EPT];
  const RouterArgs& a = A.r;
  const int t = blockIdx.x / RS, q = blockIdx.x - t * RS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = A.H;
  const size_t base = (size_t)t * H;
  const float inv_h = 1.0f / (float)H;
  // Every load is issued before the first use: the row (branch partials, stream, gains)
  // first, as it is needed first, then the router lines.  Part q scores experts 8q .. 8q+7:
  // rows 8(q&1) .. +7 of 16-row tile q>>1, which fill one 128-byte line of every 8-wide k
  // group of the packed router weight.  Lane l of wave w takes line (it*4 + w)*8 + l/8
  // (k = 8 x line .. +7) and expert 8q + l%8, so each load instruction reads 1 KB of whole
  // lines.
  float pb[NB][EPT], s[EPT], gp[EPT], gq[EPT];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int i0 = (v * 256 + tid) * VW;
#pragma unroll
    for (int p = 0; p < NB; ++p) load_f32v<VW>(A.branch + p * A.branch_stride + base + i0, &pb[p][v * VW]);
    load_f32v<VW>(A.stream_in + base + i0, &s[v * VW]);
    load_f32v<VW>(A.g_post + i0, &gp[v * VW]);
    load_f32v<VW>(A.g_pre + i0, &gq[v * VW]);
  }
  const int KT = H >> 5;
  const auto rw = rsrc(a.w, (uint32_t)((size_t)((a.E + 15) >> 4) * KT * 1024));
  u32x4_t wv[EPT];
#pragma unroll
  for (int it = 0; it < EPT; ++it) {
    const int line = (it * 4 + wave) * 8 + (lane >> 3);
    const uint32_t off = (uint32_t)(((q >> 1) * KT + (line >> 2)) * 1024 + (line & 3) * 256 +
                                    (q & 1) * 128 + (lane & 7) * 16);
    wv[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, kStream));
  }
  __builtin_amdgcn_sched_barrier(0);
  float u[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    u[e] = pb[0][e];
#pragma unroll
    for (int p = 1; p < NB; ++p) u[e] += pb[p][e];
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) ss += u[e] * u[e];
  ss = sd::block_sum<4>(ss, red);
  const float r1 = rsqrtf(ss * inv_h + A.eps);
  ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    s[e] += u[e] * r1 * gp[e];
    ss += s[e] * s[e];
  }
  ss = sd::block_sum<4>(ss, red);
  const float r2 = rsqrtf(ss * inv_h + A.eps);
  float x[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) x[e] = s[e] * r2 * gq[e];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int i0 = (v * 256 + tid) * VW;
#pragma unroll
    for (int jj = 0; jj < VW; ++jj) s_x[i0 + jj] = x[v * VW + jj];
  }
  // this part's share of the outputs: vectors v with v % RS == q
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    if (v % RS != q) continue;
    const size_t i0 = base + (size_t)(v * 256 + tid) * VW;
    uint16_t hi[VW], lo[VW];
    _Float16 h16[VW], l16[VW];
    if constexpr (VW == 4) {
      *(f32x4_t*)(A.stream + i0) = f32x4_t{s[v * 4], s[v * 4 + 1], s[v * 4 + 2], s[v * 4 + 3]};
    } else {
#pragma unroll
      for (int jj = 0; jj < VW; ++jj) A.stream[i0 + jj] = s[v * VW + jj];
    }
#pragma unroll
    for (int jj = 0; jj < VW; ++jj) {
      sd::split_bf16(x[v * VW + jj], hi[jj], lo[jj]);
      sd::split_f16(x[v * VW + jj], h16[jj], l16[jj]);
    }
    if (A.out != nullptr) {
      store16<VW>(A.out + i0, hi);
      store16<VW>(A.out_lo + i0, lo);
    }
    store16<VW>((uint16_t*)A.x16 + i0, (const uint16_t*)h16);
    store16<VW>((uint16_t*)A.x16_lo + i0, (const uint16_t*)l16);
  }
  __syncthreads();
  // logits of the part's experts from the normalised row: fp32 products, lane sums over
  // its lines, then the 8 lanes of an expert, then the 4 waves
  float acc = 0.f;
#pragma unroll
  for (int it = 0; it < EPT; ++it) {
    const int k0 = ((it * 4 + wave) * 8 + (lane >> 3)) * 8;
    const f32x4_t x0 = *(const f32x4_t*)(s_x + k0), x1 = *(const f32x4_t*)(s_x + k0 + 4);
    const u32x4_t w = wv[it];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float wl = __uint_as_float(w[h] << 16), wh = __uint_as_float(w[h] & 0xffff0000u);
      const float xl = h < 2 ? x0[2 * h] : x1[2 * h - 4], xh = h < 2 ? x0[2 * h + 1] : x1[2 * h - 3];
      acc += wl * xl;
      acc += wh * xh;
    }
  }
  acc += sd::lane_xor<8>(acc);
  acc += sd::lane_xor<16>(acc);
  acc += sd::lane_xor<32>(acc);
  if (lane < 8) s_z[wave][lane] = acc;
  __syncthreads();
  if (tid < 8 && 8 * q + tid < a.E)
    a.part[(size_t)t * a.E + 8 * q + tid] = (s_z[0][tid] + s_z[1][tid]) + (s_z[2][tid] + s_z[3][tid]);
}

__global__ void k_zero_i32(int* p) { *p = 0; }

// ---------------------------------------------------------------- expert GEMMs
// Weights are packed tiles of 16 rows x 128 weights (layout in sdverify.h): per tile 1 KB
// of codes, lane l's 16 bytes holding weights 32(l/16) .. +31 of row l%16, and 128 B of
// scales, lane l's 2 bytes at 2l.  Lane (i, G)'s four f16x8 operands of a tile cover k =
// 32G + 8m, m = 0..3; the activation operand takes the same k order.
//
// A work unit is (active expert, 16-row tile); a persistent grid walks the units with KS
// waves splitting K (NU tiles each).  The routing metadata is staged in LDS once per
// workgroup, and the next unit's weights are loaded while the current unit is reduced, so
// the weight stream does not drain between units.  Pooled tokens are the B operand, 8 per column tile as hi/lo fp16 terms (columns
// 0-7 / 8-15); operand rows that do not exist are read through buffer loads whose range
// check returns zero without a memory access.


template <class M>
__device__ __forceinline__ void stage_meta(const MoeArgs& a, M& m) {
  const int nk = a.b * a.k;
  for (int p = threadIdx.x; p <= a.E; p += blockDim.x) m.active[p] = a.active[p];
  for (int p = threadIdx.x; p < a.E; p += blockDim.x) {
    m.cnt[p] = a.counts[p];
    m.off[p] = a.offsets[p];
    m.g13[p] = a.w13_gscale[p];
    m.g2[p] = a.w2_gscale[p];
  }
  for (int p = threadIdx.x; p < nk; p += blockDim.x) m.tos[p] = a.tos[p];
  __syncthreads();
  if constexpr (std::is_same<M, MoeMetaG>::value) build_groups(m, a.E);
}

template <int NU>
struct Slice {
  u32x4_t codes[NU];
  uint32_t scales[NU];
};

// Packed weights of one expert as buffer resources (codes, scales).
struct ExpertRes {
  __amdgpu_buffer_rsrc_t c, s;
};

__device__ __forceinline__ ExpertRes expert_res(const uint8_t* codes, const uint8_t* scales,
                                                size_t code_bytes, int e) {
  ExpertRes r;
  r.c = rsrc(codes + (size_t)e * code_bytes, (uint32_t)code_bytes);
  r.s = rsrc(scales + (size_t)e * (code_bytes / 8), (uint32_t)(code_bytes / 8));
  return r;
}

// The wave's NU consecutive tiles from tile index `t0` of the expert; t0 < 0 loads zeros
// without touching memory (a prefetch past the last unit), so the load count never
// depends on a branch and every wait stays exact.
// The offset is a per-lane part (the lane's bytes in a tile, or out of range) plus a
// wave-uniform tile offset, so the loads need no per-lane address arithmetic.
template <int NU>
__device__ __forceinline__ void load_slice(Slice<NU>& s, const ExpertRes& r, int t0, int lane) {
  const uint32_t lc = t0 < 0 ? kOob : 16u * lane, ls = t0 < 0 ? kOob : 2u * lane;
  const uint32_t t = t0 < 0 ? 0u : (uint32_t)t0;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    s.codes[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r.c, lc, (t + u) * 1024u, kStream));
    s.scales[u] = __builtin_amdgcn_raw_buffer_load_b16(r.s, ls, (t + u) * 128u, kStream);
  }
}

// B operand: f16x8 m of tile u at byte offset off + (128u + 8m) * 2 of one buffer that
// holds the hi terms and, lo_off bytes further, the lo terms (each lane's offset picks).
template <int NU>
__device__ __forceinline__ void load_bx(f16x8_t (&bx)[NU][4], __amdgpu_buffer_rsrc_t r,
                                        uint32_t off) {
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      bx[u][m] = __builtin_bit_cast(
          f16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, off + (uint32_t)(128 * u + 8 * m) * 2, 0, 0));
}

// A unit: row tile nt of expert group gi (expert e, pooled rows off .. off + Te - 1).
// Without a group list (MoeMeta), group gi is active expert gi.
struct Unit {
  int gi, e, nt, Te, off;
};

template <class M>
__device__ __forceinline__ Unit unit_of(const M& m, int u, int NT) {
  Unit r;
  r.gi = __builtin_amdgcn_readfirstlane(u / NT);
  r.nt = __builtin_amdgcn_readfirstlane(u - r.gi * NT);
  if constexpr (std::is_same<M, MoeMetaG>::value) {
    r.e = __builtin_amdgcn_readfirstlane(m.gexp[r.gi]);
    r.Te = __builtin_amdgcn_readfirstlane(m.gcnt[r.gi]);
    r.off = __builtin_amdgcn_readfirstlane(m.goff[r.gi]);
  } else {
    r.e = __builtin_amdgcn_readfirstlane(m.active[r.gi]);
    r.Te = __builtin_amdgcn_readfirstlane(m.cnt[r.e]);
    r.off = __builtin_amdgcn_readfirstlane(m.off[r.e]);
  }
  return r;
}

// (wave-uniform: the walk's loop control then stays scalar)
template <class M>
__device__ __forceinline__ int groups_of(const M& m, int E) {
  if constexpr (std::is_same<M, MoeMetaG>::value) return __builtin_amdgcn_readfirstlane(m.ng);
  else return __builtin_amdgcn_readfirstlane(m.active[E]);
}

// The unit after U in the walk: the next tile of U's group, or the first tile of the next
// group (only then are the maps in LDS read again).  U must not be the walk's last unit.
template <class M>
__device__ __forceinline__ Unit next_unit(const M& m, const Unit& U, int NT) {
  if (U.nt + 1 < NT) {  // wave-uniform
    Unit V = U;
    V.nt = U.nt + 1;
    return V;
  }
  return unit_of(m, (U.gi + 1) * NT, NT);
}

// Workgroup w walks the contiguous unit range [begin, end): consecutive units mostly share
// an expert group, so the activation operand is reloaded only when the group changes.
// Ranges go out XCD by XCD: the workgroups of one XCD walk one contiguous part of the
// units, so when an expert's weights are walked once per expert group, the groups' reads
// of a tile come from workgroups of one XCD at about the same time and share its L2.
__device__ __forceinline__ void unit_range(int n_units, int& begin, int& end) {
  const int r = xcd_rank(blockIdx.x, gridDim.x);
  begin = (int)(((long)r * n_units) / gridDim.x);
  end = (int)(((long)(r + 1) * n_units) / gridDim.x);
}

// W13 (gate rows [0, I), up rows [I, 2I)) + SwiGLU.  K = H = 128 * NU * KS.
//
// Row block j (8 rows) of an expert group is one MFMA A tile: gate rows 8j .. 8j + 7 in tile
// rows 0-7 and the up rows of the same index in tile rows 8-15, so one accumulator carries
// both and each output lane finds its SwiGLU partner 32 lanes away.  A unit is the pair of
// blocks 2p, 2p + 1, which together read packed gate tile p and up tile p.  Workgroups split
// the walk in blocks, so a range may start or end half-way through a unit: the missing block
// loads nothing and stores nothing.  With 19 experts of I = 1536 the longest range is then
// 7.5 units against 7.125 on average, where whole units gave 8.
template <int NU, int KS, bool RT, bool GRP>
__global__ __launch_bounds__(64 * KS) void k_moe_w13(MoeArgs a) {
  constexpr int NR = KS > 1 ? KS - 1 : 1;
  __shared__ MoeMetaT<GRP> meta;
  __shared__ f32x4_t red[2][NR][2][64];
  __shared__ RouteLdsT<64 * 32> R;  // routing (RT): b <= 64 rows, E <= 32 experts
  // workgroup 0 writes the routing's ids and softmax weights after its last unit: only
  // later kernels read them, and no workgroup's weight stream waits for them
  auto route_weights = [&]() {
    if constexpr (RT)
      if (blockIdx.x == 0)
        for (int p = threadIdx.x; p < a.r.b * a.r.k; p += blockDim.x) route_weight<32>(a.r, R, p);
  };
  if constexpr (RT) {
    // every workgroup routes from the router's logits (the same arithmetic, so the same
    // maps); workgroup 0 also writes the maps for the W2 kernel and the unpooler
    // the global scales are read before the routing and staged after it, so their loads go
    // out with the logits' (a barrier inside the routing keeps them there)
    const int ge = min((int)threadIdx.x, a.E - 1);
    const float g13v = a.w13_gscale[ge], g2v = a.w2_gscale[ge];
    route_phase2<32, 64 * KS, false>(a.r, 1, R, blockIdx.x == 0, &meta);
    if ((int)threadIdx.x < a.E) {
      meta.g13[threadIdx.x] = g13v;
      meta.g2[threadIdx.x] = g2v;
    }
    if constexpr (GRP) {
      build_groups(meta, a.E);  // its barriers also cover the scales
    } else {
      __syncthreads();
    }
  } else {
    stage_meta(a, meta);
  }
  const int NT = a.I >> 4;  // units (16-row tile pairs) per expert group
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, G = lane >> 4;
  const bool lo = (i >> 3) != 0;
  const int K = a.H, KT = K >> 7, kw = wave * NU;
  const size_t code_bytes = (size_t)a.I * K;  // 2I rows x K/2 bytes per expert
  // hi terms at x16, lo terms x16_lo_off bytes further in the same buffer (or none)
  const uint32_t xbytes = (uint32_t)(a.b * K * 2);
  const auto rx = rsrc(a.x16, a.x16_lo_off + xbytes);
  // this lane's row of block 2p (+1) is row i % 8 (+8) of packed gate tile p (i < 8) or of
  // up tile p (i >= 8); the up tiles follow the I / 16 gate tiles.  A load's offset is this
  // per-lane constant (byte of the lane's row within tile 0 of its matrix half) plus a
  // wave-uniform tile offset, so a unit's loads need no per-lane address arithmetic.
  const int l_base = (lane & 48) + (i & 7);
  const uint32_t lane_c = (i < 8 ? 0u : (uint32_t)(NT * KT) * 1024u) + 16u * l_base;
  const uint32_t lane_s = (i < 8 ? 0u : (uint32_t)(NT * KT) * 128u) + 2u * l_base;

  // lane's B byte offset for unit U (column tile 0: at most 8 pooled rows per group)
  auto b_off = [&](const Unit& U) -> uint32_t {
    const int slot = i & 7;
    if (slot >= U.Te || (lo && a.x16_lo_off == 0)) return kOob;
    return (lo ? a.x16_lo_off : 0u) +
           (uint32_t)(((size_t)meta.tos[U.off + slot] * K + kw * 128 + 32 * G) * 2);
  };
  // weights of blocks 2 U.nt (+1) where valid (else zeros, no memory traffic: the
  // out-of-range part of the offset is the per-lane one)
  auto load_a = [&](Slice<NU>& sa, Slice<NU>& sb, const Unit& U, bool va, bool vb) {
    const ExpertRes r = expert_res(a.w13_codes, a.w13_scales, code_bytes, U.e);
    const uint32_t t0 = (uint32_t)(U.nt * KT + kw);
    const uint32_t ca = va ? lane_c : kOob, cb = vb ? lane_c + 128u : kOob;
    const uint32_t sa_o = va ? lane_s : kOob, sb_o = vb ? lane_s + 16u : kOob;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const uint32_t t = t0 + (uint32_t)u;
      sa.codes[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r.c, ca, t * 1024u, kStream));
      sb.codes[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r.c, cb, t * 1024u, kStream));
      sa.scales[u] = __builtin_amdgcn_raw_buffer_load_b16(r.s, sa_o, t * 128u, kStream);
      sb.scales[u] = __builtin_amdgcn_raw_buffer_load_b16(r.s, sb_o, t * 128u, kStream);
    }
  };
  auto compute = [&](const Slice<NU>& sa, const Slice<NU>& sb, const f16x8_t (&bx)[NU][4],
                     const Unit& U, bool va, bool vb, int buf) {
    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      f16x8_t da[4], db[4];
      sd::dequant_unit(sa.codes[u], sa.scales[u], da);
      sd::dequant_unit(sb.codes[u], sb.scales[u], db);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(da[m], bx[u][m], acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(db[m], bx[u][m], acc[1], 0, 0, 0);
      }
    }
    // block j's sum is finished by wave j (one wave when KS == 1): every other wave leaves
    // its partial of the block in LDS, in the block's slot order of the other waves
    const int jw = KS > 1 ? (wave < 2 ? wave : -1) : 0;  // the block this wave finishes
    if (KS > 1) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (wave != j) red[buf][wave - (wave > j ? 1 : 0)][j][lane] = acc[j];
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (KS > 1 ? jw != j : false) continue;  // wave-uniform
      f32x4_t v = acc[j], up;
#pragma unroll
      for (int w = 0; w < KS - 1; ++w) v += red[buf][w][j][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] += sd::lane_xor<8>(v[r]);  // hi + lo columns
        up[r] = sd::lane_xor<32>(v[r]);  // tile rows 8-15: the up rows
      }
      const int slot = i;
      if (i < 8 && G < 2 && slot < U.Te && (j == 0 ? va : vb)) {
        const float sc = SD_X16_UNSCALE * meta.g13[U.e];
        const int n = (2 * U.nt + j) * 8 + 4 * G;  // lane rows n .. n+3 of the gate (and up) block
        const size_t o = (size_t)(U.off + slot) * a.I + n;
        _Float16 hh[4], hl[4];
        uint16_t hb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gv = v[r] * sc, uv = up[r] * sc;
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
  };

  // this workgroup's blocks [hb, he) in the walk, as units [u, end)
  int hb, he;
  unit_range(groups_of(meta, a.E) * 2 * NT, hb, he);
  hb = __builtin_amdgcn_readfirstlane(hb);
  he = __builtin_amdgcn_readfirstlane(he);
  if (hb >= he) {
    route_weights();
    return;
  }
  int u = hb >> 1;
  const int end = (he + 1) >> 1;
  auto va_of = [&](int p) { return 2 * p >= hb && p < end; };
  auto vb_of = [&](int p) { return 2 * p + 1 < he; };
  Slice<NU> a0, b0, a1, b1;
  f16x8_t bx[NU][4];  // the current group's activations
  // two-deep pipeline: every load is unconditional (a missing next unit loads zeros from
  // no memory), so the wait before each compute covers exactly the unit it uses
  Unit U0 = unit_of(meta, u, NT), U1;
  int bg = -1;  // expert group whose activations are in bx
  load_a(a0, b0, U0, va_of(u), vb_of(u));
  while (true) {
    if (U0.gi != bg) { load_bx<NU>(bx, rx, b_off(U0)); bg = U0.gi; }
    const int n1 = u + 1;
    U1 = n1 < end ? next_unit(meta, U0, NT) : U0;  // past the end: loads nothing
    load_a(a1, b1, U1, va_of(n1), vb_of(n1));
    compute(a0, b0, bx, U0, va_of(u), vb_of(u), 0);
    if (n1 >= end) break;
    if (U1.gi != bg) { load_bx<NU>(bx, rx, b_off(U1)); bg = U1.gi; }
    const int n2 = n1 + 1;
    U0 = n2 < end ? next_unit(meta, U1, NT) : U1;
    load_a(a0, b0, U0, va_of(n2), vb_of(n2));
    compute(a1, b1, bx, U1, va_of(n1), vb_of(n1), 1);
    if (n2 >= end) break;
    u = n2;
  }
  route_weights();
}

// W2: y[slot, n] = h[slot] . W2_e[n], fp32.  K = I = 128 * NU * KS.
template <int NCT, int NU, int KS, bool GRP>
__global__ __launch_bounds__(64 * KS) void k_moe_w2(MoeArgs a) {
  constexpr bool PB = NCT == 1;
  constexpr int NR = KS > 1 ? KS - 1 : 1;
  __shared__ MoeMetaT<GRP> meta;
  __shared__ f32x4_t red[PB ? 2 : 1][NR][NCT][64];
  stage_meta(a, meta);
  const int NT = a.H >> 4;
  const int n_units = groups_of(meta, a.E) * NT;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, G = lane >> 4;
  const bool lo = (i >> 3) != 0;
  const int K = a.I, KT = K >> 7, kw = wave * NU;
  const size_t code_bytes = (size_t)a.H * K / 2;
  // hi terms at h16, lo terms h16_lo_off bytes further in the same buffer
  const uint32_t hbytes = (uint32_t)(a.b * a.k * K * 2);
  const auto rx = rsrc(a.h16, a.h16_lo_off + hbytes);

  auto b_off = [&](const Unit& U, int c) -> uint32_t {
    const int slot = 8 * c + (i & 7);
    if (slot >= U.Te) return kOob;
    return (lo ? a.h16_lo_off : 0u) + (uint32_t)(((size_t)(U.off + slot) * K + kw * 128 + 32 * G) * 2);
  };
  auto load_a = [&](Slice<NU>& sw, const Unit& U, bool valid) {
    const ExpertRes r = expert_res(a.w2_codes, a.w2_scales, code_bytes, U.e);
    load_slice<NU>(sw, r, valid ? U.nt * KT + kw : -1, lane);
  };
  auto load_b0 = [&](f16x8_t (&bx)[NU][4], const Unit& U) { load_bx<NU>(bx, rx, b_off(U, 0)); };
  auto compute = [&](const Slice<NU>& sw, f16x8_t (&bx0)[NU][4], const Unit& U, int buf) {
    f32x4_t acc[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nct = (U.Te + 7) >> 3;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      if (c >= nct) break;
      // column tile 0 was loaded before the next unit's prefetch (bx0); later tiles here
      f16x8_t bl[NU][4];
      if (!PB && c > 0) load_bx<NU>(bl, rx, b_off(U, c));
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        f16x8_t dw[4];
        sd::dequant_unit(sw.codes[u], sw.scales[u], dw);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              dw[m], (PB || c == 0) ? bx0[u][m] : bl[u][m], acc[c], 0, 0, 0);
      }
    }
    if (KS > 1) {
      if (wave > 0) {
#pragma unroll
        for (int c = 0; c < NCT; ++c) {  // only the unit's column tiles
          if (c >= nct) break;
          red[buf][wave - 1][c][lane] = acc[c];
        }
      }
      __syncthreads();
    }
    if (wave == 0) {
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        if (c >= nct) break;
#pragma unroll
        for (int w = 0; w < KS - 1; ++w) acc[c] += red[buf][w][c][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[c][r] += sd::lane_xor<8>(acc[c][r]);
      }
      if (i < 8) {
        const float sc = SD_X16_UNSCALE * meta.g2[U.e];
        const int n = U.nt * 16 + 4 * G;
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          const int slot = 8 * c + i;
          if (slot >= U.Te) continue;
          *(f32x4_t*)(a.y + (size_t)(U.off + slot) * a.H + n) = acc[c] * sc;
        }
      }
    }
    if (!PB && KS > 1) __syncthreads();
  };

  Slice<NU> w0, w1;
  f16x8_t bx[NU][4];  // column tile 0's activations of the unit being computed
  int u, end;
  unit_range(n_units, u, end);
  u = __builtin_amdgcn_readfirstlane(u);
  end = __builtin_amdgcn_readfirstlane(end);
  if (u >= end) return;
  Unit U0 = unit_of(meta, u, NT), U1;
  int bg = -1;
  load_a(w0, U0, true);
  while (true) {
    if (!PB || U0.gi != bg) { load_b0(bx, U0); bg = U0.gi; }
    const int n1 = u + 1;
    U1 = n1 < end ? next_unit(meta, U0, NT) : U0;  // past the end: loads nothing
    load_a(w1, U1, n1 < end);
    __builtin_amdgcn_sched_barrier(0);  // the prefetch leaves before the compute starts
    compute(w0, bx, U0, 0);
    if (n1 >= end) break;
    if (!PB || U1.gi != bg) { load_b0(bx, U1); bg = U1.gi; }
    const int n2 = n1 + 1;
    U0 = n2 < end ? next_unit(meta, U1, NT) : U1;
    load_a(w0, U0, n2 < end);
    __builtin_amdgcn_sched_barrier(0);
    compute(w1, bx, U1, PB ? 1 : 0);
    if (n2 >= end) break;
    u = n2;
  }
}

// ---------------------------------------------------------------- unpooler
// out[t, n] = sum_j w[t, j] * y[slot_of[t, j], n], j in order, fp32.  4 features/thread;
// K = top_k is a template parameter so every slot id, then every row, is in flight at once.
template <int K>
__global__ __launch_bounds__(256) void k_unpool(int H, const float* __restrict__ y,
                                                const float* __restrict__ w,
                                                const int* __restrict__ slot_of,
                                                float* __restrict__ out) {
  const int t = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  int sl[K];
  float wj[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    sl[j] = slot_of[t * K + j];
    wj[j] = w[t * K + j];
  }
  f32x4_t v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) v[j] = *(const f32x4_t*)(y + (size_t)sl[j] * H + n);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < K; ++j) acc += wj[j] * v[j];
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

// A K split of an expert GEMM: K = 128 * NU * KS with NU <= 4 tiles per wave.
struct Split { int nu, ks; };
Split split_for(int K) {
  const int g = K / 128;
  for (int ks = 8; ks >= 1; ks >>= 1)
    if (K % 128 == 0 && g % ks == 0 && g / ks >= 1 && g / ks <= 4) return {g / ks, ks};
  return {0, 0};
}

#define SD_SPLITS(X) X(1, 1) X(1, 2) X(1, 4) X(1, 8) X(2, 1) X(2, 2) X(2, 4) X(2, 8) \
                     X(3, 1) X(3, 2) X(3, 4) X(3, 8) X(4, 1) X(4, 2) X(4, 4) X(4, 8)

int cus() {
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

template <bool GRP>
hipError_t launch_experts(const MoeArgs& a, hipStream_t st) {
  const Split s13 = split_for(a.H), s2 = split_for(a.I);
  // persistent grids: the live units are at most E * tiles
  const int g13 = min(cus(), a.E * (a.I / 16));
  const int g2 = min(2 * cus(), a.E * (a.H / 16));  // two per CU: measured fastest
  bool done = false;
#define SD_W13(NU, KS)                                                                     \
  if (!done && s13.nu == NU && s13.ks == KS) {                                             \
    if (a.route)                                                                           \
      hipLaunchKernelGGL((k_moe_w13<NU, KS, true, GRP>), dim3(g13), dim3(64 * KS), 0, st, a); \
    else                                                                                   \
      hipLaunchKernelGGL((k_moe_w13<NU, KS, false, GRP>), dim3(g13), dim3(64 * KS), 0, st, a); \
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
    hipLaunchKernelGGL((k_moe_w2<1, NU, KS, GRP>), dim3(g2), dim3(64 * KS), 0, st, a);     \
    done = true;                                                                          \
  }
  SD_SPLITS(SD_W2)
#undef SD_W2
  if (!done) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

bool moe_shape_supported(int H, int I) { return split_for(H).nu > 0 && split_for(I).nu > 0; }

hipError_t launch_router(const RouterArgs& a, hipStream_t st) {
  const int ntiles = (a.E + 15) / 16, ks = a.H / 256;
  const dim3 grid(ntiles * ks), block(256);
  if (a.b <= 8) hipLaunchKernelGGL(k_router<1>, grid, block, 0, st, a);
  else if (a.b <= 16) hipLaunchKernelGGL(k_router<2>, grid, block, 0, st, a);
  else if (a.b <= 32) hipLaunchKernelGGL(k_router<4>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(k_router<8>, grid, block, 0, st, a);
  return hipGetLastError();
}

int norm_router_parts(int H, int E, int b, int k) {
  if (H % 256 || b > 64 || b * k > 512 || k > 8) return 0;
  const int ept = H / 256;
  if (ept != 16 && ept != 1) return 0;  // instantiated widths: H = 4096 and H = 256
  const int vw = ept % 4 == 0 ? 4 : (ept % 2 == 0 ? 2 : 1), nv = ept / vw;
  // RS parts of 8 experts each; an odd part would leave half of its tile's lines to nobody
  for (int rs : {1, 2, 4})
    if (nv % rs == 0 && E <= 8 * rs) return rs;
  return 0;
}

hipError_t launch_norm_router(const NormRouterArgs& a, int nbranch, hipStream_t st) {
  const int rs = norm_router_parts(a.H, a.r.E, a.r.b, a.r.k);
  if (rs == 0 || (nbranch != 1 && nbranch != 4)) return hipErrorInvalidValue;
  if ((a.out == nullptr) != (a.out_lo == nullptr)) return hipErrorInvalidValue;
  // the parts of a row each read the whole incoming row and write their share of the new one
  if (a.stream_in == nullptr || (rs > 1 && a.stream_in == a.stream)) return hipErrorInvalidValue;
  const dim3 grid(a.r.b * rs), block(256);
#define SD_NR(EPT, NB, RS)                                                             \
  if (a.H == 256 * EPT && nbranch == NB && rs == RS) {                                 \
    hipLaunchKernelGGL((k_norm_router<EPT, NB, RS>), grid, block, 0, st, a);           \
    return hipGetLastError();                                                          \
  }
  SD_NR(16, 4, 4) SD_NR(16, 1, 4) SD_NR(16, 4, 2) SD_NR(16, 1, 2) SD_NR(16, 4, 1) SD_NR(16, 1, 1)
  SD_NR(1, 4, 1) SD_NR(1, 1, 1)
#undef SD_NR
  return hipErrorInvalidValue;
}

hipError_t launch_zero_i32(int* p, hipStream_t st) {
  hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(1), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_moe_experts(const MoeArgs& in, hipStream_t st) {
  MoeArgs a = in;
  const size_t xb = (size_t)a.b * a.H * 2, hb = (size_t)a.b * a.k * a.I * 2;
  // lo terms must follow the hi terms in one buffer (the workspace lays them out so)
  if (a.x16_lo != nullptr) {
    if (a.x16_lo < a.x16 + (size_t)a.b * a.H || (size_t)((const char*)a.x16_lo - (const char*)a.x16) + xb >= 0x80000000u)
      return hipErrorInvalidValue;
    a.x16_lo_off = (uint32_t)((const char*)a.x16_lo - (const char*)a.x16);
  } else {
    a.x16_lo_off = 0;
  }
  if (a.h16_lo < a.h16 + (size_t)a.b * a.k * a.I || (size_t)((const char*)a.h16_lo - (const char*)a.h16) + hb >= 0x80000000u)
    return hipErrorInvalidValue;
  a.h16_lo_off = (uint32_t)((const char*)a.h16_lo - (const char*)a.h16);
  // every unit is one expert group of at most 8 pooled rows (one MFMA column tile), so
  // one kernel pair serves every batch: an expert with more rows is read once per group;
  // with b <= 8 every expert is one group and the kernels build no group list
  return a.b > 8 ? launch_experts<true>(a, st) : launch_experts<false>(a, st);
}

hipError_t launch_unpool(int b, int H, int k, const float* y, const float* w, const int* slot_of,
                         float* out, hipStream_t st) {
  const dim3 grid((H / 4 + 255) / 256, b), block(256);
  switch (k) {
#define SD_UNPOOL(KV) \
  case KV: hipLaunchKernelGGL(k_unpool<KV>, grid, block, 0, st, H, y, w, slot_of, out); break;
    SD_UNPOOL(1) SD_UNPOOL(2) SD_UNPOOL(3) SD_UNPOOL(4)
    SD_UNPOOL(5) SD_UNPOOL(6) SD_UNPOOL(7) SD_UNPOOL(8)
#undef SD_UNPOOL
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_debug_dequant(int n, int k, const uint8_t* codes, const uint8_t* scales,
                                float gscale, float* out, hipStream_t st) {
  const int units = n * (k / 32);
  hipLaunchKernelGGL(k_debug_dequant, dim3((units + 255) / 256), dim3(256), 0, st, n, k, codes,
                     scales, gscale, out);
  return hipGetLastError();
}
