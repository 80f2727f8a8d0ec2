// K-C: paged verify attention, split over KV blocks, then an LSE combine with the output
// gate fused in.
//
// Page "vllm.models.muse_spark.nvidia.specialized_decode.runtime.decode": the attention
// block is QKV front -> attn2 -> o_proj (module docstring); attn2 reads block-table decode
// metadata for one request verifying q tokens (plan, decode_metadata).  The verify rows
// are causal: row j sees positions 0 .. p_j of its request.
//
// Work split: workgroup (chunk, kv head g, request r) covers `chunk_blocks` KV blocks; its
// 4 waves take 32-token windows (two blocks) in turn.  Every window is read once and
// shared by all QG = (Hq/Hkv) * q_rows queries of (r, g) through MFMA:
//   S^T[token, query] = K[token, :] . Q^T       (A = K rows, B = Q^T; 16x16x32 bf16)
//   O^T[dim, query]  += V^T[dim, token] . P^T   (A = V^T, B = P^T)
// K rows of a window are assigned to the two S tiles so that a lane's 8 S values are the
// 8 consecutive tokens 8G .. 8G+7 of one query: after exp they are that lane's P^T
// B operand as is, and the V^T operand is 16 contiguous bytes of the dim-major V block.
// Q and P enter as bf16 hi/lo terms (two MFMAs each), so the only 16-bit quantities are
// the cached K and V themselves.  Masked scores become -inf by selection and V of tokens
// past the request's end is zeroed by selection, so NaN in unused cache slots never
// reaches the result.
#include "sd_common.h"

namespace {

constexpr float LOG2E = 1.4426950408889634f;

template <int D, int NQT>
__global__ __launch_bounds__(256) void k_attn_split(AttnArgs a, int chunk_blocks, int n_chunks) {
  constexpr int QG = 16 * NQT;
  constexpr int NC = D / 32;   // MFMA steps over the head dim
  constexpr int NDT = D / 16;  // output dim tiles
  constexpr int DL = D / 4;    // dims per lane group
  __shared__ float s_acc[4][QG][D];
  __shared__ float s_m[4][QG], s_l[4][QG];

  const int chunk = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int L = min(a.seq_lens[r], a.max_blocks * 16);  // never read past the table row
  const int nblk = (L + 15) >> 4;
  const int blk_begin = chunk * chunk_blocks;
  if (blk_begin >= nblk) return;  // past this request's end (uniform per workgroup)
  const int blk_end = min(blk_begin + chunk_blocks, nblk);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = lane & 15, G = lane >> 4;
  const int group = a.Hq / a.Hkv;

  // Q^T B operands (hi and lo terms) and the causal bound of the lane's query column
  bf16x8_t bq[NQT][NC], bql[NQT][NC];
  int qpos[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int qi = 16 * qt + i;
    const int hh = qi / a.q_rows, jr = qi - hh * a.q_rows;
    const int row = r * a.q_rows + jr;
    const size_t qo = ((size_t)row * a.Hq + g * group + hh) * D + G * DL;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bq[qt][c] = *(const bf16x8_t*)(a.q + qo + 8 * c);
      bql[qt][c] = *(const bf16x8_t*)(a.q_lo + qo + 8 * c);
    }
    qpos[qt] = a.positions[row];
  }
  const float sl2 = a.scale * LOG2E;

  float mrun[NQT], lsum[NQT];
  f32x4_t acc[NDT][NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    mrun[qt] = -INFINITY;
    lsum[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt][qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8_t zero8 = {};
  const int* bt = a.block_table + (size_t)r * a.max_blocks;
  const size_t kv_head_stride = (size_t)16 * D;  // elements per (block, head)

  for (int wb = blk_begin + 2 * wave; wb < blk_end; wb += 8) {
    const bool has1 = wb + 1 < blk_end;
    const int pb0 = bt[wb];
    const int pb1 = has1 ? bt[wb + 1] : pb0;
    const int tok_base = wb * 16;
    // K rows: tile t, row i <-> window token 8*(i/4) + 4t + i%4
    bf16x8_t ka[2][NC];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int tw = 8 * (i >> 2) + 4 * t + (i & 3);
      const bool ok = tok_base + tw < L;
      const int pb = (tw >> 4) ? pb1 : pb0;
      const uint16_t* kp = a.k_cache + ((size_t)pb * a.Hkv + g) * kv_head_stride +
                           (size_t)(tw & 15) * D + G * DL;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        ka[t][c] = ok ? __builtin_nontemporal_load((const bf16x8_t*)(kp + 8 * c)) : zero8;
    }
    // V^T rows: dim 16dt + i, window tokens 8G .. 8G+7
    bf16x8_t va[NDT];
    {
      const int tok0 = tok_base + 8 * G;
      const int pb = (G >> 1) ? pb1 : pb0;
      const uint16_t* vp =
          a.v_cache + ((size_t)pb * a.Hkv + g) * kv_head_stride + (size_t)i * 16 + 8 * (G & 1);
      const int nvalid = L - tok0;  // tokens of this lane's 8 that exist
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        bf16x8_t v = nvalid > 0 ? __builtin_nontemporal_load((const bf16x8_t*)(vp + (size_t)dt * 256))
                                : zero8;
        if (nvalid < 8) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e >= nvalid) v[e] = (__bf16)0.0f;
        }
        va[dt] = v;
      }
    }
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      f32x4_t s[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4_t sh = {0.f, 0.f, 0.f, 0.f}, slo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          sh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[t][c], bq[qt][c], sh, 0, 0, 0);
          slo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[t][c], bql[qt][c], slo, 0, 0, 0);
        }
        s[t] = sh + slo;
      }
      // lane's scores: token tok_base + 8G + 4t + rr for query column 16qt + i
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int tok = tok_base + 8 * G + 4 * t + rr;
          const float v = tok <= qpos[qt] ? s[t][rr] * sl2 : -INFINITY;
          s[t][rr] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrun[qt], mx);
      const float alpha = mnew == -INFINITY ? 1.f : exp2f(mrun[qt] - mnew);
      bf16x8_t pb, pbl;
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float p = s[t][rr] == -INFINITY ? 0.f : exp2f(s[t][rr] - mnew);
          psum += p;
          const __bf16 ph = (__bf16)p;
          pb[4 * t + rr] = ph;
          pbl[4 * t + rr] = (__bf16)(p - (float)ph);
        }
      lsum[qt] = lsum[qt] * alpha + psum;
      mrun[qt] = mnew;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        acc[dt][qt] *= alpha;
        acc[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], pb, acc[dt][qt], 0, 0, 0);
        acc[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], pbl, acc[dt][qt], 0, 0, 0);
      }
    }
  }
  // per-wave state -> LDS; the lane's column is query 16qt + i, rows are dims 16dt + 4G + rr
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    float l = lsum[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int qi = 16 * qt + i;
    if (G == 0) {
      s_m[wave][qi] = mrun[qt];
      s_l[wave][qi] = l;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) s_acc[wave][qi][16 * dt + 4 * G + rr] = acc[dt][qt][rr];
  }
  __syncthreads();
  // combine the 4 waves; write one partial (m, l, acc) per query
  const size_t pidx = ((size_t)r * a.Hkv + g) * n_chunks + chunk;
  float* pacc = a.part_acc + pidx * QG * D;
  float* pml = a.part_ml + pidx * QG * 2;
  for (int e = threadIdx.x; e < QG * D; e += 256) {
    const int qi = e / D, d = e - qi * D;
    float M = s_m[0][qi];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, s_m[w][qi]);
    float v = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = exp2f(s_m[w][qi] - M);
        v += f * s_acc[w][qi][d];
        l += f * s_l[w][qi];
      }
    }
    pacc[e] = v;
    if (d == 0) {
      pml[2 * qi] = M;
      pml[2 * qi + 1] = l;
    }
  }
}

// One workgroup of D threads per (row, query head): LSE-combine the chunks, normalise,
// apply the output gate o * sigmoid(o_gate), store bf16 hi/lo terms.
__global__ __launch_bounds__(128) void k_attn_combine(AttnArgs a, int chunk_blocks, int n_chunks,
                                                      int qg) {
  const int t = blockIdx.x / a.Hq, h = blockIdx.x - t * a.Hq;
  const int d = threadIdx.x;
  const int r = t / a.q_rows, jr = t - r * a.q_rows;
  const int group = a.Hq / a.Hkv;
  const int g = h / group, hh = h - g * group;
  const int qi = hh * a.q_rows + jr;
  const int L = min(a.seq_lens[r], a.max_blocks * 16);
  const int nc = (((L + 15) >> 4) + chunk_blocks - 1) / chunk_blocks;
  const size_t p0 = ((size_t)r * a.Hkv + g) * n_chunks;
  __shared__ float s_w[1024], s_l[1024], s_red[2];
  // chunk maxima and sums: one load per chunk, spread over the threads
  float mloc = -INFINITY;
  for (int c = d; c < nc; c += blockDim.x) {
    const float m = a.part_ml[((p0 + c) * qg + qi) * 2];
    s_w[c] = m;
    s_l[c] = a.part_ml[((p0 + c) * qg + qi) * 2 + 1];
    mloc = fmaxf(mloc, m);
  }
  mloc = sd::wave_max(mloc);
  if ((d & 63) == 0) s_red[d >> 6] = mloc;
  __syncthreads();
  const float M = blockDim.x > 64 ? fmaxf(s_red[0], s_red[1]) : s_red[0];
  __syncthreads();
  for (int c = d; c < nc; c += blockDim.x)
    s_w[c] = s_w[c] == -INFINITY ? 0.f : exp2f(s_w[c] - M);
  __syncthreads();
  // independent loads across chunks: 4 accumulators
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, l = 0.f;
  const float* pa = a.part_acc + (p0 * qg + qi) * a.D + d;
  const size_t cs = (size_t)qg * a.D;  // chunk stride
  int c = 0;
  for (; c + 4 <= nc; c += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += s_w[c + u] * pa[(c + u) * cs];
  }
  for (; c < nc; ++c) acc[0] += s_w[c] * pa[c * cs];
  for (int cc = 0; cc < nc; ++cc) l += s_w[cc] * s_l[cc];
  const float o = (acc[0] + acc[1] + acc[2] + acc[3]) / l;
  const float gate = a.gate[(size_t)t * a.gate_stride + h * a.D + d];
  const float sig = 1.0f / (1.0f + __expf(-gate));
  uint16_t hi, lo;
  sd::split_bf16(o * sig, hi, lo);
  const size_t oi = (size_t)t * a.Hq * a.D + h * a.D + d;
  a.out[oi] = hi;
  a.out_lo[oi] = lo;
}

}  // namespace

AttnPlan attn_plan(const sd_dims& d, int n_req, int max_seq_len) {
  AttnPlan p;
  const int max_blocks = (max_seq_len + 15) / 16;
  const long units = (long)n_req * d.n_kv_heads * max_blocks;
  int cb = 8;                      // 4 waves x one 2-block window
  while (units / cb > 512 && cb < 4096) cb *= 2;
  p.chunk_blocks = cb;
  p.n_chunks = (max_blocks + cb - 1) / cb;
  p.qg = (d.n_q_heads / d.n_kv_heads) * d.q_rows;
  return p;
}

hipError_t launch_attention(const AttnArgs& a, const AttnPlan& p, hipStream_t st) {
  const dim3 grid(p.n_chunks, a.Hkv, a.n_req), block(256);
#define SD_ATTN(DD, NQ)                                                                    \
  hipLaunchKernelGGL((k_attn_split<DD, NQ>), grid, block, 0, st, a, p.chunk_blocks, p.n_chunks)
  if (a.D == 128 && p.qg == 32) SD_ATTN(128, 2);
  else if (a.D == 128 && p.qg == 16) SD_ATTN(128, 1);
  else if (a.D == 64 && p.qg == 32) SD_ATTN(64, 2);
  else if (a.D == 64 && p.qg == 16) SD_ATTN(64, 1);
  else if (a.D == 64 && p.qg == 64) SD_ATTN(64, 4);
  else return hipErrorInvalidValue;
#undef SD_ATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int b = a.n_req * a.q_rows;
  hipLaunchKernelGGL(k_attn_combine, dim3(b * a.Hq), dim3(a.D), 0, st, a, p.chunk_blocks,
                     p.n_chunks, p.qg);
  return hipGetLastError();
}
