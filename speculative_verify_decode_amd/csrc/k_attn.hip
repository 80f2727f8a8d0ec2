// K-C: paged verify attention, split over KV blocks, then an LSE combine with the output
// gate fused in.  The split kernel's prologue is also the QKV projection's epilogue: it
// sums the projection's K-slice partials, applies the per-head RMSNorm and RoPE to its
// query group and stores the new tokens' K/V into the cache.
//
// Page "vllm.models.muse_spark.nvidia.specialized_decode.runtime.decode": the attention
// block is QKV front -> attn2 -> o_proj (module docstring); attn2 reads block-table decode
// metadata for one request verifying q tokens (plan, decode_metadata).  The verify rows
// are causal: row j sees positions 0 .. p_j of its request.
//
// Work split: workgroup (slot, kv head g) covers one chunk of KV blocks of one request (the
// chunk map below assigns slots to requests); its 4 waves take 32-token windows (two
// blocks) in turn.  In MFMA step c over the head dim,
// lane group G holds dims 32c + 8G .. +7 of K and of Q (any dim order serves if both
// operands share it), so each K load instruction reads 64 contiguous bytes of 16 rows.  Every window is read once and
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
constexpr int kMaxChunkBlocks = 2048;
constexpr int kMaxReqChunks = 1024;  // chunks of one request (the combine's LDS statistics)
constexpr int kQRows = 8;  // verify rows per request (the host accepts only 8)

// cos and sin of the RoPE angle pos * freq: the angle is reduced modulo 2 pi in double (it
// reaches ~1.3e5 rad, where fp32 would lose ~1e-2 rad), the reduced angle taken in fp32.
__device__ __forceinline__ void rope_cs(int pos, double freq, float& c, float& s) {
  constexpr double kTwoPi = 6.283185307179586232, kTwoPiLo = 2.4492935982947064e-16;
  const double ang = (double)pos * freq;
  const double k = rint(ang * 0.15915494309189535);
  const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPi, ang));
  sincosf((float)r, &s, &c);
}

// The first block a request's rows can see: with a sliding window w, the lowest position
// of the request's rows (seq_len - q_rows) minus w - 1; block 0 otherwise.
__device__ __forceinline__ int first_block(const AttnArgs& a, int r) {
  if (a.window <= 0) return 0;
  const int L = min(a.seq_lens[r], a.max_blocks * 16);
  return max(0, L - a.q_rows - a.window + 1) >> 4;
}

// Rows of request r: the first row and the count.  Without query_start q_rows rows start
// at r * q_rows; with it (partial drafts) the range query_start[r] .. query_start[r+1] - 1,
// clamped so that base + j stays in 0 .. b - 1 for every j < n (and base itself when n = 0).
struct ReqRows {
  int base, n;
};
__device__ __forceinline__ ReqRows req_rows(const AttnArgs& a, int r) {
  if (a.query_start == nullptr) return {r * a.q_rows, a.q_rows};
  const int s0 = min(max(a.query_start[r], 0), a.b - 1);
  return {s0, min(max(a.query_start[r + 1] - s0, 0), min(a.q_rows, a.b - s0))};
}

// ceil(n / d) for n >= 0, d >= 1, with rd the fp32 reciprocal of d: the fp32 quotient is
// close to floor(n / d) (within one below 2^20), and the remainder corrects it exactly.
__device__ __forceinline__ int ceil_div_small(int n, int d, float rd) {
  int q = (int)((float)n * rd);
  int rem = n - q * d;
  while (rem < 0) { q -= 1; rem += d; }
  while (rem >= d) { q += 1; rem -= d; }
  return q + (rem > 0 ? 1 : 0);
}

// How the KV blocks of several requests map onto the nslot chunk slots of a KV head.  Every
// request's visible blocks (from its first visible block to its last) are cut into chunks of
// one size cb: the smallest multiple of 8 blocks, at most cb_host, whose chunks fit the
// slots, so the workgroups of long and short requests get near-equal work.  Request r owns
// slots off .. off + nch - 1 (request order).  cb_host always fits: the host sizes it for
// every request at max_seq_len.  Lane r of the calling wave holds request r's off and nch
// (n_req <= 64); every wave that calls this derives the same map.
struct ChunkMap {
  int cb;
  int off, nch;  // this lane's request (0, 0 for lanes past n_req)
};
__device__ ChunkMap chunk_map(const AttnArgs& a, int cb_host, int nslot) {
  const int lane = threadIdx.x & 63;
  int span = 0;
  if (lane < a.n_req) {
    const int L = min(a.seq_lens[lane], a.max_blocks * 16);
    span = max(((L + 15) >> 4) - first_block(a, lane), 0);
  }
  int S = span, smax = span;
  auto step = [&](int oS, int om) {
    S += oS;
    smax = max(smax, om);
  };
  step(sd::lane_xor<32>(S), sd::lane_xor<32>(smax));
  step(sd::lane_xor<16>(S), sd::lane_xor<16>(smax));
  step(sd::lane_xor<8>(S), sd::lane_xor<8>(smax));
  step(sd::lane_xor<4>(S), sd::lane_xor<4>(smax));
  step(sd::lane_xor<2>(S), sd::lane_xor<2>(smax));
  step(sd::lane_xor<1>(S), sd::lane_xor<1>(smax));
  S = __builtin_amdgcn_readfirstlane(S);
  smax = __builtin_amdgcn_readfirstlane(smax);
  // candidate sizes cb0 + 8 lane, from the least that could fit (and gives no request more
  // than kMaxReqChunks chunks)
  const int cb0 = max(max(8, (((S + nslot - 1) / nslot) + 7) & ~7),
                      (((smax + kMaxReqChunks - 1) / kMaxReqChunks) + 7) & ~7);
  const int cand = cb0 + 8 * lane;
  const float rc = 1.0f / (float)cand;
  int need = 0;
  for (int q = 0; q < a.n_req; ++q) need += ceil_div_small(__builtin_amdgcn_readlane(span, q), cand, rc);
  const uint64_t fits = __builtin_amdgcn_ballot_w64(need <= nslot && cand <= cb_host);
  ChunkMap m;
  m.cb = fits != 0 ? cb0 + 8 * (int)__builtin_ctzll(fits) : cb_host;
  m.nch = lane < a.n_req ? (span + m.cb - 1) / m.cb : 0;
  const int inc = sd::wave_scan_incl(m.nch);  // inclusive prefix sum over the lanes
  m.off = inc - m.nch;
  // seq_lens beyond the host's max_seq_len could ask for more slots than there are: such
  // chunks get none (the slot range of every request stays inside the nslot slots)
  m.off = min(m.off, nslot);
  m.nch = min(m.nch, nslot - m.off);
  return m;
}

// Workgroup (slot, kv head g): chunk `chunk` of request r, blocks [chunk * cb, +cb) from the
// request's first visible block (one request: r = 0, chunk = slot, cb = cb_host; several:
// the chunk map's), one workgroup per CU at most.  The chunk's block ids (clamped to the pool) and the query
// group (hi/lo, computed from the projection partials) are staged in LDS first; NP is the
// number of K-slice partials.  Each of the 4 waves then streams 2-block windows
// w = 2 * wave + 8 j, loading window j + 1 while window j is in the matrix cores.  Loads
// are unconditional: tokens past the request's end are masked after loading (scores by
// selection to -inf, V by selection to 0).  K and V are read once: non-temporal loads.
//
// GEN selects the general form (a sliding window or partial drafts): the first visible
// block and the request's rows then come from device metadata, one more scalar round trip
// before the first window.  Without it, and with one request, the chunk's block range and
// rows follow from the launch alone, and every scalar load the first two windows need
// (their four block ids, seq_len) goes out in one batch right after the kernel arguments.
template <int D, int NQT, bool GEN, int NP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_attn_split(AttnArgs a, int cb_host, int nslot) {
  constexpr int QG = 16 * NQT;
  constexpr int NC = D / 32;   // MFMA steps over the head dim
  constexpr int NDT = D / 16;  // output dim tiles
  constexpr int QP = D + 8;    // padded LDS row of the query terms
  constexpr int AP = D + 4;    // padded LDS row of the cross-wave accumulators
  __shared__ float s_acc[4][QG][AP];
  __shared__ float s_m[4][QG], s_l[4][QG];
  __shared__ uint16_t s_q[2][QG][QP];
  __shared__ int s_bt[kMaxChunkBlocks];
  __shared__ float s_cos[kQRows][D / 2], s_sin[kQRows][D / 2];
  __shared__ __align__(16) uint16_t s_kn[kQRows][D], s_vn[kQRows][D];  // new tokens' K, V
  __shared__ int s_kok[kQRows];  // row j's new K/V is stored (its slot is not negative)

  // (slot, head) from the XCD rank: the nslot workgroups of a KV head share an XCD, so the
  // head's projection partials (read by every slot of the head) fill one L2 once
  const int rank = xcd_rank(blockIdx.y * nslot + blockIdx.x, nslot * gridDim.y);
  const int slot = rank % nslot, g = rank / nslot;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // the slot's request and chunk: one request takes the slots as its chunks of cb_host
  // blocks; several share them through the chunk map (an unused slot has no work)
  int r = 0, chunk = slot, cb = cb_host;
  if (a.n_req > 1) {  // uniform
    const ChunkMap cm = chunk_map(a, cb_host, nslot);
    const uint64_t own = __builtin_amdgcn_ballot_w64(lane < a.n_req && cm.off <= slot &&
                                                     slot < cm.off + cm.nch);
    if (own == 0) return;  // uniform per workgroup, before any barrier
    r = (int)__builtin_ctzll(own);
    chunk = slot - __builtin_amdgcn_readlane(cm.off, r);
    cb = cm.cb;
  }
  const int i = lane & 15, G = lane >> 4;
  const int group = a.Hq / a.Hkv;
  // chunks start at the request's first visible block (block 0 without a window)
  const int blk_begin = (GEN ? first_block(a, r) : 0) + chunk * cb;
  const float sl2 = a.scale * LOG2E;
  const size_t kvh = (size_t)16 * D;  // elements per (block, head)
  const int* btr = a.block_table + (size_t)r * a.max_blocks;

  struct Win {
    bf16x8_t k[2][NC];
    bf16x8_t v[NDT];
  };
  // window of blocks (pb0, pb1): 32 tokens, K rows and V^T rows in MFMA operand order
  auto load_win = [&](Win& W, int pb0, int pb1) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // K rows: tile t, row i <-> window token 8 * (i / 4) + 4 t + i % 4
      const int tw = 8 * (i >> 2) + 4 * t + (i & 3);
      const int pb = (tw >> 4) ? pb1 : pb0;
      const uint16_t* kp = a.k_cache + ((size_t)pb * a.Hkv + g) * kvh + (size_t)(tw & 15) * D + 8 * G;
#pragma unroll
      for (int c = 0; c < NC; ++c) W.k[t][c] = __builtin_nontemporal_load((const bf16x8_t*)(kp + 32 * c));
    }
    // V^T rows: dim 16 dt + i, window tokens 8G .. 8G+7
    const int pb = (G >> 1) ? pb1 : pb0;
    const uint16_t* vp = a.v_cache + ((size_t)pb * a.Hkv + g) * kvh + (size_t)i * 16 + 8 * (G & 1);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) W.v[dt] = __builtin_nontemporal_load((const bf16x8_t*)(vp + (size_t)dt * 256));
  };
  auto clamp_blk = [&](int id) { return min(max(id, 0), a.num_blocks - 1); };

  // Order matters, as loads complete in order: the scalar loads (block ids of the first two
  // windows, seq_len, positions), then the projection partials this workgroup needs, then
  // the first window; the query terms (and, where this workgroup's blocks hold the new
  // tokens, their K/V) are computed while the window is in flight.  The new tokens' K/V go
  // into the cache and into LDS; after one barrier every later window (the second one
  // included) reads them from the cache, and the first window, read before they were
  // stored, is patched from LDS.  Block ids are clamped into the pool and tokens past the
  // request's end are masked, so a window past the end reads harmless data; a second window
  // past the end re-reads the first one's blocks, which merge with the loads in flight.
  // Query column jr of the group is row base + jr of the step; the columns of a partial
  // draft past its count read its last row and are masked below (position -1).
  const ReqRows rq = GEN ? req_rows(a, r) : ReqRows{r * a.q_rows, a.q_rows};
  auto row_of = [&](int jr) { return rq.base + min(jr, max(rq.n - 1, 0)); };
  const int ncb = min(cb, a.max_blocks - blk_begin);  // <= 0 only past the table's end
  const int bt0 = btr[min(blk_begin + min(tid, max(ncb - 1, 0)), a.max_blocks - 1)];
  int qpos[NQT], qlow[NQT];  // visible tokens: qlow < tok <= qpos
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int qi = 16 * qt + i, jr = qi - (qi / a.q_rows) * a.q_rows;
    const int p = a.positions[row_of(jr)];
    qpos[qt] = jr < rq.n ? p : -1;  // a column past the request's rows sees no token
  }
  // the block ids of both windows are read unconditionally (each index is clamped into the
  // table row), so no id load waits for seq_len
  Win W0, W1;
  const int wb0 = blk_begin + 2 * wave, wb1 = wb0 + 8;
  const int mb = a.max_blocks - 1;
  const int id0 = btr[min(wb0, mb)], id1 = btr[min(wb0 + 1, mb)];
  const int id2 = btr[min(wb1, mb)], id3 = btr[min(wb1 + 1, mb)];
  const int L = min(a.seq_lens[r], a.max_blocks * 16);  // never read past the table row
  const int nblk = (L + 15) >> 4;
  const bool w1_in = wb1 < nblk;

  // Projection partials.  Query terms: thread (column qi, part qp) takes the rotate-half
  // pairs (d, d + D/2), d = qp + TPQ m, of its column's head and row.  New tokens: thread
  // (row j, lane l) takes the pairs d = l + 32 m of K and V head g of the request's row j
  // (every workgroup loads them; only those holding new tokens use them).
  constexpr int HALF = D / 2;
  constexpr int TPQ = 256 / QG;    // threads per query column
  constexpr int DPT = HALF / TPQ;  // query pairs per thread
  constexpr int KPT = HALF / 32;   // K/V pairs per thread
  const int N = (2 * a.Hq + 2 * a.Hkv) * D;
  const int qi_t = tid / TPQ, qp = tid - qi_t * TPQ;
  const int hh_t = qi_t / a.q_rows, jr_t = qi_t - hh_t * a.q_rows;
  const int jn = tid >> 5, ln = tid & 31;
  const int krow = rq.base + min(jn, max(rq.n - 1, 0));
  float uq[NP][2][DPT], uk[NP][2][KPT], uv[NP][2][KPT];
  {
    const float* qsrc = a.qkv + (size_t)row_of(jr_t) * N + (size_t)(g * group + hh_t) * D;
    const float* ksrc = a.qkv + (size_t)krow * N + (size_t)(a.Hq + g) * D;
    const float* vsrc = ksrc + (size_t)a.Hkv * D;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int m = 0; m < DPT; ++m) uq[p][h2][m] = qsrc[p * a.part_stride + qp + TPQ * m + h2 * HALF];
#pragma unroll
        for (int m = 0; m < KPT; ++m) {
          uk[p][h2][m] = ksrc[p * a.part_stride + ln + 32 * m + h2 * HALF];
          uv[p][h2][m] = vsrc[p * a.part_stride + ln + 32 * m + h2 * HALF];
        }
      }
  }
  const int kpos = a.positions[krow];
  const int64_t kslot = a.slot_mapping[krow];
  constexpr int NE = (kQRows * HALF + 255) / 256;  // RoPE table entries per thread
  int epos[NE];
  double efreq[NE];  // kernel-argument reads are memory loads too
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int idx = min(tid + 256 * e, kQRows * HALF - 1);
    epos[e] = a.positions[row_of(idx / HALF)];
    efreq[e] = a.freq[idx % HALF];
  }
  load_win(W0, clamp_blk(id0), clamp_blk(id1));

  // query terms: slices summed in order from 0, per-head weightless RMSNorm over the
  // column's TPQ aligned lanes
  float x1[DPT], x2[DPT];
#pragma unroll
  for (int m = 0; m < DPT; ++m) {
    x1[m] = 0.f;
    x2[m] = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      x1[m] += uq[p][0][m];
      x2[m] += uq[p][1][m];
    }
  }
  if (a.qk_norm) {
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < DPT; ++m) ss += x1[m] * x1[m] + x2[m] * x2[m];
    ss = sd::group_sum<TPQ>(ss);
    const float rn = rsqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int m = 0; m < DPT; ++m) {
      x1[m] *= rn;
      x2[m] *= rn;
    }
  }
  // RoPE cos / sin of the request's rows: entry (jr, d) for the rotate-half pair d of row jr
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int idx = tid + 256 * e, jr = idx / HALF, d = idx - jr * HALF;
    if (idx < kQRows * HALF) rope_cs(epos[e], efreq[e], s_cos[jr][d], s_sin[jr][d]);
  }
  if (tid < ncb) s_bt[tid] = clamp_blk(bt0);
  for (int j = tid + 256; j < ncb; j += 256) s_bt[j] = clamp_blk(btr[blk_begin + j]);  // long chunks
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) qlow[qt] = a.window > 0 ? qpos[qt] - a.window : -1;

  // the new tokens sit at positions L - n .. L - 1 of the request (one workgroup per KV
  // head holds each of them)
  const int Ln0 = L - rq.n;
  const bool has_new = blk_begin < nblk && 16 * min(blk_begin + cb, nblk) > Ln0;
  if (has_new) {  // uniform
    // the new tokens are the request's rows: their RoPE entries are the table's, row jn
    __syncthreads();
    float k1[KPT], k2[KPT];
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      k1[m] = 0.f;
      k2[m] = 0.f;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        k1[m] += uk[p][0][m];
        k2[m] += uk[p][1][m];
      }
    }
    if (a.qk_norm) {  // each 32-lane group is one row
      float sk = 0.f;
#pragma unroll
      for (int m = 0; m < KPT; ++m) sk += k1[m] * k1[m] + k2[m] * k2[m];
      sk = sd::group_sum<32>(sk);
      const float rk = rsqrtf(sk / (float)D + a.eps);
#pragma unroll
      for (int m = 0; m < KPT; ++m) {
        k1[m] *= rk;
        k2[m] *= rk;
      }
    }
    if (ln == 0) s_kok[jn] = jn < rq.n && kslot >= 0;
    if (jn < rq.n) {
      const bool store =
          kslot >= 0 && (kpos >> 4) >= blk_begin && (kpos >> 4) < blk_begin + cb;
      const int64_t blk = kslot >> 4;
      const int off = (int)(kslot & 15);
      uint16_t* kp = a.k_cache + ((size_t)(blk * a.Hkv + g) * 16 + off) * D;
      uint16_t* vp = a.v_cache + (size_t)(blk * a.Hkv + g) * D * 16 + off;
#pragma unroll
      for (int m = 0; m < KPT; ++m) {
        const int d = ln + 32 * m;
        const float c = s_cos[jn][d], sn = s_sin[jn][d];
        float v1 = 0.f, v2 = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          v1 += uv[p][0][m];
          v2 += uv[p][1][m];
        }
        const uint16_t ka = sd::f2bf(k1[m] * c - k2[m] * sn), kb = sd::f2bf(k2[m] * c + k1[m] * sn);
        const uint16_t va = sd::f2bf(v1), vb = sd::f2bf(v2);
        s_kn[jn][d] = ka;
        s_kn[jn][d + HALF] = kb;
        s_vn[jn][d] = va;
        s_vn[jn][d + HALF] = vb;
        if (store) {
          kp[d] = ka;
          kp[d + HALF] = kb;
          vp[(size_t)d * 16] = va;
          vp[(size_t)(d + HALF) * 16] = vb;
        }
      }
    }
  }
  __syncthreads();  // angles and the new tokens' K/V staged; the new tokens stored
  load_win(W1, clamp_blk(w1_in ? id2 : id0), clamp_blk(w1_in ? id3 : id1));
  // the first window may hold the old cache contents of new tokens that are now stored
  if (has_new && 16 * wb0 + 32 > Ln0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int tk = 16 * wb0 + 8 * (i >> 2) + 4 * t + (i & 3) - Ln0;
      if (tk >= 0 && tk < rq.n && s_kok[tk]) {
#pragma unroll
        for (int c = 0; c < NC; ++c) W0.k[t][c] = *(const bf16x8_t*)&s_kn[tk][32 * c + 8 * G];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tv = 16 * wb0 + 8 * G + e - Ln0;
      if (tv >= 0 && tv < rq.n && s_kok[tv]) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) W0.v[dt][e] = __builtin_bit_cast(__bf16, s_vn[tv][16 * dt + i]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < DPT; ++m) {  // rotated query terms as bf16 hi/lo in LDS
    const int d = qp + TPQ * m;
    const float c = s_cos[jr_t][d], sn = s_sin[jr_t][d];
    const float y1 = x1[m] * c - x2[m] * sn, y2 = x2[m] * c + x1[m] * sn;
    uint16_t h1, l1, h2, l2;
    sd::split_bf16(y1, h1, l1);
    sd::split_bf16(y2, h2, l2);
    s_q[0][qi_t][d] = h1;
    s_q[1][qi_t][d] = l1;
    s_q[0][qi_t][d + HALF] = h2;
    s_q[1][qi_t][d + HALF] = l2;
  }
  __syncthreads();
  if (blk_begin >= nblk) return;  // past this request's end (uniform per workgroup)
  const int blk_end = min(blk_begin + cb, nblk);
  // later windows take their block ids from LDS (a window's second block past blk_end
  // re-reads its first)
  auto load_at = [&](Win& W, int wb) {
    load_win(W, s_bt[wb - blk_begin], s_bt[min(wb + 1, blk_end - 1) - blk_begin]);
  };

  float mrun[NQT], lsum[NQT];
  f32x4_t acc[NDT][NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    mrun[qt] = -INFINITY;
    lsum[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt][qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](Win& W, int wb) {
    const int tok_base = wb * 16;
    // V of tokens past the request's end is zeroed (the cache there may hold anything)
    const int nvalid = L - (tok_base + 8 * G);
    if (nvalid < 8) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= nvalid) W.v[dt][e] = (__bf16)0.0f;
    }
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      f32x4_t sh[2], slo[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) sh[t] = slo[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8_t qh = *(const bf16x8_t*)&s_q[0][16 * qt + i][32 * c + 8 * G];
        const bf16x8_t ql = *(const bf16x8_t*)&s_q[1][16 * qt + i][32 * c + 8 * G];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          sh[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(W.k[t][c], qh, sh[t], 0, 0, 0);
          slo[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(W.k[t][c], ql, slo[t], 0, 0, 0);
        }
      }
      // lane's scores: token tok_base + 8G + 4t + rr for query column 16qt + i
      float sc[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int tok = tok_base + 8 * G + 4 * t + rr;
          const float v = (tok <= qpos[qt] && tok > qlow[qt]) ? (sh[t][rr] + slo[t][rr]) * sl2
                                                               : -INFINITY;
          sc[t][rr] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, sd::lane_xor<16>(mx));
      mx = fmaxf(mx, sd::lane_xor<32>(mx));
      // lazy rescaling: a column's reference maximum moves only when a score exceeds it by
      // more than 2^8 (in exp2 units), so p <= 256 and the accumulators are rescaled rarely;
      // exp2(s - m) with any fixed m gives the same normalised result
      const bool grow = mx > mrun[qt] + 8.0f;
      const float mnew = grow ? mx : mrun[qt];
      const float alpha = (grow && mrun[qt] != -INFINITY) ? exp2f(mrun[qt] - mnew) : 1.f;
      bf16x8_t pb, pbl;
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float p = sc[t][rr] == -INFINITY ? 0.f : exp2f(sc[t][rr] - mnew);
          psum += p;
          const __bf16 ph = (__bf16)p;
          pb[4 * t + rr] = ph;
          pbl[4 * t + rr] = (__bf16)(p - (float)ph);
        }
      lsum[qt] = lsum[qt] * alpha + psum;
      mrun[qt] = mnew;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {  // wave-uniform
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt][qt] *= alpha;
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        acc[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(W.v[dt], pb, acc[dt][qt], 0, 0, 0);
        acc[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(W.v[dt], pbl, acc[dt][qt], 0, 0, 0);
      }
    }
  };

  // W0 holds window wb and W1 window wb + 8; each prefetch sits on its own path, so every
  // wait before a compute covers exactly the window it uses
  int wb = wb0;
  if (wb < blk_end) {
    while (true) {
      compute(W0, wb);
      const int w1 = wb + 8;
      if (w1 >= blk_end) break;
      const int w2 = w1 + 8;
      if (w2 >= blk_end) {
        compute(W1, w1);
        break;
      }
      load_at(W0, w2);
      compute(W1, w1);
      const int w3 = w2 + 8;
      if (w3 >= blk_end) {
        compute(W0, w2);
        break;
      }
      load_at(W1, w3);
      wb = w2;
    }
  }

  // cross-wave combine: rescale each wave's state to the chunk maximum, then add
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    float l = lsum[qt];
    l += sd::lane_xor<16>(l);
    l += sd::lane_xor<32>(l);
    lsum[qt] = l;
    if (G == 0) s_m[wave][16 * qt + i] = mrun[qt];
  }
  __syncthreads();
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int qi = 16 * qt + i;
    const float M = fmaxf(fmaxf(s_m[0][qi], s_m[1][qi]), fmaxf(s_m[2][qi], s_m[3][qi]));
    const float f = mrun[qt] == -INFINITY ? 0.f : exp2f(mrun[qt] - M);
    if (G == 0) s_l[wave][qi] = lsum[qt] * f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *(f32x4_t*)&s_acc[wave][qi][16 * dt + 4 * G] = acc[dt][qt] * f;
  }
  __syncthreads();
  const size_t pidx = (size_t)g * nslot + slot;
  float* pacc = a.part_acc + pidx * QG * D;
  float* pml = a.part_ml + pidx * QG * 2;
  for (int e = tid * 4; e < QG * D; e += 1024) {
    const int qi = e / D, d = e - qi * D;
    f32x4_t v = *(const f32x4_t*)&s_acc[0][qi][d];
    v += *(const f32x4_t*)&s_acc[1][qi][d];
    v += *(const f32x4_t*)&s_acc[2][qi][d];
    v += *(const f32x4_t*)&s_acc[3][qi][d];
    *(f32x4_t*)(pacc + e) = v;
    if (d == 0) {
      pml[2 * qi] = fmaxf(fmaxf(s_m[0][qi], s_m[1][qi]), fmaxf(s_m[2][qi], s_m[3][qi]));
      pml[2 * qi + 1] = s_l[0][qi] + s_l[1][qi] + s_l[2][qi] + s_l[3][qi];
    }
  }
}

// One workgroup of D threads per (query column, query head) of each request: LSE-combine
// the chunks, normalise, apply the output gate o * sigmoid(o_gate), store bf16 hi/lo terms.
// With one request, the first pass of chunk values (32 per thread), each thread's chunk
// statistics (one (m, l) pair per load) and the gate are loaded before seq_len is known:
// they read the chunk slots the launch allocates, and the slots past the request's chunk
// count are dropped by selection afterwards, so whatever they hold never reaches the result
// (with several, the chunk map comes first: its slots depend on every request's length).  Thread c turns
// chunk c's statistics into its weight exp2(m_c - M) (in LDS) and w_c * l_c (block-summed).
// GEN as for the split: partial drafts map the column to its row through query_start, and
// columns past a request's rows exit after issuing their loads.
template <bool GEN, int NP>
__global__ __launch_bounds__(128) void k_attn_combine(AttnArgs a, int cb_host, int nslot, int qg) {
  constexpr int PASS = 32;
  __shared__ __align__(16) float s_w[1024];
  __shared__ float s_lc[1024];
  __shared__ float s_red[4];
  const int tp = blockIdx.x / a.Hq, h = blockIdx.x - tp * a.Hq;
  const int d = threadIdx.x;
  const int r = tp / a.q_rows, jr = tp - r * a.q_rows;
  const int group = a.Hq / a.Hkv;
  const int g = h / group, hh = h - g * group;
  const int qi = hh * a.q_rows + jr;
  // the request's chunk slots: with one request all nslot slots (the chunks past its end
  // are dropped below); with several, the chunk map's
  int off = 0, nmax = nslot, cbm = cb_host;
  if (a.n_req > 1) {  // uniform
    const ChunkMap cm = chunk_map(a, cb_host, nslot);
    off = min(__builtin_amdgcn_readlane(cm.off, r), nslot - 1);
    nmax = max(min(__builtin_amdgcn_readlane(cm.nch, r), nslot - off), 1);
    cbm = cm.cb;
  }
  const size_t p0 = (size_t)g * nslot + off;
  const float* pa = a.part_acc + (p0 * qg + qi) * a.D + d;
  const size_t cs = (size_t)qg * a.D;  // chunk stride
  float vals[PASS];
#pragma unroll
  for (int u = 0; u < PASS; ++u) vals[u] = pa[min(u, nmax - 1) * cs];
  const float2 ml0 = *(const float2*)&a.part_ml[((p0 + min(d, nmax - 1)) * qg + qi) * 2];
  const ReqRows rq = GEN ? req_rows(a, r) : ReqRows{r * a.q_rows, a.q_rows};
  const int t = rq.base + min(jr, max(rq.n - 1, 0));  // the step row of this column
  float gate = 0.f;  // the output gate, slices summed in order
  {
    float gp[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p)
      gp[p] = a.gate[(size_t)p * a.part_stride + (size_t)t * a.gate_stride + h * a.D + d];
#pragma unroll
    for (int p = 0; p < NP; ++p) gate += gp[p];
  }
  const int L = min(a.seq_lens[r], a.max_blocks * 16);
  const int nc = max(min((((L + 15) >> 4) - (GEN ? first_block(a, r) : 0) + cbm - 1) / cbm,
                         nmax), 1);
  if (jr >= rq.n) return;  // uniform per workgroup, before any barrier
  // chunk statistics: thread c holds (m_c, l_c) of chunks c, c + D, ...
  // (the first chunk's pair is the one loaded above, kept out of the loop so it stays a
  // register value)
  s_w[d] = ml0.x;  // d < blockDim <= 1024; entries past nc are never used
  s_lc[d] = ml0.y;
  float mloc = d < nc ? ml0.x : -INFINITY;
  for (int c = d + (int)blockDim.x; c < nc; c += blockDim.x) {
    const float2 ml = *(const float2*)&a.part_ml[((p0 + c) * qg + qi) * 2];
    s_w[c] = ml.x;
    s_lc[c] = ml.y;
    mloc = fmaxf(mloc, ml.x);
  }
  mloc = sd::wave_max(mloc);
  if ((d & 63) == 0) s_red[d >> 6] = mloc;
  __syncthreads();
  const float M = blockDim.x > 64 ? fmaxf(s_red[0], s_red[1]) : s_red[0];
  float wl = 0.f;
  for (int c = d; c < nc; c += blockDim.x) {
    const float m = s_w[c];
    const float w = m == -INFINITY ? 0.f : exp2f(m - M);
    s_w[c] = w;
    wl += w * s_lc[c];
  }
  wl = sd::wave_sum(wl);
  __syncthreads();  // s_red reuse and s_w complete
  if ((d & 63) == 0) s_red[2 + (d >> 6)] = wl;
  __syncthreads();
  const float l = blockDim.x > 64 ? s_red[2] + s_red[3] : s_red[2];
  float o = 0.f;
  for (int c0 = 0; c0 < nc; c0 += PASS) {
    if (c0 > 0) {
#pragma unroll
      for (int u = 0; u < PASS; ++u) vals[u] = pa[min(c0 + u, nc - 1) * cs];
    }
#pragma unroll
    for (int u4 = 0; u4 < PASS / 4; ++u4) {
      const f32x4_t w4 = *(const f32x4_t*)&s_w[c0 + 4 * u4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c0 + 4 * u4 + j < nc) o += w4[j] * vals[4 * u4 + j];
    }
  }
  o /= l;
  const float sig = 1.0f / (1.0f + __expf(-gate));
  uint16_t hi, lo;
  sd::split_bf16(o * sig, hi, lo);
  const size_t oi = (size_t)t * a.Hq * a.D + h * a.D + d;
  a.out[oi] = hi;
  a.out_lo[oi] = lo;
}

}  // namespace

AttnPlan attn_plan(const sd_dims& d, int n_req, int max_seq_len, int window) {
  AttnPlan p;
  int span = (max_seq_len + 15) / 16;
  if (window > 0) span = min(span, (int)(((long)window + d.q_rows - 1 + 15) / 16) + 1);
  const long units = (long)n_req * d.n_kv_heads * span;
  // about one workgroup per CU (4 waves x 2-block windows, so a multiple of 8 blocks)
  int cb = 8;
  while (units / cb > 256 && cb < kMaxChunkBlocks) cb *= 2;
  p.chunk_blocks = cb;
  p.n_chunks = (span + cb - 1) / cb;
  p.qg = (d.n_q_heads / d.n_kv_heads) * d.q_rows;
  return p;
}

int attn_chunk_bound(const sd_dims& d, int n_req, int max_seq_len) {
  // a plan's chunks are at most units / cb + 1 <= 256 / (n_req * Hkv) + 1 when cb stops
  // below the cap, and span / kMaxChunkBlocks + 1 at the cap; the full span is one plan
  const int full = attn_plan(d, n_req, max_seq_len, 0).n_chunks;
  const int small = 256 / max(1, n_req * d.n_kv_heads) + 1;
  const int capped = (max_seq_len + 15) / 16 / kMaxChunkBlocks + 1;
  return max(full, max(small, capped));
}

hipError_t launch_attention(const AttnArgs& a, const AttnPlan& p, hipStream_t st) {
  // nslot chunk slots per KV head: as many workgroups as n_req requests of n_chunks chunks
  const int nslot = p.n_chunks * a.n_req;
  if (p.n_chunks > kMaxReqChunks) return hipErrorInvalidValue;
  const dim3 grid(nslot, a.Hkv), block(256);
  const bool gen = a.window > 0 || a.query_start != nullptr;
  if (a.nparts != 1 && a.nparts != 4) return hipErrorInvalidValue;
#define SD_ATTN_NP(DD, NQ, GN)                                                             \
  do {                                                                                     \
    if (a.nparts == 4)                                                                     \
      hipLaunchKernelGGL((k_attn_split<DD, NQ, GN, 4>), grid, block, 0, st, a,             \
                         p.chunk_blocks, nslot);                                           \
    else                                                                                   \
      hipLaunchKernelGGL((k_attn_split<DD, NQ, GN, 1>), grid, block, 0, st, a,             \
                         p.chunk_blocks, nslot);                                           \
  } while (0)
#define SD_ATTN(DD, NQ)                                                                    \
  do {                                                                                     \
    if (gen) SD_ATTN_NP(DD, NQ, true);                                                     \
    else SD_ATTN_NP(DD, NQ, false);                                                        \
  } while (0)
  if (a.D == 128 && p.qg == 32) SD_ATTN(128, 2);
  else if (a.D == 128 && p.qg == 16) SD_ATTN(128, 1);
  else if (a.D == 64 && p.qg == 32) SD_ATTN(64, 2);
  else if (a.D == 64 && p.qg == 16) SD_ATTN(64, 1);
  else if (a.D == 64 && p.qg == 64) SD_ATTN(64, 4);
  else return hipErrorInvalidValue;
#undef SD_ATTN
#undef SD_ATTN_NP
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 cgrid(a.n_req * a.q_rows * a.Hq), cblock(a.D);
#define SD_COMB(GN, NPV)                                                                   \
  hipLaunchKernelGGL((k_attn_combine<GN, NPV>), cgrid, cblock, 0, st, a, p.chunk_blocks,     \
                     nslot, p.qg)
  if (gen && a.nparts == 4) SD_COMB(true, 4);
  else if (gen) SD_COMB(true, 1);
  else if (a.nparts == 4) SD_COMB(false, 4);
  else SD_COMB(false, 1);
#undef SD_COMB
  return hipGetLastError();
}
