// Attention-state memory: cosine-argmax centroid lookup and lossless merge.
//
// "Context Memorization for Efficient Long Context Generation", method step 3:
// a decode query selects the centroid with the largest cosine similarity and
// fetches that entry's stored state (abar, Zbar); step 4 merges it with the
// query's own attention state (a, Z) weighting each output by its normaliser.
// Centroids are kept per KV head (the page's GQA extension); every query head
// searches its KV head's codebook with its own query.
//
// Kernels
//   asm_lookup_partial  per (KV head, four blocks of 16 queries, chunk of 256
//                       centroids): S = Q C^T on v_mfma_f32_16x16x32_bf16 with the
//                       queries as rows; each centroid tile is loaded once (all of
//                       a wave's tiles up front) and serves the four query blocks;
//                       each lane scores one centroid column against four queries
//                       per block, scales by 1/|c_k| (the |q| factor is common to
//                       all k), keeps the best (score, lowest k), and the workgroup
//                       reduces to one candidate per query and chunk.
//   asm_finalize        per query: best over chunks -> idx; gather abar[idx],
//                       log Zbar[idx]; merge with (self_out, self_lse).
#include <string.h>

#include "common.h"

namespace kvb {

constexpr int kAsmWaves = 4;
constexpr int kAsmChunk = 256;  // centroids per workgroup
constexpr int kAsmIt = kAsmChunk / (16 * kAsmWaves);  // 16-centroid tiles per wave
constexpr int kAsmQB = 4;  // blocks of 16 queries per workgroup (share each centroid load)

struct AsmArgs {
  const uint16_t* q;
  const uint16_t* cent;
  const uint16_t* abar;
  const float* log_zbar;
  const float* self_out;
  const float* self_lse;
  float* out;
  float* out_lse;
  int32_t* idx;
  float* cand_score;  // [Hkv][QB*16][KC]
  int32_t* cand_idx;
  int32_t B, Hq, Hkv, D, K, G, QB, KC;
};

__device__ __forceinline__ bool better(float s, int k, float bs, int bk) {
  return s > bs || (s == bs && k < bk);
}

template <int D>
__global__ __launch_bounds__(64 * kAsmWaves) void asm_lookup_partial(AsmArgs a) {
  constexpr int KK = D / 32;
  __shared__ float red_s[kAsmWaves][kAsmQB * 16];
  __shared__ int red_k[kAsmWaves][kAsmQB * 16];

  const int chunk = blockIdx.x, g = blockIdx.y, qz = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lg = lane >> 4, lc = lane & 15;
  const int nq = a.B * a.G;

  // A operands: query row lc of each of this workgroup's kAsmQB query blocks (zero
  // past the last query)
  u32x4 qa[kAsmQB][KK];
#pragma unroll
  for (int j = 0; j < kAsmQB; ++j) {
    const int qi = (qz * kAsmQB + j) * 16 + lc;
    const bool ok = qi < nq;
    const int b = ok ? qi / a.G : 0, jj = ok ? qi - (qi / a.G) * a.G : 0;
    const uint16_t* qp = a.q + ((size_t)(b * a.Hq + g * a.G + jj)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qa[j][kk] = ok ? *(const u32x4*)(qp + 32 * kk + 8 * lg) : z;
    }
  }

  float best[kAsmQB][4];
  int bestk[kAsmQB][4];
#pragma unroll
  for (int j = 0; j < kAsmQB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      best[j][i] = kNegInf;
      bestk[j][i] = 0x7FFFFFFF;
    }
  const uint16_t* cb = a.cent + (size_t)g * a.K * D;
  const int k0 = chunk * kAsmChunk;
  const int k1 = min(k0 + kAsmChunk, a.K);
  // every centroid tile of this wave is loaded before any is scored (one memory
  // round trip); columns past the codebook read its last row and are never scored
  u32x4 cv[kAsmIt][KK];
#pragma unroll
  for (int it = 0; it < kAsmIt; ++it) {
    const int kr = min(k0 + 16 * (wave + kAsmWaves * it) + lc, a.K - 1);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      cv[it][kk] = *(const u32x4*)(cb + (size_t)kr * D + 32 * kk + 8 * lg);
  }
#pragma unroll
  for (int it = 0; it < kAsmIt; ++it) {
    const int kc = k0 + 16 * (wave + kAsmWaves * it) + lc;  // this lane's centroid column
    // |c|^2 of the column: 8 dims per lane per k-step, then over the 4 lane groups
    float n2 = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float lo = bf16_bits_to_f32(cv[it][kk][w] & 0xFFFFu);
        const float hi = bf16_bits_to_f32(cv[it][kk][w] >> 16);
        n2 = fmaf(lo, lo, n2);
        n2 = fmaf(hi, hi, n2);
      }
    n2 += __shfl_xor(n2, 16, 64);
    n2 += __shfl_xor(n2, 32, 64);
    const float inv = n2 > 0.f ? rsqrtf(n2) : 0.f;
    const bool live = kc < k1 && n2 > 0.f;
    // the centroid tile is the B operand of every query block's product
#pragma unroll
    for (int j = 0; j < kAsmQB; ++j) {
      f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) S = mfma_16x16x32_bf16(qa[j][kk], cv[it][kk], S);
      if (live) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sc = S[i] * inv;
          if (better(sc, kc, best[j][i], bestk[j][i])) {
            best[j][i] = sc;
            bestk[j][i] = kc;
          }
        }
      }
    }
  }
  // reduce over the 16 centroid columns (lanes with equal lg)
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
#pragma unroll
    for (int j = 0; j < kAsmQB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float os = __shfl_xor(best[j][i], o, 64);
        const int ok = __shfl_xor(bestk[j][i], o, 64);
        if (better(os, ok, best[j][i], bestk[j][i])) {
          best[j][i] = os;
          bestk[j][i] = ok;
        }
      }
  }
  if (lc == 0) {
#pragma unroll
    for (int j = 0; j < kAsmQB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        red_s[wave][16 * j + 4 * lg + i] = best[j][i];
        red_k[wave][16 * j + 4 * lg + i] = bestk[j][i];
      }
  }
  __syncthreads();
  if (threadIdx.x < kAsmQB * 16) {
    const int r = threadIdx.x;
    float bs = red_s[0][r];
    int bk = red_k[0][r];
    for (int w = 1; w < kAsmWaves; ++w)
      if (better(red_s[w][r], red_k[w][r], bs, bk)) {
        bs = red_s[w][r];
        bk = red_k[w][r];
      }
    const int row = qz * kAsmQB * 16 + r;  // query row (block row * 16 + lane)
    if (row < a.QB * 16) {
      const size_t o = ((size_t)g * a.QB * 16 + row) * a.KC + chunk;
      a.cand_score[o] = bs;
      a.cand_idx[o] = bk;
    }
  }
}

// Step 4 for query (b, h) with stored entry k of KV head g: merge (self_out,
// self_lse) with (abar[k], log Zbar[k]) by their normalisers.  One wave.
__device__ __forceinline__ void merge_entry(const AsmArgs& a, int bh, int g, int k, int lane) {
  const int D = a.D;
  const float lz = a.log_zbar[(size_t)g * a.K + k];
  const float ls = a.self_lse[bh];
  const float M = fmaxf(ls, lz);
  float w1 = 0.f, w2 = 0.f, lse_out = kNegInf;
  if (M != kNegInf) {
    w1 = ls == kNegInf ? 0.f : __expf(ls - M);
    w2 = lz == kNegInf ? 0.f : __expf(lz - M);
    lse_out = M + __logf(w1 + w2);
  }
  const float inv = (w1 + w2) > 0.f ? 1.f / (w1 + w2) : 0.f;
  const uint16_t* ab = a.abar + ((size_t)g * a.K + k) * D;
  for (int d = lane; d < D; d += 64) {
    const float so = a.self_out[(size_t)bh * D + d];
    const float av = bf16_bits_to_f32(ab[d]);
    a.out[(size_t)bh * D + d] = fmaf(w1, so, w2 * av) * inv;
  }
  if (lane == 0) a.out_lse[bh] = lse_out;
}

// One wave per query (b, h): pick the best candidate, gather, merge.
__global__ __launch_bounds__(64) void asm_finalize(AsmArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh - (bh / a.Hq) * a.Hq;
  const int g = h / a.G, j = h - g * a.G;
  const int qi = b * a.G + j;
  const int lane = threadIdx.x;
  const int D = a.D;
  // |q|^2 (zero query -> index 0)
  float q2 = 0.f;
  for (int d = lane; d < D; d += 64) {
    const float x = bf16_bits_to_f32(a.q[(size_t)bh * D + d]);
    q2 = fmaf(x, x, q2);
  }
  q2 = wave_sum(q2);
  float bs = kNegInf;
  int bk = 0x7FFFFFFF;
  const size_t base = ((size_t)g * a.QB * 16 + qi) * a.KC;
  for (int c = lane; c < a.KC; c += 64) {
    const float s = a.cand_score[base + c];
    const int k = a.cand_idx[base + c];
    if (better(s, k, bs, bk)) {
      bs = s;
      bk = k;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float os = __shfl_xor(bs, o, 64);
    const int ok = __shfl_xor(bk, o, 64);
    if (better(os, ok, bs, bk)) {
      bs = os;
      bk = ok;
    }
  }
  const int k = (q2 > 0.f && bk != 0x7FFFFFFF) ? bk : 0;
  if (a.idx && lane == 0) a.idx[bh] = k;
  merge_entry(a, bh, g, k, lane);
}

// ------------------------------------------------------------------ two-level lookup
// Same page, technical-novelty section: a hierarchical index replaces the linear
// scan.  Entries are stored cluster by cluster (offs[j] .. offs[j+1]-1 hold the
// entries of first-level cluster j; kid gives each stored entry's original index).
//   asm_hier_select    per (query, KV head): cosine against the K1 first-level
//                      centroids, then the m best (equal similarities: lower
//                      cluster first) -> sel.
//   asm_hier_score     per (cluster, KV head): the cluster's entries against the
//                      queries that kept it (MFMA); each query's best entry as an
//                      atomic maximum of (ordered cosine, ~original index), so equal
//                      cosines go to the lowest original index whatever the order.
//   asm_hier_finalize  per query: index, gather, merge (as the linear lookup).
constexpr int kHierMaxK1 = 512;

struct HierArgs {
  AsmArgs a;                // q, abar and log_zbar (original order), self state, outputs
  const uint16_t* c1;       // [Hkv][K1][D]
  const int32_t* offs;      // [Hkv][K1 + 1]
  const uint16_t* stored;   // [Hkv][K][D], cluster by cluster
  const int32_t* kid;       // [Hkv][K]
  int32_t* sel;             // [Hkv][NQ][m]
  unsigned long long* best; // [Hkv][NQ]
  int32_t K1, m, NQ;
};

// Order-preserving float -> unsigned map (+0 and -0 equal).
__device__ __forceinline__ uint32_t ordf(float x) {
  uint32_t b = __float_as_uint(x);
  if ((b << 1) == 0) b = 0;
  return (b >> 31) ? ~b : (b | 0x80000000u);
}

// Query row lc of a 16-query tile as the MFMA A operand (zero when absent).
template <int D>
__device__ __forceinline__ void load_query_rows(const AsmArgs& a, int g, int qi, bool ok, int lg,
                                                u32x4* qa) {
  constexpr int KK = D / 32;
  const int b = ok ? qi / a.G : 0, jj = ok ? qi - (qi / a.G) * a.G : 0;
  const uint16_t* qp = a.q + ((size_t)(b * a.Hq + g * a.G + jj)) * D;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    u32x4 z = {0u, 0u, 0u, 0u};
    qa[kk] = ok ? *(const u32x4*)(qp + 32 * kk + 8 * lg) : z;
  }
}

// Column lc of a 16-vector tile as the MFMA B operand, and its squared norm.
template <int D>
__device__ __forceinline__ float load_columns(const uint16_t* row, int lg, u32x4* cv) {
  constexpr int KK = D / 32;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) cv[kk] = *(const u32x4*)(row + 32 * kk + 8 * lg);
  float n2 = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float lo = bf16_bits_to_f32(cv[kk][w] & 0xFFFFu);
      const float hi = bf16_bits_to_f32(cv[kk][w] >> 16);
      n2 = fmaf(lo, lo, n2);
      n2 = fmaf(hi, hi, n2);
    }
  n2 += __shfl_xor(n2, 16, 64);
  n2 += __shfl_xor(n2, 32, 64);
  return n2;
}

// One wave per (query, KV head): the first-level cosines (lane l scores clusters
// l, l + 64, ...), then the m best by repeated wave-wide selection.
template <int D>
__global__ __launch_bounds__(64) void asm_hier_select(HierArgs h) {
  constexpr int kMaxPer = kHierMaxK1 / 64;
  __shared__ float qs[D];
  const AsmArgs& a = h.a;
  const int qi = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
  const int b = qi / a.G, jj = qi - (qi / a.G) * a.G;
  const uint16_t* qp = a.q + ((size_t)(b * a.Hq + g * a.G + jj)) * D;
  for (int d = lane; d < D; d += 64) qs[d] = bf16_bits_to_f32(qp[d]);
  __syncthreads();
  const uint16_t* cb = h.c1 + (size_t)g * h.K1 * D;
  float sc[kMaxPer];
#pragma unroll
  for (int e = 0; e < kMaxPer; ++e) {
    sc[e] = kNegInf;
    const int j = lane + 64 * e;
    if (j < h.K1) {
      const u32x4* row = (const u32x4*)(cb + (size_t)j * D);
      u32x4 rv[D / 8];
#pragma unroll
      for (int c = 0; c < D / 8; ++c) rv[c] = row[c];
      float dot = 0.f, n2 = 0.f;
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        const u32x4 v = rv[c];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float lo = bf16_bits_to_f32(v[w] & 0xFFFFu);
          const float hi = bf16_bits_to_f32(v[w] >> 16);
          dot = fmaf(qs[8 * c + 2 * w], lo, dot);
          dot = fmaf(qs[8 * c + 2 * w + 1], hi, dot);
          n2 = fmaf(lo, lo, n2);
          n2 = fmaf(hi, hi, n2);
        }
      }
      sc[e] = n2 > 0.f ? dot * rsqrtf(n2) : kNegInf;
    }
  }
  // the m largest in (similarity desc, j asc) order, by wave ballots: u = ordered
  // bits of the similarity; T = the m-th largest u by bisection; keep every u > T
  // and the lowest-j entries with u == T until m are kept.  Lane l holds clusters
  // l + 64 e, so e-major lane order is j order.
  uint32_t u[kMaxPer];
#pragma unroll
  for (int e = 0; e < kMaxPer; ++e) u[e] = ordf(sc[e]);
  // (64 e < K1 is uniform: the slices past the last cluster are skipped)
  auto count_ge = [&](uint32_t th) -> int {
    int c = 0;
#pragma unroll
    for (int e = 0; e < kMaxPer; ++e)
      if (64 * e < h.K1) c += __popcll(__ballot(lane + 64 * e < h.K1 && u[e] >= th));
    return c;
  };
  unsigned long long lo = 0, hi = 0xFFFFFFFFull;  // count_ge(lo) >= m throughout
  while (lo < hi) {
    const unsigned long long mid = (lo + hi + 1) >> 1;
    if (count_ge((uint32_t)mid) >= h.m) lo = mid;
    else hi = mid - 1;
  }
  const uint32_t T = (uint32_t)lo;
  int above = 0;
#pragma unroll
  for (int e = 0; e < kMaxPer; ++e)
    if (64 * e < h.K1) above += __popcll(__ballot(lane + 64 * e < h.K1 && u[e] > T));
  int slot = 0, ties = h.m - above;
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int e = 0; e < kMaxPer; ++e) {
    if (64 * e >= h.K1) break;
    const bool valid = lane + 64 * e < h.K1;
    const unsigned long long eq = __ballot(valid && u[e] == T);
    const int eq_before = __popcll(eq & below);
    const bool keep = (valid && u[e] > T) || (valid && u[e] == T && eq_before < ties);
    const unsigned long long kb = __ballot(keep);
    if (keep) h.sel[((size_t)g * h.NQ + qi) * h.m + slot + __popcll(kb & below)] = lane + 64 * e;
    slot += __popcll(kb);
    ties -= min(ties, __popcll(eq));
  }
  if (lane == 0) h.best[(size_t)g * h.NQ + qi] = 0ull;
}

// One workgroup per (cluster, KV head): find the queries that kept the cluster
// (a scan of the selections, up to kHierRound queries per round), copy their rows
// to LDS, then score the cluster's entries against them on MFMA: each wave loads
// its 16-entry tiles once and runs every 16-query tile of the list against them;
// each query's best (ordered cosine, ~original index) is an LDS atomic maximum,
// then one global atomic maximum per listed query.
constexpr int kHierRound = 256;

template <int D>
__global__ __launch_bounds__(256) void asm_hier_score(HierArgs h) {
  constexpr int KK = D / 32;
  constexpr int kRowW = D / 8;  // 16-byte pieces per query row
  __shared__ int qlist[kHierRound];
  __shared__ int nlist;
  // one 16-byte pad per row: the 16 rows of a tile read from different banks
  __shared__ __attribute__((aligned(16))) u32x4 qrows[kHierRound][kRowW + 1];
  __shared__ unsigned long long qbest[kHierRound];
  const AsmArgs& a = h.a;
  const int j = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int nq = a.B * a.G;
  const int32_t* offs = h.offs + (size_t)g * (h.K1 + 1);
  const int32_t* sel = h.sel + (size_t)g * h.NQ * h.m;
  const uint16_t* cb = h.stored + (size_t)g * a.K * D;
  const int32_t* kid = h.kid + (size_t)g * a.K;
  const int o0 = offs[j], o1 = offs[j + 1];
  // the first kPre x 256 selections are loaded together with the cluster's range
  constexpr int kPre = 8;
  int sv0[kPre];
  {
    const int pf = min(nq, kHierRound) * h.m;
#pragma unroll
    for (int e = 0; e < kPre; ++e) sv0[e] = tid + 256 * e < pf ? sel[tid + 256 * e] : -1;
  }
  const int m0 = min(max(o0, 0), a.K), m1 = min(max(o1, m0), a.K);
  if (m0 >= m1) return;
  for (int base = 0; base < nq; base += kHierRound) {
    if (tid == 0) nlist = 0;
    qbest[tid] = 0ull;  // kHierRound == blockDim
    __syncthreads();
    // a query keeps a cluster at most once: scan its selections in memory order
    const int p1 = min(nq, base + kHierRound) * h.m;
    int pstart = base * h.m + tid;
    if (base == 0) {
#pragma unroll
      for (int e = 0; e < kPre; ++e)
        if (sv0[e] == j) qlist[atomicAdd(&nlist, 1)] = (tid + 256 * e) / h.m;
      pstart += kPre * 256;
    }
    for (int p0 = pstart; p0 < p1; p0 += kPre * 256) {
      int sv[kPre];
#pragma unroll
      for (int e = 0; e < kPre; ++e) sv[e] = p0 + 256 * e < p1 ? sel[p0 + 256 * e] : -1;
#pragma unroll
      for (int e = 0; e < kPre; ++e)
        if (sv[e] == j) qlist[atomicAdd(&nlist, 1)] = (p0 + 256 * e) / h.m;
    }
    __syncthreads();
    const int nl = nlist;
    if (nl == 0) continue;  // uniform
    // the listed queries' rows -> LDS (rows past the list up to the tile edge: 0)
    const int nlt = (nl + 15) & ~15;
    for (int e = tid; e < nlt * kRowW; e += 256) {
      const int r = e / kRowW, c = e - r * kRowW;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < nl) {
        const int qi = qlist[r];
        const int b = qi / a.G, jj = qi - (qi / a.G) * a.G;
        v = *(const u32x4*)(a.q + ((size_t)(b * a.Hq + g * a.G + jj)) * D + 8 * c);
      }
      qrows[r][c] = v;
    }
    __syncthreads();
    // Entries are the MFMA's A rows and queries its B columns, so lane (g4, c)
    // holds entries 4 g4 .. 4 g4 + 3 of a tile for query c.  Wave w takes entry
    // tiles w, w + 4, ...
    for (int mt = m0 + 16 * wave; mt < m1; mt += 64) {
      u32x4 cv[KK];
      int kd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kd[i] = kid[min(mt + 4 * lg + i, m1 - 1)];
      const float n2 = load_columns<D>(cb + (size_t)min(mt + lc, m1 - 1) * D, lg, cv);
      float inv[4];
      bool live[4], nz[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int me = 4 * lg + i;             // entry row of S[i]
        const float n2e = __shfl(n2, me, 64);  // lanes 0..15 hold the 16 norms
        live[i] = mt + me < m1;
        nz[i] = n2e > 0.f;                     // a zero entry scores -inf
        inv[i] = nz[i] ? rsqrtf(n2e) : 0.f;
      }
      for (int qt = 0; qt < nl; qt += 16) {
        u32x4 qb[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qb[kk] = qrows[qt + lc][4 * kk + lg];
        f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) S = mfma_16x16x32_bf16(cv[kk], qb[kk], S);
        unsigned long long pk = 0ull;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (live[i]) {
            const float sc = nz[i] ? S[i] * inv[i] : kNegInf;
            const unsigned long long key =
                ((unsigned long long)ordf(sc) << 32) | (0xFFFFFFFFu - (uint32_t)kd[i]);
            pk = key > pk ? key : pk;
          }
        }
        unsigned long long o2 = __shfl_xor(pk, 16, 64);
        pk = o2 > pk ? o2 : pk;
        o2 = __shfl_xor(pk, 32, 64);
        pk = o2 > pk ? o2 : pk;
        if (lg == 0 && qt + lc < nl && pk != 0ull) atomicMax(&qbest[qt + lc], pk);
      }
    }
    __syncthreads();
    for (int r = tid; r < nl; r += 256)
      if (qbest[r] != 0ull) atomicMax(&h.best[(size_t)g * h.NQ + qlist[r]], qbest[r]);
    __syncthreads();
  }
}

__global__ __launch_bounds__(64) void asm_hier_finalize(HierArgs h) {
  const AsmArgs& a = h.a;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, hh = bh - (bh / a.Hq) * a.Hq;
  const int g = hh / a.G, jj = hh - g * a.G;
  const int qi = b * a.G + jj;
  const int lane = threadIdx.x;
  float q2 = 0.f;
  for (int d = lane; d < a.D; d += 64) {
    const float x = bf16_bits_to_f32(a.q[(size_t)bh * a.D + d]);
    q2 = fmaf(x, x, q2);
  }
  q2 = wave_sum(q2);
  const unsigned long long pk = h.best[(size_t)g * h.NQ + qi];
  int k = 0;
  if (q2 > 0.f && pk != 0ull) {
    k = (int)(0xFFFFFFFFu - (uint32_t)(pk & 0xFFFFFFFFull));
    k = min(max(k, 0), a.K - 1);
  }
  if (a.idx && lane == 0) a.idx[bh] = k;
  merge_entry(a, bh, g, k, lane);
}

void asm_dims(int B, int Hq, int Hkv, int K, int& G, int& QB, int& KC) {
  G = Hq / Hkv;
  QB = (B * G + 15) / 16;
  KC = (K + kAsmChunk - 1) / kAsmChunk;
}

void launch_asm_candidates(const uint16_t* q, int B, int Hq, int Hkv, int D,
                           const uint16_t* centroids, int K, float* cand_score,
                           int32_t* cand_idx, hipStream_t s) {
  AsmArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.cent = centroids;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.K = K;
  asm_dims(B, Hq, Hkv, K, a.G, a.QB, a.KC);
  a.cand_score = cand_score;
  a.cand_idx = cand_idx;
  dim3 grid(a.KC, Hkv, (a.QB + kAsmQB - 1) / kAsmQB);
  TraceScope tr(kTrAsmLookup, s);
  if (D == 128)
    hipLaunchKernelGGL(asm_lookup_partial<128>, grid, dim3(64 * kAsmWaves), 0, s, a);
  else
    hipLaunchKernelGGL(asm_lookup_partial<64>, grid, dim3(64 * kAsmWaves), 0, s, a);
}

}  // namespace kvb

using namespace kvb;

extern "C" size_t asm_lookup_merge_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t K) {
  (void)D;
  // the entry's limits: B * G query rows per KV head at most 65536, K below 2^24
  if (B < 1 || Hq < 1 || Hkv < 1 || K < 1 || K >= (1 << 24) || Hq % Hkv ||
      (long long)B * (Hq / Hkv) > 65536)
    return 0;
  int G, QB, KC;
  asm_dims(B, Hq, Hkv, K, G, QB, KC);
  const size_t n = (size_t)Hkv * QB * 16 * KC;
  return kWsHeader + 2 * align_up(n * 4, 256);
}

extern "C" int32_t asm_lookup_merge(const void* q, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                    const void* centroids, const void* abar,
                                    const float* log_zbar, int32_t K, const float* self_out,
                                    const float* self_lse, float* out, float* out_lse,
                                    int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !centroids || !abar || !log_zbar || !self_out || !self_lse || !out || !out_lse)
    return KVB_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || K < 1 || K >= (1 << 24)) return KVB_EINVAL;
  if (D != 64 && D != 128) return KVB_EUNSUPPORTED;
  if ((long long)B * (Hq / Hkv) > 65536) return KVB_EINVAL;
  const size_t need = asm_lookup_merge_workspace(B, Hq, Hkv, D, K);
  if (!ws || ws_bytes < need) return KVB_EWORKSPACE;
  int32_t st = check_device();
  if (st) return st;
  AsmArgs a;
  a.q = (const uint16_t*)q;
  a.cent = (const uint16_t*)centroids;
  a.abar = (const uint16_t*)abar;
  a.log_zbar = log_zbar;
  a.self_out = self_out;
  a.self_lse = self_lse;
  a.out = out;
  a.out_lse = out_lse;
  a.idx = idx;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.K = K;
  asm_dims(B, Hq, Hkv, K, a.G, a.QB, a.KC);
  const size_t n = (size_t)Hkv * a.QB * 16 * a.KC;
  a.cand_score = (float*)((char*)ws + kWsHeader);
  a.cand_idx = (int32_t*)((char*)ws + kWsHeader + align_up(n * 4, 256));
  hipStream_t s = (hipStream_t)stream;
  dim3 grid(a.KC, Hkv, (a.QB + kAsmQB - 1) / kAsmQB);
  {
    TraceScope tr(kTrAsmLookup, s);
    if (D == 128)
      hipLaunchKernelGGL(asm_lookup_partial<128>, grid, dim3(64 * kAsmWaves), 0, s, a);
    else
      hipLaunchKernelGGL(asm_lookup_partial<64>, grid, dim3(64 * kAsmWaves), 0, s, a);
  }
  TraceScope tr(kTrAsmFinalize, s);
  hipLaunchKernelGGL(asm_finalize, dim3(B * Hq), dim3(64), 0, s, a);
  return launch_status();
}

static size_t hier_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t m, int& NQ,
                          size_t& o_sel, size_t& o_best) {
  const int G = Hq / Hkv;
  NQ = B * G;
  o_sel = kWsHeader;
  o_best = o_sel + align_up((size_t)Hkv * NQ * m * 4, 256);
  return o_best + align_up((size_t)Hkv * NQ * 8, 256);
}

extern "C" size_t asm_lookup_merge_hier_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t K1,
                                                  int32_t m) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || K1 < 1 || K1 > kHierMaxK1 || m < 1 || m > K1 ||
      (long long)B * (Hq / Hkv) > 65536)
    return 0;
  int NQ;
  size_t a, b;
  return hier_layout(B, Hq, Hkv, m, NQ, a, b);
}

extern "C" int32_t asm_lookup_merge_hier(const void* q, int32_t B, int32_t Hq, int32_t Hkv,
                                         int32_t D, const void* c1, int32_t K1,
                                         const int32_t* offs, const void* centroids,
                                         const int32_t* kid, int32_t K, int32_t m,
                                         const void* abar, const float* log_zbar,
                                         const float* self_out, const float* self_lse,
                                         float* out, float* out_lse, int32_t* idx, void* ws,
                                         size_t ws_bytes, void* stream) {
  if (!q || !c1 || !offs || !centroids || !kid || !abar || !log_zbar || !self_out ||
      !self_lse || !out || !out_lse)
    return KVB_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || K < 1 || K >= (1 << 24)) return KVB_EINVAL;
  if (K1 < 1 || K1 > kHierMaxK1 || m < 1 || m > K1) return KVB_EINVAL;
  if (D != 64 && D != 128) return KVB_EUNSUPPORTED;
  if ((long long)B * (Hq / Hkv) > 65536) return KVB_EINVAL;
  int NQ;
  size_t o_sel, o_best;
  const size_t need = hier_layout(B, Hq, Hkv, m, NQ, o_sel, o_best);
  if (!ws || ws_bytes < need) return KVB_EWORKSPACE;
  int32_t st = check_device();
  if (st) return st;
  HierArgs h;
  memset(&h, 0, sizeof(h));
  AsmArgs& a = h.a;
  a.q = (const uint16_t*)q;
  a.cent = nullptr;
  a.abar = (const uint16_t*)abar;
  a.log_zbar = log_zbar;
  a.self_out = self_out;
  a.self_lse = self_lse;
  a.out = out;
  a.out_lse = out_lse;
  a.idx = idx;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.K = K;
  a.G = Hq / Hkv;
  h.c1 = (const uint16_t*)c1;
  h.offs = offs;
  h.stored = (const uint16_t*)centroids;
  h.kid = kid;
  char* w = (char*)ws;
  h.sel = (int32_t*)(w + o_sel);
  h.best = (unsigned long long*)(w + o_best);
  h.K1 = K1;
  h.m = m;
  h.NQ = NQ;
  hipStream_t s = (hipStream_t)stream;
  {
    TraceScope tr(kTrAsmLookup, s);
    if (D == 128)
      hipLaunchKernelGGL(asm_hier_select<128>, dim3(NQ, Hkv), dim3(64), 0, s, h);
    else
      hipLaunchKernelGGL(asm_hier_select<64>, dim3(NQ, Hkv), dim3(64), 0, s, h);
  }
  {
    TraceScope tr(kTrAsmLookup, s);
    if (D == 128)
      hipLaunchKernelGGL(asm_hier_score<128>, dim3(K1, Hkv), dim3(256), 0, s, h);
    else
      hipLaunchKernelGGL(asm_hier_score<64>, dim3(K1, Hkv), dim3(256), 0, s, h);
  }
  TraceScope tr(kTrAsmFinalize, s);
  hipLaunchKernelGGL(asm_hier_finalize, dim3(B * Hq), dim3(64), 0, s, h);
  return launch_status();
}
