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
//   asm_lookup_partial  per (KV head, block of 16 queries, chunk of centroids):
//                       S = Q C^T on v_mfma_f32_16x16x32_bf16 with the queries as
//                       rows; each lane scores one centroid column against four
//                       queries, scales by 1/|c_k| (the |q| factor is common to all
//                       k), keeps the best (score, lowest k), and the workgroup
//                       reduces to one candidate per query and chunk.
//   asm_finalize        per query: best over chunks -> idx; gather abar[idx],
//                       log Zbar[idx]; merge with (self_out, self_lse).
#include "common.h"

namespace kvb {

constexpr int kAsmWaves = 4;
constexpr int kAsmChunk = 1024;  // centroids per workgroup

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
  __shared__ float red_s[kAsmWaves][16];
  __shared__ int red_k[kAsmWaves][16];

  const int chunk = blockIdx.x, g = blockIdx.y, qb = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lg = lane >> 4, lc = lane & 15;
  const int nq = a.B * a.G;

  // A operand: query row lc of this block (zero past the last query)
  const int qi = qb * 16 + lc;
  u32x4 qa[KK];
  {
    const bool ok = qi < nq;
    const int b = ok ? qi / a.G : 0, j = ok ? qi - (qi / a.G) * a.G : 0;
    const uint16_t* qp = a.q + ((size_t)(b * a.Hq + g * a.G + j)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qa[kk] = ok ? *(const u32x4*)(qp + 32 * kk + 8 * lg) : z;
    }
  }

  float best[4];
  int bestk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    best[i] = kNegInf;
    bestk[i] = 0x7FFFFFFF;
  }
  const uint16_t* cb = a.cent + (size_t)g * a.K * D;
  const int k0 = chunk * kAsmChunk;
  const int k1 = min(k0 + kAsmChunk, a.K);
  for (int kt = k0 + wave * 16; kt < k1; kt += 16 * kAsmWaves) {
    const int kc = kt + lc;  // this lane's centroid column
    const int kr = min(kc, a.K - 1);
    u32x4 cv[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) cv[kk] = *(const u32x4*)(cb + (size_t)kr * D + 32 * kk + 8 * lg);
    // |c|^2 of the column: 8 dims per lane per k-step, then over the 4 lane groups
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
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) S = mfma_16x16x32_bf16(qa[kk], cv[kk], S);
    const float inv = n2 > 0.f ? rsqrtf(n2) : 0.f;
    if (kc < k1 && n2 > 0.f) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = S[i] * inv;
        if (better(sc, kc, best[i], bestk[i])) {
          best[i] = sc;
          bestk[i] = kc;
        }
      }
    }
  }
  // reduce over the 16 centroid columns (lanes with equal lg)
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float os = __shfl_xor(best[i], o, 64);
      const int ok = __shfl_xor(bestk[i], o, 64);
      if (better(os, ok, best[i], bestk[i])) {
        best[i] = os;
        bestk[i] = ok;
      }
    }
  }
  if (lc == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red_s[wave][4 * lg + i] = best[i];
      red_k[wave][4 * lg + i] = bestk[i];
    }
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    float bs = red_s[0][threadIdx.x];
    int bk = red_k[0][threadIdx.x];
    for (int w = 1; w < kAsmWaves; ++w)
      if (better(red_s[w][threadIdx.x], red_k[w][threadIdx.x], bs, bk)) {
        bs = red_s[w][threadIdx.x];
        bk = red_k[w][threadIdx.x];
      }
    const size_t o = ((size_t)g * a.QB * 16 + qb * 16 + threadIdx.x) * a.KC + chunk;
    a.cand_score[o] = bs;
    a.cand_idx[o] = bk;
  }
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
  int k = (q2 > 0.f && bk != 0x7FFFFFFF) ? bk : 0;
  if (a.idx && lane == 0) a.idx[bh] = k;
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
    a.out[(size_t)bh * D + d] = (w1 * so + w2 * av) * inv;
  }
  if (lane == 0) a.out_lse[bh] = lse_out;
}

static void asm_dims(int B, int Hq, int Hkv, int K, int& G, int& QB, int& KC) {
  G = Hq / Hkv;
  QB = (B * G + 15) / 16;
  KC = (K + kAsmChunk - 1) / kAsmChunk;
}

}  // namespace kvb

using namespace kvb;

extern "C" size_t asm_lookup_merge_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t K) {
  (void)D;
  if (B < 1 || Hq < 1 || Hkv < 1 || K < 1 || Hq % Hkv) return 0;
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
  dim3 grid(a.KC, Hkv, a.QB);
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
