// One-wave candidate scan of the ASM cosine lookup ("Context Memorization for
// Efficient Long Context Generation", method step 3; GQA: one codebook per KV
// head), for kv_attn_decode_asm: a task is (128-centroid chunk, KV head, 64 query
// rows); the wave scores its 128 x 64 cosines on MFMA, four 16-centroid tiles in
// flight at a time, and writes, per query row, the best (score, lowest index) of
// the chunk.  (64-centroid tasks took 53.6 us per split launch on the ASM
// workload, 128-centroid ones 51.6 us, 256-centroid ones 51.9 us.)  Scores are q . c_k / |c_k| (|q| is
// common to a query row, so it does not change the row's argmax).  The merge kernel
// of the attention picks each row's best over the chunks (same rule).
#pragma once

#include "common.h"

namespace kvb {

constexpr int kScanChunk = 128;  // centroids per task (eight 16-column tiles, two rounds)
constexpr int kScanQB = 4;       // 16-query blocks per task

struct AsmScanArgs {
  const uint16_t* q;     // [B][Hq][D] bf16
  const uint16_t* cent;  // [Hkv][K][D] bf16
  float* cand_score;     // [Hkv][QB * 16][KC]
  int32_t* cand_idx;
  int32_t B, Hq, Hkv, K, G, QB, KC, tasks;
};

__device__ __forceinline__ bool scan_better(float s, int k, float bs, int bk) {
  return s > bs || (s == bs && k < bk);
}

template <int D>
__device__ __forceinline__ void asm_scan_wave(const AsmScanArgs& a, int task) {
  constexpr int KK = D / 32;
  if (task >= a.tasks) return;
  const int chunk = task % a.KC;
  const int rest = task / a.KC;
  const int g = rest % a.Hkv, qz = rest / a.Hkv;
  const int lane = threadIdx.x & 63;
  const int lg = lane >> 4, lc = lane & 15;
  const int nq = a.B * a.G;
  // A operands: query row lc of each of the task's query blocks (zero past the last)
  u32x4 qa[kScanQB][KK];
#pragma unroll
  for (int j = 0; j < kScanQB; ++j) {
    const int qi = (qz * kScanQB + j) * 16 + lc;
    const bool ok = qi < nq;
    const int b = ok ? qi / a.G : 0, jj = ok ? qi - (qi / a.G) * a.G : 0;
    const uint16_t* qp = a.q + ((size_t)(b * a.Hq + g * a.G + jj)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qa[j][kk] = ok ? *(const u32x4*)(qp + 32 * kk + 8 * lg) : z;
    }
  }
  const uint16_t* cb = a.cent + (size_t)g * a.K * D;
  const int k0 = chunk * kScanChunk;
  const int k1 = min(k0 + kScanChunk, a.K);
  float best[kScanQB][4];
  int bestk[kScanQB][4];
#pragma unroll
  for (int j = 0; j < kScanQB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      best[j][i] = kNegInf;
      bestk[j][i] = 0x7FFFFFFF;
    }
  for (int t0 = 0; t0 < kScanChunk / 16; t0 += 4) {  // four centroid tiles per round
  u32x4 cv[4][KK];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int kr = min(k0 + 16 * (t0 + it) + lc, a.K - 1);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) cv[it][kk] = *(const u32x4*)(cb + (size_t)kr * D + 32 * kk + 8 * lg);
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int kc = k0 + 16 * (t0 + it) + lc;  // this lane's centroid column
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
#pragma unroll
    for (int j = 0; j < kScanQB; ++j) {
      f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) S = mfma_16x16x32_bf16(qa[j][kk], cv[it][kk], S);
      if (live) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sc = S[i] * inv;
          if (scan_better(sc, kc, best[j][i], bestk[j][i])) {
            best[j][i] = sc;
            bestk[j][i] = kc;
          }
        }
      }
    }
  }
  }
  // over the 16 centroid columns (lanes with equal lg), then lane lc == 0 writes
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
#pragma unroll
    for (int j = 0; j < kScanQB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float os = __shfl_xor(best[j][i], o, 64);
        const int ok = __shfl_xor(bestk[j][i], o, 64);
        if (scan_better(os, ok, best[j][i], bestk[j][i])) {
          best[j][i] = os;
          bestk[j][i] = ok;
        }
      }
  }
  if (lc == 0) {
#pragma unroll
    for (int j = 0; j < kScanQB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (qz * kScanQB + j) * 16 + 4 * lg + i;  // query row of the output
        if (row < a.QB * 16) {
          const size_t o = ((size_t)g * a.QB * 16 + row) * a.KC + chunk;
          a.cand_score[o] = best[j][i];
          a.cand_idx[o] = bestk[j][i];
        }
      }
  }
}

}  // namespace kvb
