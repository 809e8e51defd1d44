// Attention-state memory construction (offline calibration) on the GPU.
//
// "Context Memorization for Efficient Long Context Generation": method step 1
// (each calibration query's attention state over the prefix, a = attn(q, K_p, V_p)
// with its normaliser Z), the chunked construction of the experiments (the prefix
// encoded in chunks whose states are merged), and step 2 (K-means over the
// collected queries; a cluster's query centroid is the mean of its members and
// its stored state the merge of their states).  Calibration queries, centroids
// and states are kept per KV head (the page's GQA extension).
//
// Kernels
//   asm_prefix_chunk<D>  per (KV head, 256 queries, prefix chunk), 8 waves: attention on
//                        v_mfma_f32_16x16x32_bf16 with the keys as rows.  S^T =
//                        K Q^T leaves every lane four keys of one query, which is
//                        the B-operand layout of O^T = V^T P^T once the two 16-key
//                        halves of a 32-key step are interleaved in the contraction
//                        index (the A operand, V^T, uses the same interleave); V is
//                        transposed (to fp16) by a pre-pass; K and V^T tiles go to
//                        XOR-swizzled LDS rows by global_load_lds.  The value
//                        product runs on v_mfma_f32_16x16x32_f16 (P rounded to fp16).
//   asm_prefix_merge<D>  per (KV head, query): merge of the chunks' states.
//   km_prep<D>           fp32 centroids -> bf16 hi, bf16 lo = c - hi, |c|^2.
//   km_assign<D>         per (KV head, 256 points): |c|^2 - 2 x.c for every
//                        centroid on MFMA (x is exact in bf16; c = hi + lo keeps
//                        16 significant bits), argmin with the lowest index on ties;
//                        centroid tiles go HBM -> LDS by global_load_lds into
//                        XOR-swizzled rows, double-buffered.
//   km_reduce<D, MERGE>  per (KV head, 64 clusters): scans the assignment in index
//                        order and accumulates each cluster's members in a fixed
//                        order (no float atomics, so results repeat bit for bit);
//                        MERGE = false writes member means as the new centroids
//                        (and their hi/lo/|c|^2), MERGE = true the merged states.
#include <string.h>

#include "common.h"

namespace kvb {

constexpr int kPfxQB = 256;     // queries per workgroup (8 waves x 2 tiles of 16)
constexpr int kPfxKT = 64;      // keys per LDS tile
constexpr int kKmPB = 256;      // points per workgroup (4 waves x 4 tiles of 16)
constexpr int kKmCT = 64;       // centroids per LDS tile
constexpr int kMaxPoints = 1 << 24;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

struct PrefixArgs {
  const uint16_t* q;   // [H][N][D]
  const uint16_t* k;   // [H][L][D]
  const uint16_t* v;   // [H][L][D]
  uint16_t* vt;        // [H][C][D][Lc]: V^T per chunk in fp16, keys interleaved (vt_prepare)
  uint32_t* rmax;      // [H][C][Lc / 64][D]: max |v| per 64-key tile and dimension (bits)
  int32_t* sexp;       // [H][C][D]: V^T row d of the chunk holds v * 2^-sexp (vt_prepare)
  int32_t* status;     // workspace status word (KVB_ERANGE for a non-finite v)
  float* out;          // [C][H][N][D]
  float* out_lse;      // [C][H][N]
  int32_t H, N, L, C, csize, Lc;
  float scale_log2;    // scale * log2(e)
};

// Position of chunk-local key kk in a V^T row: inside each 32-key block, keys
// 4g..4g+3 and 16+4g..16+4g+3 fill positions 8g..8g+7, the contraction slots lane
// group g supplies to O^T = V^T P^T (P^T arrives in the S^T accumulator layout).
__device__ __forceinline__ int vt_position(int kk) {
  const int w = kk & 31, g = (w & 15) >> 2, j = (w & 3) + (w >> 4) * 4;
  return (kk & ~31) + 8 * g + j;
}

// Per (KV head, chunk, 64-key tile): max |v| of every dimension over the tile's keys
// (float bits, which order like the values for |v|; NaN above +inf).
template <int D>
__global__ __launch_bounds__(256) void vt_range(PrefixArgs p) {
  __shared__ uint32_t part[256];
  const int tiles = p.Lc / 64;
  const int tt = blockIdx.x % tiles, hc = blockIdx.x / tiles;
  const int c = hc % p.C, h = hc / p.C;
  const int c0 = c * p.csize, c1 = min(p.L, c0 + p.csize);
  const int tid = threadIdx.x, d = tid % D, k0 = tid / D;
  constexpr int KS = 256 / D;  // keys read at a time
  uint32_t m = 0u;
  for (int r = k0; r < 64; r += KS) {
    const int gk = c0 + tt * 64 + r;
    if (gk < c1) m = max(m, (uint32_t)(p.v[((size_t)h * p.L + gk) * D + d] & 0x7FFFu) << 16);
  }
  part[tid] = m;
  __syncthreads();
  if (tid < D) {
    for (int j = 1; j < KS; ++j) m = max(m, part[tid + j * D]);
    p.rmax[((size_t)hc * tiles + tt) * D + tid] = m;
  }
}

// The power-of-two exponent s that brings max |v| = m (float bits) into [2^14, 2^15)
// (clamped to [-100, 113], the exponents a float multiplier can carry), so v * 2^-s
// is finite in fp16 and small dimensions keep fp16's full precision; kVtBad for a
// non-finite m.
constexpr int kVtBad = 1 << 20;
__device__ __forceinline__ int vt_exponent(uint32_t m) {
  const int e = (int)(m >> 23) - 127;  // floor(log2 m) for a normal m
  if (e >= 128) return kVtBad;
  return min(max(e - 14, -100), 113);
}

// V [H][L][D] bf16 -> V^T [H][C][D][Lc] fp16 (chunk-local keys at vt_position, zero
// past the chunk's end).  Row d of a chunk is scaled by 2^-s_d so that the chunk's
// max |v| in dimension d (vt_range) lies in [2^14, 2^15): every finite bf16 value
// fits, and a scaling by a power of two changes no significant bit of a bf16 value
// (the chunk kernel multiplies row d of its output back; inside float32's range the
// product and its accumulation scale exactly).  A non-finite v saturates and sets
// the status word.  One workgroup per (KV head,
// chunk, 64-key tile).  The tile is staged in LDS with rows of 32 keys and above
// swapped in 16-byte column pairs (chunk c at c ^ 1): a wave's transposed reads
// take rows k and k + 32 together, which would otherwise share banks.
template <int D>
__global__ __launch_bounds__(256) void vt_prepare(PrefixArgs p) {
  constexpr int RP = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t vs[64 * RP];
  __shared__ float s_mul[D];
  __shared__ int s_bad;
  const int tiles = p.Lc / 64;
  const int tt = blockIdx.x % tiles, hc = blockIdx.x / tiles;
  const int c = hc % p.C, h = hc / p.C;
  const int c0 = c * p.csize, c1 = min(p.L, c0 + p.csize);
  const int tid = threadIdx.x;
  constexpr int CPR = D / 8;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (tid < D) {
    uint32_t m = 0u;
    for (int t2 = 0; t2 < tiles; ++t2) m = max(m, p.rmax[((size_t)hc * tiles + t2) * D + tid]);
    int e = vt_exponent(m);
    if (e == kVtBad) {
      s_bad = 1;
      e = 0;
    }
    s_mul[tid] = __int_as_float((127 - e) << 23);  // 2^-e
    if (tt == 0) p.sexp[(size_t)hc * D + tid] = e;
  }
#pragma unroll
  for (int j = 0; j < 64 * CPR / 256; ++j) {
    const int ci = tid + 256 * j, r = ci / CPR, col = ci % CPR;
    const int gk = c0 + tt * 64 + r;
    const u32x4 x = gk < c1 ? *(const u32x4*)(p.v + ((size_t)h * p.L + gk) * D + col * 8)
                            : u32x4{0, 0, 0, 0};
    *(u32x4*)&vs[r * RP + ((col ^ ((r >> 5) & 1)) << 3)] = x;
  }
  __syncthreads();
  uint16_t* dst = p.vt + ((size_t)h * p.C + c) * D * p.Lc + tt * 64;
#pragma unroll
  for (int j = 0; j < D * 8 / 256; ++j) {
    const int ci = tid + 256 * j, d = ci / 8, q = ci % 8;  // positions 8q..8q+7 of row d
    uint32_t w[4];
    bool sat = false;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      // inverse of vt_position inside a 32-key block: position 8g + j -> key
      const int p0 = 8 * q + e, p1 = p0 + 1;
      const int k0 = (p0 & ~31) + 4 * ((p0 & 31) >> 3) + (p0 & 3) + ((p0 & 4) ? 16 : 0);
      const int k1 = (p1 & ~31) + 4 * ((p1 & 31) >> 3) + (p1 & 3) + ((p1 & 4) ? 16 : 0);
      const int c0s = (((d >> 3) ^ ((k0 >> 5) & 1)) << 3) + (d & 7);
      const int c1s = (((d >> 3) ^ ((k1 >> 5) & 1)) << 3) + (d & 7);
      const float x0 = bf16_bits_to_f32(vs[k0 * RP + c0s]) * s_mul[d];
      const float x1 = bf16_bits_to_f32(vs[k1 * RP + c1s]) * s_mul[d];
      sat |= !(fabsf(x0) <= 65504.f) || !(fabsf(x1) <= 65504.f);
      w[e / 2] = pack_f16x2(fminf(fmaxf(x0, -65504.f), 65504.f),
                            fminf(fmaxf(x1, -65504.f), 65504.f));
    }
    if (sat || (tid == 0 && s_bad)) p.status[0] = KVB_ERANGE;
    *(u32x4*)(dst + (size_t)d * p.Lc + 8 * q) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// LDS 16-byte slot holding chunk c of K row r (XOR swizzle: the 16 rows one MFMA
// operand read touches land in distinct banks).
template <int D>
__device__ __forceinline__ int k_slot(int r, int c) {
  if constexpr (D == 128)
    return c ^ (r & 15);
  else
    return c ^ ((r >> 1) & 7);
}
__device__ __forceinline__ int vt_slot(int d, int c) { return c ^ ((d >> 1) & 7); }

template <int D>
__global__ __launch_bounds__(512) void asm_prefix_chunk(PrefixArgs p) {
  constexpr int DS = D / 32;          // 32-wide contraction steps of S^T
  constexpr int DT = D / 16;          // 16-row tiles of O^T
  constexpr int KRB = D * 2;          // K row bytes
  constexpr int KCPR = D / 8;         // 16-byte chunks per K row
  constexpr int KB = kPfxKT * KRB;    // K tile bytes
  constexpr int VB = D * kPfxKT * 2;  // V^T tile bytes (D rows of 64 keys)
  constexpr int KI = KB / 1024, VI = VB / 1024;  // 1 KB DMA instructions per tile
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * (KB + VB)];

  const int H = p.H;
  const int h = blockIdx.x % H, qb = blockIdx.x / H, c = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int c0 = c * p.csize;
  const int c1 = min(p.L, c0 + p.csize);
  const int nt = c1 > c0 ? (c1 - c0 + kPfxKT - 1) / kPfxKT : 0;
  const uint16_t* kh = p.k + (size_t)h * p.L * D;
  const uint16_t* vth = p.vt + ((size_t)h * p.C + c) * D * p.Lc;

  // B operand of S^T: query column lc of each of the wave's two tiles
  u32x4 qr[2][DS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int n = qb * kPfxQB + wave * 32 + qt * 16 + lc;
    const uint16_t* qp = p.q + ((size_t)h * p.N + n) * D + 8 * lg;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qr[qt][ds] = n < p.N ? *(const u32x4*)(qp + ds * 32) : u32x4{0, 0, 0, 0};
  }

  f32x4 o[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt][0] = o[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {kNegInf, kNegInf}, ls[2] = {0.f, 0.f};

  // Tile t's K rows (rows past the prefix end read its last row; their scores
  // are masked) and V^T block into LDS buffer `buf`, HBM -> LDS directly.
  auto issue = [&](int t, int buf) {
    unsigned char* kb = lds + buf * (KB + VB);
    unsigned char* vb = kb + KB;
    for (int i = wave; i < KI; i += kPfxQB / 32) {
      const int r = i * (1024 / KRB) + lane / KCPR, slot = lane % KCPR;
      const int gk = min(c0 + t * kPfxKT + r, p.L - 1);
      __builtin_amdgcn_global_load_lds((glb_void_t*)(kh + (size_t)gk * D + k_slot<D>(r, slot) * 8),
                                       (lds_void_t*)(kb + i * 1024), 16, 0, 0);
    }
    for (int i = wave; i < VI; i += kPfxQB / 32) {
      const int d = i * 8 + lane / 8, slot = lane % 8;
      __builtin_amdgcn_global_load_lds(
          (glb_void_t*)(vth + (size_t)d * p.Lc + t * kPfxKT + vt_slot(d, slot) * 8),
          (lds_void_t*)(vb + i * 1024), 16, 0, 0);
    }
  };

  if (nt > 0) issue(0, 0);
  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    // this wave's transfers for tile t have landed (the compiler does not track
    // LDS written by global_load_lds); the barrier makes every wave's visible and
    // frees the other buffer (its tile was computed by everyone)
    wait_vmem_all();
    __syncthreads();
    if (t + 1 < nt) issue(t + 1, buf ^ 1);
    const unsigned char* kb = lds + buf * (KB + VB);
    const unsigned char* vb = kb + KB;

    // S^T tiles: rows = keys kt*16 + 4lg + i, column = this lane's query
    f32x4 s[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt][0] = s[kt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = kt * 16 + lc;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const u32x4 a = *(const u32x4*)(kb + r * KRB + 16 * k_slot<D>(r, ds * 4 + lg));
        s[kt][0] = mfma_16x16x32_bf16(a, qr[0][ds], s[kt][0]);
        s[kt][1] = mfma_16x16x32_bf16(a, qr[1][ds], s[kt][1]);
      }
    }
    const int valid = c1 - (c0 + t * kPfxKT);  // >= 1
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = s[kt][qt][i] * p.scale_log2;
          if (kt * 16 + 4 * lg + i >= valid) x = kNegInf;
          s[kt][qt][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m[qt], mx);
      const float alpha = exp2_fast(m[qt] - mn);
      m[qt] = mn;
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = exp2_fast(s[kt][qt][i] - mn);
          s[kt][qt][i] = pv;
          sum += pv;
        }
      ls[qt] = ls[qt] * alpha + sum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][qt] *= alpha;
    }

    // O^T += V^T P^T over two 32-key steps; contraction slot 8lg + j holds key
    // 32ks + 4lg + j (j < 4) or 32ks + 16 + 4lg + (j - 4)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // P in fp16 (11 significant bits; a single bf16 rounding of the weights would
      // cost up to ~2e-3 of the output's scale), V^T in fp16
      u32x4 pf[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const f32x4 x0 = s[2 * ks][qt], x1 = s[2 * ks + 1][qt];
        pf[qt] = u32x4{pack_f16x2(x0[0], x0[1]), pack_f16x2(x0[2], x0[3]),
                       pack_f16x2(x1[0], x1[1]), pack_f16x2(x1[2], x1[3])};
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 16 + lc;
        const u32x4 a = *(const u32x4*)(vb + d * 128 + 16 * vt_slot(d, 4 * ks + lg));
        o[dt][0] = mfma_16x16x32_f16(a, pf[0], o[dt][0]);
        o[dt][1] = mfma_16x16x32_f16(a, pf[1], o[dt][1]);
      }
    }
  }

#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float l = ls[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int n = qb * kPfxQB + wave * 32 + qt * 16 + lc;
    if (n >= p.N) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const size_t row = ((size_t)c * H + h) * p.N + n;
    float* dst = p.out + row * D + 4 * lg;
    // V^T row d held v * 2^-s_d (vt_prepare): scale output element d back (no V and
    // no exponents for an empty prefix)
    const i32x4* se = (const i32x4*)(p.sexp + ((size_t)h * p.C + c) * D + 4 * lg);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const i32x4 e4 = p.L > 0 ? se[dt * 4] : i32x4{0, 0, 0, 0};
      f32x4 x = o[dt][qt] * inv;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] *= __int_as_float((127 + e4[i]) << 23);
      *(f32x4*)(dst + dt * 16) = x;
    }
    if (lg == 0) p.out_lse[row] = l > 0.f ? m[qt] * kLn2 + logf(l) : kNegInf;
  }
}

// Merge of C chunk states per (KV head, query) in chunk order: sixteen lanes per
// row, D/16 consecutive elements per lane.
template <int D>
__global__ __launch_bounds__(256) void asm_prefix_merge(const float* part, const float* plse,
                                                       float* a, float* lse, int32_t rows,
                                                       int32_t C) {
  constexpr int V = D / 16;
  const int lane = threadIdx.x & 63, lg = lane >> 4, lc = lane & 15;
  const int r = blockIdx.x * 16 + (threadIdx.x >> 6) * 4 + lg;
  if (r >= rows) return;
  float M = kNegInf;
  for (int c = 0; c < C; ++c) M = fmaxf(M, plse[(size_t)c * rows + r]);
  float acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = 0.f;
  float Z = 0.f;
  if (M != kNegInf) {
    for (int c = 0; c < C; ++c) {
      const float w = exp2_fast((plse[(size_t)c * rows + r] - M) * kLog2e);
      const float* src = part + ((size_t)c * rows + r) * D + lc * V;
      Z += w;
#pragma unroll
      for (int j = 0; j < V; j += 4) {
        const f32x4 x = *(const f32x4*)(src + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[j + e] += w * x[e];
      }
    }
  }
  const float inv = Z > 0.f ? 1.f / Z : 0.f;
  float* dst = a + (size_t)r * D + lc * V;
#pragma unroll
  for (int j = 0; j < V; j += 4)
    *(f32x4*)(dst + j) = f32x4{acc[j] * inv, acc[j + 1] * inv, acc[j + 2] * inv, acc[j + 3] * inv};
  if (lc == 0) lse[r] = Z > 0.f ? M + logf(Z) : kNegInf;
}

struct KmArgs {
  const uint16_t* x;   // [H][N][D] points (bf16)
  float* cent;         // [H][K][D] centroids (fp32)
  uint16_t* hi;        // [H][K][D] bf16 of the centroids, read by km_assign
  uint16_t* hi_out;    // where km_reduce writes hi (hi, or the caller's bf16 copy)
  uint16_t* lo;        // [H][K][D] bf16 of (c - hi)
  float* cnorm;        // [H][K]  |c|^2
  int32_t* assign;     // [H][N]
  int32_t* counts;     // [H][K] or null
  const float* a;      // [H][N][D] states (merge mode)
  const float* lse;    // [H][N]
  uint16_t* abar;      // [H][K][D] bf16
  float* log_zbar;     // [H][K]
  int32_t H, N, K;
};

// Writes hi, lo and |c|^2 of one centroid row held by 16 lanes (lane lc holds the
// D/16 consecutive elements starting at lc * D/16); the caller's 16 lanes must be
// active together.
template <int D>
__device__ __forceinline__ void km_prep_row(const KmArgs& k, size_t row, const float* v, int lc,
                                            uint16_t* hi_dst) {
  constexpr int V = D / 16;
  uint32_t hb[V / 2], lb[V / 2];
  float sq = 0.f;
#pragma unroll
  for (int j = 0; j < V; j += 2) {
    split_bf16x2(v[j], v[j + 1], hb[j / 2], lb[j / 2]);
    sq = fmaf(v[j], v[j], sq);
    sq = fmaf(v[j + 1], v[j + 1], sq);
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) sq += __shfl_xor(sq, o, 64);
  const size_t off = row * D + (size_t)lc * V;
  if constexpr (V == 8) {
    *(u32x4*)(hi_dst + off) = u32x4{hb[0], hb[1], hb[2], hb[3]};
    *(u32x4*)(k.lo + off) = u32x4{lb[0], lb[1], lb[2], lb[3]};
  } else {
    *(uint2*)(hi_dst + off) = uint2{hb[0], hb[1]};
    *(uint2*)(k.lo + off) = uint2{lb[0], lb[1]};
  }
  if (lc == 0) k.cnorm[row] = sq;
}

template <int D>
__global__ __launch_bounds__(256) void km_prep(KmArgs k) {
  constexpr int V = D / 16;
  const int lane = threadIdx.x & 63, lg = lane >> 4, lc = lane & 15;
  const size_t row = (size_t)blockIdx.x * 16 + (threadIdx.x >> 6) * 4 + lg;
  if (row >= (size_t)k.H * k.K) return;
  float v[V];
  const float* src = k.cent + row * D + lc * V;
#pragma unroll
  for (int j = 0; j < V; j += 4) {
    const f32x4 x = *(const f32x4*)(src + j);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[j + e] = x[e];
  }
  km_prep_row<D>(k, row, v, lc, k.hi);
}

template <int D>
__global__ __launch_bounds__(256) void km_assign(KmArgs k) {
  constexpr int DS = D / 32;
  constexpr int RB = D * 2;           // centroid row bytes
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int TB = kKmCT * RB;      // bytes of one tile of one part
  constexpr int NI = TB / 1024;       // 1 KB DMA instructions per part and tile
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2][2 * TB];
  __shared__ __attribute__((aligned(16))) float Cn[2][kKmCT];

  const int H = k.H, K = k.K;
  const int h = blockIdx.x % H, pb = blockIdx.x / H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int nt = (K + kKmCT - 1) / kKmCT;
  const uint16_t* hh = k.hi + (size_t)h * K * D;
  const uint16_t* lh = k.lo + (size_t)h * K * D;
  const float* nh = k.cnorm + (size_t)h * K;

  u32x4 xr[4][DS];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    const int n = pb * kKmPB + wave * 64 + pt * 16 + lc;
    const uint16_t* xp = k.x + ((size_t)h * k.N + n) * D + 8 * lg;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      xr[pt][ds] = n < k.N ? *(const u32x4*)(xp + ds * 32) : u32x4{0, 0, 0, 0};
  }
  float best[4];
  int bi[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    best[pt] = __builtin_huge_valf();
    bi[pt] = 0x7FFFFFFF;
  }

  // Tile t's hi and lo rows HBM -> LDS (rows past K repeat row K-1: their norm is
  // replaced by +inf below), and their norms; XOR-swizzled 16-byte slots.
  auto issue = [&](int t, int buf) {
    for (int i = wave; i < NI; i += 4) {
      const int r = i * (1024 / RB) + lane / CPR, slot = lane % CPR;
      const int c = (CPR == 16) ? (slot ^ (r & 15)) : (slot ^ ((r >> 1) & 7));
      const size_t src = (size_t)min(t * kKmCT + r, K - 1) * D + c * 8;
      __builtin_amdgcn_global_load_lds((glb_void_t*)(hh + src), (lds_void_t*)(lds[buf] + i * 1024),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((glb_void_t*)(lh + src),
                                       (lds_void_t*)(lds[buf] + TB + i * 1024), 16, 0, 0);
    }
    if (wave == 0)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(nh + min(t * kKmCT + lane, K - 1)),
                                       (lds_void_t*)Cn[buf], 4, 0, 0);
  };

  issue(0, 0);
  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    // this wave's transfers for tile t have landed (LDS written by global_load_lds
    // is not tracked by the compiler); the barrier makes every wave's visible and
    // frees the other buffer
    wait_vmem_all();
    __syncthreads();
    if (t + 1 < nt) issue(t + 1, buf ^ 1);
    const unsigned char* ch = lds[buf];
    const unsigned char* cl = lds[buf] + TB;

#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      f32x4 s[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) s[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = ct * 16 + lc;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const int cc = ds * 4 + lg;
        const int slot = (CPR == 16) ? (cc ^ (row & 15)) : (cc ^ ((row >> 1) & 7));
        const u32x4 ah = *(const u32x4*)(ch + row * RB + 16 * slot);
        const u32x4 al = *(const u32x4*)(cl + row * RB + 16 * slot);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) s[pt] = mfma_16x16x32_bf16(ah, xr[pt][ds], s[pt]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) s[pt] = mfma_16x16x32_bf16(al, xr[pt][ds], s[pt]);
      }
      const f32x4 cn = *(const f32x4*)&Cn[buf][ct * 16 + 4 * lg];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = t * kKmCT + ct * 16 + 4 * lg + i;
        const float cni = kk < K ? cn[i] : __builtin_huge_valf();
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const float d = fmaf(-2.f, s[pt][i], cni);
          if (d < best[pt]) {
            best[pt] = d;
            bi[pt] = kk;
          }
        }
      }
    }
  }

#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float d2 = __shfl_xor(best[pt], o, 64);
      const int i2 = __shfl_xor(bi[pt], o, 64);
      if (d2 < best[pt] || (d2 == best[pt] && i2 < bi[pt])) {
        best[pt] = d2;
        bi[pt] = i2;
      }
    }
    const int n = pb * kKmPB + wave * 64 + pt * 16 + lc;
    if (lg == 0 && n < k.N) k.assign[(size_t)h * k.N + n] = bi[pt];
  }
}

// One workgroup of 16 waves per (KV head, 64 clusters); wave w owns clusters
// k0 + w + 16c (c = 0..3).  The assignment is taken in passes of 16 x 1024 labels:
// wave w scans the pass's w-th run of 1024 labels (all loaded up front) and lists,
// in index order, those that fall in the block's clusters in its own LDS region.
// After one barrier each wave walks the regions in wave order (that is, in index
// order), copies its own clusters' members to a private buffer and works them off
// sixteen at a time, lane group lg taking every fourth, so that every sum is
// formed in an order fixed by N and the assignment alone.
template <int D, bool MERGE>
__global__ __launch_bounds__(1024) void km_reduce(KmArgs k) {
  constexpr int V = D / 16;
  constexpr int kRun = 1024;  // labels per wave per pass
  constexpr int kWaveBuf = 256;  // per-wave member buffer
  __shared__ uint32_t list[16 * kRun];
  __shared__ uint32_t wbuf[16 * kWaveBuf];
  __shared__ int wcnt[16];
  const int H = k.H;
  const int h = blockIdx.x % H, k0 = (blockIdx.x / H) * 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int32_t* lab = k.assign + (size_t)h * k.N;

  float acc[4][V];
  float mm[4], ss[4];
  int cnt[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int j = 0; j < V; ++j) acc[c][j] = 0.f;
    mm[c] = kNegInf;
    ss[c] = 0.f;
    cnt[c] = 0;
  }

  // This wave's members, in index order, buffered in `mine` and worked off sixteen
  // at a time: lane group lg takes entries lg, lg + 4, ... of each batch (all row
  // loads of a batch are in flight together).
  uint32_t* mine = wbuf + wave * kWaveBuf;
  auto work_off = [&](int nm) {
    for (int b0 = 0; b0 < nm; b0 += 16) {
      uint32_t e[4];
      float val[4][V];
      float vl[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int j = b0 + 4 * bb + lg;
        e[bb] = j < nm ? mine[j] : 0xFFFFFFFFu;
        vl[bb] = kNegInf;
#pragma unroll
        for (int q = 0; q < V; ++q) val[bb][q] = 0.f;
        if (e[bb] == 0xFFFFFFFFu) continue;
        const size_t pi = (size_t)h * k.N + (e[bb] >> 6);
        if constexpr (MERGE) {
          const float* sp = k.a + pi * D + lc * V;
#pragma unroll
          for (int q = 0; q < V; q += 4) {
            const f32x4 x = *(const f32x4*)(sp + q);
#pragma unroll
            for (int r = 0; r < 4; ++r) val[bb][q + r] = x[r];
          }
          vl[bb] = k.lse[pi];
        } else {
          const uint16_t* xp = k.x + pi * D + lc * V;
          uint32_t w[V / 2];
          if constexpr (V == 8) {
            const u32x4 x = *(const u32x4*)xp;
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] = x[r];
          } else {
            const uint2 x = *(const uint2*)xp;
            w[0] = x.x;
            w[1] = x.y;
          }
#pragma unroll
          for (int r = 0; r < V / 2; ++r) {
            val[bb][2 * r] = bf16_bits_to_f32(w[r] & 0xFFFFu);
            val[bb][2 * r + 1] = bf16_bits_to_f32(w[r] >> 16);
          }
        }
      }
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        if (e[bb] == 0xFFFFFFFFu) continue;
        const int cs = (int)((e[bb] & 63u) >> 4);
        // selects rather than a branch per cluster: keeps acc[][] in registers
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bool hit = c == cs;
          cnt[c] += hit ? 1 : 0;
          if constexpr (MERGE) {
            const bool use = hit && vl[bb] != kNegInf;
            const float mn = use ? fmaxf(mm[c], vl[bb]) : mm[c];
            const float sc = use ? exp2_fast((mm[c] - mn) * kLog2e) : 1.f;
            const float wi = use ? exp2_fast((vl[bb] - mn) * kLog2e) : 0.f;
#pragma unroll
            for (int q = 0; q < V; ++q)
              acc[c][q] = use ? acc[c][q] * sc + wi * val[bb][q] : acc[c][q];
            ss[c] = use ? ss[c] * sc + wi : ss[c];
            mm[c] = mn;
          } else {
#pragma unroll
            for (int q = 0; q < V; ++q) acc[c][q] = hit ? acc[c][q] + val[bb][q] : acc[c][q];
          }
        }
      }
    }
  };

  for (int s0 = 0; s0 < k.N; s0 += 16 * kRun) {
    const int r0 = s0 + wave * kRun;
    int labv[kRun / 64];
#pragma unroll
    for (int r = 0; r < kRun / 64; ++r) {
      const int i = r0 + r * 64 + lane;
      labv[r] = i < k.N ? lab[i] : -1;
    }
    int n = 0;
#pragma unroll
    for (int r = 0; r < kRun / 64; ++r) {
      const int i = r0 + r * 64 + lane;
      const int loc = labv[r] - k0;
      const bool in = labv[r] >= 0 && (unsigned)loc < 64u;
      const uint64_t bal = __ballot(in);
      if (in) list[wave * kRun + n + __popcll(bal & ((1ull << lane) - 1ull))] =
          ((uint32_t)i << 6) | loc;
      n += __popcll(bal);
    }
    if (lane == 0) wcnt[wave] = n;
    __syncthreads();
    // collect this wave's clusters' members from the regions, in wave (= index) order
    int nm = 0;
    for (int w2 = 0; w2 < 16; ++w2) {
      const int n2 = wcnt[w2];
      for (int j0 = 0; j0 < n2; j0 += 64) {
        const bool ok = j0 + lane < n2;
        const uint32_t ev = ok ? list[w2 * kRun + j0 + lane] : 0u;
        const bool my = ok && (int)(ev & 15u) == wave;
        const uint64_t bal = __ballot(my);
        if (my) mine[nm + __popcll(bal & ((1ull << lane) - 1ull))] = ev;
        nm += __popcll(bal);
        if (nm > kWaveBuf - 64) {
          work_off(nm);
          nm = 0;
        }
      }
    }
    work_off(nm);
    __syncthreads();  // regions and counts are rewritten by the next pass
  }

  // combine the four lane groups (xor 16, then xor 32)
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      if constexpr (MERGE) {
        const float m2 = __shfl_xor(mm[c], o, 64), s2 = __shfl_xor(ss[c], o, 64);
        const float mn = fmaxf(mm[c], m2);
        const float e1 = mn == kNegInf ? 0.f : exp2_fast((mm[c] - mn) * kLog2e);
        const float e2 = mn == kNegInf ? 0.f : exp2_fast((m2 - mn) * kLog2e);
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const float a2 = __shfl_xor(acc[c][j], o, 64);
          acc[c][j] = __fmul_rn(acc[c][j], e1) + __fmul_rn(a2, e2);
        }
        ss[c] = __fmul_rn(ss[c], e1) + __fmul_rn(s2, e2);
        mm[c] = mn;
      } else {
#pragma unroll
        for (int j = 0; j < V; ++j) acc[c][j] += __shfl_xor(acc[c][j], o, 64);
      }
      cnt[c] += __shfl_xor(cnt[c], o, 64);
    }
  }

  // lane group c writes cluster c of this wave
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int kk = k0 + wave + 16 * c;
    if (lg != c || kk >= k.K) continue;
    const size_t row = (size_t)h * k.K + kk;
    if constexpr (MERGE) {
      const bool any = ss[c] > 0.f;
      const float inv = any ? 1.f / ss[c] : 0.f;
      uint32_t w[V / 2];
#pragma unroll
      for (int q = 0; q < V / 2; ++q)
        w[q] = f32_to_bf16_rne(acc[c][2 * q] * inv) | (f32_to_bf16_rne(acc[c][2 * q + 1] * inv) << 16);
      uint16_t* dst = k.abar + row * D + lc * V;
      if constexpr (V == 8)
        *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
      else
        *(uint2*)dst = uint2{w[0], w[1]};
      if (lc == 0) k.log_zbar[row] = any ? mm[c] + logf(ss[c]) : kNegInf;
    } else {
      float v[V];
      float* cp = k.cent + row * D + lc * V;
      if (cnt[c] > 0) {
        const float fc = (float)cnt[c];
#pragma unroll
        for (int j = 0; j < V; ++j) v[j] = acc[c][j] / fc;
#pragma unroll
        for (int j = 0; j < V; j += 4) *(f32x4*)(cp + j) = f32x4{v[j], v[j + 1], v[j + 2], v[j + 3]};
      } else {
#pragma unroll
        for (int j = 0; j < V; j += 4) {
          const f32x4 x = *(const f32x4*)(cp + j);
#pragma unroll
          for (int q = 0; q < 4; ++q) v[j + q] = x[q];
        }
      }
      km_prep_row<D>(k, row, v, lc, k.hi_out);
      if (lc == 0 && k.counts) k.counts[row] = cnt[c];
    }
  }
}

static int prefix_chunks(int L, int chunks, int& csize) {
  if (L <= 0) {
    csize = 1;
    return 1;
  }
  csize = (int)(((long long)L + chunks - 1) / chunks);
  return (L + csize - 1) / csize;
}

static bool build_dims_ok(int H, int N, int D) {
  if (H < 1 || N < 1 || N >= kMaxPoints) return false;
  if ((long long)H * N >= (1ll << 30)) return false;
  (void)D;
  return true;
}

// Workspace of the prefix-state computation: V^T per chunk, then (more than one
// chunk) the chunk states and their lse.
static size_t prefix_layout(int H, int N, int D, int L, int chunks, int& C, int& csize, int& Lc,
                            size_t& o_vt, size_t& o_part, size_t& o_plse, size_t* o_rmax = nullptr,
                            size_t* o_sexp = nullptr) {
  C = prefix_chunks(L, chunks, csize);
  Lc = (csize + kPfxKT - 1) / kPfxKT * kPfxKT;
  const size_t rows = (size_t)H * N;
  o_vt = kWsHeader;
  o_part = o_vt + (L > 0 ? align_up((size_t)H * C * D * Lc * 2, 256) : 0);
  o_plse = o_part + (C > 1 ? align_up((size_t)C * rows * D * 4, 256) : 0);
  const size_t rm = o_plse + (C > 1 ? align_up((size_t)C * rows * 4, 256) : 0);
  const size_t se = rm + (L > 0 ? align_up((size_t)H * C * (Lc / kPfxKT) * D * 4, 256) : 0);
  if (o_rmax) *o_rmax = rm;
  if (o_sexp) *o_sexp = se;
  return se + (L > 0 ? align_up((size_t)H * C * D * 4, 256) : 0);
}

static int32_t launch_prefix(const void* q, int32_t H, int32_t N, int32_t D, const void* k,
                             const void* v, int32_t L, int32_t chunks, float scale, float* a,
                             float* lse, void* ws, int32_t* status, hipStream_t s) {
  int C, csize, Lc;
  size_t o_vt, o_part, o_plse, o_rmax, o_sexp;
  prefix_layout(H, N, D, L, chunks, C, csize, Lc, o_vt, o_part, o_plse, &o_rmax, &o_sexp);
  PrefixArgs p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.vt = (uint16_t*)((char*)ws + o_vt);
  p.rmax = (uint32_t*)((char*)ws + o_rmax);
  p.sexp = (int32_t*)((char*)ws + o_sexp);
  p.status = status;
  p.H = H;
  p.N = N;
  p.L = L;
  p.C = C;
  p.csize = csize;
  p.Lc = Lc;
  p.scale_log2 = scale * kLog2e;
  const size_t rows = (size_t)H * N;
  if (C == 1) {
    p.out = a;
    p.out_lse = lse;
  } else {
    p.out = (float*)((char*)ws + o_part);
    p.out_lse = (float*)((char*)ws + o_plse);
  }
  if (L > 0) {
    TraceScope tr(kTrAsmVt, s);
    const dim3 g((unsigned)((size_t)H * C * (Lc / kPfxKT)));
    if (D == 128) {
      hipLaunchKernelGGL(vt_range<128>, g, dim3(256), 0, s, p);
      hipLaunchKernelGGL(vt_prepare<128>, g, dim3(256), 0, s, p);
    } else {
      hipLaunchKernelGGL(vt_range<64>, g, dim3(256), 0, s, p);
      hipLaunchKernelGGL(vt_prepare<64>, g, dim3(256), 0, s, p);
    }
  }
  const dim3 grid(H * ((N + kPfxQB - 1) / kPfxQB), C);
  {
    TraceScope tr(kTrAsmPrefix, s);
    if (D == 128)
      hipLaunchKernelGGL(asm_prefix_chunk<128>, grid, dim3(kPfxQB * 2), 0, s, p);
    else
      hipLaunchKernelGGL(asm_prefix_chunk<64>, grid, dim3(kPfxQB * 2), 0, s, p);
  }
  if (C > 1) {
    TraceScope tr(kTrAsmPrefixMerge, s);
    const dim3 g2((unsigned)((rows + 15) / 16));
    if (D == 128)
      hipLaunchKernelGGL(asm_prefix_merge<128>, g2, dim3(256), 0, s, p.out, p.out_lse, a, lse,
                         (int32_t)rows, C);
    else
      hipLaunchKernelGGL(asm_prefix_merge<64>, g2, dim3(256), 0, s, p.out, p.out_lse, a, lse,
                         (int32_t)rows, C);
  }
  return launch_status();
}

static size_t km_layout(int H, int K, int D, size_t& o_hi, size_t& o_lo, size_t& o_n) {
  const size_t cells = (size_t)H * K * D;
  o_hi = kWsHeader;
  o_lo = o_hi + align_up(cells * 2, 256);
  o_n = o_lo + align_up(cells * 2, 256);
  return o_n + align_up((size_t)H * K * 4, 256);
}

static void km_launch_assign(const KmArgs& k, int D, hipStream_t s) {
  TraceScope tr(kTrKmAssign, s);
  const dim3 g(k.H * ((k.N + kKmPB - 1) / kKmPB));
  if (D == 128)
    hipLaunchKernelGGL(km_assign<128>, g, dim3(256), 0, s, k);
  else
    hipLaunchKernelGGL(km_assign<64>, g, dim3(256), 0, s, k);
}

static void km_launch_reduce(const KmArgs& k, int D, bool merge, hipStream_t s) {
  TraceScope tr(merge ? kTrAsmAggregate : kTrKmUpdate, s);
  const dim3 g(k.H * ((k.K + 63) / 64));
  if (merge) {
    if (D == 128)
      hipLaunchKernelGGL((km_reduce<128, true>), g, dim3(1024), 0, s, k);
    else
      hipLaunchKernelGGL((km_reduce<64, true>), g, dim3(1024), 0, s, k);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((km_reduce<128, false>), g, dim3(1024), 0, s, k);
    else
      hipLaunchKernelGGL((km_reduce<64, false>), g, dim3(1024), 0, s, k);
  }
}

static int32_t launch_kmeans(const void* x, int32_t H, int32_t N, int32_t D, float* cent,
                             int32_t K, int32_t iters, int32_t* assign, int32_t* counts,
                             void* cent_bf16, void* ws, hipStream_t s) {
  size_t o_hi, o_lo, o_n;
  km_layout(H, K, D, o_hi, o_lo, o_n);
  KmArgs k;
  memset(&k, 0, sizeof(k));
  k.x = (const uint16_t*)x;
  k.cent = cent;
  k.hi = (uint16_t*)((char*)ws + o_hi);
  k.lo = (uint16_t*)((char*)ws + o_lo);
  k.cnorm = (float*)((char*)ws + o_n);
  k.assign = assign;
  k.counts = counts;
  k.H = H;
  k.N = N;
  k.K = K;
  k.hi_out = k.hi;
  {
    TraceScope tr(kTrKmUpdate, s);
    const dim3 g((unsigned)(((size_t)H * K + 15) / 16));
    if (D == 128)
      hipLaunchKernelGGL(km_prep<128>, g, dim3(256), 0, s, k);
    else
      hipLaunchKernelGGL(km_prep<64>, g, dim3(256), 0, s, k);
  }
  for (int it = 0; it < iters; ++it) {
    km_launch_assign(k, D, s);
    k.hi_out = (it == iters - 1 && cent_bf16) ? (uint16_t*)cent_bf16 : k.hi;
    km_launch_reduce(k, D, false, s);
  }
  return launch_status();
}

static int32_t launch_aggregate(const int32_t* assign, const float* a, const float* lse,
                                int32_t H, int32_t N, int32_t D, int32_t K, void* abar,
                                float* log_zbar, hipStream_t s) {
  KmArgs k;
  memset(&k, 0, sizeof(k));
  k.assign = (int32_t*)assign;
  k.a = a;
  k.lse = lse;
  k.abar = (uint16_t*)abar;
  k.log_zbar = log_zbar;
  k.H = H;
  k.N = N;
  k.K = K;
  km_launch_reduce(k, D, true, s);
  return launch_status();
}

}  // namespace kvb

using namespace kvb;

extern "C" size_t asm_prefix_states_workspace(int32_t H, int32_t N, int32_t D, int32_t L,
                                              int32_t chunks) {
  if (!build_dims_ok(H, N, D) || L < 0 || L >= (1 << 30) || chunks < 1 || (D != 64 && D != 128))
    return 0;
  int C, csize, Lc;
  size_t a, b, c;
  return prefix_layout(H, N, D, L, chunks, C, csize, Lc, a, b, c);
}

extern "C" int32_t asm_prefix_states(const void* q, int32_t H, int32_t N, int32_t D,
                                     const void* k, const void* v, int32_t L, int32_t chunks,
                                     float scale, float* a, float* lse, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (!q || !a || !lse || (L > 0 && (!k || !v))) return KVB_EINVAL;
  if (!build_dims_ok(H, N, D) || L < 0 || L >= (1 << 30) || chunks < 1 || chunks > 65535)
    return KVB_EINVAL;
  if (D != 64 && D != 128) return KVB_EUNSUPPORTED;
  if ((long long)H * ((N + kPfxQB - 1) / kPfxQB) >= (1ll << 31)) return KVB_EINVAL;
  const size_t need = asm_prefix_states_workspace(H, N, D, L, chunks);
  if (!ws || ws_bytes < need) return KVB_EWORKSPACE;
  int32_t st = check_device();
  if (st) return st;
  if (!(scale > 0.f)) scale = 1.f / sqrtf((float)D);
  return launch_prefix(q, H, N, D, k, v, L, chunks, scale, a, lse, ws, (int32_t*)ws,
                       (hipStream_t)stream);
}

extern "C" size_t asm_kmeans_workspace(int32_t H, int32_t K, int32_t D) {
  if (H < 1 || K < 1 || K >= kMaxPoints || (D != 64 && D != 128)) return 0;
  size_t a, b, c;
  return km_layout(H, K, D, a, b, c);
}

extern "C" int32_t asm_kmeans(const void* x, int32_t H, int32_t N, int32_t D, float* centroids,
                              int32_t K, int32_t iters, int32_t* assign, int32_t* counts,
                              void* centroids_bf16, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !centroids || !assign) return KVB_EINVAL;
  if (!build_dims_ok(H, N, D) || K < 1 || K >= kMaxPoints || iters < 1 || iters > 100000)
    return KVB_EINVAL;
  if ((long long)H * K >= (1ll << 30)) return KVB_EINVAL;
  if (D != 64 && D != 128) return KVB_EUNSUPPORTED;
  const size_t need = asm_kmeans_workspace(H, K, D);
  if (!ws || ws_bytes < need) return KVB_EWORKSPACE;
  int32_t st = check_device();
  if (st) return st;
  return launch_kmeans(x, H, N, D, centroids, K, iters, assign, counts, centroids_bf16, ws,
                       (hipStream_t)stream);
}

extern "C" int32_t asm_aggregate_states(const int32_t* assign, const float* a, const float* lse,
                                        int32_t H, int32_t N, int32_t D, int32_t K, void* abar,
                                        float* log_zbar, void* stream) {
  if (!assign || !a || !lse || !abar || !log_zbar) return KVB_EINVAL;
  if (!build_dims_ok(H, N, D) || K < 1 || K >= kMaxPoints) return KVB_EINVAL;
  if ((long long)H * K >= (1ll << 30)) return KVB_EINVAL;
  if (D != 64 && D != 128) return KVB_EUNSUPPORTED;
  int32_t st = check_device();
  if (st) return st;
  return launch_aggregate(assign, a, lse, H, N, D, K, abar, log_zbar, (hipStream_t)stream);
}

static size_t build_layout(int32_t H, int32_t N, int32_t D, int32_t L, int32_t chunks, int32_t K,
                           size_t& o_a, size_t& o_l, size_t& o_p, size_t& o_k) {
  const size_t rows = (size_t)H * N;
  o_a = kWsHeader;
  o_l = o_a + align_up(rows * D * 4, 256);
  o_p = o_l + align_up(rows * 4, 256);
  o_k = o_p + align_up(asm_prefix_states_workspace(H, N, D, L, chunks), 256);
  return o_k + asm_kmeans_workspace(H, K, D);
}

extern "C" size_t asm_build_memory_workspace(int32_t H, int32_t N, int32_t D, int32_t L,
                                             int32_t chunks, int32_t K) {
  if (!asm_prefix_states_workspace(H, N, D, L, chunks) || !asm_kmeans_workspace(H, K, D))
    return 0;
  size_t a, b, c, d;
  return build_layout(H, N, D, L, chunks, K, a, b, c, d);
}

extern "C" int32_t asm_build_memory(const void* q, int32_t H, int32_t N, int32_t D,
                                    const void* k, const void* v, int32_t L, int32_t chunks,
                                    float scale, float* centroids, int32_t K, int32_t iters,
                                    void* centroids_bf16, void* abar, float* log_zbar,
                                    int32_t* assign, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !centroids || !centroids_bf16 || !abar || !log_zbar || !assign) return KVB_EINVAL;
  if (L > 0 && (!k || !v)) return KVB_EINVAL;
  if (!build_dims_ok(H, N, D) || L < 0 || L >= (1 << 30) || chunks < 1 || chunks > 65535)
    return KVB_EINVAL;
  if (K < 1 || K >= kMaxPoints || (long long)H * K >= (1ll << 30) || iters < 1 || iters > 100000)
    return KVB_EINVAL;
  if (D != 64 && D != 128) return KVB_EUNSUPPORTED;
  const size_t need = asm_build_memory_workspace(H, N, D, L, chunks, K);
  if (!ws || ws_bytes < need) return KVB_EWORKSPACE;
  int32_t st = check_device();
  if (st) return st;
  if (!(scale > 0.f)) scale = 1.f / sqrtf((float)D);
  size_t o_a, o_l, o_p, o_k;
  build_layout(H, N, D, L, chunks, K, o_a, o_l, o_p, o_k);
  char* w = (char*)ws;
  float* a = (float*)(w + o_a);
  float* lse = (float*)(w + o_l);
  hipStream_t s = (hipStream_t)stream;
  st = launch_prefix(q, H, N, D, k, v, L, chunks, scale, a, lse, w + o_p, (int32_t*)w, s);
  if (st) return st;
  st = launch_kmeans(q, H, N, D, centroids, K, iters, assign, nullptr, centroids_bf16, w + o_k, s);
  if (st) return st;
  return launch_aggregate(assign, a, lse, H, N, D, K, abar, log_zbar, s);
}
