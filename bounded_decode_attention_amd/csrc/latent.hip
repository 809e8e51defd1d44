// Latent memory of evicted tokens: decayed outer-product fast weights and the
// gated residual read-out.
//
// "IndexMem: Learned KV-Cache Eviction with Latent Memory for Long-Context LLM
// Inference", technical summary, section 2, part B: each evicted token updates a
// fixed-size state matrix M and a stabiliser vector b online by an outer-product
// accumulation with decay; a projection and a gate g(q) read the memory and the
// attention output becomes o_attn + g(q) m(q).  Per KV head, with phi(x) =
// elu(x) + 1 and evicted tokens taken in slot order, n of them:
//   M <- lam^n M + sum_j lam^(n-1-j) phi(k_j) v_j^T,   b <- lam^n b + sum_j lam^(n-1-j) phi(k_j);
//   r = M^T phi(q) / (b . phi(q) + eps),  m = W_o r,  g = sigmoid(w_g . q + c_g).
//
// Kernels
//   latent_list            per (head, 256 slots): slot s of a head the plan evicts is
//                          evicted iff it is not in the plan's ascending kept list
//                          (binary search); its rank among the evicted slots is s
//                          minus the kept slots below it.
//   latent_absorb_part<D>  per (head, 4096 evicted tokens): rows gathered 64 at a
//                          time (slot indices fetched a tile ahead of the rows);
//                          phi(k) times its decay weight (relative to the chunk end)
//                          is split into two bf16 parts and, with v, transposed 4x8
//                          per thread into LDS as [d][token]; the chunk's
//                          Phi^T V (D x D) accumulates on v_mfma_f32_16x16x32_bf16,
//                          its sum of weighted phi(k) in float32.
//   latent_absorb_combine  per (head, 1024 state elements): lam^n * old plus the
//                          chunk partials scaled by lam^(tokens after the chunk), in
//                          chunk order.
//   latent_read<D>         per (sequence, KV head): for each of the G query heads
//                          r, m, g as above; out += g m.
#include <string.h>

#include "common.h"

namespace kvb {

constexpr int kLatChunk = 4096;  // evicted tokens per partial
constexpr int kLatTile = 64;     // tokens per LDS tile

struct LatentArgs {
  const uint16_t* k;
  const uint16_t* v;
  int32_t cap;
  const UnitInfo* info;
  const int32_t* keep_src;
  int32_t Mk;
  int32_t* ev;       // [U][cap] evicted slots in order
  int32_t* ev_n;     // [U]
  float* part;       // [U][S][D*D + D]
  int32_t S;         // partial slots per head
  float log2_lam;
  float* mem_M;      // [U][D][D]
  float* mem_b;      // [U][D]
};

__global__ __launch_bounds__(256) void latent_list(LatentArgs a) {
  const int u = blockIdx.y;
  const UnitInfo inf = a.info[u];
  const bool ev = inf.mode == MODE_EVICT;
  const int n = ev ? min(inf.n, a.cap) : 0;
  const int kept = ev ? min(inf.kept, a.Mk) : 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.ev_n[u] = n - kept;
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= n) return;
  const int32_t* ks = a.keep_src + (size_t)u * a.Mk;
  int lo = 0, hi = kept;  // first index with ks[idx] >= s
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (ks[mid] < s) lo = mid + 1;
    else hi = mid;
  }
  if (lo < kept && ks[lo] == s) return;
  a.ev[(size_t)u * a.cap + (s - lo)] = s;
}

__device__ __forceinline__ float phi_elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// 16-byte LDS slot holding token chunk c (8 tokens) of row d (rows of 64 tokens).
__device__ __forceinline__ int lat_slot(int d, int c) { return c ^ ((d >> 1) & 7); }

template <int D>
__global__ __launch_bounds__(256) void latent_absorb_part(LatentArgs a) {
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int NT = D / 16;           // 16-wide tiles per dimension
  constexpr int TPW = NT * NT / 4;     // output tiles per wave
  constexpr int RB = kLatTile * 2;     // LDS row bytes (64 tokens, bf16)
  __shared__ __attribute__((aligned(16))) unsigned char ph[D * RB];
  __shared__ __attribute__((aligned(16))) unsigned char pl[D * RB];
  __shared__ __attribute__((aligned(16))) unsigned char vt[D * RB];
  __shared__ float bred[16][D];

  const int u = blockIdx.y, c = blockIdx.x;
  const int ne = a.ev_n[u];
  const int j0 = c * kLatChunk;
  if (j0 >= ne) return;
  const int j1 = min(ne, j0 + kLatChunk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  // each thread: 4 consecutive tokens (quad qd) x one 16-byte chunk ch, of k and of v
  const int qd = tid & 15, ch = tid >> 4;
  const bool act = ch < CPR;
  const int32_t* evl = a.ev + (size_t)u * a.cap;
  const size_t uoff = (size_t)u * a.cap * D + (act ? ch : 0) * 8;

  f32x4 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float bs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) bs[e] = 0.f;

  int idx[4];
  u32x4 kr[4], vr[4];
  auto load_idx = [&](int t0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int jj = t0 + 4 * qd + r;
      // (the clamp only guards the read; every listed slot is below cap)
      idx[r] = (act && jj < j1) ? min(evl[jj], a.cap - 1) : -1;
    }
  };
  auto load_rows = [&]() {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const size_t off = uoff + (size_t)(idx[r] < 0 ? 0 : idx[r]) * D;
      kr[r] = idx[r] >= 0 ? *(const u32x4*)(a.k + off) : u32x4{0, 0, 0, 0};
      vr[r] = idx[r] >= 0 ? *(const u32x4*)(a.v + off) : u32x4{0, 0, 0, 0};
    }
  };

  load_idx(j0);
  load_rows();
  if (j0 + kLatTile < j1) load_idx(j0 + kLatTile);
  for (int t0 = j0; t0 < j1; t0 += kLatTile) {
    __syncthreads();  // the previous tile's operands are consumed
    if (act) {
      float f[4][8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jj = t0 + 4 * qd + r;
        const bool ok = jj < j1;
        const float wt = ok ? exp2_fast((float)(j1 - 1 - jj) * a.log2_lam) : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (kr[r][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          f[r][e] = ok ? wt * phi_elu1(bf16_bits_to_f32(bits)) : 0.f;
          bs[e] += f[r][e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = ch * 8 + e;
        const int off = d * RB + 16 * lat_slot(d, qd >> 1) + 8 * (qd & 1);
        uint32_t wh[2], wl[2], wv[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t h0 = f32_to_bf16_rne(f[2 * q][e]), h1 = f32_to_bf16_rne(f[2 * q + 1][e]);
          const uint32_t l0 = f32_to_bf16_rne(f[2 * q][e] - bf16_bits_to_f32(h0));
          const uint32_t l1 = f32_to_bf16_rne(f[2 * q + 1][e] - bf16_bits_to_f32(h1));
          wh[q] = h0 | (h1 << 16);
          wl[q] = l0 | (l1 << 16);
          const uint32_t x0 = vr[2 * q][e >> 1], x1 = vr[2 * q + 1][e >> 1];
          wv[q] = (e & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (x1 << 16));
        }
        *(uint2*)(ph + off) = uint2{wh[0], wh[1]};
        *(uint2*)(pl + off) = uint2{wl[0], wl[1]};
        *(uint2*)(vt + off) = uint2{wv[0], wv[1]};
      }
    }
    __syncthreads();
    if (t0 + kLatTile < j1) {
      load_rows();                                         // tile t+1 (indices ready)
      if (t0 + 2 * kLatTile < j1) load_idx(t0 + 2 * kLatTile);  // indices of tile t+2
    }
    // Phi^T V: output tile (d1 tile, d2 tile), contraction over this tile's tokens
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tt = wave * TPW + i, dt1 = tt / NT, dt2 = tt % NT;
      const int d1 = dt1 * 16 + lc, d2 = dt2 * 16 + lc;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int cc = 4 * ks + lg;
        const u32x4 ah = *(const u32x4*)(ph + d1 * RB + 16 * lat_slot(d1, cc));
        const u32x4 al = *(const u32x4*)(pl + d1 * RB + 16 * lat_slot(d1, cc));
        const u32x4 bv = *(const u32x4*)(vt + d2 * RB + 16 * lat_slot(d2, cc));
        acc[i] = mfma_16x16x32_bf16(ah, bv, acc[i]);
        acc[i] = mfma_16x16x32_bf16(al, bv, acc[i]);
      }
    }
  }

  float* out = a.part + ((size_t)u * a.S + c) * (D * D + D);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tt = wave * TPW + i, dt1 = tt / NT, dt2 = tt % NT;
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(size_t)(dt1 * 16 + 4 * lg + r) * D + dt2 * 16 + lc] = acc[i][r];
  }
  // weighted phi(k) sums: the 16 quad threads of each chunk, in quad order
  if (act) {
#pragma unroll
    for (int e = 0; e < 8; ++e) bred[qd][ch * 8 + e] = bs[e];
  }
  __syncthreads();
  if (tid < D) {
    float s2 = 0.f;
#pragma unroll
    for (int o = 0; o < 16; ++o) s2 += bred[o][tid];
    out[D * D + tid] = s2;
  }
}

// Final state per (head, 1024 elements of M then b).
__global__ __launch_bounds__(256) void latent_absorb_combine(LatentArgs a, int D) {
  const int u = blockIdx.y;
  const int ne = a.ev_n[u];
  if (ne <= 0) return;
  const int E = D * D + D;
  const int S = (ne + kLatChunk - 1) / kLatChunk;
  const float decay_all = exp2_fast((float)ne * a.log2_lam);
  const float* pu = a.part + (size_t)u * a.S * E;
  for (int e = blockIdx.x * 1024 + threadIdx.x; e < min(E, (int)(blockIdx.x + 1) * 1024);
       e += 256) {
    float* dst = e < D * D ? a.mem_M + (size_t)u * D * D + e : a.mem_b + (size_t)u * D + (e - D * D);
    float acc = decay_all * *dst;
    for (int c = 0; c < S; ++c) {
      const int j1 = min(ne, (c + 1) * kLatChunk);
      acc += exp2_fast((float)(ne - j1) * a.log2_lam) * pu[(size_t)c * E + e];
    }
    *dst = acc;
  }
}

struct LatentReadArgs {
  const uint16_t* q;     // [B][Hq][D]
  const float* mem_M;    // [B*Hkv][D][D]
  const float* mem_b;    // [B*Hkv][D]
  const float* W_o;      // [D][D]
  const float* w_g;      // [Hq][D]
  const float* c_g;      // [Hq]
  float* out;            // [B][Hq][D]
  int32_t Hq, Hkv, G;
  float eps;
};

// One workgroup (4 waves) per (sequence, KV head); wave w reads for query heads
// w, w + 4, ... of the group.  Lanes hold D/64 consecutive elements.
template <int D>
__global__ __launch_bounds__(256) void latent_read(LatentReadArgs a) {
  constexpr int V = D / 64;
  __shared__ float fq[4][D];
  __shared__ float rr[4][D];
  const int u = blockIdx.x;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float* Mu = a.mem_M + (size_t)u * D * D;
  const float* bu = a.mem_b + (size_t)u * D;
  for (int hi = wave; hi < a.G; hi += 4) {
    const int h = g * a.G + hi;
    const uint16_t* qp = a.q + ((size_t)b * a.Hq + h) * D;
    float qv[V], f[V];
    float den = 0.f, gd = 0.f;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      qv[j] = bf16_bits_to_f32(qp[lane * V + j]);
      f[j] = phi_elu1(qv[j]);
      fq[wave][lane * V + j] = f[j];
      den = fmaf(bu[lane * V + j], f[j], den);
      gd = fmaf(a.w_g[(size_t)h * D + lane * V + j], qv[j], gd);
    }
    den = wave_sum(den) + a.eps;
    gd = wave_sum(gd) + a.c_g[h];
    const float gate = 1.f / (1.f + __expf(-gd));
    __builtin_amdgcn_wave_barrier();  // this wave's phi(q) is in LDS
    // r[d2] = sum_d1 M[d1][d2] f[d1] / den
    float r[V];
#pragma unroll
    for (int j = 0; j < V; ++j) r[j] = 0.f;
#pragma unroll 4
    for (int d1 = 0; d1 < D; ++d1) {
      const float fv = fq[wave][d1];
#pragma unroll
      for (int j = 0; j < V; ++j) r[j] = fmaf(Mu[(size_t)d1 * D + lane * V + j], fv, r[j]);
    }
#pragma unroll
    for (int j = 0; j < V; ++j) rr[wave][lane * V + j] = r[j] / den;
    __builtin_amdgcn_wave_barrier();
    // m[d] = sum_e W_o[d][e] r[e]
    float* op = a.out + ((size_t)b * a.Hq + h) * D;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int d = lane * V + j;
      const float* wr = a.W_o + (size_t)d * D;
      float m = 0.f;
#pragma unroll 4
      for (int e = 0; e < D; ++e) m = fmaf(wr[e], rr[wave][e], m);
      op[d] += gate * m;
    }
  }
}

static size_t latent_layout(const kvb_cache* c, int& S, size_t& o_ev, size_t& o_n,
                            size_t& o_part) {
  const size_t U = (size_t)c->B * c->Hkv;
  S = (c->cap + kLatChunk - 1) / kLatChunk;
  o_ev = kWsHeader;
  o_n = o_ev + align_up(U * c->cap * 4, 256);
  o_part = o_n + align_up(U * 4, 256);
  return o_part + align_up(U * S * ((size_t)c->D * c->D + c->D) * 4, 256);
}

}  // namespace kvb

using namespace kvb;

extern "C" size_t kv_latent_absorb_workspace(const kvb_cache* cache) {
  if (!cache || cache->B < 1 || cache->Hkv < 1 || cache->cap < 1 || cache->D < 8) return 0;
  int S;
  size_t a, b, c;
  return latent_layout(cache, S, a, b, c);
}

extern "C" int32_t kv_latent_absorb(const kvb_cache* cache, int32_t M, const void* ws_evict,
                                    size_t ws_evict_bytes, float lam, float* mem_M, float* mem_b,
                                    void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (M < 0 || !mem_M || !mem_b || !ws_evict) return KVB_EINVAL;
  if (!(lam > 0.f && lam <= 1.f)) return KVB_EINVAL;
  if (cache->dtype != KVB_BF16 || (cache->D != 64 && cache->D != 128)) return KVB_EUNSUPPORTED;
  if (ws_evict_bytes < kv_evict_workspace(cache, M)) return KVB_EWORKSPACE;
  int S;
  size_t o_ev, o_n, o_part;
  const size_t need = latent_layout(cache, S, o_ev, o_n, o_part);
  if (!ws || ws_bytes < need) return KVB_EWORKSPACE;
  st = check_device();
  if (st) return st;
  const EvictView e = evict_view(cache, M, ws_evict);
  LatentArgs a;
  memset(&a, 0, sizeof(a));
  a.k = (const uint16_t*)cache->k;
  a.v = (const uint16_t*)cache->v;
  a.cap = cache->cap;
  a.info = e.info;
  a.keep_src = e.keep_src;
  a.Mk = e.Mk;
  char* w = (char*)ws;
  a.ev = (int32_t*)(w + o_ev);
  a.ev_n = (int32_t*)(w + o_n);
  a.part = (float*)(w + o_part);
  a.S = S;
  a.log2_lam = log2f(lam);
  a.mem_M = mem_M;
  a.mem_b = mem_b;
  const int U = cache->B * cache->Hkv;
  hipStream_t s = (hipStream_t)stream;
  TraceScope tr(kTrLatentAbsorb, s);
  hipLaunchKernelGGL(latent_list, dim3((cache->cap + 255) / 256, U), dim3(256), 0, s, a);
  if (cache->D == 128)
    hipLaunchKernelGGL(latent_absorb_part<128>, dim3(S, U), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(latent_absorb_part<64>, dim3(S, U), dim3(256), 0, s, a);
  const int E = cache->D * cache->D + cache->D;
  hipLaunchKernelGGL(latent_absorb_combine, dim3((E + 1023) / 1024, U), dim3(256), 0, s, a,
                     cache->D);
  return launch_status();
}

extern "C" int32_t kv_latent_read(const void* q, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                  const float* mem_M, const float* mem_b, const float* W_o,
                                  const float* w_g, const float* c_g, float eps, float* out,
                                  void* stream) {
  if (!q || !mem_M || !mem_b || !W_o || !w_g || !c_g || !out) return KVB_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || (long long)B * Hkv >= (1 << 24)) return KVB_EINVAL;
  if (!(eps >= 0.f)) return KVB_EINVAL;
  if (D != 64 && D != 128) return KVB_EUNSUPPORTED;
  int32_t st = check_device();
  if (st) return st;
  LatentReadArgs a;
  a.q = (const uint16_t*)q;
  a.mem_M = mem_M;
  a.mem_b = mem_b;
  a.W_o = W_o;
  a.w_g = w_g;
  a.c_g = c_g;
  a.out = out;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.eps = eps;
  hipStream_t s = (hipStream_t)stream;
  TraceScope tr(kTrLatentRead, s);
  if (D == 128)
    hipLaunchKernelGGL(latent_read<128>, dim3(B * Hkv), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(latent_read<64>, dim3(B * Hkv), dim3(256), 0, s, a);
  return launch_status();
}
