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
//                          evicted iff the plan does not keep it; its rank among the
//                          evicted slots is s minus the kept slots below it (from the
//                          plan's per-32-slot keep masks and counts, or a binary
//                          search of its ascending kept list).
//   latent_absorb_part<D>  per (head, 2048 evicted tokens), 8 waves: rows gathered
//                          64 at a time (slot indices fetched a tile ahead of the
//                          rows); phi(k) times its decay weight (relative to the
//                          chunk end) is split into two bf16 parts and, with v,
//                          transposed 2x8 per thread into LDS as [d][token]; the chunk's
//                          Phi^T V (D x D) accumulates on v_mfma_f32_16x16x32_bf16,
//                          its sum of weighted phi(k) in float32.
//   latent_absorb_small<D> per (head with at most 32 evicted tokens, 1024 state
//                          elements): the listed tokens' weighted phi(k) and v staged
//                          in LDS, the state updated directly (float32); the chunk
//                          kernels skip such heads.
//   latent_absorb_combine  per (head, 1024 state elements): lam^n * old plus the
//                          chunk partials scaled by lam^(tokens after the chunk), in
//                          chunk order.
//   latent_read<D>         per (sequence, KV head): for each of the G query heads
//                          r, m, g as above; out += g m.
#include <string.h>

#include "common.h"

namespace kvb {

constexpr int kLatChunk = 2048;  // evicted tokens per partial
constexpr int kLatTile = 64;     // tokens per LDS tile
constexpr int kLatSmall = 32;    // heads with at most this many evicted: direct update

struct LatentArgs {
  const uint16_t* k;
  const uint16_t* v;
  int32_t cap;
  const UnitInfo* info;
  const int32_t* keep_src;
  int32_t Mk;
  const uint32_t* tile_mask;  // [U][Tc] keep bits per 32 slots, or null
  const int32_t* tile_base;   // [U][Tc] kept slots before each tile
  int32_t Tc;
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
  int lo;  // kept slots below s
  if (a.tile_mask) {
    const uint32_t m = a.tile_mask[(size_t)u * a.Tc + (s >> 5)];
    const uint32_t bit = 1u << (s & 31);
    if (m & bit) return;
    lo = a.tile_base[(size_t)u * a.Tc + (s >> 5)] + __popc(m & (bit - 1u));
  } else {
    const int32_t* ks = a.keep_src + (size_t)u * a.Mk;
    int l = 0, h = kept;  // first index with ks[idx] >= s
    while (l < h) {
      const int mid = (l + h) >> 1;
      if (ks[mid] < s) l = mid + 1;
      else h = mid;
    }
    if (l < kept && ks[l] == s) return;
    lo = l;
  }
  const int slot = inf.ostart + s;  // the head's slot (around the end of its slots)
  a.ev[(size_t)u * a.cap + (s - lo)] = slot < a.cap ? slot : slot - a.cap;
}

__device__ __forceinline__ float phi_elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// 16-byte LDS slot holding token chunk c (8 tokens) of row d (rows of 64 tokens).
// The operand reads (rows 16T .. 16T + 15, one chunk) hit 16 distinct (row parity,
// slot) pairs, and the stores (rows e, e + 8, ..., one chunk) all 8 slots, twice.
__device__ __forceinline__ int lat_slot(int d, int c) { return c ^ (((d >> 1) ^ (d >> 4)) & 7); }

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4)))
void latent_absorb_part(LatentArgs a) {
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int NT = D / 16;           // 16-wide tiles per dimension
  constexpr int TPW = NT * NT / 8;     // output tiles per wave (8 waves)
  constexpr int RB = kLatTile * 2;     // LDS row bytes (64 tokens, bf16)
  __shared__ __attribute__((aligned(16))) unsigned char ph[D * RB];
  __shared__ __attribute__((aligned(16))) unsigned char pl[D * RB];
  __shared__ __attribute__((aligned(16))) unsigned char vt[D * RB];

  const int u = blockIdx.y, c = blockIdx.x;
  const int ne = a.ev_n[u];
  const int j0 = c * kLatChunk;
  if (j0 >= ne || ne <= kLatSmall) return;
  const int j1 = min(ne, j0 + kLatChunk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  // each thread: tokens qd and qd + 32 of the tile x one 16-byte chunk ch, of k and
  // of v; consecutive threads take consecutive chunks of a row, so one wave's load
  // reads whole rows.  An LDS word holds tokens (qd, qd + 32) of one dimension: the
  // token order inside a tile is the same for both operands of the product.
  const int ch = tid % CPR, qd = tid / CPR;
  const bool act = qd < 32;  // (all threads for D = 128)
  const int32_t* evl = a.ev + (size_t)u * a.cap;
  const size_t uoff = (size_t)u * a.cap * D + (act ? ch : 0) * 8;

  f32x4 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float bs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) bs[e] = 0.f;

  // two tiles of rows in flight: buffer P = (tile index & 1).  Each step first
  // fetches the slot indices of the tile three ahead, then issues the rows of the
  // tile two ahead from indices fetched one step earlier; loads are unconditional
  // (past the chunk end they repeat its last token, whose weight is zero) and a
  // loaded index is not touched until the next step, so no wait drains the rows
  // in flight.
  int rawi[2][2];
  u32x4 kr[2][2], vr[2][2];
  auto load_idx = [&](int P, int t0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) rawi[P][r] = evl[min(t0 + (act ? qd : 0) + 32 * r, j1 - 1)];
  };
  auto load_rows = [&](int P) {
    if (!act) return;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      // (the clamp only guards the read; every listed slot is below cap)
      const size_t off = uoff + (size_t)min(rawi[P][r], a.cap - 1) * D;
      kr[P][r] = *(const u32x4*)(a.k + off);
      vr[P][r] = *(const u32x4*)(a.v + off);
    }
  };
  auto step = [&](const int P, int t0) {
    barrier_lds();  // the previous tile's operands are consumed (rows stay in flight)
    if (act) {
      float wt[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int jj = t0 + qd + 32 * r;
        wt[r] = jj < j1 ? exp2_fast((float)(j1 - 1 - jj) * a.log2_lam) : 0.f;
      }
      // one dimension at a time: the 2 tokens' weighted phi(k), split, and v (a
      // token past the chunk end has weight 0, so its phi(k) column is 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float f[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const uint32_t bits = (kr[P][r][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          f[r] = wt[r] * phi_elu1(bf16_bits_to_f32(bits));
          bs[e] += f[r];
        }
        const int d = ch * 8 + e;
        const int off = d * RB + 16 * lat_slot(d, qd >> 2) + 4 * (qd & 3);
        uint32_t wh, wl;
        split_bf16x2(f[0], f[1], wh, wl);
        const uint32_t x0 = vr[P][0][e >> 1], x1 = vr[P][1][e >> 1];
        const uint32_t wv = (e & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (x1 << 16));
        *(uint32_t*)(ph + off) = wh;
        *(uint32_t*)(pl + off) = wl;
        *(uint32_t*)(vt + off) = wv;
      }
    }
    barrier_lds();
    load_idx(P ^ 1, t0 + 3 * kLatTile);    // indices of tile t0 + 3T
    load_rows(P);                          // tile t0 + 2T (indices fetched last step)
    // Phi^T V over this tile's tokens: wave output tile tt = wave * TPW + i is
    // (d1 tile tt / NT, d2 tile tt % NT)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int cc = 4 * ks + lg;
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int tt = wave * TPW + i;
        const int d1 = (tt / NT) * 16 + lc, d2 = (tt % NT) * 16 + lc;
        const u32x4 ah = *(const u32x4*)(ph + d1 * RB + 16 * lat_slot(d1, cc));
        const u32x4 al = *(const u32x4*)(pl + d1 * RB + 16 * lat_slot(d1, cc));
        const u32x4 bv = *(const u32x4*)(vt + d2 * RB + 16 * lat_slot(d2, cc));
        acc[i] = mfma_16x16x32_bf16(ah, bv, acc[i]);
        acc[i] = mfma_16x16x32_bf16(al, bv, acc[i]);
      }
    }
  };

  load_idx(0, j0);
  load_rows(0);
  load_idx(1, j0 + kLatTile);
  load_rows(1);
  load_idx(0, j0 + 2 * kLatTile);
  for (int t0 = j0; t0 < j1; t0 += 2 * kLatTile) {
    step(0, t0);
    if (t0 + kLatTile < j1) step(1, t0 + kLatTile);
  }

  float* out = a.part + ((size_t)u * a.S + c) * (D * D + D);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tt = wave * TPW + i, dt1 = tt / NT, dt2 = tt % NT;
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(size_t)(dt1 * 16 + 4 * lg + r) * D + dt2 * 16 + lc] = acc[i][r];
  }
  // weighted phi(k) sums: the 32 pair threads of each chunk, in pair order (the
  // reduction reuses the first operand buffer once every wave is past its reads)
  float(*bred)[D] = (float(*)[D])ph;
  __syncthreads();
  if (act) {
#pragma unroll
    for (int e = 0; e < 8; ++e) bred[qd][ch * 8 + e] = bs[e];
  }
  __syncthreads();
  if (tid < D) {
    float s2 = 0.f;
#pragma unroll
    for (int o = 0; o < 32; ++o) s2 += bred[o][tid];
    out[D * D + tid] = s2;
  }
}

// Heads with 1..kLatSmall evicted tokens: the listed evicted slots' weighted phi(k)
// and v are staged in LDS (float32) and this block's state elements are updated in
// place, summing the tokens in order.
template <int D>
__global__ __launch_bounds__(256) void latent_absorb_small(LatentArgs a) {
  __shared__ int evs[kLatSmall];
  __shared__ float fk[kLatSmall][D];
  __shared__ float fv[kLatSmall][D];
  const int u = blockIdx.y;
  const UnitInfo inf = a.info[u];
  if (inf.mode != MODE_EVICT) return;
  const int n = min(inf.n, a.cap), kept = min(inf.kept, a.Mk);
  const int ne = n - kept;
  if (ne <= 0 || ne > kLatSmall) return;
  const int tid = threadIdx.x;
  if (tid < ne) evs[tid] = min(a.ev[(size_t)u * a.cap + tid], a.cap - 1);
  __syncthreads();
  for (int e = tid; e < ne * D; e += 256) {
    const int j = e / D, d = e - j * D;
    const size_t row = ((size_t)u * a.cap + evs[j]) * D + d;
    const float wt = exp2_fast((float)(ne - 1 - j) * a.log2_lam);
    fk[j][d] = wt * phi_elu1(bf16_bits_to_f32(a.k[row]));
    fv[j][d] = bf16_bits_to_f32(a.v[row]);
  }
  __syncthreads();
  // this block's 1024 elements of (M, b), four per thread, loads first
  const float decay_all = exp2_fast((float)ne * a.log2_lam);
  const int E = D * D + D;
  float old[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = blockIdx.x * 1024 + r * 256 + tid;
    old[r] = e < D * D ? a.mem_M[(size_t)u * D * D + e]
                       : (e < E ? a.mem_b[(size_t)u * D + (e - D * D)] : 0.f);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = blockIdx.x * 1024 + r * 256 + tid;
    if (e >= E) continue;
    float acc = decay_all * old[r];
    if (e < D * D) {
      const int d1 = e / D, d2 = e - d1 * D;
      for (int j = 0; j < ne; ++j) acc = fmaf(fk[j][d1], fv[j][d2], acc);
      a.mem_M[(size_t)u * D * D + e] = acc;
    } else {
      for (int j = 0; j < ne; ++j) acc += fk[j][e - D * D];
      a.mem_b[(size_t)u * D + (e - D * D)] = acc;
    }
  }
}

// Final state per (head, 1024 elements of M then b).
__global__ __launch_bounds__(256) void latent_absorb_combine(LatentArgs a, int D) {
  const int u = blockIdx.y;
  const int ne = a.ev_n[u];
  if (ne <= kLatSmall) return;
  const int E = D * D + D;
  const int S = (ne + kLatChunk - 1) / kLatChunk;
  const float decay_all = exp2_fast((float)ne * a.log2_lam);
  const float* pu = a.part + (size_t)u * a.S * E;
  for (int e = blockIdx.x * 1024 + threadIdx.x; e < min(E, (int)(blockIdx.x + 1) * 1024);
       e += 256) {
    float* dst = e < D * D ? a.mem_M + (size_t)u * D * D + e : a.mem_b + (size_t)u * D + (e - D * D);
    float acc = decay_all * *dst;
    for (int c0 = 0; c0 < S; c0 += 8) {
      float x[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = c0 + q < S ? pu[(size_t)(c0 + q) * E + e] : 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (c0 + q >= S) break;
        const int j1 = min(ne, (c0 + q + 1) * kLatChunk);
        acc += exp2_fast((float)(ne - j1) * a.log2_lam) * x[q];
      }
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
  if (!cache_dims_ok(cache) || cache->D < 8) return 0;
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
  a.tile_mask = e.tile_mask;
  a.tile_base = e.tile_base;
  a.Tc = e.Tc;
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
    hipLaunchKernelGGL(latent_absorb_small<128>, dim3((128 * 128 + 128 + 1023) / 1024, U),
                       dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(latent_absorb_small<64>, dim3((64 * 64 + 64 + 1023) / 1024, U), dim3(256),
                       0, s, a);
  if (cache->D == 128)
    hipLaunchKernelGGL(latent_absorb_part<128>, dim3(S, U), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(latent_absorb_part<64>, dim3(S, U), dim3(512), 0, s, a);
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
