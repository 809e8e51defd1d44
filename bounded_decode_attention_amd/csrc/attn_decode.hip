// Decode-step GQA attention with the retention bias, split over the KV axis.
//
// Logit of token i for a decode query at position t ("Cache What Lasts", section
// 2.1, retention-gated attention):  s_i = scale * q.k_i + (t - pos_i) * log beta_i.
// Each split emits an attention state (a, m, Z) and the states are combined with
// the merge operator of "Context Memorization for Efficient Long Context
// Generation" (method step 2; online-softmax identity in its background section).
//
// Kernels
//   kv_append          one new token per KV head at slot len; len += 1.
//   attn_split_mfma    bf16, D in {64,128}, group G in {1,2,4,8}: one wave per
//                      (KV head, split).  QK^T and PV run on v_mfma_f32_16x16x32_bf16.
//   attn_split_generic any dtype / D <= 256 / G <= 16; one wave per split, one
//                      token at a time (used for float32 caches and odd shapes).
//   attn_merge         merge of the splits' states, in split order.
//
// MFMA tile layout (32 tokens per iteration, one wave).  The 16 MFMA columns hold
// the G query heads (columns 0..G-1) and the same G heads again (G..2G-1); the
// second copy carries the low-order bf16 part of the probabilities in PV, so
// P ~= P_hi + P_lo is applied with ~16 significant bits while V stays bf16.
//   QK^T: A = K rows (lane l: token row l%16, dims 8*(l/16) + 32*kk .. +8), read
//         straight from HBM (each instruction covers 16 rows x 64 contiguous B);
//         B = q columns.  Output lane (g=l/16, c=l%16) holds S[token 4g+r][head c].
//   PV:   O^T[dim][col] += V^T[dim][token] * P^T[token][col].  P^T is consumed in
//         place: lane (g, c) already holds column c's probabilities of tokens
//         {4g..4g+3, 16+4g..16+4g+3}, which become its 8 k-slots.  V^T is read from
//         an LDS copy of the V tile (written with coalesced 16-byte stores); LDS rows
//         are permuted and padded so that the four lane groups read four disjoint
//         32-byte bank groups.
#include <string.h>

#include <mutex>

#include "common.h"
#include "asm_scan.h"

namespace kvb {

struct AttnArgs {
  const void* k;
  const void* v;
  const float* log_beta;
  const int32_t* pos;
  const int32_t* len;
  const int32_t* start;  // [U] first live slot per head, or null (0)
  const void* q;
  const int32_t* t;
  float* part_a;   // [B][Hq][P][D]
  float* part_ml;  // [B][Hq][P][2]  (m, Z)
  int32_t B, Hkv, cap, D, Hq, G, P;
  float scale_log2;  // scale * log2(e)
  // tile range of this launch and its first split index (pipelined kernel): splits
  // p_off .. p_off + gridDim.x - 1 take tiles tile_lo, tile_lo + 1, ... round robin
  int32_t tile_lo, tile_hi, p_off;
  // fused compaction (MOVE launches only)
  FusedPlan plan;
  void* kw;  // K, V written through these (the same buffers as k, v)
  void* vw;
  float* lbw;
  int32_t* posw;
  // when non-null, the first split of each head records the head's len here (the
  // merge then appends the decode token and needs the length before it)
  int32_t* n_rec;
  // when non-null, the call's workspace status word: the first workgroup resets it
  // to KVB_OK (the merge, a later launch of the same call, may set an error)
  int32_t* status = nullptr;
  // one-eviction candidates (kv_attn_decode_plan_one): [U][P] per split; null: none
  OneCand* cand = nullptr;
  // paged cache (kv_attn_decode_paged): page table, fills, pages in use per head,
  // the caller's free pages for the decode token
  const int32_t* pg_table = nullptr;
  const int32_t* pg_fill = nullptr;
  const int32_t* pg_n = nullptr;
  const int32_t* pg_spare = nullptr;
  int32_t pg_max = 0;
};

// ------------------------------------------------------------------ append
// Resets a call's workspace status word (a store, not a memset node, so the call
// can be captured in a graph); the append kernel then reports full heads in it.
__global__ __launch_bounds__(64) void status_reset(int32_t* status) {
  if (threadIdx.x == 0) status[0] = KVB_OK;
}

__global__ __launch_bounds__(64) void kv_append(void* k, void* v, float* log_beta, int32_t* pos,
                                                int32_t* len, const int32_t* start, int32_t cap,
                                                int32_t row_words, const void* k_new,
                                                const void* v_new, const float* lb_new,
                                                const int32_t* t, int32_t Hkv, int32_t* status) {
  const int u = blockIdx.x;
  const int s0 = head_start(start, u);
  const int n = len[u];
  if (n >= cap) {
    if (threadIdx.x == 0) status[0] = KVB_ECAPACITY;
    return;
  }
  const int s = s0 + n < cap ? s0 + n : s0 + n - cap;  // slot of the new token
  const size_t dst = ((size_t)u * cap + s) * row_words;
  const uint32_t* kn = (const uint32_t*)k_new + (size_t)u * row_words;
  const uint32_t* vn = (const uint32_t*)v_new + (size_t)u * row_words;
  for (int w = threadIdx.x; w < row_words; w += 64) {
    ((uint32_t*)k)[dst + w] = kn[w];
    ((uint32_t*)v)[dst + w] = vn[w];
  }
  if (threadIdx.x == 0) {
    pos[(size_t)u * cap + s] = t[u / Hkv];
    if (log_beta) log_beta[(size_t)u * cap + s] = lb_new[u];
  }
  __syncthreads();
  if (threadIdx.x == 0) len[u] = n + 1;
}

// Token range of split p of a head with n live tokens: whole 32-token tiles,
// spread as evenly as possible over the P splits.
__device__ __forceinline__ void split_range(int n, int p, int P, int& lo, int& hi) {
  const int tiles = (n + 31) >> 5;
  const int t0 = (int)(((long long)tiles * p) / P);
  const int t1 = (int)(((long long)tiles * (p + 1)) / P);
  lo = t0 * 32;
  hi = min(t1 * 32, n);
}

// LDS row of tile token tt (0..31): transposes (tt/4)%4 with tt%4 so that the
// tokens one PV k-slot reads across the four lane groups sit in adjacent rows.
__device__ __forceinline__ int lds_row(int tt) {
  return ((tt >> 2) & 3) + ((tt & 3) << 2) + (tt & 16);
}

// ------------------------------------------------------------------ MFMA split
template <int D, int G>
__global__ __launch_bounds__(64) void attn_split_mfma(AttnArgs a) {
  constexpr int KK = D / 32;     // QK k-steps
  constexpr int NB = D / 16;     // PV output dim blocks
  constexpr int CH = D / 8;      // 16-byte chunks per row
  constexpr int RPI = 64 / CH;   // rows per V load instruction
  constexpr int NV = 32 / RPI;   // V load instructions per tile
  constexpr int RS = 2 * D + 32; // LDS row stride (bytes)
  static_assert(2 * G <= 16, "group too large for the hi/lo column split");

  __shared__ __attribute__((aligned(16))) unsigned char vtile[32 * RS];

  const int u = blockIdx.y;
  const int p = blockIdx.x;
  const int b = u / a.Hkv;
  const int g = u - b * a.Hkv;
  const int lane = threadIdx.x;
  const int lg = lane >> 4;
  const int lc = lane & 15;

  const int s0 = head_start(a.start, u);
  const int n = min(a.len[u], a.cap);
  if (a.n_rec && blockIdx.x == 0 && threadIdx.x == 0) a.n_rec[u] = a.len[u];
  if (a.status && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.status[0] = KVB_OK;
  int lo, end;
  split_range(n, p, a.P, lo, end);
  // 16-byte loads of log beta / pos need a 4-slot aligned head base
  const size_t row0 = (size_t)u * a.cap + s0;  // the head's first live slot
  const bool vec_ok = (row0 & 3) == 0;
  // rows at or past capu continue at the start of the head's slots
  const int capu = a.cap - s0;
  auto wr = [&](int r) { return r < capu ? r : r - a.cap; };

  // q as the B operand: column lc is head lc (lc < G), head lc-G (G <= lc < 2G), or 0.
  const int hcol = lc < G ? lc : (lc < 2 * G ? lc - G : -1);
  u32x4 qv[KK];
  {
    const uint16_t* qp =
        (const uint16_t*)a.q + ((size_t)(b * a.Hq + g * G + (hcol < 0 ? 0 : hcol))) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qv[kk] = hcol >= 0 ? *(const u32x4*)(qp + 32 * kk + 8 * lg) : z;
    }
  }

  const uint16_t* kb = (const uint16_t*)a.k + row0 * D;
  const uint16_t* vb = (const uint16_t*)a.v + row0 * D;
  const float* lbb = a.log_beta ? a.log_beta + row0 : nullptr;
  const int32_t* pb = a.pos + row0;
  const int qpos = a.t[b];
  const float sc = a.scale_log2;

  float m2 = kNegInf;  // running max of this column's logits (log2 units)
  float lsum = 0.f;    // this lane's share of Z (its 8 tokens per tile)
  f32x4 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int tb = lo; tb < end; tb += 32) {
    const bool full = tb + 32 <= end;
    const int last = end - 1;

    // ---- global loads: K (MFMA A layout), V (coalesced rows), bias inputs
    u32x4 kr[2][KK];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int row = tb + 16 * j + lc;
      if (!full) row = min(row, last);
      row = wr(row);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kr[j][kk] = *(const u32x4*)(kb + (ptrdiff_t)row * D + 32 * kk + 8 * lg);
    }
    u32x4 vr[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int row = tb + RPI * i + lane / CH;
      if (!full) row = min(row, last);
      row = wr(row);
      vr[i] = *(const u32x4*)(vb + (ptrdiff_t)row * D + 8 * (lane % CH));
    }
    float lbv[2][4];
    int pv[2][4];
    if (lbb) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r0 = tb + 16 * j + 4 * lg;
        if (full && vec_ok && r0 + 4 <= capu) {
          const f32x4 l4 = *(const f32x4*)(lbb + r0);
          const i32x4 p4 = *(const i32x4*)(pb + r0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            lbv[j][r] = l4[r];
            pv[j][r] = p4[r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = wr(min(r0 + r, last));
            lbv[j][r] = lbb[row];
            pv[j][r] = pb[row];
          }
        }
      }
    }

    // ---- V tile to LDS (row-permuted)
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int tt = RPI * i + lane / CH;
      *(u32x4*)(vtile + lds_row(tt) * RS + 16 * (lane % CH)) = vr[i];
    }

    // ---- S = K q^T on MFMA
    f32x4 S[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      S[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) S[j] = mfma_16x16x32_bf16(kr[j][kk], qv[kk], S[j]);
    }

    // ---- logits (log2 units), online max
    float s[2][4];
    float mt = kNegInf;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = tb + 16 * j + 4 * lg + r;
        float bias = 0.f;
        if (lbb) {
          const int d = qpos - pv[j][r];
          bias = d != 0 ? (float)d * lbv[j][r] : 0.f;
        }
        float x = fmaf(S[j][r], sc, bias * kLog2e);
        if (tok >= end) x = kNegInf;
        s[j][r] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    if (mt > m2) {
      const float alpha = (m2 == kNegInf) ? 0.f : exp2_fast(m2 - mt);
#pragma unroll
      for (int i = 0; i < NB; ++i) acc[i] *= alpha;
      lsum *= alpha;
      m2 = mt;
    }
    const float mref = (m2 == kNegInf) ? 0.f : m2;

    // ---- probabilities -> bf16 hi (columns < G) / lo (columns G..2G-1) B operand
    uint32_t pw[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t h[2];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int e = 2 * e2 + w;
        const float x = exp2_fast((e < 4 ? s[0][e] : s[1][e - 4]) - mref);
        lsum += x;
        const uint32_t xb = __float_as_uint(x);
        const uint32_t hi = xb >> 16;
        const uint32_t lo16 = f32_to_bf16_rne(x - __uint_as_float(xb & 0xFFFF0000u));
        h[w] = lc < G ? hi : lo16;
      }
      pw[e2] = h[0] | (h[1] << 16);
    }
    const u32x4 pb4 = {pw[0], pw[1], pw[2], pw[3]};

    // ---- O^T += V^T P^T on MFMA; V^T gathered from LDS
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const unsigned char* col = vtile + 2 * (16 * nb + lc);
      uint32_t vw[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int e0 = 2 * e2, e1 = 2 * e2 + 1;
        const int t0 = e0 < 4 ? 4 * lg + e0 : 16 + 4 * lg + e0 - 4;
        const int t1 = e1 < 4 ? 4 * lg + e1 : 16 + 4 * lg + e1 - 4;
        const uint32_t v0 = *(const uint16_t*)(col + lds_row(t0) * RS);
        const uint32_t v1 = *(const uint16_t*)(col + lds_row(t1) * RS);
        vw[e2] = v0 | (v1 << 16);
      }
      const u32x4 va = {vw[0], vw[1], vw[2], vw[3]};
      acc[nb] = mfma_16x16x32_bf16(va, pb4, acc[nb]);
    }
  }

  // ---- epilogue: Z over the four lane groups; hi + lo columns; normalise; store
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  // lane (g, c < G) adds the low-part column c + G held by lane + G; the shuffles
  // run with every lane active (ds_bpermute only reads active lanes)
  const int src = lane + G < 64 ? lane + G : lane;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[nb][i] = (acc[nb][i] + __shfl(acc[nb][i], src, 64)) * inv;
  if (lc < G) {
    const int h = g * G + lc;
    const size_t sidx = ((size_t)(b * a.Hq + h)) * a.P + p;
    float* pa = a.part_a + sidx * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) *(f32x4*)(pa + 16 * nb + 4 * lg) = acc[nb];
    if (lg == 0) {
      a.part_ml[2 * sidx] = m2 == kNegInf ? kNegInf : m2 * kLn2;
      a.part_ml[2 * sidx + 1] = lsum;
    }
  }
}

// ------------------------------------------------------------------ pipelined split (D = 128)
// Same math and MFMA layout as attn_split_mfma, in a two-stage pipeline: while
// tile i is computed, tile i+1's K rows are in flight into a second register set
// and its V rows into a second LDS buffer.  V goes HBM -> LDS directly
// (global_load_lds_dwordx4: lane l of DMA instruction i lands at byte 16*l of that
// instruction's 1 KB block), so it needs no VGPRs and no ds_write.  Instruction i
// carries tile rows 4i..4i+3 and its block starts at i*1056 bytes: the 32-byte
// pad puts the four lane groups of every transposed read in disjoint bank groups.
// The two buffers are distinct arrays and the loop is unrolled by two.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kVBlk = 1056;  // bytes per V DMA instruction block (1 KB + pad)
// Cache-policy operand of the V transfers: the non-temporal (streaming) hint.  Each
// V row is read once per launch; marking the stream non-temporal took the 32K
// layer from 372 to 331 us (5.9 -> 6.6 TB/s) with bit-identical results.  The same
// hint on the K register loads helped less with it than without it, so K loads
// stay plain.
constexpr int kNonTemporal = 2;

struct KTile {
  u32x4 k[2][4];
  float lb[2][4];
  int ps[2][4];
  uint32_t mk;  // fused compaction: the tile's keep mask and first destination
  int bs;
};

// Issues every load of one tile with no branches.  Rows past the split end are
// clamped to its last row (cache hits); with VEC (capacity % 4 == 0, heads at slot 0)
// log beta and pos are read four at a time from base min(r0, cap - 4), which equals
// r0 for every slot below cap.  Rows are relative to the head's first live slot;
// row r lies at r - cap from it once r reaches capu = cap - first slot (the head
// continues at the start of its slots).
template <bool VEC, bool MOVE>
__device__ __forceinline__ void issue_tile128(const uint16_t* kb, const uint16_t* vb,
                                              const float* lbb, const int32_t* pb, int tb,
                                              int end, int capu, int cap, int lane, KTile& t,
                                              lds_u8* __restrict__ vlds, const uint32_t* tmask,
                                              const int32_t* tbase) {
  const int lg = lane >> 4, lc = lane & 15;
  const int last = end - 1;
  auto wr = [&](int r) { return r < capu ? r : r - cap; };
  if constexpr (MOVE) {
    // with the tile's own loads, so the move step adds no wait of its own
    const int tl = min(tb, last) >> 5;
    t.mk = tmask[tl];
    t.bs = tbase[tl];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = wr(min(tb + 16 * j + lc, last));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      t.k[j][kk] = *(const u32x4*)(kb + (ptrdiff_t)row * 128 + 32 * kk + 8 * lg);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = wr(min(tb + 4 * i + lg, last));
    __builtin_amdgcn_global_load_lds((glb_void_t*)(vb + (ptrdiff_t)row * 128 + 8 * lc),
                                     (lds_void_t*)(vlds + i * kVBlk), 16, 0, kNonTemporal);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r0 = tb + 16 * j + 4 * lg;
    if constexpr (VEC) {
      const int rb = min(r0, capu - 4);
      const f32x4 l4 = __builtin_nontemporal_load((const f32x4*)(lbb + rb));
      const i32x4 p4 = __builtin_nontemporal_load((const i32x4*)(pb + rb));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        t.lb[j][r] = l4[r];
        t.ps[j][r] = p4[r];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wr(min(r0 + r, last));
        t.lb[j][r] = lbb[row];
        t.ps[j][r] = pb[row];
      }
    }
  }
}

template <int G>
__device__ __forceinline__ void compute_tile128(const KTile& t, const lds_u8* __restrict__ vlds, int tb,
                                                int end, int lane, const u32x4* qv, float sc,
                                                int qpos, bool has_lb, float& m2, float& lsum,
                                                f32x4* acc) {
  const int lg = lane >> 4, lc = lane & 15;
  f32x4 S[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    S[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) S[j] = mfma_16x16x32_bf16(t.k[j][kk], qv[kk], S[j]);
  }
  float s[2][4];
  float mt = kNegInf;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = tb + 16 * j + 4 * lg + r;
      float bias = 0.f;
      if (has_lb) {
        const int d = qpos - t.ps[j][r];
        bias = d != 0 ? (float)d * t.lb[j][r] : 0.f;
      }
      float x = fmaf(S[j][r], sc, bias * kLog2e);
      if (tok >= end) x = kNegInf;
      s[j][r] = x;
      mt = fmaxf(mt, x);
    }
  }
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  if (mt > m2) {
    const float alpha = (m2 == kNegInf) ? 0.f : exp2_fast(m2 - mt);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= alpha;
    lsum *= alpha;
    m2 = mt;
  }
  const float mref = (m2 == kNegInf) ? 0.f : m2;
  uint32_t pw[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    uint32_t h[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int e = 2 * e2 + w;
      const float x = exp2_fast((e < 4 ? s[0][e] : s[1][e - 4]) - mref);
      lsum += x;
      const uint32_t xb = __float_as_uint(x);
      const uint32_t hi = xb >> 16;
      const uint32_t lo16 = f32_to_bf16_rne(x - __uint_as_float(xb & 0xFFFF0000u));
      h[w] = lc < G ? hi : lo16;
    }
    pw[e2] = h[0] | (h[1] << 16);
  }
  const u32x4 pb4 = {pw[0], pw[1], pw[2], pw[3]};
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const lds_u8* col = vlds + 2 * (16 * nb + lc);
    uint32_t vw[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const int e0 = 2 * e2, e1 = 2 * e2 + 1;
      const int t0 = e0 < 4 ? 4 * lg + e0 : 16 + 4 * lg + e0 - 4;
      const int t1 = e1 < 4 ? 4 * lg + e1 : 16 + 4 * lg + e1 - 4;
      typedef __attribute__((address_space(3))) const uint16_t lds_u16;
      const uint32_t v0 = *(lds_u16*)(col + (t0 >> 2) * kVBlk + (t0 & 3) * 256);
      const uint32_t v1 = *(lds_u16*)(col + (t1 >> 2) * kVBlk + (t1 & 3) * 256);
      vw[e2] = v0 | (v1 << 16);
    }
    const u32x4 va = {vw[0], vw[1], vw[2], vw[3]};
    acc[nb] = mfma_16x16x32_bf16(va, pb4, acc[nb]);
  }
}

// One-eviction candidate over one tile: the lowest (retention key, position) among
// the tile's rows below `end` that this lane's group holds (rows 16j + 4g + r), with
// its row.  The key (t - pos) * log beta is formed exactly in double (a < 2^30
// integer times a float), 0 at distance 0 or without a retention array; -0 compares
// equal to +0.
template <bool LB>
__device__ __forceinline__ void sel_tile128(const KTile& t, int tb, int end, int lane, int qpos,
                                            double& bk, int& bp, int& bs) {
  const int lg = lane >> 4;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = tb + 16 * j + 4 * lg + r;
      const int ps = t.ps[j][r];
      const int d = qpos - ps;
      const double key = (LB && d != 0) ? (double)d * (double)t.lb[j][r] : 0.0;
      if (tok < end && (key < bk || (key == bk && ps < bp))) {
        bk = key;
        bp = ps;
        bs = tok;
      }
    }
  }
}

// Writes the kept rows of one tile to their compacted slots: K from the registers
// the QK MFMA read (lane (g, c): row 16j + c, dims 32kk + 8g), V from the tile's LDS
// block (lane l of block i: row 4i + l/16, 16-byte chunk l%16), log beta and pos
// from the bias registers (lanes with c == 0: rows 16j + 4g + r).  Destination of
// tile row r: base + number of kept rows of the tile before r.
template <bool LB>
__device__ __forceinline__ void move_tile128(const KTile& t, const lds_u8* __restrict__ vlds,
                                             uint32_t mask, int base, int lane, uint16_t* kw,
                                             uint16_t* vw, float* lbw, int32_t* pw) {
  const int lg = lane >> 4, lc = lane & 15;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * j + lc;
    if ((mask >> r) & 1u) {
      const int dst = base + __popc(mask & ((1u << r) - 1u));
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) *(u32x4*)(kw + (size_t)dst * 128 + 32 * kk + 8 * lg) = t.k[j][kk];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + lg;
    if ((mask >> r) & 1u) {
      const int dst = base + __popc(mask & ((1u << r) - 1u));
      typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
      *(u32x4*)(vw + (size_t)dst * 128 + 8 * lc) = *(lds_u32x4*)(vlds + i * kVBlk + 16 * lane);
    }
  }
  if (lc == 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = 16 * j + 4 * lg + rr;
        if ((mask >> r) & 1u) {
          const int dst = base + __popc(mask & ((1u << r) - 1u));
          if (LB) lbw[dst] = t.lb[j][rr];
          pw[dst] = t.ps[j][rr];
        }
      }
  }
}

// One split (p, head u) of the pipelined kernel; the launch has gridDim.x splits per
// head.  A device function so that a launch can also carry other work (the ASM
// candidate scan of kv_attn_decode_asm) in workgroups of its own.
template <int G, bool LB, bool VEC, bool MOVE, bool SEL = false>
__device__ __forceinline__ void pipe128_split(const AttnArgs& a, const int p, const int u) {
  static_assert(2 * G <= 16, "group too large for the hi/lo column split");
  __shared__ __attribute__((aligned(16))) unsigned char vbufA_[8 * kVBlk];
  __shared__ __attribute__((aligned(16))) unsigned char vbufB_[8 * kVBlk];
  lds_u8* vbufA = (lds_u8*)vbufA_;
  lds_u8* vbufB = (lds_u8*)vbufB_;
  const int b = u / a.Hkv;
  const int g = u - b * a.Hkv;
  const int lane = threadIdx.x;
  const int lg = lane >> 4;
  const int lc = lane & 15;
  const int s0 = head_start(a.start, u);
  const int capu = a.cap - s0;  // rows before the head wraps to the start of its slots
  const int n = min(a.len[u], a.cap);
  if (a.n_rec && p == 0 && threadIdx.x == 0) a.n_rec[u] = a.len[u];
  if (a.status && p == 0 && u == 0 && threadIdx.x == 0) a.status[0] = KVB_OK;
  const int end = n;
  const size_t row0 = (size_t)u * a.cap + s0;  // the head's first live slot

  const int hcol = lc < G ? lc : (lc < 2 * G ? lc - G : -1);
  u32x4 qv[4];
  {
    const uint16_t* qp =
        (const uint16_t*)a.q + ((size_t)(b * a.Hq + g * G + (hcol < 0 ? 0 : hcol))) * 128;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qv[kk] = hcol >= 0 ? *(const u32x4*)(qp + 32 * kk + 8 * lg) : z;
    }
  }
  const uint16_t* kb = (const uint16_t*)a.k + row0 * 128;
  const uint16_t* vb = (const uint16_t*)a.v + row0 * 128;
  // without a retention array the bias loads read pos twice (harmless, unused)
  const int32_t* pb = a.pos + row0;
  const float* lbb = LB ? a.log_beta + row0 : (const float*)pb;
  const int qpos = a.t[b];
  const float sc = a.scale_log2;

  float m2 = kNegInf, lsum = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one-eviction candidate of this split (SEL)
  double bk = __builtin_huge_val();
  int bp = 0x7FFFFFFF, bs = 0x7FFFFFFF;

  // Tiles in pairs (A, B) with one loop exit, so each register set keeps its
  // registers.
  KTile tA, tB;
  // Split p takes tiles lo + p, lo + p + P, ... of the head (round-robin), so the
  // waves of one head read neighbouring tiles at the same time.
  const int Pl = gridDim.x;
  const int T = min((n + 31) >> 5, a.tile_hi);
  const int t_first = a.tile_lo + p;
  const int ntiles = t_first < T ? (T - t_first + Pl - 1) / Pl : 0;
  const int step = 32 * Pl;
  // fused compaction: this head's plan
  bool mv = false;
  const uint32_t* tmask = nullptr;
  const int32_t* tbase = nullptr;
  uint16_t* kw = nullptr;
  uint16_t* vw = nullptr;
  float* lbw = nullptr;
  int32_t* pw = nullptr;
  if (MOVE) {
    mv = a.plan.info[u].mode == MODE_EVICT;
    tmask = a.plan.tile_mask + (size_t)u * a.plan.Tc;
    tbase = a.plan.tile_base + (size_t)u * a.plan.Tc;
    kw = (uint16_t*)a.kw + row0 * 128;
    vw = (uint16_t*)a.vw + row0 * 128;
    lbw = LB ? a.lbw + row0 : nullptr;
    pw = a.posw + row0;
  }
  auto moves = [&](const KTile& tt, const lds_u8* __restrict__ vl) {
    if (MOVE && mv) {
      // tile-uniform values: keep them in scalar registers
      const uint32_t m = __builtin_amdgcn_readfirstlane(tt.mk);
      if (m) move_tile128<LB>(tt, vl, m, __builtin_amdgcn_readfirstlane(tt.bs), lane, kw, vw, lbw, pw);
    }
  };
  if (ntiles > 0) {
    // Per tile: wait for its loads (the only ones outstanding), write its kept rows,
    // issue the next tile's loads into the other register set and LDS buffer, then
    // compute from this tile's registers and buffer while those loads are in
    // flight.  The wait is explicit: the compiler does not order LDS reads after
    // global_load_lds transfers into the same LDS.  The scheduling barriers keep
    // the next tile's arithmetic from being hoisted above its wait.
    int tb = 32 * t_first;
    issue_tile128<VEC, MOVE>(kb, vb, lbb, pb, tb, end, capu, a.cap, lane, tA, vbufA, tmask, tbase);
    for (int k = 0; k < (ntiles >> 1); ++k) {
      wait_vmem_all();
      moves(tA, vbufA);
      issue_tile128<VEC, MOVE>(kb, vb, lbb, pb, tb + step, end, capu, a.cap, lane, tB, vbufB, tmask, tbase);
      compute_tile128<G>(tA, vbufA, tb, end, lane, qv, sc, qpos, LB, m2, lsum, acc);
      if (SEL) sel_tile128<LB>(tA, tb, end, lane, qpos, bk, bp, bs);
      wait_vmem_all();
      moves(tB, vbufB);
      issue_tile128<VEC, MOVE>(kb, vb, lbb, pb, tb + 2 * step, end, capu, a.cap, lane, tA, vbufA, tmask,
                               tbase);
      compute_tile128<G>(tB, vbufB, tb + step, end, lane, qv, sc, qpos, LB, m2, lsum, acc);
      if (SEL) sel_tile128<LB>(tB, tb + step, end, lane, qpos, bk, bp, bs);
      tb += 2 * step;
    }
    if (ntiles & 1) {
      wait_vmem_all();
      moves(tA, vbufA);
      compute_tile128<G>(tA, vbufA, tb, end, lane, qv, sc, qpos, LB, m2, lsum, acc);
      if (SEL) sel_tile128<LB>(tA, tb, end, lane, qpos, bk, bp, bs);
    }
  }
  if constexpr (SEL) {
    // the four lane groups' candidates
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1)
      one_better(bk, bp, bs, __shfl_xor(bk, o, 64), __shfl_xor(bp, o, 64), __shfl_xor(bs, o, 64));
    if (lane == 0) {
      OneCand c;
      c.key = bk;
      c.slot = bs;
      c.pos = bp;
      a.cand[(size_t)u * a.P + a.p_off + p] = c;
    }
  }
  // staged rows (source below the attended boundary): scratch -> destination.
  // This split copies entries p, p + Pl, ...; each row is 32 pieces of 16 bytes
  // (K then V) plus an 8-byte tail, and four pieces per lane are loaded before
  // any is stored, so a few round trips cover the split's share.
  if (MOVE && mv) {
    const int ns = a.plan.stage_n[u];
    const int ne = ns > p ? (ns - p + Pl - 1) / Pl : 0;
    const int2* sl = a.plan.stage_list + (size_t)u * a.plan.Mk;
    const unsigned char* sbase = a.plan.scratch + (size_t)u * a.plan.Mk * a.plan.srow;
    constexpr int kPer = 4;
    for (int q0 = 0; q0 < 32 * ne; q0 += 64 * kPer) {
      u32x4 x[kPer];
      int dst[kPer];
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int q = q0 + 64 * r + lane;
        const int e = min(q >> 5, ne - 1), pc = q & 31;
        const int2 sd = sl[p + e * Pl];
        dst[r] = q < 32 * ne ? sd.y : -1;
        x[r] = *(const u32x4*)(sbase + (size_t)sd.y * a.plan.srow + 16 * pc);
      }
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int pc = (q0 + 64 * r + lane) & 31;
        if (dst[r] >= 0)
          *(u32x4*)((pc < 16 ? kw : vw) + (size_t)dst[r] * 128 + 8 * (pc & 15)) = x[r];
      }
    }
    for (int e = lane; e < ne; e += 64) {
      const int d = sl[p + e * Pl].y;
      const int32_t* tl = (const int32_t*)(sbase + (size_t)d * a.plan.srow + 256 + 256);
      const int32_t l0 = tl[0], p0 = tl[1];
      if (LB) lbw[d] = __int_as_float(l0);
      pw[d] = p0;
    }
  }

  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int src = lane + G < 64 ? lane + G : lane;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[nb][i] = (acc[nb][i] + __shfl(acc[nb][i], src, 64)) * inv;
  if (lc < G) {
    const int h = g * G + lc;
    const size_t sidx = ((size_t)(b * a.Hq + h)) * a.P + a.p_off + p;
    float* pa = a.part_a + sidx * 128;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) *(f32x4*)(pa + 16 * nb + 4 * lg) = acc[nb];
    if (lg == 0) {
      a.part_ml[2 * sidx] = m2 == kNegInf ? kNegInf : m2 * kLn2;
      a.part_ml[2 * sidx + 1] = lsum;
    }
  }
}

template <int G, bool LB, bool VEC, bool MOVE, bool SEL = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_split_pipe128(AttnArgs a) {
  pipe128_split<G, LB, VEC, MOVE, SEL>(a, blockIdx.x, blockIdx.y);
}

// The splits plus the ASM lookup's candidate scan in one launch: rows y < crow of
// the grid are scan tasks (one wave each, dispatched first), the rest the splits of
// head y - crow.  The scan's few microseconds of latency-bound work then overlap
// the splits instead of preceding them as a launch of their own.
template <int G, bool LB, bool VEC>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_split_asm(AttnArgs a, AsmScanArgs c, int crow) {
  if ((int)blockIdx.y < crow) {
    asm_scan_wave<128>(c, (int)(blockIdx.y * gridDim.x + blockIdx.x));
    return;
  }
  pipe128_split<G, LB, VEC, false>(a, blockIdx.x, (int)blockIdx.y - crow);
}

// ------------------------------------------------------------------ paged split
// Loads of one page of a paged cache: physical page rows pr .. pr + 31 of the head,
// the first fill of them live; rows past fill repeat the last live one (their
// logits are masked by the caller), so every address stays inside the page.  Log
// beta and pos are read four at a time (a page starts on a multiple of 32 slots).
__device__ __forceinline__ void issue_page128(const uint16_t* kb, const uint16_t* vb,
                                              const float* lbb, const int32_t* pb, int pr,
                                              int fill, int lane, KTile& t,
                                              lds_u8* __restrict__ vlds) {
  const int lg = lane >> 4, lc = lane & 15;
  const int last = max(fill, 1) - 1;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = pr + min(16 * j + lc, last);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      t.k[j][kk] = *(const u32x4*)(kb + (ptrdiff_t)row * 128 + 32 * kk + 8 * lg);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = pr + min(4 * i + lg, last);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(vb + (ptrdiff_t)row * 128 + 8 * lc),
                                     (lds_void_t*)(vlds + i * kVBlk), 16, 0, kNonTemporal);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rb = pr + 16 * j + 4 * lg;
    const f32x4 l4 = __builtin_nontemporal_load((const f32x4*)(lbb + rb));
    const i32x4 p4 = __builtin_nontemporal_load((const i32x4*)(pb + rb));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      t.lb[j][r] = l4[r];
      t.ps[j][r] = p4[r];
    }
  }
}

// One split (p, head u) of the attention over a paged cache: split p takes the
// head's logical pages p, p + P, ... (each one 32-slot tile), with the same
// two-stage pipeline and arithmetic as pipe128_split.  The split's page numbers
// and fills are loaded 64 at a time (lane i: the split's i-th page) and read per
// page with a lane read.
template <int G, bool LB>
__device__ __forceinline__ void pipe128_paged(const AttnArgs& a, const int p, const int u) {
  static_assert(2 * G <= 16, "group too large for the hi/lo column split");
  __shared__ __attribute__((aligned(16))) unsigned char vbufA_[8 * kVBlk];
  __shared__ __attribute__((aligned(16))) unsigned char vbufB_[8 * kVBlk];
  lds_u8* vbufA = (lds_u8*)vbufA_;
  lds_u8* vbufB = (lds_u8*)vbufB_;
  const int b = u / a.Hkv;
  const int g = u - b * a.Hkv;
  const int lane = threadIdx.x;
  const int lg = lane >> 4;
  const int lc = lane & 15;
  const int np = min(max(a.pg_n[u], 0), a.pg_max);
  const int pages = a.cap / 32;
  const int32_t* ptab = a.pg_table + (size_t)u * a.pg_max;
  const int32_t* pfil = a.pg_fill + (size_t)u * a.pg_max;
  if (a.n_rec && p == 0 && lane == 0) {
    // the merge appends the decode token: record whether it has room (the last page
    // has a free slot, or the caller's free page can be appended)
    const bool room = (np > 0 && pfil[np - 1] < 32) ||
                      (a.pg_spare && a.pg_spare[u] >= 0 && a.pg_spare[u] < pages && np < a.pg_max);
    a.n_rec[u] = room ? min(max(a.len[u], 0), a.cap - 1) : a.cap;
  }
  if (a.status && p == 0 && u == 0 && lane == 0) a.status[0] = KVB_OK;
  const size_t head0 = (size_t)u * a.cap;

  const int hcol = lc < G ? lc : (lc < 2 * G ? lc - G : -1);
  u32x4 qv[4];
  {
    const uint16_t* qp =
        (const uint16_t*)a.q + ((size_t)(b * a.Hq + g * G + (hcol < 0 ? 0 : hcol))) * 128;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qv[kk] = hcol >= 0 ? *(const u32x4*)(qp + 32 * kk + 8 * lg) : z;
    }
  }
  const uint16_t* kb = (const uint16_t*)a.k + head0 * 128;
  const uint16_t* vb = (const uint16_t*)a.v + head0 * 128;
  const int32_t* pb = a.pos + head0;
  const float* lbb = LB ? a.log_beta + head0 : (const float*)pb;
  const int qpos = a.t[b];
  const float sc = a.scale_log2;

  float m2 = kNegInf, lsum = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int Pl = gridDim.x;
  const int ntiles = p < np ? (np - p + Pl - 1) / Pl : 0;
  int pe = 0, pf = 0;  // lane i: page and fill of the split's tile (64 c + i)
  auto load_pages = [&](int k0) {
    const int idx = p + (k0 + lane) * Pl;
    pe = idx < np ? min(max(ptab[idx], 0), pages - 1) : 0;
    pf = idx < np ? min(max(pfil[idx], 0), 32) : 0;
  };
  auto page_of = [&](int k, int& pr, int& f) {
    if ((k & 63) == 0 && k > 0) load_pages(k);
    pr = 32 * __builtin_amdgcn_readlane(pe, k & 63);
    f = __builtin_amdgcn_readlane(pf, k & 63);
  };
  KTile tA, tB;
  if (ntiles > 0) {
    load_pages(0);
    int prA, fA, prB, fB;
    page_of(0, prA, fA);
    issue_page128(kb, vb, lbb, pb, prA, fA, lane, tA, vbufA);
    int k = 0;
    for (; k + 1 < ntiles; k += 2) {
      wait_vmem_all();
      page_of(k + 1, prB, fB);
      issue_page128(kb, vb, lbb, pb, prB, fB, lane, tB, vbufB);
      compute_tile128<G>(tA, vbufA, 0, fA, lane, qv, sc, qpos, LB, m2, lsum, acc);
      wait_vmem_all();
      if (k + 2 < ntiles) {
        page_of(k + 2, prA, fA);
        issue_page128(kb, vb, lbb, pb, prA, fA, lane, tA, vbufA);
      }
      compute_tile128<G>(tB, vbufB, 0, fB, lane, qv, sc, qpos, LB, m2, lsum, acc);
    }
    if (k < ntiles) {
      wait_vmem_all();
      compute_tile128<G>(tA, vbufA, 0, fA, lane, qv, sc, qpos, LB, m2, lsum, acc);
    }
  }

  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int src = lane + G < 64 ? lane + G : lane;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[nb][i] = (acc[nb][i] + __shfl(acc[nb][i], src, 64)) * inv;
  if (lc < G) {
    const int h = g * G + lc;
    const size_t sidx = ((size_t)(b * a.Hq + h)) * a.P + p;
    float* pa = a.part_a + sidx * 128;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) *(f32x4*)(pa + 16 * nb + 4 * lg) = acc[nb];
    if (lg == 0) {
      a.part_ml[2 * sidx] = m2 == kNegInf ? kNegInf : m2 * kLn2;
      a.part_ml[2 * sidx + 1] = lsum;
    }
  }
}

template <int G, bool LB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_split_paged(AttnArgs a) {
  pipe128_paged<G, LB>(a, blockIdx.x, blockIdx.y);
}

// The candidate scan alone (one wave per task), where the splits are not the
// pipelined kernel.
template <int D>
__global__ __launch_bounds__(64) void asm_scan_kernel(AsmScanArgs c) {
  asm_scan_wave<D>(c, (int)blockIdx.x);
}

// ------------------------------------------------------------------ generic split
template <typename T, int DPL, int MAXG>
__global__ __launch_bounds__(64) void attn_split_generic(AttnArgs a) {
  const int u = blockIdx.y;
  const int p = blockIdx.x;
  const int b = u / a.Hkv;
  const int g = u - b * a.Hkv;
  const int lane = threadIdx.x;
  const int D = a.D, G = a.G;
  const int s0 = head_start(a.start, u);
  const int n = min(a.len[u], a.cap);
  if (a.n_rec && blockIdx.x == 0 && threadIdx.x == 0) a.n_rec[u] = a.len[u];
  if (a.status && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.status[0] = KVB_OK;
  int lo, end;
  split_range(n, p, a.P, lo, end);
  const size_t row0 = (size_t)u * a.cap + s0;  // the head's first live slot

  auto ld = [](const T* ptr) -> float {
    if constexpr (sizeof(T) == 2) return bf16_bits_to_f32(*(const uint16_t*)ptr);
    else return *(const float*)ptr;
  };

  float qf[MAXG][DPL];
#pragma unroll
  for (int h = 0; h < MAXG; ++h)
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
      const int d = lane + 64 * j;
      qf[h][j] = (h < G && d < D)
                     ? ld((const T*)a.q + ((size_t)(b * a.Hq + g * G + h)) * D + d)
                     : 0.f;
    }
  float m[MAXG], Z[MAXG], acc[MAXG][DPL];
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
    m[h] = kNegInf;
    Z[h] = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[h][j] = 0.f;
  }
  const T* kb = (const T*)a.k + row0 * D;
  const T* vb = (const T*)a.v + row0 * D;
  const float* lbb = a.log_beta ? a.log_beta + row0 : nullptr;
  const int32_t* pb = a.pos + row0;
  const int qpos = a.t[b];

  for (int tok = lo; tok < end; ++tok) {
    // the head continues at the start of its slots past the end
    const ptrdiff_t r = tok < a.cap - s0 ? tok : tok - a.cap;
    float kf[DPL], vf[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
      const int d = lane + 64 * j;
      kf[j] = d < D ? ld(kb + r * D + d) : 0.f;
      vf[j] = d < D ? ld(vb + r * D + d) : 0.f;
    }
    float bias = 0.f;
    if (lbb) {
      const int dd = qpos - pb[r];
      bias = dd != 0 ? (float)dd * lbb[r] : 0.f;
    }
#pragma unroll
    for (int h = 0; h < MAXG; ++h) {
      if (h < G) {
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < DPL; ++j) part = fmaf(qf[h][j], kf[j], part);
        const float s = fmaf(wave_sum(part), a.scale_log2, bias * kLog2e);
        const float mn = fmaxf(m[h], s);
        if (mn != kNegInf) {
          const float alpha = m[h] == kNegInf ? 0.f : exp2_fast(m[h] - mn);
          const float pr = exp2_fast(s - mn);
          Z[h] = Z[h] * alpha + pr;
#pragma unroll
          for (int j = 0; j < DPL; ++j) acc[h][j] = fmaf(acc[h][j], alpha, pr * vf[j]);
          m[h] = mn;
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
    if (h < G) {
      const size_t sidx = ((size_t)(b * a.Hq + g * G + h)) * a.P + p;
      const float inv = Z[h] > 0.f ? 1.f / Z[h] : 0.f;
#pragma unroll
      for (int j = 0; j < DPL; ++j) {
        const int d = lane + 64 * j;
        if (d < D) a.part_a[sidx * D + d] = acc[h][j] * inv;
      }
      if (lane == 0) {
        a.part_ml[2 * sidx] = m[h] == kNegInf ? kNegInf : m[h] * kLn2;
        a.part_ml[2 * sidx + 1] = Z[h];
      }
    }
  }
}

// ------------------------------------------------------------------ merge
// One workgroup of NT threads per (b, h) folds the P split states with the merge
// operator (NT = 512 for many splits, else 256).  Weights w_p = Z_p e^{m_p - M}
// are staged in LDS; thread group q (NT / D groups) sums w_p a_p over its
// contiguous share of the splits with 16 loads in flight; the maximum and the
// weight total are tree reductions and the groups' sums are added in group order,
// so the result does not depend on timing.
constexpr int kMergeMaxP = 4096;

// The decode token, merged as a one-token state and appended to the cache by the
// merge (kv_attn_decode with k_new): its logit is scale * q.k_new (no bias: its
// distance is 0), its value v_new.
struct NewTok {
  const void* k_new;   // [U][D] cache dtype, or null (no decode token)
  const void* v_new;
  const float* lb_new; // [U] or null
  const int32_t* t;    // [B]
  const void* q;       // [B][Hq][D] cache dtype
  const int32_t* n_rec;  // [U] len before the append (recorded by the split kernel)
  void* k;
  void* v;
  float* log_beta;
  int32_t* pos;
  int32_t* len;
  const int32_t* start;  // [U] first live slot per head, or null (0)
  int32_t* status;
  int32_t cap, Hkv, elem;
  float scale;         // natural-log scale of q.k
  // paged cache: the token goes into the last page or the caller's free page
  int32_t* pg_table;
  int32_t* pg_fill;
  int32_t* pg_n;
  const int32_t* pg_spare;
  int32_t pg_max;
};

__device__ __forceinline__ float load_elem(const void* p, size_t i, int elem) {
  return elem == 2 ? bf16_bits_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

// Word tid of head u's decode-token K and V rows, for the merge block that appends
// it (loaded with the merge's first round of loads; D * elem / 4 <= D words, so
// every word has a thread).
__device__ __forceinline__ void token_words(const NewTok& nt, int u, int D, int tid, bool mine,
                                            uint32_t& kx, uint32_t& vx) {
  kx = vx = 0u;
  const int words = D * nt.elem / 4;
  if (mine && tid < words) {
    kx = ((const uint32_t*)nt.k_new)[(size_t)u * words + tid];
    vx = ((const uint32_t*)nt.v_new)[(size_t)u * words + tid];
  }
}

// The decode token of head u into a paged cache, by the nthr threads of the merge
// workgroup of the head's first query head (the split kernel found room: the last
// page has a free slot, or the caller's free page can be appended to the table).
// kx, vx: word tid of the token's K and V rows (loaded by the caller; every word of
// the row has a thread).
__device__ __forceinline__ void paged_append(const NewTok& nt, int u, int tid, uint32_t kx,
                                             uint32_t vx) {
  const int np = min(max(nt.pg_n[u], 0), nt.pg_max);
  const int lf = np > 0 ? min(max(nt.pg_fill[(size_t)u * nt.pg_max + np - 1], 0), 32) : 32;
  const bool last = np > 0 && lf < 32;
  const int page = last ? nt.pg_table[(size_t)u * nt.pg_max + np - 1] : nt.pg_spare[u];
  const int pages = nt.cap / 32;
  const int slot = min(max(page, 0), pages - 1) * 32 + (last ? lf : 0);
  const int words = 128 * nt.elem / 4;
  const size_t dst = ((size_t)u * nt.cap + slot) * words;
  if (tid < words) {
    ((uint32_t*)nt.k)[dst + tid] = kx;
    ((uint32_t*)nt.v)[dst + tid] = vx;
  }
  if (tid == 0) {
    nt.pos[(size_t)u * nt.cap + slot] = nt.t[u / nt.Hkv];
    if (nt.log_beta) nt.log_beta[(size_t)u * nt.cap + slot] = nt.lb_new[u];
    if (last) {
      nt.pg_fill[(size_t)u * nt.pg_max + np - 1] = lf + 1;
    } else {
      nt.pg_table[(size_t)u * nt.pg_max + np] = page;
      nt.pg_fill[(size_t)u * nt.pg_max + np] = 1;
      nt.pg_n[u] = np + 1;
    }
    nt.len[u] = nt.n_rec[u] + 1;
  }
}

// Sum and maximum over a workgroup of NT threads: wave butterflies, then the NT / 64
// wave results from LDS in wave order (two barriers; `s` may be reused after).
template <int NT>
__device__ __forceinline__ float merge_block_sum(float x, float* s) {
  x = wave_sum(x);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = x;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += s[i];
  __syncthreads();
  return t;
}

template <int NT>
__device__ __forceinline__ float merge_block_max(float x, float* s) {
  x = wave_max(x);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = x;
  __syncthreads();
  float t = kNegInf;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t = fmaxf(t, s[i]);
  __syncthreads();
  return t;
}

template <int kMergeThreads>
__global__ __launch_bounds__(kMergeThreads) void attn_merge(const float* part_a,
                                                            const float* part_ml, int P, int D,
                                                            float* out, float* lse,
                                                            const UnitInfo* info, int32_t* len,
                                                            int G, NewTok nt, AsmTail at) {
  __shared__ float w[kMergeMaxP];
  __shared__ int s_k;  // the lookup's entry (with an ASM tail)
  __shared__ float red[kMergeThreads / 64];
  __shared__ float gsum[kMergeThreads];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const float* ml = part_ml + (size_t)bh * P * 2;
  const float* pa = part_a + (size_t)bh * P * D;
  const int NG = kMergeThreads / D;  // thread groups over the splits
  const int q = tid / D, d = tid - q * D;
  const int p0 = q < NG ? (int)((long long)P * q / NG) : 0;
  const int p1 = q < NG ? (int)((long long)P * (q + 1) / NG) : 0;
  // the split outputs do not depend on the weights: load the first batch now
  constexpr int kB = 16;
  float x[kB];
#pragma unroll
  for (int e = 0; e < kB; ++e) x[e] = p0 + e < p1 ? pa[(size_t)(p0 + e) * D + d] : 0.f;
  // the decode token's logit (when it is appended here)
  const int u = bh / G;
  uint32_t tkx, tvx;
  token_words(nt, u, D, tid, nt.k_new && bh % G == 0, tkx, tvx);
  bool incl = false;
  float s_new = kNegInf;
  if (nt.k_new) {
    incl = nt.n_rec[u] < nt.cap;
    float pr = 0.f;
    if (incl && tid < D)
      pr = load_elem(nt.q, (size_t)bh * D + tid, nt.elem) *
           load_elem(nt.k_new, (size_t)u * D + tid, nt.elem);
    pr = merge_block_sum<kMergeThreads>(pr, red);
    if (incl) s_new = pr * nt.scale;
  }
  float mx = kNegInf;
  for (int p = tid; p < P; p += kMergeThreads)
    if (ml[2 * p + 1] > 0.f) mx = fmaxf(mx, ml[2 * p]);
  const float M = fmaxf(merge_block_max<kMergeThreads>(mx, red), s_new);
  float ws = 0.f;
  for (int p = tid; p < P; p += kMergeThreads) {
    const float Zp = ml[2 * p + 1];
    const float wp = (Zp > 0.f && M != kNegInf) ? Zp * __expf(ml[2 * p] - M) : 0.f;
    w[p] = wp;
    ws += wp;
  }
  const float wsum = merge_block_sum<kMergeThreads>(ws, red);  // also orders the w[] stores
  const float w_new = incl ? __expf(s_new - M) : 0.f;
  const float W = wsum + w_new;
  float o = 0.f;
#pragma unroll
  for (int e = 0; e < kB; ++e)
    if (p0 + e < p1) o = fmaf(w[p0 + e], x[e], o);
  for (int pb = p0 + kB; pb < p1; pb += kB) {
#pragma unroll
    for (int e = 0; e < kB; ++e) x[e] = pb + e < p1 ? pa[(size_t)(pb + e) * D + d] : 0.f;
#pragma unroll
    for (int e = 0; e < kB; ++e)
      if (pb + e < p1) o = fmaf(w[pb + e], x[e], o);
  }
  // ASM tail (the lookup's step 4): the best candidate entry of this query head
  if (at.cand_score && tid < 64) {
    const int b = bh / at.Hq, h = bh - b * at.Hq;
    const int g = h / G, j = h - g * G;
    float q2 = 0.f;
    for (int d = tid; d < D; d += 64) {
      const float x = bf16_bits_to_f32(at.q[(size_t)bh * D + d]);
      q2 = fmaf(x, x, q2);
    }
    q2 = wave_sum(q2);
    float bs = kNegInf;
    int bk = 0x7FFFFFFF;
    const size_t base = ((size_t)g * at.QB * 16 + b * G + j) * at.KC;
    for (int c = tid; c < at.KC; c += 64) {
      const float sc = at.cand_score[base + c];
      const int k = at.cand_idx[base + c];
      if (sc > bs || (sc == bs && k < bk)) {
        bs = sc;
        bk = k;
      }
    }
#pragma unroll
    for (int o2 = 32; o2 >= 1; o2 >>= 1) {
      const float os = __shfl_xor(bs, o2, 64);
      const int ok = __shfl_xor(bk, o2, 64);
      if (os > bs || (os == bs && ok < bk)) {
        bs = os;
        bk = ok;
      }
    }
    if (tid == 0) {
      const int k = (q2 > 0.f && bk != 0x7FFFFFFF) ? bk : 0;
      s_k = k;
      if (at.idx) at.idx[bh] = k;
    }
  }
  gsum[tid] = o;
  __syncthreads();
  const float lse_self = W > 0.f ? M + __logf(W) : kNegInf;
  // merge with the entry's stored state by the normalisers (as asm_lookup_merge)
  float w1 = 0.f, w2 = 0.f, lse_out = lse_self;
  const uint16_t* ab = nullptr;
  if (at.cand_score) {
    const int h = bh - (bh / at.Hq) * at.Hq, g = h / G;
    const float lz = at.log_zbar[(size_t)g * at.K + s_k];
    const float Mx = fmaxf(lse_self, lz);
    lse_out = kNegInf;
    if (Mx != kNegInf) {
      w1 = lse_self == kNegInf ? 0.f : __expf(lse_self - Mx);
      w2 = lz == kNegInf ? 0.f : __expf(lz - Mx);
      lse_out = Mx + __logf(w1 + w2);
    }
    ab = at.abar + ((size_t)g * at.K + s_k) * D;
  }
  if (tid < D) {
    float acc = 0.f;
    for (int g = 0; g < NG; ++g) acc += gsum[g * D + tid];
    if (incl) acc = fmaf(w_new, load_elem(nt.v_new, (size_t)u * D + tid, nt.elem), acc);
    float so = W > 0.f ? acc / W : 0.f;
    if (ab) {
      const float inv = (w1 + w2) > 0.f ? 1.f / (w1 + w2) : 0.f;
      so = fmaf(w1, so, w2 * bf16_bits_to_f32(ab[tid])) * inv;
    }
    out[(size_t)bh * D + tid] = so;
  }
  if (tid == 0) lse[bh] = lse_out;
  // append the decode token (first query head of each KV head); every split has
  // read the old len, and the other merge blocks use the recorded one
  if (nt.k_new && bh % G == 0 && nt.pg_table) {
    if (incl) paged_append(nt, u, tid, tkx, tvx);
    else if (tid == 0) nt.status[0] = KVB_ECAPACITY;
  } else if (nt.k_new && bh % G == 0) {
    if (!incl) {
      if (tid == 0) nt.status[0] = KVB_ECAPACITY;
    } else {
      const int n0 = nt.n_rec[u];
      int s0 = head_start(nt.start, u) + n0;  // slot of the decode token
      if (s0 >= nt.cap) s0 -= nt.cap;
      const int words = D * nt.elem / 4;
      const size_t dst = ((size_t)u * nt.cap + s0) * words;
      if (tid < words) {
        ((uint32_t*)nt.k)[dst + tid] = tkx;
        ((uint32_t*)nt.v)[dst + tid] = tvx;
      }
      if (tid == 0) {
        nt.pos[(size_t)u * nt.cap + s0] = nt.t[u / nt.Hkv];
        if (nt.log_beta) nt.log_beta[(size_t)u * nt.cap + s0] = nt.lb_new[u];
        nt.len[u] = n0 + 1;
      }
    }
  }
  // fused compaction: the head's new length (every split has read the old one)
  if (info && tid == 0 && bh % G == 0) {
    if (info[u].mode == MODE_EVICT) len[u] = info[u].kept;
  }
}

// The merge for at most 64 splits and D in {64, 128}: one thread per output
// dimension, reductions over the splits by wave shuffles (wave 0, one split per
// lane) instead of workgroup-wide trees, so the chain is one round of loads (split
// states, decode token, lookup candidates), a few shuffles, the chosen entry's
// gather and the stores.  Same arithmetic per output as attn_merge up to the
// order of the per-dimension sum (here split by split, in order).
template <int D, int kB>
__global__ __launch_bounds__(D) void attn_merge_small(const float* part_a, const float* part_ml,
                                                      int P, float* out, float* lse,
                                                      const UnitInfo* info, int32_t* len,
                                                      int G, NewTok nt, AsmTail at, OnePlan op) {
  constexpr int NW = D / 64;
  __shared__ int s_e;
  __shared__ float s_w[64];
  __shared__ float s_red[2][NW];
  __shared__ float s_mw[2];
  __shared__ int s_k;
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* ml = part_ml + (size_t)bh * P * 2;
  const float* pa = part_a + (size_t)bh * P * D;
  const int u = bh / G;
  // every load of the first round: this dimension's split outputs (the first kB:
  // all of them when P <= kB), the split (m, Z) in wave 0, the decode token's q.k
  // product terms and its row, the candidates
  float x[kB];
#pragma unroll
  for (int e = 0; e < kB; ++e) x[e] = e < P ? pa[(size_t)e * D + tid] : 0.f;
  uint32_t tkx, tvx;
  token_words(nt, u, D, tid, nt.k_new && bh % G == 0, tkx, tvx);
  float mp = kNegInf, zp = 0.f;
  if (wave == 0 && lane < P) {
    mp = ml[2 * lane];
    zp = ml[2 * lane + 1];
  }
  bool incl = false;
  float pr = 0.f;
  if (nt.k_new) {
    incl = nt.n_rec[u] < nt.cap;
    if (incl)
      pr = load_elem(nt.q, (size_t)bh * D + tid, nt.elem) *
           load_elem(nt.k_new, (size_t)u * D + tid, nt.elem);
  }
  // the one-eviction candidates (the head's first query head plans)
  const bool plans = op.cand && bh % G == 0;
  OneCand oc;
  if (plans) oc = one_plan_load(op, u, tid);
  float q2 = 0.f;
  float cs = kNegInf;
  int ck = 0x7FFFFFFF;
  const int bq = bh / (at.cand_score ? at.Hq : 1);
  const int hq = bh - bq * (at.cand_score ? at.Hq : 1);
  if (at.cand_score) {
    const float xq = bf16_bits_to_f32(at.q[(size_t)bh * D + tid]);
    q2 = xq * xq;
    if (wave == 0) {
      const int g = hq / G, j = hq - g * G;
      const size_t base = ((size_t)g * at.QB * 16 + bq * G + j) * at.KC;
      for (int c = lane; c < at.KC; c += 64) {
        const float sc = at.cand_score[base + c];
        const int k = at.cand_idx[base + c];
        if (sc > cs || (sc == cs && k < ck)) {
          cs = sc;
          ck = k;
        }
      }
    }
  }
  // decode-token logit and |q|^2 over the workgroup
  pr = wave_sum(pr);
  q2 = wave_sum(q2);
  if (lane == 0) {
    s_red[0][wave] = pr;
    s_red[1][wave] = q2;
  }
  __syncthreads();
  float s_new = kNegInf;
  if (incl) {
    float dsum = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) dsum += s_red[0][w2];
    s_new = dsum * nt.scale;
  }
  // split maximum, weights and total, and the lookup's best entry (wave 0)
  if (wave == 0) {
    const float Mp = wave_max(zp > 0.f ? mp : kNegInf);
    const float M = fmaxf(Mp, s_new);
    const float wp = (zp > 0.f && M != kNegInf) ? zp * __expf(mp - M) : 0.f;
    const float W = wave_sum(wp);
    if (lane < P) s_w[lane] = wp;
    if (lane == 0) {
      s_mw[0] = M;
      s_mw[1] = W;
    }
    if (at.cand_score) {
#pragma unroll
      for (int o2 = 32; o2 >= 1; o2 >>= 1) {
        const float os = __shfl_xor(cs, o2, 64);
        const int ok = __shfl_xor(ck, o2, 64);
        if (os > cs || (os == cs && ok < ck)) {
          cs = os;
          ck = ok;
        }
      }
      if (lane == 0) {
        float qq = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) qq += s_red[1][w2];
        const int k = (qq > 0.f && ck != 0x7FFFFFFF) ? ck : 0;
        s_k = k;
        if (at.idx) at.idx[bh] = k;
      }
    }
  }
  __syncthreads();
  const float M = s_mw[0];
  const float w_new = incl ? __expf(s_new - M) : 0.f;
  const float W = s_mw[1] + w_new;
  float o = 0.f;
#pragma unroll
  for (int e = 0; e < kB; ++e)
    if (e < P) o = fmaf(s_w[e], x[e], o);
  for (int pb = kB; pb < P; pb += kB) {
#pragma unroll
    for (int e = 0; e < kB; ++e) x[e] = pb + e < P ? pa[(size_t)(pb + e) * D + tid] : 0.f;
#pragma unroll
    for (int e = 0; e < kB; ++e)
      if (pb + e < P) o = fmaf(s_w[pb + e], x[e], o);
  }
  if (incl) o = fmaf(w_new, load_elem(nt.v_new, (size_t)u * D + tid, nt.elem), o);
  float so = W > 0.f ? o / W : 0.f;
  const float lse_self = W > 0.f ? M + __logf(W) : kNegInf;
  float lse_out = lse_self;
  if (at.cand_score) {
    // merge with the entry's stored state by the normalisers (as asm_lookup_merge)
    const int g = hq / G;
    const int k = s_k;
    const float lz = at.log_zbar[(size_t)g * at.K + k];
    const float av = bf16_bits_to_f32(at.abar[((size_t)g * at.K + k) * D + tid]);
    const float Mx = fmaxf(lse_self, lz);
    float w1 = 0.f, w2 = 0.f;
    lse_out = kNegInf;
    if (Mx != kNegInf) {
      w1 = lse_self == kNegInf ? 0.f : __expf(lse_self - Mx);
      w2 = lz == kNegInf ? 0.f : __expf(lz - Mx);
      lse_out = Mx + __logf(w1 + w2);
    }
    const float inv = (w1 + w2) > 0.f ? 1.f / (w1 + w2) : 0.f;
    so = fmaf(w1, so, w2 * av) * inv;
  }
  out[(size_t)bh * D + tid] = so;
  if (tid == 0) lse[bh] = lse_out;
  // kv_attn_decode_evict_one: a head with M + 1 live tokens (the decode token
  // included) loses the lowest (key, position) among the splits' candidates and the
  // decode token; decided before the decode token is written, since it may take the
  // evicted slot
  int ev = -1, n_ev = 0;
  if (plans && op.fill_M >= 0) {
    int n0 = 0, n;
    if (nt.k_new) {
      n0 = min(max(nt.n_rec[u], 0), nt.cap);
      n = incl ? n0 + 1 : n0;
    } else {
      n = min(max(op.len[u], 0), op.cap);
    }
    if (tid < 64) {
      double bk = oc.key;
      int bp = oc.pos, bs = oc.slot;
      if (tid == 0 && nt.k_new && incl) one_better(bk, bp, bs, 0.0, nt.t[u / nt.Hkv], n0);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1)
        one_better(bk, bp, bs, __shfl_xor(bk, o, 64), __shfl_xor(bp, o, 64),
                   __shfl_xor(bs, o, 64));
      if (tid == 0) {
        int e = -1;
        if (n == op.fill_M + 1) {
          e = min(max(bs, 0), n - 1);
          if (op.evicted_pos && op.max_evict > 0)
            op.evicted_pos[(size_t)u * op.max_evict] = bp;
        }
        if (op.n_evicted)
          op.n_evicted[u] = e >= 0 ? 1 : (n <= op.fill_M ? 0 : -(n - op.fill_M));
        s_e = e;
      }
    }
    __syncthreads();
    ev = s_e;
    n_ev = n;
  }
  // append the decode token (first query head of each KV head); every split has
  // read the old len, and the other merge blocks use the recorded one.  With an
  // eviction above the token goes into the evicted slot (not at all when it is the
  // evicted one) and len stays.
  if (nt.k_new && bh % G == 0 && nt.pg_table) {
    if (incl) paged_append(nt, u, tid, tkx, tvx);
    else if (tid == 0) nt.status[0] = KVB_ECAPACITY;
  } else if (nt.k_new && bh % G == 0) {
    if (!incl) {
      if (tid == 0) nt.status[0] = KVB_ECAPACITY;
    } else {
      const int n0 = nt.n_rec[u];
      if (ev != n0) {
        int s0 = head_start(nt.start, u) + (ev >= 0 ? ev : n0);  // slot of the decode token
        if (s0 >= nt.cap) s0 -= nt.cap;
        const int words = D * nt.elem / 4;
        const size_t dst = ((size_t)u * nt.cap + s0) * words;
        if (tid < words) {
          ((uint32_t*)nt.k)[dst + tid] = tkx;
          ((uint32_t*)nt.v)[dst + tid] = tvx;
        }
        if (tid == 0) {
          nt.pos[(size_t)u * nt.cap + s0] = nt.t[u / nt.Hkv];
          if (nt.log_beta) nt.log_beta[(size_t)u * nt.cap + s0] = nt.lb_new[u];
          nt.len[u] = ev >= 0 ? n0 : n0 + 1;
        }
      }
    }
  }
  if (ev >= 0 && !(nt.k_new && incl)) {
    // no decode token written here: the last live row moves into the evicted slot
    const int n = n_ev;
    const int s0 = op.start ? min(max(op.start[u], 0), op.cap - 1) : 0;
    auto slot = [&](int i) { return s0 + i < op.cap ? s0 + i : s0 + i - op.cap; };
    const size_t row0 = (size_t)u * op.cap;
    if (ev != n - 1) {
      const int words = op.row_bytes / 4;
      const size_t se = (row0 + slot(ev)) * words, sl = (row0 + slot(n - 1)) * words;
      for (int w = tid; w < words; w += D) {
        const uint32_t kx = ((const uint32_t*)op.k)[sl + w];
        const uint32_t vx = ((const uint32_t*)op.v)[sl + w];
        ((uint32_t*)op.k)[se + w] = kx;
        ((uint32_t*)op.v)[se + w] = vx;
      }
      if (tid == 0) {
        if (op.log_beta) op.log_beta[row0 + slot(ev)] = op.log_beta[row0 + slot(n - 1)];
        op.pos[row0 + slot(ev)] = op.pos[row0 + slot(n - 1)];
      }
    }
    if (tid == 0) op.len[u] = n - 1;
  }
  // fused compaction: the head's new length (every split has read the old one)
  if (info && tid == 0 && bh % G == 0) {
    if (info[u].mode == MODE_EVICT) len[u] = info[u].kept;
  }
  // the one-eviction plan (kv_attn_decode_plan_one), by the head's first query head:
  // the splits' candidates and, when appended here, the decode token (key 0, the
  // head's last slot)
  if (plans && op.fill_M < 0) {
    int n;
    bool has_new = false;
    if (nt.k_new) {
      const int n0 = min(max(nt.n_rec[u], 0), nt.cap);
      n = incl ? n0 + 1 : n0;
      has_new = incl;
    } else {
      n = min(max(op.len[u], 0), op.cap);
    }
    one_plan_head(op, u, n, has_new, 0.0, has_new ? nt.t[u / nt.Hkv] : 0, oc, tid, D, &s_e);
  }
}

// ------------------------------------------------------------------ host
// Returns true when the merge also made the one-eviction plan (`one`).
static bool launch_merge(const float* part_a, const float* part_ml, int P, int D, float* out,
                         float* lse, const UnitInfo* info, int32_t* len, int G, int BH,
                         hipStream_t s, const NewTok* nt = nullptr,
                         const AsmTail* tail = nullptr, const OnePlan* one = nullptr) {
  NewTok none;
  memset(&none, 0, sizeof(none));
  const NewTok& n = nt ? *nt : none;
  AsmTail no_tail;
  memset(&no_tail, 0, sizeof(no_tail));
  const AsmTail& at = tail ? *tail : no_tail;
  OnePlan no_plan;
  memset(&no_plan, 0, sizeof(no_plan));
  const OnePlan& op = one ? *one : no_plan;
  // the small merge loads every split's output in one round (16 or 64 per thread)
  if (P <= 64 && D == 128) {
    if (P <= 16)
      hipLaunchKernelGGL((attn_merge_small<128, 16>), dim3(BH), dim3(128), 0, s, part_a,
                         part_ml, P, out, lse, info, len, G, n, at, op);
    else
      hipLaunchKernelGGL((attn_merge_small<128, 64>), dim3(BH), dim3(128), 0, s, part_a,
                         part_ml, P, out, lse, info, len, G, n, at, op);
    return true;
  }
  if (P <= 64 && D == 64) {
    if (P <= 16)
      hipLaunchKernelGGL((attn_merge_small<64, 16>), dim3(BH), dim3(64), 0, s, part_a, part_ml,
                         P, out, lse, info, len, G, n, at, op);
    else
      hipLaunchKernelGGL((attn_merge_small<64, 64>), dim3(BH), dim3(64), 0, s, part_a, part_ml,
                         P, out, lse, info, len, G, n, at, op);
    return true;
  }
  if (P > 128)
    hipLaunchKernelGGL(attn_merge<512>, dim3(BH), dim3(512), 0, s, part_a, part_ml, P, D, out,
                       lse, info, len, G, n, at);
  else
    hipLaunchKernelGGL(attn_merge<256>, dim3(BH), dim3(256), 0, s, part_a, part_ml, P, D, out,
                       lse, info, len, G, n, at);
  return false;
}

static bool mfma_supported(const kvb_cache* c, int G) {
  return c->dtype == KVB_BF16 && (c->D == 64 || c->D == 128) &&
         (G == 1 || G == 2 || G == 4 || G == 8);
}

// 16-byte loads of log beta and pos: every head's first live slot must be a
// multiple of 4 (per-head starts are not known on the host).
static bool vec_bias_loads(const kvb_cache* c) {
  return c->cap % 4 == 0 && c->cap >= 4 && c->start == nullptr;
}

template <int D, int G>
static void launch_mfma(const AttnArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_split_mfma<D, G>), grid, dim3(64), 0, s, a);
}

static int32_t launch_split(const kvb_cache* c, const AttnArgs& a, hipStream_t s,
                            const AsmScanArgs* scan = nullptr, const OnePlan* one = nullptr) {
  dim3 grid(a.P, c->B * c->Hkv);
  const long long crow_ll = scan ? ((long long)scan->tasks + a.P - 1) / a.P : 0;
  if (scan && c->dtype == KVB_BF16 && c->D == 128 &&
      (a.G == 1 || a.G == 2 || a.G == 4 || a.G == 8) &&
      crow_ll + (long long)c->B * c->Hkv <= 65535) {
    // the candidate scan rides in the first rows of the split launch
    const int crow = (int)crow_ll;
    dim3 g2(a.P, crow + c->B * c->Hkv);
#define KVB_ASM_CASE(GG)                                                                   \
  if (a.G == GG) {                                                                         \
    const bool lb = c->log_beta != nullptr, vec = vec_bias_loads(c);                      \
    if (lb && vec) hipLaunchKernelGGL((attn_split_asm<GG, true, true>), g2, dim3(64), 0, s, a, *scan, crow);   \
    else if (lb) hipLaunchKernelGGL((attn_split_asm<GG, true, false>), g2, dim3(64), 0, s, a, *scan, crow);   \
    else if (vec) hipLaunchKernelGGL((attn_split_asm<GG, false, true>), g2, dim3(64), 0, s, a, *scan, crow);  \
    else hipLaunchKernelGGL((attn_split_asm<GG, false, false>), g2, dim3(64), 0, s, a, *scan, crow);          \
    return KVB_OK;                                                                         \
  }
    KVB_ASM_CASE(1) KVB_ASM_CASE(2) KVB_ASM_CASE(4) KVB_ASM_CASE(8)
#undef KVB_ASM_CASE
  }
  if (scan) {
    // other shapes: the scan as a launch of its own before the splits
    if (c->D == 128)
      hipLaunchKernelGGL(asm_scan_kernel<128>, dim3(scan->tasks), dim3(64), 0, s, *scan);
    else
      hipLaunchKernelGGL(asm_scan_kernel<64>, dim3(scan->tasks), dim3(64), 0, s, *scan);
  }
  if (a.cand && c->dtype == KVB_BF16 && c->D == 128 &&
      (a.G == 1 || a.G == 2 || a.G == 4 || a.G == 8)) {
    // the splits also find the one-eviction candidates
#define KVB_SEL_CASE(GG)                                                                   \
  if (a.G == GG) {                                                                         \
    const bool lb = c->log_beta != nullptr, vec = vec_bias_loads(c);                      \
    if (lb && vec) hipLaunchKernelGGL((attn_split_pipe128<GG, true, true, false, true>), grid, dim3(64), 0, s, a);   \
    else if (lb) hipLaunchKernelGGL((attn_split_pipe128<GG, true, false, false, true>), grid, dim3(64), 0, s, a);   \
    else if (vec) hipLaunchKernelGGL((attn_split_pipe128<GG, false, true, false, true>), grid, dim3(64), 0, s, a);  \
    else hipLaunchKernelGGL((attn_split_pipe128<GG, false, false, false, true>), grid, dim3(64), 0, s, a);          \
    return KVB_OK;                                                                         \
  }
    KVB_SEL_CASE(1) KVB_SEL_CASE(2) KVB_SEL_CASE(4) KVB_SEL_CASE(8)
#undef KVB_SEL_CASE
  }
  if (one) {
    // other kernels: the candidates from a scan of log beta and pos of their own
    launch_one_scan(c, a.t, *one, s);
  }
  if (mfma_supported(c, a.G)) {
#define KVB_PIPE_CASE(GG)                                                                  \
  if (c->D == 128 && a.G == GG) {                                                          \
    const bool lb = c->log_beta != nullptr, vec = vec_bias_loads(c);                      \
    if (lb && vec) hipLaunchKernelGGL((attn_split_pipe128<GG, true, true, false>), grid, dim3(64), 0, s, a);   \
    else if (lb) hipLaunchKernelGGL((attn_split_pipe128<GG, true, false, false>), grid, dim3(64), 0, s, a);   \
    else if (vec) hipLaunchKernelGGL((attn_split_pipe128<GG, false, true, false>), grid, dim3(64), 0, s, a);  \
    else hipLaunchKernelGGL((attn_split_pipe128<GG, false, false, false>), grid, dim3(64), 0, s, a);          \
    return KVB_OK;                                                                         \
  }
    KVB_PIPE_CASE(1) KVB_PIPE_CASE(2) KVB_PIPE_CASE(4) KVB_PIPE_CASE(8)
#undef KVB_PIPE_CASE
#define KVB_MFMA_CASE(DD, GG) \
  if (c->D == DD && a.G == GG) { launch_mfma<DD, GG>(a, grid, s); return KVB_OK; }
    KVB_MFMA_CASE(64, 1) KVB_MFMA_CASE(64, 2) KVB_MFMA_CASE(64, 4) KVB_MFMA_CASE(64, 8)
#undef KVB_MFMA_CASE
  }
  const int dpl = (c->D + 63) / 64;
#define KVB_GEN_CASE(TT, DPL)                                                           \
  if (dpl == DPL) {                                                                     \
    hipLaunchKernelGGL((attn_split_generic<TT, DPL, 16>), grid, dim3(64), 0, s, a);    \
    return KVB_OK;                                                                      \
  }
  if (c->dtype == KVB_F32) {
    KVB_GEN_CASE(float, 1) KVB_GEN_CASE(float, 2) KVB_GEN_CASE(float, 3) KVB_GEN_CASE(float, 4)
  } else {
    KVB_GEN_CASE(__bf16, 1) KVB_GEN_CASE(__bf16, 2) KVB_GEN_CASE(__bf16, 3)
    KVB_GEN_CASE(__bf16, 4)
  }
#undef KVB_GEN_CASE
  return KVB_EUNSUPPORTED;
}

static int32_t launch_paged(const kvb_cache* c, const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.P, c->B * c->Hkv);
  const bool lb = c->log_beta != nullptr;
#define KVB_PAGED_CASE(GG)                                                                 \
  if (a.G == GG) {                                                                         \
    if (lb) hipLaunchKernelGGL((attn_split_paged<GG, true>), grid, dim3(64), 0, s, a);     \
    else hipLaunchKernelGGL((attn_split_paged<GG, false>), grid, dim3(64), 0, s, a);       \
    return KVB_OK;                                                                         \
  }
  KVB_PAGED_CASE(1) KVB_PAGED_CASE(2) KVB_PAGED_CASE(4) KVB_PAGED_CASE(8)
#undef KVB_PAGED_CASE
  return KVB_EUNSUPPORTED;
}

// Candidate-scan dimensions of kv_attn_decode_asm: QB blocks of 16 query rows per KV
// head, KC chunks of kScanChunk centroids, one task per (chunk, head, 64 rows).
static AsmScanArgs scan_dims(int B, int Hq, int Hkv, int K) {
  AsmScanArgs c;
  memset(&c, 0, sizeof(c));
  c.B = B;
  c.Hq = Hq;
  c.Hkv = Hkv;
  c.K = K;
  c.G = Hq / Hkv;
  c.QB = (B * c.G + 15) / 16;
  c.KC = (K + kScanChunk - 1) / kScanChunk;
  c.tasks = c.KC * Hkv * ((c.QB + kScanQB - 1) / kScanQB);
  return c;
}

// About one round of resident waves (2 per SIMD on 256 CUs): fewer, longer splits
// stream better than many short ones (on the 32K layer 16 splits per head take 331
// us, 32 take 337 us, 64 take 374 us), and keep the merged partial states small.  A
// split covers at least 256 slots (two 128-token tiles): on short heads one-tile
// splits spend their time in set-up and partial-state writes.
static int32_t auto_splits(const kvb_cache* c) {
  const long long units = (long long)c->B * c->Hkv;
  if (units < 1) return 1;
  const long long tiles = c->cap / 256;
  long long P = (2048 + units - 1) / units;
  if (P > tiles) P = tiles;
  if (P > 1024) P = 1024;
  if (P < 1) P = 1;
  return (int32_t)P;
}

}  // namespace kvb

using namespace kvb;

extern "C" int32_t kv_attn_decode_splits(const kvb_cache* cache, int32_t Hq) {
  (void)Hq;
  if (!cache_dims_ok(cache)) return 0;
  return auto_splits(cache);
}

extern "C" size_t kv_attn_decode_workspace(const kvb_cache* cache, int32_t Hq, int32_t num_splits) {
  if (!cache_dims_ok(cache) || Hq < 1 || num_splits < 0) return 0;
  const size_t P = num_splits > 0 ? (size_t)num_splits : (size_t)auto_splits(cache);
  const size_t S = (size_t)cache->B * Hq * P;
  return kWsHeader + align_up(S * cache->D * sizeof(float), 256) +
         align_up(S * 2 * sizeof(float), 256) + align_up((size_t)cache->B * cache->Hkv * 4, 256);
}

extern "C" int32_t kv_append(const kvb_cache* cache, const void* k_new, const void* v_new,
                             const float* log_beta_new, const int32_t* t, void* ws,
                             size_t ws_bytes, void* stream) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (!k_new || !v_new || !t || (cache->log_beta && !log_beta_new)) return KVB_EINVAL;
  if (!ws || ws_bytes < kWsHeader) return KVB_EWORKSPACE;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  const int elem = cache->dtype == KVB_BF16 ? 2 : 4;
  TraceScope tr(kTrAppend, s);
  hipLaunchKernelGGL(status_reset, dim3(1), dim3(64), 0, s, (int32_t*)ws);
  hipLaunchKernelGGL(kv_append, dim3(cache->B * cache->Hkv), dim3(64), 0, s, cache->k, cache->v,
                     cache->log_beta, cache->pos, cache->len, cache->start, cache->cap,
                     cache->D * elem / 4,
                     k_new, v_new, log_beta_new, t, cache->Hkv, (int32_t*)ws);
  return launch_status();
}

// The decode attention; with an ASM tail its merge also merges each query head's
// chosen codebook entry (kv_attn_decode_asm).
static int32_t attn_decode_impl(const kvb_cache* cache, const void* q, int32_t Hq,
                                const int32_t* t, float scale, const void* k_new,
                                const void* v_new, const float* log_beta_new,
                                int32_t num_splits, float* out, float* lse, void* ws,
                                size_t ws_bytes, hipStream_t stream, const AsmTail* tail,
                                int32_t* status = nullptr,
                                const AsmScanArgs* scan = nullptr,
                                const OnePlan* one = nullptr, const kvb_pages* pages = nullptr,
                                const int32_t* spare = nullptr) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (!q || !t || !out || !lse || Hq < 1 || Hq % cache->Hkv != 0) return KVB_EINVAL;
  if (((uintptr_t)q & 15u) != 0) return KVB_EINVAL;  // query rows read 16 bytes at a time
  if ((k_new == nullptr) != (v_new == nullptr)) return KVB_EINVAL;
  if (k_new && cache->log_beta && !log_beta_new) return KVB_EINVAL;
  if (num_splits < 0 || num_splits > 4096) return KVB_EINVAL;
  const int G = Hq / cache->Hkv;
  if (!mfma_supported(cache, G) && (G > 16 || cache->D > 256)) return KVB_EUNSUPPORTED;
  const int P = num_splits > 0 ? num_splits : auto_splits(cache);
  const size_t need = kv_attn_decode_workspace(cache, Hq, P);
  if (!ws || ws_bytes < need) return KVB_EWORKSPACE;
  if ((st = check_device())) return st;

  hipStream_t s = stream;
  const size_t S = (size_t)cache->B * Hq * P;
  AttnArgs a;
  a.k = cache->k;
  a.v = cache->v;
  a.log_beta = cache->log_beta;
  a.pos = cache->pos;
  a.len = cache->len;
  a.start = cache->start;
  a.q = q;
  a.t = t;
  a.part_a = (float*)((char*)ws + kWsHeader);
  a.part_ml = (float*)((char*)ws + kWsHeader + align_up(S * cache->D * sizeof(float), 256));
  a.B = cache->B;
  a.Hkv = cache->Hkv;
  a.cap = cache->cap;
  a.D = cache->D;
  a.Hq = Hq;
  a.G = G;
  a.P = P;
  a.scale_log2 = (scale > 0.f ? scale : 1.0f / sqrtf((float)cache->D)) * kLog2e;
  a.tile_lo = 0;
  a.tile_hi = 1 << 30;
  a.p_off = 0;
  if (!status) status = (int32_t*)ws;
  a.status = status;
  if (one) a.cand = (OneCand*)one->cand;

  // with a decode token: attend over the cached tokens (the splits record each
  // head's len), then the merge adds the token's own state and appends it
  NewTok nt;
  memset(&nt, 0, sizeof(nt));
  a.n_rec = nullptr;
  if (k_new) {
    a.n_rec = (int32_t*)((char*)ws + kWsHeader + align_up(S * cache->D * sizeof(float), 256) +
                         align_up(S * 2 * sizeof(float), 256));
    nt.k_new = k_new;
    nt.v_new = v_new;
    nt.lb_new = log_beta_new;
    nt.t = t;
    nt.q = q;
    nt.n_rec = a.n_rec;
    nt.k = cache->k;
    nt.v = cache->v;
    nt.log_beta = cache->log_beta;
    nt.pos = cache->pos;
    nt.len = cache->len;
    nt.start = cache->start;
    nt.status = status;
    nt.cap = cache->cap;
    nt.Hkv = cache->Hkv;
    nt.elem = cache->dtype == KVB_BF16 ? 2 : 4;
    nt.scale = a.scale_log2 * kLn2;
  }
  if (pages) {
    a.pg_table = pages->table;
    a.pg_fill = pages->fill;
    a.pg_n = pages->n_pages;
    a.pg_spare = spare;
    a.pg_max = pages->max_pages;
    nt.pg_table = pages->table;
    nt.pg_fill = pages->fill;
    nt.pg_n = pages->n_pages;
    nt.pg_spare = spare;
    nt.pg_max = pages->max_pages;
    TraceScope tr(kTrAttnSplit, s);
    if ((st = launch_paged(cache, a, s))) return st;
  } else {
    TraceScope tr(kTrAttnSplit, s);
    if ((st = launch_split(cache, a, s, scan, one))) return st;
  }
  TraceScope tr(kTrAttnMerge, s);
  const bool planned = launch_merge(a.part_a, a.part_ml, P, cache->D, out, lse, nullptr,
                                    nullptr, G, cache->B * Hq, s, k_new ? &nt : nullptr, tail,
                                    one);
  if (one && !planned) launch_one_plan(cache, t, *one, s);
  return launch_status();
}

extern "C" int32_t kv_attn_decode(const kvb_cache* cache, const void* q, int32_t Hq,
                                  const int32_t* t, float scale, const void* k_new,
                                  const void* v_new, const float* log_beta_new,
                                  int32_t num_splits, float* out, float* lse, void* ws,
                                  size_t ws_bytes, void* stream) {
  return attn_decode_impl(cache, q, Hq, t, scale, k_new, v_new, log_beta_new, num_splits, out,
                          lse, ws, ws_bytes, (hipStream_t)stream, nullptr);
}

// Splits of the paged attention: about 2048 workgroups, at most one per 8 pages a
// head can hold, never more than kv_attn_decode_workspace's own default.
static int32_t paged_splits(const kvb_cache* c, const kvb_pages* pg) {
  const long long units = (long long)c->B * c->Hkv;
  long long P = (2048 + units - 1) / units;
  const long long per = pg->max_pages / 8;
  if (P > per) P = per;
  if (P > auto_splits(c)) P = auto_splits(c);
  if (P < 1) P = 1;
  return (int32_t)P;
}

extern "C" int32_t kv_attn_decode_paged(const kvb_cache* cache, const kvb_pages* pages,
                                        const void* q, int32_t Hq, const int32_t* t, float scale,
                                        const void* k_new, const void* v_new,
                                        const float* log_beta_new, const int32_t* spare,
                                        int32_t num_splits, float* out, float* lse, void* ws,
                                        size_t ws_bytes, void* stream) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (!pages || !pages->table || !pages->fill || !pages->n_pages || pages->max_pages < 1)
    return KVB_EINVAL;
  if (cache->start || cache->cap % 32 != 0) return KVB_EINVAL;
  if (Hq < 1 || Hq % cache->Hkv != 0) return KVB_EINVAL;
  if (!mfma_supported(cache, Hq / cache->Hkv) || cache->D != 128) return KVB_EUNSUPPORTED;
  if (num_splits < 0 || num_splits > 4096) return KVB_EINVAL;
  const int32_t P = num_splits > 0 ? num_splits : paged_splits(cache, pages);
  return attn_decode_impl(cache, q, Hq, t, scale, k_new, v_new, log_beta_new, P, out, lse, ws,
                          ws_bytes, (hipStream_t)stream, nullptr, nullptr, nullptr, nullptr,
                          pages, spare);
}

extern "C" int32_t kv_attn_decode_plan_one(const kvb_cache* cache, const void* q, int32_t Hq,
                                           const int32_t* t, float scale, const void* k_new,
                                           const void* v_new, const float* log_beta_new,
                                           int32_t num_splits, float* out, float* lse, void* ws,
                                           size_t ws_bytes, void* ws_evict,
                                           size_t ws_evict_bytes, void* stream) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (num_splits < 0 || num_splits > 4096) return KVB_EINVAL;
  if ((long long)cache->B * cache->Hkv > 65535) return KVB_EUNSUPPORTED;
  const int32_t P = num_splits > 0 ? num_splits : auto_splits(cache);
  if (!ws_evict || ws_evict_bytes < kv_evict_one_workspace(cache, P)) return KVB_EWORKSPACE;
  const OnePlan op = one_plan_args(cache, P, ws_evict);
  return attn_decode_impl(cache, q, Hq, t, scale, k_new, v_new, log_beta_new, P, out, lse, ws,
                          ws_bytes, (hipStream_t)stream, nullptr, nullptr, nullptr, &op);
}

// kv_attn_decode_evict_one's workspace: the attention's, then the candidates.
extern "C" size_t kv_attn_decode_evict_one_workspace(const kvb_cache* cache, int32_t Hq,
                                                     int32_t num_splits) {
  if (!cache_dims_ok(cache) || Hq < 1 || Hq % cache->Hkv != 0) return 0;
  const size_t a = kv_attn_decode_workspace(cache, Hq, num_splits);
  if (a == 0 || num_splits < 0 || num_splits > 4096) return 0;
  const size_t P = num_splits > 0 ? (size_t)num_splits : (size_t)auto_splits(cache);
  return a + align_up((size_t)cache->B * cache->Hkv * P * sizeof(OneCand), 256);
}

extern "C" int32_t kv_attn_decode_evict_one(const kvb_cache* cache, const void* q, int32_t Hq,
                                            const int32_t* t, float scale, const void* k_new,
                                            const void* v_new, const float* log_beta_new,
                                            int32_t M, int32_t num_splits, float* out,
                                            float* lse, int32_t* evicted_pos, int32_t max_evict,
                                            int32_t* n_evicted, void* ws, size_t ws_bytes,
                                            void* stream) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (num_splits < 0 || num_splits > 4096 || M < 0 || max_evict < 0) return KVB_EINVAL;
  if ((long long)cache->B * cache->Hkv > 65535) return KVB_EUNSUPPORTED;
  const int32_t P = num_splits > 0 ? num_splits : auto_splits(cache);
  const size_t need = kv_attn_decode_evict_one_workspace(cache, Hq, P);
  if (need == 0) return KVB_EINVAL;
  if (!ws || ws_bytes < need) return KVB_EWORKSPACE;
  OnePlan op;
  memset(&op, 0, sizeof(op));
  op.cand = (const OneCand*)((char*)ws + kv_attn_decode_workspace(cache, Hq, P));
  op.k = cache->k;
  op.v = cache->v;
  op.log_beta = cache->log_beta;
  op.pos = cache->pos;
  op.start = cache->start;
  op.len = cache->len;
  op.P = P;
  op.cap = cache->cap;
  op.row_bytes = cache->D * (cache->dtype == KVB_BF16 ? 2 : 4);
  op.fill_M = M;
  op.evicted_pos = evicted_pos;
  op.max_evict = max_evict;
  op.n_evicted = n_evicted;
  return attn_decode_impl(cache, q, Hq, t, scale, k_new, v_new, log_beta_new, P, out, lse, ws,
                          ws_bytes, (hipStream_t)stream, nullptr, nullptr, nullptr, &op);
}

// ------------------------------------------------------------------ no-alloc entry
// Scratch of kv_attn_decode_noalloc: a device global, so each GPU the library runs
// on holds its own copy (zero-filled .bss of the code object) until the process
// ends.  In host code the array's name only stands for the symbol: its device
// address, per device, comes from hipGetSymbolAddress (made once per device, with
// that device current) and is what the kernels get.
namespace kvb {
static __device__ __align__(256) unsigned char scratch[KVB_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

static int32_t scratch_of_current_device(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return KVB_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVB_EDEVICE;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return KVB_OK;
}
}  // namespace kvb

extern "C" int32_t kv_attn_decode_noalloc(const kvb_cache* cache, const void* q, int32_t Hq,
                                          const int32_t* t, float scale, const void* k_new,
                                          const void* v_new, const float* log_beta_new,
                                          int32_t num_splits, float* out, float* lse,
                                          int32_t* status, void* stream) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (!q || !t || !out || !lse || Hq < 1 || Hq % cache->Hkv != 0) return KVB_EINVAL;
  if (num_splits < 0 || num_splits > 4096) return KVB_EINVAL;
  const size_t need = kv_attn_decode_workspace(cache, Hq, num_splits);
  if (need == 0 || need > KVB_NOALLOC_SCRATCH_BYTES) return KVB_EWORKSPACE;
  if ((st = check_device())) return st;
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws))) return st;
  return attn_decode_impl(cache, q, Hq, t, scale, k_new, v_new, log_beta_new, num_splits, out,
                          lse, ws, KVB_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream, nullptr,
                          status);
}

// Default split count of kv_attn_decode_asm: where the codebook scan rides in the
// split launch (bf16, D = 128), its tasks take wave slots of the same round, so the
// splits get at most what one round of resident waves (2 per SIMD on 256 CUs)
// leaves, rounded down to a power of two, never more than kv_attn_decode's default.
// On the ASM workload (512 scan tasks, 256 heads of 2049 tokens): 4 splits per head
// 507 steps/s, 5: 498, 6 (one full round): 496, 8 (kv_attn_decode's default): 479.
// The size limits kv_attn_decode_asm checks, for its host-only queries.
static bool asm_dims_ok(const kvb_cache* c, int32_t Hq, int32_t K) {
  return cache_dims_ok(c) && K >= 1 && K < (1 << 24) && Hq >= 1 && Hq % c->Hkv == 0 &&
         (long long)c->B * (Hq / c->Hkv) <= 65536;
}

static int32_t asm_splits(const kvb_cache* c, int32_t Hq, int32_t K) {
  const int32_t P = auto_splits(c);
  const int G = Hq / c->Hkv;
  if (c->dtype != KVB_BF16 || c->D != 128 || (G != 1 && G != 2 && G != 4 && G != 8)) return P;
  const long long tasks = scan_dims(c->B, Hq, c->Hkv, K).tasks;
  const long long units = (long long)c->B * c->Hkv;
  if (tasks >= 2048) return P;
  long long left = (2048 - tasks) / units;
  if (left > P) left = P;
  int32_t p2 = 1;
  while (2LL * p2 <= left) p2 *= 2;
  return p2;
}

extern "C" int32_t kv_attn_decode_asm_splits(const kvb_cache* cache, int32_t Hq, int32_t K) {
  if (!asm_dims_ok(cache, Hq, K)) return 0;
  return asm_splits(cache, Hq, K);
}

extern "C" size_t kv_attn_decode_asm_workspace(const kvb_cache* cache, int32_t Hq,
                                               int32_t num_splits, int32_t K) {
  if (!asm_dims_ok(cache, Hq, K) || num_splits < 0) return 0;
  if (num_splits == 0) num_splits = asm_splits(cache, Hq, K);
  const size_t wa = kv_attn_decode_workspace(cache, Hq, num_splits);
  if (!wa) return 0;
  const AsmScanArgs c = scan_dims(cache->B, Hq, cache->Hkv, K);
  const size_t n = (size_t)cache->Hkv * c.QB * 16 * c.KC;
  return align_up(wa, 256) + 2 * align_up(n * 4, 256);
}

extern "C" int32_t kv_attn_decode_asm(const kvb_cache* cache, const void* q, int32_t Hq,
                                      const int32_t* t, float scale, const void* k_new,
                                      const void* v_new, const float* log_beta_new,
                                      int32_t num_splits, const void* centroids,
                                      const void* abar, const float* log_zbar, int32_t K,
                                      float* out, float* lse, int32_t* idx, void* ws,
                                      size_t ws_bytes, void* stream) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (!q || !centroids || !abar || !log_zbar) return KVB_EINVAL;
  if (cache->dtype != KVB_BF16) return KVB_EUNSUPPORTED;  // q and the codebook are bf16
  if (K < 1 || K >= (1 << 24) || Hq < 1 || Hq % cache->Hkv) return KVB_EINVAL;
  if ((long long)cache->B * (Hq / cache->Hkv) > 65536) return KVB_EINVAL;
  if (num_splits < 0 || num_splits > 4096) return KVB_EINVAL;
  const int P = num_splits > 0 ? num_splits : asm_splits(cache, Hq, K);
  const size_t need = kv_attn_decode_asm_workspace(cache, Hq, P, K);
  if (!ws || ws_bytes < need) return KVB_EWORKSPACE;
  if ((st = check_device())) return st;
  AsmScanArgs sc = scan_dims(cache->B, Hq, cache->Hkv, K);
  const size_t wa = align_up(kv_attn_decode_workspace(cache, Hq, P), 256);
  const size_t n = (size_t)cache->Hkv * sc.QB * 16 * sc.KC;
  sc.q = (const uint16_t*)q;
  sc.cent = (const uint16_t*)centroids;
  sc.cand_score = (float*)((char*)ws + wa);
  sc.cand_idx = (int32_t*)((char*)ws + wa + align_up(n * 4, 256));
  AsmTail at;
  at.cand_score = sc.cand_score;
  at.cand_idx = sc.cand_idx;
  at.q = (const uint16_t*)q;
  at.abar = (const uint16_t*)abar;
  at.log_zbar = log_zbar;
  at.idx = idx;
  at.K = K;
  at.KC = sc.KC;
  at.QB = sc.QB;
  at.Hq = Hq;
  // the lookup needs only q and the codebook: its candidate scan runs in the first
  // workgroups of the split launch, and the attention's merge finishes the lookup.
  // (As a launch of its own before the splits it added ~13 us of latency to the
  // layer; beside them on a second stream it was starved by their workgroups.)
  return attn_decode_impl(cache, q, Hq, t, scale, k_new, v_new, log_beta_new, P, out, lse, ws,
                          wa, (hipStream_t)stream, &at, nullptr, &sc);
}

// ------------------------------------------------------------------ fused attention + compaction
namespace kvb {

template <int G>
static void launch_pipe_move(const kvb_cache* c, const AttnArgs& a, dim3 grid, hipStream_t s,
                             bool move) {
  const bool lb = c->log_beta != nullptr, vec = c->cap % 4 == 0 && c->cap >= 4;
  if (move) {
    if (lb && vec) hipLaunchKernelGGL((attn_split_pipe128<G, true, true, true>), grid, dim3(64), 0, s, a);
    else if (lb) hipLaunchKernelGGL((attn_split_pipe128<G, true, false, true>), grid, dim3(64), 0, s, a);
    else if (vec) hipLaunchKernelGGL((attn_split_pipe128<G, false, true, true>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((attn_split_pipe128<G, false, false, true>), grid, dim3(64), 0, s, a);
  } else {
    if (lb && vec) hipLaunchKernelGGL((attn_split_pipe128<G, true, true, false>), grid, dim3(64), 0, s, a);
    else if (lb) hipLaunchKernelGGL((attn_split_pipe128<G, true, false, false>), grid, dim3(64), 0, s, a);
    else if (vec) hipLaunchKernelGGL((attn_split_pipe128<G, false, true, false>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((attn_split_pipe128<G, false, false, false>), grid, dim3(64), 0, s, a);
  }
}

static void launch_pipe_any(const kvb_cache* c, const AttnArgs& a, dim3 grid, hipStream_t s,
                            bool move) {
  switch (a.G) {
    case 1: launch_pipe_move<1>(c, a, grid, s, move); break;
    case 2: launch_pipe_move<2>(c, a, grid, s, move); break;
    case 4: launch_pipe_move<4>(c, a, grid, s, move); break;
    default: launch_pipe_move<8>(c, a, grid, s, move); break;
  }
}

}  // namespace kvb

extern "C" int32_t kv_attn_decode_compact(const kvb_cache* cache, const void* q, int32_t Hq,
                                          const int32_t* t, float scale, int32_t M,
                                          int32_t num_splits, int32_t phase, float* out,
                                          float* lse, void* ws, size_t ws_bytes, void* ws_evict,
                                          size_t ws_evict_bytes, void* stream) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (!q || !t || !out || !lse || Hq < 1 || Hq % cache->Hkv != 0 || M < 0) return KVB_EINVAL;
  if (num_splits < 0 || num_splits > 4096 || phase < 0 || phase > 2) return KVB_EINVAL;
  const int G = Hq / cache->Hkv;
  if (!mfma_supported(cache, G) && (G > 16 || cache->D > 256)) return KVB_EUNSUPPORTED;
  const int P = num_splits > 0 ? num_splits : auto_splits(cache);
  if (!ws || ws_bytes < kv_attn_decode_workspace(cache, Hq, P)) return KVB_EWORKSPACE;
  if (!ws_evict || ws_evict_bytes < kv_evict_workspace(cache, M)) return KVB_EWORKSPACE;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  // (per-head starts: the unfused path)
  const bool fused = cache->dtype == KVB_BF16 && cache->D == 128 &&
                     (G == 1 || G == 2 || G == 4 || G == 8) && P >= 2 && plan_in_lds(cache) &&
                     cache->start == nullptr;
  if (!fused) {
    // same result through the unfused kernels: attention, then the planned moves
    if (phase == 1) return KVB_OK;
    st = kv_attn_decode(cache, q, Hq, t, scale, nullptr, nullptr, nullptr, P, out, lse, ws,
                        ws_bytes, stream);
    if (st) return st;
    return kv_evict_apply(cache, M, ws_evict, ws_evict_bytes, stream);
  }
  // Phase 1 covers few tiles but runs beside the planner: half the splits keep
  // enough waves in flight for it (measured on the 32K workload).
  const int Ta = fused_za(M, cache->cap) / 32;
  int Pa = P / 2;
  if (Pa > Ta) Pa = Ta;
  Pa = Pa < 1 ? 1 : (Pa > P - 1 ? P - 1 : Pa);
  const int Pb = P - Pa;
  const size_t S = (size_t)cache->B * Hq * P;
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.k = cache->k;
  a.v = cache->v;
  a.log_beta = cache->log_beta;
  a.pos = cache->pos;
  a.len = cache->len;
  a.start = cache->start;
  a.q = q;
  a.t = t;
  a.part_a = (float*)((char*)ws + kWsHeader);
  a.part_ml = (float*)((char*)ws + kWsHeader + align_up(S * cache->D * sizeof(float), 256));
  a.B = cache->B;
  a.Hkv = cache->Hkv;
  a.cap = cache->cap;
  a.D = cache->D;
  a.Hq = Hq;
  a.G = G;
  a.P = P;
  a.scale_log2 = (scale > 0.f ? scale : 1.0f / sqrtf((float)cache->D)) * kLog2e;
  const int U = cache->B * cache->Hkv;
  if (phase != 2) {  // tiles below the destination boundary: attention only
    a.tile_lo = 0;
    a.tile_hi = Ta;
    a.p_off = 0;
    TraceScope tr(kTrAttnSplit, s);
    launch_pipe_any(cache, a, dim3(Pa, U), s, false);
  }
  if (phase != 1) {  // the remaining tiles, with their kept rows written to place
    a.tile_lo = Ta;
    a.tile_hi = 1 << 30;
    a.p_off = Pa;
    a.plan = fused_plan(cache, M, ws_evict);
    launch_fused_stage(cache, M, ws_evict, s);
    a.kw = cache->k;
    a.vw = cache->v;
    a.lbw = cache->log_beta;
    a.posw = cache->pos;
    {
      TraceScope tr(kTrAttnFused, s);
      launch_pipe_any(cache, a, dim3(Pb, U), s, true);
    }
    TraceScope tr(kTrAttnMerge, s);
    launch_merge(a.part_a, a.part_ml, P, cache->D, out, lse, a.plan.info, cache->len, G,
                 cache->B * Hq, s);
  }
  return launch_status();
}
