// Shared device and host helpers for the kvbound HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvbound.h"

namespace kvb {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Workspace header: the first 256 bytes of every workspace are reserved
// (status word and alignment); operation data starts at kWsHeader.
constexpr size_t kWsHeader = 256;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// 2^x on the transcendental unit (v_exp_f32); inputs here are <= 0 or -inf.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats to packed bf16 (a in the low half), round to nearest-even, on the
// hardware conversion (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// hi = bf16(a), bf16(b) packed; lo = bf16 of the remainders, packed: a = hi + lo to
// about 16 significant bits.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

// bf16 bits of x rounded to nearest-even (x finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Wait for every outstanding vector memory operation (s_waitcnt vmcnt(0), other
// counters untouched), fenced against instruction scheduling on both sides.  LDS
// filled by global_load_lds is not tracked by the compiler's own waits.
__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier for LDS traffic only: after it every wave's LDS writes are
// complete and visible, while global loads a wave has in flight stay in flight
// (__syncthreads() fences global memory too and so waits for them).
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two floats to packed fp16 (a in the low half), round to nearest-even.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x4 mfma_16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Per-head eviction plan header (workspace), written by the planners.
enum { MODE_NOOP = 0, MODE_EVICT = 1, MODE_ERASE = 2 };
// First live slot of head u: live slots are start[u] .. start[u] + len[u] - 1
// (every head starts at slot 0 without a start array).
__device__ __forceinline__ int head_start(const int32_t* start, int u) {
  return start ? start[u] : 0;
}

struct UnitInfo {
  uint64_t kstar;  // ordered 64-bit key of the threshold element
  int32_t sstar;   // its slot
  int32_t mode;
  int32_t n;       // live slots before
  int32_t kept;    // live slots after
  int32_t nstart;  // first live slot after the compaction
  int32_t ostart;  // first live slot before it (the start array is rewritten by the
                   // compaction, so its workgroups read this copy)
};
static_assert(sizeof(UnitInfo) == 32, "UnitInfo layout");

// ASM lookup's candidates and stored states, for the attention merge that also
// performs the lookup's merge (kv_attn_decode_asm): per query row of KV head g the
// best (score, lowest index) of KC chunk candidates at
// [g][qrow][c] (qrow = b * G + j), then entry k's (abar, log Zbar).
struct AsmTail {
  const float* cand_score;  // null: no lookup merge
  const int32_t* cand_idx;
  const uint16_t* q;        // [B][Hq][D] bf16 (zero query -> entry 0)
  const uint16_t* abar;     // [Hkv][K][D] bf16
  const float* log_zbar;    // [Hkv][K]
  int32_t* idx;             // [B][Hq] or null
  int32_t K, KC, QB, Hq;
};

// Lookup candidates (the first kernel of asm_lookup_merge): per KV head, query row
// and 256-centroid chunk, the best cosine and its index.
void asm_dims(int B, int Hq, int Hkv, int K, int& G, int& QB, int& KC);
void launch_asm_candidates(const uint16_t* q, int B, int Hq, int Hkv, int D,
                           const uint16_t* centroids, int K, float* cand_score,
                           int32_t* cand_idx, hipStream_t s);

// Compaction state a fused attention launch reads from an eviction plan: per
// 32-slot tile the keep mask and the destination of its first kept row, and the
// kept rows whose source lies below `za` (staged in scratch by the planner).
struct FusedPlan {
  const UnitInfo* info;
  const uint32_t* tile_mask;  // [U][Tc]
  const int32_t* tile_base;   // [U][Tc]
  const int32_t* stage_n;     // [U]
  const int2* stage_list;     // [U][Mk]  (src, dst)
  const unsigned char* scratch;  // [U][Mk][srow] by destination
  int32_t Tc, Mk, srow;
};

// Host: the boundary below which a fused attention + compaction launch attends
// before it moves any row (all destinations lie below it): M rounded up to a tile.
inline int fused_za(int M, int cap) {
  const int m = M < cap ? M : cap;
  return (m + 31) / 32 * 32;
}
bool plan_in_lds(const kvb_cache* c);
FusedPlan fused_plan(const kvb_cache* c, int32_t M, void* ws);
// Host: where an eviction plan (kv_evict_plan with budget M) keeps, per head, its
// UnitInfo and the kept source slots in ascending order ([U][Mk], first `kept`
// entries valid when mode == MODE_EVICT).
struct EvictView {
  const UnitInfo* info;
  const int32_t* keep_src;
  int32_t Mk;
  // per 32-slot tile of an evicted head: keep bits and kept slots before the tile
  // (written by the LDS planner only: null when the plan came from the other path)
  const uint32_t* tile_mask;
  const int32_t* tile_base;
  int32_t Tc;
};
EvictView evict_view(const kvb_cache* c, int32_t M, const void* ws);
// Copies the fused apply's staged rows (kept rows below the boundary that move) to
// the plan's scratch; must run after kv_evict_plan and before any row is written.
void launch_fused_stage(const kvb_cache* c, int32_t M, void* ws, hipStream_t s);

// One-eviction planning (kv_attn_decode_plan_one -> kv_evict_one_apply).
// Candidates: per head and split, the slot (relative to the head's first live slot)
// with the lowest (retention key, position) among the slots the split attended
// (positions are distinct, so the order is total); key +inf, position and slot
// INT32_MAX for a split with no slot.
struct OneCand {
  double key;
  int32_t slot;
  int32_t pos;
};
static_assert(sizeof(OneCand) == 16, "OneCand layout");
// Per head: the evicted slot e (relative) among n live slots, the direction of the
// shift (up: rows [0, e) one slot toward the last slot; else rows (e, n) one slot
// toward the first), its chunk count and the head's first slot.
struct OneInfo {
  int32_t e, n, up, nch, s0, pad0, pad1, pad2;
};
static_assert(sizeof(OneInfo) == 32, "OneInfo layout");
// What the planner needs: the candidates, where the plan goes (info, and the staged
// rows: the source row b_c = e -+ (c + 1) R of every shift chunk c with a successor,
// which chunk c + 1's destinations overwrite), and the cache.  With fill_M >= 0
// (kv_attn_decode_evict_one) there is no plan: a head with fill_M + 1 live tokens
// evicts at once, the decode token (or the last live row) taking the evicted slot,
// and the outputs are written.
struct OnePlan {
  const OneCand* cand;   // [U][P]; null: no planning
  OneInfo* info;         // [U]
  unsigned char* scratch;  // [U][SC][srow]: K row, V row, (log beta, pos)
  void* k;
  void* v;
  float* log_beta;
  int32_t* pos;
  const int32_t* start;
  int32_t* len;
  int32_t P, cap, R, SC, srow, row_bytes;
  int32_t fill_M;
  int32_t* evicted_pos;  // [U][max_evict] or null
  int32_t max_evict;
  int32_t* n_evicted;    // [U] or null
};
// Host: the plan arguments of a one-eviction workspace (P candidates per head).
OnePlan one_plan_args(const kvb_cache* c, int32_t P, void* ws);
// Candidates by a scan of log beta and pos alone (splits other than the pipelined
// kernel's): chunk p of each head's live slots gives entry p.
void launch_one_scan(const kvb_cache* c, const int32_t* t, const OnePlan& p, hipStream_t s);
// The plan by a kernel of its own (merges that do not plan), after the merge: the
// candidates and the head's last live slot; with p.fill_M >= 0 the eviction by fill.
void launch_one_plan(const kvb_cache* c, const int32_t* t, const OnePlan& p, hipStream_t s);

// Keeps the lower of (bk, bp) and (k, ps) in (key, position) order, with its slot.
__device__ __forceinline__ void one_better(double& bk, int& bp, int& bs, double k, int ps,
                                           int s) {
  if (k < bk || (k == bk && ps < bp)) {
    bk = k;
    bp = ps;
    bs = s;
  }
}

// This thread's candidate of head u for one_plan_head (threads below min(P, 64); the
// others hold no candidate), loaded early so that its latency overlaps other work.
__device__ __forceinline__ OneCand one_plan_load(const OnePlan& p, int u, int tid) {
  OneCand c;
  c.key = __builtin_huge_val();
  c.slot = 0x7FFFFFFF;
  c.pos = 0x7FFFFFFF;
  if (tid < 64 && tid < p.P) c = p.cand[(size_t)u * p.P + tid];
  return c;
}

// The plan of head u, by all nthr threads of one workgroup (nthr a multiple of 64,
// every thread calls it): the lowest (key, position) over the P candidates (own:
// this thread's one_plan_load) and, with has_last, slot n - 1 with key last_key and
// position last_pos; then the staged rows (shift only) and the head's OneInfo.
// s_e: a __shared__ int of the caller.
__device__ __forceinline__ void one_plan_head(const OnePlan& p, int u, int n, bool has_last,
                                              double last_key, int last_pos, OneCand own,
                                              int tid, int nthr, int* s_e) {
  const int s0 = p.start ? min(max(p.start[u], 0), p.cap - 1) : 0;
  if (tid < 64) {
    double bk = own.key;
    int bp = own.pos, bs = own.slot;
    for (int i = tid + 64; i < p.P; i += 64) {
      const OneCand c = p.cand[(size_t)u * p.P + i];
      one_better(bk, bp, bs, c.key, c.pos, c.slot);
    }
    if (tid == 0 && has_last && n > 0) one_better(bk, bp, bs, last_key, last_pos, n - 1);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
      one_better(bk, bp, bs, __shfl_xor(bk, o, 64), __shfl_xor(bp, o, 64), __shfl_xor(bs, o, 64));
    if (tid == 0) *s_e = n > 0 ? min(max(bs, 0), n - 1) : 0;
  }
  __syncthreads();
  const int e = *s_e;
  const bool up = p.start != nullptr && e < n - 1 - e;
  const int moved = n > 0 ? (up ? e : n - 1 - e) : 0;
  const int nch = (moved + p.R - 1) / p.R;
  const int ppr = p.row_bytes / 16;
  const int per = 2 * ppr + 1;  // 16-byte pieces of K and V, then (log beta, pos)
  const int items = nch > 1 ? (nch - 1) * per : 0;
  const size_t row0 = (size_t)u * p.cap;
  const unsigned char* kb = (const unsigned char*)p.k + row0 * p.row_bytes;
  const unsigned char* vb = (const unsigned char*)p.v + row0 * p.row_bytes;
  unsigned char* sc = p.scratch + (size_t)u * p.SC * p.srow;
  constexpr int kIn = 4;
  for (int i0 = 0; i0 < items; i0 += nthr * kIn) {
    u32x4 x[kIn];
#pragma unroll
    for (int q = 0; q < kIn; ++q) {
      const int it = min(i0 + q * nthr + tid, items - 1);
      const int c = it / per, pt = it - c * per;
      int sl = s0 + (up ? e - (c + 1) * p.R : e + (c + 1) * p.R);
      if (sl >= p.cap) sl -= p.cap;
      if (pt < 2 * ppr)
        x[q] = *(const u32x4*)((pt < ppr ? kb : vb) + (size_t)sl * p.row_bytes + 16 * (pt % ppr));
      else
        x[q] = u32x4{p.log_beta ? __float_as_uint(p.log_beta[row0 + sl]) : 0u,
                     (uint32_t)p.pos[row0 + sl], 0u, 0u};
    }
#pragma unroll
    for (int q = 0; q < kIn; ++q) {
      const int it = i0 + q * nthr + tid;
      if (it >= items) continue;
      const int c = it / per, pt = it - c * per;
      *(u32x4*)(sc + (size_t)c * p.srow +
                (pt < 2 * ppr ? (pt < ppr ? 0 : p.row_bytes) + 16 * (pt % ppr) : 2 * p.row_bytes)) =
          x[q];
    }
  }
  if (tid == 0) {
    const OneInfo inf = {e, n, up ? 1 : 0, nch, s0, 0, 0, 0};
    p.info[u] = inf;
  }
}

// Host: 0 if the current device is gfx950, else KVB_EDEVICE (cached per device).
int32_t check_device();

// Host: validate a cache descriptor (pointers, sizes, dtype/D support).
int32_t check_cache(const kvb_cache* c, bool need_kv);
// check_cache's size checks alone (no pointers): what a host-only size query needs
// before it computes with the descriptor's dimensions.
bool cache_dims_ok(const kvb_cache* c);

// Kernel-launch tracing (see kvb_trace_enable): records a HIP event pair on the
// launch stream around each traced kernel while enabled.
enum TraceKernel {
  kTrAttnSplit = 1, kTrAttnMerge = 2, kTrAppend = 4, kTrEvictSelect = 8, kTrKeepCount = 16,
  kTrKeepEmit = 32, kTrCompactMove = 64, kTrAsmLookup = 128, kTrAsmFinalize = 256,
  kTrAttnFused = 512, kTrAsmPrefix = 1024, kTrAsmPrefixMerge = 2048, kTrKmAssign = 4096,
  kTrKmUpdate = 8192, kTrAsmAggregate = 16384, kTrAsmVt = 32768,
  kTrLatentAbsorb = 65536, kTrLatentRead = 131072, kTrEvictOne = 262144,
  kTrEraseSearch = 524288, kTrErasePlan = 1048576, kTrOneShift = 4194304,
  kTrErasePages = 8388608
};
struct TraceScope {
  TraceScope(int kernel, hipStream_t s);
  ~TraceScope();
  int slot;
  hipStream_t stream;
};

inline int32_t launch_status() {
  return hipGetLastError() == hipSuccess ? KVB_OK : KVB_ELAUNCH;
}

}  // namespace kvb
