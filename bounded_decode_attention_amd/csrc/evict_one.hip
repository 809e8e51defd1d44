// The steady state of bounded decoding ("Cache What Lasts", section 2.2, inference:
// each decode step puts one token into a head that holds M, and the token with
// the lowest retention score beta_i^(t-i) leaves), with the selection folded into
// the attention so that no pass over the head's keys runs on its own.  The
// attention's splits find, per head, the attended slot with the lowest (kappa,
// position), kappa = (t - pos) * log beta exact in double, from the log beta and pos
// values each split loads for the bias anyway; one candidate per split.  Then:
//
//   kv_attn_decode_evict_one  the merge (or one_plan after merges that do not
//                 plan) reduces the candidates and the decode token to the evicted
//                 slot e and writes the decode token into e instead of appending
//                 it (fill): nothing else moves, and the live slots are no longer
//                 in position order;
//   kv_attn_decode_plan_one + kv_evict_one_apply  the order-keeping form: the
//                 merge reduces the candidates to e, picks the shorter side (with
//                 a start array the rows before e move up one slot when there are
//                 fewer of them, else the rows after e move down one slot) and
//                 copies the few rows the shift cannot read in place to scratch;
//                 one_shift moves the rows, one workgroup per chunk of R rows, and
//                 sets len, start and the outputs.
//
// In-place safety of the shift: chunk c of a head moves its R source rows one slot
// toward e's side.  Its destinations overlap its own sources (read into registers
// before any store, behind a barrier) and exactly one source row of the chunk
// before it: the row b_(c-1) = e -+ cR at the boundary (the first row of the
// previous chunk moving up, the last one moving down).  The plan copies b_c of
// every chunk c with a successor to scratch, and chunk c reads that row from there.
//
// one_scan forms the candidates from log beta and pos alone, for the split kernels
// that do not produce them.
#include "common.h"

namespace kvb {

struct OneLayout {
  size_t info, scratch, cand;
  int R, SC, srow, row_bytes, X;
};

constexpr int kShiftThreads = 256;
constexpr int kShiftPieces = 8;  // 16-byte pieces per thread per chunk

static OneLayout one_layout(const kvb_cache* c) {
  OneLayout L;
  const size_t U = (size_t)c->B * c->Hkv;
  L.row_bytes = c->D * (c->dtype == KVB_BF16 ? 2 : 4);
  L.srow = 2 * L.row_bytes + 16;
  const int cols = 2 * (L.row_bytes / 16);
  const int rpp = kShiftThreads / cols;
  L.R = rpp * kShiftPieces;
  if (L.R > kShiftThreads) L.R = kShiftThreads;  // one thread per row tail
  // rows one eviction can move: n - 1 <= cap - 1 toward the first slot; with a start
  // array the shorter side, at most (cap - 1) / 2
  const long long most = c->start ? (c->cap - 1) / 2 : c->cap - 1;
  L.X = (int)((most + L.R - 1) / L.R);
  if (L.X < 1) L.X = 1;
  L.SC = L.X > 1 ? L.X - 1 : 1;
  L.info = kWsHeader;
  L.scratch = L.info + align_up(U * sizeof(OneInfo), 256);
  L.cand = L.scratch + align_up(U * L.SC * (size_t)L.srow, 256);
  return L;
}

OnePlan one_plan_args(const kvb_cache* c, int32_t P, void* ws) {
  const OneLayout L = one_layout(c);
  OnePlan p;
  p.cand = (const OneCand*)((char*)ws + L.cand);
  p.info = (OneInfo*)((char*)ws + L.info);
  p.scratch = (unsigned char*)ws + L.scratch;
  p.k = c->k;
  p.v = c->v;
  p.log_beta = c->log_beta;
  p.pos = c->pos;
  p.start = c->start;
  p.len = c->len;
  p.P = P;
  p.cap = c->cap;
  p.R = L.R;
  p.SC = L.SC;
  p.srow = L.srow;
  p.row_bytes = L.row_bytes;
  p.fill_M = -1;
  p.evicted_pos = nullptr;
  p.max_evict = 0;
  p.n_evicted = nullptr;
  return p;
}

__device__ __forceinline__ double one_key(bool has_lb, int d, float lb) {
  return (has_lb && d != 0) ? (double)d * (double)lb : 0.0;
}

// ---------------------------------------------------------------- candidates
// Chunk p (of gridDim.x) of head u's live slots: the lowest (key, slot).
__global__ __launch_bounds__(256) void one_scan(OnePlan pl, const int32_t* t, int32_t Hkv) {
  __shared__ double sk[4];
  __shared__ int sp[4], ss[4];
  const int p = blockIdx.x, u = blockIdx.y, P = gridDim.x, tid = threadIdx.x;
  const int n = min(max(pl.len[u], 0), pl.cap);
  const int s0 = pl.start ? min(max(pl.start[u], 0), pl.cap - 1) : 0;
  const int lo = (int)((long long)n * p / P), hi = (int)((long long)n * (p + 1) / P);
  const int tq = t[u / Hkv];
  const size_t row0 = (size_t)u * pl.cap;
  double bk = __builtin_huge_val();
  int bp = 0x7FFFFFFF, bs = 0x7FFFFFFF;
  for (int i = lo + tid; i < hi; i += 256) {
    const int sl = s0 + i < pl.cap ? s0 + i : s0 + i - pl.cap;
    const int ps = pl.pos[row0 + sl];
    one_better(bk, bp, bs,
               one_key(pl.log_beta != nullptr, tq - ps, pl.log_beta ? pl.log_beta[row0 + sl] : 0.f),
               ps, i);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
    one_better(bk, bp, bs, __shfl_xor(bk, o, 64), __shfl_xor(bp, o, 64), __shfl_xor(bs, o, 64));
  if ((tid & 63) == 0) {
    sk[tid >> 6] = bk;
    sp[tid >> 6] = bp;
    ss[tid >> 6] = bs;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) one_better(bk, bp, bs, sk[w], sp[w], ss[w]);
    OneCand c;
    c.key = bk;
    c.slot = bs;
    c.pos = bp;
    ((OneCand*)pl.cand)[(size_t)u * P + p] = c;
  }
}

void launch_one_scan(const kvb_cache* c, const int32_t* t, const OnePlan& p, hipStream_t s) {
  hipLaunchKernelGGL(one_scan, dim3(p.P, c->B * c->Hkv), dim3(256), 0, s, p, t, c->Hkv);
}

// The plan of head blockIdx.x after a merge that does not plan: its candidates and
// its last live slot (the decode token if the call appended one).  With fill_M >= 0
// the eviction itself: a head with fill_M + 1 live tokens loses the lowest, and its
// last live row takes that slot.
__global__ __launch_bounds__(64) void one_plan(OnePlan pl, const int32_t* t, int32_t Hkv) {
  __shared__ int s_e;
  const int u = blockIdx.x, tid = threadIdx.x;
  const int n = min(max(pl.len[u], 0), pl.cap);
  const int s0 = pl.start ? min(max(pl.start[u], 0), pl.cap - 1) : 0;
  auto slot = [&](int i) { return s0 + i < pl.cap ? s0 + i : s0 + i - pl.cap; };
  const size_t row0 = (size_t)u * pl.cap;
  double lk = 0.0;
  int lp = 0;
  if (n > 0) {
    const size_t i = row0 + slot(n - 1);
    lp = pl.pos[i];
    lk = one_key(pl.log_beta != nullptr, t[u / Hkv] - lp, pl.log_beta ? pl.log_beta[i] : 0.f);
  }
  const OneCand own = one_plan_load(pl, u, tid);
  if (pl.fill_M < 0) {
    one_plan_head(pl, u, n, true, lk, lp, own, tid, 64, &s_e);
    return;
  }
  if (n != pl.fill_M + 1) {
    if (tid == 0 && pl.n_evicted) pl.n_evicted[u] = n <= pl.fill_M ? 0 : -(n - pl.fill_M);
    return;
  }
  double bk = own.key;
  int bp = own.pos, bs = own.slot;
  for (int i = tid + 64; i < pl.P; i += 64) {
    const OneCand c = pl.cand[(size_t)u * pl.P + i];
    one_better(bk, bp, bs, c.key, c.pos, c.slot);
  }
  if (tid == 0) one_better(bk, bp, bs, lk, lp, n - 1);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
    one_better(bk, bp, bs, __shfl_xor(bk, o, 64), __shfl_xor(bp, o, 64), __shfl_xor(bs, o, 64));
  const int e = min(max(bs, 0), n - 1);
  // the last live row moves into slot e (nothing moves when e is the last slot)
  if (e != n - 1) {
    const int se = slot(e), sl = slot(n - 1);
    const int ppr = pl.row_bytes / 16;
    for (int i = tid; i < 2 * ppr; i += 64) {
      unsigned char* tb = (unsigned char*)(i < ppr ? pl.k : pl.v) + row0 * pl.row_bytes;
      const int pc = i < ppr ? i : i - ppr;
      *(u32x4*)(tb + (size_t)se * pl.row_bytes + 16 * pc) =
          *(const u32x4*)(tb + (size_t)sl * pl.row_bytes + 16 * pc);
    }
    if (tid == 0) {
      if (pl.log_beta) pl.log_beta[row0 + se] = pl.log_beta[row0 + sl];
      pl.pos[row0 + se] = pl.pos[row0 + sl];
    }
  }
  if (tid == 0) {
    pl.len[u] = n - 1;
    if (pl.n_evicted) pl.n_evicted[u] = 1;
    if (pl.evicted_pos && pl.max_evict > 0) pl.evicted_pos[(size_t)u * pl.max_evict] = bp;
  }
}

void launch_one_plan(const kvb_cache* c, const int32_t* t, const OnePlan& p, hipStream_t s) {
  hipLaunchKernelGGL(one_plan, dim3(c->B * c->Hkv), dim3(64), 0, s, p, t, c->Hkv);
}

// ---------------------------------------------------------------- apply
struct ApplyArgs {
  void* k;
  void* v;
  float* log_beta;
  int32_t* pos;
  int32_t* len;
  int32_t* start;
  int32_t* evicted_pos;
  int32_t* n_out;
  const OneInfo* info;
  const unsigned char* scratch;  // [U][SC][srow]
  int32_t cap, M, max_evict, row_bytes, srow, R, SC;
};

// Chunk c (blockIdx.x) of head u (blockIdx.y): source rows [lo, hi) move one slot
// (up: +1, toward the last slot; down: -1).  Thread layout as in compact_move:
// piece column tid % cols fixed per thread, rows tid / cols + q * rpp.  Chunk 0
// also sets the head's len, start and outputs (it is the only writer of slot e).
__global__ __launch_bounds__(kShiftThreads) __attribute__((amdgpu_waves_per_eu(8)))
void one_shift(ApplyArgs a) {
  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const OneInfo inf = a.info[u];
  const int n = min(max(inf.n, 0), a.cap);
  if (n != a.M + 1) {  // nothing to evict (n <= M), or more than one (n > M + 1)
    if (c == 0 && tid == 0 && a.n_out) a.n_out[u] = n <= a.M ? 0 : -(n - a.M);
    return;
  }
  // the planner's rule, recomputed from its e and first slot (so every index below
  // stays inside the cache and the scratch whatever the workspace holds)
  const int e = min(max(inf.e, 0), n - 1);
  const int s0 = min(max(inf.s0, 0), a.cap - 1);
  auto slot = [&](int i) { return s0 + i < a.cap ? s0 + i : s0 + i - a.cap; };
  const size_t row0 = (size_t)u * a.cap;
  const bool up = a.start != nullptr && e < n - 1 - e;
  const int moved = up ? e : n - 1 - e;
  const int nch = (moved + a.R - 1) / a.R;
  int32_t epos = 0;
  if (c == 0 && tid == 0) epos = a.pos[row0 + slot(e)];  // before slot e is written
  if (c == 0 && tid == 0) {
    if (a.n_out) a.n_out[u] = 1;
    a.len[u] = n - 1;
    if (up) a.start[u] = s0 + 1 < a.cap ? s0 + 1 : 0;
  }
  if (c < nch) {
    int lo, hi;
    if (up) {
      hi = e - c * a.R;
      lo = max(hi - a.R, 0);
    } else {
      lo = e + 1 + c * a.R;
      hi = min(lo + a.R, n);
    }
    const int rows = hi - lo;
    // the source row the next chunk's destinations take, staged by the plan
    const bool has_stage = c + 1 < nch;
    const int brow = up ? lo : hi - 1;
    const int dir = up ? 1 : -1;
    const int ppr = a.row_bytes / 16;
    const int cols = 2 * ppr;
    const int rpp = kShiftThreads / cols;
    const int col = tid % cols, r0 = tid / cols;
    const bool isv = col >= ppr;
    const int pc = isv ? col - ppr : col;
    unsigned char* tb = (unsigned char*)(isv ? a.v : a.k) + row0 * a.row_bytes;
    const unsigned char* st = a.scratch + ((size_t)u * a.SC + c) * a.srow;
    u32x4 buf[kShiftPieces];
#pragma unroll
    for (int q = 0; q < kShiftPieces; ++q) {
      const int row = r0 + q * rpp;
      buf[q] = u32x4{0u, 0u, 0u, 0u};
      if (r0 < rpp && row < rows) {
        const int src = lo + row;
        const unsigned char* from = (has_stage && src == brow)
                                        ? st + (isv ? a.row_bytes : 0) + 16 * pc
                                        : tb + (size_t)slot(src) * a.row_bytes + 16 * pc;
        buf[q] = __builtin_nontemporal_load((const u32x4*)from);
      }
    }
    int32_t tl = 0, tp = 0;
    if (tid < rows) {
      const int src = lo + tid;
      if (has_stage && src == brow) {
        const int32_t* t2 = (const int32_t*)(st + 2 * a.row_bytes);
        tl = t2[0];
        tp = t2[1];
      } else {
        tl = a.log_beta ? __float_as_int(a.log_beta[row0 + slot(src)]) : 0;
        tp = a.pos[row0 + slot(src)];
      }
    }
    // every source of the chunk in registers before any destination is written
    wait_vmem_all();
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kShiftPieces; ++q) {
      const int row = r0 + q * rpp;
      if (r0 < rpp && row < rows)
        *(u32x4*)(tb + (size_t)slot(lo + row + dir) * a.row_bytes + 16 * pc) = buf[q];
    }
    if (tid < rows) {
      const int dst = slot(lo + tid + dir);
      if (a.log_beta) a.log_beta[row0 + dst] = __int_as_float(tl);
      a.pos[row0 + dst] = tp;
    }
  }
  if (c == 0 && tid == 0 && a.evicted_pos && a.max_evict > 0)
    a.evicted_pos[(size_t)u * a.max_evict] = epos;
}

}  // namespace kvb

using namespace kvb;

extern "C" size_t kv_evict_one_workspace(const kvb_cache* cache, int32_t num_splits) {
  if (check_cache(cache, false) != KVB_OK || num_splits < 0 || num_splits > 4096) return 0;
  const int32_t P = num_splits > 0 ? num_splits : kv_attn_decode_splits(cache, cache->Hkv);
  const OneLayout L = one_layout(cache);
  return L.cand + align_up((size_t)cache->B * cache->Hkv * P * sizeof(OneCand), 256);
}

extern "C" int32_t kv_evict_one_apply(const kvb_cache* cache, const int32_t* t, int32_t M,
                                      int32_t* evicted_pos, int32_t max_evict,
                                      int32_t* n_evicted, void* ws, size_t ws_bytes,
                                      void* stream) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (!t || M < 0 || max_evict < 0) return KVB_EINVAL;
  const OneLayout L = one_layout(cache);
  const size_t U = (size_t)cache->B * cache->Hkv;
  if (U > 65535) return KVB_EUNSUPPORTED;
  if (!ws || ws_bytes < L.cand) return KVB_EWORKSPACE;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  ApplyArgs a;
  a.k = cache->k;
  a.v = cache->v;
  a.log_beta = cache->log_beta;
  a.pos = cache->pos;
  a.len = cache->len;
  a.start = cache->start;
  a.evicted_pos = evicted_pos;
  a.n_out = n_evicted;
  a.info = (const OneInfo*)((char*)ws + L.info);
  a.scratch = (const unsigned char*)ws + L.scratch;
  a.cap = cache->cap;
  a.M = M;
  a.max_evict = max_evict;
  a.row_bytes = L.row_bytes;
  a.srow = L.srow;
  a.R = L.R;
  a.SC = L.SC;
  TraceScope tr(kTrOneShift, s);
  hipLaunchKernelGGL(one_shift, dim3(L.X, (unsigned)U), dim3(kShiftThreads), 0, s, a);
  return launch_status();
}
