// Retention-score eviction to a budget, MEMENTO range erasure, and the stable
// in-place compaction both share.
//
// Eviction ("Cache What Lasts", section 2.2, inference): a head holding n > M
// tokens loses the n - M with the lowest retention score beta_i^(t-i).  Tokens
// are ranked by kappa_i = (t - pos_i) * log beta_i (the log of that score,
// computed exactly in double: a <= 30-bit integer times a 24-bit significand),
// ties broken by lower position first.  Erasure ("MEMENTO: Teaching LLMs to
// Manage Their Own Context", blocks and compression; system engineering) drops
// every slot whose position lies in one of the sequence's half-open ranges.
//
// Kernels
//   sel_init, sel_hist0, sel_refine x2, sel_finish
//                  (heads too long for the LDS planner) find the threshold element
//                  (kappa*, slot*) -- the (n-M)-th in (kappa, slot) order -- by radix
//                  passes on the float32-rounded key (a monotone map of kappa), many
//                  workgroups per head, until the bucket holding it has at most 4096
//                  members, whose slots are listed and the selection finished in
//                  LDS on their exact keys; if more than 4096 share the 22-bit
//                  bucket, exact passes on the 64-bit key and a slot pass over the
//                  head.  The result: a keep bit per slot, kept slots per chunk.
//   keep_count     (erase) per 4096-slot chunk: number of kept slots.
//   keep_emit      per chunk: exclusive scan -> destination slot of every kept
//                  row (keep_src[dst] = src); evicted positions; rows whose source
//                  would be overwritten by another workgroup's writes are copied
//                  to scratch first (see compact_move).
//   compact_move   per group of MOVE_ROWS destination rows: read every source row
//                  (from the cache, or from scratch for staged rows), barrier, write.
//
// In-place safety: kept row j moves from slot os + src_j to slot ns + j (os, ns: the
// head's first live slot before and after; equal unless the head has a start array
// and is compacted toward its last slot, ns = os + evicted; slots count around the
// head's ring).  A workgroup owns the destination rows [j0, j0 + R); the only rows
// it writes are its own.  Toward the first slot (src_j >= j) a source can be
// clobbered only inside a later group's destination range; toward the last slot
// (src_j <= j + evicted) only inside an earlier group's.  Those sources are staged
// to scratch by the planner (staged_row), before any move starts.  Sources inside
// the group's own range are read before the barrier.
#include <string.h>

#include "common.h"

namespace kvb {


constexpr int kChunk = 4096;      // slots per keep_count / keep_emit workgroup
constexpr int kChunkThreads = 256;
constexpr int kPerThread = kChunk / kChunkThreads;
constexpr int kSelThreads = 1024;
// byte offset of the erase path's largest-kept-count word in the workspace header
constexpr size_t kWsMaxKept = 128;

// ---------------------------------------------------------------- keys
// A head's per-slot array seen from its first live slot: index i is i slots past
// it, continuing at the start of the head's slots once i reaches capu = cap - first
// slot.
template <typename T>
struct Ring {
  T* p;
  int capu, cap;
  __device__ __forceinline__ T& operator[](int i) const { return p[i < capu ? i : i - cap]; }
  // the same element read with the non-temporal (streaming) hint: whole-head scans
  __device__ __forceinline__ T ld(int i) const {
    return __builtin_nontemporal_load(&p[i < capu ? i : i - cap]);
  }
  __device__ __forceinline__ explicit operator bool() const { return p != nullptr; }
};

template <typename LB, typename PS>
__device__ __forceinline__ double retention_key(const LB& lb, const PS& ps, int i, int tq) {
  if (!lb) return 0.0;
  const int d = tq - ps[i];
  if (d == 0) return 0.0;
  return (double)d * (double)lb[i];
}

// Order-preserving maps of a double / float to unsigned integers (+0 and -0
// map to the same value).
__device__ __forceinline__ uint64_t ord64(double k) {
  uint64_t b = (uint64_t)__double_as_longlong(k);
  if ((b << 1) == 0) b = 0;
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ __forceinline__ uint32_t ord32f(float k) {
  uint32_t b = __float_as_uint(k);
  if ((b << 1) == 0) b = 0;
  return (b >> 31) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ uint32_t ord32(double k) {
  return ord32f((float)k);  // round to nearest: monotone in k
}
// Inverse of ord64 (up to the sign of zero).
__device__ __forceinline__ double unord64(uint64_t o) {
  const uint64_t b = (o >> 63) ? (o & 0x7fffffffffffffffull) : ~o;
  return __longlong_as_double((long long)b);
}

// The retention key d * log beta (d = t - pos) and its float32 rounding.  The
// exact key is the double product (exact while |d| < 2^29).  For |d| <= 2^24, d is
// exact in float32 and one float32 multiply rounds the exact product once, which
// is what rounding the double product to float32 does; so the float32 key, which all
// the radix passes look at, costs one float multiply.  No log beta (lb null):
// every key is 0.
template <typename LB>
__device__ __forceinline__ double key_f64(const LB& lb, int d, float b) {
  return (!lb || d == 0) ? 0.0 : (double)d * (double)b;
}
template <typename LB>
__device__ __forceinline__ uint32_t key_ord32(const LB& lb, int d, float b) {
  if (!lb || d == 0) return 0x80000000u;  // ord32f(0)
  if (d <= (1 << 24) && d >= -(1 << 24)) return ord32f((float)d * b);
  return ord32((double)d * (double)b);
}
// key_ord32 of a thread's N slots: the float multiply for all, then (only in a
// wave holding one) the distances beyond 2^24 from the double product.
template <int N, typename LB>
__device__ __forceinline__ void keys_ord32(const LB& lb, const int* d, const float* b,
                                           uint32_t* k) {
  bool far = false;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    k[e] = (!lb || d[e] == 0) ? 0x80000000u : ord32f((float)d[e] * b[e]);
    far |= d[e] > (1 << 24) || d[e] < -(1 << 24);
  }
  if (__ballot(far) != 0) {
#pragma unroll
    for (int e = 0; e < N; ++e)
      if (d[e] > (1 << 24) || d[e] < -(1 << 24)) k[e] = key_ord32(lb, d[e], b[e]);
  }
}

// ---------------------------------------------------------------- block helpers
template <int NT>
__device__ __forceinline__ int block_excl_scan(int x, int* smem, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) smem[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int i = 0; i < NT / 64; ++i) {
      s += smem[i];
      smem[i] = s;
    }
  }
  __syncthreads();
  const int off = w > 0 ? smem[w - 1] : 0;
  total = smem[NT / 64 - 1];
  __syncthreads();
  return off + v - x;
}

template <int NT>
__device__ __forceinline__ int block_sum(int x, int* smem) {
  int total;
  (void)block_excl_scan<NT>(x, smem, total);
  return total;
}

// Find the histogram bucket holding the r-th (1-based) element; returns the bucket
// and replaces r by the rank inside it.  hist has nb bins (nb <= 2 * NT).
template <int NT>
__device__ __forceinline__ int select_bucket(const uint32_t* hist, int nb, int& r, int* smem,
                                             int* out) {
  const int per = (nb + NT - 1) / NT;
  const int b0 = threadIdx.x * per;
  int c = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < nb) c += (int)hist[b0 + i];
  int total;
  const int excl = block_excl_scan<NT>(c, smem, total);
  if (r > excl && r <= excl + c) {
    int acc = excl;
    for (int i = 0; i < per; ++i) {
      const int h = (int)hist[b0 + i];
      if (r <= acc + h) {
        out[0] = b0 + i;
        out[1] = r - acc;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
  const int bucket = min(max(out[0], 0), nb - 1);  // always found when r <= count
  r = out[1];
  __syncthreads();
  return bucket;
}

// The blocks of bsz slots of an n-slot head that workgroup x takes: block x, and
// (with fold) the last workgroup with work also takes the head's last block when
// that one is short (at most bsz / 4 slots), so that a head a few slots past a
// multiple of bsz does not need one more workgroup, which would wait for a free
// slot on the chip when the grid exceeds what the chip holds at once.  (The
// selection kernels fit a 128K-slot layer at once, where the folded workgroup's
// second pass costs more than it saves.)  Returns (first, last); last < first: no
// work.
__device__ __forceinline__ int2 wg_blocks(int x, int n, int bsz, bool fold_short = true) {
  const int nb = (n + bsz - 1) / bsz;
  const bool fold = fold_short && nb >= 2 && n - (nb - 1) * bsz <= bsz / 4;
  const int lastwg = fold ? nb - 2 : nb - 1;
  if (x > lastwg) return make_int2(0, -1);
  return make_int2(x, x == lastwg ? nb - 1 : x);
}

// ---------------------------------------------------------------- select
// Chunked selection for heads too long for the LDS planner.  Several workgroups
// per head (slices of kSelSlice slots): a histogram pass of the top 11 bits of
// the float32-rounded key (sel_hist0) added into a per-head global histogram;
// then two refine launches.  Each refine workgroup loads its slice's keys, replays
// the earlier passes' bucket choices from the global histograms while the loads
// are in flight (deterministic, so no launch in between is needed), and either
// lists the slots of the bucket holding the threshold once it has at most
// kSelCand members (recording the level in the head's SelHead, and marking the
// slots above the bucket in the head's keep bits), or adds the next 11-bit
// histogram pass.  A refine launch after the listing one reads that record and
// exits.  (Letting the last workgroup of a pass record the choice instead needs a
// device-wide release fence in every workgroup, which writes back the L2 of its
// XCD and made the pass several times slower.)  One workgroup per head then
// finishes the selection from the list in LDS and marks the bucket's kept
// members; if more than kSelCand keys share the 22-bit bucket, that workgroup
// runs exact passes over the whole head instead.
constexpr int kSelB = 16;       // slots per thread per round
constexpr int kSelCand = 4096;  // bucket size finished from a list
constexpr int kSelNT = 256;     // threads of the slice kernels
constexpr int kSelRounds = 2;   // rounds per slice workgroup
constexpr int kSelRefines = 2;  // refine launches (histogram passes of 11 + 11 bits)
constexpr int kSelHistWords = kSelRefines * 2048;  // per head: pass p's bins at p * 2048
constexpr int kSelSlice = kSelRounds * kSelNT * kSelB;  // slots per slice workgroup
static_assert(kSelNT * kSelB == kChunk, "a round covers one keep_emit chunk");

struct SelHead {      // per head
  int32_t nlist;      // members listed
  int32_t level;      // the refine launch that listed them (0: not listed)
  uint32_t prefix;    // the bucket listed: its top pbits bits of the float32 key
  int32_t pbits, r, cnt;  // rank of the threshold inside it, its size
  int32_t pad[2];
};

struct SelArgs {
  const float* log_beta;
  const int32_t* pos;
  const int32_t* len;
  const int32_t* start;
  const int32_t* tq;
  uint32_t* hist;        // [U][kSelRefines][2048]
  SelHead* head;         // [U]
  int32_t* ls;           // [U][kSelCand] the listed slots
  UnitInfo* info;
  int32_t* n_out;
  int32_t* counts;       // [U][C] kept slots per kChunk-slot chunk (for keep_emit)
  uint32_t* keepbits;    // [U][W] bit i % 32 of word i / 32: slot i is kept
  int32_t cap, Hkv, M, C, W;
};

// Distances d = t - pos and log betas of the slots base + e * NT + tid, e < kSelB:
// every load of the round is issued before any is used.  Slots past n repeat slot
// n - 1 (callers skip them).
template <int NT, typename LB, typename PS>
__device__ __forceinline__ void sel_load(const LB& lb, const PS& ps, int base, int n, int tpos,
                                         int* d, float* b) {
#pragma unroll
  for (int e = 0; e < kSelB; ++e) {
    const int i = min(base + e * NT + (int)threadIdx.x, n - 1);
    d[e] = ps.ld(i);
    b[e] = lb ? lb.ld(i) : 0.f;
  }
#pragma unroll
  for (int e = 0; e < kSelB; ++e) d[e] = tpos - d[e];
}

// Whether float32-ordered key k32 starts with the pbits-bit prefix.
__device__ __forceinline__ bool has_prefix(uint32_t k32, uint32_t prefix, int pbits) {
  return pbits == 0 || (pbits == 32 ? k32 : (k32 >> (32 - pbits))) == prefix;
}

struct SelPos {
  uint32_t prefix;  // the fixed top pbits bits of the float32 key
  int pbits;
  int r;    // 1-based rank of the threshold among the keys with that prefix
  int cnt;  // keys with that prefix
  // the prefix as a mask and value over the whole key: k32 has the prefix iff
  // (k32 & pmask) == pval, and lies in a higher bucket iff (k32 & pmask) > pval
  __device__ __forceinline__ uint32_t pmask() const { return pbits == 0 ? 0u : ~0u << (32 - pbits); }
  __device__ __forceinline__ uint32_t pval() const { return pbits == 0 ? 0u : prefix << (32 - pbits); }
};

// The bucket choices of passes 0 .. upto-1, from the head's histograms (whole
// workgroup; stops early once the bucket is small enough to list).
template <int NT>
__device__ SelPos sel_replay(const uint32_t* gh, int upto, int n, int M, int* smem, int* out) {
  SelPos sp = {0u, 0, n - M, n};
  for (int p = 0; p < upto && sp.cnt > kSelCand; ++p) {
    const int width = p == 2 ? 10 : 11;
    const uint32_t* h = gh + p * 2048;
    const int b = select_bucket<NT>(h, 1 << width, sp.r, smem, out);
    sp.cnt = (int)h[b];
    sp.prefix = (sp.prefix << width) | (uint32_t)b;
    sp.pbits += width;
  }
  return sp;
}

// Clears the head's histograms, record and chunk counts.
__global__ __launch_bounds__(kSelNT) void sel_init(SelArgs a) {
  const int u = blockIdx.x;
  for (int i = threadIdx.x; i < kSelHistWords; i += kSelNT) a.hist[(size_t)u * kSelHistWords + i] = 0u;
  for (int i = threadIdx.x; i < a.C; i += kSelNT) a.counts[(size_t)u * a.C + i] = 0;
  if (threadIdx.x < (int)(sizeof(SelHead) / 4)) ((int32_t*)(a.head + u))[threadIdx.x] = 0;
}

// The slice's keys, all loads in flight at once: round rr holds slots base0 +
// rr * kChunk + e * kSelNT + tid.
template <typename LB, typename PS>
__device__ __forceinline__ void slice_load(const LB& lb, const PS& ps, int base0, int n, int tpos,
                                           int (&d)[kSelRounds][kSelB],
                                           float (&b)[kSelRounds][kSelB]) {
#pragma unroll
  for (int rr = 0; rr < kSelRounds; ++rr) {
#pragma unroll
    for (int e = 0; e < kSelB; ++e) {
      const int i = min(base0 + rr * kChunk + e * kSelNT + (int)threadIdx.x, n - 1);
      d[rr][e] = ps.ld(i);
      b[rr][e] = lb ? lb.ld(i) : 0.f;
    }
  }
#pragma unroll
  for (int rr = 0; rr < kSelRounds; ++rr)
#pragma unroll
    for (int e = 0; e < kSelB; ++e) d[rr][e] = tpos - d[rr][e];
}

// Adds the slice's keys with the given prefix to the head's histogram of the
// width bits below it (LDS first, then one global add per non-empty bin).  (Four
// copies of every bin, to spread a wave's same-bin atomics, made the pass slower:
// the larger LDS footprint costs more occupancy than the conflicts it saves.)
__device__ __forceinline__ void slice_hist(const uint32_t (&k)[kSelRounds][kSelB], int base0,
                                           int n, const SelPos& sp, int width, uint32_t* h,
                                           uint32_t* gh) {
  const int tid = threadIdx.x;
  const int nb = 1 << width;
  const int shift = 32 - sp.pbits - width;
  const uint32_t pm = sp.pmask(), pv = sp.pval();
  for (int i = tid; i < nb; i += kSelNT) h[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < kSelRounds; ++rr)
#pragma unroll
    for (int e = 0; e < kSelB; ++e) {
      if (base0 + rr * kChunk + e * kSelNT + tid >= n || (k[rr][e] & pm) != pv) continue;
      atomicAdd(&h[(k[rr][e] >> shift) & (uint32_t)(nb - 1)], 1u);
    }
  __syncthreads();
  for (int i = tid; i < nb; i += kSelNT)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// The float32-ordered keys of the loaded slots.
template <typename LB>
__device__ __forceinline__ void slice_keys(const LB& lb, const int (&d)[kSelRounds][kSelB],
                                           const float (&b)[kSelRounds][kSelB],
                                           uint32_t (&k)[kSelRounds][kSelB]) {
#pragma unroll
  for (int rr = 0; rr < kSelRounds; ++rr) keys_ord32<kSelB>(lb, d[rr], b[rr], k[rr]);
}

// Pass 0: the top 11 bits of every key of the workgroup's slices.  Heads of at
// most kSelCand slots are listed whole by the first refine launch.
// (At most 96 registers, so that five workgroups fit a compute unit and every
// slice of a 128K-slot layer is resident at once.)
__global__ __launch_bounds__(kSelNT) __attribute__((amdgpu_waves_per_eu(5, 8))) void sel_hist0(SelArgs a) {
  __shared__ uint32_t h[2048];
  const int u = blockIdx.y;
  const int n = min(a.len[u], a.cap);
  const int2 br = wg_blocks(blockIdx.x, n, kSelSlice, false);
  if (n <= a.M || n <= kSelCand || br.y < br.x) return;
  const int s0 = head_start(a.start, u);
  const Ring<const float> lb{a.log_beta ? a.log_beta + (size_t)u * a.cap + s0 : nullptr,
                             a.cap - s0, a.cap};
  const Ring<const int32_t> ps{a.pos + (size_t)u * a.cap + s0, a.cap - s0, a.cap};
  const SelPos sp = {0u, 0, 0, n};
#pragma unroll 1
  for (int blk = br.x; blk <= br.y; ++blk) {
    int d[kSelRounds][kSelB];
    float b[kSelRounds][kSelB];
    slice_load(lb, ps, blk * kSelSlice, n, a.tq[u / a.Hkv], d, b);
    uint32_t k[kSelRounds][kSelB];
    slice_keys(lb, d, b, k);
    slice_hist(k, blk * kSelSlice, n, sp, 11, h, a.hist + (size_t)u * kSelHistWords);
  }
}

// Refine launch `pass` (1, 2) over the workgroup's slices: lists the slots of
// the threshold's bucket if it is small enough after the first `pass` passes (and
// no earlier launch listed it), else adds histogram pass `pass`.  The list goes
// to LDS first and takes one global reservation per workgroup (a per-head counter
// taking every wave's reservation serialises at one address); members past the
// LDS list take a global reservation per wave.  The listing launch also stores,
// per kChunk-slot chunk, the slots whose key lies above the bucket (kept whatever
// the threshold inside it; sel_finish adds the bucket's kept members).  Only the
// float32 keys stay in registers once formed; sel_finish forms the members' exact
// keys.  (At most 96 registers, as sel_hist0.)
constexpr int kCollectLds = 2048;
__global__ __launch_bounds__(kSelNT) __attribute__((amdgpu_waves_per_eu(5, 8))) void sel_refine(SelArgs a, int pass) {
  __shared__ int smem[kSelNT / 64];
  __shared__ int out[4];
  __shared__ __align__(16) uint32_t lds[2048];  // the histogram, or the list
  static_assert(kCollectLds <= 2048, "the list fits the histogram's space");
  int* cs = (int*)lds;
  __shared__ int nloc, gbase;
  const int u = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int n = min(a.len[u], a.cap);
  const int2 br = wg_blocks(blockIdx.x, n, kSelSlice, false);
  if (n <= a.M || br.y < br.x) return;
  const int lvl = a.head[u].level;
  if (lvl != 0 && lvl < pass) return;  // listed by an earlier launch
  const int s0 = head_start(a.start, u);
  const Ring<const float> lb{a.log_beta ? a.log_beta + (size_t)u * a.cap + s0 : nullptr,
                             a.cap - s0, a.cap};
  const Ring<const int32_t> ps{a.pos + (size_t)u * a.cap + s0, a.cap - s0, a.cap};
  const int tpos = a.tq[u / a.Hkv];
  int d[kSelRounds][kSelB];
  float b[kSelRounds][kSelB];
  slice_load(lb, ps, br.x * kSelSlice, n, tpos, d, b);  // in flight during the replay
  if (tid == 0) nloc = 0;
  uint32_t* gh = a.hist + (size_t)u * kSelHistWords;
  const SelPos sp = sel_replay<kSelNT>(gh, pass, n, a.M, smem, out);
  __syncthreads();  // nloc cleared (the replay may take no pass)
  // more than kSelCand keys share one float32 key after the last pass: sel_finish
  // takes the head
  const bool listing = sp.cnt <= kSelCand;
  if (!listing && pass == kSelRefines) return;
  if (listing && blockIdx.x == 0 && tid == 0) {
    SelHead* hd = a.head + u;
    hd->level = pass;
    hd->prefix = sp.prefix;
    hd->pbits = sp.pbits;
    hd->r = sp.r;
    hd->cnt = sp.cnt;
  }
  constexpr int kCps = kSelSlice / kChunk;  // chunks per slice
  const uint32_t pm = sp.pmask(), pv = sp.pval();
  for (int blk = br.x;;) {
    const int base0 = blk * kSelSlice;
    uint32_t k[kSelRounds][kSelB];
    slice_keys(lb, d, b, k);
    if (!listing) {
      slice_hist(k, base0, n, sp, pass == 2 ? 10 : 11, lds, gh + pass * 2048);
    } else {
      int above[kCps];
#pragma unroll
      for (int rr = 0; rr < kCps; ++rr) above[rr] = 0;
#pragma unroll
      for (int rr = 0; rr < kCps; ++rr) {
        const int base = base0 + rr * kChunk;
        if (base >= n) break;
        uint32_t mbits = 0;  // bit e: slot base + e * kSelNT + tid is a member
#pragma unroll
        for (int e = 0; e < kSelB; ++e) {
          const bool live = base + e * kSelNT + tid < n;
          const uint32_t kp = k[rr][e] & pm;
          mbits |= (live && kp == pv) ? 1u << e : 0u;
          // keys above the bucket: kept (sel_finish adds the bucket's kept members)
          const unsigned long long ab = __ballot(live && kp > pv);
          above[rr] += (live && kp > pv) ? 1 : 0;
          const int w0 = (base + e * kSelNT + (tid & ~63)) >> 5;
          if (lane == 0 && w0 + 1 < a.W) {
            uint32_t* kb = a.keepbits + (size_t)u * a.W + w0;
            kb[0] = (uint32_t)ab;
            kb[1] = (uint32_t)(ab >> 32);
          } else if (lane == 0 && w0 < a.W) {
            a.keepbits[(size_t)u * a.W + w0] = (uint32_t)ab;
          }
        }
        // the wave's members take consecutive list positions: one reservation per
        // wave
        const int c = __popc(mbits);
        int incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o, 64);
          if (lane >= o) incl += y;
        }
        const int wtot = __shfl(incl, 63, 64);
        if (wtot == 0) continue;
        int wb = 0;
        if (lane == 63) wb = atomicAdd(&nloc, wtot);
        wb = __shfl(wb, 63, 64);
        // members whose LDS position lies past the list go straight to the head's
        // list (one reservation per wave); the LDS positions below kCollectLds are
        // all written, so the flush below copies min(nloc, kCollectLds) entries
        const int over = min(max(0, wb + wtot - kCollectLds), wtot);
        int gb = 0;
        if (over > 0 && lane == 63) gb = atomicAdd(&a.head[u].nlist, over);
        gb = __shfl(gb, 63, 64);
        int j = wb + incl - c;
#pragma unroll
        for (int e = 0; e < kSelB; ++e) {
          if (!((mbits >> e) & 1u)) continue;
          const int i = base + e * kSelNT + tid;
          if (j < kCollectLds) {
            cs[j] = i;
          } else {
            const int g = gb + (j - max(wb, kCollectLds));
            if (g < kSelCand) a.ls[(size_t)u * kSelCand + g] = i;  // always: cnt in all
          }
          ++j;
        }
      }
#pragma unroll
      for (int c = 0; c < kCps; ++c) {
        const int tot = block_sum<kSelNT>(above[c], smem);
        if (tid == 0 && base0 / kChunk + c < a.C) a.counts[(size_t)u * a.C + base0 / kChunk + c] = tot;
      }
    }
    if (++blk > br.y) break;
    slice_load(lb, ps, blk * kSelSlice, n, tpos, d, b);
  }
  if (!listing) return;
  __syncthreads();
  const int nl = min(nloc, kCollectLds);
  if (nl == 0) return;
  if (tid == 0) gbase = atomicAdd(&a.head[u].nlist, nl);
  __syncthreads();
  int32_t* ls = a.ls + (size_t)u * kSelCand;
  for (int j = tid; j < nl; j += kSelNT) {
    const int g = gbase + j;
    if (g < kSelCand) ls[g] = cs[j];  // always: exactly cnt members over all slices
  }
}

// One workgroup per head: the threshold (kappa*, slot*) from the list, or from
// exact passes over the head when more than kSelCand keys share its float32 key.
__global__ __launch_bounds__(kSelThreads) void sel_finish(SelArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ unsigned long long ck[kSelCand];
  __shared__ int cs[kSelCand];
  __shared__ unsigned long long kext[2];
  __shared__ unsigned long long wext[2][kSelThreads / 64];
  __shared__ int smem[kSelThreads / 64];
  __shared__ int out[4];
  const int u = blockIdx.x, tid = threadIdx.x;
  const int s0 = head_start(a.start, u);
  const int n = min(a.len[u], a.cap);
  const SelHead hd = a.head[u];  // issued early: its latency overlaps the checks below
  if (n <= a.M) {
    if (tid == 0) {
      UnitInfo z = {0ull, -1, MODE_NOOP, n, n, s0, s0};
      a.info[u] = z;
      if (a.n_out) a.n_out[u] = 0;
    }
    return;
  }
  if (tid == 0) {
    out[2] = -1;
    kext[0] = ~0ull;
    kext[1] = 0ull;
  }
  __syncthreads();
  // the listed bucket, or (none listed) the float32 key more than kSelCand share
  const SelPos sp = hd.level != 0
                        ? SelPos{hd.prefix, hd.pbits, hd.r, hd.cnt}
                        : sel_replay<kSelThreads>(a.hist + (size_t)u * kSelHistWords, kSelRefines, n,
                                                  a.M, smem, out);
  int r = sp.r;
  unsigned long long K;
  int sstar = -1;
  if (sp.cnt <= kSelCand) {
    // the r-th of the listed members in (key, slot) order: radix on the key below
    // the members' common top bits, then on the slot among equal keys
    const int nc = min(min(hd.nlist, sp.cnt), kSelCand);
    // every load in flight at once, then the smallest and largest key by wave
    // shuffles and one LDS slot per wave
    constexpr int kPer = kSelCand / kSelThreads;
    const Ring<const float> lb{a.log_beta ? a.log_beta + (size_t)u * a.cap + s0 : nullptr,
                               a.cap - s0, a.cap};
    const Ring<const int32_t> ps{a.pos + (size_t)u * a.cap + s0, a.cap - s0, a.cap};
    const int tpos = a.tq[u / a.Hkv];
    int sv[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int j = tid + e * kSelThreads;
      sv[e] = j < nc ? a.ls[(size_t)u * kSelCand + j] : 0;
    }
    int dv[kPer];
    float bv[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      dv[e] = ps[sv[e]];
      bv[e] = lb ? lb[sv[e]] : 0.f;
    }
    unsigned long long kv[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) kv[e] = ord64(key_f64(lb, tpos - dv[e], bv[e]));
    unsigned long long lo = ~0ull, hi = 0ull;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int j = tid + e * kSelThreads;
      if (j < nc) {
        ck[j] = kv[e];
        cs[j] = sv[e];
        lo = kv[e] < lo ? kv[e] : lo;
        hi = kv[e] > hi ? kv[e] : hi;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long l2 = __shfl_xor(lo, o, 64), h2 = __shfl_xor(hi, o, 64);
      lo = l2 < lo ? l2 : lo;
      hi = h2 > hi ? h2 : hi;
    }
    if ((tid & 63) == 0) {
      wext[0][tid >> 6] = lo;
      wext[1][tid >> 6] = hi;
    }
    __syncthreads();
    unsigned long long kmin = ~0ull, kmax = 0ull;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) {
      kmin = wext[0][w] < kmin ? wext[0][w] : kmin;
      kmax = wext[1][w] > kmax ? wext[1][w] : kmax;
    }
    K = kmin;
    bool unique = false;  // the bucket narrowed to one member: it is the threshold
    if (kmin != kmax) {
      int top = 63 - __clzll((long long)(kmin ^ kmax));  // highest differing bit
      unsigned long long pfx = top == 63 ? 0ull : kmin >> (top + 1);
      for (; top >= 0; top -= 11) {
        const int width = top + 1 < 11 ? top + 1 : 11;
        const int shift = top + 1 - width;
        for (int i = tid; i < 2048; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        for (int j = tid; j < nc; j += kSelThreads) {
          const unsigned long long k64 = ck[j];
          if (top == 63 || (k64 >> (top + 1)) == pfx)
            atomicAdd(&hist[(k64 >> shift) & ((1u << width) - 1u)], 1u);
        }
        __syncthreads();
        const int bk = select_bucket<kSelThreads>(hist, 1 << width, r, smem, out);
        pfx = (pfx << width) | (unsigned long long)bk;
        const bool one = hist[bk] == 1;
        __syncthreads();  // every count read before the next pass clears them
        if (one) {  // r == 1: the one member with this prefix
          for (int j = tid; j < nc; j += kSelThreads)
            if ((ck[j] >> shift) == pfx) out[2] = j;
          __syncthreads();
          K = ck[out[2]];
          sstar = cs[out[2]];
          unique = true;
          break;
        }
      }
      if (!unique) K = pfx;
    }
    // slot: the r-th smallest among the members whose key is K (slots < 2^30)
    uint32_t sp2 = 0;
    for (int pass = 0; pass < 3 && !unique; ++pass) {
      const int shift = 20 - 10 * pass;
      for (int i = tid; i < 1024; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int j = tid; j < nc; j += kSelThreads) {
        if (ck[j] != K) continue;
        const uint32_t sl = (uint32_t)cs[j];
        if (pass == 0 || (sl >> (shift + 10)) == sp2) atomicAdd(&hist[(sl >> shift) & 1023u], 1u);
      }
      __syncthreads();
      const int bk = select_bucket<kSelThreads>(hist, 1024, r, smem, out);
      sp2 = (sp2 << 10) | (uint32_t)bk;
    }
    if (!unique) sstar = (int)sp2;
    // the bucket's kept members into their chunks' counts (sel_refine wrote the
    // counts of the keys above the bucket): summed in LDS, then one add per chunk
    const bool in_lds = a.C <= 2048;
    if (in_lds) {
      for (int i = tid; i < a.C; i += kSelThreads) hist[i] = 0u;
      __syncthreads();
    }
    for (int j = tid; j < nc; j += kSelThreads)
      if (ck[j] > K || (ck[j] == K && cs[j] > sstar)) {
        atomicOr(&a.keepbits[(size_t)u * a.W + cs[j] / 32], 1u << (cs[j] & 31));
        if (in_lds) atomicAdd(&hist[cs[j] / kChunk], 1u);
        else atomicAdd(&a.counts[(size_t)u * a.C + cs[j] / kChunk], 1);
      }
    if (in_lds) {
      __syncthreads();
      for (int i = tid; i < a.C; i += kSelThreads)
        if (hist[i]) a.counts[(size_t)u * a.C + i] += (int)hist[i];
    }
  } else {
    // more than kSelCand keys share the threshold's bucket (the top sp.pbits bits
    // of the float32 key): the exact key by radix passes over the head (skipped
    // when those keys are all equal), then the slot of the r-th of its ties in
    // slot order
    const uint32_t pm = sp.pmask(), pv = sp.pval();
    const Ring<const float> lb{a.log_beta ? a.log_beta + (size_t)u * a.cap + s0 : nullptr,
                               a.cap - s0, a.cap};
    const Ring<const int32_t> ps{a.pos + (size_t)u * a.cap + s0, a.cap - s0, a.cap};
    const int tpos = a.tq[u / a.Hkv];
    unsigned long long lo = ~0ull, hi = 0ull;
    for (int base = 0; base < n; base += kSelThreads * kSelB) {
      int dd[kSelB];
      float bb[kSelB];
      sel_load<kSelThreads>(lb, ps, base, n, tpos, dd, bb);
#pragma unroll
      for (int e = 0; e < kSelB; ++e) {
        if (base + e * kSelThreads + tid >= n || (key_ord32(lb, dd[e], bb[e]) & pm) != pv) continue;
        const unsigned long long k64 = ord64(key_f64(lb, dd[e], bb[e]));
        lo = k64 < lo ? k64 : lo;
        hi = k64 > hi ? k64 : hi;
      }
    }
    if (lo != ~0ull) {
      atomicMin(&kext[0], lo);
      atomicMax(&kext[1], hi);
    }
    __syncthreads();
    K = kext[0];
    if (K != kext[1]) {
      unsigned long long pfx = 0;
      for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        for (int base = 0; base < n; base += kSelThreads * kSelB) {
          int dd[kSelB];
          float bb[kSelB];
          sel_load<kSelThreads>(lb, ps, base, n, tpos, dd, bb);
#pragma unroll
          for (int e = 0; e < kSelB; ++e) {
            if (base + e * kSelThreads + tid >= n || (key_ord32(lb, dd[e], bb[e]) & pm) != pv) continue;
            const unsigned long long k64 = ord64(key_f64(lb, dd[e], bb[e]));
            if (pass == 0 || (k64 >> (shift + 8)) == pfx)
              atomicAdd(&hist[(k64 >> shift) & 255u], 1u);
          }
        }
        __syncthreads();
        const int bk = select_bucket<kSelThreads>(hist, 256, r, smem, out);
        pfx = (pfx << 8) | (unsigned long long)bk;
      }
      K = pfx;
    }
    // a round's ties are counted at once; only the round holding the r-th is
    // walked in slot order (row e of a round = slots base + e * kSelThreads + tid)
    int seen = 0;
    for (int base = 0; base < n && sstar < 0; base += kSelThreads * kSelB) {
      int dd[kSelB];
      float bb[kSelB];
      sel_load<kSelThreads>(lb, ps, base, n, tpos, dd, bb);
      bool f[kSelB];
      int c = 0;
#pragma unroll
      for (int e = 0; e < kSelB; ++e) {
        f[e] = base + e * kSelThreads + tid < n && ord64(key_f64(lb, dd[e], bb[e])) == K;
        c += f[e] ? 1 : 0;
      }
      const int total = block_sum<kSelThreads>(c, smem);
      if (seen + total < r) {
        seen += total;
        continue;
      }
      for (int e = 0; e < kSelB; ++e) {
        int tot_e;
        const int excl = block_excl_scan<kSelThreads>(f[e] ? 1 : 0, smem, tot_e);
        if (f[e] && seen + excl + 1 == r) out[2] = base + e * kSelThreads + tid;
        __syncthreads();
        if (seen + tot_e >= r) {
          sstar = out[2];
          break;
        }
        seen += tot_e;
      }
    }
    // kept slots (sel_refine did not mark them for this head): their bits, and
    // their number per chunk counted in LDS for windows of 2048 chunks
    uint32_t* cc = hist;
    for (int cw = 0; cw < a.C; cw += 2048) {
      for (int i = tid; i < 2048; i += kSelThreads) cc[i] = 0u;
      __syncthreads();
      const int lo = cw * kChunk, hi2 = min(n, (cw + 2048) * kChunk);
      for (int base = lo; base < hi2; base += kSelThreads * kSelB) {
        int dd[kSelB];
        float bb[kSelB];
        sel_load<kSelThreads>(lb, ps, base, hi2, tpos, dd, bb);
#pragma unroll
        for (int e = 0; e < kSelB; ++e) {
          const int i = base + e * kSelThreads + tid;
          bool kept = false;
          if (i < hi2) {
            const unsigned long long k64 = ord64(key_f64(lb, dd[e], bb[e]));
            kept = k64 > K || (k64 == K && i > sstar);
            if (kept) atomicAdd(&cc[i / kChunk - cw], 1u);
          }
          const unsigned long long kb = __ballot(kept);  // the wave's 64 slots
          const int w0 = (i - (tid & 63)) >> 5;
          if ((tid & 63) == 0 && i < hi2) {
            a.keepbits[(size_t)u * a.W + w0] = (uint32_t)kb;
            if (w0 + 1 < a.W) a.keepbits[(size_t)u * a.W + w0 + 1] = (uint32_t)(kb >> 32);
          }
        }
      }
      __syncthreads();
      for (int c = tid; c < 2048 && cw + c < a.C; c += kSelThreads)
        a.counts[(size_t)u * a.C + cw + c] = (int)cc[c];
      __syncthreads();
    }
  }
  if (tid == 0) {
    UnitInfo v = {K, sstar, MODE_EVICT, n, a.M, s0, s0};
    a.info[u] = v;
  }
}

// ---------------------------------------------------------------- staging rule
// Kept row j moves from slot os + src (os: the head's first live slot before the
// compaction) to slot ns + j (ns: after it).  compact_move's workgroups own groups
// of mr destinations and write only those; a source that lies inside another
// group's destination range could be overwritten before it is read, so it is
// copied to scratch (by destination index) before any move starts.  Moving toward
// the head's first slot (ns <= os, src >= j) the endangered sources lie in later
// groups' ranges, below ns + kept; moving toward the end (ns > os, src <= j) in
// earlier groups' ranges, at or above ns.
__device__ __forceinline__ bool staged_row(int os, int ns, int src, int j, int kept, int mr) {
  const int sa = os + src, da = ns + j;
  if (sa == da) return false;
  const int g0 = ns + (j / mr) * mr;  // the group's first destination slot
  if (ns <= os) return sa >= g0 + mr && sa < ns + kept;
  return sa < g0 && sa >= ns;
}



// ---------------------------------------------------------------- fused LDS planner
// One 1024-thread workgroup per head, for heads whose float32-rounded keys fit in
// LDS (gfx950: 160 KB).  Same selection as evict_select, then the head's own scan:
// keep flags in slot order -> destination of every kept row (keep_src), evicted
// positions, and staging of cross-workgroup hazard rows -- no chunk kernels needed.
// Keys sit at LDS index i + i/32 so that both the strided passes and the
// per-thread contiguous ranges of the scan are free of bank conflicts.
__device__ __forceinline__ int skew(int i) { return i + (i >> 5); }

struct PlanArgs {
  const float* log_beta;
  const int32_t* pos;
  const int32_t* len;
  const int32_t* start;  // [U] or null
  const int32_t* tq;
  UnitInfo* info;
  int32_t* keep_src;
  int32_t* evicted_pos;
  int32_t* n_out;
  unsigned char* scratch;
  uint32_t* tile_mask;  // [U][Tc]
  int32_t* tile_base;   // [U][Tc]
  int32_t* stage_n;     // [U]
  int2* stage_list;     // [U][Mk]: every kept row below za that moves (fused apply)
  int2* copy_list;      // [U][Mk]: the subset compact_move reads from scratch
  const void* k;
  const void* v;
  int32_t cap, Hkv, M, Mk, max_evict, row_bytes, srow, move_rows, za, Tc;
  int32_t vec;  // capacity % 4 == 0: log beta and pos read 16 bytes at a time
};

constexpr int kCand = 2048;  // candidate list: slots of the selected top-11-bit bucket

__global__ __launch_bounds__(kSelThreads) void evict_plan_lds(PlanArgs a) {
  extern __shared__ uint32_t keys[];  // ord32 keys at skew(i)
  __shared__ uint32_t hist[2048];     // histograms; tie flags; later each tile's first destination
  __shared__ int cand[kCand];         // candidate slots; later each tile's keep mask
  __shared__ int smem[kSelThreads / 64];
  __shared__ int out[4];
  __shared__ unsigned long long mm[2];
  __shared__ int ncand, nflag, nstage, ncopy;
  __shared__ int efirst, elast;  // first and last evicted slot

  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int s0 = head_start(a.start, u);
  const size_t row0 = (size_t)u * a.cap + s0;  // the head's first live slot
  const int capu = a.cap - s0;                 // slots before the head wraps
  const int n = min(a.len[u], a.cap);
  const int M = a.M;
  if (tid == 0) {
    out[0] = 0;
    out[1] = 1;
    out[2] = -1;
    mm[0] = ~0ull;
    mm[1] = 0ull;
    ncand = 0;
    nflag = 0;
    nstage = 0;
    ncopy = 0;
    efirst = 0x7FFFFFFF;
    elast = -1;
  }
  if (n <= M) {
    if (tid == 0) {
      UnitInfo z = {0ull, -1, MODE_NOOP, n, n, s0, s0};
      a.info[u] = z;
      if (a.n_out) a.n_out[u] = 0;
    }
    return;
  }
  const Ring<const float> lb{a.log_beta ? a.log_beta + row0 : nullptr, capu, a.cap};
  const Ring<const int32_t> ps{a.pos + row0, capu, a.cap};
  const int tpos = a.tq[u / a.Hkv];
  int r = n - M;
  auto key32 = [&](float l, int p) -> uint32_t { return key_ord32(lb, tpos - p, l); };

  // One eviction (the steady state: n = M + 1): the threshold is the minimum of
  // (key, slot), found by reductions instead of radix passes.
  const bool one = r == 1;
  uint32_t kmin = 0xFFFFFFFFu;  // this thread's smallest float32-ordered key
  // ---- pass 0: keys to LDS + histogram of the top 11 bits.  All of a round's
  // loads are issued before any key is formed (the loop is latency bound otherwise).
  for (int i = tid; i < 2048; i += kSelThreads) hist[i] = 0;
  __syncthreads();
  if (a.vec && n <= capu) {
    // 16-byte loads of aligned quads (capacity % 4 == 0, so a quad holding a live
    // slot lies inside the head's rows; the head does not wrap): quad j holds slots
    // 4j - a0 .. 4j - a0 + 3
    const int a0 = (int)(row0 & 3);
    const float* lbq = lb ? lb.p - a0 : nullptr;
    const int32_t* psq = ps.p - a0;
    const int nq = (n + a0 + 3) >> 2;
    constexpr int kQ = 8;
    for (int j0 = tid; j0 < nq; j0 += kQ * kSelThreads) {
      f32x4 l4[kQ];
      i32x4 p4[kQ];
#pragma unroll
      for (int e = 0; e < kQ; ++e) {
        const int j = min(j0 + e * kSelThreads, nq - 1);
        l4[e] = lbq ? *(const f32x4*)(lbq + 4 * j) : f32x4{0.f, 0.f, 0.f, 0.f};
        p4[e] = *(const i32x4*)(psq + 4 * j);
      }
#pragma unroll
      for (int e = 0; e < kQ; ++e) {
        const int j = j0 + e * kSelThreads;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = 4 * j + c - a0;
          if (j < nq && i >= 0 && i < n) {
            const uint32_t k32 = key32(l4[e][c], p4[e][c]);
            keys[skew(i)] = k32;
            if (one) kmin = min(kmin, k32);
            else atomicAdd(&hist[k32 >> 21], 1u);
          }
        }
      }
    }
  } else {
    constexpr int kRounds = 16;
    for (int i0 = tid; i0 < n; i0 += kRounds * kSelThreads) {
      float lv[kRounds];
      int pv[kRounds];
#pragma unroll
      for (int e = 0; e < kRounds; ++e) {
        const int i = min(i0 + e * kSelThreads, n - 1);
        lv[e] = lb ? lb[i] : 0.f;
        pv[e] = ps[i];
      }
#pragma unroll
      for (int e = 0; e < kRounds; ++e) {
        const int i = i0 + e * kSelThreads;
        if (i < n) {
          const uint32_t k32 = key32(lv[e], pv[e]);
          keys[skew(i)] = k32;
          if (one) kmin = min(kmin, k32);
          else atomicAdd(&hist[k32 >> 21], 1u);
        }
      }
    }
  }
  __syncthreads();
  uint32_t t32;
  unsigned long long K;
  if (one) {
    // the smallest float32 key, then the smallest exact key among its ties, then
    // the lowest slot among those
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    if (lane == 0) hist[wv] = kmin;
    __syncthreads();
    t32 = hist[0];
    for (int w2 = 1; w2 < kSelThreads / 64; ++w2) t32 = min(t32, hist[w2]);
    for (int i = tid; i < n; i += kSelThreads)
      if (keys[skew(i)] == t32) atomicMin(&mm[0], ord64(retention_key(lb, ps, i, tpos)));
    __syncthreads();
    K = mm[0];
    if (tid == 0) out[2] = 0x7FFFFFFF;
    __syncthreads();
    for (int i = tid; i < n; i += kSelThreads)
      if (keys[skew(i)] == t32 && ord64(retention_key(lb, ps, i, tpos)) == K) atomicMin(&out[2], i);
  } else {
  int bucket = select_bucket<kSelThreads>(hist, 2048, r, smem, out);
  const uint32_t b0 = (uint32_t)bucket;
  const int c0 = (int)hist[b0];
  if (c0 <= kCand) {
    // ---- the bucket's slots to a list; the remaining passes and the ties use it
    constexpr int kU = 8;  // LDS reads in flight per thread
    for (int i0 = tid; i0 < n; i0 += kU * kSelThreads) {
      uint32_t kk[kU];
#pragma unroll
      for (int e = 0; e < kU; ++e) kk[e] = keys[skew(min(i0 + e * kSelThreads, n - 1))];
#pragma unroll
      for (int e = 0; e < kU; ++e) {
        const int i = i0 + e * kSelThreads;
        if (i < n && (kk[e] >> 21) == b0) cand[atomicAdd(&ncand, 1)] = i;
      }
    }
    __syncthreads();
    const int nc = ncand;
    uint32_t prefix = b0;
    for (int pass = 1; pass < 3; ++pass) {
      const int shift = pass == 1 ? 10 : 0;
      const int bits = pass == 1 ? 11 : 10;
      const int nb = 1 << bits;
      for (int i = tid; i < nb; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int e = tid; e < nc; e += kSelThreads) {
        const uint32_t k32 = keys[skew(cand[e])];
        if ((k32 >> (shift + bits)) == prefix) atomicAdd(&hist[(k32 >> shift) & (nb - 1)], 1u);
      }
      __syncthreads();
      bucket = select_bucket<kSelThreads>(hist, nb, r, smem, out);
      prefix = (prefix << bits) | (uint32_t)bucket;
    }
    t32 = prefix;
    // exact keys of the float32 ties
    for (int e = tid; e < nc; e += kSelThreads) {
      const int i = cand[e];
      if (keys[skew(i)] != t32) continue;
      const unsigned long long k64 = ord64(retention_key(lb, ps, i, tpos));
      atomicMin(&mm[0], k64);
      atomicMax(&mm[1], k64);
    }
    __syncthreads();
    K = mm[0];
    if (K != mm[1]) {
      unsigned long long pfx = 0;
      for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        for (int e = tid; e < nc; e += kSelThreads) {
          const int i = cand[e];
          if (keys[skew(i)] != t32) continue;
          const unsigned long long k64 = ord64(retention_key(lb, ps, i, tpos));
          if (pass == 0 || (k64 >> (shift + 8)) == pfx) atomicAdd(&hist[(k64 >> shift) & 255u], 1u);
        }
        __syncthreads();
        const int bk = select_bucket<kSelThreads>(hist, 256, r, smem, out);
        pfx = (pfx << 8) | (unsigned long long)bk;
      }
      K = pfx;
    }
    // the r-th (slot order) of the candidates whose exact key is K
    for (int e = tid; e < nc; e += kSelThreads) {
      const int i = cand[e];
      const bool f = keys[skew(i)] == t32 && ord64(retention_key(lb, ps, i, tpos)) == K;
      hist[e] = f ? 1u : 0u;
      if (f) atomicAdd(&nflag, 1);
    }
    __syncthreads();
    const int nf = nflag;
    for (int e = tid; e < nc; e += kSelThreads) {
      if (!hist[e]) continue;
      const int i = cand[e];
      int rank = 0;
      if (nf > 1)
        for (int f2 = 0; f2 < nc; ++f2) rank += (hist[f2] && cand[f2] < i) ? 1 : 0;
      if (rank + 1 == r) out[2] = i;
    }
  } else {
    // ---- large bucket: passes 1, 2 over all keys in LDS
    uint32_t prefix = b0;
    for (int pass = 1; pass < 3; ++pass) {
      const int shift = pass == 1 ? 10 : 0;
      const int bits = pass == 1 ? 11 : 10;
      const int nb = 1 << bits;
      for (int i = tid; i < nb; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kSelThreads) {
        const uint32_t k32 = keys[skew(i)];
        if ((k32 >> (shift + bits)) == prefix) atomicAdd(&hist[(k32 >> shift) & (nb - 1)], 1u);
      }
      __syncthreads();
      bucket = select_bucket<kSelThreads>(hist, nb, r, smem, out);
      prefix = (prefix << bits) | (uint32_t)bucket;
    }
    t32 = prefix;
    for (int i = tid; i < n; i += kSelThreads) {
      if (keys[skew(i)] != t32) continue;
      const unsigned long long k64 = ord64(retention_key(lb, ps, i, tpos));
      atomicMin(&mm[0], k64);
      atomicMax(&mm[1], k64);
    }
    __syncthreads();
    K = mm[0];
    if (K != mm[1]) {
      unsigned long long pfx = 0;
      for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kSelThreads) {
          if (keys[skew(i)] != t32) continue;
          const unsigned long long k64 = ord64(retention_key(lb, ps, i, tpos));
          if (pass == 0 || (k64 >> (shift + 8)) == pfx) atomicAdd(&hist[(k64 >> shift) & 255u], 1u);
        }
        __syncthreads();
        const int bk = select_bucket<kSelThreads>(hist, 256, r, smem, out);
        pfx = (pfx << 8) | (unsigned long long)bk;
      }
      K = pfx;
    }
    // slot of the r-th tie (slot order) with exact key K: contiguous ranges
    const int ipt = (n + kSelThreads - 1) / kSelThreads;
    const int lo = min(n, tid * ipt), hi = min(n, lo + ipt);
    int c = 0;
    for (int i = lo; i < hi; ++i)
      if (keys[skew(i)] == t32 && ord64(retention_key(lb, ps, i, tpos)) == K) ++c;
    int tot;
    const int before = block_excl_scan<kSelThreads>(c, smem, tot);
    if (r > before && r <= before + c) {
      int seen = before;
      for (int i = lo; i < hi; ++i)
        if (keys[skew(i)] == t32 && ord64(retention_key(lb, ps, i, tpos)) == K && ++seen == r) {
          out[2] = i;
          break;
        }
    }
  }
  }  // general case
  __syncthreads();
  const int sstar = out[2];

  // ---- keep masks per 32-slot tile (one ballot covers two tiles), tile bases by a
  // scan, then per slot: destination (keep_src), evicted position, and two lists:
  // kept rows below za that move (the fused apply writes into [0, za) while reading
  // the rest, so it copies them to scratch first; za >= kept bounds every
  // destination), and the subset compact_move reads from scratch.
  uint32_t* tmask = (uint32_t*)cand;  // kCand >= tiles: the keys fit in LDS
  const int T = (n + 31) >> 5;
  {
    // wave wv takes 64-slot blocks wv, wv + 16, ...; four blocks per round
    constexpr int kW = kSelThreads / 64, kU = 4;
    const int nb64 = (n + 63) >> 6;
    for (int b0r = wv; b0r < nb64; b0r += kU * kW) {
      uint32_t kk[kU];
#pragma unroll
      for (int e = 0; e < kU; ++e) kk[e] = keys[skew(min(64 * (b0r + e * kW) + lane, n - 1))];
#pragma unroll
      for (int e = 0; e < kU; ++e) {
        const int blk = b0r + e * kW;
        const int i = 64 * blk + lane;
        bool k = kk[e] > t32;
        if (kk[e] == t32 && i < n) {  // float32 tie: the exact key decides
          const unsigned long long k64 = ord64(retention_key(lb, ps, i, tpos));
          k = k64 > K || (k64 == K && i > sstar);
        }
        k = k && i < n;
        const unsigned long long bal = __ballot(k);
        if (lane == 0 && blk < nb64) {
          tmask[2 * blk] = (uint32_t)bal;
          if (2 * blk + 1 < T) tmask[2 * blk + 1] = (uint32_t)(bal >> 32);
        }
      }
    }
  }
  __syncthreads();
  const int tpt = (T + kSelThreads - 1) / kSelThreads;
  const int tl0 = min(T, tid * tpt), tl1 = min(T, tl0 + tpt);
  int kc = 0;
  for (int tl = tl0; tl < tl1; ++tl) kc += __popc(tmask[tl]);
  int kept_all;
  int dst = block_excl_scan<kSelThreads>(kc, smem, kept_all);
  int ef = 0x7FFFFFFF, el = -1;
  for (int tl = tl0; tl < tl1; ++tl) {
    const uint32_t m = tmask[tl];
    hist[tl] = (uint32_t)dst;
    a.tile_mask[(size_t)u * a.Tc + tl] = m;
    a.tile_base[(size_t)u * a.Tc + tl] = dst;
    dst += __popc(m);
    const int live = min(32, n - 32 * tl);
    const uint32_t evb = ~m & (live == 32 ? 0xFFFFFFFFu : ((1u << live) - 1u));
    if (evb) {
      ef = min(ef, 32 * tl + __ffs(evb) - 1);
      el = max(el, 32 * tl + 31 - __clz(evb));
    }
  }
  if (el >= 0) {
    atomicMin(&efirst, ef);
    atomicMax(&elast, el);
  }
  __syncthreads();
  const int kept = min(kept_all, a.Mk);
  // With a start array the head is compacted toward whichever end moves fewer
  // rows: toward its first slot the kept rows after the first evicted slot move,
  // toward its last slot the kept rows before the last evicted slot (the first
  // slot then advances by the evicted count, around the end of the head's slots).
  // nstart is kept unwrapped (s0 <= nstart < s0 + cap) for the staging rule.
  int nstart = s0;
  if (a.start && elast >= 0) {
    const int nev = n - kept;
    const int fwd = kept - efirst;
    const int bwd = elast + 1 - nev;
    if (bwd < fwd) nstart = s0 + nev;
  }
  int2* slist = a.stage_list + (size_t)u * a.Mk;
  int2* clist = a.copy_list + (size_t)u * a.Mk;
  {
    constexpr int kU = 4;
    for (int i0 = tid; i0 < n; i0 += kU * kSelThreads) {
      uint32_t mk[kU];
      int bs[kU];
#pragma unroll
      for (int e = 0; e < kU; ++e) {
        const int tl = min(i0 + e * kSelThreads, n - 1) >> 5;
        mk[e] = tmask[tl];
        bs[e] = (int)hist[tl];
      }
#pragma unroll
      for (int e = 0; e < kU; ++e) {
        const int i = i0 + e * kSelThreads;
        if (i >= n) continue;
        const int s2 = i & 31;
        const int before = bs[e] + __popc(mk[e] & ((1u << s2) - 1u));
        if ((mk[e] >> s2) & 1u) {
          if (before < a.Mk) {
            a.keep_src[(size_t)u * a.Mk + before] = i;
            if (i != before && i < a.za) slist[atomicAdd(&nstage, 1)] = make_int2(i, before);
            if (staged_row(s0, nstart, i, before, kept, a.move_rows))
              clist[atomicAdd(&ncopy, 1)] = make_int2(i, before);
          }
        } else if (a.evicted_pos) {
          const int ev = i - before;
          if (ev < a.max_evict) a.evicted_pos[(size_t)u * a.max_evict + ev] = ps[i];
        }
      }
    }
  }
  __syncthreads();
  // ---- the rows compact_move will read from scratch, copied there: 16-byte pieces
  // (K, V) and the 8-byte row tails; each thread loads a batch before storing any.
  // (The fused apply copies the rest of the stage list itself.)
  {
    const int ns = min(ncopy, a.Mk);
    const int ppr = a.row_bytes / 16;
    const int per = 2 * ppr + 1;
    const unsigned char* kb = (const unsigned char*)a.k + row0 * a.row_bytes;
    const unsigned char* vb = (const unsigned char*)a.v + row0 * a.row_bytes;
    constexpr int kB = 8;
    for (int q0 = tid; q0 < ns * per; q0 += kB * kSelThreads) {
      u32x4 x[kB];
      unsigned char* to[kB];
#pragma unroll
      for (int e = 0; e < kB; ++e) {
        const int q = q0 + e * kSelThreads;
        to[e] = nullptr;
        if (q < ns * per) {
          const int en = q / per, part = q - en * per;
          const int2 sd = clist[en];
          unsigned char* sp = a.scratch + ((size_t)u * a.Mk + sd.y) * a.srow;
          if (part < 2 * ppr) {
            const bool isv = part >= ppr;
            const int pc = isv ? part - ppr : part;
            const ptrdiff_t rs = sd.x < capu ? sd.x : sd.x - a.cap;
            x[e] = *(const u32x4*)((isv ? vb : kb) + rs * a.row_bytes + 16 * pc);
            to[e] = sp + (isv ? a.row_bytes : 0) + 16 * pc;
          } else {
            x[e] = u32x4{lb ? __float_as_uint(lb[sd.x]) : 0u, (uint32_t)ps[sd.x], 0u, 0u};
            to[e] = sp + 2 * a.row_bytes;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < kB; ++e) {
        if (!to[e]) continue;
        if (q0 + e * kSelThreads < ns * per &&
            (q0 + e * kSelThreads) % per == 2 * ppr) {
          *(uint2*)to[e] = make_uint2(x[e][0], x[e][1]);
        } else {
          *(u32x4*)to[e] = x[e];
        }
      }
    }
  }
  if (tid == 0) {
    UnitInfo v = {K, sstar, MODE_EVICT, n, kept, nstart, s0};
    a.info[u] = v;
    a.stage_n[u] = min(nstage, a.Mk);
    if (a.n_out) a.n_out[u] = n - kept_all;
  }
}

// ---------------------------------------------------------------- keep predicate
struct KeepArgs {
  const float* log_beta;
  const int32_t* pos;
  int32_t* len;
  int32_t* start;           // [U] or null
  const int32_t* tq;
  const int32_t* ranges;    // erase: [B][R][2]
  const int32_t* n_ranges;  // erase: [B]
  UnitInfo* info;
  int32_t* counts;          // [U][C]
  int32_t* keep_src;        // [U][Mk]
  unsigned char* scratch;   // [U][Mk][srow]
  int32_t* evicted_pos;     // [U][max_evict] or null
  int32_t* n_out;           // [U] or null
  const uint32_t* keepbits;  // evict: [U][W] from the selection
  const void* k;
  const void* v;
  int32_t cap, Hkv, R, C, W, Mk, max_evict, row_bytes, srow, move_rows;
};

// Copies the ns staged rows of head u to scratch with the whole workgroup (stg(en)
// gives entry en's source slot and destination row): consecutive threads take
// consecutive 16-byte pieces of a row, so a load instruction covers whole lines of a few rows
// (a thread per row touches 64 rows per instruction); each thread's batch of
// pieces is loaded before any of it is stored.
template <int NT, typename Ent>
__device__ __forceinline__ void stage_list_rows(const KeepArgs& a, int u, int s0, Ent stg,
                                                int ns) {
  const int ppr = a.row_bytes / 16;   // pieces per tensor row
  const int per = 2 * ppr;            // K then V
  const size_t ub = (size_t)u * a.cap;
  constexpr int kB = 4;
  for (int q0 = threadIdx.x; q0 < ns * per; q0 += kB * NT) {
    u32x4 x[kB];
    unsigned char* to[kB];
#pragma unroll
    for (int e = 0; e < kB; ++e) {
      const int q = q0 + e * NT;
      to[e] = nullptr;
      if (q < ns * per) {
        const int en = q / per, part = q - en * per;
        const int2 sd = stg(en);
        const size_t row = ub + (s0 + sd.x < a.cap ? s0 + sd.x : s0 + sd.x - a.cap);
        const bool isv = part >= ppr;
        const int pc = isv ? part - ppr : part;
        x[e] = *(const u32x4*)((const unsigned char*)(isv ? a.v : a.k) + row * a.row_bytes + 16 * pc);
        to[e] = a.scratch + ((size_t)u * a.Mk + sd.y) * a.srow + (isv ? a.row_bytes : 0) + 16 * pc;
      }
    }
#pragma unroll
    for (int e = 0; e < kB; ++e)
      if (to[e]) *(u32x4*)to[e] = x[e];
  }
  for (int en = threadIdx.x; en < ns; en += NT) {  // the 8-byte tails
    const int2 sd = stg(en);
    const size_t row = ub + (s0 + sd.x < a.cap ? s0 + sd.x : s0 + sd.x - a.cap);
    const uint32_t l = a.log_beta ? __float_as_uint(a.log_beta[row]) : 0u;
    const uint32_t p = (uint32_t)a.pos[row];
    *(uint2*)(a.scratch + ((size_t)u * a.Mk + sd.y) * a.srow + 2 * a.row_bytes) = make_uint2(l, p);
  }
}

// Index of the first range whose end lies above p (nr if none); the ranges are
// sorted and disjoint.
__device__ __forceinline__ int first_range_ending_after(const int32_t* rg, int nr, int p) {
  int lo = 0, hi = nr;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (rg[2 * mid + 1] <= p) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Erase keep flags of the thread's kPerThread consecutive slots i0 ..
// i0 + kPerThread - 1 (i0 = chunk start + tid * kPerThread), as a bit mask.
template <int MODE>
__device__ __forceinline__ uint32_t keep_flags(const KeepArgs& a, int u, int i0, int n) {
  static_assert(MODE == MODE_ERASE, "eviction flags come from the selection's keep bits");
  const int s0 = head_start(a.start, u);
  const Ring<const int32_t> ps{a.pos + (size_t)u * a.cap + s0, a.cap - s0, a.cap};
  uint32_t fm = 0;  // bit e: slot i0 + e is kept
  // positions increase along the slots: one search for the thread's first slot,
  // then the range index only moves forward
  const int b = u / a.Hkv;
  const int32_t* rg = a.ranges + (size_t)b * a.R * 2;
  const int nr = a.n_ranges[b];
  int pv[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) pv[e] = i0 + e < n ? ps[i0 + e] : 0;
  int ri = i0 < n ? first_range_ending_after(rg, nr, pv[0]) : nr;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int p = pv[e];
    while (ri < nr && rg[2 * ri + 1] <= p) ++ri;
    fm |= (i0 + e < n && !(ri < nr && rg[2 * ri] <= p)) ? 1u << e : 0u;
  }
  return fm;
}

template <int MODE>
__global__ __launch_bounds__(kChunkThreads) void keep_count(KeepArgs a) {
  __shared__ int smem[kChunkThreads / 64];
  const int u = blockIdx.y, c = blockIdx.x;
  const int n = min(a.len[u], a.cap);
  const int base = c * kChunk;
  int cnt = 0;
  if (base < n) cnt = __popc(keep_flags<MODE>(a, u, base + threadIdx.x * kPerThread, n));
  const int tot = block_sum<kChunkThreads>(cnt, smem);
  if (threadIdx.x == 0) a.counts[(size_t)u * a.C + c] = tot;
}

template <int MODE>
__global__ __launch_bounds__(kChunkThreads) void keep_emit(KeepArgs a) {
  __shared__ int smem[kChunkThreads / 64];
  // this chunk's staged rows: source offset in the chunk << 16 | destination
  // offset among the chunk's kept rows (both below kChunk)
  static_assert(kChunk <= 65536, "16-bit offsets");
  __shared__ uint32_t stg[kChunk];
  __shared__ int nstg;
  const int u = blockIdx.y, c = blockIdx.x;
  if (MODE == MODE_EVICT && a.info[u].mode == MODE_NOOP) return;
  const int s0 = head_start(a.start, u);
  const int n = min(a.len[u], a.cap);
  // kept rows before this chunk, and in total
  int before = 0, all = 0;
  for (int j = threadIdx.x; j < a.C; j += kChunkThreads) {
    const int x = a.counts[(size_t)u * a.C + j];
    all += x;
    if (j < c) before += x;
  }
  before = block_sum<kChunkThreads>(before, smem);
  all = block_sum<kChunkThreads>(all, smem);
  if (c == 0 && threadIdx.x == 0) {
    a.info[u].kept = all;
    a.info[u].nstart = s0;
    a.info[u].ostart = s0;
    if (MODE == MODE_ERASE) a.info[u].mode = MODE_ERASE;
    if (a.n_out) a.n_out[u] = n - all;
  }
  const int2 br = wg_blocks(c, n, kChunk);  // this chunk, and a short last one
  const Ring<const int32_t> ps{a.pos + (size_t)u * a.cap + s0, a.cap - s0, a.cap};
  for (int ch = br.x; ch <= br.y; ++ch) {
    const int base = ch * kChunk;
    if (threadIdx.x == 0) nstg = 0;
    const int i0 = base + threadIdx.x * kPerThread;
    uint32_t fm = 0;  // bit e: slot i0 + e is kept
    if constexpr (MODE == MODE_EVICT) {
      static_assert(kPerThread == 16, "half a word of keep bits per thread");
      if (i0 < n) {
        fm = (a.keepbits[(size_t)u * a.W + (i0 >> 5)] >> (i0 & 31)) & 0xFFFFu;
        if (n - i0 < 16) fm &= (1u << (n - i0)) - 1u;
      }
    } else {
      fm = keep_flags<MODE>(a, u, i0, n);
    }
    const int cnt = __popc(fm);
    int total;
    int dst = before + block_excl_scan<kChunkThreads>(cnt, smem, total);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int i = i0 + e;
      if ((fm >> e) & 1u) {
        if (dst < a.Mk) {  // always true when the threshold is consistent
          a.keep_src[(size_t)u * a.Mk + dst] = i;
          if (staged_row(s0, s0, i, dst, all, a.move_rows))
            stg[atomicAdd(&nstg, 1)] = (uint32_t)(i - base) << 16 | (uint32_t)(dst - before);
        }
        ++dst;
      } else if (i < n && MODE == MODE_EVICT && a.evicted_pos) {
        const int ev = i - dst;  // evicted slots before i
        if (ev < a.max_evict) a.evicted_pos[(size_t)u * a.max_evict + ev] = ps[i];
      }
    }
    __syncthreads();
    // the staged rows to scratch (by destination)
    stage_list_rows<kChunkThreads>(
        a, u, s0,
        [&](int en) {
          const uint32_t e = stg[en];
          return make_int2(base + (int)(e >> 16), before + (int)(e & 0xffffu));
        },
        nstg);
    before += total;
    __syncthreads();  // the list read before the next chunk's flags reuse it
  }
}

// ---------------------------------------------------------------- erase by range endpoints
// Positions increase along a head's live slots, so the slots an erase range [s, e)
// covers form one run, [lb(s), lb(e)) with lb(x) = number of live slots whose position
// is below x, and the kept slots are the runs between consecutive ranges.  Instead of
// testing every slot, erase_search finds lb at each range endpoint and erase_plan
// lays the kept runs end to end (keep_src, staging, the head's new length); the
// rows then move with compact_move as for an eviction.
constexpr int kEraseMaxR = 4096;  // ranges per sequence on this path (LDS tables)

// One wave per (endpoint, head): 64 evenly spaced probes per round cut the search
// interval 64-fold (four dependent loads for a 1M-slot head).  Invariant: slots
// below lo have positions below x, slots at or above hi do not.  The probes that
// fall below x are a prefix of the lanes; malformed (unsorted) positions still give
// a value in [0, n] after at most ~log64(n) + 1 rounds.
__global__ __launch_bounds__(256) void erase_search(KeepArgs a, int32_t* ep, int32_t* max_kept) {
  const int u = blockIdx.y;
  const int b = u / a.Hkv;
  const int e = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *max_kept = 0;
  const int nr = max(0, min(a.n_ranges[b], a.R));
  if (e >= 2 * nr) return;
  const int x = a.ranges[(size_t)b * a.R * 2 + e];
  const int s0 = head_start(a.start, u);
  const Ring<const int32_t> ps{a.pos + (size_t)u * a.cap + s0, a.cap - s0, a.cap};
  const int n = min(a.len[u], a.cap);
  int lo = 0, hi = n;
  while (lo < hi) {
    const int step = (hi - lo + 63) >> 6;
    const int i = lo + lane * step;
    const bool below = i < hi && ps[i] < x;
    const int c = __popcll(__ballot(below));
    if (c == 0) break;                   // the probe at lo is not below x: lb = lo
    const int nxt = lo + c * step;       // first probe not below x (or past hi)
    lo = lo + (c - 1) * step + 1;
    hi = min(hi, nxt);
  }
  if (lane == 0) ep[(size_t)u * 2 * a.R + e] = lo;
}

// Grid (kErasePlanBlocks, heads).  Kept run k is [a_k, b_k) with a_0 = 0,
// a_k = lb(e_{k-1}), b_k = lb(s_k), b_nr = n; its rows go to slots d_k .. d_k +
// (b_k - a_k) - 1, d_k the exclusive prefix of the run lengths.  Each workgroup
// builds the (small) run table in LDS once, then writes keep_src for destination
// blocks of one row per thread, strided over the grid.  The rows compact_move must
// not read in place (staged_row) are those whose source lies below the kept count,
// so they belong to the runs starting there and sit at the first destinations; a
// second pass copies them to scratch in 16-row slices strided over the grid, so
// that the copying is spread over every workgroup of the head instead of falling
// on the first few.
constexpr int kErasePlanBlocks = 64;
constexpr int kEraseSlice = 16;  // staged rows per slice in the copy pass
__global__ __launch_bounds__(kChunkThreads) void erase_plan(KeepArgs a, const int32_t* ep,
                                                            int32_t* max_kept) {
  __shared__ int s_a[kEraseMaxR + 1];
  __shared__ int s_d[kEraseMaxR + 1];
  __shared__ int smem[kChunkThreads / 64];
  __shared__ int s_stage_end;
  const int u = blockIdx.y;
  const int b = u / a.Hkv;
  const int tid = threadIdx.x;
  const int nr = max(0, min(a.n_ranges[b], a.R));
  const int n = min(a.len[u], a.cap);
  const int s0 = head_start(a.start, u);
  const int32_t* e = ep + (size_t)u * 2 * a.R;
  if (tid == 0) s_stage_end = 0;
  int carry = 0;
  for (int k0 = 0; k0 <= nr; k0 += kChunkThreads) {
    const int k = k0 + tid;
    int len = 0;
    if (k <= nr) {
      const int ak = k == 0 ? 0 : e[2 * k - 1];
      const int bk = k == nr ? n : e[2 * k];
      len = max(bk - ak, 0);
      s_a[k] = ak;
    }
    int tot;
    const int ex = block_excl_scan<kChunkThreads>(len, smem, tot);
    if (k <= nr) s_d[k] = carry + ex;
    carry += tot;
  }
  const int kept = min(carry, n);
  __syncthreads();
  // one past the last destination whose row may be staged: over the runs that
  // move, the end of each one's rows with sources below the kept count (does not
  // assume the runs are ordered)
  for (int k = tid; k <= nr; k += kChunkThreads) {
    const int len = (k < nr ? s_d[k + 1] : carry) - s_d[k];
    if (len > 0 && s_a[k] < kept && s_a[k] != s_d[k])
      atomicMax(&s_stage_end, s_d[k] + min(len, kept - s_a[k]));
  }
  if (blockIdx.x == 0 && tid == 0) {
    UnitInfo inf = a.info[u];
    inf.mode = MODE_ERASE;
    inf.n = n;
    inf.kept = kept;
    inf.nstart = s0;
    inf.ostart = s0;
    a.info[u] = inf;
    if (a.n_out) a.n_out[u] = n - kept;
    atomicMax(max_kept, kept);
  }
  __syncthreads();
  const int jmax = min(kept, a.Mk);
  // the last run starting at or below destination j (runs of length 0 share
  // their start with the next one)
  auto source_of = [&](int j) {
    int lo = 0, hi = nr;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_d[mid] <= j) lo = mid;
      else hi = mid - 1;
    }
    return s_a[lo] + (j - s_d[lo]);
  };
  for (int j = blockIdx.x * kChunkThreads + tid; j < jmax; j += gridDim.x * kChunkThreads)
    a.keep_src[(size_t)u * a.Mk + j] = source_of(j);

  // copy pass: kChunkThreads / kEraseSlice threads per row, 16-byte pieces of K
  // then V; every thread loads its pieces before storing them
  constexpr int kTpr = kChunkThreads / kEraseSlice;
  const int send = min(s_stage_end, jmax);
  const int ppr = a.row_bytes / 16, per = 2 * ppr;
  const size_t ub = (size_t)u * a.cap;
  const int sub = tid % kTpr;
  for (int z0 = blockIdx.x * kEraseSlice; z0 < send; z0 += gridDim.x * kEraseSlice) {
    const int j = z0 + tid / kTpr;
    if (j >= send) continue;
    const int src = source_of(j);
    if (!staged_row(s0, s0, src, j, kept, a.move_rows)) continue;
    const size_t row = ub + (s0 + src < a.cap ? s0 + src : s0 + src - a.cap);
    unsigned char* sp = a.scratch + ((size_t)u * a.Mk + j) * a.srow;
    for (int p0 = sub; p0 < per; p0 += 4 * kTpr) {
      u32x4 x[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int pc = p0 + t * kTpr;
        if (pc < per) {
          const bool isv = pc >= ppr;
          x[t] = *(const u32x4*)((const unsigned char*)(isv ? a.v : a.k) + row * a.row_bytes +
                                 16 * (isv ? pc - ppr : pc));
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int pc = p0 + t * kTpr;
        if (pc < per) *(u32x4*)(sp + 16 * pc) = x[t];  // K then V, as in the cache
      }
    }
    if (sub == 0) {
      const uint32_t l = a.log_beta ? __float_as_uint(a.log_beta[row]) : 0u;
      *(uint2*)(sp + 2 * a.row_bytes) = make_uint2(l, (uint32_t)a.pos[row]);
    }
  }
}

// ---------------------------------------------------------------- move
constexpr int kMoveThreads = 256;
// 16-byte pieces per thread per group (groups of 64 destination rows for D = 128 in
// bf16), stores with the non-temporal hint.  Alone, plain stores and 32-row groups
// were faster (99 against 117 us on the 32K layer); inside the decode step, where
// the compactions run beside the next layers' planners, this form gave the shortest
// step (16.4-16.8 against 17.0 ms).
constexpr int kMovePieces = 8;

// Thread layout: piece column pc = tid % (2*ppr) (K chunks, then V chunks) is fixed
// per thread; the thread moves that column of rows tid / (2*ppr) + q * rpp,
// q < kMovePieces (rpp = rows per pass).  All reads of the group are issued
// before the barrier, all writes after it.
__global__ __launch_bounds__(kMoveThreads) void compact_move(KeepArgs a, int U, int check_mode,
                                                              const int32_t* max_kept) {
  const int cpu = (a.Mk + a.move_rows - 1) / a.move_rows;
  const int ppr = a.row_bytes / 16;   // 16-byte pieces per row per tensor
  const int cols = 2 * ppr;
  const int rpp = kMoveThreads / cols; // rows per pass
  const int tid = threadIdx.x;
  const int col = tid % cols;
  const int r0 = tid / cols;
  const bool isv = col >= ppr;
  const int pc = isv ? col - ppr : col;
  // one item per workgroup: item w = (head u, group ch), groups of a head on
  // neighbouring workgroups; when the grid strides (many more groups than
  // workgroups), heads fastest, so the groups that hold rows (the first kept /
  // move_rows of every head) are the first items, spread over the grid
  const bool strided = U * cpu > (int)gridDim.x;
  // with heads fastest, the items past the largest kept count hold no rows
  int items = U * cpu;
  if (strided && max_kept) items = min(items, U * ((*max_kept + a.move_rows - 1) / a.move_rows));
  for (int w = blockIdx.x; w < items; w += gridDim.x) {
    const int u = strided ? w % U : w / cpu, ch = strided ? w / U : w % cpu;
    const UnitInfo inf = a.info[u];
    if (check_mode && inf.mode == MODE_NOOP) continue;
    const int kept = min(inf.kept, a.Mk);
    const int os = inf.ostart, ns = inf.nstart;
    // slots are kept unwrapped below (< 2 cap); addresses wrap
    auto wrap = [&](int x) { return x < a.cap ? x : x - a.cap; };
    if (ch == 0 && tid == 0) {
      a.len[u] = kept;
      if (a.start) a.start[u] = wrap(ns);
    }
    const int j0 = ch * a.move_rows;
    if (j0 >= kept) continue;
    const int rows = min(a.move_rows, kept - j0);
    const int32_t* ks = a.keep_src + (size_t)u * a.Mk;
    // (os + src) - (ns + j) never decreases along the destinations and ends at or
    // above 0 toward the first slot, at or below 0 toward the end: a group whose
    // last (first) row stays in place moves no row
    if (ns <= os ? os + ks[j0 + rows - 1] == ns + j0 + rows - 1 : os + ks[j0] == ns + j0) continue;
    const unsigned char* scr = a.scratch + (size_t)u * a.Mk * a.srow;
    unsigned char* tb = (unsigned char*)(isv ? a.v : a.k) + (size_t)u * a.cap * a.row_bytes;
    float* lbb = a.log_beta ? (float*)a.log_beta + (size_t)u * a.cap : nullptr;
    int32_t* pb = (int32_t*)a.pos + (size_t)u * a.cap;
    // this group's staged sources (staged_row for the group's rows): the slots of
    // the other groups' destinations that can be overwritten first
    const int st_lo = ns <= os ? ns + j0 + a.move_rows : ns;
    const int st_hi = ns <= os ? ns + kept : ns + j0;

    int src[kMovePieces];
#pragma unroll
    for (int q = 0; q < kMovePieces; ++q) {
      const int row = r0 + q * rpp;
      src[q] = (r0 < rpp && row < rows) ? ks[j0 + row] : -1;
    }
    bool mv[kMovePieces];  // this piece's row moves
    u32x4 buf[kMovePieces];
#pragma unroll
    for (int q = 0; q < kMovePieces; ++q) {
      const int j = j0 + r0 + q * rpp;
      const int sa = os + src[q];
      mv[q] = src[q] >= 0 && sa != ns + j;
      const bool staged = sa >= st_lo && sa < st_hi;
      const unsigned char* from =
          staged ? scr + (size_t)j * a.srow + (isv ? a.row_bytes : 0) + 16 * pc
                 : tb + (size_t)wrap(sa) * a.row_bytes + 16 * pc;
      buf[q] = mv[q] ? __builtin_nontemporal_load((const u32x4*)from) : u32x4{0u, 0u, 0u, 0u};
    }
    int32_t tail_lb = 0, tail_pos = 0, tail_dst = -1;
    if (tid < rows) {
      const int j = j0 + tid;
      const int sr = ks[j];
      if (os + sr != ns + j) {
        if (os + sr >= st_lo && os + sr < st_hi) {
          const int32_t* tl = (const int32_t*)(scr + (size_t)j * a.srow + 2 * a.row_bytes);
          tail_lb = tl[0];
          tail_pos = tl[1];
        } else {
          tail_lb = lbb ? __float_as_int(lbb[wrap(os + sr)]) : 0;
          tail_pos = pb[wrap(os + sr)];
        }
        tail_dst = wrap(ns + j);
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kMovePieces; ++q) {
      const int j = j0 + r0 + q * rpp;
      if (mv[q])
        __builtin_nontemporal_store(buf[q],
                                    (u32x4*)(tb + (size_t)wrap(ns + j) * a.row_bytes + 16 * pc));
    }
    if (tail_dst >= 0) {
      if (lbb) lbb[tail_dst] = __int_as_float(tail_lb);
      pb[tail_dst] = tail_pos;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- one eviction
// kv_evict_one: a head exactly one token over its budget loses the token with the
// lowest (kappa, slot) -- the same rule as the general selection with n - M = 1 --
// and the gap closes by shifting the shorter side one slot (with a start array:
// the rows before it up, start + 1, when there are fewer of them than after it;
// otherwise the rows after it down), the direction the general planner picks for
// one eviction.  One 1024-thread workgroup per head: an argmin over the head's keys
// (coalesced, 16 slots in flight per thread), then the shift in chunks of rows,
// each chunk read into registers completely before any of it is written.
struct OneArgs {
  void* k;
  void* v;
  float* log_beta;
  int32_t* pos;
  int32_t* len;
  int32_t* start;
  const int32_t* tq;
  int32_t* evicted_pos;
  int32_t* n_out;
  int32_t cap, Hkv, M, max_evict, row_bytes;
};
constexpr int kOneItems = 8;  // 16-byte items per thread per chunk

__global__ __launch_bounds__(kSelThreads) void evict_one(OneArgs a) {
  __shared__ unsigned long long wkey[kSelThreads / 64];
  __shared__ int wslot[kSelThreads / 64];
  __shared__ int es;
  const int u = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int s0 = head_start(a.start, u);
  const int n = min(a.len[u], a.cap);
  if (n <= a.M || n > a.M + 1) {
    if (tid == 0 && a.n_out) a.n_out[u] = n <= a.M ? 0 : -(n - a.M);
    return;
  }
  const size_t row0 = (size_t)u * a.cap;
  const Ring<const float> lb{a.log_beta ? a.log_beta + row0 + s0 : nullptr, a.cap - s0, a.cap};
  const Ring<const int32_t> ps{a.pos + row0 + s0, a.cap - s0, a.cap};
  const int tpos = a.tq[u / a.Hkv];

  // ---- the slot with the lowest (exact key, slot)
  unsigned long long bk = ~0ull;
  int bs = 0x7FFFFFFF;
  for (int base = 0; base < n; base += kSelThreads * kSelB) {
    int dd[kSelB];
    float bb[kSelB];
    sel_load<kSelThreads>(lb, ps, base, n, tpos, dd, bb);
#pragma unroll
    for (int e = 0; e < kSelB; ++e) {
      const int i = base + e * kSelThreads + tid;
      if (i >= n) continue;
      const unsigned long long k64 = ord64(key_f64(lb, dd[e], bb[e]));
      if (k64 < bk || (k64 == bk && i < bs)) {
        bk = k64;
        bs = i;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long ok = __shfl_xor(bk, o, 64);
    const int os = __shfl_xor(bs, o, 64);
    if (ok < bk || (ok == bk && os < bs)) {
      bk = ok;
      bs = os;
    }
  }
  if (lane == 0) {
    wkey[w] = bk;
    wslot[w] = bs;
  }
  __syncthreads();
  if (tid == 0) {
    unsigned long long k = wkey[0];
    int sl = wslot[0];
    for (int i = 1; i < kSelThreads / 64; ++i)
      if (wkey[i] < k || (wkey[i] == k && wslot[i] < sl)) {
        k = wkey[i];
        sl = wslot[i];
      }
    es = sl;
    if (a.evicted_pos && a.max_evict > 0) a.evicted_pos[(size_t)u * a.max_evict] = ps[sl];
    if (a.n_out) a.n_out[u] = 1;
  }
  wait_vmem_all();
  __syncthreads();
  const int e = es;

  // ---- close the gap: rows (e, n) down one slot, or rows [0, e) up one
  const bool up = a.start != nullptr && e < n - 1 - e;
  const int ppr = a.row_bytes / 16;
  const int per = 2 * ppr + 1;  // 16-byte pieces of K and V, then (log beta, pos)
  const int R = (kSelThreads * kOneItems) / per;  // rows per chunk
  unsigned char* kb = (unsigned char*)a.k + row0 * a.row_bytes;
  unsigned char* vb = (unsigned char*)a.v + row0 * a.row_bytes;
  float* lbb = a.log_beta ? a.log_beta + row0 : nullptr;
  int32_t* pb = a.pos + row0;
  const int first = up ? 0 : e + 1, last = up ? e : n;  // rows [first, last) move
  const int nchunks = (last - first + R - 1) / R;
  // down: ascending chunks; up: descending.  Chunk c + 1's sources never overlap
  // chunk c's destinations, and chunk c's sources are all in registers (every
  // thread waited, then the barrier) before chunk c + 1 -- whose destinations take
  // chunk c's last source -- stores; so chunk c + 1 is loaded while c is stored.
  auto chunk = [&](int c, int& r0, int& r1) {
    r0 = up ? max(last - (c + 1) * R, first) : first + c * R;
    r1 = up ? last - c * R : min(first + (c + 1) * R, last);
  };
  auto load = [&](int c, u32x4* buf) {
    int r0, r1;
    chunk(c, r0, r1);
    const int items = (r1 - r0) * per;
#pragma unroll
    for (int q = 0; q < kOneItems; ++q) {
      const int it = tid + q * kSelThreads;
      buf[q] = u32x4{0u, 0u, 0u, 0u};
      if (it < items) {
        const int row = r0 + it / per;
        const int pt = it - (it / per) * per;
        const int sj = s0 + row;
        const int src = sj < a.cap ? sj : sj - a.cap;
        if (pt < 2 * ppr) {
          const bool isv = pt >= ppr;
          buf[q] = *(const u32x4*)((isv ? vb : kb) + (size_t)src * a.row_bytes +
                                   16 * (isv ? pt - ppr : pt));
        } else {
          buf[q] = u32x4{lbb ? __float_as_uint(lbb[src]) : 0u, (uint32_t)pb[src], 0u, 0u};
        }
      }
    }
  };
  auto store = [&](int c, const u32x4* buf) {
    int r0, r1;
    chunk(c, r0, r1);
    const int items = (r1 - r0) * per;
#pragma unroll
    for (int q = 0; q < kOneItems; ++q) {
      const int it = tid + q * kSelThreads;
      if (it >= items) continue;
      const int row = r0 + it / per;
      const int pt = it - (it / per) * per;
      const int dj = s0 + (up ? row + 1 : row - 1);
      const int dst = dj < a.cap ? dj : dj - a.cap;
      if (pt < 2 * ppr) {
        const bool isv = pt >= ppr;
        *(u32x4*)((isv ? vb : kb) + (size_t)dst * a.row_bytes + 16 * (isv ? pt - ppr : pt)) =
            buf[q];
      } else {
        if (lbb) lbb[dst] = __uint_as_float(buf[q][0]);
        pb[dst] = (int32_t)buf[q][1];
      }
    }
  };
  u32x4 b0[kOneItems], b1[kOneItems];
  if (nchunks > 0) load(0, b0);
  for (int c = 0; c < nchunks; c += 2) {
    wait_vmem_all();
    __syncthreads();
    if (c + 1 < nchunks) load(c + 1, b1);
    store(c, b0);
    if (c + 1 >= nchunks) break;
    wait_vmem_all();
    __syncthreads();
    if (c + 2 < nchunks) load(c + 2, b0);
    store(c + 1, b1);
  }
  if (tid == 0) {
    a.len[u] = n - 1;
    if (up) a.start[u] = s0 + 1 < a.cap ? s0 + 1 : 0;
  }
}

// ---------------------------------------------------------------- host
// Dynamic LDS available to evict_plan_lds (static LDS of the kernel excluded).
static size_t plan_lds_limit() {
  static size_t limit = 0;
  if (limit == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
        v > 0) {
      hipFuncAttributes fa;
      size_t static_lds = 64 * 1024;  // conservative if the query fails
      if (hipFuncGetAttributes(&fa, (const void*)evict_plan_lds) == hipSuccess)
        static_lds = fa.sharedSizeBytes;
      limit = (size_t)v > static_lds + 256 ? (size_t)v - static_lds - 256 : 1;
      if (hipFuncSetAttribute((const void*)evict_plan_lds,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)limit) != hipSuccess)
        limit = 1;
    } else {
      limit = 1;
    }
  }
  return limit;
}

struct CompactLayout {
  size_t info, counts, keep_src, scratch, tile_mask, tile_base, stage_n, stage_list, copy_list,
      sel_hist, sel_nlist, sel_ls, sel_bits, total;
  int C, W, Mk, srow, move_rows, row_bytes, Tc;
};

static CompactLayout compact_layout(const kvb_cache* c, int Mk) {
  CompactLayout L;
  const size_t U = (size_t)c->B * c->Hkv;
  L.row_bytes = c->D * (c->dtype == KVB_BF16 ? 2 : 4);
  L.srow = 2 * L.row_bytes + 16;
  L.C = (c->cap + kChunk - 1) / kChunk;
  L.Mk = Mk < 1 ? 1 : Mk;
  {
    const int cols = 2 * (L.row_bytes / 16);
    const int rpp = kMoveThreads / cols;
    L.move_rows = rpp * kMovePieces;
    if (L.move_rows > kMoveThreads) L.move_rows = kMoveThreads;  // one thread per row tail
  }
  L.Tc = (c->cap + 31) / 32;
  L.info = kWsHeader;
  L.counts = L.info + align_up(U * sizeof(UnitInfo), 256);
  L.keep_src = L.counts + align_up(U * L.C * sizeof(int32_t), 256);
  L.scratch = L.keep_src + align_up(U * L.Mk * sizeof(int32_t), 256);
  L.tile_mask = L.scratch + align_up(U * L.Mk * (size_t)L.srow, 256);
  L.tile_base = L.tile_mask + align_up(U * L.Tc * sizeof(uint32_t), 256);
  L.stage_n = L.tile_base + align_up(U * L.Tc * sizeof(int32_t), 256);
  L.stage_list = L.stage_n + align_up(U * sizeof(int32_t), 256);
  L.copy_list = L.stage_list + align_up(U * L.Mk * sizeof(int2), 256);
  L.sel_hist = L.copy_list + align_up(U * L.Mk * sizeof(int2), 256);
  // the chunked selection's histograms and list: only for heads the LDS planner
  // cannot take
  const bool chunked = !plan_in_lds(c);
  L.sel_nlist = L.sel_hist + (chunked ? align_up(U * kSelHistWords * sizeof(uint32_t), 256) : 0);
  L.sel_ls = L.sel_nlist + (chunked ? align_up(U * sizeof(SelHead), 256) : 0);
  L.W = (c->cap + 31) / 32;
  L.sel_bits = L.sel_ls + (chunked ? align_up(U * kSelCand * sizeof(int32_t), 256) : 0);
  L.total = L.sel_bits + (chunked ? align_up(U * L.W * sizeof(uint32_t), 256) : 0);
  return L;
}

static KeepArgs keep_args(const kvb_cache* c, const CompactLayout& L, void* ws) {
  KeepArgs a;
  memset(&a, 0, sizeof(a));
  char* w = (char*)ws;
  a.log_beta = c->log_beta;
  a.pos = c->pos;
  a.len = c->len;
  a.start = c->start;
  a.info = (UnitInfo*)(w + L.info);
  a.counts = (int32_t*)(w + L.counts);
  a.keep_src = (int32_t*)(w + L.keep_src);
  a.scratch = (unsigned char*)(w + L.scratch);
  a.k = c->k;
  a.v = c->v;
  a.cap = c->cap;
  a.Hkv = c->Hkv;
  a.C = L.C;
  a.W = L.W;
  a.Mk = L.Mk;
  a.row_bytes = L.row_bytes;
  a.srow = L.srow;
  a.move_rows = L.move_rows;
  return a;
}

static void launch_keep_chunks(const kvb_cache* c, const KeepArgs& a, int mode, hipStream_t s) {
  const int U = c->B * c->Hkv;
  dim3 grid(a.C, U);
  if (mode == MODE_EVICT) {
    // the chunk counts come from the selection (sel_refine, sel_finish)
    { TraceScope tr(kTrKeepEmit, s);
      hipLaunchKernelGGL(keep_emit<MODE_EVICT>, grid, dim3(kChunkThreads), 0, s, a); }
  } else {
    { TraceScope tr(kTrKeepCount, s);
      hipLaunchKernelGGL(keep_count<MODE_ERASE>, grid, dim3(kChunkThreads), 0, s, a); }
    { TraceScope tr(kTrKeepEmit, s);
      hipLaunchKernelGGL(keep_emit<MODE_ERASE>, grid, dim3(kChunkThreads), 0, s, a); }
  }
}

static void launch_move(const kvb_cache* c, const KeepArgs& a, int mode, hipStream_t s,
                        const int32_t* max_kept = nullptr, int max_blocks = 16384) {
  const int U = c->B * c->Hkv;
  const long long items = (long long)U * ((a.Mk + a.move_rows - 1) / a.move_rows);
  // one group per workgroup (many in flight hide the read latency) up to max_blocks
  // workgroups; past that the kernel strides over the groups (heads fastest, so the
  // groups with rows to move, the first of every head, come first, and with
  // max_kept the loop ends after the last of them)
  const int blocks = (int)(items < max_blocks ? items : max_blocks);
  TraceScope tr(kTrCompactMove, s);
  hipLaunchKernelGGL(compact_move, dim3(blocks), dim3(kMoveThreads), 0, s, a, U,
                     mode == MODE_EVICT ? 1 : 0, max_kept);
}

// Eviction plan: selection, destinations, evicted positions, staging.  Reads the
// cache, writes only the workspace and the caller's outputs.
static int32_t evict_plan(const kvb_cache* cache, const CompactLayout& L, const int32_t* t,
                          int32_t M, int32_t* evicted_pos, int32_t max_evict,
                          int32_t* n_evicted, void* ws, hipStream_t s) {
  KeepArgs a = keep_args(cache, L, ws);
  a.tq = t;
  a.evicted_pos = evicted_pos;
  a.max_evict = max_evict;
  a.n_out = n_evicted;
  const size_t lds_keys = ((size_t)cache->cap + cache->cap / 32 + 1) * sizeof(uint32_t);
  if (plan_in_lds(cache)) {
    PlanArgs pa;
    pa.log_beta = cache->log_beta;
    pa.pos = cache->pos;
    pa.len = cache->len;
    pa.start = cache->start;
    pa.tq = t;
    pa.info = a.info;
    pa.keep_src = a.keep_src;
    pa.evicted_pos = evicted_pos;
    pa.n_out = n_evicted;
    pa.scratch = a.scratch;
    pa.k = cache->k;
    pa.v = cache->v;
    pa.cap = cache->cap;
    pa.Hkv = cache->Hkv;
    pa.M = M;
    pa.Mk = a.Mk;
    pa.max_evict = max_evict;
    pa.row_bytes = a.row_bytes;
    pa.srow = a.srow;
    pa.move_rows = a.move_rows;
    char* w = (char*)ws;
    pa.tile_mask = (uint32_t*)(w + L.tile_mask);
    pa.tile_base = (int32_t*)(w + L.tile_base);
    pa.stage_n = (int32_t*)(w + L.stage_n);
    pa.stage_list = (int2*)(w + L.stage_list);
    pa.copy_list = (int2*)(w + L.copy_list);
    pa.Tc = L.Tc;
    pa.za = fused_za(M, cache->cap);
    pa.vec = cache->cap % 4 == 0;
    TraceScope tr(kTrEvictSelect, s);
    hipLaunchKernelGGL(evict_plan_lds, dim3(cache->B * cache->Hkv), dim3(kSelThreads), lds_keys, s,
                       pa);
  } else {
    SelArgs sa;
    char* w = (char*)ws;
    sa.log_beta = cache->log_beta;
    sa.pos = cache->pos;
    sa.len = cache->len;
    sa.start = cache->start;
    sa.tq = t;
    sa.hist = (uint32_t*)(w + L.sel_hist);
    sa.head = (SelHead*)(w + L.sel_nlist);
    sa.ls = (int32_t*)(w + L.sel_ls);
    sa.keepbits = (uint32_t*)(w + L.sel_bits);
    sa.W = L.W;
    sa.info = a.info;
    sa.n_out = n_evicted;
    sa.counts = a.counts;
    sa.C = a.C;
    sa.cap = cache->cap;
    sa.Hkv = cache->Hkv;
    sa.M = M;
    const int U = cache->B * cache->Hkv;
    const dim3 slices((cache->cap + kSelSlice - 1) / kSelSlice, U);
    {
      TraceScope tr(kTrEvictSelect, s);
      hipLaunchKernelGGL(sel_init, dim3(U), dim3(kSelNT), 0, s, sa);
      hipLaunchKernelGGL(sel_hist0, slices, dim3(kSelNT), 0, s, sa);
      for (int pass = 1; pass <= kSelRefines; ++pass)
        hipLaunchKernelGGL(sel_refine, slices, dim3(kSelNT), 0, s, sa, pass);
      hipLaunchKernelGGL(sel_finish, dim3(U), dim3(kSelThreads), 0, s, sa);
    }
    KeepArgs ka = a;
    ka.keepbits = sa.keepbits;
    launch_keep_chunks(cache, ka, MODE_EVICT, s);
  }
  return launch_status();
}

// Whether kv_evict_plan uses the LDS planner (which also prepares the fused
// attention + compaction path) for this cache.
bool plan_in_lds(const kvb_cache* c) {
  const size_t lds_keys = ((size_t)c->cap + c->cap / 32 + 1) * sizeof(uint32_t);
  return lds_keys <= plan_lds_limit() && (c->cap + 31) / 32 <= kCand;
}

// Copies the stage list (kept rows below za that move) to scratch by destination
// index, for the fused apply: one workgroup per (head, 64 entries); sources are
// slots from the head's first live slot.  Each thread issues a batch of loads
// before storing any.
__global__ __launch_bounds__(256) void stage_copy(const UnitInfo* info, const int32_t* count,
                                                  const int2* list, unsigned char* scratch,
                                                  const void* k, const void* v,
                                                  const float* log_beta, const int32_t* pos,
                                                  int cap, int Mk, int srow, int row_bytes) {
  const int u = blockIdx.y;
  const UnitInfo inf = info[u];
  if (inf.mode != MODE_EVICT) return;
  const int ns = min(count[u], Mk);
  const int e0 = blockIdx.x * 64;
  if (e0 >= ns) return;
  const int ppr = row_bytes / 16, per = 2 * ppr + 1;
  const int total = (min(ns, e0 + 64) - e0) * per;
  const size_t row0 = (size_t)u * cap + inf.ostart;
  const unsigned char* kb = (const unsigned char*)k + row0 * row_bytes;
  const unsigned char* vb = (const unsigned char*)v + row0 * row_bytes;
  const int2* sl = list + (size_t)u * Mk;
  constexpr int kB = 9;  // 64 rows of 33 pieces (D = 128 bf16) in one batch
  for (int q0 = threadIdx.x; q0 < total; q0 += kB * 256) {
    u32x4 x[kB];
    unsigned char* to[kB];
    bool tail[kB];
#pragma unroll
    for (int e = 0; e < kB; ++e) {
      const int q = q0 + e * 256;
      to[e] = nullptr;
      tail[e] = false;
      if (q < total) {
        const int en = e0 + q / per, part = q - (q / per) * per;
        const int2 sd = sl[en];
        unsigned char* sp = scratch + ((size_t)u * Mk + sd.y) * srow;
        const ptrdiff_t rs = inf.ostart + sd.x < cap ? sd.x : sd.x - cap;  // around the end
        if (part < 2 * ppr) {
          const bool isv = part >= ppr;
          const int pc = isv ? part - ppr : part;
          x[e] = *(const u32x4*)((isv ? vb : kb) + rs * row_bytes + 16 * pc);
          to[e] = sp + (isv ? row_bytes : 0) + 16 * pc;
        } else {
          x[e] = u32x4{log_beta ? __float_as_uint(log_beta[row0 + rs]) : 0u,
                       (uint32_t)pos[row0 + rs], 0u, 0u};
          to[e] = sp + 2 * row_bytes;
          tail[e] = true;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < kB; ++e) {
      if (!to[e]) continue;
      if (tail[e]) *(uint2*)to[e] = make_uint2(x[e][0], x[e][1]);
      else *(u32x4*)to[e] = x[e];
    }
  }
}

void launch_fused_stage(const kvb_cache* c, int32_t M, void* ws, hipStream_t s) {
  const CompactLayout L = compact_layout(c, M < c->cap ? M : c->cap);
  char* w = (char*)ws;
  const int U = c->B * c->Hkv;
  dim3 grid((L.Mk + 63) / 64, U);
  hipLaunchKernelGGL(stage_copy, grid, dim3(256), 0, s, (const UnitInfo*)(w + L.info),
                     (const int32_t*)(w + L.stage_n), (const int2*)(w + L.stage_list),
                     (unsigned char*)(w + L.scratch), c->k, c->v, c->log_beta, c->pos, c->cap,
                     L.Mk, L.srow, L.row_bytes);
}

FusedPlan fused_plan(const kvb_cache* c, int32_t M, void* ws) {
  const CompactLayout L = compact_layout(c, M < c->cap ? M : c->cap);
  const char* w = (const char*)ws;
  FusedPlan f;
  f.info = (const UnitInfo*)(w + L.info);
  f.tile_mask = (const uint32_t*)(w + L.tile_mask);
  f.tile_base = (const int32_t*)(w + L.tile_base);
  f.stage_n = (const int32_t*)(w + L.stage_n);
  f.stage_list = (const int2*)(w + L.stage_list);
  f.scratch = (const unsigned char*)(w + L.scratch);
  f.Tc = L.Tc;
  f.Mk = L.Mk;
  f.srow = L.srow;
  return f;
}

EvictView evict_view(const kvb_cache* c, int32_t M, const void* ws) {
  const CompactLayout L = compact_layout(c, M < c->cap ? M : c->cap);
  const char* w = (const char*)ws;
  EvictView e;
  e.info = (const UnitInfo*)(w + L.info);
  e.keep_src = (const int32_t*)(w + L.keep_src);
  e.Mk = L.Mk;
  const bool lds = plan_in_lds(c);
  e.tile_mask = lds ? (const uint32_t*)(w + L.tile_mask) : nullptr;
  e.tile_base = lds ? (const int32_t*)(w + L.tile_base) : nullptr;
  e.Tc = L.Tc;
  return e;
}

static int32_t evict_validate(const kvb_cache* cache, int32_t M, size_t ws_bytes, const void* ws,
                              CompactLayout& L) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (M < 0) return KVB_EINVAL;
  L = compact_layout(cache, M < cache->cap ? M : cache->cap);
  if (!ws || ws_bytes < L.total) return KVB_EWORKSPACE;
  return KVB_OK;
}

}  // namespace kvb

using namespace kvb;

extern "C" size_t kv_evict_workspace(const kvb_cache* cache, int32_t M) {
  if (!cache_dims_ok(cache) || M < 0 || cache->D < 8) return 0;
  return compact_layout(cache, M < cache->cap ? M : cache->cap).total;
}

extern "C" size_t kv_erase_workspace(const kvb_cache* cache) {
  if (!cache_dims_ok(cache) || cache->D < 8) return 0;
  return compact_layout(cache, cache->cap).total;
}

extern "C" int32_t kv_evict_plan(const kvb_cache* cache, const int32_t* t, int32_t M,
                                 int32_t* evicted_pos, int32_t max_evict, int32_t* n_evicted,
                                 void* ws, size_t ws_bytes, void* stream) {
  CompactLayout L;
  int32_t st = evict_validate(cache, M, ws_bytes, ws, L);
  if (st) return st;
  if (!t || max_evict < 0 || (evicted_pos && max_evict == 0)) return KVB_EINVAL;
  if ((st = check_device())) return st;
  return evict_plan(cache, L, t, M, evicted_pos, max_evict, n_evicted, ws, (hipStream_t)stream);
}

extern "C" int32_t kv_evict_apply(const kvb_cache* cache, int32_t M, void* ws, size_t ws_bytes,
                                  void* stream) {
  CompactLayout L;
  int32_t st = evict_validate(cache, M, ws_bytes, ws, L);
  if (st) return st;
  if ((st = check_device())) return st;
  launch_move(cache, keep_args(cache, L, ws), MODE_EVICT, (hipStream_t)stream);
  return launch_status();
}

extern "C" int32_t kv_evict_to_budget(const kvb_cache* cache, const int32_t* t, int32_t M,
                                      int32_t* evicted_pos, int32_t max_evict,
                                      int32_t* n_evicted, void* ws, size_t ws_bytes,
                                      void* stream) {
  int32_t st = kv_evict_plan(cache, t, M, evicted_pos, max_evict, n_evicted, ws, ws_bytes, stream);
  if (st) return st;
  return kv_evict_apply(cache, M, ws, ws_bytes, stream);
}

extern "C" int32_t kv_evict_one(const kvb_cache* cache, const int32_t* t, int32_t M,
                                int32_t* evicted_pos, int32_t max_evict, int32_t* n_evicted,
                                void* stream) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (!t || M < 0 || max_evict < 0 || (evicted_pos && max_evict == 0)) return KVB_EINVAL;
  if ((st = check_device())) return st;
  OneArgs a;
  a.k = cache->k;
  a.v = cache->v;
  a.log_beta = cache->log_beta;
  a.pos = cache->pos;
  a.len = cache->len;
  a.start = cache->start;
  a.tq = t;
  a.evicted_pos = evicted_pos;
  a.n_out = n_evicted;
  a.cap = cache->cap;
  a.Hkv = cache->Hkv;
  a.M = M;
  a.max_evict = max_evict;
  a.row_bytes = cache->D * (cache->dtype == KVB_BF16 ? 2 : 4);
  hipStream_t s = (hipStream_t)stream;
  TraceScope tr(kTrEvictOne, s);
  hipLaunchKernelGGL(evict_one, dim3(cache->B * cache->Hkv), dim3(kSelThreads), 0, s, a);
  return launch_status();
}

extern "C" int32_t kv_erase_ranges(const kvb_cache* cache, const int32_t* ranges,
                                   const int32_t* n_ranges, int32_t R, int32_t* n_erased,
                                   void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (R < 0 || !n_ranges || (R > 0 && !ranges)) return KVB_EINVAL;
  const CompactLayout L = compact_layout(cache, cache->cap);
  if (!ws || ws_bytes < L.total) return KVB_EWORKSPACE;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  KeepArgs a = keep_args(cache, L, ws);
  a.ranges = ranges;
  a.n_ranges = n_ranges;
  a.R = R;
  a.n_out = n_erased;
  const int U = cache->B * cache->Hkv;
  if (R <= kEraseMaxR && 2 * (size_t)R <= (size_t)L.Tc) {
    // endpoint table in the (otherwise unused) tile-mask area; the largest kept
    // count in the header
    int32_t* ep = (int32_t*)((char*)ws + L.tile_mask);
    int32_t* max_kept = (int32_t*)((char*)ws + kWsMaxKept);
    if (R > 0) {
      TraceScope tr(kTrEraseSearch, s);
      hipLaunchKernelGGL(erase_search, dim3((2 * R + 3) / 4, U), dim3(256), 0, s, a, ep,
                         max_kept);
    } else {
      TraceScope tr(kTrEraseSearch, s);
      hipLaunchKernelGGL(erase_search, dim3(1, U), dim3(256), 0, s, a, ep, max_kept);
    }
    {
      TraceScope tr(kTrErasePlan, s);
      hipLaunchKernelGGL(erase_plan, dim3(kErasePlanBlocks, U), dim3(kChunkThreads), 0, s, a, ep,
                         max_kept);
    }
    launch_move(cache, a, MODE_ERASE, s, max_kept, 4096);
    return launch_status();
  }
  launch_keep_chunks(cache, a, MODE_ERASE, s);
  launch_move(cache, a, MODE_ERASE, s);
  return launch_status();
}
