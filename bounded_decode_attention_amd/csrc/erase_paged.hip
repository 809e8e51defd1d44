// MEMENTO range erasure over a paged cache, block by block ("MEMENTO: Teaching
// LLMs to Manage Their Own Context", blocks and compression; system engineering:
// a finished thinking block leaves the KV cache as a whole within the same
// generate call).  A head's live tokens sit in 32-slot pages listed in position
// order by its page table; a page keeps its live rows in its first fill slots.
// Erasure keeps a token iff its position lies in none of the sequence's ranges, as
// the contiguous form does, but works on pages:
//
//   a page none of whose rows is kept leaves the table (its rows are not read
//     beyond the first and last position, and not written);
//   a page all of whose rows are kept stays as it is;
//   a page with both keeps its kept rows, in order, in its first slots -- the only
//     rows that move, each within its own page.
//
// A caller that starts every thinking block and every memento on a fresh page
// erases whole pages only: the erase then rewrites the page table and moves no row.
//
// Kernels (one thread per logical page, 256 pages per workgroup):
//   pg_classify  reads each page's physical number, fill and first and last
//                position; a page whose position span meets no range keeps every
//                row, one inside a single range keeps none, otherwise its rows are
//                walked against the ranges (positions ascend within a page).
//                Writes the kept-row count and mask and a copy of the table to the
//                workspace, and per workgroup the pages that stay and the rows
//                before and after.
//   pg_apply     each workgroup sums the counts of the workgroups before it (the
//                new index of its first surviving page), scans its pages and
//                writes the new table and fills in place (it reads only the
//                workspace copies), then compacts its partial pages through LDS
//                (all reads of a page before any of its writes).  Workgroup 0 of a
//                head writes n_pages, len and n_erased.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace kvb {

constexpr int kPgThreads = 256;
constexpr int kPgMaxRowBytes = 1024;  // f32, D = 256

struct PgArgs {
  int32_t* table;
  int32_t* fill;
  int32_t* n_pages;
  void* k;
  void* v;
  float* log_beta;
  int32_t* pos;
  int32_t* len;
  const int32_t* ranges;
  const int32_t* n_ranges;
  int32_t* n_erased;
  int32_t R, Hkv, cap, max_pages, NB, row_bytes;
  int32_t* kc;       // [U][max_pages] kept rows of each logical page, -1 past n_pages
  int32_t* tcopy;    // [U][max_pages] the table before the erase
  uint32_t* mask;    // [U][max_pages] kept rows (bit r: row r of the page)
  int32_t* blk;      // [U][NB][3] surviving pages, rows before, rows after
};

struct PgLayout {
  size_t kc, tcopy, mask, blk, total;
  int NB;
};

static PgLayout pg_layout(const kvb_cache* c, const kvb_pages* pg) {
  PgLayout L;
  const size_t U = (size_t)c->B * c->Hkv;
  const size_t mp = (size_t)pg->max_pages;
  L.NB = (int)((mp + kPgThreads - 1) / kPgThreads);
  size_t o = kWsHeader;
  L.kc = o;
  o += align_up(U * mp * 4, 256);
  L.tcopy = o;
  o += align_up(U * mp * 4, 256);
  L.mask = o;
  o += align_up(U * mp * 4, 256);
  L.blk = o;
  o += align_up(U * L.NB * 3 * 4, 256);
  L.total = o;
  return L;
}

// First range of the sequence whose end lies above p (ranges are sorted and
// disjoint, so their ends ascend); nr when there is none.
__device__ __forceinline__ int range_after(const int32_t* rg, int nr, int p) {
  int lo = 0, hi = nr;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (rg[2 * mid + 1] > p) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// Sum of x over the workgroup (all kPgThreads threads call it).
__device__ __forceinline__ int pg_block_sum(int x, int* s_red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[w] = x;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < kPgThreads / 64; ++i) t += s_red[i];
  return t;
}

// Kept rows of one page (count and mask) from its f positions pr[0 .. f).
__device__ __forceinline__ int page_keep(const int32_t* rg, int nr, const int32_t* pr, int f,
                                         uint32_t& m) {
  m = 0u;
  if (f <= 0) return 0;
  const int p0 = pr[0], pl = pr[f - 1];
  int j = range_after(rg, nr, p0);
  if (j >= nr || rg[2 * j] > pl) {
    m = f == 32 ? 0xFFFFFFFFu : (1u << f) - 1u;  // no range meets the page's positions
    return f;
  }
  if (rg[2 * j] <= p0 && rg[2 * j + 1] > pl) return 0;  // one range covers them
  int kc = 0;
  for (int r = 0; r < f; ++r) {
    const int p = pr[r];
    while (j < nr && rg[2 * j + 1] <= p) ++j;
    if (!(j < nr && rg[2 * j] <= p)) {
      m |= 1u << r;
      ++kc;
    }
  }
  return kc;
}

constexpr int kPgLdsRanges = 1024;  // ranges searched in LDS (more: from global memory)

__global__ __launch_bounds__(kPgThreads) void pg_classify(PgArgs a) {
  __shared__ int s_red[kPgThreads / 64];
  __shared__ int32_t s_rg[2 * kPgLdsRanges];
  const int u = blockIdx.y;
  const int b = u / a.Hkv;
  const int i = blockIdx.x * kPgThreads + threadIdx.x;
  const int np = min(max(a.n_pages[u], 0), a.max_pages);
  const int pages = a.cap / 32;
  const int nr = min(max(a.n_ranges[b], 0), a.R);
  const int32_t* rg = a.ranges + (size_t)b * a.R * 2;
  const bool in_lds = nr <= kPgLdsRanges;
  if (in_lds)
    for (int x = threadIdx.x; x < 2 * nr; x += kPgThreads) s_rg[x] = rg[x];
  int kc = -1, f = 0, pe = 0;
  size_t e = 0;
  if (i < a.max_pages) {
    e = (size_t)u * a.max_pages + i;
    pe = a.table[e];
    if (i < np) f = min(max(a.fill[e], 0), 32);
  }
  __syncthreads();
  if (i < a.max_pages) {
    a.tcopy[e] = pe;
    uint32_t m = 0u;
    if (i < np) {
      const int32_t* pr = a.pos + (size_t)u * a.cap + 32 * (size_t)min(max(pe, 0), pages - 1);
      kc = in_lds ? page_keep(s_rg, nr, pr, f, m) : page_keep(rg, nr, pr, f, m);
    }
    a.kc[e] = kc;
    a.mask[e] = m;
  }
  const int surv = pg_block_sum(kc > 0 ? 1 : 0, s_red);
  const int before = pg_block_sum(f, s_red);
  const int after = pg_block_sum(max(kc, 0), s_red);
  if (threadIdx.x == 0) {
    int32_t* o = a.blk + ((size_t)u * a.NB + blockIdx.x) * 3;
    o[0] = surv;
    o[1] = before;
    o[2] = after;
  }
}

__global__ __launch_bounds__(kPgThreads) void pg_apply(PgArgs a) {
  __shared__ int s_red[kPgThreads / 64];
  __shared__ int s_wave[kPgThreads / 64];
  __shared__ int s_list[kPgThreads];
  __shared__ int s_nlist;
  __shared__ uint4 s_rows[32 * kPgMaxRowBytes / 16];
  const int u = blockIdx.y;
  const int tid = threadIdx.x;
  const int32_t* blk = a.blk + (size_t)u * a.NB * 3;
  int base = 0;
  for (int k = tid; k < (int)blockIdx.x; k += kPgThreads) base += blk[3 * k];
  base = pg_block_sum(base, s_red);
  if (blockIdx.x == 0) {
    int pages = 0, before = 0, after = 0;
    for (int k = tid; k < a.NB; k += kPgThreads) {
      pages += blk[3 * k];
      before += blk[3 * k + 1];
      after += blk[3 * k + 2];
    }
    pages = pg_block_sum(pages, s_red);
    before = pg_block_sum(before, s_red);
    after = pg_block_sum(after, s_red);
    if (tid == 0) {
      a.n_pages[u] = pages;
      a.len[u] = after;
      if (a.n_erased) a.n_erased[u] = before - after;
    }
  }
  if (tid == 0) s_nlist = 0;
  const int i = blockIdx.x * kPgThreads + tid;
  const size_t e = (size_t)u * a.max_pages + i;
  const int kc = i < a.max_pages ? a.kc[e] : -1;
  const bool surv = kc > 0;
  // exclusive scan of the surviving pages over the workgroup
  const unsigned long long bal = __ballot(surv);
  const int lane = tid & 63, w = tid >> 6;
  const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) s_wave[w] = __popcll(bal);
  __syncthreads();
  int off = base + in_wave;
  for (int k = 0; k < w; ++k) off += s_wave[k];
  int pe = 0;
  uint32_t m = 0u;
  if (surv) {
    pe = a.tcopy[e];
    m = a.mask[e];
    a.table[(size_t)u * a.max_pages + off] = pe;
    a.fill[(size_t)u * a.max_pages + off] = kc;
    const uint32_t prefix = kc == 32 ? 0xFFFFFFFFu : (1u << kc) - 1u;
    if (m != prefix) s_list[atomicAdd(&s_nlist, 1)] = i;
  }
  __syncthreads();
  // partial pages: kept rows to the page's first slots, through LDS
  const int nl = s_nlist;
  const int pages = a.cap / 32;
  const int units = a.row_bytes / 16;  // 16-byte pieces per row
  for (int li = 0; li < nl; ++li) {
    const size_t el = (size_t)u * a.max_pages + s_list[li];
    const uint32_t lm = a.mask[el];
    const size_t row0 = (size_t)u * a.cap + 32 * (size_t)min(max(a.tcopy[el], 0), pages - 1);
    const int kept = __popc(lm);
    for (int which = 0; which < 2; ++which) {
      uint4* base_ptr = (uint4*)((char*)(which ? a.v : a.k) + row0 * a.row_bytes);
      for (int x = tid; x < 32 * units; x += kPgThreads) {
        const int r = x / units, c = x - r * units;
        if (lm >> r & 1u) {
          const int d = __popc(lm & ((1u << r) - 1u));
          s_rows[d * units + c] = base_ptr[(size_t)r * units + c];
        }
      }
      __syncthreads();
      for (int x = tid; x < kept * units; x += kPgThreads) base_ptr[x] = s_rows[x];
      __syncthreads();
    }
    int32_t pv = 0;
    float lv = 0.f;
    const bool mine = tid < 32 && (lm >> tid & 1u);
    if (mine) {
      pv = a.pos[row0 + tid];
      if (a.log_beta) lv = a.log_beta[row0 + tid];
    }
    __syncthreads();
    if (mine) {
      const int d = __popc(lm & ((1u << tid) - 1u));
      a.pos[row0 + d] = pv;
      if (a.log_beta) a.log_beta[row0 + d] = lv;
    }
    __syncthreads();
  }
}

}  // namespace kvb

using namespace kvb;

extern "C" size_t kv_erase_paged_workspace(const kvb_cache* cache, const kvb_pages* pages) {
  if (!cache_dims_ok(cache) || !pages || pages->max_pages < 1) return 0;
  return pg_layout(cache, pages).total;
}

extern "C" int32_t kv_erase_ranges_paged(const kvb_cache* cache, const kvb_pages* pages,
                                         const int32_t* ranges, const int32_t* n_ranges,
                                         int32_t R, int32_t* n_erased, void* ws,
                                         size_t ws_bytes, void* stream) {
  int32_t st = check_cache(cache, true);
  if (st) return st;
  if (!pages || !pages->table || !pages->fill || !pages->n_pages || pages->max_pages < 1)
    return KVB_EINVAL;
  if (cache->start || cache->cap % 32 != 0) return KVB_EINVAL;
  if (R < 0 || !n_ranges || (R > 0 && !ranges)) return KVB_EINVAL;
  const int row_bytes = cache->D * (cache->dtype == KVB_BF16 ? 2 : 4);
  if (row_bytes % 16 != 0 || row_bytes > kPgMaxRowBytes) return KVB_EUNSUPPORTED;
  const long long U = (long long)cache->B * cache->Hkv;
  if (U > 65535) return KVB_EUNSUPPORTED;
  const PgLayout L = pg_layout(cache, pages);
  if (!ws || ws_bytes < L.total) return KVB_EWORKSPACE;
  if ((st = check_device())) return st;
  PgArgs a;
  a.table = pages->table;
  a.fill = pages->fill;
  a.n_pages = pages->n_pages;
  a.k = cache->k;
  a.v = cache->v;
  a.log_beta = cache->log_beta;
  a.pos = cache->pos;
  a.len = cache->len;
  a.ranges = ranges;
  a.n_ranges = n_ranges;
  a.n_erased = n_erased;
  a.R = R;
  a.Hkv = cache->Hkv;
  a.cap = cache->cap;
  a.max_pages = pages->max_pages;
  a.NB = L.NB;
  a.row_bytes = row_bytes;
  a.kc = (int32_t*)((char*)ws + L.kc);
  a.tcopy = (int32_t*)((char*)ws + L.tcopy);
  a.mask = (uint32_t*)((char*)ws + L.mask);
  a.blk = (int32_t*)((char*)ws + L.blk);
  hipStream_t s = (hipStream_t)stream;
  TraceScope tr(kTrErasePages, s);
  const dim3 grid(L.NB, (unsigned)U);
  hipLaunchKernelGGL(pg_classify, grid, dim3(kPgThreads), 0, s, a);
  hipLaunchKernelGGL(pg_apply, grid, dim3(kPgThreads), 0, s, a);
  return launch_status();
}
