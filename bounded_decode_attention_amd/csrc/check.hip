// Device-side precondition check of a cache descriptor (the conditions the calls
// take as given because testing them on the host would need a synchronisation).
// One workgroup per KV head reads the head's live positions and log beta values
// once (coalesced) and writes the head's violation bits; nothing else is written,
// so the call needs no workspace and can be issued before any other call.
#include "common.h"

namespace kvb {

constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void check_cache_kernel(
    const float* log_beta, const int32_t* pos, const int32_t* len, const int32_t* start,
    int32_t cap, int32_t Hkv, const int32_t* t, const int32_t* ranges,
    const int32_t* n_ranges, int32_t R, int32_t* flags) {
  __shared__ int s_flags;
  const int u = blockIdx.x;
  const int b = u / Hkv;
  if (threadIdx.x == 0) s_flags = 0;
  __syncthreads();
  int f = 0;
  int n = len[u];
  if (n < 0 || n > cap) {
    f |= KVB_CHECK_LEN;
    n = n < 0 ? 0 : cap;
  }
  int s0 = 0;
  if (start) {
    s0 = start[u];
    if (s0 < 0 || s0 >= cap) {
      f |= KVB_CHECK_START;
      s0 = 0;
    }
  }
  const size_t row0 = (size_t)u * cap;
  auto slot = [&](int i) { return s0 + i < cap ? s0 + i : s0 + i - cap; };
  const int tb = t ? t[b] : 0;
  for (int i = threadIdx.x; i < n; i += kCheckThreads) {
    const int p = pos[row0 + slot(i)];
    if (i + 1 < n && pos[row0 + slot(i + 1)] <= p) f |= KVB_CHECK_POS_ORDER;
    if (t && p > tb) f |= KVB_CHECK_POS_AFTER_T;
    if (log_beta) {
      const float l = log_beta[row0 + slot(i)];
      if (l != l) f |= KVB_CHECK_LOG_BETA_NAN;
      else if (l > 0.f) f |= KVB_CHECK_LOG_BETA_POSITIVE;
    }
  }
  if (n_ranges) {
    const int nr = n_ranges[b];
    if (nr < 0 || nr > R) f |= KVB_CHECK_RANGES;
    const int m = nr < 0 ? 0 : (nr > R ? R : nr);
    const int32_t* rg = ranges + (size_t)b * R * 2;
    for (int r = threadIdx.x; r < m; r += kCheckThreads) {
      if (rg[2 * r] >= rg[2 * r + 1]) f |= KVB_CHECK_RANGES;
      if (r + 1 < m && rg[2 * r + 1] > rg[2 * r + 2]) f |= KVB_CHECK_RANGES;
    }
  }
  if (f) atomicOr(&s_flags, f);
  __syncthreads();
  if (threadIdx.x == 0) flags[u] = s_flags;
}

// The paged form: one workgroup per KV head, one thread per (logical page, row),
// the page's rows coalesced.  A physical page listed twice, or pages out of
// position order, show as positions that do not increase along the sequence.
__global__ __launch_bounds__(kCheckThreads) void check_pages_kernel(
    const float* log_beta, const int32_t* pos, const int32_t* len, int32_t cap, int32_t Hkv,
    const int32_t* table, const int32_t* fill, const int32_t* n_pages, int32_t max_pages,
    const int32_t* t, int32_t* flags) {
  __shared__ int s_flags, s_total;
  const int u = blockIdx.x;
  const int b = u / Hkv;
  if (threadIdx.x == 0) {
    s_flags = 0;
    s_total = 0;
  }
  __syncthreads();
  int f = 0;
  int np = n_pages[u];
  if (np < 0 || np > max_pages) {
    f |= KVB_CHECK_PAGES;
    np = np < 0 ? 0 : max_pages;
  }
  const int pages = cap / 32;
  const size_t row0 = (size_t)u * cap;
  const int32_t* tab = table + (size_t)u * max_pages;
  const int32_t* fil = fill + (size_t)u * max_pages;
  const int tb = t ? t[b] : 0;
  // page i's physical page and fill, or -1 when malformed (reported, not read)
  auto page = [&](int i, int& fl) {
    const int pe = tab[i];
    fl = fil[i];
    return (pe < 0 || pe >= pages || fl < 1 || fl > 32) ? -1 : pe;
  };
  int total = 0;
  for (int x = threadIdx.x; x < 32 * np; x += kCheckThreads) {
    const int i = x >> 5, r = x & 31;
    int fl;
    const int pe = page(i, fl);
    if (pe < 0) {
      if (r == 0) f |= KVB_CHECK_PAGES;
      continue;
    }
    if (r >= fl) continue;
    if (r == 0) total += fl;
    const size_t at = row0 + 32 * (size_t)pe + r;
    const int p = pos[at];
    if (r + 1 < fl) {
      if (pos[at + 1] <= p) f |= KVB_CHECK_POS_ORDER;
    } else if (i + 1 < np) {
      int fn;
      const int pn = page(i + 1, fn);
      if (pn >= 0 && pos[row0 + 32 * (size_t)pn] <= p) f |= KVB_CHECK_POS_ORDER;
    }
    if (t && p > tb) f |= KVB_CHECK_POS_AFTER_T;
    if (log_beta) {
      const float l = log_beta[at];
      if (l != l) f |= KVB_CHECK_LOG_BETA_NAN;
      else if (l > 0.f) f |= KVB_CHECK_LOG_BETA_POSITIVE;
    }
  }
  if (f) atomicOr(&s_flags, f);
  if (total) atomicAdd(&s_total, total);
  __syncthreads();
  if (threadIdx.x == 0) flags[u] = s_flags | (s_total != len[u] ? KVB_CHECK_LEN : 0);
}

}  // namespace kvb

using namespace kvb;

extern "C" int32_t kv_check_pages(const kvb_cache* cache, const kvb_pages* pages,
                                  const int32_t* t, int32_t* flags, void* stream) {
  int32_t st = check_cache(cache, false);
  if (st) return st;
  if (!flags || !pages || !pages->table || !pages->fill || !pages->n_pages ||
      pages->max_pages < 1 || pages->max_pages > (1 << 25) || cache->cap % 32 != 0 ||
      cache->start)
    return KVB_EINVAL;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(check_pages_kernel, dim3(cache->B * cache->Hkv), dim3(kCheckThreads), 0, s,
                     cache->log_beta, cache->pos, cache->len, cache->cap, cache->Hkv,
                     pages->table, pages->fill, pages->n_pages, pages->max_pages, t, flags);
  return launch_status();
}

extern "C" int32_t kv_check_cache(const kvb_cache* cache, const int32_t* t, const int32_t* ranges,
                                  const int32_t* n_ranges, int32_t R, int32_t* flags,
                                  void* stream) {
  int32_t st = check_cache(cache, false);
  if (st) return st;
  if (!flags || R < 0 || (n_ranges && R > 0 && !ranges)) return KVB_EINVAL;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(check_cache_kernel, dim3(cache->B * cache->Hkv), dim3(kCheckThreads), 0, s,
                     cache->log_beta, cache->pos, cache->len, cache->start, cache->cap,
                     cache->Hkv, t, ranges, n_ranges, R, flags);
  return launch_status();
}
