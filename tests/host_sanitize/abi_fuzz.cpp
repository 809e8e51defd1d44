// Host-side checker of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// The library's host code (argument validation, workspace sizing, the trace table,
// the device check) is compiled with both sanitizers and without its kernels, and
// linked into this program, which runs on a machine with no GPU.  Every entry point
// is called with a well-formed argument set whose device pointers are fake (distinct,
// 16-byte aligned addresses that are never mapped), then with each argument replaced
// in turn by values that break it (NULL, misaligned, zero, negative, huge, NaN), then
// with seeded random combinations of such replacements.  Every call must return one
// of the documented kvb_status codes; a dereference of a fake pointer, an overflow in
// a size computation or any other report of either sanitizer aborts the run.  A call
// that passes validation needs the device and returns KVB_EDEVICE; none may return
// KVB_OK with work to do, since nothing can be launched here.
//
// Output: one line "calls=<n> edevice=<n> rejected=<n>" on success.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <functional>
#include <string>
#include <vector>

#include "kvbound.h"

extern "C" const char* __asan_default_options() { return "detect_leaks=0"; }

namespace {

// fake device addresses: far from anything the process maps, 1 MiB apart
void* fake(int i) { return (void*)(uintptr_t)(0x5f0000000000ull + (uint64_t)i * 0x100000ull); }

struct Args {
  kvb_cache c;
  kvb_pages pg;
  const void* q;
  const int32_t* t;
  float scale, lam, eps;
  const void *k_new, *v_new;
  const float* lb_new;
  int32_t Hq, M, splits, max_evict, R, K, K1, m, B, Hkv, D, H, N, L, chunks, iters, phase;
  int32_t *evicted_pos, *n_evicted, *flags, *status, *idx, *assign, *counts;
  const int32_t *ranges, *n_ranges, *spare, *offs, *kid;
  float *out, *lse, *out_lse, *mem_M, *mem_b, *a, *centroids, *log_zbar_w;
  const float *self_out, *self_lse, *log_zbar, *W_o, *w_g, *c_g;
  const void *cent, *abar, *c1, *x, *kk, *vv;
  void *abar_w, *cent_bf16;
  void* ws;
  size_t wsb;
  void* ws2;
  size_t wsb2;
  void* stream;
};

Args base() {
  Args a;
  memset(&a, 0, sizeof(a));
  int f = 0;
  a.c.k = fake(f++);
  a.c.v = fake(f++);
  a.c.log_beta = (float*)fake(f++);
  a.c.pos = (int32_t*)fake(f++);
  a.c.len = (int32_t*)fake(f++);
  a.c.B = 2;
  a.c.Hkv = 2;
  a.c.cap = 4096;
  a.c.D = 128;
  a.c.dtype = KVB_BF16;
  a.c.start = nullptr;
  a.pg.table = (int32_t*)fake(f++);
  a.pg.fill = (int32_t*)fake(f++);
  a.pg.n_pages = (int32_t*)fake(f++);
  a.pg.max_pages = 128;
  a.q = fake(f++);
  a.t = (const int32_t*)fake(f++);
  a.scale = 0.0f;
  a.lam = 0.99f;
  a.eps = 1e-6f;
  a.k_new = fake(f++);
  a.v_new = fake(f++);
  a.lb_new = (const float*)fake(f++);
  a.Hq = 8;
  a.M = 1024;
  a.splits = 0;
  a.max_evict = 4096;
  a.R = 16;
  a.K = 256;
  a.K1 = 16;
  a.m = 4;
  a.B = 2;
  a.Hkv = 2;
  a.D = 128;
  a.H = 2;
  a.N = 1024;
  a.L = 512;
  a.chunks = 2;
  a.iters = 3;
  a.phase = 1;
  a.evicted_pos = (int32_t*)fake(f++);
  a.n_evicted = (int32_t*)fake(f++);
  a.flags = (int32_t*)fake(f++);
  a.status = (int32_t*)fake(f++);
  a.idx = (int32_t*)fake(f++);
  a.assign = (int32_t*)fake(f++);
  a.counts = (int32_t*)fake(f++);
  a.ranges = (const int32_t*)fake(f++);
  a.n_ranges = (const int32_t*)fake(f++);
  a.spare = (const int32_t*)fake(f++);
  a.offs = (const int32_t*)fake(f++);
  a.kid = (const int32_t*)fake(f++);
  a.out = (float*)fake(f++);
  a.lse = (float*)fake(f++);
  a.out_lse = (float*)fake(f++);
  a.mem_M = (float*)fake(f++);
  a.mem_b = (float*)fake(f++);
  a.a = (float*)fake(f++);
  a.centroids = (float*)fake(f++);
  a.log_zbar_w = (float*)fake(f++);
  a.self_out = (const float*)fake(f++);
  a.self_lse = (const float*)fake(f++);
  a.log_zbar = (const float*)fake(f++);
  a.W_o = (const float*)fake(f++);
  a.w_g = (const float*)fake(f++);
  a.c_g = (const float*)fake(f++);
  a.cent = fake(f++);
  a.abar = fake(f++);
  a.c1 = fake(f++);
  a.x = fake(f++);
  a.kk = fake(f++);
  a.vv = fake(f++);
  a.abar_w = fake(f++);
  a.cent_bf16 = fake(f++);
  a.ws = fake(f++);
  a.wsb = (size_t)1 << 40;
  a.ws2 = fake(f++);
  a.wsb2 = (size_t)1 << 40;
  a.stream = nullptr;
  return a;
}

using Mut = std::function<void(Args&)>;

int32_t sat(long long x) { return (int32_t)(x > INT32_MAX ? INT32_MAX : x < INT32_MIN ? INT32_MIN : x); }

// replacement values
const int32_t kInts[] = {0, -1, 1, 3, 7, 64, 65, 100000, 1 << 20, 1 << 30, INT32_MAX, INT32_MIN};
const float kFloats[] = {NAN, INFINITY, -INFINITY, 0.0f, -1.0f, 1e30f};
const size_t kSizes[] = {0, 1, 255, (size_t)1 << 20, SIZE_MAX};

template <typename P>
void ptr_muts(std::vector<Mut>& v, P Args::*field) {
  v.push_back([field](Args& a) { a.*field = nullptr; });
  v.push_back([field](Args& a) { a.*field = (P)((uintptr_t)(a.*field) + 8); });
  v.push_back([field](Args& a) { a.*field = (P)((uintptr_t)(a.*field) + 2); });
}
template <typename P>
void cptr_muts(std::vector<Mut>& v, P kvb_cache::*field) {
  v.push_back([field](Args& a) { a.c.*field = nullptr; });
  v.push_back([field](Args& a) { a.c.*field = (P)((uintptr_t)(a.c.*field) + 8); });
  v.push_back([field](Args& a) { a.c.*field = (P)((uintptr_t)(a.c.*field) + 4); });
}

std::vector<Mut> mutations() {
  std::vector<Mut> v;
  cptr_muts(v, &kvb_cache::k);
  cptr_muts(v, &kvb_cache::v);
  cptr_muts(v, &kvb_cache::log_beta);
  cptr_muts(v, &kvb_cache::pos);
  cptr_muts(v, &kvb_cache::len);
  v.push_back([](Args& a) { a.c.start = (int32_t*)fake(900); });
  for (int32_t x : kInts) {
    v.push_back([x](Args& a) { a.c.B = x; });
    v.push_back([x](Args& a) { a.c.Hkv = x; });
    v.push_back([x](Args& a) { a.c.cap = x; });
    v.push_back([x](Args& a) { a.c.D = x; });
    v.push_back([x](Args& a) { a.c.dtype = x; });
    v.push_back([x](Args& a) { a.pg.max_pages = x; });
    for (int32_t Args::*f : {&Args::Hq, &Args::M, &Args::splits, &Args::max_evict, &Args::R,
                             &Args::K, &Args::K1, &Args::m, &Args::B, &Args::Hkv, &Args::D,
                             &Args::H, &Args::N, &Args::L, &Args::chunks, &Args::iters,
                             &Args::phase})
      v.push_back([x, f](Args& a) { a.*f = x; });
  }
  v.push_back([](Args& a) { a.c.dtype = KVB_F32; a.c.D = 64; });
  v.push_back([](Args& a) { a.c.dtype = KVB_F32; a.c.D = 256; });
  v.push_back([](Args& a) { a.c.dtype = KVB_F32; a.c.D = 264; });
  v.push_back([](Args& a) { a.c.D = 64; a.D = 64; });
  v.push_back([](Args& a) { a.c.B = 1 << 15; a.c.Hkv = 1 << 15; });
  v.push_back([](Args& a) { a.c.B = 1 << 10; a.c.Hkv = 1 << 10; a.c.cap = (1 << 30) - 32; });
  v.push_back([](Args& a) { a.c.start = (int32_t*)fake(900); a.pg.max_pages = 1; });
  v.push_back([](Args& a) { a.Hq = sat((long long)a.c.Hkv * 3); });
  v.push_back([](Args& a) { a.Hq = sat((long long)a.c.Hkv * 64); });
  v.push_back([](Args& a) { a.M = a.c.cap; });
  v.push_back([](Args& a) { a.M = sat((long long)a.c.cap + 1); });
  v.push_back([](Args& a) { a.R = 4097; });
  v.push_back([](Args& a) { a.K = 1 << 24; a.K1 = 1 << 12; a.m = 1 << 12; });
  v.push_back([](Args& a) { a.N = INT32_MAX; a.L = INT32_MAX; a.chunks = INT32_MAX; });
  for (float x : kFloats) {
    v.push_back([x](Args& a) { a.scale = x; });
    v.push_back([x](Args& a) { a.lam = x; });
    v.push_back([x](Args& a) { a.eps = x; });
  }
  for (size_t x : kSizes) {
    v.push_back([x](Args& a) { a.wsb = x; });
    v.push_back([x](Args& a) { a.wsb2 = x; });
  }
  ptr_muts(v, &Args::q);
  ptr_muts(v, &Args::t);
  ptr_muts(v, &Args::k_new);
  ptr_muts(v, &Args::v_new);
  ptr_muts(v, &Args::lb_new);
  ptr_muts(v, &Args::ws);
  ptr_muts(v, &Args::ws2);
  ptr_muts(v, &Args::out);
  ptr_muts(v, &Args::lse);
  ptr_muts(v, &Args::out_lse);
  ptr_muts(v, &Args::evicted_pos);
  ptr_muts(v, &Args::n_evicted);
  ptr_muts(v, &Args::flags);
  ptr_muts(v, &Args::status);
  ptr_muts(v, &Args::idx);
  ptr_muts(v, &Args::assign);
  ptr_muts(v, &Args::counts);
  ptr_muts(v, &Args::ranges);
  ptr_muts(v, &Args::n_ranges);
  ptr_muts(v, &Args::spare);
  ptr_muts(v, &Args::offs);
  ptr_muts(v, &Args::kid);
  ptr_muts(v, &Args::mem_M);
  ptr_muts(v, &Args::mem_b);
  ptr_muts(v, &Args::a);
  ptr_muts(v, &Args::centroids);
  ptr_muts(v, &Args::log_zbar_w);
  ptr_muts(v, &Args::self_out);
  ptr_muts(v, &Args::self_lse);
  ptr_muts(v, &Args::log_zbar);
  ptr_muts(v, &Args::W_o);
  ptr_muts(v, &Args::w_g);
  ptr_muts(v, &Args::c_g);
  ptr_muts(v, &Args::cent);
  ptr_muts(v, &Args::abar);
  ptr_muts(v, &Args::c1);
  ptr_muts(v, &Args::x);
  ptr_muts(v, &Args::kk);
  ptr_muts(v, &Args::vv);
  ptr_muts(v, &Args::abar_w);
  ptr_muts(v, &Args::cent_bf16);
  v.push_back([](Args& a) { a.pg.table = nullptr; });
  v.push_back([](Args& a) { a.pg.fill = nullptr; });
  v.push_back([](Args& a) { a.pg.n_pages = nullptr; });
  return v;
}

struct Call {
  const char* name;
  std::function<int32_t(Args&)> fn;
};

std::vector<Call> calls() {
  std::vector<Call> v;
  v.push_back({"kv_attn_decode", [](Args& a) {
                 return kv_attn_decode(&a.c, a.q, a.Hq, a.t, a.scale, a.k_new, a.v_new, a.lb_new,
                                       a.splits, a.out, a.lse, a.ws, a.wsb, a.stream);
               }});
  v.push_back({"kv_attn_decode(no decode token)", [](Args& a) {
                 return kv_attn_decode(&a.c, a.q, a.Hq, a.t, a.scale, nullptr, nullptr, nullptr,
                                       a.splits, a.out, a.lse, a.ws, a.wsb, a.stream);
               }});
  v.push_back({"kv_attn_decode(NULL cache)", [](Args& a) {
                 return kv_attn_decode(nullptr, a.q, a.Hq, a.t, a.scale, nullptr, nullptr, nullptr,
                                       a.splits, a.out, a.lse, a.ws, a.wsb, a.stream);
               }});
  v.push_back({"kv_attn_decode_noalloc", [](Args& a) {
                 return kv_attn_decode_noalloc(&a.c, a.q, a.Hq, a.t, a.scale, a.k_new, a.v_new,
                                               a.lb_new, a.splits, a.out, a.lse, a.status, a.stream);
               }});
  v.push_back({"kv_check_cache", [](Args& a) {
                 return kv_check_cache(&a.c, a.t, a.ranges, a.n_ranges, a.R, a.flags, a.stream);
               }});
  v.push_back({"kv_check_cache(no ranges)", [](Args& a) {
                 return kv_check_cache(&a.c, a.t, nullptr, nullptr, 0, a.flags, a.stream);
               }});
  v.push_back({"kv_check_pages", [](Args& a) {
                 return kv_check_pages(&a.c, &a.pg, a.t, a.flags, a.stream);
               }});
  v.push_back({"kv_check_pages(NULL pages)", [](Args& a) {
                 return kv_check_pages(&a.c, nullptr, a.t, a.flags, a.stream);
               }});
  v.push_back({"kv_append", [](Args& a) {
                 return kv_append(&a.c, a.k_new, a.v_new, a.lb_new, a.t, a.ws, a.wsb, a.stream);
               }});
  v.push_back({"kv_evict_to_budget", [](Args& a) {
                 return kv_evict_to_budget(&a.c, a.t, a.M, a.evicted_pos, a.max_evict, a.n_evicted,
                                           a.ws, a.wsb, a.stream);
               }});
  v.push_back({"kv_evict_to_budget(no outputs)", [](Args& a) {
                 return kv_evict_to_budget(&a.c, a.t, a.M, nullptr, 0, nullptr, a.ws, a.wsb,
                                           a.stream);
               }});
  v.push_back({"kv_evict_plan", [](Args& a) {
                 return kv_evict_plan(&a.c, a.t, a.M, a.evicted_pos, a.max_evict, a.n_evicted, a.ws,
                                      a.wsb, a.stream);
               }});
  v.push_back({"kv_evict_apply", [](Args& a) {
                 return kv_evict_apply(&a.c, a.M, a.ws, a.wsb, a.stream);
               }});
  v.push_back({"kv_evict_one", [](Args& a) {
                 return kv_evict_one(&a.c, a.t, a.M, a.evicted_pos, a.max_evict, a.n_evicted,
                                     a.stream);
               }});
  v.push_back({"kv_attn_decode_evict_one", [](Args& a) {
                 return kv_attn_decode_evict_one(&a.c, a.q, a.Hq, a.t, a.scale, a.k_new, a.v_new,
                                                 a.lb_new, a.M, a.splits, a.out, a.lse,
                                                 a.evicted_pos, a.max_evict, a.n_evicted, a.ws,
                                                 a.wsb, a.stream);
               }});
  v.push_back({"kv_attn_decode_plan_one", [](Args& a) {
                 return kv_attn_decode_plan_one(&a.c, a.q, a.Hq, a.t, a.scale, a.k_new, a.v_new,
                                                a.lb_new, a.splits, a.out, a.lse, a.ws, a.wsb,
                                                a.ws2, a.wsb2, a.stream);
               }});
  v.push_back({"kv_evict_one_apply", [](Args& a) {
                 return kv_evict_one_apply(&a.c, a.t, a.M, a.evicted_pos, a.max_evict, a.n_evicted,
                                           a.ws2, a.wsb2, a.stream);
               }});
  v.push_back({"kv_attn_decode_compact", [](Args& a) {
                 return kv_attn_decode_compact(&a.c, a.q, a.Hq, a.t, a.scale, a.M, a.splits,
                                               a.phase, a.out, a.lse, a.ws, a.wsb, a.ws2, a.wsb2,
                                               a.stream);
               }});
  v.push_back({"kv_attn_decode_paged", [](Args& a) {
                 return kv_attn_decode_paged(&a.c, &a.pg, a.q, a.Hq, a.t, a.scale, a.k_new,
                                             a.v_new, a.lb_new, a.spare, a.splits, a.out, a.lse,
                                             a.ws, a.wsb, a.stream);
               }});
  v.push_back({"kv_attn_decode_paged(NULL pages)", [](Args& a) {
                 return kv_attn_decode_paged(&a.c, nullptr, a.q, a.Hq, a.t, a.scale, nullptr,
                                             nullptr, nullptr, nullptr, a.splits, a.out, a.lse,
                                             a.ws, a.wsb, a.stream);
               }});
  v.push_back({"kv_erase_ranges_paged", [](Args& a) {
                 return kv_erase_ranges_paged(&a.c, &a.pg, a.ranges, a.n_ranges, a.R, a.n_evicted,
                                              a.ws, a.wsb, a.stream);
               }});
  v.push_back({"kv_erase_ranges", [](Args& a) {
                 return kv_erase_ranges(&a.c, a.ranges, a.n_ranges, a.R, a.n_evicted, a.ws, a.wsb,
                                        a.stream);
               }});
  v.push_back({"asm_lookup_merge", [](Args& a) {
                 return asm_lookup_merge(a.q, a.B, a.Hq, a.Hkv, a.D, a.cent, a.abar, a.log_zbar,
                                         a.K, a.self_out, a.self_lse, a.out, a.out_lse, a.idx, a.ws,
                                         a.wsb, a.stream);
               }});
  v.push_back({"kv_attn_decode_asm", [](Args& a) {
                 return kv_attn_decode_asm(&a.c, a.q, a.Hq, a.t, a.scale, a.k_new, a.v_new,
                                           a.lb_new, a.splits, a.cent, a.abar, a.log_zbar, a.K,
                                           a.out, a.lse, a.idx, a.ws, a.wsb, a.stream);
               }});
  v.push_back({"asm_lookup_merge_hier", [](Args& a) {
                 return asm_lookup_merge_hier(a.q, a.B, a.Hq, a.Hkv, a.D, a.c1, a.K1, a.offs,
                                              a.cent, a.kid, a.K, a.m, a.abar, a.log_zbar,
                                              a.self_out, a.self_lse, a.out, a.out_lse, a.idx,
                                              a.ws, a.wsb, a.stream);
               }});
  v.push_back({"asm_prefix_states", [](Args& a) {
                 return asm_prefix_states(a.q, a.H, a.N, a.D, a.kk, a.vv, a.L, a.chunks, a.scale,
                                          a.a, a.out_lse, a.ws, a.wsb, a.stream);
               }});
  v.push_back({"asm_kmeans", [](Args& a) {
                 return asm_kmeans(a.x, a.H, a.N, a.D, a.centroids, a.K, a.iters, a.assign,
                                   a.counts, a.cent_bf16, a.ws, a.wsb, a.stream);
               }});
  v.push_back({"asm_aggregate_states", [](Args& a) {
                 return asm_aggregate_states(a.assign, a.a, a.out_lse, a.H, a.N, a.D, a.K,
                                             a.abar_w, a.log_zbar_w, a.stream);
               }});
  v.push_back({"asm_build_memory", [](Args& a) {
                 return asm_build_memory(a.q, a.H, a.N, a.D, a.kk, a.vv, a.L, a.chunks, a.scale,
                                         a.centroids, a.K, a.iters, a.cent_bf16, a.abar_w,
                                         a.log_zbar_w, a.assign, a.ws, a.wsb, a.stream);
               }});
  v.push_back({"kv_latent_absorb", [](Args& a) {
                 return kv_latent_absorb(&a.c, a.M, a.ws2, a.wsb2, a.lam, a.mem_M, a.mem_b, a.ws,
                                         a.wsb, a.stream);
               }});
  v.push_back({"kv_latent_read", [](Args& a) {
                 return kv_latent_read(a.q, a.B, a.Hq, a.Hkv, a.D, a.mem_M, a.mem_b, a.W_o, a.w_g,
                                       a.c_g, a.eps, a.out, a.stream);
               }});
  // host-only queries: any value is fine, the sanitizers judge them
  v.push_back({"workspace sizes", [](Args& a) {
                 volatile size_t s = 0;
                 s += kv_attn_decode_workspace(&a.c, a.Hq, a.splits);
                 s += kv_evict_workspace(&a.c, a.M);
                 s += kv_erase_workspace(&a.c);
                 s += asm_lookup_merge_workspace(a.B, a.Hq, a.Hkv, a.D, a.K);
                 s += asm_lookup_merge_hier_workspace(a.B, a.Hq, a.Hkv, a.K1, a.m);
                 s += asm_prefix_states_workspace(a.H, a.N, a.D, a.L, a.chunks);
                 s += asm_kmeans_workspace(a.H, a.K, a.D);
                 s += kv_latent_absorb_workspace(&a.c);
                 s += asm_build_memory_workspace(a.H, a.N, a.D, a.L, a.chunks, a.K);
                 s += kv_attn_decode_evict_one_workspace(&a.c, a.Hq, a.splits);
                 s += kv_evict_one_workspace(&a.c, a.splits);
                 s += kv_erase_paged_workspace(&a.c, &a.pg);
                 s += kv_attn_decode_asm_workspace(&a.c, a.Hq, a.splits, a.K);
                 s += kv_attn_decode_workspace(nullptr, a.Hq, a.splits);
                 s += kv_evict_workspace(nullptr, a.M);
                 s += kv_erase_paged_workspace(&a.c, nullptr);
                 volatile int32_t n = kv_attn_decode_splits(&a.c, a.Hq);
                 n = kv_attn_decode_asm_splits(&a.c, a.Hq, a.K);
                 n = kv_attn_decode_splits(nullptr, a.Hq);
                 (void)n;
                 (void)s;
                 return (int32_t)KVB_EDEVICE;
               }});
  return v;
}

uint64_t rng = 0x9e3779b97f4a7c15ull;
uint32_t next_u32() {  // splitmix64
  uint64_t z = (rng += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return (uint32_t)((z ^ (z >> 31)) >> 32);
}

long n_calls = 0, n_edevice = 0, n_rejected = 0;

void check(const Call& c, Args& a, const std::string& what) {
  const int32_t st = c.fn(a);
  ++n_calls;
  if (st == KVB_EDEVICE) ++n_edevice;
  else if (st < 0 && st >= KVB_ERANGE) ++n_rejected;
  else {
    fprintf(stderr, "FAIL %s (%s): returned %d without a device\n", c.name, what.c_str(), st);
    exit(2);
  }
  (void)kvb_strerror(st);
}

}  // namespace

int main(int argc, char** argv) {
  const long n_random = argc > 1 ? atol(argv[1]) : 20000;
  for (int s = -64; s <= 64; ++s)
    if (!kvb_strerror(s)) {
      fprintf(stderr, "FAIL kvb_strerror(%d) is NULL\n", s);
      return 2;
    }
  (void)kvb_strerror(INT32_MIN);
  (void)kvb_strerror(INT32_MAX);

  // trace table: bounds and sequences without a device
  for (int32_t cap : {INT32_MIN, -1, 0, 1, 64, (1 << 20) + 1, INT32_MAX}) {
    for (int32_t mask : {0, 1, -1}) {
      (void)kvb_trace_enable(cap, mask);
      int32_t ids[4];
      float ms[4];
      (void)kvb_trace_read(ids, ms, 4);
      (void)kvb_trace_read(nullptr, nullptr, 0);
      (void)kvb_trace_read(ids, ms, -1);
      kvb_trace_reset();
    }
  }
  kvb_trace_disable();
  kvb_trace_disable();

  const std::vector<Mut> muts = mutations();
  const std::vector<Call> cs = calls();
  // the well-formed set reaches the device check in every call
  for (const Call& c : cs) {
    Args a = base();
    const int32_t st = c.fn(a);
    if (st != KVB_EDEVICE && strstr(c.name, "NULL") == nullptr) {
      fprintf(stderr, "FAIL %s: well-formed arguments returned %d, not KVB_EDEVICE\n", c.name,
              st);
      return 2;
    }
  }
  // one argument broken at a time
  for (const Call& c : cs)
    for (size_t i = 0; i < muts.size(); ++i) {
      Args a = base();
      muts[i](a);
      check(c, a, "mutation " + std::to_string(i));
    }
  // seeded random combinations of two to six broken arguments
  for (long r = 0; r < n_random; ++r) {
    Args a = base();
    const int k = 2 + (int)(next_u32() % 5);
    std::string what = "combination";
    for (int j = 0; j < k; ++j) {
      const size_t i = next_u32() % muts.size();
      muts[i](a);
      what += " " + std::to_string(i);
    }
    check(cs[next_u32() % cs.size()], a, what);
  }
  printf("calls=%ld edevice=%ld rejected=%ld mutations=%zu entry_points=%zu\n", n_calls,
         n_edevice, n_rejected, muts.size(), cs.size());
  return 0;
}
