/*
 * kvbound -- decode-step attention over a memory-bounded KV cache, for MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a DEVICE pointer unless the comment says
 * "host".  Every call is asynchronous on `stream` (a hipStream_t passed as
 * void*; NULL means the default stream), performs no host synchronisation, and
 * allocates nothing: scratch memory is the caller's workspace `ws` of at least
 * the size the matching *_workspace() function returns (the one exception,
 * kv_attn_decode_noalloc, uses a fixed device-resident scratch array instead).
 * Host-side state is limited to: a per-device cache of the gfx950 check (written
 * once per device, idempotent), the kvb_trace_* event table (process-global, not
 * thread-safe; tracing is a measurement aid), and the per-device address of the
 * no-alloc scratch array (guarded by a mutex).  Results never depend on earlier
 * calls except through the caller's buffers.  Calls on different streams must not
 * share a workspace or a cache.
 *
 * Errors: arguments are validated on the host before anything is launched; a
 * failed check returns a negative kvb_status and leaves all memory untouched.
 * Conditions that live in device memory (e.g. `len`) cannot be checked on the
 * host without a synchronisation; their handling is stated per call.
 *
 * Sources of the operations (web pages, cited by title and section):
 *  [TRIM]  "Cache What Lasts: Token Retention for Memory-Bounded KV Cache in LLMs",
 *          section 2.1 (retention-gated attention: logit q.k + (t-i) log beta_i)
 *          and section 2.2 (inference: over budget M, evict the lowest beta_i^(t-i)).
 *  [ASM]   "Context Memorization for Efficient Long Context Generation",
 *          background (online-softmax identity), method steps 1-4 (attention state
 *          (a, Z), merge operator, cosine-argmax retrieval, merge with the query's
 *          own state), technical novelty (GQA: centroids per KV head).
 *  [IDX]   "IndexMem: Learned KV-Cache Eviction with Latent Memory for Long-Context
 *          LLM Inference", technical summary, section 2 part B (latent memory of
 *          evicted tokens: decayed outer-product fast weights, gated read-out).
 *  [MEM]   "MEMENTO: Teaching LLMs to Manage Their Own Context", blocks and
 *          compression (a finished thinking block's KV entries are removed once its
 *          memento exists) and system engineering (entries physically removed
 *          within one generate call).
 */
#ifndef KVBOUND_H
#define KVBOUND_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVB_OK = 0,
  KVB_EINVAL = -1,       /* a NULL pointer, a size out of range, Hq % Hkv != 0 ... */
  KVB_EUNSUPPORTED = -2, /* dtype / head_dim / group size combination not built */
  KVB_ECAPACITY = -3,    /* cache capacity too small for the request            */
  KVB_EWORKSPACE = -4,   /* ws is NULL or ws_bytes below the required size       */
  KVB_EDEVICE = -5,      /* no usable HIP device, or the device is not gfx950    */
  KVB_ELAUNCH = -6,      /* a kernel launch failed (hipGetLastError)            */
  KVB_ERANGE = -7        /* (workspace status word only) an input value outside the
                            range a kernel's arithmetic supports; it was saturated */
} kvb_status;

typedef enum { KVB_F32 = 0, KVB_BF16 = 1 } kvb_dtype;

/* Size of the device-resident scratch array behind kv_attn_decode_noalloc. */
#define KVB_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * One layer's KV cache; a plain descriptor, read during the call, not retained.
 *   k, v      [B][Hkv][cap][D] elements of `dtype`, dense row-major (one row = one
 *             token of one KV head, D contiguous values).
 *   log_beta  [B][Hkv][cap] float32 natural log of the retention score beta_i of
 *             each slot ([TRIM] 2.1), values in [-inf, 0]; NULL means beta == 1
 *             (no retention bias; eviction then keeps the newest tokens).
 *   pos       [B][Hkv][cap] int32 absolute token position of each slot.  Within
 *             the live slots of a head positions must be strictly increasing.
 *   len       [B][Hkv] int32 live slots per head, device resident; slots at and
 *             beyond len are unspecified.
 *   start     [B][Hkv] int32 first live slot per head, device resident, or NULL
 *             (every head starts at slot 0).  A head's cap slots form a ring: its
 *             i-th live token (position order) is in slot (start[u] + i) mod cap;
 *             the other slots are unspecified.  Requires 0 <= start[u] < cap.
 *             With a start array, eviction compacts each head toward whichever
 *             end moves fewer rows and updates start (see kv_evict_to_budget);
 *             the decode token goes to slot (start + len) mod cap.  Without one,
 *             head u's live slots are 0 .. len[u] - 1.
 * The caller owns all of it.  Requires 1 <= B, Hkv; 1 <= cap < 2^30;
 * D in {64, 128} for KVB_BF16 (any 1 <= D <= 256 for KVB_F32); D % 8 == 0;
 * k, v, log_beta and pos 16-byte aligned (KVB_EINVAL otherwise), as is the query
 * of the attention calls.
 */
typedef struct {
  void* k;
  void* v;
  float* log_beta;
  int32_t* pos;
  int32_t* len;
  int32_t B, Hkv, cap, D;
  int32_t dtype; /* kvb_dtype */
  int32_t* start;
} kvb_cache;

/*
 * Paged form of a cache ([MEM] system engineering: entries removed by whole blocks
 * within one generate call).  A head's live tokens sit in pages of 32 slots; the
 * page table lists its pages in position order.  Physical page p of head u is slots
 * [32p, 32p + 32) of that head's cap slots in the kvb_cache arrays; a page holds
 * its live tokens in its first fill slots, in position order.
 *   table      [B][Hkv][max_pages] int32 physical page of each logical page
 *   fill       [B][Hkv][max_pages] int32 live slots of each logical page, 1..32
 *   n_pages    [B][Hkv] int32 logical pages in use (0..max_pages)
 *   max_pages  entries per head of table and fill
 * The kvb_cache's len holds each head's live-token total (the sum of its fills);
 * its start must be NULL.  Physical pages must lie below cap / 32 and be distinct.
 */
typedef struct {
  int32_t* table;
  int32_t* fill;
  int32_t* n_pages;
  int32_t max_pages;
} kvb_pages;

/* Violation bits written by kv_check_cache, per KV head. */
enum {
  KVB_CHECK_LEN = 1,               /* len < 0 or len > cap                                */
  KVB_CHECK_START = 2,             /* start outside [0, cap)                              */
  KVB_CHECK_POS_ORDER = 4,         /* live positions not strictly increasing along slots  */
  KVB_CHECK_POS_AFTER_T = 8,       /* a live position above t[b] (negative distance)      */
  KVB_CHECK_LOG_BETA_NAN = 16,     /* a live log beta is NaN                              */
  KVB_CHECK_LOG_BETA_POSITIVE = 32,/* a live log beta above 0 (beta > 1)                  */
  KVB_CHECK_RANGES = 64,           /* the sequence's erase ranges: s >= e, unsorted or
                                      overlapping, or n_ranges[b] outside [0, R]          */
  KVB_CHECK_PAGES = 128            /* kv_check_pages: n_pages outside [0, max_pages], a
                                      physical page outside [0, cap / 32) or a fill
                                      outside [1, 32] (the page is then not read)         */
};

/* Human-readable name of a status code (static storage; never NULL). */
const char* kvb_strerror(int32_t status);

/* Number of KV splits kv_attn_decode uses for num_splits == 0 (host only): about
 * 2048 / (B * Hkv), at least one, at most one per 256 slots of capacity. */
int32_t kv_attn_decode_splits(const kvb_cache* cache, int32_t Hq);

/* Workspace sizes in bytes (host only; no device access).  0 when the dimensions are
 * ones the matching call rejects (a descriptor outside the kvb_cache limits, a
 * negative split count, more query rows per KV head than the lookups take). */
size_t kv_attn_decode_workspace(const kvb_cache* cache, int32_t Hq, int32_t num_splits);
size_t kv_evict_workspace(const kvb_cache* cache, int32_t M);
size_t kv_erase_workspace(const kvb_cache* cache);
size_t asm_lookup_merge_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t K);
size_t asm_lookup_merge_hier_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t K1,
                                       int32_t m);
size_t asm_prefix_states_workspace(int32_t H, int32_t N, int32_t D, int32_t L, int32_t chunks);
size_t asm_kmeans_workspace(int32_t H, int32_t K, int32_t D);
size_t kv_latent_absorb_workspace(const kvb_cache* cache);
size_t asm_build_memory_workspace(int32_t H, int32_t N, int32_t D, int32_t L, int32_t chunks,
                                  int32_t K);

/*
 * Decode-step grouped-query attention with the retention bias, split over the KV
 * axis ([TRIM] 2.1; [ASM] background and method steps 1-2).
 *
 * Optional decode token: if k_new != NULL, each head (b, g) gets k_new[b][g],
 * v_new[b][g] (and log_beta_new[b][g] when the cache has log_beta) at slot
 * len[b][g] (start + len mod cap with a start array) with pos = t[b], then
 * len[b][g] += 1, and the attention below covers
 * it.  A head whose len already equals cap is not appended to (its len stays, the
 * token is not attended, and the workspace status word -- the int32 at byte offset
 * 0 of ws -- becomes KVB_ECAPACITY; the caller must keep cap > len).  Every call
 * first resets that word to KVB_OK on the device (a kernel store, so the call can
 * be captured in a HIP graph), so after the call's work completes it holds this
 * call's outcome.  The splits cover the cached slots; the token's own
 * state (logit scale * q.k_new, no bias at distance 0) is merged last, and the row
 * is written by the merge, after every split has read the cache.
 *
 * Then for every query head h of sequence b (KV head g = h / (Hq/Hkv)) over the
 * live slots i < len[b][g]:
 *   s_i   = scale * (q[b][h] . k_i) + (t[b] - pos_i) * log_beta_i
 *           (the bias term is 0 when t[b] == pos_i or log_beta is NULL)
 *   out   = sum_i e^{s_i} v_i / sum_i e^{s_i},   lse = log sum_i e^{s_i}.
 * The live slots are cut into 32-slot tiles dealt to num_splits splits (round
 * robin for D = 128, contiguous runs otherwise); each split yields a partial
 * state (a, m, Z) (a normalised over its tiles, m its max logit, Z = sum e^{s-m}),
 * and the states are combined with the merge operator
 * ((Z_A a_A + Z_B a_B)/(Z_A + Z_B), Z_A + Z_B) in split order (deterministic).
 * An empty head (len == 0, or every weight 0) gives out = 0, lse = -inf.
 *
 *   q          [B][Hq][D] in the cache dtype
 *   Hq         query heads; Hq % Hkv == 0
 *   t          [B] int32 position of each sequence's decode token
 *   scale      dot-product scale; <= 0 selects 1/sqrt(D)
 *   k_new, v_new [B][Hkv][D] cache dtype, or both NULL (no append)
 *   log_beta_new [B][Hkv] float32; required with k_new iff cache->log_beta != NULL
 *   num_splits 0 = kv_attn_decode_splits(); else 1..4096
 *   out        [B][Hq][D] float32;  lse [B][Hq] float32
 *   ws         workspace of kv_attn_decode_workspace(cache, Hq, num_splits) bytes;
 *              after the call it holds the split states: a [B][Hq][num_splits][D]
 *              float32 at byte offset 256, then (m, Z) [B][Hq][num_splits][2]
 *              float32 at the next 256-byte boundary, then (with a decode token)
 *              each head's len before the append [B][Hkv] int32 at the next.
 */
int32_t kv_attn_decode(const kvb_cache* cache, const void* q, int32_t Hq, const int32_t* t,
                       float scale, const void* k_new, const void* v_new,
                       const float* log_beta_new, int32_t num_splits, float* out, float* lse,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * kv_attn_decode without a workspace argument and without any allocation, for
 * callers that cannot allocate: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results as
 * kv_attn_decode (bit for bit, for the same num_splits); the split states live in
 * a device-resident array of KVB_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU
 * holds from the library's load until the process ends.  The array's device
 * address is looked up once per device on the first call made with that device
 * current.
 *   status  [1] int32 device pointer or NULL: receives the call's status word
 *           (KVB_OK, or KVB_ECAPACITY when a head was full; reset by every call);
 *           NULL keeps it in the scratch array, where the caller cannot read it.
 * Returns KVB_EWORKSPACE, launching nothing, when the call would need more than
 * KVB_NOALLOC_SCRATCH_BYTES (kv_attn_decode_workspace(cache, Hq, num_splits) >
 * KVB_NOALLOC_SCRATCH_BYTES; e.g. B * Hq * num_splits * (D + 2) * 4 bytes of split
 * states).  Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that overlap in time on one GPU (different streams, or different
 * host threads) race and give undefined results; serialise them.
 */
int32_t kv_attn_decode_noalloc(const kvb_cache* cache, const void* q, int32_t Hq,
                               const int32_t* t, float scale, const void* k_new,
                               const void* v_new, const float* log_beta_new,
                               int32_t num_splits, float* out, float* lse, int32_t* status,
                               void* stream);

/*
 * Device-side check of the preconditions the other calls take as given ([TRIM] 2.1:
 * positions i <= t and retention scores beta in (0, 1]; [MEM] erase ranges as sorted
 * disjoint half-open position intervals).  For every KV head u = (b, g), flags[u]
 * receives the OR of the KVB_CHECK_* bits the head violates over its live slots
 * (0: none).  A debugging aid: it reads each head's positions and
 * log beta once, writes only flags, and allocates nothing.
 *   t         [B] int32 decode positions, or NULL (no distance check)
 *   ranges    [B][R][2] int32 and n_ranges [B] int32 (as for kv_erase_ranges), or
 *             n_ranges NULL (no range check)
 *   flags     [B][Hkv] int32 (device)
 * Malformed values are only reported: every read stays inside the descriptor's
 * arrays (len is clamped to [0, cap], start to 0 when out of range).
 */
int32_t kv_check_cache(const kvb_cache* cache, const int32_t* t, const int32_t* ranges,
                       const int32_t* n_ranges, int32_t R, int32_t* flags, void* stream);

/*
 * kv_check_cache for the paged form (see kvb_pages; [MEM] system engineering): per
 * KV head, the OR of KVB_CHECK_PAGES (malformed table entry, fill or n_pages),
 * KVB_CHECK_LEN (len differs from the sum of the fills), KVB_CHECK_POS_ORDER
 * (positions not strictly increasing along the head's pages in table order, which is
 * also how a physical page listed twice shows), KVB_CHECK_POS_AFTER_T (with t) and
 * the log beta bits, over the live rows of the well-formed pages.
 *   t      [B] int32 or NULL;  flags [B][Hkv] int32 (device)
 * Requires cap % 32 == 0, start == NULL and max_pages <= 2^25 (KVB_EINVAL otherwise;
 * no head holds more than cap / 32 < 2^25 distinct pages).  Every read stays
 * inside the arrays: n_pages is clamped to [0, max_pages] and a malformed page is
 * not read.
 */
int32_t kv_check_pages(const kvb_cache* cache, const kvb_pages* pages, const int32_t* t,
                       int32_t* flags, void* stream);

/*
 * Append one token per KV head: the same append kv_attn_decode performs when
 * given k_new (slot len, pos = t[b], len += 1; a full head is skipped).  For
 * callers that start eviction planning (kv_evict_plan) as soon as the token is in
 * the cache, concurrently with the attention that follows.
 *   k_new, v_new [B][Hkv][D] cache dtype; log_beta_new [B][Hkv] f32 (required iff
 *   cache->log_beta != NULL); t [B] int32; ws: at least 256 bytes (status word:
 *   reset to KVB_OK by the call, KVB_ECAPACITY if a head was full).
 */
int32_t kv_append(const kvb_cache* cache, const void* k_new, const void* v_new,
                  const float* log_beta_new, const int32_t* t, void* ws, size_t ws_bytes,
                  void* stream);

/*
 * Evict every head over budget to exactly M live slots, then compact in place
 * ([TRIM] 2.2).
 *
 * For a head with n = len > M the key of slot i is
 *   kappa_i = (t[b] - pos_i) * log_beta_i   (exact in double; +0 when t[b] == pos_i
 *                                            or log_beta is NULL; -0 equals +0),
 * the logarithm of the retention score beta_i^(t-i).  The n - M slots that come
 * first in (kappa, pos) ascending order are evicted (ties: lower position first).
 * The surviving rows (k, v, log_beta, pos) move, in their slot order, to slots
 * [0, M) and len becomes M.  Heads with len <= M are untouched.
 * With a start array (slots relative to start, around the ring): a head whose
 * cache fits the single-workgroup planner (about 34K slots on gfx950) is compacted
 * toward whichever end moves fewer rows -- toward its first slot (start kept; the
 * kept rows after the first evicted slot move) or toward its last slot (start +=
 * number evicted, mod cap; the kept rows before the last evicted slot move).  At
 * budget M with one token over, that moves min(e, M - e) rows for an eviction at
 * slot e instead of M - e.  Larger heads are compacted toward their first slot.
 *
 *   t          [B] int32 current token position of each sequence
 *   M          budget, >= 0
 *   evicted_pos [B][Hkv][max_evict] int32 or NULL: the evicted positions of each
 *              head in ascending order; only the first max_evict are written.
 *   n_evicted  [B][Hkv] int32 or NULL: number evicted per head.
 *   ws         workspace of kv_evict_workspace(cache, M) bytes.
 * Preconditions (not checked): positions strictly increasing over live slots,
 * pos <= t, no NaN in log_beta.
 */
int32_t kv_evict_to_budget(const kvb_cache* cache, const int32_t* t, int32_t M,
                           int32_t* evicted_pos, int32_t max_evict, int32_t* n_evicted,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * kv_evict_to_budget in two phases, so that eviction can overlap attention.
 * kv_evict_plan selects the evicted slots and the destination of every kept row,
 * writes evicted_pos / n_evicted, and copies into ws the few kept rows whose
 * source a later move would overwrite; it reads the cache and does not modify it.
 * kv_evict_apply then moves the rows and sets len.  Use the same cache, M and ws
 * for both, apply ordered after plan; between them the cache may be read (e.g. by
 * kv_attn_decode without k_new) but not written.
 */
int32_t kv_evict_plan(const kvb_cache* cache, const int32_t* t, int32_t M, int32_t* evicted_pos,
                      int32_t max_evict, int32_t* n_evicted, void* ws, size_t ws_bytes,
                      void* stream);
int32_t kv_evict_apply(const kvb_cache* cache, int32_t M, void* ws, size_t ws_bytes, void* stream);

/*
 * kv_evict_to_budget for the steady state of bounded decoding, where each step
 * puts a head at most one token over its budget ([TRIM] 2.2, inference: one token
 * in, the lowest-retention token out): in one launch, with no workspace.  A head
 * with n = M + 1 live tokens loses the slot with the lowest (kappa, slot)
 * (kappa as for kv_evict_to_budget) and is compacted exactly as
 * kv_evict_to_budget compacts it: with a start array the rows before the evicted
 * slot move up one slot (start + 1, mod cap) when there are fewer of them than
 * rows after it, otherwise the rows after it move down one slot.  Heads with
 * n <= M are left as they are (n_evicted 0); heads with n > M + 1 are also left as
 * they are, with n_evicted = -(n - M) (use kv_evict_to_budget for them).
 *   t, M, evicted_pos, max_evict, n_evicted as kv_evict_to_budget (at most one
 *   position is written per head).
 */
int32_t kv_evict_one(const kvb_cache* cache, const int32_t* t, int32_t M, int32_t* evicted_pos,
                     int32_t max_evict, int32_t* n_evicted, void* stream);

/*
 * The steady state of bounded decoding, with the eviction's selection folded into
 * the attention ([TRIM] 2.1 and 2.2, inference: one token in, the lowest-retention
 * token out).  The attention's KV splits find, per head, the attended slot with the
 * lowest (kappa, position) (kappa as for kv_evict_to_budget, at t[b]) from the log
 * beta and pos values they load for the retention bias anyway; the merge reduces
 * them and the decode token to the head's evicted slot (ties: lower position first).
 * The attention itself is kv_attn_decode's (same kernels, results bit for bit).
 *
 * kv_attn_decode_evict_one: one call.  Attention with the decode token as
 * kv_attn_decode (k_new may be NULL), then every head with n = M + 1 live tokens
 * (the decode token included) evicts its lowest token, and the decode token is
 * written into the evicted slot instead of being appended (not written at all when
 * it is the evicted token itself; without a decode token the head's last live row
 * moves into the evicted slot): one row per head, len ends at M.  The live tokens
 * are those kv_evict_to_budget keeps; the slots no longer hold them in position
 * order.  The eviction rule compares positions, not slots, so a cache kept this way
 * stays correct for kv_attn_decode, kv_attn_decode_evict_one and kv_append (which
 * need no order); kv_evict_to_budget, kv_evict_plan/apply, kv_evict_one,
 * kv_attn_decode_plan_one, kv_erase_ranges and kv_latent_absorb need position order
 * (kv_check_cache reports KVB_CHECK_POS_ORDER).  Positions must stay distinct.
 * Heads with n <= M get the plain append (n_evicted 0); heads with n > M + 1 too
 * (n_evicted -(n - M)).
 *   M            budget, >= 0
 *   evicted_pos  [B][Hkv][max_evict] int32 or NULL: the evicted position (first entry)
 *   n_evicted    [B][Hkv] int32 or NULL
 *   ws           kv_attn_decode_evict_one_workspace(cache, Hq, num_splits) bytes
 *                (kv_attn_decode's workspace followed by the candidates)
 *
 * kv_attn_decode_plan_one + kv_evict_one_apply: the order-keeping form, in two
 * calls.  kv_attn_decode_plan_one is kv_attn_decode that also plans every head's
 * eviction into ws_evict: the evicted slot, the direction of the shift, and copies
 * of the few rows the shift cannot read in place; it writes nothing else of the
 * cache than kv_attn_decode does.  kv_evict_one_apply then carries out the plan in
 * every head with n = M + 1 live tokens (n as planned), with the same evicted slot,
 * direction and layout, bit for bit, as kv_evict_one / kv_evict_to_budget: with a
 * start array the rows before the evicted slot move up one slot (start + 1, mod
 * cap) when there are fewer of them than rows after it, otherwise the rows after it
 * move down one slot; len becomes M.  Heads with n <= M are left alone (n_evicted
 * 0); heads with n > M + 1 too (n_evicted -(n - M)).  One launch, many workgroups
 * per head.  Between the two calls the cache must not be written; apply may run on
 * another stream once the attention call's work is complete, e.g. beside the next
 * layer's attention.  Using a ws_evict that no kv_attn_decode_plan_one call on this
 * cache filled gives unspecified evictions (every access stays inside the cache and
 * the workspace).
 *   ws_evict    kv_evict_one_workspace(cache, num_splits) bytes, one per cache whose
 *               apply may still be pending
 *   t, M, evicted_pos, max_evict, n_evicted as kv_evict_one (apply; at most one
 *   position is written per head).
 *
 * Both forms: num_splits as kv_attn_decode (0 = kv_attn_decode_splits()); other
 * arguments as kv_attn_decode; supported for B * Hkv <= 65535.
 */
size_t kv_attn_decode_evict_one_workspace(const kvb_cache* cache, int32_t Hq,
                                          int32_t num_splits);
int32_t kv_attn_decode_evict_one(const kvb_cache* cache, const void* q, int32_t Hq,
                                 const int32_t* t, float scale, const void* k_new,
                                 const void* v_new, const float* log_beta_new, int32_t M,
                                 int32_t num_splits, float* out, float* lse,
                                 int32_t* evicted_pos, int32_t max_evict, int32_t* n_evicted,
                                 void* ws, size_t ws_bytes, void* stream);
size_t kv_evict_one_workspace(const kvb_cache* cache, int32_t num_splits);
int32_t kv_attn_decode_plan_one(const kvb_cache* cache, const void* q, int32_t Hq,
                                const int32_t* t, float scale, const void* k_new,
                                const void* v_new, const float* log_beta_new,
                                int32_t num_splits, float* out, float* lse, void* ws,
                                size_t ws_bytes, void* ws_evict, size_t ws_evict_bytes,
                                void* stream);
int32_t kv_evict_one_apply(const kvb_cache* cache, const int32_t* t, int32_t M,
                           int32_t* evicted_pos, int32_t max_evict, int32_t* n_evicted,
                           void* ws_evict, size_t ws_evict_bytes, void* stream);

/*
 * Attention and the planned compaction in one pass over the cache ([TRIM] 2.1 and
 * 2.2): the result equals kv_attn_decode (no append) followed by kv_evict_apply,
 * for a plan made by kv_evict_plan(cache, t, M, ..., ws_evict) with no cache write
 * in between.  Attention reads every K/V row once; each kept row is written to its
 * compacted slot from the data the attention already loaded, so the separate
 * re-read of kept rows disappears.  All destinations lie below M rounded up to 32
 * slots; those tiles are attended first (phase 1), the rest afterwards (phase 2,
 * which first copies the kept rows below that boundary that move to the plan's
 * scratch, then moves rows, merges the split states and sets len).
 *   phase 0  both phases on `stream` (the plan must be complete before the call)
 *   phase 1  attention over the first tiles only; needs no plan, so it may run
 *            concurrently with kv_evict_plan (which only reads the cache)
 *   phase 2  the rest; the plan must be complete; ws must hold phase 1's states
 * Other arguments as kv_attn_decode (num_splits >= 2 for the fused kernels; the
 * same num_splits and ws in both phases); ws_evict is the plan's workspace.
 * Falls back to kv_attn_decode + kv_evict_apply (phase 1 then does nothing) for
 * dtype/D/group combinations without the fused kernel, caches whose plan does not
 * fit the single-workgroup planner, and caches with a start array.
 */
int32_t kv_attn_decode_compact(const kvb_cache* cache, const void* q, int32_t Hq, const int32_t* t,
                               float scale, int32_t M, int32_t num_splits, int32_t phase,
                               float* out, float* lse, void* ws, size_t ws_bytes, void* ws_evict,
                               size_t ws_evict_bytes, void* stream);

/*
 * kv_attn_decode over a paged cache (see kvb_pages; bf16, D = 128, Hq / Hkv in
 * {1, 2, 4, 8}): the same attention over each head's live tokens, taken page by
 * page.  A decode token (k_new != NULL) is written into the last page when it has
 * room, otherwise into the caller's free physical page spare[b][g] (appended to
 * the table; spare NULL or < 0, or a full table: the token is neither stored nor
 * attended and the status word becomes KVB_ECAPACITY), with pos = t[b]; len and
 * the page arrays are updated.
 *   spare      [B][Hkv] int32 or NULL: a physical page the head does not use (not
 *              checked; kv_check_pages reports a page listed twice)
 *   ws         kv_attn_decode_workspace(cache, Hq, num_splits) bytes
 * Other arguments as kv_attn_decode; num_splits 0 takes about 2048 / (B * Hkv)
 * splits, at most one per 8 pages of max_pages.  Like kv_attn_decode it allocates
 * nothing and issues no memset, so it can be captured in a graph.
 */
int32_t kv_attn_decode_paged(const kvb_cache* cache, const kvb_pages* pages, const void* q,
                             int32_t Hq, const int32_t* t, float scale, const void* k_new,
                             const void* v_new, const float* log_beta_new,
                             const int32_t* spare, int32_t num_splits, float* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * kv_erase_ranges over a paged cache, block-granular ([MEM] blocks and compression;
 * system engineering): a page whose live positions all lie in the sequence's
 * ranges leaves the table (its rows are not touched; the page is free for the
 * caller), a page none of whose positions does stays as it is, and a page with
 * both keeps its surviving rows, in order, in its first slots (the only rows that
 * move).  The table keeps the remaining pages in order; n_pages, fill and len are
 * updated.  A cache whose erased blocks start and end on page boundaries moves no
 * row at all.
 *   ranges, n_ranges, R, n_erased  as kv_erase_ranges (at most 4096 ranges per
 *              sequence)
 *   ws         kv_erase_paged_workspace(cache, pages) bytes
 */
size_t kv_erase_paged_workspace(const kvb_cache* cache, const kvb_pages* pages);
int32_t kv_erase_ranges_paged(const kvb_cache* cache, const kvb_pages* pages,
                              const int32_t* ranges, const int32_t* n_ranges, int32_t R,
                              int32_t* n_erased, void* ws, size_t ws_bytes, void* stream);

/*
 * Erase position ranges from every KV head of a sequence and compact in place
 * ([MEM] blocks and compression; system engineering).
 *
 *   ranges     [B][R][2] int32 half-open position ranges [s, e) per sequence,
 *              sorted by s, pairwise disjoint, s < e.
 *   n_ranges   [B] int32 ranges used per sequence (0..R).
 *   R          row stride of `ranges` (>= 0).
 *   n_erased   [B][Hkv] int32 or NULL: slots removed per head.
 * A slot is kept iff its position lies in none of its sequence's ranges; kept
 * rows keep their slot order and fill slots [0, kept); len becomes kept.
 *   ws         workspace of kv_erase_workspace(cache) bytes.
 */
int32_t kv_erase_ranges(const kvb_cache* cache, const int32_t* ranges, const int32_t* n_ranges,
                        int32_t R, int32_t* n_erased, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * Attention-state memory lookup and merge ([ASM] method steps 3 and 4; GQA
 * extension).  For every query head h of sequence b (KV head g = h / (Hq/Hkv)):
 *   idx = argmax_k cos(q[b][h], centroids[g][k])   (ties: lowest k; the stored
 *         centroid values are used as they are; a zero query gives idx 0)
 *   (out, out_lse) = merge((self_out, self_lse), (abar[g][idx], log_zbar[g][idx]))
 * where merge weights each output by its normaliser: with Z = e^self_lse and
 * Zbar = e^log_zbar, out = (Z self_out + Zbar abar) / (Z + Zbar),
 * out_lse = log(Z + Zbar).  self_lse = -inf means no own tokens.
 *
 *   q          [B][Hq][D] bf16;  centroids, abar [Hkv][K][D] bf16;  log_zbar [Hkv][K] f32
 *   self_out   [B][Hq][D] f32;   self_lse [B][Hq] f32 (e.g. kv_attn_decode's out, lse)
 *   out        [B][Hq][D] f32;   out_lse [B][Hq] f32 (may alias self_out / self_lse)
 *   idx        [B][Hq] int32 or NULL
 *   D == 128 or 64; 1 <= K < 2^24; (Hq / Hkv) * B <= 65536.
 *   ws         workspace of asm_lookup_merge_workspace(B, Hq, Hkv, D, K) bytes.
 */
int32_t asm_lookup_merge(const void* q, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                         const void* centroids, const void* abar, const float* log_zbar,
                         int32_t K, const float* self_out, const float* self_lse, float* out,
                         float* out_lse, int32_t* idx, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * kv_attn_decode followed by asm_lookup_merge on its output, in three launches
 * instead of four ([ASM] method steps 1-4): the lookup's candidate scan (it needs
 * only q and the codebook) runs first, and the attention's split merge also picks
 * each query head's entry and merges it.  Results equal the two calls' (same
 * arithmetic); out and lse hold the merged state, idx the chosen entries.
 *   Arguments as kv_attn_decode (bf16 cache, D 128 or 64) and asm_lookup_merge
 *   (centroids, abar [Hkv][K][D] bf16; log_zbar [Hkv][K] f32; 1 <= K < 2^24).
 *   num_splits 0: kv_attn_decode_asm_splits(): for D = 128 at most what one round
 *              of resident waves (2048) leaves beside the scan's tasks, per head,
 *              rounded down to a power of two; otherwise as kv_attn_decode.
 *   ws         workspace of kv_attn_decode_asm_workspace(cache, Hq, num_splits, K)
 *              bytes; the attention's part (and status word) comes first.
 */
size_t kv_attn_decode_asm_workspace(const kvb_cache* cache, int32_t Hq, int32_t num_splits,
                                    int32_t K);
/* Number of KV splits kv_attn_decode_asm uses for num_splits == 0 (host only; 0 for
 * invalid arguments). */
int32_t kv_attn_decode_asm_splits(const kvb_cache* cache, int32_t Hq, int32_t K);
int32_t kv_attn_decode_asm(const kvb_cache* cache, const void* q, int32_t Hq, const int32_t* t,
                           float scale, const void* k_new, const void* v_new,
                           const float* log_beta_new, int32_t num_splits,
                           const void* centroids, const void* abar, const float* log_zbar,
                           int32_t K, float* out, float* lse, int32_t* idx, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * The same lookup and merge through a two-level index ([ASM] technical novelty:
 * hierarchical lookup; experiments: expanding the top 16 first-level centroids
 * matches the linear lookup's top-1).  Per query head h of sequence b (KV head g):
 *   1. cos(q, c1[g][j]) for the K1 first-level centroids; keep the m largest
 *      (equal similarities: the lower j first);
 *   2. idx = the original index of the entry with the largest cos(q, c) among the
 *      entries of the kept clusters (equal similarities: the lowest original
 *      index); a zero query, or kept clusters without entries, give idx 0;
 *   3. merge with (abar[g][idx], log_zbar[g][idx]) as asm_lookup_merge does.
 *
 *   c1         [Hkv][K1][D] bf16 first-level centroids, 1 <= K1 <= 512, 1 <= m <= K1
 *   offs       [Hkv][K1 + 1] int32: the entries of cluster j are stored at positions
 *              offs[j] .. offs[j+1]-1 (non-decreasing, offs[0] = 0, offs[K1] = K;
 *              values outside [0, K] are clamped)
 *   centroids  [Hkv][K][D] bf16, stored cluster by cluster
 *   kid        [Hkv][K] int32: original index (0 .. K-1) of each stored entry
 *   abar, log_zbar  by original index, as for asm_lookup_merge
 *   other arguments as asm_lookup_merge.
 *   ws         workspace of asm_lookup_merge_hier_workspace(B, Hq, Hkv, K1, m) bytes.
 */
int32_t asm_lookup_merge_hier(const void* q, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                              const void* c1, int32_t K1, const int32_t* offs,
                              const void* centroids, const int32_t* kid, int32_t K, int32_t m,
                              const void* abar, const float* log_zbar, const float* self_out,
                              const float* self_lse, float* out, float* out_lse, int32_t* idx,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * Attention states of calibration queries over a prefix ([ASM] method step 1, and
 * the chunked construction of the experiments: the prefix encoded in chunks whose
 * states are merged).  Per KV head h and query n:
 *   a[h][n]   = sum_i e^{s_i} v_i / sum_i e^{s_i},  s_i = scale * (q[h][n] . k[h][i]),
 *   lse[h][n] = log sum_i e^{s_i}  (the page's Z in log form).
 * The L prefix tokens are cut into ceil(L / csize) consecutive chunks of csize =
 * ceil(L / chunks) tokens (the last may be shorter); each chunk's state is
 * computed on its own and the states are merged in chunk order with the merge
 * operator.  L == 0 gives a = 0, lse = -inf.  Scores use bf16 MFMA products with
 * float32 accumulation; the value product runs in fp16 (float32 accumulation): the
 * softmax weights rounded to fp16, v converted to fp16 after scaling each chunk's
 * dimension d by the power of two that brings that dimension's max |v| into
 * [2^14, 2^15), which the output undoes: every finite bf16 v is carried exactly.  A non-finite v saturates and sets the workspace status word, the int32 at
 * byte offset 0, to KVB_ERANGE (the call never clears it).
 *   q        [H][N][D] bf16 (the KV head's calibration queries; for GQA the group's
 *            query heads stacked along N)
 *   k, v     [H][L][D] bf16 (may be NULL when L == 0)
 *   chunks   1..65535; scale: <= 0 selects 1/sqrt(D); D is 64 or 128; N < 2^24
 *   a        [H][N][D] float32;  lse [H][N] float32
 *   ws       asm_prefix_states_workspace(H, N, D, L, chunks) bytes (the chunk states
 *            when there is more than one chunk).
 */
int32_t asm_prefix_states(const void* q, int32_t H, int32_t N, int32_t D, const void* k,
                          const void* v, int32_t L, int32_t chunks, float scale, float* a,
                          float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * K-means over each KV head's calibration queries ([ASM] method step 2: the
 * collected queries are clustered and a cluster's query centroid is the mean of
 * its members).  Lloyd iterations from the caller's initial centroids: every
 * iteration assigns each point to the centroid at the smallest Euclidean
 * distance (equal distances to the lowest index), then moves every centroid to
 * the mean of its members; a centroid without members stays where it is.
 * Distances are ranked by |c|^2 - 2 x.c in float32, x.c formed from the bf16 point
 * and the centroid split into two bf16 parts (16 significant bits); member sums
 * are float32 in an order fixed by N and the assignment, so results repeat bit
 * for bit.
 *   x          [H][N][D] bf16 points
 *   centroids  [H][K][D] float32: initial centroids in, final centroids out
 *   iters      1..100000 iterations; K < 2^24
 *   assign     [H][N] int32 out: the last iteration's assignment
 *   counts     [H][K] int32 out (may be NULL): member counts of that assignment
 *   centroids_bf16 [H][K][D] bf16 out (may be NULL): final centroids rounded to
 *              nearest-even bf16 (the codebook format asm_lookup_merge reads)
 *   ws         asm_kmeans_workspace(H, K, D) bytes
 */
int32_t asm_kmeans(const void* x, int32_t H, int32_t N, int32_t D, float* centroids, int32_t K,
                   int32_t iters, int32_t* assign, int32_t* counts, void* centroids_bf16,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * Attention-aware aggregation ([ASM] method step 2 and technical novelty: a
 * cluster's stored state is the merge of its members' states, not their average).
 * For cluster k of KV head h, over the points n with assign[h][n] == k:
 *   log_zbar[h][k] = log sum_n e^{lse[h][n]},
 *   abar[h][k]     = sum_n e^{lse[h][n]} a[h][n] / sum_n e^{lse[h][n]}  (bf16, RNE);
 * a cluster with no member (or only members with lse = -inf) gets abar = 0,
 * log_zbar = -inf.  Labels outside 0..K-1 belong to no cluster.  Members are
 * merged in an order fixed by N and the assignment (float32, bit-repeatable).
 *   assign [H][N] int32; a [H][N][D] float32; lse [H][N] float32
 *   abar   [H][K][D] bf16 out;  log_zbar [H][K] float32 out
 */
int32_t asm_aggregate_states(const int32_t* assign, const float* a, const float* lse, int32_t H,
                             int32_t N, int32_t D, int32_t K, void* abar, float* log_zbar,
                             void* stream);

/*
 * The whole offline build of an attention-state memory for one layer ([ASM]
 * method steps 1-2): asm_prefix_states of the calibration queries q over the
 * prefix (k, v) in `chunks` chunks, asm_kmeans of the same queries for `iters`
 * iterations from the initial `centroids`, then asm_aggregate_states of the
 * states by the final assignment.  The outputs are the codebook the lookup reads:
 * centroids_bf16 [H][K][D] bf16, abar [H][K][D] bf16, log_zbar [H][K] float32,
 * plus the float32 centroids (in place) and the assignment [H][N] int32.
 *   ws  asm_build_memory_workspace(H, N, D, L, chunks, K) bytes (its status word as
 *       for asm_prefix_states); after the call it holds the per-query states: a [H][N][D] float32 at byte offset 256,
 *       lse [H][N] float32 at the next 256-byte boundary.
 * Other arguments as for the three calls above.
 */
int32_t asm_build_memory(const void* q, int32_t H, int32_t N, int32_t D, const void* k,
                         const void* v, int32_t L, int32_t chunks, float scale, float* centroids,
                         int32_t K, int32_t iters, void* centroids_bf16, void* abar,
                         float* log_zbar, int32_t* assign, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * Latent memory of evicted tokens, update ([IDX] section 2, part B: evicted tokens
 * update a fixed-size state matrix M and a stabiliser vector b online, by an
 * outer-product accumulation with decay).  Per KV head u, for the slots the plan
 * in ws_evict evicts (kv_evict_plan with the same cache and M), in slot order,
 * j = 0..n-1, with phi(x) = elu(x) + 1:
 *   M[u] <- lam^n M[u] + sum_j lam^(n-1-j) phi(k_j) v_j^T
 *   b[u] <- lam^n b[u] + sum_j lam^(n-1-j) phi(k_j)
 * A head the plan leaves alone is not touched.  Call after kv_evict_plan and before
 * kv_evict_apply (it reads the evicted rows in place).  phi(k) enters the matrix
 * product as two bf16 parts (float32 accumulation); b is accumulated in float32.
 *   cache      bf16, D = 64 or 128
 *   ws_evict   the plan's workspace (ws_evict_bytes >= kv_evict_workspace(cache, M))
 *   lam        decay per absorbed token, 0 < lam <= 1
 *   mem_M      [B][Hkv][D][D] float32, in/out;  mem_b [B][Hkv][D] float32, in/out
 *   ws         kv_latent_absorb_workspace(cache) bytes
 */
int32_t kv_latent_absorb(const kvb_cache* cache, int32_t M, const void* ws_evict,
                         size_t ws_evict_bytes, float lam, float* mem_M, float* mem_b, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * Latent memory read-out added to the attention output ([IDX] section 2, part B:
 * o = o_attn + g(q) m(q), a projection and a gate reading the memory).  For query
 * head h of sequence b (KV head u = b * Hkv + h / (Hq / Hkv)), f = phi(q[b][h]):
 *   r = M[u]^T f / (b[u] . f + eps),  m = W_o r,  g = 1 / (1 + e^-(w_g[h] . q + c_g[h])),
 *   out[b][h] += g * m   (out holds o_attn on entry).
 *   q      [B][Hq][D] bf16;  D = 64 or 128
 *   W_o    [D][D] float32 (row-major, m = W_o r);  w_g [Hq][D], c_g [Hq] float32
 *   eps    >= 0 (the caller keeps b . f + eps > 0; with an empty memory and eps = 0
 *          the read is 0/0)
 *   out    [B][Hq][D] float32, in/out
 */
int32_t kv_latent_read(const void* q, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                       const float* mem_M, const float* mem_b, const float* W_o, const float* w_g,
                       const float* c_g, float eps, float* out, void* stream);

/*
 * Kernel timing (a measurement aid; off by default; not thread-safe).
 * kvb_trace_enable(capacity, mask) creates `capacity` HIP event pairs; from then
 * on every launch of a kernel selected by `mask` records one pair on the launch
 * stream around that launch, until the pairs run out.  mask bits: 1 attention
 * split kernel, 2 split merge, 4 append, 8 eviction select, 16 keep count,
 * 32 keep emit, 64 compaction move, 128 ASM lookup, 256 ASM finalize, 512 the
 * attention split kernel that also moves kept rows (kv_attn_decode_compact),
 * 1024 prefix-state chunk kernel, 2048 prefix chunk merge, 4096 K-means
 * assignment, 8192 K-means centroid update (and the initial centroid split),
 * 16384 state aggregation, 32768 the value transpose before the prefix-state
 * chunk kernel, 65536 latent-memory update (all its kernels), 131072 latent-memory
 * read.
 * kvb_trace_read waits for the recorded pairs and writes, for the first `max`,
 * the kernel bit and the elapsed milliseconds (-1 if unavailable); it returns
 * how many it wrote (host arrays).  kvb_trace_reset reuses the pairs from the
 * start; kvb_trace_disable destroys them.  Returns KVB_OK, KVB_EINVAL
 * (capacity outside 0..2^20) or KVB_EDEVICE.
 */
int32_t kvb_trace_enable(int32_t capacity, int32_t kernel_mask);
int32_t kvb_trace_read(int32_t* kernel_ids, float* ms, int32_t max);
void kvb_trace_reset(void);
void kvb_trace_disable(void);

#ifdef __cplusplus
}
#endif

#endif /* KVBOUND_H */
