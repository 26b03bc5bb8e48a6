/*
 * kvq.h — decode attention over a mixed-precision, group-quantized KV cache (AMD CDNA4).
 *
 * Plain C ABI. No exception crosses it; every call that can fail returns a kvq_status and
 * leaves a thread-local message for kvq_last_error(). Pointers are plain addresses: those
 * named *_dev are device (HBM) addresses, everything else is host memory. Streams are
 * hipStream_t handles passed as void* (NULL = the default stream).
 *
 * The method (sources: the RateQuant and InnerQ pages):
 *   - keys are quantized in groups of 32 consecutive head_dim channels of one token, values
 *     in groups of 32 consecutive tokens of one channel: grouping along the inner dimension
 *     of q.K^T and P.V (InnerQ, abstract and "Core claim");
 *   - each group is asymmetric min/max, or in hybrid mode the lower-error of symmetric and
 *     asymmetric (InnerQ, technique (i)), with float16 scale s and zero z;
 *   - the first n_sink tokens and the most recent n_recent..n_recent+31 tokens stay in 16
 *     bits (InnerQ, technique (ii));
 *   - bits per KV head come from the distortion model D(b) = alpha * beta^-b fitted on a
 *     calibration slice and allocated by reverse waterfilling / greedy integer allocation
 *     (RateQuant, sections 3.1, 3.3, 3.4);
 *   - decode reads the packed codes with dequantization fused into q.K^T and P.V, split-K
 *     over tokens, merged by log-sum-exp (InnerQ, "Algorithm 1 ... decode phase");
 *   - optionally, per-channel key normalization folded into the query (InnerQ, technique
 *     (iii)); several query tokens per row decoded causally at once; rows of different
 *     lengths in one cache (ragged batches); a paged body (pages of 64 tokens placed by a
 *     per-row page table) for serving engines that hand out cache memory page by page.
 *
 * Ownership: the caller allocates and frees every device buffer (cache blob, inputs,
 * outputs, workspace). The library never allocates or frees device memory and keeps no
 * global state besides the thread-local error string.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_MAX_KV_HEADS 128
#define KVQ_GROUP 32

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_ARG = -1,         /* bad argument or shape; nothing was enqueued */
  KVQ_ERR_BUDGET = -2,      /* n*b_lo > total or total > n*b_hi */
  KVQ_ERR_CAPACITY = -3,    /* append would exceed the cache capacity */
  KVQ_ERR_RANGE = -4,       /* a quantized input was non-finite or |x| > 2^14 */
  KVQ_ERR_UNSUPPORTED = -5, /* a configuration this build does not implement */
  KVQ_ERR_DEVICE = -6,      /* a HIP call failed; kvq_last_error() has HIP's message */
  KVQ_ERR_PAGE = -7         /* paged cache: an append or decode reached a tile with no page mapped */
} kvq_status;

typedef enum { KVQ_F16 = 0, KVQ_BF16 = 1 } kvq_dtype;
enum { KVQ_QUANT_ASYM = 0, KVQ_QUANT_HYBRID = 1 };
/* Flag OR'ed into kvq_config.quant: per-channel key normalization (InnerQ technique (iii), its
 * "Core claim" and abstract). The first kvq_append on an empty cache stores, per row, KV head
 * and channel c, n_c = the smallest power of two >= max |k_c| over the tokens of that call
 * (1 if that max is 0; fp32, region KN). From then on every quantized key group holds
 * k_c / n_c instead of k_c, and decode scores the packed keys with q_c * n_c: the
 * normalization is folded into the query. Both steps are exact because n_c is a power of two.
 * 16-bit sink, window and unquantized-head keys are stored and used as they are. */
enum { KVQ_KEY_NORM = 0x100 };
enum { KVQ_AXIS_KEY = 0, KVQ_AXIS_VALUE = 1 };
enum { KVQ_ALLOC_CAP_W = 1u }; /* w_i <- min(w_i, 5 * mean(w)) before allocating (RateQuant W.14) */

/* Cache geometry. Host memory, owned by the caller. */
typedef struct {
  int32_t batch;        /* rows B >= 1 */
  int32_t n_kv_heads;   /* Hkv, 1..KVQ_MAX_KV_HEADS */
  int32_t n_q_heads;    /* Hq, a multiple of Hkv; query head i reads KV head i / (Hq/Hkv) */
  int32_t head_dim;     /* D: 64 or 128 */
  int32_t capacity;     /* maximum tokens per row */
  int32_t group;        /* must be KVQ_GROUP (32) */
  int32_t n_sink;       /* first tokens kept in 16 bits, >= 0 */
  int32_t n_recent;     /* recent tokens kept in 16 bits, >= 0 (the window holds
                           n_recent..n_recent+31 once the body has started) */
  int32_t dtype;        /* kvq_dtype of keys, values and queries */
  int32_t quant;        /* KVQ_QUANT_ASYM or KVQ_QUANT_HYBRID, optionally | KVQ_KEY_NORM */
  uint8_t k_bits[KVQ_MAX_KV_HEADS]; /* per KV head: 2..8, or 16 = unquantized */
  uint8_t v_bits[KVQ_MAX_KV_HEADS];
} kvq_config;

/* A cache handle: the caller's POD. `dev` is a device blob of `bytes` bytes laid out by
 * kvq_cache_init (n_pages = 0) or kvq_cache_init_paged (n_pages > 0); `len` is the token
 * count of every row. kvq_append changes `len`, so calls on one cache must be serialized by
 * the caller (same stream, or host order). */
typedef struct {
  kvq_config cfg;
  void* dev;
  uint64_t bytes;
  int32_t len;
  int32_t n_pages;
} kvq_cache;

/* Blob bytes needed for `cfg` (0 if cfg is invalid; kvq_last_error() says why). */
size_t kvq_cache_bytes(const kvq_config* cfg);

/* Validate cfg, write the blob header and region table into dev_mem (synchronously on
 * `stream`), clear the sticky range flag, and set cache->len = 0. dev_mem must be at least
 * kvq_cache_bytes(cfg) bytes and 256-byte aligned. */
kvq_status kvq_cache_init(kvq_cache* cache, const kvq_config* cfg, void* dev_mem, size_t bytes,
                          void* stream);

/* Paged caches. The quantized body (regions 0..4) of every row is cut into tiles of 64
 * tokens (two 32-token groups of values); tile t of row b lives in page page[b][t] of a pool
 * of n_pages pages that every row shares. Each KV head has its own pools (its pages differ in
 * size with its bit widths) and one page index serves all heads of a row. Sink, ring and norm
 * regions stay per (row, head). Bytes inside a page are laid out as in a contiguous cache's
 * tile, so paged and contiguous caches hold the same codes and decode to the same outputs.
 * The page table (int32 [batch][page_stride], page_stride = the tiles of a row holding
 * `capacity` tokens) lives in the blob; kvq_cache_init_paged sets every entry to -1
 * (unmapped). kvq_cache_map_pages rejects one page given to two tiles of the same call;
 * a page shared with a (row, tile) mapped by another call is the caller's error (the library
 * keeps no host copy of the table). A flush into an unmapped tile writes nothing, and a decode
 * that reads one gets meaningless values for it (the read stays inside the pools); both set a
 * sticky flag that kvq_cache_check reports as KVQ_ERR_PAGE. All other calls (append, ragged,
 * multi-token, decode, step) take paged caches as they are.
 * Motivation: a fixed bit budget per token and head is what lets serving engines hand out
 * cache memory in fixed-size blocks (NOVA-KV page, "If this is right"); the page mechanics
 * are this library's. */

/* Blob bytes for a paged cache of n_pages pages (1 <= n_pages; every pool under 2 GiB);
 * 0 on bad arguments. */
size_t kvq_cache_bytes_paged(const kvq_config* cfg, int32_t n_pages);

/* As kvq_cache_init, for a paged cache of n_pages pages; also writes the page table with
 * every entry -1. Synchronous on `stream`. */
kvq_status kvq_cache_init_paged(kvq_cache* cache, const kvq_config* cfg, int32_t n_pages, void* dev_mem,
                                size_t bytes, void* stream);

/* Map tiles first_tile .. first_tile + n_tiles - 1 of `row` to pages[0 .. n_tiles - 1]
 * (host array; each entry in [0, n_pages), or -1 to unmap; no page twice). Tile t holds body tokens
 * 64t .. 64t + 63 of the row, i.e. tokens n_sink + 64t .. of the sequence; a row holding T
 * tokens needs its first ceil(body(T) / 64) tiles mapped, body(T) as in the decode
 * description. KVQ_ERR_ARG, with nothing written, if after the call one page would hold two
 * tiles (of this or any other row): the call reads the table back to check. Copies
 * synchronously on `stream` (host order with earlier work on it). */
kvq_status kvq_cache_map_pages(const kvq_cache* cache, int32_t row, int32_t first_tile, int32_t n_tiles,
                               const int32_t* pages, void* stream);

/* Calibration + distortion fit (RateQuant sections 3.1, 3.4, 4.1, W.10).
 * x_dev: [n_heads][n_tokens][head_dim] 16-bit (dtype), one calibration slice per head.
 * axis KVQ_AXIS_KEY groups 32 channels of a token; KVQ_AXIS_VALUE groups 32 tokens of a
 * channel (n_tokens must then be a multiple of 32). For every head and b = b_lo..b_hi the
 * device computes each group's squared quantization error in float64 (quant = asym or
 * hybrid) and adds them per 256 groups in a fixed order; the host adds those sums in
 * order, divides by n_tokens*head_dim to get D(b),
 * fits ln D(b) = ln alpha - b ln beta by least squares and applies the beta fallback
 * (R^2 < 0.96: beta = min(beta, mean beta of the well-fitted heads)).
 * Outputs alpha, beta, r2: host arrays [n_heads]. Needs 2 <= b_lo, b_lo + 2 <= b_hi <= 8 and
 * 1 <= n_heads <= 65535 (a whole model's (layer, KV head) pairs fit in one call).
 * ws_dev: device scratch of at least kvq_calibrate_workspace_bytes(...) bytes.
 * BLOCKS until the result is on the host. A head whose inputs are out of range makes the
 * call return KVQ_ERR_RANGE. */
size_t kvq_calibrate_workspace_bytes(int32_t n_heads, int32_t n_tokens, int32_t head_dim,
                                     int32_t b_lo, int32_t b_hi);
kvq_status kvq_calibrate_fit(const void* x_dev, int32_t dtype, int32_t n_heads,
                             int32_t n_tokens, int32_t head_dim, int32_t axis, int32_t quant,
                             int32_t b_lo, int32_t b_hi, void* ws_dev, size_t ws_bytes,
                             double* alpha, double* beta, double* r2, void* stream);

/* Bit allocation (RateQuant sections 3.1, 3.3, B.1, B.3, U): host only, pure.
 * Minimizes sum_i w_i alpha_i beta_i^-b_i over integers b_lo <= b_i <= b_hi with
 * sum b_i = total_bits: every head starts at b_lo and a max-heap hands out the remaining
 * bits one at a time to the largest marginal gain w a beta^-b (1 - 1/beta) (ties: lowest
 * index). bits_cont_out (nullable) receives the continuous reverse-waterfilling solution.
 * alpha >= 0, beta > 1, w > 0, 2 <= b_lo <= b_hi <= 8; flags: KVQ_ALLOC_CAP_W. */
kvq_status kvq_allocate_bits(int32_t n, const double* alpha, const double* beta,
                             const double* w, int32_t total_bits, int32_t b_lo, int32_t b_hi,
                             uint32_t flags, uint8_t* bits_out, double* bits_cont_out);

/* Decision margin of an integer allocation (RateQuant section 3.3): host only, pure.
 * bits: an allocation of the same inputs (for instance from kvq_allocate_bits). With
 * key_i(b) = ln(w_i alpha_i beta_i^-b (1 - 1/beta_i)), the marginal key of head i's (b+1)-th
 * bit evaluated as kvq_allocate_bits does, *margin_out = min over heads with bits_i > b_lo of
 * key_i(bits_i - 1) minus max over heads with bits_i < b_hi of key_i(bits_i): how far, in log
 * units, the last bit handed out beat the best bit left. It is >= 0 for a greedy allocation,
 * 0 exactly at a tie, +inf when no bit was handed out or every head is at b_hi. Model
 * parameters known only to a relative error e move each key by about (1 + b_hi) e, so two
 * such inputs can allocate differently only when the margin is below a few times that (fits
 * computed with differently ordered sums agree to ~1e-13). Same argument rules as
 * kvq_allocate_bits, plus b_lo <= bits_i <= b_hi. */
kvq_status kvq_allocation_margin(int32_t n, const double* alpha, const double* beta, const double* w,
                                 const uint8_t* bits, int32_t b_lo, int32_t b_hi, uint32_t flags,
                                 double* margin_out);

/* Append n_new tokens to every row (InnerQ techniques (i)-(ii); asynchronous on stream).
 * k_dev, v_dev: [batch][n_kv_heads][n_new][head_dim] 16-bit. Tokens 0..n_sink-1 of a row
 * go to the sink; later tokens enter the recent ring; whenever the ring holds
 * n_recent + 32 tokens its oldest 32 are quantized and packed as one body block.
 * len + n_new must not exceed capacity (else KVQ_ERR_CAPACITY, nothing enqueued).
 * Out-of-range quantized inputs set the cache's sticky flag (see kvq_cache_check). */
kvq_status kvq_append(kvq_cache* cache, const void* k_dev, const void* v_dev, int32_t n_new,
                      void* stream);

/* Split-K decode attention for one query token per row (InnerQ Algorithm 1 structure).
 * q_dev: [batch][n_q_heads][head_dim] 16-bit; out_dev: [batch][n_q_heads][head_dim] fp32.
 * The packed body tiles of each (row, KV head) are cut into n_splits (1..256) contiguous
 * ranges, and the 16-bit sink + recent window is dealt out over the same workgroups in
 * 16-token units; each workgroup yields one partial (m, l, o), and a second launch merges
 * the partials by log-sum-exp. scale <= 0 means 1/sqrt(D).
 * workspace_dev: at least kvq_decode_workspace_bytes(cache, n_splits) bytes, 256-byte
 * aligned, holding the split partials between the decode and merge launches (no
 * initialization needed). Calls that share a workspace must not run concurrently.
 * Asynchronous on stream. len must be >= 1. */
size_t kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t n_splits);
kvq_status kvq_decode_attention(const kvq_cache* cache, const void* q_dev, float* out_dev,
                                int32_t n_splits, float scale, void* workspace_dev,
                                size_t ws_bytes, void* stream);

/* kvq_decode_attention without a workspace, for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid hipMalloc): the split
 * partials go to a static device array of 4 MiB that the library holds on every GPU it runs
 * on until the process ends (looked up once per device, on the first call there). Nothing is
 * allocated or freed. A call whose partials, kvq_decode_workspace_bytes(cache, n_splits),
 * exceed 4 MiB returns KVQ_ERR_ARG and enqueues nothing. Every call on one GPU uses that
 * GPU's array: calls that overlap on one GPU (other streams, other threads) race and must be
 * serialized by the caller. The array needs no initialization. Otherwise the same arguments,
 * rules, kernels and results as kvq_decode_attention. */
kvq_status kvq_decode_attention_noalloc(const kvq_cache* cache, const void* q_dev, float* out_dev,
                                        int32_t n_splits, float scale, void* stream);

/* The two launches of kvq_decode_attention, for callers that schedule or time them apart:
 * kvq_decode_splitk writes the n_splits partials (m, l, o) of every query head into the
 * workspace; kvq_decode_merge combines them into out_dev. Same arguments and rules as
 * kvq_decode_attention; the merge must see the same cache, n_splits and workspace as the
 * split-K call before it on the stream. */
kvq_status kvq_decode_splitk(const kvq_cache* cache, const void* q_dev, int32_t n_splits,
                             float scale, void* workspace_dev, size_t ws_bytes, void* stream);
kvq_status kvq_decode_merge(const kvq_cache* cache, float* out_dev, int32_t n_splits,
                            void* workspace_dev, size_t ws_bytes, void* stream);

/* Ragged batches: rows of different lengths in one cache (serving several sequences that
 * started at different times). The caller keeps each row's length in a host array
 * row_len[batch] (all 0 after kvq_cache_init) and passes it to these calls, which do not use
 * or change cache->len; a cache is used either through these calls or through the uniform
 * ones. Any number of rows: the library launches them in groups of 64 on the stream.
 * kvq_append_ragged: row b appends n_new[b] >= 0 tokens, the first n_new[b] of its n_max input
 * slots: k_dev, v_dev [batch][n_kv_heads][n_max][head_dim] 16-bit. Each row follows the rules
 * of kvq_append on its own (sink, ring, 32-token flushes; with KVQ_KEY_NORM the norms come
 * from the row's first non-empty append). The caller then adds n_new[b] to row_len[b].
 * Host arrays are read before the call returns; KVQ_ERR_CAPACITY if a row would exceed it.
 * kvq_decode_ragged: one query token per row, row b attending to its row_len[b] >= 1 tokens;
 * q, out, workspace and rules as for kvq_decode_attention. */
kvq_status kvq_append_ragged(const kvq_cache* cache, const int32_t* row_len, const int32_t* n_new,
                             const void* k_dev, const void* v_dev, int32_t n_max, void* stream);
kvq_status kvq_decode_ragged(const kvq_cache* cache, const int32_t* row_len, const void* q_dev, float* out_dev,
                             int32_t n_splits, float scale, void* workspace_dev, size_t ws_bytes, void* stream);

/* Decode attention for the last n_qtok cached tokens of every row at once (multi-token or
 * speculative decode; the InnerQ Algorithm 1 structure per query token). q_dev:
 * [batch][n_qtok][n_q_heads][head_dim] 16-bit, out_dev: same shape fp32. Query token i of a
 * row is the (len - n_qtok + i)-th token and attends causally: to tokens 0 .. len - n_qtok + i.
 * The n_qtok x G query rows of a KV head share one pass over its cache: up to 4 rows run on the
 * single-query kernel's 4-row MFMA tile, 5 to 16 rows (for instance 4 GQA heads x 4 tokens) on
 * a 16-row tile; n_qtok * (n_q_heads / n_kv_heads) > 16 returns KVQ_ERR_UNSUPPORTED. The newest n_qtok - 1 tokens must still be in the 16-bit window
 * (true when n_recent >= n_qtok - 1), else KVQ_ERR_UNSUPPORTED. n_qtok == 1 is exactly
 * kvq_decode_attention. Workspace: kvq_decode_multi_workspace_bytes(cache, n_splits, n_qtok)
 * bytes; other arguments and rules as for kvq_decode_attention. */
size_t kvq_decode_multi_workspace_bytes(const kvq_cache* cache, int32_t n_splits, int32_t n_qtok);
kvq_status kvq_decode_multi(const kvq_cache* cache, const void* q_dev, int32_t n_qtok, float* out_dev,
                            int32_t n_splits, float scale, void* workspace_dev, size_t ws_bytes,
                            void* stream);

/* One decode step (InnerQ Algorithm 1 with techniques (i)-(ii)): append n_new tokens (exactly
 * as kvq_append) and run decode attention for the query over all len + n_new tokens (exactly
 * as kvq_decode_attention), in one call. With n_new == 1 and the token past the sink, the
 * split-K launch reads the window as it stands and takes the new token straight from
 * k_dev / v_dev as one more softmax term, and the merge launch copies it into its recent-ring
 * slot; the step is then those two launches, plus the quantize launch when a 32-token block
 * leaves the window. Same arguments, ownership and rules as the two calls; arguments are
 * checked before anything is enqueued. Asynchronous on stream; cache->len grows by n_new.
 * k_dev / v_dev must stay valid until the merge launch has run. */
kvq_status kvq_decode_step(kvq_cache* cache, const void* k_dev, const void* v_dev, int32_t n_new,
                           const void* q_dev, float* out_dev, int32_t n_splits, float scale,
                           void* workspace_dev, size_t ws_bytes, void* stream);

/* Synchronize `stream`, read the sticky flags; KVQ_ERR_RANGE if an input was out of range,
 * else KVQ_ERR_PAGE if a paged cache's append or decode reached an unmapped tile. */
kvq_status kvq_cache_check(const kvq_cache* cache, void* stream);

/* Byte offset, from the blob start, of region `region` (0..9: key codes, key meta, value
 * codes, value meta, hybrid flags, sink keys, sink values, ring keys, ring values, key
 * norms) of (row, kv_head), and its size; returns 0 and sets *size = 0 on bad arguments.
 * Contiguous caches only; a paged blob's region table (uint64 [batch][n_kv_heads][10] at
 * byte 256 of the blob) names the pools and regions of a paged cache. */
uint64_t kvq_region_offset(const kvq_config* cfg, int32_t row, int32_t kv_head, int32_t region,
                           uint64_t* size);

/* Message of the last non-OK status on this thread ("" if none). */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */
