// C ABI entry points of libkvq (declared in include/kvq.h): argument checks on the host,
// then kernel launches on the caller's stream. No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "kvq_internal.h"

using namespace kvq;

namespace {

kvq_status hip_fail(hipError_t e, const char* what) {
  return fail(KVQ_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

kvq_status check_launch(int e, const char* what) {
  if (e != (int)hipSuccess) return hip_fail((hipError_t)e, what);
  return KVQ_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

kvq_status check_cache(const kvq_cache* c) {
  if (!c) return fail(KVQ_ERR_ARG, "cache is NULL");
  kvq_status st = check_config(&c->cfg);
  if (st != KVQ_OK) return st;
  if (!c->dev) return fail(KVQ_ERR_ARG, "cache has no device memory");
  if (c->len < 0 || c->len > c->cfg.capacity) return fail(KVQ_ERR_ARG, "cache len out of range");
  if (c->n_pages < 0) return fail(KVQ_ERR_ARG, "negative n_pages");
  if (c->bytes < plan_layout(c->cfg, nullptr, c->n_pages)) return fail(KVQ_ERR_ARG, "cache blob too small");
  return KVQ_OK;
}

const uint64_t* table_ptr(const kvq_cache* c) {
  return reinterpret_cast<const uint64_t*>(static_cast<const char*>(c->dev) + kHeaderBytes);
}
// The page table of a paged cache into a launch plan (null for contiguous caches).
template <class Plan>
void set_pages(const kvq_cache* c, Plan& p) {
  if (c->n_pages <= 0) return;
  uint64_t pt_off = 0;
  plan_layout(c->cfg, nullptr, c->n_pages, &pt_off);
  p.pages = reinterpret_cast<const int32_t*>(static_cast<const char*>(c->dev) + pt_off);
  p.page_stride = page_stride(c->cfg);
  p.n_pages = c->n_pages;
}

uint32_t* flag_ptr(const kvq_cache* c) {
  return reinterpret_cast<uint32_t*>(static_cast<char*>(c->dev) + offsetof(BlobHeader, range_flag));
}

}  // namespace

extern "C" {

const char* kvq_last_error(void) { return last_error(); }

size_t kvq_cache_bytes(const kvq_config* cfg) {
  if (check_config(cfg) != KVQ_OK) return 0;
  return (size_t)plan_layout(*cfg, nullptr);
}

uint64_t kvq_region_offset(const kvq_config* cfg, int32_t row, int32_t kv_head, int32_t region,
                           uint64_t* size) {
  if (size) *size = 0;
  if (check_config(cfg) != KVQ_OK) return 0;
  if (row < 0 || row >= cfg->batch || kv_head < 0 || kv_head >= cfg->n_kv_heads || region < 0 ||
      region >= kRegions) {
    set_error("region index out of range");
    return 0;
  }
  std::vector<uint64_t> off((size_t)cfg->batch * cfg->n_kv_heads * kRegions);
  plan_layout(*cfg, off.data());
  uint64_t sz[kRegions];
  region_sizes(*cfg, kv_head, sz);
  if (size) *size = sz[region];
  return off[((size_t)row * cfg->n_kv_heads + kv_head) * kRegions + region];
}

}  // extern "C"

namespace {

kvq_status check_pages(const kvq_config* cfg, int32_t n_pages) {
  if (n_pages < 1) return fail(KVQ_ERR_ARG, "n_pages must be >= 1");
  for (int h = 0; h < cfg->n_kv_heads; ++h) {
    uint64_t sz[kRegions];
    region_sizes(*cfg, h, sz, n_pages);
    for (int r = KC; r <= FL; ++r)
      if (sz[r] > 0x7FFFFFFFull) return fail(KVQ_ERR_ARG, "a page pool would exceed 2 GiB");
  }
  return KVQ_OK;
}

// Header, region table and (paged caches) a page table of -1 entries, copied synchronously.
kvq_status init_blob(kvq_cache* cache, const kvq_config* cfg, int32_t n_pages, void* dev_mem, size_t bytes,
                     void* stream) {
  if (!cache) return fail(KVQ_ERR_ARG, "cache is NULL");
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (n_pages > 0 && (st = check_pages(cfg, n_pages)) != KVQ_OK) return st;
  if (!dev_mem || !aligned(dev_mem, 256)) return fail(KVQ_ERR_ARG, "dev_mem must be 256-byte aligned");
  const size_t n_off = (size_t)cfg->batch * cfg->n_kv_heads * kRegions;
  std::vector<uint64_t> host(kHeaderBytes / 8 + n_off, 0);
  uint64_t pt_off = 0;
  const uint64_t total = plan_layout(*cfg, host.data() + kHeaderBytes / 8, n_pages, &pt_off);
  if (bytes < total) return fail(KVQ_ERR_ARG, "dev_mem smaller than the cache's size");
  BlobHeader hdr{};
  hdr.magic = kMagic;
  hdr.version = kVersion;
  hdr.range_flag = 0;
  hdr.n_regions = kRegions;
  hdr.batch = cfg->batch;
  hdr.n_kv_heads = cfg->n_kv_heads;
  hdr.head_dim = cfg->head_dim;
  hdr.capacity = cfg->capacity;
  hdr.table_offset = kHeaderBytes;
  hdr.total_bytes = total;
  hdr.page_table_offset = pt_off;
  hdr.n_pages = n_pages;
  hdr.page_stride = n_pages > 0 ? page_stride(*cfg) : 0;
  std::memcpy(host.data(), &hdr, sizeof(hdr));
  hipError_t e = hipMemcpyAsync(dev_mem, host.data(), host.size() * 8, hipMemcpyHostToDevice,
                                as_stream(stream));
  std::vector<int32_t> table(n_pages > 0 ? (size_t)cfg->batch * hdr.page_stride : 0, -1);
  if (e == hipSuccess && !table.empty())
    e = hipMemcpyAsync(static_cast<char*>(dev_mem) + pt_off, table.data(), table.size() * 4,
                       hipMemcpyHostToDevice, as_stream(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "cache init copy");
  cache->cfg = *cfg;
  cache->dev = dev_mem;
  cache->bytes = bytes;
  cache->len = 0;
  cache->n_pages = n_pages;
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_cache_init(kvq_cache* cache, const kvq_config* cfg, void* dev_mem, size_t bytes,
                          void* stream) {
  return init_blob(cache, cfg, 0, dev_mem, bytes, stream);
}

size_t kvq_cache_bytes_paged(const kvq_config* cfg, int32_t n_pages) {
  if (check_config(cfg) != KVQ_OK || check_pages(cfg, n_pages) != KVQ_OK) return 0;
  return (size_t)plan_layout(*cfg, nullptr, n_pages);
}

kvq_status kvq_cache_init_paged(kvq_cache* cache, const kvq_config* cfg, int32_t n_pages, void* dev_mem,
                                size_t bytes, void* stream) {
  if (n_pages < 1) return fail(KVQ_ERR_ARG, "n_pages must be >= 1");
  return init_blob(cache, cfg, n_pages, dev_mem, bytes, stream);
}

kvq_status kvq_cache_map_pages(const kvq_cache* cache, int32_t row, int32_t first_tile, int32_t n_tiles,
                               const int32_t* pages, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (cache->n_pages <= 0) return fail(KVQ_ERR_ARG, "not a paged cache");
  const int stride = page_stride(cache->cfg);
  if (row < 0 || row >= cache->cfg.batch) return fail(KVQ_ERR_ARG, "row out of range");
  if (n_tiles < 0 || first_tile < 0 || (int64_t)first_tile + n_tiles > stride)
    return fail(KVQ_ERR_ARG, "tiles out of range (a row has " + std::to_string(stride) + ")");
  if (n_tiles == 0) return KVQ_OK;
  if (!pages) return fail(KVQ_ERR_ARG, "pages is NULL");
  for (int i = 0; i < n_tiles; ++i)
    if (pages[i] < -1 || pages[i] >= cache->n_pages)
      return fail(KVQ_ERR_ARG, "page index out of range at " + std::to_string(i));
  uint64_t pt_off = 0;
  plan_layout(cache->cfg, nullptr, cache->n_pages, &pt_off);
  char* table = static_cast<char*>(cache->dev) + pt_off;
  // The table as it will be after this call must give no page to two tiles (of any row):
  // read it back, apply the new entries on the host and count every page's uses.
  const size_t entries = (size_t)cache->cfg.batch * stride;
  std::vector<int32_t> after(entries);
  hipError_t e = hipMemcpyAsync(after.data(), table, entries * 4, hipMemcpyDeviceToHost, as_stream(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "page table read");
  std::copy(pages, pages + n_tiles, after.begin() + (size_t)row * stride + first_tile);
  std::vector<int64_t> owner(cache->n_pages, -1);
  for (size_t i = 0; i < entries; ++i) {
    const int32_t pg = after[i];
    if (pg < 0) continue;
    if (pg >= cache->n_pages) return fail(KVQ_ERR_ARG, "the page table holds an out-of-range page");
    if (owner[pg] >= 0) {
      const size_t j = (size_t)owner[pg];
      return fail(KVQ_ERR_ARG, "page " + std::to_string(pg) + " would hold two tiles: row " + std::to_string(j / stride) +
                                   " tile " + std::to_string(j % stride) + " and row " + std::to_string(i / stride) +
                                   " tile " + std::to_string(i % stride));
    }
    owner[pg] = (int64_t)i;
  }
  char* dst = table + ((size_t)row * stride + first_tile) * 4;
  e = hipMemcpyAsync(dst, pages, (size_t)n_tiles * 4, hipMemcpyHostToDevice, as_stream(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "page table copy");
  return KVQ_OK;
}

kvq_status kvq_cache_check(const kvq_cache* cache, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  uint32_t flag = 0;
  hipError_t e = hipMemcpyAsync(&flag, flag_ptr(cache), 4, hipMemcpyDeviceToHost, as_stream(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "cache check");
  if (flag & 1u) return fail(KVQ_ERR_RANGE, "a quantized input was non-finite or |x| > 2^14");
  if (flag & 2u) return fail(KVQ_ERR_PAGE, "an append reached a tile with no page mapped");
  return KVQ_OK;
}

kvq_status kvq_append(kvq_cache* cache, const void* k_dev, const void* v_dev, int32_t n_new,
                      void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (n_new < 0) return fail(KVQ_ERR_ARG, "n_new must be >= 0");
  if (n_new == 0) return KVQ_OK;
  if (!k_dev || !v_dev) return fail(KVQ_ERR_ARG, "NULL input");
  if (!aligned(k_dev, 16) || !aligned(v_dev, 16)) return fail(KVQ_ERR_ARG, "inputs must be 16-byte aligned");
  const kvq_config& c = cache->cfg;
  if ((int64_t)cache->len + n_new > c.capacity) return fail(KVQ_ERR_CAPACITY, "append exceeds capacity");
  AppendPlan p{};
  p.k_in = k_dev;
  p.v_in = v_dev;
  p.blob = static_cast<char*>(cache->dev);
  p.off = table_ptr(cache);
  set_pages(cache, p);
  p.range_flag = flag_ptr(cache);
  p.B = c.batch;
  p.H = c.n_kv_heads;
  p.D = c.head_dim;
  p.n_new = n_new;
  p.len0 = cache->len;
  p.len1 = cache->len + n_new;
  p.body0 = (int)body_len(p.len0, c.n_sink, c.n_recent);
  p.body1 = (int)body_len(p.len1, c.n_sink, c.n_recent);
  p.n_sink = c.n_sink;
  p.n_recent = c.n_recent;
  p.dtype = c.dtype;
  p.hybrid = quant_mode(c) == KVQ_QUANT_HYBRID;
  p.key_norm = key_norm(c);
  std::memcpy(p.k_bits, c.k_bits, sizeof(p.k_bits));
  std::memcpy(p.v_bits, c.v_bits, sizeof(p.v_bits));
  // The key norms come from the first append, before any block of it is quantized.
  if (p.key_norm && p.len0 == 0) {
    st = check_launch(launch_key_norms(p, stream), "key norm launch");
    if (st != KVQ_OK) return st;
  }
  // Blocks leaving the ring are quantized first; the window copy runs after it on the same
  // stream, so new ring tokens never overwrite ring slots that a flushed block still reads.
  if (p.body1 > p.body0) {
    st = check_launch(launch_append_flush(p, stream), "append flush launch");
    if (st != KVQ_OK) return st;
  }
  st = check_launch(launch_append_window(p, stream), "append window launch");
  if (st != KVQ_OK) return st;
  cache->len = p.len1;
  return KVQ_OK;
}

kvq_status kvq_append_ragged(const kvq_cache* cache, const int32_t* row_len, const int32_t* n_new,
                             const void* k_dev, const void* v_dev, int32_t n_max, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  const kvq_config& c = cache->cfg;
  if (!row_len || !n_new) return fail(KVQ_ERR_ARG, "NULL row_len or n_new");
  if (n_max < 0) return fail(KVQ_ERR_ARG, "n_max must be >= 0");
  bool any = false;
  for (int b = 0; b < c.batch; ++b) {
    if (row_len[b] < 0 || n_new[b] < 0 || n_new[b] > n_max) return fail(KVQ_ERR_ARG, "row length or n_new out of range");
    if ((int64_t)row_len[b] + n_new[b] > c.capacity) return fail(KVQ_ERR_CAPACITY, "append exceeds capacity");
    any |= n_new[b] > 0;
  }
  if (!any) return KVQ_OK;
  if (!k_dev || !v_dev) return fail(KVQ_ERR_ARG, "NULL input");
  if (!aligned(k_dev, 16) || !aligned(v_dev, 16)) return fail(KVQ_ERR_ARG, "inputs must be 16-byte aligned");
  // The per-row counts travel in the launch plan (kMaxRaggedRows of them), so a larger batch
  // runs as consecutive groups of rows: each group's plan sees its rows as rows 0.. through
  // offset region table, page table and input pointers. Groups touch disjoint rows.
  const size_t row_elems = (size_t)c.n_kv_heads * n_max * c.head_dim;  // 16-bit input elements per row
  const uint64_t* tab = table_ptr(cache);
  for (int r0 = 0; r0 < c.batch; r0 += kMaxRaggedRows) {
    const int nr = std::min(kMaxRaggedRows, c.batch - r0);
    AppendPlan p{};
    p.k_in = static_cast<const uint16_t*>(k_dev) + (size_t)r0 * row_elems;
    p.v_in = static_cast<const uint16_t*>(v_dev) + (size_t)r0 * row_elems;
    p.blob = static_cast<char*>(cache->dev);
    p.off = tab + (size_t)r0 * c.n_kv_heads * kRegions;
    set_pages(cache, p);
    if (p.pages) p.pages += (size_t)r0 * p.page_stride;
    p.range_flag = flag_ptr(cache);
    p.B = nr;
    p.H = c.n_kv_heads;
    p.D = c.head_dim;
    p.n_new = n_max;  // the input's token stride
    p.n_sink = c.n_sink;
    p.n_recent = c.n_recent;
    p.dtype = c.dtype;
    p.hybrid = quant_mode(c) == KVQ_QUANT_HYBRID;
    p.key_norm = key_norm(c);
    std::memcpy(p.k_bits, c.k_bits, sizeof(p.k_bits));
    std::memcpy(p.v_bits, c.v_bits, sizeof(p.v_bits));
    p.ragged = 1;
    bool flush = false, first_here = false, any_here = false;
    for (int b = 0; b < nr; ++b) {
      p.row_len0[b] = row_len[r0 + b];
      p.row_new[b] = n_new[r0 + b];
      const RowAppend a = host_row_append(p, b);
      flush |= a.body1 > a.body0;
      first_here |= a.len0 == 0 && a.n > 0;
      any_here |= a.n > 0;
    }
    if (!any_here) continue;
    // same order as kvq_append: norms of rows appended for the first time, flushes, window copies
    if (p.key_norm && first_here) {
      st = check_launch(launch_key_norms(p, stream), "key norm launch");
      if (st != KVQ_OK) return st;
    }
    if (flush) {
      st = check_launch(launch_append_flush(p, stream), "append flush launch");
      if (st != KVQ_OK) return st;
    }
    st = check_launch(launch_append_window(p, stream), "append window launch");
    if (st != KVQ_OK) return st;
  }
  return KVQ_OK;
}

size_t kvq_decode_multi_workspace_bytes(const kvq_cache* cache, int32_t n_splits, int32_t n_qtok) {
  if (check_cache(cache) != KVQ_OK) return 0;
  if (n_splits < 1 || n_splits > 256) {
    set_error("n_splits must be in 1..256");
    return 0;
  }
  if (n_qtok < 1 || n_qtok * (cache->cfg.n_q_heads / cache->cfg.n_kv_heads) > kMaxDenseRows) {
    set_error("n_qtok must be >= 1 and n_qtok * (query heads per KV head) <= 16");
    return 0;
  }
  const kvq_config& c = cache->cfg;
  const size_t parts = (size_t)n_splits;
  const size_t rows = (size_t)c.batch * n_qtok * c.n_q_heads;
  return align_up(parts * rows * c.head_dim * 4) + align_up(parts * rows * 2 * 4);
}

size_t kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t n_splits) {
  return kvq_decode_multi_workspace_bytes(cache, n_splits, 1);
}

}  // extern "C"

namespace {

// Checks shared by the decode entry points; fills the launch plan.
kvq_status decode_plan(const kvq_cache* cache, const void* q_dev, float* out_dev, int32_t n_splits, float scale,
                       void* ws, size_t ws_bytes, DecodePlan& p, int32_t n_qtok = 1) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (cache->len < 1) return fail(KVQ_ERR_ARG, "decode on an empty cache");
  if (!ws) return fail(KVQ_ERR_ARG, "NULL workspace");
  if (n_splits < 1 || n_splits > 256) return fail(KVQ_ERR_ARG, "n_splits must be in 1..256");
  if ((q_dev && !aligned(q_dev, 16)) || (out_dev && !aligned(out_dev, 16)) || !aligned(ws, 256))
    return fail(KVQ_ERR_ARG, "q/out must be 16-byte and workspace 256-byte aligned");
  if (!(std::isfinite(scale))) return fail(KVQ_ERR_ARG, "scale must be finite");
  const size_t need = kvq_decode_multi_workspace_bytes(cache, n_splits, n_qtok);
  if (need == 0) return fail(KVQ_ERR_ARG, last_error());
  if (ws_bytes < need) return fail(KVQ_ERR_ARG, "workspace too small");
  const kvq_config& c = cache->cfg;
  p = DecodePlan{};
  p.blob = static_cast<const char*>(cache->dev);
  p.off = table_ptr(cache);
  set_pages(cache, p);
  p.flag = flag_ptr(cache);
  p.q = q_dev;
  p.out = out_dev;
  const size_t parts = (size_t)n_splits;
  const size_t rows = (size_t)c.batch * n_qtok * c.n_q_heads;
  p.ws_o = static_cast<float*>(ws);
  p.ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(parts * rows * c.head_dim * 4));
  p.B = c.batch;
  p.H = c.n_kv_heads;
  p.Hq = c.n_q_heads;
  p.G = c.n_q_heads / c.n_kv_heads;
  p.Q = n_qtok;
  p.D = c.head_dim;
  p.T = cache->len;
  p.body = (int)body_len(cache->len, c.n_sink, c.n_recent);
  p.n_sink_live = std::min(cache->len, c.n_sink);
  p.n_win = cache->len - p.n_sink_live - p.body;
  p.n_sink_cfg = c.n_sink;
  p.ring = ring_slots(c.n_recent);
  p.n_splits = n_splits;
  p.ring0 = p.body % p.ring;
  p.n_tiles = (p.body + kTile - 1) / kTile;
  p.n_wtiles = (p.n_sink_live + p.n_win + kWinTile - 1) / kWinTile;
  p.tiles_per_split = (p.n_tiles + n_splits - 1) / n_splits;
  p.dtype = c.dtype;
  p.key_norm = key_norm(c);
  const float s = scale > 0.0f ? scale : 1.0f / std::sqrt((float)c.head_dim);
  p.scale_log2 = s * 1.4426950408889634f;
  std::memcpy(p.k_bits, c.k_bits, sizeof(p.k_bits));
  std::memcpy(p.v_bits, c.v_bits, sizeof(p.v_bits));
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_decode_splitk(const kvq_cache* cache, const void* q_dev, int32_t n_splits, float scale,
                             void* ws, size_t ws_bytes, void* stream) {
  if (!q_dev) return fail(KVQ_ERR_ARG, "NULL q");
  DecodePlan p;
  kvq_status st = decode_plan(cache, q_dev, nullptr, n_splits, scale, ws, ws_bytes, p);
  if (st != KVQ_OK) return st;
  return check_launch(launch_decode_splitk(p, stream), "decode launch");
}

kvq_status kvq_decode_merge(const kvq_cache* cache, float* out_dev, int32_t n_splits, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!out_dev) return fail(KVQ_ERR_ARG, "NULL out");
  DecodePlan p;
  kvq_status st = decode_plan(cache, nullptr, out_dev, n_splits, 0.0f, ws, ws_bytes, p);
  if (st != KVQ_OK) return st;
  return check_launch(launch_decode_merge(p, stream), "merge launch");
}

kvq_status kvq_decode_step(kvq_cache* cache, const void* k_dev, const void* v_dev, int32_t n_new,
                           const void* q_dev, float* out_dev, int32_t n_splits, float scale, void* ws,
                           size_t ws_bytes, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (!q_dev || !out_dev) return fail(KVQ_ERR_ARG, "NULL pointer");
  const kvq_config& c = cache->cfg;
  const int len0 = cache->len, len1 = len0 + n_new;
  // (with key normalization the norms come from the first append: that one is not fused)
  const bool fused = n_new == 1 && len0 >= c.n_sink && !(key_norm(c) && len0 == 0);
  if (!fused) {
    st = kvq_append(cache, k_dev, v_dev, n_new, stream);
    if (st != KVQ_OK) return st;
    return kvq_decode_attention(cache, q_dev, out_dev, n_splits, scale, ws, ws_bytes, stream);
  }
  if (!k_dev || !v_dev) return fail(KVQ_ERR_ARG, "NULL input");
  if (!aligned(k_dev, 16) || !aligned(v_dev, 16)) return fail(KVQ_ERR_ARG, "inputs must be 16-byte aligned");
  if ((int64_t)len1 > c.capacity) return fail(KVQ_ERR_CAPACITY, "append exceeds capacity");
  // validate the decode arguments on the cache as it will be after the append (nothing has
  // been enqueued yet, and cache->len is restored if they are rejected)
  kvq_cache after = *cache;
  after.len = len1;
  DecodePlan d;
  st = decode_plan(&after, q_dev, out_dev, n_splits, scale, ws, ws_bytes, d);
  if (st != KVQ_OK) return st;
  AppendPlan a{};
  a.k_in = k_dev;
  a.v_in = v_dev;
  a.blob = static_cast<char*>(cache->dev);
  a.off = table_ptr(cache);
  set_pages(cache, a);
  a.range_flag = flag_ptr(cache);
  a.B = c.batch;
  a.H = c.n_kv_heads;
  a.D = c.head_dim;
  a.n_new = 1;
  a.len0 = len0;
  a.len1 = len1;
  a.body0 = (int)body_len(len0, c.n_sink, c.n_recent);
  a.body1 = (int)body_len(len1, c.n_sink, c.n_recent);
  a.n_sink = c.n_sink;
  a.n_recent = c.n_recent;
  a.dtype = c.dtype;
  a.hybrid = quant_mode(c) == KVQ_QUANT_HYBRID;
  a.key_norm = key_norm(c);
  std::memcpy(a.k_bits, c.k_bits, sizeof(a.k_bits));
  std::memcpy(a.v_bits, c.v_bits, sizeof(a.v_bits));
  if (a.body1 > a.body0) {  // a block leaves the window: quantize it first
    st = check_launch(launch_append_flush(a, stream), "append flush launch");
    if (st != KVQ_OK) return st;
  }
  if (d.n_win > 0) {
    // the new token is the last window token: the decode kernel takes it from the inputs as
    // one more softmax term, reads the window as it stands before the append, and writes the
    // token into its ring slot
    d.new_k = k_dev;
    d.new_v = v_dev;
    d.new_slot = (len1 - 1 - c.n_sink) % ring_slots(c.n_recent);
    d.n_win -= 1;
    d.n_wtiles = (d.n_sink_live + d.n_win + kWinTile - 1) / kWinTile;
  }
  cache->len = len1;
  st = check_launch(launch_decode_splitk(d, stream), "decode launch");
  if (st != KVQ_OK) return st;
  return check_launch(launch_decode_merge(d, stream), "merge launch");
}

kvq_status kvq_decode_ragged(const kvq_cache* cache, const int32_t* row_len, const void* q_dev, float* out_dev,
                             int32_t n_splits, float scale, void* ws, size_t ws_bytes, void* stream) {
  if (!q_dev || !out_dev || !row_len) return fail(KVQ_ERR_ARG, "NULL pointer");
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  const kvq_config& c = cache->cfg;
  for (int b = 0; b < c.batch; ++b)
    if (row_len[b] < 1 || row_len[b] > c.capacity) return fail(KVQ_ERR_ARG, "every row needs 1..capacity tokens");
  // plan on a copy whose len is a valid stand-in; the kernels take each row's own length
  kvq_cache any = *cache;
  any.len = row_len[0];
  DecodePlan full;
  st = decode_plan(&any, q_dev, out_dev, n_splits, scale, ws, ws_bytes, full);
  if (st != KVQ_OK) return st;
  // The row lengths travel in the launch plan (kMaxRaggedRows of them), so a larger batch runs
  // as consecutive groups of rows, each a split-K launch and a merge whose plan sees its rows
  // as rows 0.. through offset region table, page table, q and out pointers. The groups reuse
  // the front of the workspace one after the other on the stream.
  for (int r0 = 0; r0 < c.batch; r0 += kMaxRaggedRows) {
    const int nr = std::min(kMaxRaggedRows, c.batch - r0);
    DecodePlan p = full;
    p.ragged = 1;
    p.B = nr;
    p.off = full.off + (size_t)r0 * c.n_kv_heads * kRegions;
    if (p.pages) p.pages += (size_t)r0 * p.page_stride;
    p.q = static_cast<const uint16_t*>(q_dev) + (size_t)r0 * c.n_q_heads * c.head_dim;
    p.out = out_dev + (size_t)r0 * c.n_q_heads * c.head_dim;
    const size_t rows = (size_t)nr * c.n_q_heads;
    p.ws_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(p.ws_o) + align_up((size_t)n_splits * rows * c.head_dim * 4));
    for (int b = 0; b < nr; ++b) p.row_len[b] = row_len[r0 + b];
    st = check_launch(launch_decode_splitk(p, stream), "decode launch");
    if (st != KVQ_OK) return st;
    st = check_launch(launch_decode_merge(p, stream), "merge launch");
    if (st != KVQ_OK) return st;
  }
  return KVQ_OK;
}

kvq_status kvq_decode_multi(const kvq_cache* cache, const void* q_dev, int32_t n_qtok, float* out_dev,
                            int32_t n_splits, float scale, void* ws, size_t ws_bytes, void* stream) {
  if (!q_dev || !out_dev) return fail(KVQ_ERR_ARG, "NULL pointer");
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  const kvq_config& c = cache->cfg;
  if (n_qtok < 1) return fail(KVQ_ERR_ARG, "n_qtok must be >= 1");
  const int rows = n_qtok * (c.n_q_heads / c.n_kv_heads);
  if (rows > kMaxDenseRows)
    return fail(KVQ_ERR_UNSUPPORTED, "n_qtok * (query heads per KV head) must be <= 16");
  if (cache->len < n_qtok) return fail(KVQ_ERR_ARG, "the cache holds fewer tokens than n_qtok");
  DecodePlan p;
  st = decode_plan(cache, q_dev, out_dev, n_splits, scale, ws, ws_bytes, p, n_qtok);
  if (st != KVQ_OK) return st;
  // the causal mask is applied to the 16-bit window only: the newest n_qtok - 1 tokens must
  // not have been quantized into the body yet
  if (p.body > 0 && p.n_win < n_qtok - 1)
    return fail(KVQ_ERR_UNSUPPORTED, "n_qtok - 1 exceeds the tokens of the recent window");
  // up to 4 rows: the single-query kernel's 4-row tile; more: the 16-row tile
  st = check_launch(rows <= kMaxQueryRows ? launch_decode_splitk(p, stream) : launch_decode_dense(p, stream),
                    "decode launch");
  if (st != KVQ_OK) return st;
  return check_launch(launch_decode_merge(p, stream), "merge launch");
}

kvq_status kvq_decode_attention(const kvq_cache* cache, const void* q_dev, float* out_dev,
                                int32_t n_splits, float scale, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!q_dev || !out_dev) return fail(KVQ_ERR_ARG, "NULL pointer");
  DecodePlan p;
  kvq_status st = decode_plan(cache, q_dev, out_dev, n_splits, scale, ws, ws_bytes, p);
  if (st != KVQ_OK) return st;
  st = check_launch(launch_decode_splitk(p, stream), "decode launch");
  if (st != KVQ_OK) return st;
  return check_launch(launch_decode_merge(p, stream), "merge launch");
}

kvq_status kvq_decode_attention_noalloc(const kvq_cache* cache, const void* q_dev, float* out_dev,
                                        int32_t n_splits, float scale, void* stream) {
  if (!q_dev || !out_dev) return fail(KVQ_ERR_ARG, "NULL pointer");
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  const size_t need = kvq_decode_workspace_bytes(cache, n_splits);
  if (need == 0) return fail(KVQ_ERR_ARG, last_error());
  void* ws = nullptr;
  size_t cap = 0;
  const int e = static_scratch(&ws, &cap);
  if (e != (int)hipSuccess) return hip_fail((hipError_t)e, "static decode scratch");
  if (need > cap)
    return fail(KVQ_ERR_ARG, "the split partials need " + std::to_string(need) + " bytes; the static scratch holds " +
                                 std::to_string(cap) + " (use kvq_decode_attention with a workspace)");
  return kvq_decode_attention(cache, q_dev, out_dev, n_splits, scale, ws, cap, stream);
}

size_t kvq_calibrate_workspace_bytes(int32_t n_heads, int32_t n_tokens, int32_t head_dim,
                                     int32_t b_lo, int32_t b_hi) {
  if (n_heads < 1 || n_tokens < 1 || head_dim < 32 || head_dim % kGroup || b_hi < b_lo) return 0;
  const size_t groups = (size_t)n_tokens * head_dim / kGroup;
  const size_t blocks = (groups + kCalibThreads - 1) / kCalibThreads;
  return align_up((size_t)n_heads * (b_hi - b_lo + 1) * blocks * 8) + kAlign;
}

kvq_status kvq_calibrate_fit(const void* x_dev, int32_t dtype, int32_t n_heads, int32_t n_tokens,
                             int32_t head_dim, int32_t axis, int32_t quant, int32_t b_lo,
                             int32_t b_hi, void* ws, size_t ws_bytes, double* alpha,
                             double* beta, double* r2, void* stream) {
  if (!x_dev || !ws || !alpha || !beta || !r2) return fail(KVQ_ERR_ARG, "NULL pointer");
  if (dtype != KVQ_F16 && dtype != KVQ_BF16) return fail(KVQ_ERR_ARG, "bad dtype");
  if (n_heads < 1 || n_tokens < 1) return fail(KVQ_ERR_ARG, "n_heads and n_tokens must be >= 1");
  if (head_dim < 32 || head_dim % kGroup || head_dim > 4096)
    return fail(KVQ_ERR_ARG, "head_dim must be a multiple of 32");
  if (axis != KVQ_AXIS_KEY && axis != KVQ_AXIS_VALUE) return fail(KVQ_ERR_ARG, "bad axis");
  if (axis == KVQ_AXIS_VALUE && n_tokens % kGroup)
    return fail(KVQ_ERR_ARG, "value calibration needs n_tokens % 32 == 0");
  if (quant != KVQ_QUANT_ASYM && quant != KVQ_QUANT_HYBRID) return fail(KVQ_ERR_ARG, "bad quant");
  if (!(2 <= b_lo && b_lo + 2 <= b_hi && b_hi <= 8)) return fail(KVQ_ERR_ARG, "need 2 <= b_lo, b_lo + 2 <= b_hi <= 8");
  if (!aligned(x_dev, 16) || !aligned(ws, 256)) return fail(KVQ_ERR_ARG, "misaligned pointer");
  const size_t need = kvq_calibrate_workspace_bytes(n_heads, n_tokens, head_dim, b_lo, b_hi);
  if (ws_bytes < need) return fail(KVQ_ERR_ARG, "workspace too small");
  const int nb = b_hi - b_lo + 1;
  const int64_t groups = (int64_t)n_tokens * head_dim / kGroup;
  const int64_t blocks = (groups + kCalibThreads - 1) / kCalibThreads;
  if (blocks > INT32_MAX || n_heads > 65535) return fail(KVQ_ERR_ARG, "calibration slice too large");
  CalibPlan p{};
  p.x = x_dev;
  p.part = static_cast<double*>(ws);
  p.range_flag = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + need - kAlign);
  p.n_heads = n_heads;
  p.n_tokens = n_tokens;
  p.D = head_dim;
  p.axis = axis;
  p.hybrid = quant == KVQ_QUANT_HYBRID;
  p.dtype = dtype;
  p.b_lo = b_lo;
  p.nb = nb;
  p.n_groups = groups;
  p.n_blocks = (int)blocks;
  hipStream_t s = as_stream(stream);
  hipError_t e = hipMemsetAsync(p.range_flag, 0, 4, s);
  if (e != hipSuccess) return hip_fail(e, "calibrate flag clear");
  kvq_status st = check_launch(launch_calib(p, stream), "calibrate launch");
  if (st != KVQ_OK) return st;
  std::vector<double> part((size_t)n_heads * nb * blocks);
  uint32_t flag = 0;
  e = hipMemcpyAsync(part.data(), p.part, part.size() * 8, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&flag, p.range_flag, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "calibrate copy-back");
  if (flag) return fail(KVQ_ERR_RANGE, "calibration input non-finite or |x| > 2^14");
  // D(b) = (sum of the per-group SSE: workgroup sums added in workgroup order) / element count
  std::vector<double> D((size_t)n_heads * nb);
  const double n_el = (double)n_tokens * head_dim;
  for (int h = 0; h < n_heads; ++h)
    for (int i = 0; i < nb; ++i) {
      const double* g = part.data() + ((size_t)h * nb + i) * blocks;
      double tot = 0.0;
      for (int64_t k = 0; k < blocks; ++k) tot = tot + g[k];
      D[(size_t)h * nb + i] = tot / n_el;
    }
  return fit_distortion(n_heads, nb, D.data(), b_lo, alpha, beta, r2);
}

}  // extern "C"
