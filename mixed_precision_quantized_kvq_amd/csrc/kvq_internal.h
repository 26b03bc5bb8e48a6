// Internal declarations shared by the host side and the kernel launchers of libkvq.
// Not part of the public ABI (see include/kvq.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "kvq.h"

namespace kvq {

constexpr int kGroup = 32;        // quantization group size (keys: channels, values: tokens)
constexpr int kTile = 64;         // body tokens per key tile (one wavefront, one token per lane)
// 16-bit window tokens per unit of decode work (a unit is dealt to one wavefront; units
// smaller than a body tile spread the window's bytes over many wavefronts)
#ifndef KVQ_WIN_TILE
#define KVQ_WIN_TILE 16
#endif
constexpr int kWinTile = KVQ_WIN_TILE;
constexpr int kMaxQueryRows = 4;  // query rows per KV head in one decode launch (heads x tokens)
constexpr int kMaxDenseRows = 16;  // the same for the multi-token launch with the 16-row tile
constexpr int kMaxRaggedRows = 64;  // rows of a ragged call (per-row lengths travel as kernel arguments)
constexpr int kRegions = 10;
constexpr uint64_t kAlign = 256;  // every region starts on a 256-byte boundary
constexpr uint64_t kHeaderBytes = 256;
constexpr uint32_t kMagic = 0x3151564Bu;  // "KVQ1"
constexpr uint32_t kVersion = 3;        // 2: region KN (key norms) added; 3: paged caches
constexpr float kRangeLimit = 16384.0f;   // |x| <= 2^14 for quantized heads

enum Region { KC = 0, KM, VC, VM, FL, SK, SV, RK, RV, KN };

// Quantizer mode and flags packed in kvq_config.quant.
inline int quant_mode(const kvq_config& c) { return c.quant & 0xFF; }
inline bool key_norm(const kvq_config& c) { return (c.quant & KVQ_KEY_NORM) != 0; }

// Blob header (first 256 bytes of every cache blob). The region table follows it.
struct BlobHeader {
  uint32_t magic;
  uint32_t version;
  uint32_t range_flag;   // sticky: set by the device when a quantized input is out of range
  uint32_t n_regions;
  int32_t batch, n_kv_heads, head_dim, capacity;
  uint64_t table_offset; // byte offset of uint64 off[batch][n_kv_heads][kRegions]
  uint64_t total_bytes;
  // paged caches (n_pages > 0): int32 page[batch][page_stride] at page_table_offset; -1 = unmapped
  uint64_t page_table_offset;
  int32_t n_pages, page_stride;
};

inline uint64_t align_up(uint64_t x, uint64_t a = kAlign) { return (x + a - 1) / a * a; }

// Tokens quantized into the body after T tokens: whole 32-token blocks that have left the
// recent window (the window then holds n_recent..n_recent+31 tokens).
inline int64_t body_len(int64_t T, int64_t n_sink, int64_t n_recent) {
  int64_t r = T - n_sink - n_recent;
  return r <= 0 ? 0 : (r / kGroup) * kGroup;
}
inline int ring_slots(int n_recent) { return n_recent + kGroup; }

// Sizes of the kRegions regions of one (row, KV head).
// Paged caches (n_pages > 0): the body regions KC..FL are pools of n_pages 64-token tiles.
void region_sizes(const kvq_config& cfg, int kv_head, uint64_t sz[kRegions], int n_pages = 0);
// Body tiles of a full row: the page table's row stride.
int page_stride(const kvq_config& cfg);
// Full layout: off[(row*H + head)*kRegions + region], returns the total blob size.
// Paged caches: every row's entries for KC..FL name its head's pools, and *pt_off (nullable)
// receives the page table's offset.
uint64_t plan_layout(const kvq_config& cfg, uint64_t* off /* nullable */, int n_pages = 0,
                     uint64_t* pt_off = nullptr);

// Validation (sets the error string and returns a status).
kvq_status check_config(const kvq_config* cfg);

// Error handling.
void set_error(const std::string& msg);
kvq_status fail(kvq_status st, const std::string& msg);
const char* last_error();

// Host algorithms (kvq_host.cpp).
kvq_status fit_distortion(int n_heads, int nb, const double* D /*[n_heads][nb]*/, int b_lo,
                          double* alpha, double* beta, double* r2);

// ---------------------------------------------------------------------------------------
// Kernel launchers (device code in *.hip). All return hipError_t as int.
// ---------------------------------------------------------------------------------------

// Parameters of one append launch, computed on the host.
struct AppendPlan {
  const void* k_in;      // [B][H][n_new][D]
  const void* v_in;
  char* blob;            // device blob base
  const uint64_t* off;   // device region table
  uint32_t* range_flag;  // device sticky flag
  // paged caches: the body tile t of row b lives in page pages[b * page_stride + t] of each
  // head's pools (null for contiguous caches)
  const int32_t* pages;
  int page_stride, n_pages;
  int B, H, D, n_new;
  int len0, len1;        // token counts before / after
  int body0, body1;      // body lengths before / after
  int n_sink, n_recent;
  int dtype, hybrid;
  int key_norm;          // keys of quantized heads are divided by the stored per-channel norms
  alignas(4) uint8_t k_bits[KVQ_MAX_KV_HEADS];  // word-aligned: kernels read them a word at a time
  alignas(4) uint8_t v_bits[KVQ_MAX_KV_HEADS];
  // ragged rows: row b holds row_len0[b] tokens and appends row_new[b] (its first ones of the
  // n_new input slots); len0, len1, body0 and body1 above are then ignored
  int ragged;
  int32_t row_len0[kMaxRaggedRows];
  int32_t row_new[kMaxRaggedRows];
};
// Token counts of one row for an append: before / after, body before / after, new tokens.
struct RowAppend {
  int len0, len1, body0, body1, n;
};
inline RowAppend host_row_append(const AppendPlan& p, int b) {
  if (!p.ragged) return RowAppend{p.len0, p.len1, p.body0, p.body1, p.n_new};
  const int l0 = p.row_len0[b], n = p.row_new[b];
  return RowAppend{l0, l0 + n, (int)body_len(l0, p.n_sink, p.n_recent), (int)body_len(l0 + n, p.n_sink, p.n_recent), n};
}
int launch_append_flush(const AppendPlan& p, void* stream);
int launch_append_window(const AppendPlan& p, void* stream);
int launch_key_norms(const AppendPlan& p, void* stream);  // first append: per-channel key norms

constexpr int kCalibThreads = 256;  // groups per calibration workgroup
struct CalibPlan {
  const void* x;          // [n_heads][n_tokens][D]
  double* part;           // [n_heads][nb][n_blocks]: per-workgroup sums of group errors
  uint32_t* range_flag;   // device
  int n_heads, n_tokens, D, axis, hybrid, dtype, b_lo, nb, n_blocks;
  int64_t n_groups;
};
int launch_calib(const CalibPlan& p, void* stream);

struct DecodePlan {
  const char* blob;
  const uint64_t* off;
  const void* q;         // [B][Hq][D]
  float* out;            // [B][Hq][D]
  float* ws_o;           // [P][B][Hq][D]
  float* ws_ml;          // [P][B][Hq][2]
  const int32_t* pages;  // paged caches: as in AppendPlan (null for contiguous caches)
  int page_stride, n_pages;
  uint32_t* flag;        // the cache's sticky flag: bit 1 is set when a tile read is unmapped
  int B, H, Hq, G, D, T, body, n_sink_live, n_win, n_sink_cfg, ring;
  int Q;                 // query tokens per row: the last Q cached tokens, attended causally
  int ring0;             // ring slot of the oldest live window token (body mod ring)
  int n_splits, n_tiles, n_wtiles;  // partials, 64-token body tiles, kWinTile-token window units
  int tiles_per_split;   // body tiles per split (the window tiles are dealt out separately)
  int dtype;
  int key_norm;          // packed keys are k / n: their scores use q * n
  float scale_log2;      // softmax scale times log2(e)
  // fused decode step: the token being appended ([B][H][1][D], 16-bit), not counted in n_win.
  // The last split of each (row, head) attends to it; the merge launch writes it into ring
  // slot new_slot.
  // Null when not fused.
  const void* new_k;
  const void* new_v;
  int new_slot;
  alignas(4) uint8_t k_bits[KVQ_MAX_KV_HEADS];  // word-aligned: kernels read them a word at a time
  alignas(4) uint8_t v_bits[KVQ_MAX_KV_HEADS];
  // ragged rows: row b holds row_len[b] tokens, and T, body, n_sink_live, n_win, ring0,
  // n_tiles, n_wtiles and tiles_per_split above are ignored (each workgroup derives its row's)
  int ragged;
  int32_t row_len[kMaxRaggedRows];
};
int launch_decode_splitk(const DecodePlan& p, void* stream);

int launch_decode_merge(const DecodePlan& p, void* stream);
// Multi-token decode with up to kMaxDenseRows query rows per KV head: writes the split
// partials, like launch_decode_splitk.
int launch_decode_dense(const DecodePlan& p, void* stream);
// Device address and size of this device's static decode scratch (set up on first use per
// device); returns a hipError_t as int.
int static_scratch(void** ptr, size_t* bytes);

}  // namespace kvq
