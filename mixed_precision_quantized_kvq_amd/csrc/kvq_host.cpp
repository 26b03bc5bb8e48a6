// Host-side algorithms of libkvq: layout planning, configuration checks, the distortion
// fit and the bit allocator. Pure C++ (no device code); compiled with -ffp-contract=off so
// every floating-point step rounds exactly as written.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <queue>
#include <string>
#include <vector>

#include "kvq_internal.h"

namespace kvq {

// ------------------------------------------------------------------------- errors ------
static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }
kvq_status fail(kvq_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}
const char* last_error() { return g_last_error.c_str(); }

// ------------------------------------------------------------------------- layout ------
// Per (row, KV head) the blob holds, in this order, each region 256-byte aligned:
//   KC key codes   b-bit heads: tiles of 64 tokens; a token's W = D*b/32 words are cut into
//                  16-byte chunks and chunk q of all 64 tokens is contiguous (one 16-byte
//                  load per lane when lane = token). 16-bit heads: [body][D] 16-bit.
//   KM key meta    [token][D/32] x (fp16 s | fp16 z << 16)
//   VC value codes b-bit heads: [tile][channel][2 blocks][b words]; 16-bit: [body][D]
//   VM value meta  [tile][channel][2 blocks] x (s | z << 16)
//   FL hybrid flags [block][D/32 key words | D/32 value words] (hybrid caches only)
//   SK, SV sink    [n_sink][D] 16-bit
//   RK, RV ring    [n_recent + 32][D] 16-bit; token t >= n_sink sits in slot (t-n_sink) mod R
//   KN key norms   [D] fp32 (caches with KVQ_KEY_NORM, quantized key heads only)
//   Paged caches hold KC..FL as pools of n_pages tiles in the same per-tile order (a 16-bit
//   head's page holds 64 rows), one set of pools per head, shared by all rows.
int page_stride(const kvq_config& cfg) {
  return (int)((body_len(cfg.capacity, cfg.n_sink, cfg.n_recent) / kGroup + 1) / 2);
}

void region_sizes(const kvq_config& cfg, int h, uint64_t sz[kRegions], int n_pages) {
  const uint64_t D = (uint64_t)cfg.head_dim;
  const uint64_t bmax = n_pages > 0 ? (uint64_t)n_pages * kTile
                                    : (uint64_t)body_len(cfg.capacity, cfg.n_sink, cfg.n_recent);
  const uint64_t nblk = bmax / kGroup;
  const uint64_t ntile = (nblk + 1) / 2;
  const uint64_t kb = cfg.k_bits[h], vb = cfg.v_bits[h];
  sz[KC] = kb == 16 ? bmax * D * 2 : ntile * kTile * D * kb / 8;
  sz[KM] = kb == 16 ? 0 : ntile * kTile * (D / kGroup) * 4;
  sz[VC] = vb == 16 ? bmax * D * 2 : ntile * kTile * D * vb / 8;
  sz[VM] = vb == 16 ? 0 : ntile * 2 * D * 4;
  sz[FL] = quant_mode(cfg) == KVQ_QUANT_HYBRID ? nblk * 2 * (D / kGroup) * 4 : 0;
  sz[SK] = sz[SV] = (uint64_t)cfg.n_sink * D * 2;
  sz[RK] = sz[RV] = (uint64_t)ring_slots(cfg.n_recent) * D * 2;
  sz[KN] = key_norm(cfg) && kb != 16 ? D * 4 : 0;
}

uint64_t plan_layout(const kvq_config& cfg, uint64_t* off, int n_pages, uint64_t* pt_off) {
  const uint64_t B = cfg.batch, H = cfg.n_kv_heads;
  uint64_t pos = align_up(kHeaderBytes + B * H * kRegions * 8);
  if (n_pages <= 0) {
    for (uint64_t b = 0; b < B; ++b)
      for (uint64_t h = 0; h < H; ++h) {
        uint64_t sz[kRegions];
        region_sizes(cfg, (int)h, sz);
        for (int r = 0; r < kRegions; ++r) {
          if (off) off[(b * H + h) * kRegions + r] = pos;
          pos = align_up(pos + sz[r]);
        }
      }
    if (pt_off) *pt_off = 0;
    return pos;
  }
  // pools KC..FL of each head, then the windows and norms of each (row, head), then the table
  for (uint64_t h = 0; h < H; ++h) {
    uint64_t sz[kRegions];
    region_sizes(cfg, (int)h, sz, n_pages);
    for (int r = KC; r <= FL; ++r) {
      for (uint64_t b = 0; b < B && off; ++b) off[(b * H + h) * kRegions + r] = pos;
      pos = align_up(pos + sz[r]);
    }
  }
  for (uint64_t b = 0; b < B; ++b)
    for (uint64_t h = 0; h < H; ++h) {
      uint64_t sz[kRegions];
      region_sizes(cfg, (int)h, sz, n_pages);
      for (int r = SK; r < kRegions; ++r) {
        if (off) off[(b * H + h) * kRegions + r] = pos;
        pos = align_up(pos + sz[r]);
      }
    }
  if (pt_off) *pt_off = pos;
  return align_up(pos + B * (uint64_t)page_stride(cfg) * 4);
}

static bool bits_ok(int b) { return (b >= 2 && b <= 8) || b == 16; }

kvq_status check_config(const kvq_config* c) {
  if (!c) return fail(KVQ_ERR_ARG, "config is NULL");
  if (c->batch < 1) return fail(KVQ_ERR_ARG, "batch must be >= 1");
  if (c->n_kv_heads < 1 || c->n_kv_heads > KVQ_MAX_KV_HEADS)
    return fail(KVQ_ERR_ARG, "n_kv_heads must be in 1..128");
  if (c->n_q_heads < c->n_kv_heads || c->n_q_heads % c->n_kv_heads)
    return fail(KVQ_ERR_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
  if (c->n_q_heads / c->n_kv_heads > 4)
    return fail(KVQ_ERR_UNSUPPORTED, "more than 4 query heads per KV head is not implemented");
  if (c->group != kGroup) return fail(KVQ_ERR_UNSUPPORTED, "group must be 32");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(KVQ_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->capacity < 1) return fail(KVQ_ERR_ARG, "capacity must be >= 1");
  if (c->n_sink < 0 || c->n_recent < 0) return fail(KVQ_ERR_ARG, "negative window size");
  if (c->n_sink > (1 << 20) || c->n_recent > (1 << 20))
    return fail(KVQ_ERR_ARG, "window too large");
  if (c->dtype != KVQ_F16 && c->dtype != KVQ_BF16) return fail(KVQ_ERR_ARG, "bad dtype");
  if ((quant_mode(*c) != KVQ_QUANT_ASYM && quant_mode(*c) != KVQ_QUANT_HYBRID) ||
      (c->quant & ~(0xFF | KVQ_KEY_NORM)))
    return fail(KVQ_ERR_ARG, "bad quant mode");
  for (int h = 0; h < c->n_kv_heads; ++h)
    if (!bits_ok(c->k_bits[h]) || !bits_ok(c->v_bits[h]))
      return fail(KVQ_ERR_ARG, "bits must be 2..8 or 16 (head " + std::to_string(h) + ")");
  const double bytes = (double)plan_layout(*c, nullptr);
  if (bytes > 1.0e15) return fail(KVQ_ERR_ARG, "cache too large");
  return KVQ_OK;
}

// ------------------------------------------------------------------------- fit ---------
// Least squares of y = ln D(b) on x = b (RateQuant: D(b) = alpha * beta^-b, section 3.1),
// then the fallback for poor fits (section W.10): R^2 < 0.96 -> beta = min(beta, beta_bar),
// beta_bar = mean beta of the well-fitted heads (all non-degenerate heads if none).
// A head with some D(b) <= 0 is exactly representable: alpha = 0, beta = 4, R^2 = 1.
// A fitted beta <= 1 is a poor fit that takes beta_bar (min() would keep an invalid model).
kvq_status fit_distortion(int n_heads, int nb, const double* D, int b_lo, double* alpha,
                          double* beta, double* r2) {
  std::vector<char> degen(n_heads, 0);
  for (int h = 0; h < n_heads; ++h) {
    const double* d = D + (size_t)h * nb;
    bool deg = false;
    for (int i = 0; i < nb; ++i)
      if (!(d[i] > 0.0) || std::isinf(d[i])) deg = true;
    if (deg) {
      degen[h] = 1;
      alpha[h] = 0.0;
      beta[h] = 4.0;
      r2[h] = 1.0;
      continue;
    }
    double xbar = 0.0, ybar = 0.0;
    for (int i = 0; i < nb; ++i) {
      xbar += (double)(b_lo + i);
      ybar += std::log(d[i]);
    }
    xbar /= nb;
    ybar /= nb;
    double sxy = 0.0, sxx = 0.0;
    for (int i = 0; i < nb; ++i) {
      const double x = (double)(b_lo + i), y = std::log(d[i]);
      sxy += (x - xbar) * (y - ybar);
      sxx += (x - xbar) * (x - xbar);
    }
    const double slope = sxy / sxx;
    const double icpt = ybar - slope * xbar;
    double ss_res = 0.0, ss_tot = 0.0;
    for (int i = 0; i < nb; ++i) {
      const double x = (double)(b_lo + i), y = std::log(d[i]);
      const double r = y - (icpt + slope * x);
      ss_res += r * r;
      ss_tot += (y - ybar) * (y - ybar);
    }
    r2[h] = ss_tot == 0.0 ? 1.0 : 1.0 - ss_res / ss_tot;
    alpha[h] = std::exp(icpt);
    beta[h] = std::exp(-slope);
  }
  const double kR2 = 0.96;
  double sum = 0.0;
  int cnt = 0;
  for (int h = 0; h < n_heads; ++h)
    if (!degen[h] && r2[h] >= kR2 && beta[h] > 1.0) {
      sum += beta[h];
      ++cnt;
    }
  if (cnt == 0)
    for (int h = 0; h < n_heads; ++h)
      if (!degen[h] && beta[h] > 1.0) {
        sum += beta[h];
        ++cnt;
      }
  const double bbar = cnt ? sum / cnt : 4.0;
  for (int h = 0; h < n_heads; ++h) {
    if (degen[h]) continue;
    if (beta[h] <= 1.0)
      beta[h] = bbar;
    else if (r2[h] < kR2)
      beta[h] = std::min(beta[h], bbar);
  }
  return KVQ_OK;
}

}  // namespace kvq

// ------------------------------------------------------------------------- allocation --
// RateQuant sections 3.1 / 3.3 / B.1 / B.3 / U: minimize sum w_i a_i beta_i^-b_i subject to
// sum b_i = total and b_lo <= b_i <= b_hi. Integer: greedy over marginal gains with a
// max-heap, optimal because the gains decrease in b (the exponential model is convex).
// Continuous: reverse waterfilling, solved exactly over the breakpoints of sum b_i(theta).
namespace {

double marginal_key(double w, double a, double bt, int b) {
  // ln(w * a * beta^-b * (1 - 1/beta)), evaluated left to right; ln 0 = -inf
  const double la = a > 0.0 ? std::log(a) : -std::numeric_limits<double>::infinity();
  return ((std::log(w) + la) + std::log(1.0 - 1.0 / bt)) - (double)b * std::log(bt);
}

struct HeapItem {
  double key;
  int head;
};
struct HeapLess {  // max-heap on key; equal keys: lowest head index on top
  bool operator()(const HeapItem& x, const HeapItem& y) const {
    if (x.key != y.key) return x.key < y.key;
    return x.head > y.head;
  }
};

void waterfill(int n, const double* alpha, const double* beta, const double* w, int total,
               int b_lo, int b_hi, double* out) {
  // b_i(theta) = clip((c_i - theta) / l_i, b_lo, b_hi), c_i = ln(w_i a_i l_i), l_i = ln beta_i
  std::vector<double> c(n), l(n);
  std::vector<double> pts;
  const double ninf = -std::numeric_limits<double>::infinity();
  for (int i = 0; i < n; ++i) {
    l[i] = std::log(beta[i]);
    c[i] = alpha[i] > 0.0 ? std::log(w[i] * alpha[i] * l[i]) : ninf;
    if (c[i] != ninf) {
      pts.push_back(c[i] - b_hi * l[i]);  // below this theta the head sits at b_hi
      pts.push_back(c[i] - b_lo * l[i]);  // above this theta the head sits at b_lo
    }
  }
  auto bits_at = [&](double th, int i) {
    if (c[i] == ninf) return (double)b_lo;
    return std::min((double)b_hi, std::max((double)b_lo, (c[i] - th) / l[i]));
  };
  auto sum_at = [&](double th) {
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += bits_at(th, i);
    return s;
  };
  // Heads with alpha = 0 have nothing to gain; as in the greedy form they take bits only once
  // every other head sits at b_hi, and then share the remainder evenly.
  int n_deg = 0;
  double full = 0.0;
  for (int i = 0; i < n; ++i) {
    if (c[i] == ninf) {
      ++n_deg;
      full += b_lo;
    } else {
      full += b_hi;
    }
  }
  if ((double)total >= full) {
    const double extra = n_deg ? ((double)total - full) / n_deg : 0.0;
    for (int i = 0; i < n; ++i) out[i] = c[i] == ninf ? b_lo + extra : (double)b_hi;
    return;
  }
  if (pts.empty() || total == n * b_lo) {
    for (int i = 0; i < n; ++i) out[i] = b_lo;
    return;
  }
  std::sort(pts.begin(), pts.end());
  // sum_at is non-increasing in theta; find the breakpoint interval holding `total`
  double th_lo = pts.front(), th_hi = pts.back();
  if (sum_at(th_lo) <= total) {
    th_hi = th_lo;
  } else {
    for (size_t k = 1; k < pts.size(); ++k) {
      if (sum_at(pts[k]) <= total) {
        th_lo = pts[k - 1];
        th_hi = pts[k];
        break;
      }
    }
  }
  // on [th_lo, th_hi] the sum is linear: free heads contribute (c_i - theta) / l_i
  const double mid = 0.5 * (th_lo + th_hi);
  double fixed = 0.0, inv = 0.0, cl = 0.0;
  for (int i = 0; i < n; ++i) {
    const double raw = c[i] == ninf ? ninf : (c[i] - mid) / l[i];
    if (c[i] == ninf || raw <= b_lo) {
      fixed += b_lo;
    } else if (raw >= b_hi) {
      fixed += b_hi;
    } else {
      inv += 1.0 / l[i];
      cl += c[i] / l[i];
    }
  }
  double th = th_hi;
  if (inv > 0.0) th = (cl + fixed - total) / inv;
  th = std::min(std::max(th, th_lo), th_hi);
  for (int i = 0; i < n; ++i) out[i] = bits_at(th, i);
}

}  // namespace

extern "C" kvq_status kvq_allocate_bits(int32_t n, const double* alpha, const double* beta,
                                        const double* w_in, int32_t total, int32_t b_lo,
                                        int32_t b_hi, uint32_t flags, uint8_t* bits_out,
                                        double* bits_cont_out) {
  using kvq::fail;
  if (n < 1 || n > 1000000) return fail(KVQ_ERR_ARG, "n must be in 1..1e6");
  if (!alpha || !beta || !w_in || !bits_out) return fail(KVQ_ERR_ARG, "NULL array");
  if (!(2 <= b_lo && b_lo <= b_hi && b_hi <= 8)) return fail(KVQ_ERR_ARG, "need 2 <= b_lo <= b_hi <= 8");
  if (flags & ~(uint32_t)KVQ_ALLOC_CAP_W) return fail(KVQ_ERR_ARG, "unknown flags");
  for (int i = 0; i < n; ++i) {
    if (!(std::isfinite(alpha[i]) && alpha[i] >= 0.0))
      return fail(KVQ_ERR_ARG, "alpha must be finite and >= 0");
    if (!(std::isfinite(beta[i]) && beta[i] > 1.0))
      return fail(KVQ_ERR_ARG, "beta must be finite and > 1");
    if (!(std::isfinite(w_in[i]) && w_in[i] > 0.0))
      return fail(KVQ_ERR_ARG, "w must be finite and > 0");
  }
  if ((int64_t)n * b_lo > total || total > (int64_t)n * b_hi)
    return fail(KVQ_ERR_BUDGET, "budget outside [n*b_lo, n*b_hi]");
  std::vector<double> w(w_in, w_in + n);
  if (flags & KVQ_ALLOC_CAP_W) {  // RateQuant W.14: w_i <- min(w_i, 5 * mean w)
    double mean = 0.0;
    for (int i = 0; i < n; ++i) mean += w[i];
    mean /= n;
    for (int i = 0; i < n; ++i) w[i] = std::min(w[i], 5.0 * mean);
  }
  std::vector<int> bits(n, b_lo);
  std::priority_queue<HeapItem, std::vector<HeapItem>, HeapLess> heap;
  if (b_hi > b_lo)
    for (int i = 0; i < n; ++i) heap.push({marginal_key(w[i], alpha[i], beta[i], b_lo), i});
  for (int64_t r = (int64_t)total - (int64_t)n * b_lo; r > 0; --r) {
    HeapItem top = heap.top();
    heap.pop();
    const int i = top.head;
    bits[i] += 1;
    if (bits[i] < b_hi) heap.push({marginal_key(w[i], alpha[i], beta[i], bits[i]), i});
  }
  for (int i = 0; i < n; ++i) bits_out[i] = (uint8_t)bits[i];
  if (bits_cont_out) waterfill(n, alpha, beta, w.data(), total, b_lo, b_hi, bits_cont_out);
  return KVQ_OK;
}

// Decision margin of an integer allocation (RateQuant section 3.3): the smallest marginal key
// that was handed a bit minus the largest key left without one. The greedy hands bits in key
// order, so the margin of its result is >= 0, and 0 exactly where a tie was broken by index.
extern "C" kvq_status kvq_allocation_margin(int32_t n, const double* alpha, const double* beta,
                                            const double* w_in, const uint8_t* bits, int32_t b_lo,
                                            int32_t b_hi, uint32_t flags, double* margin_out) {
  using kvq::fail;
  if (n < 1 || n > 1000000) return fail(KVQ_ERR_ARG, "n must be in 1..1e6");
  if (!alpha || !beta || !w_in || !bits || !margin_out) return fail(KVQ_ERR_ARG, "NULL array");
  if (!(2 <= b_lo && b_lo <= b_hi && b_hi <= 8)) return fail(KVQ_ERR_ARG, "need 2 <= b_lo <= b_hi <= 8");
  if (flags & ~(uint32_t)KVQ_ALLOC_CAP_W) return fail(KVQ_ERR_ARG, "unknown flags");
  for (int i = 0; i < n; ++i) {
    if (!(std::isfinite(alpha[i]) && alpha[i] >= 0.0))
      return fail(KVQ_ERR_ARG, "alpha must be finite and >= 0");
    if (!(std::isfinite(beta[i]) && beta[i] > 1.0))
      return fail(KVQ_ERR_ARG, "beta must be finite and > 1");
    if (!(std::isfinite(w_in[i]) && w_in[i] > 0.0))
      return fail(KVQ_ERR_ARG, "w must be finite and > 0");
    if (bits[i] < b_lo || bits[i] > b_hi) return fail(KVQ_ERR_ARG, "bits outside [b_lo, b_hi]");
  }
  std::vector<double> w(w_in, w_in + n);
  if (flags & KVQ_ALLOC_CAP_W) {
    double mean = 0.0;
    for (int i = 0; i < n; ++i) mean += w[i];
    mean /= n;
    for (int i = 0; i < n; ++i) w[i] = std::min(w[i], 5.0 * mean);
  }
  const double inf = std::numeric_limits<double>::infinity();
  double taken = inf, left = -inf;
  bool any_taken = false, any_left = false;
  for (int i = 0; i < n; ++i) {
    if (bits[i] > b_lo) {
      taken = std::min(taken, marginal_key(w[i], alpha[i], beta[i], bits[i] - 1));
      any_taken = true;
    }
    if (bits[i] < b_hi) {
      left = std::max(left, marginal_key(w[i], alpha[i], beta[i], bits[i]));
      any_left = true;
    }
  }
  if (!any_taken || !any_left)
    *margin_out = inf;
  else if (taken == -inf && left == -inf)
    *margin_out = 0.0;  // only heads with nothing to gain (alpha = 0) took and missed bits
  else
    *margin_out = taken - left;
  return KVQ_OK;
}
