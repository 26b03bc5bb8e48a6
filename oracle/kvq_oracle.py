"""CPU oracle for decode attention over a mixed-precision, group-quantized KV cache.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke entry point and the benchmark's
CPU-baseline leg may import this module. The library (HIP kernels + C ABI) never calls it,
and this module imports nothing from the library: the two share no code. Inputs come from
the seeded generators, which hold none of the method's arithmetic.

What it computes, and where the pages define it
-----------------------------------------------
* Group-wise quantization along the inner dimension of each vector-matrix product: keys
  in groups of 32 consecutive head_dim channels of one token, values in groups of 32
  consecutive tokens of one channel (InnerQ page, abstract and "Core claim": grouping along
  the inner dimension aligns dequantization with the vector-matrix product).
* Hybrid quantization: per group, symmetric or asymmetric, chosen from the group's own
  statistics (InnerQ page, abstract, technique (i)). Reading taken: the variant with the
  lower squared error wins, ties go to asymmetric.
* 16-bit high-precision windows for attention-sink tokens and recent tokens (InnerQ page,
  abstract, technique (ii)).
* Optional per-channel key normalization computed once at prefill and folded into the
  query (InnerQ page, abstract, technique (iii), and "Core claim"). The pages give no
  formula for n_c. Reading taken: n_c is the smallest power of two >= max |k_c| over the
  tokens of the first append (1 if that max is 0). That brings every prefill channel into
  [-1, 1], as dividing by the max would, to within a factor of 2. It also makes both k_c / n_c
  and the query fold q_c * n_c exact in any binary format, so folding into the query costs
  no precision. Quantized key groups hold k_c / n_c (IEEE float32 division), and their
  attention uses n_c * (s c + z). 16-bit keys are used as they are.
* Distortion model D(b) = alpha * beta^-b fitted per head by least squares in the log
  domain, with a beta fallback for poor fits (RateQuant page, TL;DR and sections 3.1,
  3.4, W.10).
* Bit allocation: continuous reverse waterfilling and its integer greedy form (RateQuant
  page, sections 3.1, 3.3, B.1, B.3, U, W.7), optional sensitivity cap (section W.14).
* Multi-token decode: the queries of the last Q tokens, each attending causally to its own
  prefix (decode_multi; the same attention per query token).
* Attention for the decode query, in float64, over the dequantized cache (InnerQ page,
  "Algorithm 1: multi-head attention with quantized cache in the decode phase", structure
  only: the page's listing is cut off and its projections are outside this path).

Precision: the quantizer works in IEEE float32 with float16 scale and zero (the stored
precision); every squared-error sum and the attention are float64. Where a floating-point
value decides an integer (a code, a hybrid flag, a bit allocation), the arithmetic and its
order are written out so the device can reproduce it exactly.

The oracle holds only the logical content of a cache: codes, float16 scales and zeros,
hybrid flags, 16-bit rows and key norms. How the library lays those out in device memory is
its own storage format, which no page defines; the tests read device blobs through a
separate format module and compare the logical content with this module's.

parity unpinned (against the pages): the exact definition of the symmetric variant is a
reading of its own (the pages name the variant but give no formula or worked example). It
is pinned here only by internal invariants (brute-force nearest level, exact zero level,
hybrid error never above either variant's).
"""
from __future__ import annotations

import dataclasses
import itertools
import math

import numpy as np

GROUP = 32
RANGE_LIMIT = 16384.0  # |x| <= 2^14 for quantized heads (keeps s, z, x_hat finite in fp16)

# ----------------------------------------------------------------------------------------
# 16-bit widening and float16 rounding
# ----------------------------------------------------------------------------------------


def widen16(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 value of 16-bit fp16 / bf16 bit patterns."""
    raw = np.ascontiguousarray(raw, dtype=np.uint16)
    if dtype == "fp16":
        return raw.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (raw.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(f"unknown dtype {dtype}")


def f16(x) -> np.ndarray:
    """IEEE round-to-nearest-even float32 -> float16 (numpy's cast is RNE)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16)


# ----------------------------------------------------------------------------------------
# Group quantizers (InnerQ page: group-wise quantization, hybrid sym/asym technique (i))
# ----------------------------------------------------------------------------------------


def quant_asym(x: np.ndarray, b: int):
    """Asymmetric min/max quantizer of the last axis (length 32), b bits.

    s = f16(fl32(max - min) / fl32(2^b - 1)), z = f16(min + 0) (a zero minimum is stored
    as +0 whatever its sign); codes are the nearest level of
    (x - z) / s computed as fl32(fl32(x - z) * fl32(1 / s)), ties to even, clamped to
    [0, 2^b - 1]; s == 0 gives all-zero codes.  Dequantization: x_hat = c * s + z.
    Returns (codes uint8 [..., 32], s float16 [...], z float16 [...]).
    """
    x = np.asarray(x, dtype=np.float32)
    L = np.float32(2 ** b - 1)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    s = f16((mx - mn) / L)
    z = f16(mn + np.float32(0.0))   # + 0 stores a zero minimum as +0 whatever its sign
    s32 = s.astype(np.float32)
    z32 = z.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.float32(1.0) / s32
        t = (x - z32[..., None]) * r[..., None]
    c = np.clip(np.rint(t), 0, L)
    c = np.where((s32 == 0)[..., None], 0, c)
    return c.astype(np.uint8), s, z


def quant_sym(x: np.ndarray, b: int):
    """Symmetric quantizer with a zero level, stored as an offset unsigned code.

    Q = 2^(b-1) - 1, s = f16(fl32(max|x|) / fl32(Q)), q = clamp(rint(fl32(x * fl32(1/s))),
    -Q, Q), stored u = q + 2^(b-1) in [1, 2^b - 1], z = -2^(b-1) * s (exact in fp16), so
    dequantization has the same affine form u * s + z = q * s.  s == 0 gives q = 0.
    """
    x = np.asarray(x, dtype=np.float32)
    Q = np.float32(2 ** (b - 1) - 1)
    half = 2 ** (b - 1)
    m = np.abs(x).max(axis=-1)
    s = f16(m / Q)
    s32 = s.astype(np.float32)
    z = f16(np.float32(-half) * s32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.float32(1.0) / s32
        qv = np.clip(np.rint(x * r[..., None]), -Q, Q)
    qv = np.where((s32 == 0)[..., None], 0, qv)
    return (qv + half).astype(np.uint8), s, z


def dequant(codes: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """x_hat = c * s + z in float64 (exact for fp16 s, z and codes < 256)."""
    return codes.astype(np.float64) * s.astype(np.float64)[..., None] + z.astype(np.float64)[..., None]


def group_sse(x: np.ndarray, xhat: np.ndarray) -> np.ndarray:
    """Sum over the 32 group elements of (x - x_hat)^2 in float64, strictly in element
    order 0..31: each square rounded, then added (no fused multiply-add)."""
    d = np.asarray(x, dtype=np.float64) - xhat
    acc = np.zeros(d.shape[:-1], dtype=np.float64)
    for i in range(d.shape[-1]):
        sq = d[..., i] * d[..., i]
        acc = acc + sq
    return acc


def quant_group(x: np.ndarray, b: int, hybrid: bool):
    """Quantize groups (last axis = 32). Hybrid picks symmetric iff its SSE is strictly
    lower than the asymmetric one (InnerQ technique (i)); flag 1 marks symmetric."""
    ca, sa, za = quant_asym(x, b)
    if not hybrid:
        return ca, sa, za, np.zeros(ca.shape[:-1], dtype=np.uint8)
    cs, ss, zs = quant_sym(x, b)
    ea = group_sse(x, dequant(ca, sa, za))
    es = group_sse(x, dequant(cs, ss, zs))
    use_sym = es < ea
    c = np.where(use_sym[..., None], cs, ca)
    s = np.where(use_sym, ss, sa)
    z = np.where(use_sym, zs, za)
    return c, s, z, use_sym.astype(np.uint8)


# ----------------------------------------------------------------------------------------
# Bit packing: 32 codes of b bits -> b little-endian uint32 words
# ----------------------------------------------------------------------------------------


def pack(codes: np.ndarray, b: int) -> np.ndarray:
    """Code i occupies stream bits [i*b, i*b + b); stream bit k is bit (k mod 32) of word
    k // 32.  codes [..., 32] -> uint32 [..., b]."""
    codes = np.asarray(codes, dtype=np.uint64)
    lead = codes.shape[:-1]
    words = np.zeros(lead + (b,), dtype=np.uint64)
    for i in range(GROUP):
        for j in range(b):
            k = i * b + j
            bit = (codes[..., i] >> np.uint64(j)) & np.uint64(1)
            words[..., k // 32] |= bit << np.uint64(k % 32)
    return words.astype(np.uint32)


def unpack(words: np.ndarray, b: int) -> np.ndarray:
    """Inverse of pack: uint32 [..., b] -> codes uint8 [..., 32]."""
    words = np.asarray(words, dtype=np.uint64)
    lead = words.shape[:-1]
    codes = np.zeros(lead + (GROUP,), dtype=np.uint64)
    for i in range(GROUP):
        for j in range(b):
            k = i * b + j
            bit = (words[..., k // 32] >> np.uint64(k % 32)) & np.uint64(1)
            codes[..., i] |= bit << np.uint64(j)
    return codes.astype(np.uint8)


# ----------------------------------------------------------------------------------------
# Windows (InnerQ technique (ii)): sink tokens, a recent ring, 32-token body blocks
# ----------------------------------------------------------------------------------------


def body_len(T: int, n_sink: int, n_recent: int) -> int:
    """Quantized token count after T tokens: whole 32-token blocks that have left the
    recent window, so the window keeps between n_recent and n_recent + 31 tokens."""
    return GROUP * max(0, (T - n_sink - n_recent) // GROUP)


@dataclasses.dataclass
class CacheConfig:
    batch: int
    n_kv: int
    n_q: int
    head_dim: int
    capacity: int
    n_sink: int
    n_recent: int
    dtype: str
    quant: str                  # "asym" | "hybrid"
    k_bits: tuple
    v_bits: tuple
    key_norm: bool = False      # per-channel key normalization (InnerQ technique (iii))

    @property
    def groups(self) -> int:
        return self.head_dim // GROUP


@dataclasses.dataclass
class OracleCache:
    """Logical content of the cache after T tokens, per (row, KV head)."""
    cfg: CacheConfig
    T: int
    body: int
    sink_k: np.ndarray      # uint16 [B][H][min(T, n_s)][D]
    sink_v: np.ndarray
    win_k: np.ndarray       # uint16 [B][H][T - n_s - body][D], tokens n_s+body .. T-1
    win_v: np.ndarray
    # per head h: dict with quantized body (or raw 16-bit body for 16-bit heads)
    heads: list
    # per-channel key norms float32 [B][H][D] (key normalization only, else None)
    k_norm: np.ndarray | None = None


def _check_range(x: np.ndarray):
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > RANGE_LIMIT):
        raise ValueError("quantized inputs must be finite with |x| <= 2^14")


def key_norms(k_raw: np.ndarray, dtype: str) -> np.ndarray:
    """Per-channel key norms float32 [B][H][D]: the smallest power of two >= the max over
    the given tokens (those of the first append) of |k_c|; 1 where that max is 0 (InnerQ
    page, technique (iii); the power of two is this implementation's reading)."""
    m = np.abs(widen16(k_raw, dtype)).max(axis=2) if k_raw.shape[2] else np.zeros(
        (k_raw.shape[0], k_raw.shape[1], k_raw.shape[3]), dtype=np.float32)
    f, e = np.frexp(m.astype(np.float64))            # m = f * 2^e, 0.5 <= f < 1
    n = np.where(f == 0.5, m.astype(np.float64), np.ldexp(1.0, e))
    return np.where(m > 0, n, 1.0).astype(np.float32)


def build_cache(k_raw: np.ndarray, v_raw: np.ndarray, cfg: CacheConfig, norm_tokens: int | None = None) -> OracleCache:
    """State of the cache after appending tokens 0..T-1 (k_raw, v_raw [B][H][T][D] bits).

    Body keys: group (token t, channels 32g..32g+31); body values: group (channel c,
    tokens 32j..32j+31).  Heads with 16 bits keep the body unquantized. With key
    normalization, norm_tokens is the token count of the first append (default: all T)."""
    B, H, T, D = k_raw.shape
    assert v_raw.shape == k_raw.shape and H == cfg.n_kv and D == cfg.head_dim
    ns = min(T, cfg.n_sink)
    body = body_len(T, cfg.n_sink, cfg.n_recent)
    hyb = cfg.quant == "hybrid"
    kn = key_norms(k_raw[:, :, :T if norm_tokens is None else norm_tokens], cfg.dtype) if cfg.key_norm else None
    heads = []
    for h in range(H):
        e = {}
        kb, vb = cfg.k_bits[h], cfg.v_bits[h]
        kbody = k_raw[:, h, ns:ns + body, :]
        vbody = v_raw[:, h, ns:ns + body, :]
        if kb == 16:
            e["k_raw"] = kbody.copy()
        else:
            x = widen16(kbody, cfg.dtype)
            if kn is not None:
                x = (x / kn[:, h, None, :]).astype(np.float32)   # IEEE float32 division
            _check_range(x)
            xg = x.reshape(B, body, cfg.groups, GROUP)
            c, s, z, f = quant_group(xg, kb, hyb)
            e["k_codes"], e["k_s"], e["k_z"], e["k_flag"] = c, s, z, f
        if vb == 16:
            e["v_raw"] = vbody.copy()
        else:
            x = widen16(vbody, cfg.dtype)
            _check_range(x)
            # [B][body][D] -> [B][body/32][D][32]
            xg = x.reshape(B, body // GROUP, GROUP, D).transpose(0, 1, 3, 2)
            c, s, z, f = quant_group(xg, vb, hyb)
            e["v_codes"], e["v_s"], e["v_z"], e["v_flag"] = c, s, z, f
        heads.append(e)
    return OracleCache(cfg=cfg, T=T, body=body,
                       sink_k=k_raw[:, :, :ns].copy(), sink_v=v_raw[:, :, :ns].copy(),
                       win_k=k_raw[:, :, ns + body:].copy(), win_v=v_raw[:, :, ns + body:].copy(),
                       heads=heads, k_norm=kn)


def logical_kv(oc: OracleCache, b: int, h: int):
    """K_tilde, V_tilde float64 [T][D] for row b, KV head h: exact 16-bit values for sink,
    window and 16-bit heads, x_hat = c*s + z for quantized body tokens."""
    cfg = oc.cfg
    D = cfg.head_dim
    e = oc.heads[h]
    parts_k = [widen16(oc.sink_k[b, h], cfg.dtype).astype(np.float64)]
    parts_v = [widen16(oc.sink_v[b, h], cfg.dtype).astype(np.float64)]
    if "k_raw" in e:
        parts_k.append(widen16(e["k_raw"][b], cfg.dtype).astype(np.float64))
    else:
        kh = dequant(e["k_codes"][b], e["k_s"][b], e["k_z"][b]).reshape(oc.body, D)
        if oc.k_norm is not None:
            kh = kh * oc.k_norm[b, h].astype(np.float64)[None, :]   # the normalization undone
        parts_k.append(kh)
    if "v_raw" in e:
        parts_v.append(widen16(e["v_raw"][b], cfg.dtype).astype(np.float64))
    else:
        xv = dequant(e["v_codes"][b], e["v_s"][b], e["v_z"][b])     # [nblk][D][32]
        parts_v.append(xv.transpose(0, 2, 1).reshape(oc.body, D))
    parts_k.append(widen16(oc.win_k[b, h], cfg.dtype).astype(np.float64))
    parts_v.append(widen16(oc.win_v[b, h], cfg.dtype).astype(np.float64))
    return np.concatenate(parts_k, axis=0), np.concatenate(parts_v, axis=0)


# ----------------------------------------------------------------------------------------
# Decode attention in float64 (InnerQ, Algorithm 1 structure: per head q.K^T, softmax, P.V)
# ----------------------------------------------------------------------------------------


def attention_head(q: np.ndarray, Kt: np.ndarray, Vt: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of query rows q [G][D] over K_tilde, V_tilde [T][D], float64."""
    s = (q.astype(np.float64) @ Kt.T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ Vt) / p.sum(axis=1, keepdims=True)


def decode(oc: OracleCache, q_raw: np.ndarray, scale: float | None = None, rows=None, heads=None):
    """Decode output float64 [B][Hq][D] (or only the listed rows / KV heads; others NaN).

    Query head i reads KV head i // G, G = Hq / Hkv; scale defaults to 1/sqrt(D)."""
    cfg = oc.cfg
    B, Hq, D = q_raw.shape
    G = Hq // cfg.n_kv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    q = widen16(q_raw, cfg.dtype).astype(np.float64)
    out = np.full((B, Hq, D), np.nan)
    for b in (range(B) if rows is None else rows):
        for h in (range(cfg.n_kv) if heads is None else heads):
            Kt, Vt = logical_kv(oc, b, h)
            out[b, h * G:(h + 1) * G] = attention_head(q[b, h * G:(h + 1) * G], Kt, Vt, scale)
    return out


def decode_multi(oc: OracleCache, q_raw: np.ndarray, scale: float | None = None):
    """Decode output float64 [B][Q][Hq][D] for the queries q_raw [B][Q][Hq][D] of the last Q
    cached tokens: query token i is the (T - Q + i)-th token and attends to tokens
    0 .. T - Q + i only (causal decoding of several tokens at once, as in speculative
    decoding; the InnerQ Algorithm 1 structure per query token)."""
    cfg = oc.cfg
    B, Q, Hq, D = q_raw.shape
    G = Hq // cfg.n_kv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    q = widen16(q_raw, cfg.dtype).astype(np.float64)
    out = np.full((B, Q, Hq, D), np.nan)
    for b in range(B):
        for h in range(cfg.n_kv):
            Kt, Vt = logical_kv(oc, b, h)
            for i in range(Q):
                n = oc.T - Q + i + 1
                out[b, i, h * G:(h + 1) * G] = attention_head(q[b, i, h * G:(h + 1) * G], Kt[:n], Vt[:n], scale)
    return out


def partial_softmax(q: np.ndarray, Kt: np.ndarray, Vt: np.ndarray, scale: float):
    """Un-normalized partial over a token chunk: (m, l, o) with o = sum_t e^(s_t - m) v_t."""
    s = (q @ Kt.T) * scale
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return m, p.sum(axis=1), p @ Vt


def lse_merge(ms, ls, os_):
    """Combine chunk partials: m* = max m_j, l* = sum e^(m_j - m*) l_j,
    out = sum e^(m_j - m*) o_j / l*."""
    ms = np.asarray(ms)
    mstar = ms.max(axis=0)
    wts = np.exp(ms - mstar[None])
    lstar = (wts * np.asarray(ls)).sum(axis=0)
    o = (wts[..., None] * np.asarray(os_)).sum(axis=0)
    return o / lstar[..., None]


# ----------------------------------------------------------------------------------------
# Calibration and distortion fit (RateQuant page: D(b) = alpha*beta^-b, sections 3.1, 3.4,
# W.10; calibration on a small token set, section 4.1 / P)
# ----------------------------------------------------------------------------------------


def calib_group_sse(x_raw: np.ndarray, dtype: str, axis: int, b: int, hybrid: bool) -> np.ndarray:
    """Per-group SSE float64 for one head's calibration slice x [n_tokens][D].

    axis 0 (keys): groups of 32 channels of one token, ordered (token, group).
    axis 1 (values): groups of 32 tokens of one channel, ordered (token block, channel)."""
    x = widen16(x_raw, dtype)
    _check_range(x)
    n, D = x.shape
    if axis == 0:
        xg = x.reshape(n, D // GROUP, GROUP).reshape(-1, GROUP)
    else:
        xg = x.reshape(n // GROUP, GROUP, D).transpose(0, 2, 1).reshape(-1, GROUP)
    c, s, z, _ = quant_group(xg, b, hybrid)
    return group_sse(xg, dequant(c, s, z))


def calib_distortion(x_raw, dtype, axis, b_lo, b_hi, hybrid) -> np.ndarray:
    """Mean squared quantization error D(b), b = b_lo..b_hi, for one head: the per-group
    SSEs are added in group order (sequentially, float64), then divided by the element
    count."""
    n_el = x_raw.shape[0] * x_raw.shape[1]
    out = []
    for b in range(b_lo, b_hi + 1):
        sse = calib_group_sse(x_raw, dtype, axis, b, hybrid)
        tot = 0.0
        for v in sse.tolist():
            tot = tot + v
        out.append(tot / n_el)
    return np.array(out)


R2_FALLBACK = 0.96


def fit_one(bs, Ds):
    """Least squares of y = ln D(b) on x = b: returns (alpha, beta, R^2, degenerate).

    slope = sum (x - xbar)(y - ybar) / Sxx, intercept = ybar - slope * xbar,
    alpha = e^intercept, beta = e^-slope, R^2 = 1 - SS_res / SS_tot (1 when SS_tot = 0).
    Any D(b) <= 0 (an exactly representable head) is degenerate: alpha = 0, beta = 4, R^2 = 1.
    Sums run in increasing b; logs and exps are the C library's (math module)."""
    if any((not (d > 0.0)) or math.isinf(d) for d in Ds):
        return 0.0, 4.0, 1.0, True
    n = len(bs)
    xs = [float(b) for b in bs]
    ys = [math.log(d) for d in Ds]
    xbar = 0.0
    ybar = 0.0
    for x, y in zip(xs, ys):
        xbar += x
        ybar += y
    xbar /= n
    ybar /= n
    sxy = 0.0
    sxx = 0.0
    for x, y in zip(xs, ys):
        sxy += (x - xbar) * (y - ybar)
        sxx += (x - xbar) * (x - xbar)
    slope = sxy / sxx
    icpt = ybar - slope * xbar
    ss_res = 0.0
    ss_tot = 0.0
    for x, y in zip(xs, ys):
        r = y - (icpt + slope * x)
        ss_res += r * r
        ss_tot += (y - ybar) * (y - ybar)
    r2 = 1.0 if ss_tot == 0.0 else 1.0 - ss_res / ss_tot
    return math.exp(icpt), math.exp(-slope), r2, False


def fit_heads(bs, D_heads):
    """Fit every head, then the fallback for poor fits (RateQuant W.10): a head with
    R^2 < 0.96 gets beta = min(beta_fit, beta_bar), beta_bar the mean beta of this call's
    well-fitted heads (all non-degenerate heads if none fits well).  A fitted beta <= 1 (D
    not decreasing) counts as a poor fit and takes beta_bar itself, since min() would keep
    an invalid model; alpha is unchanged."""
    fits = [fit_one(bs, d) for d in D_heads]
    good = [f[1] for f in fits if not f[3] and f[2] >= R2_FALLBACK and f[1] > 1.0]
    pool = good if good else [f[1] for f in fits if not f[3] and f[1] > 1.0]
    bbar = 0.0
    for v in pool:
        bbar += v
    bbar = bbar / len(pool) if pool else 4.0
    alpha, beta, r2 = [], [], []
    for a, bt, r, deg in fits:
        if not deg:
            if bt <= 1.0:
                bt = bbar
            elif r < R2_FALLBACK:
                bt = min(bt, bbar)
        alpha.append(a)
        beta.append(bt)
        r2.append(r)
    return np.array(alpha), np.array(beta), np.array(r2)


# ----------------------------------------------------------------------------------------
# Bit allocation (RateQuant page: reverse waterfilling 3.1 / B.1; greedy 3.3 / B.3 / U / W.7)
# ----------------------------------------------------------------------------------------


def cap_weights(w):
    """Sensitivity cap w_i <- min(w_i, 5 * mean(w)) (RateQuant W.14)."""
    w = [float(x) for x in w]
    mean = 0.0
    for x in w:
        mean += x
    mean /= len(w)
    return [min(x, 5.0 * mean) for x in w]


def check_alloc_args(alpha, beta, w, total, b_lo, b_hi):
    n = len(alpha)
    if not (n >= 1 and len(beta) == n and len(w) == n):
        raise ValueError("length mismatch")
    if not (2 <= b_lo <= b_hi <= 8):
        raise ValueError("bounds")
    for a, bt, x in zip(alpha, beta, w):
        if not (math.isfinite(a) and a >= 0 and math.isfinite(bt) and bt > 1 and math.isfinite(x) and x > 0):
            raise ValueError("model parameters")
    if not (n * b_lo <= total <= n * b_hi):
        raise ValueError("budget")


def marginal_key(w, a, bt, b):
    """ln of the gain of the (b+1)-th bit, w * a * beta^-b * (1 - 1/beta), evaluated as
    ((ln w + ln a) + ln(1 - 1/beta)) - b * ln beta (C library log; ln 0 = -inf)."""
    la = math.log(a) if a > 0 else -math.inf
    return ((math.log(w) + la) + math.log(1.0 - 1.0 / bt)) - b * math.log(bt)


def allocate_greedy(alpha, beta, w, total, b_lo, b_hi, cap=False):
    """Greedy integer allocation: every head starts at b_lo; total - n*b_lo times, the head
    (below b_hi) with the largest marginal gain gets one more bit, ties to the lowest index.
    Plain linear scan over heads (the library uses a max-heap)."""
    check_alloc_args(alpha, beta, w, total, b_lo, b_hi)
    if cap:
        w = cap_weights(w)
    n = len(alpha)
    bits = [b_lo] * n
    for _ in range(total - n * b_lo):
        best, bkey = -1, None
        for i in range(n):
            if bits[i] >= b_hi:
                continue
            kk = marginal_key(w[i], alpha[i], beta[i], bits[i])
            if best < 0 or kk > bkey:
                best, bkey = i, kk
        bits[best] += 1
    return bits


def allocation_margin(alpha, beta, w, bits, b_lo, b_hi, cap=False):
    """Decision margin of an integer allocation (ln units): the smallest marginal key that
    received a bit minus the largest key left without one (keys as in allocate_greedy). The
    greedy hands out bits in key order, so its allocation has margin >= 0; a margin near 0
    means inputs perturbed by a tiny relative error may allocate differently. +inf when no bit
    was handed out or every head is at b_hi; 0 when only alpha = 0 heads took and missed bits."""
    check_alloc_args(alpha, beta, w, sum(bits), b_lo, b_hi)
    if cap:
        w = cap_weights(w)
    taken = [marginal_key(w[i], alpha[i], beta[i], bits[i] - 1) for i in range(len(bits)) if bits[i] > b_lo]
    left = [marginal_key(w[i], alpha[i], beta[i], bits[i]) for i in range(len(bits)) if bits[i] < b_hi]
    if not taken or not left:
        return math.inf
    lo, hi = min(taken), max(left)
    if lo == -math.inf and hi == -math.inf:
        return 0.0
    return lo - hi


def objective(alpha, beta, w, bits):
    return sum(wi * ai * bi ** (-b) for ai, bi, wi, b in zip(alpha, beta, w, bits))


def allocate_bruteforce(alpha, beta, w, total, b_lo, b_hi):
    """Every integer vector in [b_lo, b_hi]^n with sum = total; returns (best objective,
    list of all vectors within 1e-12 relative of it)."""
    n = len(alpha)
    best = math.inf
    vecs = []
    for v in itertools.product(range(b_lo, b_hi + 1), repeat=n):
        if sum(v) != total:
            continue
        o = objective(alpha, beta, w, v)
        vecs.append((o, v))
        best = min(best, o)
    near = [v for o, v in vecs if o <= best * (1 + 1e-12)]
    return best, near


def allocate_continuous(alpha, beta, w, total, b_lo, b_hi, cap=False, tol=1e-13):
    """Reverse waterfilling on D_i(b) = w_i a_i beta_i^-b with b_lo <= b_i <= b_hi:
    b_i(theta) = clip((ln(w_i a_i ln beta_i) - theta) / ln beta_i, b_lo, b_hi), with the
    water level theta set so that sum b_i = total.  sum b_i(theta) is non-increasing in
    theta; theta is found by bisection."""
    check_alloc_args(alpha, beta, w, total, b_lo, b_hi)
    if cap:
        w = cap_weights(w)
    n = len(alpha)
    lb = [math.log(b) for b in beta]
    c = [math.log(wi * ai * li) if ai > 0 else -math.inf for wi, ai, li in zip(w, alpha, lb)]

    def bits_at(theta):
        return [b_lo if ci == -math.inf else min(b_hi, max(b_lo, (ci - theta) / li))
                for ci, li in zip(c, lb)]

    # Heads with alpha = 0 have no distortion to remove; like the greedy form they take bits
    # only once every other head is at b_hi, the remainder shared evenly among them.
    n_deg = sum(1 for ci in c if ci == -math.inf)
    full = sum(b_hi for ci in c if ci != -math.inf) + n_deg * b_lo
    if total >= full:
        extra = (total - full) / n_deg if n_deg else 0.0
        return [float(b_hi) if ci != -math.inf else b_lo + extra for ci in c]
    if total == n * b_lo:
        return [float(b_lo)] * n
    lo = min(ci - b_hi * li for ci, li in zip(c, lb) if ci != -math.inf) - 1.0
    hi = max(ci - b_lo * li for ci, li in zip(c, lb) if ci != -math.inf) + 1.0
    for _ in range(400):
        mid = 0.5 * (lo + hi)
        if sum(bits_at(mid)) > total:
            lo = mid
        else:
            hi = mid
        if hi - lo < tol:
            break
    return bits_at(0.5 * (lo + hi))
