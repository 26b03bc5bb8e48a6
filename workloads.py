"""Seeded synthetic inputs for decode attention over a mixed-precision quantized KV cache.

This module only draws random numbers and casts them to the 16-bit storage types. It holds
none of the method's arithmetic (no quantizer, packing, allocation, fit or attention), so it
can feed both the CPU oracle and the HIP library without either importing the other.

The five workloads stand in for the evaluation settings of the RateQuant and InnerQ pages
(WikiText-2 / few-shot models are not available): head geometry 32 query / 8 KV heads /
head_dim 128 as in Llama-3-8B and Qwen3-8B, 512 calibration tokens as in RateQuant's
implementation details, and a 128K context as in the NOVA-KV review.

Every array is drawn with ``numpy.random.default_rng(seed)`` (PCG64), in the order listed
for each workload. 16-bit arrays are returned as raw ``uint16`` bit patterns together with
the dtype name ("fp16" or "bf16"), so both sides see identical bits.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make", "to_raw16", "from_raw16", "ModelCalib", "MODEL_CALIB",
           "make_model_calib"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_kv: int
    n_q: int
    head_dim: int
    tokens: int
    dtype: str                 # "fp16" | "bf16"
    n_sink: int
    n_recent: int
    quant: str                 # "asym" | "hybrid"
    n_splits: int              # split-K chunks used when timing/testing decode
    alloc: str                 # "fixed" | "joint" | "separate" | "calibrated"
    k_total: int = 0           # integer bit budget for keys (or joint budget)
    v_total: int = 0           # integer bit budget for values
    b_lo: int = 2
    b_hi: int = 4
    fixed_bits: tuple = ()     # per KV head, used when alloc == "fixed" (K and V alike)
    calib_tokens: int = 0      # calibration slice length (row 0, tokens 0..calib_tokens-1)


WORKLOADS = {
    # 1 row, GQA 2 KV heads x 2 query heads, head_dim 64, 256 tokens, fp16, 4 outlier key
    # channels x8 per KV head; head bit-widths {2,4}; 1 sink + 32 recent tokens.
    "tiny_t256": Workload("tiny_t256", 1, 2, 4, 64, 256, "fp16", 1, 32, "asym", 4,
                          "fixed", fixed_bits=(2, 4)),
    # Llama-3-8B-shaped layer: 8 rows, 32/8 heads, d 128, 8192 tokens, bf16, per-channel
    # log-normal(0, 0.5) key scales; one joint per-KV-head allocation, 2.5 average bits. The
    # description fixes no chunk count; 4 chunks give 256 workgroups, one per CU (measured
    # fastest of 1..16 on MI355X).
    "llama8b_t8k": Workload("llama8b_t8k", 8, 8, 32, 128, 8192, "bf16", 4, 128, "asym", 4,
                            "joint", k_total=20, v_total=20),
    # Qwen3-8B-shaped long context: 4 rows, 32768 tokens, separate K (3.0) / V (2.0)
    # budgets, hybrid symmetric/asymmetric groups, 16 split-K chunks.
    "qwen8b_t32k": Workload("qwen8b_t32k", 4, 8, 32, 128, 32768, "bf16", 4, 128, "hybrid", 16,
                            "separate", k_total=24, v_total=16),
    # Prefill ingest: 16 rows x 4096 tokens x 8 KV heads x d 128 bf16, calibrated on the
    # first 512 tokens of row 0; K and V budgets 20 each in {2,3,4}.
    "prefill_t4k": Workload("prefill_t4k", 16, 8, 32, 128, 4096, "bf16", 4, 128, "asym", 16,
                            "calibrated", k_total=20, v_total=20, calib_tokens=512),
    # Multi-head (no GQA) 7B-shaped layer for multi-token decode: 4 rows, 32 query = 32 KV
    # heads, d 128, 8192 tokens, bf16, per-channel log-normal(0, 0.5) key scales, heads
    # alternating 3 and 2 bits (K and V alike), 4 split-K chunks; up to 4 query tokens per
    # row fill the rows a single query leaves empty.
    "mha7b_t8k": Workload("mha7b_t8k", 4, 32, 32, 128, 8192, "bf16", 4, 128, "hybrid", 4,
                          "fixed", fixed_bits=(3, 2) * 16),
    # Extreme context: 1 row, 131072 tokens, all heads at 2 bits, fp16, 1% of (head, key
    # channel) pairs scaled x10, 64 split-K chunks.
    "long_t128k": Workload("long_t128k", 1, 8, 32, 128, 131072, "fp16", 4, 128, "asym", 64,
                           "fixed", fixed_bits=(2,) * 8),
}


def to_raw16(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32/float64 values to the 16-bit storage type (nearest-even); return bits."""
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x32.view(np.uint32).astype(np.uint64)
        # nearest-even on the upper 16 bits (inputs here are finite)
        bias = ((u >> 16) & 1) + 0x7FFF
        return ((u + bias) >> 16).astype(np.uint16)
    raise ValueError(dtype)


def from_raw16(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of 16-bit bit patterns to float32."""
    raw = np.asarray(raw, dtype=np.uint16)
    if dtype == "fp16":
        return raw.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (raw.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def make(name: str, seed: int = 0, tokens: int | None = None, batch: int | None = None) -> dict:
    """Draw the inputs of a workload.

    ``tokens`` / ``batch`` shrink the draw for quick tests (same recipe, smaller arrays).
    Returns a dict with the Workload ``spec`` and:
      k, v      uint16 [B][Hkv][T][D]   16-bit keys / values (bits)
      q         uint16 [B][Hq][D]       decode queries (bits)
      q_multi   uint16 [B][4][Hq][D]    (mha7b_t8k) queries of the last 4 tokens
      alpha, beta, w (joint) or alpha_k/beta_k/w_k/alpha_v/beta_v/w_v (separate),
      w_k / w_v (calibrated)            float64 [Hkv]
    """
    s = WORKLOADS[name]
    B = s.batch if batch is None else batch
    T = s.tokens if tokens is None else tokens
    H, Hq, D = s.n_kv, s.n_q, s.head_dim
    rng = np.random.default_rng(seed)
    out = {"spec": s, "batch": B, "tokens": T}
    if name == "tiny_t256":
        outl = np.stack([rng.choice(D, size=4, replace=False) for _ in range(H)])
        k = _normal(rng, (B, H, T, D))
        for h in range(H):
            k[:, h, :, outl[h]] *= 8.0
        v = _normal(rng, (B, H, T, D))
        q = _normal(rng, (B, Hq, D))
        out["outliers"] = outl
    elif name == "long_t128k":
        n_pairs = int(round(0.01 * H * D))
        flat = rng.choice(H * D, size=n_pairs, replace=False)
        k = _normal(rng, (B, H, T, D))
        for f in flat:
            k[:, f // D, :, f % D] *= 10.0
        v = _normal(rng, (B, H, T, D))
        q = _normal(rng, (B, Hq, D))
        out["outliers"] = np.stack([flat // D, flat % D], axis=1)
    else:
        sigma = rng.lognormal(mean=0.0, sigma=0.5, size=(H, D)).astype(np.float32)
        k = _normal(rng, (B, H, T, D))
        k *= sigma[None, :, None, :]
        v = _normal(rng, (B, H, T, D))
        q = _normal(rng, (B, Hq, D))
        out["sigma"] = sigma
        if s.alloc == "joint":
            out["alpha"] = rng.uniform(0.5, 2.0, size=H)
            out["beta"] = rng.uniform(3.6, 5.3, size=H)
            out["w"] = rng.lognormal(0.0, 1.0, size=H)
        elif s.alloc == "separate":
            for c in ("k", "v"):
                out["alpha_" + c] = rng.uniform(0.5, 2.0, size=H)
                out["beta_" + c] = rng.uniform(3.6, 5.3, size=H)
                out["w_" + c] = rng.lognormal(0.0, 1.0, size=H)
        elif s.alloc == "calibrated":
            out["w_k"] = rng.lognormal(0.0, 1.0, size=H)
            out["w_v"] = rng.lognormal(0.0, 1.0, size=H)
    if name == "mha7b_t8k":  # queries of the last 4 tokens of every row (multi-token decode)
        out["q_multi"] = to_raw16(_normal(rng, (B, 4, Hq, D)), s.dtype)
    out["k"] = to_raw16(k, s.dtype)
    del k
    out["v"] = to_raw16(v, s.dtype)
    del v
    out["q"] = to_raw16(q, s.dtype)
    return out


@dataclasses.dataclass(frozen=True)
class ModelCalib:
    """Whole-model calibration set: every (layer, KV head) pair of a model, each with the
    keys and values of `seqs` sequences of `seq_len` tokens, concatenated along tokens."""
    name: str
    layers: int
    kv_heads: int
    seqs: int
    seq_len: int
    head_dim: int
    dtype: str
    quant: str
    k_avg_bits: float          # per-pair budgets: total = avg * layers * kv_heads
    v_avg_bits: float
    b_lo: int = 2
    b_hi: int = 4

    @property
    def pairs(self) -> int:
        return self.layers * self.kv_heads

    @property
    def tokens(self) -> int:
        return self.seqs * self.seq_len


# Qwen3-8B-shaped: 36 layers x 8 KV heads = 288 pairs, 16 sequences x 512 tokens, head_dim
# 128, bf16, asymmetric quantizer, K budget 3.0 and V budget 2.5 average bits in {2, 3, 4}.
MODEL_CALIB = ModelCalib("qwen8b_model_calib", 36, 8, 16, 512, 128, "bf16", "asym", 3.0, 2.5)


def make_model_calib(spec: ModelCalib = MODEL_CALIB, seed: int = 0, pairs=None, seq_len: int | None = None) -> dict:
    """Draw a whole-model calibration set. Per pair p (layer-major), from a generator seeded
    with (seed, p): keys N(0, 1) times channel scales log-normal(0, spread_p) times a pair
    scale a_p, values N(0, 1) times a pair scale c_p. The pair parameters spread_p ~ U(0.2, 1),
    a_p, c_p ~ log-normal(0, 0.3) and the weights w_k, w_v ~ log-normal(0, 1) come from a
    generator seeded with seed, so any subset of pairs can be drawn alone (`pairs`), with
    identical bits. `seq_len` shrinks every sequence for quick tests.
    Returns dict: spec, k, v uint16 [n][seqs*seq_len][D] (bits), w_k, w_v float64 [pairs],
    k_total, v_total (integer budgets), pairs (the drawn pair indices)."""
    P, D = spec.pairs, spec.head_dim
    T = spec.seqs * (spec.seq_len if seq_len is None else seq_len)
    top = np.random.default_rng(seed)
    spread = top.uniform(0.2, 1.0, size=P)
    a = top.lognormal(0.0, 0.3, size=P)
    c = top.lognormal(0.0, 0.3, size=P)
    w_k = top.lognormal(0.0, 1.0, size=P)
    w_v = top.lognormal(0.0, 1.0, size=P)
    idx = list(range(P)) if pairs is None else list(pairs)
    k = np.empty((len(idx), T, D), dtype=np.uint16)
    v = np.empty((len(idx), T, D), dtype=np.uint16)
    for i, p in enumerate(idx):
        r = np.random.default_rng((seed, p))
        sig = np.exp(spread[p] * _normal(r, (D,))).astype(np.float32) * np.float32(a[p])
        k[i] = to_raw16(_normal(r, (T, D)) * sig[None, :], spec.dtype)
        v[i] = to_raw16(_normal(r, (T, D)) * np.float32(c[p]), spec.dtype)
    return {"spec": spec, "k": k, "v": v, "w_k": w_k, "w_v": w_v, "pairs": idx,
            "k_total": int(round(spec.k_avg_bits * P)), "v_total": int(round(spec.v_avg_bits * P))}


def random_raw16(rng: np.random.Generator, shape, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) draw in a 16-bit type (used by small property tests)."""
    return to_raw16(_normal(rng, shape) * np.float32(scale), dtype)
