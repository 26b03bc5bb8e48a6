"""Pins of the oracle's per-channel key normalization (InnerQ page, technique (iii)): computed
once from the first append, stored keys divided by it, folded back at attention (CPU).

The pins do not restate the oracle's formula. They check what normalization must do:
channel norms of 1 change nothing; scaling a key channel by a power of two (and the query
channel by its inverse) leaves codes and attention bit-identical, where plain quantization
changes; with outlier key channels the reconstruction error falls; the first append alone
sets the norms.
"""
import numpy as np

from oracle import kvq_oracle as O
from workloads import random_raw16, to_raw16


def _cfg(key_norm, k_bits=(3, 2), v_bits=(2, 4), dtype="bf16", quant="hybrid", D=64, cap=400):
    return O.CacheConfig(batch=2, n_kv=2, n_q=4, head_dim=D, capacity=cap, n_sink=2, n_recent=32,
                         dtype=dtype, quant=quant, k_bits=k_bits, v_bits=v_bits, key_norm=key_norm)


def _keys_with_unit_channel_max(rng, shape, dtype):
    """Keys whose every (row, head, channel) has max |k| exactly 1 over the tokens, except
    channel 7, all zero (its norm falls back to 1)."""
    x = rng.uniform(-0.95, 0.95, size=shape).astype(np.float32)
    B, H, T, D = shape
    t = rng.integers(0, T, size=(B, H, D))
    sign = np.where(rng.random((B, H, D)) < 0.5, -1.0, 1.0).astype(np.float32)
    for b in range(B):
        for h in range(H):
            x[b, h, t[b, h], np.arange(D)] = sign[b, h]
    x[..., 7] = 0.0
    return to_raw16(x, dtype)


def _codes(oc):
    return [oc.heads[h]["k_codes"] for h in range(len(oc.heads))]


def test_unit_norms_change_nothing():
    rng = np.random.default_rng(1)
    T = 300
    k = _keys_with_unit_channel_max(rng, (2, 2, T, 64), "bf16")
    v = random_raw16(rng, (2, 2, T, 64), "bf16")
    q = random_raw16(rng, (2, 4, 64), "bf16")
    a = O.build_cache(k, v, _cfg(False))
    b = O.build_cache(k, v, _cfg(True))
    assert np.all(b.k_norm == 1.0)
    for ca, cb in zip(_codes(a), _codes(b)):
        assert np.array_equal(ca, cb)
    assert np.array_equal(O.decode(a, q), O.decode(b, q))


def _scale_channels(raw, e, dtype):
    """Multiply channel c of the last axis by 2^e[c] (exact: no over- or underflow here)."""
    x = O.widen16(raw, dtype).astype(np.float64) * np.exp2(e)
    y = to_raw16(x.astype(np.float32), dtype)
    assert np.array_equal(O.widen16(y, dtype).astype(np.float64), x)
    return y


def test_power_of_two_channel_scaling_is_absorbed():
    # bf16: its exponent range keeps every scaled element exact
    rng = np.random.default_rng(2)
    T, D = 260, 64
    k = random_raw16(rng, (2, 2, T, D), "bf16")
    v = random_raw16(rng, (2, 2, T, D), "bf16")
    q = random_raw16(rng, (2, 4, D), "bf16")
    e = rng.integers(-3, 4, size=D).astype(np.float64)
    k2 = _scale_channels(k, e, "bf16")
    q2 = _scale_channels(q, -e, "bf16")
    cfg = _cfg(True, dtype="bf16")
    a, b = O.build_cache(k, v, cfg), O.build_cache(k2, v, cfg)
    assert np.array_equal(b.k_norm, (a.k_norm * np.exp2(e)).astype(np.float32))
    for ca, cb in zip(_codes(a), _codes(b)):
        assert np.array_equal(ca, cb)
    for h in range(2):
        assert np.array_equal(a.heads[h]["k_s"], b.heads[h]["k_s"])
        assert np.array_equal(a.heads[h]["k_z"], b.heads[h]["k_z"])
    assert np.array_equal(O.decode(a, q), O.decode(b, q2))
    # without normalization the same scaling moves the group ranges, and the codes
    cfg0 = _cfg(False, dtype="bf16")
    a0, b0 = O.build_cache(k, v, cfg0), O.build_cache(k2, v, cfg0)
    assert not all(np.array_equal(ca, cb) for ca, cb in zip(_codes(a0), _codes(b0)))


def test_outlier_channels_reconstruct_better():
    # four key channels per head scaled x8 (the tiny workload's recipe): the normalized
    # cache reconstructs the keys with a lower squared error than the plain one
    rng = np.random.default_rng(3)
    T, D = 512, 64
    x = rng.standard_normal((1, 2, T, D)).astype(np.float32)
    for h in range(2):
        x[0, h, :, rng.choice(D, size=4, replace=False)] *= 8.0
    k = to_raw16(x, "fp16")
    v = random_raw16(rng, (1, 2, T, D), "fp16")
    err = {}
    for kn in (False, True):
        cfg = O.CacheConfig(batch=1, n_kv=2, n_q=2, head_dim=D, capacity=T, n_sink=0, n_recent=0,
                            dtype="fp16", quant="asym", k_bits=(2, 3), v_bits=(2, 2), key_norm=kn)
        oc = O.build_cache(k, v, cfg)
        kx = O.widen16(k, "fp16").astype(np.float64)
        err[kn] = sum(float(np.sum((O.logical_kv(oc, 0, h)[0][:oc.body] - kx[0, h, :oc.body]) ** 2)) for h in range(2))
    assert err[True] < 0.8 * err[False], err


def test_norms_come_from_the_first_append():
    rng = np.random.default_rng(4)
    T0, T = 100, 300
    k = random_raw16(rng, (2, 2, T, 64), "bf16")
    v = random_raw16(rng, (2, 2, T, 64), "bf16")
    # later tokens carry a channel far larger than anything in the first append
    x = O.widen16(k, "bf16")
    x[:, :, T0:, 5] *= 16.0
    k = to_raw16(x, "bf16")
    cfg = _cfg(True, quant="asym")
    a = O.build_cache(k, v, cfg, norm_tokens=T0)
    b = O.build_cache(k, v, cfg)
    # norms: powers of two in [max, 2 max) of |k_c| over the first append
    m = np.abs(O.widen16(k[:, :, :T0], "bf16")).astype(np.float64).max(axis=2)
    assert np.all((a.k_norm >= m) & (a.k_norm < 2 * m))
    assert np.all(np.exp2(np.round(np.log2(a.k_norm))) == a.k_norm)
    assert np.all(b.k_norm[:, :, 5] >= 8.0 * a.k_norm[:, :, 5])
    # normalized keys past the first append exceed 1 in magnitude; the codes still rebuild
    # each key within one quantization step of its (normalized) group range, times the norm
    ns = 2
    for h, bits in enumerate(cfg.k_bits):
        kh, _ = O.logical_kv(a, 0, h)
        kx = O.widen16(k[0, h], "bf16").astype(np.float64)[ns:ns + a.body]
        xn = (kx / a.k_norm[0, h].astype(np.float64)).reshape(a.body, -1, 32)
        step = ((xn.max(axis=2) - xn.min(axis=2)) / (2**bits - 1))[:, :, None]
        bound = (step * np.ones_like(xn)).reshape(a.body, -1) * a.k_norm[0, h] * 1.01 + 1e-6
        assert np.all(np.abs(kh[ns:ns + a.body] - kx) <= bound)
