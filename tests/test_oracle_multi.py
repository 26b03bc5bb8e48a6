"""Pins of the oracle's multi-token (causal) decode (CPU): one query token is plain decode;
the newest query token sees everything; changing a window token changes exactly the query
tokens at or after it; with 16-bit heads every query token is softmax attention over its own
prefix of the raw keys and values."""
import math

import numpy as np

from oracle import kvq_oracle as O
from workloads import random_raw16


def _cfg(kb=(3, 2), vb=(2, 4), G=1, T=300):
    return O.CacheConfig(batch=2, n_kv=2, n_q=2 * G, head_dim=64, capacity=T + 8, n_sink=3, n_recent=40,
                         dtype="bf16", quant="hybrid", k_bits=kb, v_bits=vb)


def _data(seed, T, G, Q, D=64):
    rng = np.random.default_rng(seed)
    k = random_raw16(rng, (2, 2, T, D), "bf16", 2.0)
    v = random_raw16(rng, (2, 2, T, D), "bf16")
    q = random_raw16(rng, (2, Q, 2 * G, D), "bf16")
    return k, v, q


def test_one_token_is_decode():
    k, v, q = _data(1, 300, 2, 1)
    oc = O.build_cache(k, v, _cfg(G=2))
    assert np.array_equal(O.decode_multi(oc, q)[:, 0], O.decode(oc, q[:, 0]))


def test_newest_token_sees_everything():
    k, v, q = _data(2, 300, 1, 4)
    oc = O.build_cache(k, v, _cfg(G=1))
    assert np.array_equal(O.decode_multi(oc, q)[:, 3], O.decode(oc, q[:, 3]))


def test_causality():
    T, Q = 300, 4
    k, v, q = _data(3, T, 1, Q)
    cfg = _cfg(G=1, T=T)
    base = O.decode_multi(O.build_cache(k, v, cfg), q)
    for back in (1, 2, 3):  # token T - back: a recent-window token
        k2, v2 = k.copy(), v.copy()
        k2[:, :, T - back] ^= np.uint16(0x0100)
        v2[:, :, T - back] ^= np.uint16(0x0100)
        out = O.decode_multi(O.build_cache(k2, v2, cfg), q)
        first = Q - back  # the first query token that sees token T - back
        assert np.array_equal(out[:, :first], base[:, :first])
        assert np.all(np.any(out[:, first:] != base[:, first:], axis=-1))


def test_16bit_heads_prefix_attention():
    T, Q, D = 90, 3, 64
    k, v, q = _data(4, T, 1, Q)
    oc = O.build_cache(k, v, _cfg(kb=(16, 16), vb=(16, 16), G=1, T=T))
    got = O.decode_multi(oc, q)
    kf = O.widen16(k, "bf16").astype(np.float64)
    vf = O.widen16(v, "bf16").astype(np.float64)
    qf = O.widen16(q, "bf16").astype(np.float64)
    for b in range(2):
        for i in range(Q):
            n = T - Q + i + 1
            for hq in range(2):
                s = kf[b, hq, :n] @ qf[b, i, hq] / math.sqrt(D)
                w = np.exp(s - s.max())
                want = w @ vf[b, hq, :n] / w.sum()
                assert np.allclose(got[b, i, hq], want, rtol=1e-12, atol=1e-14)
