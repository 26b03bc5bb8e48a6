"""Pins of the oracle's quantizer, packing and window rule (CPU only).

Each test checks the oracle against something other than itself: IEEE-754 facts, a
brute-force nearest level, a hand-derived packing golden, the high-resolution MSE law of a
uniform quantizer, or an invariant the definition implies.
"""
import os

import numpy as np
import pytest

from oracle import kvq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- float16 rounding ----

def _rne_f16_bits(x32: np.ndarray) -> np.ndarray:
    """Independent bit-level float32 -> float16 round-to-nearest-even (finite inputs)."""
    u = x32.view(np.uint32).astype(np.int64)
    sign = (u >> 31) << 15
    e = (u >> 23) & 0xFF
    m = u & 0x7FFFFF
    out = np.zeros_like(u)
    # normal results
    ue = e - 127 + 15
    mant = m | 0x800000                      # 24-bit significand
    # shift to 11-bit significand; for subnormal results shift further
    shift = np.where(ue >= 1, 13, 13 + (1 - ue))
    shift = np.minimum(shift, 40)
    q = mant >> shift
    rem = mant - (q << shift)
    halfv = np.int64(1) << (shift - 1)
    up = (rem > halfv) | ((rem == halfv) & ((q & 1) == 1))
    q = q + up
    res = np.where(ue >= 1, ((ue - 1) << 10) + q, q)  # q may carry into exponent: fine
    res = np.where(e == 0, 0, res)                    # fp32 subnormals -> +-0
    res = np.where(res >= 0x7C00, 0x7C00, res)        # overflow -> inf
    out = sign | res
    return out.astype(np.uint16)


def test_f16_ieee_facts():
    cases = {
        1.0 + 2.0 ** -11: 1.0,                       # tie -> even (down)
        1.0 + 3 * 2.0 ** -11: 1.0 + 2.0 ** -9,       # tie -> even (up)
        65504.0: 65504.0,
        65519.0: 65504.0,
        2.0 ** -24: 2.0 ** -24,                      # smallest subnormal
        2.0 ** -25: 0.0,                             # tie with 0 -> even (0)
        1.5 * 2.0 ** -25: 2.0 ** -24,
        -3.0 * 2.0 ** -26: -2.0 ** -24,
    }
    for x, want in cases.items():
        assert float(O.f16(np.float32(x))) == want, x
    assert np.isinf(O.f16(np.float32(65520.0)))


def test_f16_matches_bit_level_rne():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 65504.0)]
    # plus every float32 in [2^-26, 2^-13] step pattern (subnormal boundary)
    lo = np.float32(2.0 ** -26).view(np.uint32)
    hi = np.float32(2.0 ** -13).view(np.uint32)
    x = np.concatenate([x, np.arange(lo, hi, 7, dtype=np.uint32).view(np.float32)])
    got = O.f16(x).view(np.uint16)
    want = _rne_f16_bits(x)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- quantizers ----------

def _groups(rng, n, dtype="fp16", scale=1.0):
    from workloads import random_raw16
    return O.widen16(random_raw16(rng, (n, 32), dtype, scale), dtype)


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_asym_is_nearest_level(b, dtype):
    rng = np.random.default_rng(b)
    x = _groups(rng, 4000, dtype, scale=3.0)
    c, s, z = O.quant_asym(x, b)
    s64 = s.astype(np.float64)[:, None]
    z64 = z.astype(np.float64)[:, None]
    levels = np.arange(2 ** b, dtype=np.float64)
    # brute force over every level in float64
    err = np.abs(x.astype(np.float64)[..., None] - (levels * s64[..., None] + z64[..., None]))
    best = err.argmin(axis=-1)
    t_exact = (x.astype(np.float64) - z64) / s64
    frac = t_exact - np.floor(t_exact)
    near_tie = np.abs(frac - 0.5) < 1e-5
    bad = (best != c) & ~near_tie
    assert not bad.any()
    # the group minimum (fp16 inputs: exactly representable) decodes to z exactly
    if dtype == "fp16":
        xhat = O.dequant(c, s, z)
        amin = x.argmin(axis=1)
        assert np.array_equal(xhat[np.arange(len(x)), amin], x.min(axis=1).astype(np.float64))
    assert c.max() <= 2 ** b - 1


def test_asym_constant_group_and_scale_zero():
    x = np.full((3, 32), 1.25, dtype=np.float32)
    c, s, z = O.quant_asym(x, 3)
    assert np.all(c == 0) and np.all(s == 0) and np.all(z.astype(np.float64) == 1.25)
    assert np.array_equal(O.dequant(c, s, z), np.full((3, 32), 1.25))


@pytest.mark.parametrize("b", [2, 3, 4, 8])
def test_sym_is_nearest_level_with_exact_zero(b):
    rng = np.random.default_rng(10 + b)
    x = _groups(rng, 3000, "bf16", 2.0)
    x[:, 5] = 0.0
    c, s, z = O.quant_sym(x, b)
    Q = 2 ** (b - 1) - 1
    assert c.min() >= 1 and c.max() <= 2 ** b - 1
    xhat = O.dequant(c, s, z)
    assert np.all(xhat[:, 5] == 0.0)
    s64 = s.astype(np.float64)[:, None]
    lev = np.arange(-Q, Q + 1, dtype=np.float64)
    err = np.abs(x.astype(np.float64)[..., None] - lev * s64[..., None])
    best = lev[err.argmin(axis=-1)]
    t_exact = x.astype(np.float64) / s64
    frac = t_exact - np.floor(t_exact)
    near_tie = np.abs(frac - 0.5) < 1e-5
    got = c.astype(np.int64) - 2 ** (b - 1)
    assert not ((best != got) & ~near_tie).any()
    # the stored affine form equals the signed level times s
    assert np.array_equal(xhat, got * s64)


def test_hybrid_takes_lower_sse():
    rng = np.random.default_rng(3)
    x = _groups(rng, 5000, "bf16")
    x[:1000, :4] *= 8.0          # outlier channels make symmetric competitive
    for b in (2, 3, 4):
        c, s, z, f = O.quant_group(x, b, hybrid=True)
        ca, sa, za = O.quant_asym(x, b)
        cs, ss, zs = O.quant_sym(x, b)
        # independent SSE (numpy pairwise sums): hybrid equals the smaller one
        ea = ((x.astype(np.float64) - O.dequant(ca, sa, za)) ** 2).sum(1)
        es = ((x.astype(np.float64) - O.dequant(cs, ss, zs)) ** 2).sum(1)
        eh = ((x.astype(np.float64) - O.dequant(c, s, z)) ** 2).sum(1)
        assert np.allclose(eh, np.minimum(ea, es), rtol=1e-12, atol=0)
        clear = np.abs(ea - es) > 1e-9 * np.maximum(ea, es)
        assert np.array_equal(f[clear].astype(bool), (es < ea)[clear])
        assert eh.mean() <= ea.mean()
    # at 2 bits on outlier-heavy groups symmetric wins often, on Gaussian groups rarely
    _, _, _, f2 = O.quant_group(x, 2, hybrid=True)
    assert f2[:1000].mean() > 0.2 and f2[1000:].mean() < 0.05


def test_mse_law_of_uniform_quantizer():
    """High-resolution law: D(b) ~ E[R^2] (n-2) / (12 n) / (2^b - 1)^2 for n = 32 Gaussian
    samples of range R (the group min/max carry ~no error), i.e. D decays close to 4^-b."""
    rng = np.random.default_rng(0)
    n_grp = 60000
    x = _groups(rng, n_grp, "fp16")
    D = [float(((x.astype(np.float64) - O.dequant(*O.quant_asym(x, b))) ** 2).mean())
         for b in range(2, 9)]
    # closed-form constant from an independent Monte-Carlo of the range only
    r = rng.standard_normal((200000, 32))
    ER2 = float(((r.max(1) - r.min(1)) ** 2).mean())
    const = ER2 * 30.0 / (12.0 * 32.0)
    scaled = [d * (2 ** b - 1) ** 2 for d, b in zip(D, range(2, 9))]
    assert abs(scaled[-1] / const - 1) < 0.02
    for v in scaled:
        assert abs(v / scaled[-1] - 1) < 0.02
    assert 3.95 <= D[5] / D[6] <= 4.10
    a, beta, r2, _ = O.fit_one(range(2, 9), D)
    assert 4.2 <= beta <= 4.5 and r2 > 0.99
    # RateQuant abstract: beta spans 3.6 .. 5.3 across quantizers; ours falls inside
    assert 3.6 <= beta <= 5.3


# ---------------------------------------------------------------- packing -------------

def _golden_words():
    out = {}
    with open(os.path.join(GOLDEN, "pack_words.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            tok = line.split()
            out[int(tok[0])] = [int(t, 16) for t in tok[1:]]
    return out


def test_pack_golden_words():
    g = _golden_words()
    for b, words in g.items():
        codes = (np.arange(32) % (2 ** b)).astype(np.uint8)
        assert O.pack(codes, b).tolist() == words
        assert np.array_equal(O.unpack(np.array(words, dtype=np.uint32), b), codes)


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 7, 8])
def test_pack_roundtrip(b):
    rng = np.random.default_rng(b)
    codes = rng.integers(0, 2 ** b, size=(500, 32)).astype(np.uint8)
    w = O.pack(codes, b)
    assert w.shape == (500, b)
    assert np.array_equal(O.unpack(w, b), codes)
    # every word bit is used exactly once: total popcount equals total code popcount
    pc = lambda a: np.unpackbits(np.ascontiguousarray(a).view(np.uint8)).sum()
    assert pc(w) == pc(codes)


# ---------------------------------------------------------------- windows -------------

def test_window_sizes_golden():
    with open(os.path.join(GOLDEN, "window_sizes.txt")) as fh:
        rows = [l.split() for l in fh if l.strip() and not l.startswith("#")]
    for T, ns, nr, body, win in (map(int, r) for r in rows):
        assert O.body_len(T, ns, nr) == body
        assert T - ns - body == win
        assert nr <= win <= nr + 31


def test_window_rule_invariants():
    for ns in (0, 1, 4):
        for nr in (0, 7, 32, 128):
            prev = 0
            for T in range(0, 700):
                bl = O.body_len(T, ns, nr)
                assert bl % 32 == 0 and bl >= prev and bl - prev in (0, 32)
                if T >= ns + nr:
                    assert nr <= T - ns - bl <= nr + 31
                else:
                    assert bl == 0
                prev = bl


def _small_cfg(k_bits, v_bits, quant="asym", D=64, H=2, cap=512, ns=1, nr=32, dtype="fp16"):
    return O.CacheConfig(batch=2, n_kv=H, n_q=2 * H, head_dim=D, capacity=cap, n_sink=ns,
                         n_recent=nr, dtype=dtype, quant=quant, k_bits=tuple(k_bits),
                         v_bits=tuple(v_bits))


def test_body_codes_never_change_after_written():
    from workloads import random_raw16
    rng = np.random.default_rng(5)
    cfg = _small_cfg((3, 16), (2, 5), quant="hybrid")
    k = random_raw16(rng, (2, 2, 400, 64), "fp16")
    v = random_raw16(rng, (2, 2, 400, 64), "fp16")
    full = O.build_cache(k, v, cfg)
    for T in (100, 177, 260, 333):
        part = O.build_cache(k[:, :, :T], v[:, :, :T], cfg)
        bl = part.body
        e0, e1 = part.heads[0], full.heads[0]
        assert np.array_equal(e0["k_codes"], e1["k_codes"][:, :bl])
        assert np.array_equal(e0["k_flag"], e1["k_flag"][:, :bl])
        assert np.array_equal(e0["v_codes"], e1["v_codes"][:, :bl // 32])
        assert np.array_equal(part.heads[1]["k_raw"], full.heads[1]["k_raw"][:, :bl])


def test_logical_cache_is_close_to_input_and_not_transposed():
    """x_hat lies within its group's half step (+ the fp16 rounding slack of s): catches a
    transposed key/value grouping or a misplaced window."""
    from workloads import random_raw16
    rng = np.random.default_rng(6)
    cfg = _small_cfg((8, 2), (8, 3))
    k = random_raw16(rng, (2, 2, 300, 64), "fp16")
    v = random_raw16(rng, (2, 2, 300, 64), "fp16")
    oc = O.build_cache(k, v, cfg)
    for h in range(2):
        for b in range(2):
            Kt, Vt = O.logical_kv(oc, b, h)
            K = O.widen16(k[b, h], "fp16").astype(np.float64)
            V = O.widen16(v[b, h], "fp16").astype(np.float64)
            assert Kt.shape == K.shape == Vt.shape
            ns, bl = 1, oc.body
            # windows are exact
            assert np.array_equal(Kt[:ns], K[:ns]) and np.array_equal(Kt[ns + bl:], K[ns + bl:])
            assert np.array_equal(Vt[ns + bl:], V[ns + bl:])
            # body: per-group error bound max-min/(2^b-1) (one full step covers s/2 + slack)
            kb, vb = cfg.k_bits[h], cfg.v_bits[h]
            Kg = K[ns:ns + bl].reshape(bl, 2, 32)
            stepk = (Kg.max(-1) - Kg.min(-1)) / (2 ** kb - 1)
            assert np.all(np.abs(Kt[ns:ns + bl].reshape(bl, 2, 32) - Kg) <= stepk[..., None] + 1e-3)
            Vg = V[ns:ns + bl].reshape(bl // 32, 32, 64)
            stepv = (Vg.max(1) - Vg.min(1)) / (2 ** vb - 1)
            assert np.all(np.abs(Vt[ns:ns + bl].reshape(bl // 32, 32, 64) - Vg) <= stepv[:, None] + 1e-3)


def test_range_check_rejects_large_inputs():
    cfg = _small_cfg((2, 2), (2, 2))
    k = np.zeros((2, 2, 100, 64), dtype=np.float32)
    k[0, 0, 50, 3] = 20000.0
    kr = k.astype(np.float16).view(np.uint16)
    with pytest.raises(ValueError):
        O.build_cache(kr, np.zeros_like(kr), cfg)
