"""Pins of the oracle's attention, split-K merge, distortion fit and bit allocation (CPU).

Attention is pinned to an independently written float64 softmax attention (torch) on
caches with nothing quantized; allocation to brute-force integer search, to the
closed-form waterfilling solution and to the AM/GM gain ratio.
"""
import math

import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O
from workloads import random_raw16


def _cfg(k_bits, v_bits, H=2, G=2, D=64, cap=1024, ns=1, nr=32, dtype="bf16", quant="asym"):
    return O.CacheConfig(batch=2, n_kv=H, n_q=G * H, head_dim=D, capacity=cap, n_sink=ns,
                         n_recent=nr, dtype=dtype, quant=quant, k_bits=tuple(k_bits),
                         v_bits=tuple(v_bits))


def _torch_attention(q, k, v, G):
    """Independent reference: torch float64 softmax(q k^T / sqrt(D)) v with explicit GQA."""
    B, Hq, D = q.shape
    qt = torch.tensor(q, dtype=torch.float64)
    kt = torch.tensor(k, dtype=torch.float64)
    vt = torch.tensor(v, dtype=torch.float64)
    out = torch.empty(B, Hq, D, dtype=torch.float64)
    for bb in range(B):
        for i in range(Hq):
            h = i // G
            w = torch.softmax((kt[bb, h] @ qt[bb, i]) / math.sqrt(D), dim=0)
            out[bb, i] = w @ vt[bb, h]
    return out.numpy()


@pytest.mark.parametrize("T", [1, 20, 33, 150, 600])
def test_all_16bit_heads_equal_plain_attention(T):
    rng = np.random.default_rng(T)
    H, G, D = 2, 3, 64
    cfg = _cfg((16, 16), (16, 16), H=H, G=G, D=D)
    k = random_raw16(rng, (2, H, T, D), "bf16", 2.0)
    v = random_raw16(rng, (2, H, T, D), "bf16")
    q = random_raw16(rng, (2, H * G, D), "bf16")
    oc = O.build_cache(k, v, cfg)
    got = O.decode(oc, q)
    want = _torch_attention(O.widen16(q, "bf16"), O.widen16(k, "bf16"), O.widen16(v, "bf16"), G)
    rms = np.sqrt((want ** 2).mean())
    assert np.abs(got - want).max() <= 1e-12 * rms


def test_no_body_quantized_heads_equal_plain_attention():
    rng = np.random.default_rng(7)
    cfg = _cfg((2, 3), (4, 2), ns=4, nr=64)
    T = 4 + 64 + 31                     # still no body block
    k = random_raw16(rng, (2, 2, T, 64), "bf16")
    v = random_raw16(rng, (2, 2, T, 64), "bf16")
    q = random_raw16(rng, (2, 4, 64), "bf16")
    oc = O.build_cache(k, v, cfg)
    assert oc.body == 0
    got = O.decode(oc, q)
    want = _torch_attention(O.widen16(q, "bf16"), O.widen16(k, "bf16"), O.widen16(v, "bf16"), 2)
    assert np.abs(got - want).max() <= 1e-12 * np.sqrt((want ** 2).mean())


def test_quantized_decode_equals_attention_on_dequantized_cache():
    """Quantized heads: the oracle's decode equals plain attention on its own logical
    cache, and the logical cache rebuilt from packed words (unpack) is identical."""
    rng = np.random.default_rng(8)
    cfg = _cfg((2, 4), (3, 2), quant="hybrid")
    T = 300
    k = random_raw16(rng, (2, 2, T, 64), "bf16")
    v = random_raw16(rng, (2, 2, T, 64), "bf16")
    q = random_raw16(rng, (2, 4, 64), "bf16")
    oc = O.build_cache(k, v, cfg)
    Ks = np.stack([np.stack([O.logical_kv(oc, b, h)[0] for h in range(2)]) for b in range(2)])
    Vs = np.stack([np.stack([O.logical_kv(oc, b, h)[1] for h in range(2)]) for b in range(2)])
    want = _torch_attention(O.widen16(q, "bf16"), Ks, Vs, 2)
    got = O.decode(oc, q)
    assert np.abs(got - want).max() <= 1e-12 * np.sqrt((want ** 2).mean())
    e = oc.heads[0]
    assert np.array_equal(O.unpack(O.pack(e["k_codes"], 2), 2), e["k_codes"])


def test_factorized_group_dot_equals_dequantized_dot():
    """q . x_hat over a key group == s (q . c) + z sum(q) (the form a fused kernel uses)."""
    rng = np.random.default_rng(9)
    x = O.widen16(random_raw16(rng, (2000, 32), "bf16"), "bf16")
    q = rng.standard_normal((2000, 32))
    for b in (2, 3, 4):
        c, s, z, _ = O.quant_group(x, b, hybrid=True)
        direct = (q * O.dequant(c, s, z)).sum(1)
        fact = s.astype(np.float64) * (q * c).sum(1) + z.astype(np.float64) * q.sum(1)
        assert np.allclose(direct, fact, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("chunks", [1, 2, 5, 16])
def test_lse_merge_equals_single_pass(chunks):
    rng = np.random.default_rng(chunks)
    T, D, G = 777, 32, 4
    q = rng.standard_normal((G, D))
    K = rng.standard_normal((T, D)) * 3
    V = rng.standard_normal((T, D))
    bounds = np.linspace(0, T, chunks + 1).astype(int)
    parts = [O.partial_softmax(q, K[a:b], V[a:b], 0.2) for a, b in zip(bounds[:-1], bounds[1:])]
    got = O.lse_merge([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])
    want = O.attention_head(q, K, V, 0.2)
    assert np.abs(got - want).max() <= 1e-13 * np.abs(want).max()


# ---------------------------------------------------------------- fit ----------------

def test_fit_recovers_exact_model():
    bs = list(range(2, 9))
    for alpha, beta in ((2.44, 4.35), (0.5, 3.6), (7.0, 5.3)):
        D = [alpha * beta ** (-b) for b in bs]
        a, bt, r2, deg = O.fit_one(bs, D)
        assert not deg and abs(a / alpha - 1) < 1e-12 and abs(bt / beta - 1) < 1e-12
        assert abs(r2 - 1) < 1e-12


def test_fit_fallback_for_poor_fits():
    bs = list(range(2, 9))
    good1 = [2.0 * 4.0 ** (-b) for b in bs]
    good2 = [1.0 * 5.0 ** (-b) for b in bs]
    bumpy = [1.0 * 6.0 ** (-b) * (3.0 if b % 2 else 0.3) for b in bs]
    a, beta, r2 = O.fit_heads(bs, [good1, good2, bumpy])
    assert r2[0] > 0.999 and r2[2] < 0.96
    assert abs(beta[0] - 4.0) < 1e-9 and abs(beta[1] - 5.0) < 1e-9
    assert abs(beta[2] - 4.5) < 1e-9          # min(beta_fit ~ 6, mean of good betas 4.5)
    zero = [0.0] * 7
    a, beta, r2 = O.fit_heads(bs, [good1, zero])
    assert a[1] == 0.0 and beta[1] == 4.0 and r2[1] == 1.0


# ---------------------------------------------------------------- allocation ---------

def _rand_model(rng, n):
    return (list(rng.uniform(0.5, 2.0, n)), list(rng.uniform(3.6, 5.3, n)),
            list(rng.lognormal(0.0, 1.0, n)))


def test_greedy_equals_bruteforce():
    rng = np.random.default_rng(11)
    n_unique = 0
    for trial in range(600):
        n = int(rng.integers(2, 7))
        b_lo, b_hi = (2, 4) if trial % 2 else (2, 8)
        if n > 4 and b_hi == 8:
            b_hi = 6
        total = int(rng.integers(n * b_lo, n * b_hi + 1))
        a, bt, w = _rand_model(rng, n)
        g = O.allocate_greedy(a, bt, w, total, b_lo, b_hi)
        assert sum(g) == total and all(b_lo <= x <= b_hi for x in g)
        best, near = O.allocate_bruteforce(a, bt, w, total, b_lo, b_hi)
        assert O.objective(a, bt, w, g) <= best * (1 + 1e-12)
        if len(near) == 1:
            n_unique += 1
            assert tuple(g) == near[0]
    assert n_unique > 500


def test_closed_form_waterfilling_beta4():
    """beta = 4, alpha = 1, no bound active: b_i = Bbar + 1/2 log2(w_i / GM(w))
    (RSAVQ appendix A.8, Lagrangian of D ~ I * 2^-2b) and the uniform/optimal distortion
    ratio equals AM(w)/GM(w) (RateQuant section 3.1 / B.2)."""
    rng = np.random.default_rng(12)
    n = 8
    w = list(rng.lognormal(0.0, 0.6, n))
    gm = math.exp(sum(math.log(x) for x in w) / n)
    am = sum(w) / n
    Bbar = 4.0
    cont = O.allocate_continuous([1.0] * n, [4.0] * n, w, int(Bbar * n), 2, 8)
    want = [Bbar + 0.5 * math.log2(x / gm) for x in w]
    assert all(2 < x < 8 for x in want)
    assert max(abs(c - x) for c, x in zip(cont, want)) < 1e-9
    d_uni = sum(x * 4.0 ** (-Bbar) for x in w)
    d_opt = sum(x * 4.0 ** (-b) for x, b in zip(w, cont))
    assert abs((d_uni / d_opt) / (am / gm) - 1) < 1e-9
    assert am / gm >= 1.0


def test_floor_budget_and_identical_heads():
    a, bt, w = [1.0] * 5, [4.0] * 5, [1.0] * 5
    assert O.allocate_greedy(a, bt, w, 10, 2, 4) == [2] * 5          # floor: ratio 1
    assert O.allocate_greedy(a, bt, w, 13, 2, 4) == [3, 3, 3, 2, 2]  # ties -> low index
    assert O.allocate_continuous(a, bt, w, 10, 2, 4) == [2.0] * 5
    assert max(abs(x - 2.6) for x in O.allocate_continuous(a, bt, w, 13, 2, 4)) < 1e-9


def test_continuous_kkt_and_integer_bracket():
    rng = np.random.default_rng(13)
    bracket_ok = 0
    for trial in range(300):
        n = int(rng.integers(2, 9))
        b_lo, b_hi = 2, (4 if trial % 2 else 8)
        total = int(rng.integers(n * b_lo, n * b_hi + 1))
        a, bt, w = _rand_model(rng, n)
        cont = O.allocate_continuous(a, bt, w, total, b_lo, b_hi)
        assert abs(sum(cont) - total) < 1e-8
        # KKT: free heads share the marginal w a ln(beta) beta^-b; bounded heads lie on the
        # right side of it
        marg = [wi * ai * math.log(bi) * bi ** (-b) for ai, bi, wi, b in zip(a, bt, w, cont)]
        free = [m for m, b in zip(marg, cont) if b_lo + 1e-9 < b < b_hi - 1e-9]
        if free:
            lam = free[0]
            assert all(abs(m / lam - 1) < 1e-6 for m in free)
            for m, b in zip(marg, cont):
                if b <= b_lo + 1e-9:
                    assert m <= lam * (1 + 1e-6)
                if b >= b_hi - 1e-9:
                    assert m >= lam * (1 - 1e-6)
        g = O.allocate_greedy(a, bt, w, total, b_lo, b_hi)
        bracket_ok += all(math.floor(c + 1e-9) <= x <= math.ceil(c - 1e-9) for c, x in zip(cont, g))
    assert bracket_ok >= 290     # an observation, not a theorem


def test_cap_weights():
    w = [1.0] * 9 + [100.0]
    cw = O.cap_weights(w)
    assert cw[:9] == [1.0] * 9 and abs(cw[9] - 5 * 109.0 / 10) < 1e-12


def test_alloc_argument_errors():
    with pytest.raises(ValueError):
        O.allocate_greedy([1.0] * 4, [4.0] * 4, [1.0] * 4, 7, 2, 4)     # below floor
    with pytest.raises(ValueError):
        O.allocate_greedy([1.0] * 4, [4.0] * 4, [1.0] * 4, 17, 2, 4)    # above ceiling
    with pytest.raises(ValueError):
        O.allocate_greedy([1.0] * 4, [1.0] * 4, [1.0] * 4, 10, 2, 4)    # beta must be > 1


def test_calibration_distortion_orders_and_law():
    rng = np.random.default_rng(14)
    x = random_raw16(rng, (512, 128), "bf16")
    Dk = O.calib_distortion(x, "bf16", 0, 2, 8, False)
    Dv = O.calib_distortion(x, "bf16", 1, 2, 8, False)
    assert np.all(np.diff(Dk) < 0) and np.all(np.diff(Dv) < 0)
    # i.i.d. data: key-axis and value-axis grouping see the same statistics
    assert np.allclose(Dk, Dv, rtol=0.05)
    a, bt, r2, _ = O.fit_one(range(2, 9), list(Dk))
    assert 4.2 <= bt <= 4.5 and r2 > 0.99


def test_calibration_grouping_direction_closed_form():
    # values are grouped along tokens (32 tokens of one channel), keys along channels (32
    # channels of one token), InnerQ page, abstract and "Core claim". Data constant along the
    # tokens of every channel makes every value group constant, so its error is exactly 0
    # (z = the group's value, s = 0), while key groups, which mix channels, are not; data
    # constant along channels does the opposite. A transposed grouping on either axis fails.
    rng = np.random.default_rng(15)
    a = rng.normal(size=64).astype(np.float16)              # one fp16 value per channel
    b = rng.normal(size=96).astype(np.float16)              # one fp16 value per token
    tok_const = np.broadcast_to(a[None, :], (96, 64)).copy().view(np.uint16)
    ch_const = np.broadcast_to(b[:, None], (96, 64)).copy().view(np.uint16)
    for bits in (2, 3, 8):
        for hyb in (False, True):
            assert np.all(O.calib_group_sse(tok_const, "fp16", 1, bits, hyb) == 0.0)
            assert np.all(O.calib_group_sse(tok_const, "fp16", 0, bits, hyb) > 0.0)
            assert np.all(O.calib_group_sse(ch_const, "fp16", 0, bits, hyb) == 0.0)
            assert np.all(O.calib_group_sse(ch_const, "fp16", 1, bits, hyb) > 0.0)
    D = O.calib_distortion(tok_const, "fp16", 1, 2, 8, False)
    assert np.all(D == 0.0)


def test_calibration_groups_brute_force_on_channel_scaled_data():
    # per-channel scales and x8 outlier channels (the key statistics of the workloads): the
    # per-group errors, in the documented order (keys: token, then group; values: token block,
    # then channel), equal a group-by-group loop over explicit index ranges
    rng = np.random.default_rng(16)
    T, D = 64, 64
    x = rng.normal(size=(T, D)) * rng.lognormal(0.0, 0.5, size=D)[None, :]
    x[:, [3, 17, 40, 41]] *= 8.0
    raw = x.astype(np.float16).view(np.uint16)
    xf = raw.view(np.float16).astype(np.float32)
    for bits in (2, 4):
        for hyb in (False, True):
            want_k, want_v = [], []
            for t in range(T):
                for g in range(D // 32):
                    want_k.append(_group_err(xf[t, 32 * g:32 * g + 32], bits, hyb))
            for j in range(T // 32):
                for c in range(D):
                    want_v.append(_group_err(xf[32 * j:32 * j + 32, c], bits, hyb))
            got_k = O.calib_group_sse(raw, "fp16", 0, bits, hyb)
            got_v = O.calib_group_sse(raw, "fp16", 1, bits, hyb)
            assert np.array_equal(got_k, np.array(want_k)), (bits, hyb)
            assert np.array_equal(got_v, np.array(want_v)), (bits, hyb)


def _group_err(g, bits, hyb):
    """Squared error of one group of 32 values, summed element by element in float64."""
    c, s, z, _ = O.quant_group(np.asarray(g, dtype=np.float32)[None, :], bits, hyb)
    xhat = [float(ci) * float(s[0]) + float(z[0]) for ci in c[0]]
    tot = 0.0
    for xi, yi in zip(g.tolist(), xhat):
        d = float(xi) - yi
        tot = tot + d * d
    return tot


def test_allocation_margin_equals_log_ratio_of_objective_changes():
    # the margin of a greedy allocation is ln(smallest objective increase from taking back one
    # handed-out bit / largest objective decrease from handing out one more), both measured
    # with the objective sum w a beta^-b itself (RateQuant page, section 3.3)
    rng = np.random.default_rng(17)
    for trial in range(200):
        n = int(rng.integers(2, 7))
        b_lo, b_hi = (2, 4) if trial % 2 else (2, 8)
        total = int(rng.integers(n * b_lo + 1, n * b_hi))
        a = list(rng.uniform(0.5, 2.0, n))
        bt = list(rng.uniform(3.6, 5.3, n))
        w = list(rng.lognormal(0.0, 1.0, n))
        bits = O.allocate_greedy(a, bt, w, total, b_lo, b_hi)
        base = O.objective(a, bt, w, bits)
        up, down = [], []
        for i in range(n):
            if bits[i] > b_lo:
                v = list(bits); v[i] -= 1
                up.append(O.objective(a, bt, w, v) - base)
            if bits[i] < b_hi:
                v = list(bits); v[i] += 1
                down.append(base - O.objective(a, bt, w, v))
        m = O.allocation_margin(a, bt, w, bits, b_lo, b_hi)
        assert m >= 0.0
        assert abs(m - math.log(min(up) / max(down))) < 1e-6, (trial, m)
