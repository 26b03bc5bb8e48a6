"""GPU parity of libkvq against the CPU oracle, through the C ABI.

Packed codes, scales/zeros, hybrid flags, windows and bit allocations must be bit-exact;
decode outputs must satisfy max|gpu - oracle| <= 2e-3 * RMS(oracle output). Inputs are the
seeded synthetic workloads (reduced sizes here; full sizes in test_gpu_fullsize.py).
"""
import sys

import numpy as np
import pytest
import torch

import mixed_precision_quantized_kvq_amd as kvq
import workloads
from oracle import kvq_oracle as O
from tests import cache_format as F
from tests.kvq_test_util import (head_slice_cfg, lib_cfg, oracle_bits, oracle_calibration,
                                 oracle_cfg, within_tol)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def gpu_cache(ocfg, k, v, chunks=None):
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    if chunks is None:
        kvq.append(cache, to_dev(k), to_dev(v))
    else:
        pos = 0
        for n in chunks:
            kvq.append(cache, to_dev(k[:, :, pos:pos + n]), to_dev(v[:, :, pos:pos + n]))
            pos += n
        assert pos == k.shape[2]
    torch.cuda.synchronize()
    kvq.cache_check(cache)
    return cache


def assert_regions_equal(cache, oc, rows=None, heads=None, map_bh=lambda b, h: (b, h)):
    """Read every (row, KV head) of the device blob through the cache format and compare its
    logical content (codes, scales, zeros, flags, 16-bit rows, norms) with the oracle's, bit
    for bit."""
    cfg = oc.cfg
    for b in (range(cfg.batch) if rows is None else rows):
        for h in (range(cfg.n_kv) if heads is None else heads):
            gb, gh = map_bh(b, h)
            regions = [cache.region(gb, gh, r).cpu().numpy() for r in range(F.N_REGIONS)]
            assert [x.size for x in regions] == F.region_sizes(cfg, h), (b, h)
            got = F.decode_head(regions, cfg, h, oc.T)
            F.assert_content_equal(got, F.oracle_head_content(oc, b, h), f"row {b} head {h}")


def gpu_decode(cache, q, n_splits, scale=0.0):
    c = cache.cfg
    out = torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32, device=DEV)
    ws = torch.zeros(kvq.decode_workspace_bytes(cache, n_splits), dtype=torch.uint8, device=DEV)
    kvq.decode_attention(cache, to_dev(q), out, n_splits, ws, scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check_decode(cache, oc, q, splits=(1, 4, 16)):
    want = O.decode(oc, q)
    for ns in splits:
        got = gpu_decode(cache, q, ns)
        ok, err, bound = within_tol(got, want)
        say(f"    decode n_splits={ns}: max err {err:.3e} (bound {bound:.3e})")
        assert ok


# ------------------------------------------------------------------------------------------

def test_tiny_workload_full():
    say("case: tiny_t256 bulk append + decode")
    w = workloads.make("tiny_t256")
    ocfg = oracle_cfg(w, *oracle_bits(w))
    oc = O.build_cache(w["k"], w["v"], ocfg)
    cache = gpu_cache(ocfg, w["k"], w["v"])
    assert cache.len == 256
    assert_regions_equal(cache, oc)
    check_decode(cache, oc, w["q"], splits=(1, 2, 4, 7))


@pytest.mark.parametrize("name,B,T", [("llama8b_t8k", 2, 1500), ("qwen8b_t32k", 1, 2600),
                                      ("long_t128k", 1, 3000)])
def test_reduced_workloads(name, B, T):
    say(f"case: {name} reduced B={B} T={T}")
    w = workloads.make(name, tokens=T, batch=B)
    s = w["spec"]
    kb, vb = oracle_bits(w)
    if s.alloc == "joint":
        gb, _ = kvq.allocate_bits(w["alpha"], w["beta"], w["w"], s.k_total, s.b_lo, s.b_hi)
        assert tuple(gb) == kb
    elif s.alloc == "separate":
        gk, _ = kvq.allocate_bits(w["alpha_k"], w["beta_k"], w["w_k"], s.k_total, s.b_lo, s.b_hi)
        gv, _ = kvq.allocate_bits(w["alpha_v"], w["beta_v"], w["w_v"], s.v_total, s.b_lo, s.b_hi)
        assert tuple(gk) == kb and tuple(gv) == vb
    ocfg = oracle_cfg(w, kb, vb)
    oc = O.build_cache(w["k"], w["v"], ocfg)
    cache = gpu_cache(ocfg, w["k"], w["v"])
    assert_regions_equal(cache, oc)
    check_decode(cache, oc, w["q"], splits=(1, s.n_splits, 33))


def test_prefill_calibrate_allocate_append_reduced():
    say("case: prefill_t4k reduced B=2 T=700 (calibrate -> allocate -> append)")
    w = workloads.make("prefill_t4k", tokens=700, batch=2)
    s = w["spec"]
    ref = oracle_calibration(w)
    got = {}
    for name, arr, axis in (("k", w["k"], kvq.AXIS_KEY), ("v", w["v"], kvq.AXIS_VALUE)):
        x = to_dev(np.ascontiguousarray(arr[0, :, :s.calib_tokens]))
        got[name] = kvq.calibrate_fit(x, s.dtype, axis, kvq.QUANT_ASYM, 2, 8)
        for i, lab in enumerate(("alpha", "beta", "r2")):
            a = np.array(got[name][i])
            bref = np.array(ref[name][i])
            assert np.allclose(a, bref, rtol=1e-13, atol=0), (name, lab, a, bref)
    kb, vb = oracle_bits(w, alpha_k=ref["k"][0], beta_k=ref["k"][1], alpha_v=ref["v"][0], beta_v=ref["v"][1])
    gk, _ = kvq.allocate_bits(got["k"][0], got["k"][1], w["w_k"], s.k_total, 2, 4)
    gv, _ = kvq.allocate_bits(got["v"][0], got["v"][1], w["w_v"], s.v_total, 2, 4)
    assert tuple(gk) == kb and tuple(gv) == vb
    ocfg = oracle_cfg(w, kb, vb)
    oc = O.build_cache(w["k"], w["v"], ocfg)
    cache = gpu_cache(ocfg, w["k"], w["v"])
    assert_regions_equal(cache, oc)
    check_decode(cache, oc, w["q"], splits=(3,))


@pytest.mark.parametrize("chunks", [[1] * 300, [7] * 42 + [6], [33, 64, 1, 100, 2, 50, 50]],
                         ids=["one-token", "seven", "ragged"])
def test_streaming_append_equals_bulk(chunks):
    say(f"case: streaming append chunks={chunks[:4]}...")
    rng = np.random.default_rng(31)
    T = sum(chunks)
    ocfg = O.CacheConfig(2, 2, 4, 64, T + 5, 3, 40, "bf16", "hybrid", (3, 2), (2, 4))
    k = workloads.random_raw16(rng, (2, 2, T, 64), "bf16", 2.0)
    v = workloads.random_raw16(rng, (2, 2, T, 64), "bf16")
    q = workloads.random_raw16(rng, (2, 4, 64), "bf16")
    oc = O.build_cache(k, v, ocfg)
    cache = gpu_cache(ocfg, k, v, chunks=chunks)
    assert_regions_equal(cache, oc)
    check_decode(cache, oc, q, splits=(2,))


def test_16bit_heads_and_mixed_widths():
    say("case: 16-bit heads + every width 2..8, hybrid, D=128")
    rng = np.random.default_rng(32)
    T = 900
    kb = (16, 2, 3, 4, 5, 6, 7, 8)
    vb = (8, 7, 16, 5, 4, 3, 2, 16)
    ocfg = O.CacheConfig(1, 8, 16, 128, T, 4, 64, "fp16", "hybrid", kb, vb)
    k = workloads.random_raw16(rng, (1, 8, T, 128), "fp16", 3.0)
    v = workloads.random_raw16(rng, (1, 8, T, 128), "fp16")
    q = workloads.random_raw16(rng, (1, 16, 128), "fp16")
    oc = O.build_cache(k, v, ocfg)
    cache = gpu_cache(ocfg, k, v, chunks=[500, 1, 399])
    assert_regions_equal(cache, oc)
    check_decode(cache, oc, q, splits=(1, 5))


def test_full_grid_all_body_paths():
    # a grid of 4 rows x 8 KV heads x 15..32 chunks (more workgroups than CUs) with every body
    # path in one launch (widths 2-4, wider widths, 16-bit sides), window units, and fused
    # decode steps across a block flush
    say("case: B=4 x 8 KV heads, all body paths, 15-32 splits, fused steps")
    rng = np.random.default_rng(33)
    T0, steps = 1100, 40
    T = T0 + steps
    kb = (2, 3, 4, 16, 5, 2, 3, 4)
    vb = (2, 3, 4, 16, 2, 8, 4, 3)
    ocfg = O.CacheConfig(4, 8, 32, 128, T, 4, 64, "bf16", "hybrid", kb, vb)
    k = workloads.random_raw16(rng, (4, 8, T, 128), "bf16", 2.0)
    v = workloads.random_raw16(rng, (4, 8, T, 128), "bf16")
    q = workloads.random_raw16(rng, (4, 32, 128), "bf16")
    ocfg0 = O.CacheConfig(4, 8, 32, 128, T, 4, 64, "bf16", "hybrid", kb, vb)
    oc = O.build_cache(k[:, :, :T0], v[:, :, :T0], ocfg0)
    cache = gpu_cache(ocfg, k[:, :, :T0], v[:, :, :T0])
    assert_regions_equal(cache, oc)
    check_decode(cache, oc, q, splits=(15, 16, 32))
    out = torch.empty((4, 32, 128), dtype=torch.float32, device=DEV)
    ws = torch.zeros(kvq.decode_workspace_bytes(cache, 16), dtype=torch.uint8, device=DEV)
    qd = to_dev(q)
    for s_ in range(steps):
        t = T0 + s_
        kvq.decode_step(cache, to_dev(np.ascontiguousarray(k[:, :, t:t + 1])),
                        to_dev(np.ascontiguousarray(v[:, :, t:t + 1])), qd, out, 16, ws)
        if s_ % 8 == 7:
            oc_t = O.build_cache(k[:, :, :t + 1], v[:, :, :t + 1], ocfg0)
            ok, err, bound = within_tol(out.cpu().numpy(), O.decode(oc_t, q))
            say(f"    step {s_}: max err {err:.3e} (bound {bound:.3e})")
            assert ok, (s_, err, bound)
    assert_regions_equal(cache, O.build_cache(k, v, ocfg))


@pytest.mark.parametrize("T", [1, 3, 4 + 32, 4 + 32 + 31, 4 + 32 + 32, 4 + 32 + 95, 200])
def test_decode_edge_lengths(T):
    say(f"case: edge length T={T}")
    rng = np.random.default_rng(T)
    ocfg = O.CacheConfig(1, 2, 2, 64, 256, 4, 32, "bf16", "asym", (2, 4), (4, 2))
    k = workloads.random_raw16(rng, (1, 2, T, 64), "bf16")
    v = workloads.random_raw16(rng, (1, 2, T, 64), "bf16")
    q = workloads.random_raw16(rng, (1, 2, 64), "bf16", 3.0)
    oc = O.build_cache(k, v, ocfg)
    cache = gpu_cache(ocfg, k, v)
    assert_regions_equal(cache, oc)
    check_decode(cache, oc, q, splits=(1, 3))


@pytest.mark.parametrize("T", [250, 700, 1333])
def test_long_window_across_splits(T):
    # a 200-token recent window (up to 4 window tiles, wrapping around the ring) shared out
    # over several splits together with the body tiles; some splits get no tile at all
    say(f"case: long window T={T}")
    rng = np.random.default_rng(70 + T)
    ocfg = O.CacheConfig(1, 2, 8, 128, 2000, 5, 200, "fp16", "hybrid", (3, 2), (2, 4))
    k = workloads.random_raw16(rng, (1, 2, T, 128), "fp16", 2.0)
    v = workloads.random_raw16(rng, (1, 2, T, 128), "fp16")
    q = workloads.random_raw16(rng, (1, 8, 128), "fp16")
    oc = O.build_cache(k, v, ocfg)
    cache = gpu_cache(ocfg, k, v, chunks=[T // 2, T - T // 2])
    assert_regions_equal(cache, oc)
    check_decode(cache, oc, q, splits=(1, 2, 3, 6, 40))


@pytest.mark.parametrize("n_recent,n_sink", [(40, 3), (0, 0), (64, 5)])
def test_decode_step_sequence(n_recent, n_sink):
    # token-by-token decode steps (append + decode in one call): every step's output against
    # the oracle on the whole prefix, crossing several 32-token flushes and the sink; at the end
    # the cache bytes equal a bulk-built cache's
    say(f"case: decode_step sequence n_recent={n_recent} n_sink={n_sink}")
    rng = np.random.default_rng(80 + n_recent)
    T0, steps = 90, 75
    T = T0 + steps
    ocfg = O.CacheConfig(2, 2, 4, 128, T + 8, n_sink, n_recent, "bf16", "hybrid", (3, 2), (2, 4))
    k = workloads.random_raw16(rng, (2, 2, T, 128), "bf16", 2.0)
    v = workloads.random_raw16(rng, (2, 2, T, 128), "bf16")
    qs = workloads.random_raw16(rng, (steps, 2, 4, 128), "bf16")
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    if T0:
        kvq.append(cache, to_dev(np.ascontiguousarray(k[:, :, :T0])), to_dev(np.ascontiguousarray(v[:, :, :T0])))
    out = torch.empty((2, 4, 128), dtype=torch.float32, device=DEV)
    ws = torch.zeros(kvq.decode_workspace_bytes(cache, 3), dtype=torch.uint8, device=DEV)
    worst = 0.0
    for s in range(steps):
        t = T0 + s
        kvq.decode_step(cache, to_dev(np.ascontiguousarray(k[:, :, t:t + 1])),
                        to_dev(np.ascontiguousarray(v[:, :, t:t + 1])), to_dev(np.ascontiguousarray(qs[s])),
                        out, 3, ws)
        assert cache.len == t + 1
        if s % 4 == 0 or s == steps - 1:
            ocfg_t = O.CacheConfig(2, 2, 4, 128, T + 8, n_sink, n_recent, "bf16", "hybrid", (3, 2), (2, 4))
            oc = O.build_cache(k[:, :, :t + 1], v[:, :, :t + 1], ocfg_t)
            ok, err, bound = within_tol(out.cpu().numpy(), O.decode(oc, qs[s]))
            worst = max(worst, err / bound)
            assert ok, (s, err, bound)
    say(f"    worst error / bound over the steps: {worst:.3e}")
    kvq.cache_check(cache)
    assert_regions_equal(cache, O.build_cache(k, v, ocfg))


def test_decode_step_unfused_paths():
    # several tokens at once, and tokens that land in the sink, take the append + decode path
    say("case: decode_step with n_new > 1 and sink tokens")
    rng = np.random.default_rng(90)
    ocfg = O.CacheConfig(1, 2, 2, 64, 300, 6, 16, "fp16", "asym", (2, 4), (4, 2))
    k = workloads.random_raw16(rng, (1, 2, 120, 64), "fp16")
    v = workloads.random_raw16(rng, (1, 2, 120, 64), "fp16")
    q = workloads.random_raw16(rng, (1, 2, 64), "fp16")
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    out = torch.empty((1, 2, 64), dtype=torch.float32, device=DEV)
    ws = torch.zeros(kvq.decode_workspace_bytes(cache, 2), dtype=torch.uint8, device=DEV)
    t = 0
    for n in (1, 1, 3, 1, 1, 1, 40, 1, 72):
        kvq.decode_step(cache, to_dev(np.ascontiguousarray(k[:, :, t:t + n])),
                        to_dev(np.ascontiguousarray(v[:, :, t:t + n])), to_dev(q), out, 2, ws)
        t += n
        oc = O.build_cache(k[:, :, :t], v[:, :, :t], ocfg)
        ok, err, bound = within_tol(out.cpu().numpy(), O.decode(oc, q))
        assert ok, (t, err, bound)
    assert_regions_equal(cache, O.build_cache(k, v, ocfg))


def test_explicit_scale():
    rng = np.random.default_rng(40)
    ocfg = O.CacheConfig(1, 1, 4, 128, 500, 4, 64, "bf16", "asym", (3,), (3,))
    k = workloads.random_raw16(rng, (1, 1, 500, 128), "bf16")
    v = workloads.random_raw16(rng, (1, 1, 500, 128), "bf16")
    q = workloads.random_raw16(rng, (1, 4, 128), "bf16")
    oc = O.build_cache(k, v, ocfg)
    cache = gpu_cache(ocfg, k, v)
    want = O.decode(oc, q, scale=0.5)
    ok, err, bound = within_tol(gpu_decode(cache, q, 4, scale=0.5), want)
    assert ok, (err, bound)


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("quant", ["asym", "hybrid"])
def test_calibrate_matches_oracle(axis, quant):
    say(f"case: calibrate axis={axis} quant={quant}")
    rng = np.random.default_rng(50 + axis)
    x = workloads.random_raw16(rng, (3, 256, 128), "bf16")
    xo = x.copy()
    # an outlier-channel head and an exactly representable head
    xf = O.widen16(x, "bf16")
    xf[1, :, :4] *= 8
    xf[2] = 0.5
    x = workloads.to_raw16(xf, "bf16")
    del xo
    hyb = quant == "hybrid"
    Ds = [O.calib_distortion(x[h], "bf16", axis, 2, 8, hyb) for h in range(3)]
    ref = O.fit_heads(list(range(2, 9)), Ds)
    got = kvq.calibrate_fit(to_dev(x), "bf16", axis, kvq.QUANT_HYBRID if hyb else kvq.QUANT_ASYM, 2, 8)
    for g, r in zip(got, ref):
        assert np.allclose(np.array(g), r, rtol=1e-13, atol=0), (g, r)
    assert got[0][2] == 0.0 and got[1][2] == 4.0


@pytest.mark.parametrize("axis", [0, 1])
def test_calibrate_fit_fallback_for_poor_fits(axis):
    """The RateQuant page's fallback (section W.10) through the library: two heads of plain
    N(0,1) data fit well; a head of values a few bf16 ulps apart (its scale rounds to zero at
    the high widths, so D(b) grows with b) fits beta <= 1 and takes the well-fitted heads'
    mean; a head of four levels plus small noise (exact grids at the even widths only) fits
    with R^2 < 0.96 and takes min(beta, that mean). alpha, beta and R^2 match the oracle's,
    and the allocation from them is the oracle's, with a decision margin far above the
    calibration's rounding."""
    say(f"case: calibration fallback heads, axis={axis}")
    rng = np.random.default_rng(55)
    n, D = 512, 128
    normal = [rng.normal(size=(n, D)) for _ in range(2)]
    tiny = 2.0 ** -13 + rng.integers(0, 5, size=(n, D)) * 2.0 ** -20
    zigzag = rng.integers(0, 4, size=(n, D)) / 3.0 + rng.normal(0.0, 1e-3, size=(n, D))
    x = workloads.to_raw16(np.stack(normal + [tiny, zigzag]).astype(np.float32), "bf16")
    Ds = [O.calib_distortion(x[h], "bf16", axis, 2, 8, False) for h in range(4)]
    raw_fits = [O.fit_one(list(range(2, 9)), list(d)) for d in Ds]
    assert raw_fits[2][1] <= 1.0 and raw_fits[3][2] < 0.96          # the crafted heads are poor fits
    ref = O.fit_heads(list(range(2, 9)), Ds)
    bbar = (ref[1][0] + ref[1][1]) / 2
    assert ref[1][2] == bbar and ref[1][3] == min(raw_fits[3][1], bbar)
    got = kvq.calibrate_fit(to_dev(x), "bf16", axis, kvq.QUANT_ASYM, 2, 8)
    for g, r in zip(got, ref):
        assert np.allclose(np.array(g), r, rtol=1e-13, atol=0), (g, r)
    w = [1.0, 0.7, 1.3, 2.0]
    want = O.allocate_greedy(list(ref[0]), list(ref[1]), w, 12, 2, 4)
    bits, _ = kvq.allocate_bits(got[0], got[1], w, 12, 2, 4)
    assert kvq.allocation_margin(ref[0], ref[1], w, want, 2, 4) > 1e-9
    assert bits == want


@pytest.mark.parametrize("quant,dtype", [("asym", "fp16"), ("hybrid", "fp16"), ("hybrid", "bf16")])
def test_edge_groups_constant_zero_negative_zero_and_range_limit(quant, dtype):
    """Groups the quantizer treats specially, through append and decode: constant groups and
    all-zero groups (s = 0, every code 0), groups of -0 and groups whose minimum is -0 (the
    zero is stored as +0), and groups reaching the input limit |x| = 2^14 (largest s and z).
    Keys are groups of 32 channels of a token, values groups of 32 tokens of a channel (InnerQ
    page, abstract and "Core claim"); hybrid caches also choose the symmetric variant per group
    (technique (i)). The logical content must match the oracle bit for bit (zeros compared
    as bits, so -0 and +0 differ) and decode must stay within tolerance per KV head."""
    say(f"case: edge groups {quant} {dtype}")
    B, H, D, T, ns, nr = 1, 3, 128, 400, 2, 32
    kb, vb = (2, 3, 8), (2, 4, 8)
    ocfg = O.CacheConfig(B, H, H, D, 512, ns, nr, dtype, quant, kb, vb)
    rng = np.random.default_rng(58)
    k = O.widen16(workloads.random_raw16(rng, (B, H, T, D), dtype), dtype)
    v = O.widen16(workloads.random_raw16(rng, (B, H, T, D), dtype), dtype)
    k[:, :, 40, 0:32] = 1.5                                   # constant key group
    k[:, :, 41, 32:64] = 0.0                                  # all +0
    k[:, :, 42, 64:96] = -0.0                                 # all -0
    k[:, :, 43, 96:128] = np.abs(k[:, :, 43, 96:128])
    k[:, :, 43, 100] = -0.0                                   # minimum is -0
    k[:, :, 44, 0:32] = -2.0                                  # negative constant
    k[:, 1, 50, 0:32] = np.where(np.arange(32) % 2, 16384.0, -16384.0)   # the input limit
    k[:, 1, 51, 32:64] = 16384.0
    k[:, 1, 52] = np.clip(np.round(k[:, 1, 52] * 5000.0), -16384.0, 16384.0)
    blk = slice(ns + 32, ns + 64)                             # value block 1 of the body
    v[:, :, blk, 5] = 0.75                                    # constant value group
    v[:, :, blk, 6] = 0.0
    v[:, :, blk, 7] = -0.0
    v[:, :, blk, 8] = np.abs(v[:, :, blk, 8])
    v[:, :, ns + 40, 8] = -0.0
    v[:, 2, ns + 64:ns + 96, 9] = np.where(np.arange(32) % 3, 16384.0, -16384.0)
    v[:, 2, ns + 96:ns + 128, 10] = -16384.0
    kr, vr = workloads.to_raw16(k, dtype), workloads.to_raw16(v, dtype)
    q = O.widen16(workloads.random_raw16(rng, (B, H, D), dtype), dtype)
    q[:, 1] *= 1e-4                                           # keep head 1's scores moderate
    qr = workloads.to_raw16(q, dtype)
    oc = O.build_cache(kr, vr, ocfg)
    for h in range(H):                                        # the oracle took the special paths
        e = oc.heads[h]
        t = lambda tok: tok - ns                               # body index of a sequence token
        assert e["k_s"][0, t(40), 0] == 0 and e["k_s"][0, t(41), 1] == 0 and e["k_s"][0, t(42), 2] == 0
        assert e["k_z"][0, t(42), 2].view(np.uint16) == 0 and e["k_z"][0, t(43), 3].view(np.uint16) == 0
        assert e["v_s"][0, 1, 5] == 0 and e["v_z"][0, 1, 7].view(np.uint16) == 0
    assert np.abs(O.widen16(kr[0, 1], dtype)).max() == 16384.0
    cache = gpu_cache(ocfg, kr, vr, chunks=[100, 1, 299])     # cache_check: no range flag at 2^14
    assert_regions_equal(cache, oc)
    want = O.decode(oc, qr)
    for ns_ in (1, 3):
        got = gpu_decode(cache, qr, ns_)
        for h in range(H):
            ok, err, bound = within_tol(got[:, h], want[:, h])
            say(f"    n_splits={ns_} head {h}: max err {err:.3e} (bound {bound:.3e})")
            assert ok


def test_range_flag_on_append_and_calibrate():
    say("case: out-of-range inputs")
    rng = np.random.default_rng(60)
    ocfg = O.CacheConfig(1, 2, 2, 64, 200, 1, 8, "fp16", "asym", (2, 16), (2, 16))
    k = O.widen16(workloads.random_raw16(rng, (1, 2, 100, 64), "fp16"), "fp16")
    k[0, 1, 50, 5] = 30000.0          # 16-bit head: allowed
    kr = workloads.to_raw16(k, "fp16")
    v = workloads.random_raw16(rng, (1, 2, 100, 64), "fp16")
    gpu_cache(ocfg, kr, v)            # cache_check passes inside
    k[0, 0, 60, 5] = 30000.0          # quantized head: flagged
    kr = workloads.to_raw16(k, "fp16")
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    kvq.append(cache, to_dev(kr), to_dev(v))
    with pytest.raises(kvq.KvqError) as e:
        kvq.cache_check(cache)
    assert e.value.status == -4
    with pytest.raises(kvq.KvqError) as e:
        kvq.calibrate_fit(to_dev(np.ascontiguousarray(kr[0])), "fp16", 0)
    assert e.value.status == -4


def test_abi_errors_enqueue_nothing():
    ocfg = O.CacheConfig(1, 1, 1, 64, 64, 1, 8, "fp16", "asym", (2,), (2,))
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    k = torch.zeros((1, 1, 65, 64), dtype=torch.int16, device=DEV)
    with pytest.raises(kvq.KvqError) as e:
        kvq.append(cache, k, k)
    assert e.value.status == -3 and cache.len == 0
    q = torch.zeros((1, 1, 64), dtype=torch.int16, device=DEV)
    out = torch.zeros((1, 1, 64), dtype=torch.float32, device=DEV)
    ws = torch.zeros(1 << 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attention(cache, q, out, 1, ws)       # empty cache
    assert e.value.status == -1


# ------------------------------------------------------------------------------------------
# Per-channel key normalization: norms from the first append, normalized body keys, the norms
# folded into the query at decode

def outlier_keys(rng, shape, dtype, n_out=4, factor=8.0):
    """N(0, 1) keys with n_out channels per (row, head) scaled by factor."""
    x = workloads.random_raw16(rng, shape, dtype)
    xf = O.widen16(x, dtype).copy()
    for b in range(shape[0]):
        for h in range(shape[1]):
            xf[b, h, :, rng.choice(shape[3], size=n_out, replace=False)] *= np.float32(factor)
    return workloads.to_raw16(xf, dtype)


@pytest.mark.parametrize("chunks", [[300], [37, 1, 100, 62, 100], [8] + [1] * 60 + [93]],
                         ids=["bulk", "ragged", "one-token"])
def test_key_norm_appends(chunks):
    say(f"case: key norm, appends {chunks[:4]}...")
    rng = np.random.default_rng(200 + len(chunks))
    T = sum(chunks)
    ocfg = O.CacheConfig(2, 2, 4, 64, T + 5, 3, 40, "bf16", "hybrid", (3, 2), (2, 4), key_norm=True)
    k = outlier_keys(rng, (2, 2, T, 64), "bf16")
    v = workloads.random_raw16(rng, (2, 2, T, 64), "bf16")
    q = workloads.random_raw16(rng, (2, 4, 64), "bf16")
    oc = O.build_cache(k, v, ocfg, norm_tokens=chunks[0])
    cache = gpu_cache(ocfg, k, v, chunks=chunks)
    assert_regions_equal(cache, oc)
    check_decode(cache, oc, q, splits=(1, 3, 8))


def test_key_norm_mixed_widths_d128():
    say("case: key norm, 16-bit heads + every width 2..8, fp16 hybrid, D=128")
    rng = np.random.default_rng(210)
    T = 900
    kb = (16, 2, 3, 4, 5, 6, 7, 8)
    vb = (8, 7, 16, 5, 4, 3, 2, 16)
    ocfg = O.CacheConfig(1, 8, 16, 128, T, 4, 64, "fp16", "hybrid", kb, vb, key_norm=True)
    k = outlier_keys(rng, (1, 8, T, 128), "fp16")
    v = workloads.random_raw16(rng, (1, 8, T, 128), "fp16")
    q = workloads.random_raw16(rng, (1, 16, 128), "fp16")
    oc = O.build_cache(k, v, ocfg, norm_tokens=500)
    cache = gpu_cache(ocfg, k, v, chunks=[500, 1, 399])
    assert_regions_equal(cache, oc)
    check_decode(cache, oc, q, splits=(1, 5, 16))


def test_key_norm_full_grid_asym():
    # every body path in one launch with normalized keys, asymmetric quantizer, bf16
    say("case: key norm, B=4 x 8 KV heads, all body paths, asym")
    rng = np.random.default_rng(211)
    T = 1100
    kb = (2, 3, 4, 16, 5, 2, 3, 4)
    vb = (2, 3, 4, 16, 2, 8, 4, 3)
    ocfg = O.CacheConfig(4, 8, 32, 128, T, 4, 64, "bf16", "asym", kb, vb, key_norm=True)
    k = outlier_keys(rng, (4, 8, T, 128), "bf16")
    v = workloads.random_raw16(rng, (4, 8, T, 128), "bf16")
    q = workloads.random_raw16(rng, (4, 32, 128), "bf16")
    oc = O.build_cache(k, v, ocfg)
    cache = gpu_cache(ocfg, k, v)
    assert_regions_equal(cache, oc)
    check_decode(cache, oc, q, splits=(15, 32))


@pytest.mark.parametrize("first", [8, 90])
def test_key_norm_decode_steps(first):
    # decode_step from an empty cache: the first call (several tokens) sets the norms, the
    # single-token steps after it take the fused path across several flushes
    say(f"case: key norm decode_step sequence, first append {first}")
    rng = np.random.default_rng(220 + first)
    steps = 75
    T = first + steps
    ocfg = O.CacheConfig(2, 2, 4, 128, T + 8, 4, 40, "bf16", "hybrid", (3, 2), (2, 4), key_norm=True)
    k = outlier_keys(rng, (2, 2, T, 128), "bf16")
    v = workloads.random_raw16(rng, (2, 2, T, 128), "bf16")
    qs = workloads.random_raw16(rng, (steps + 1, 2, 4, 128), "bf16")
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    out = torch.empty((2, 4, 128), dtype=torch.float32, device=DEV)
    ws = torch.zeros(kvq.decode_workspace_bytes(cache, 3), dtype=torch.uint8, device=DEV)
    t, worst = 0, 0.0
    for s, n in enumerate([first] + [1] * steps):
        kvq.decode_step(cache, to_dev(np.ascontiguousarray(k[:, :, t:t + n])),
                        to_dev(np.ascontiguousarray(v[:, :, t:t + n])), to_dev(np.ascontiguousarray(qs[s])),
                        out, 3, ws)
        t += n
        assert cache.len == t
        if s % 4 == 0 or t == T:
            oc = O.build_cache(k[:, :, :t], v[:, :, :t], ocfg, norm_tokens=first)
            ok, err, bound = within_tol(out.cpu().numpy(), O.decode(oc, qs[s]))
            worst = max(worst, err / bound)
            assert ok, (s, err, bound)
    say(f"    worst error / bound over the steps: {worst:.3e}")
    kvq.cache_check(cache)
    assert_regions_equal(cache, O.build_cache(k, v, ocfg, norm_tokens=first))


# ------------------------------------------------------------------------------------------
# Multi-token (causal) decode: the query rows of a KV head are its G query heads x Q tokens

@pytest.mark.parametrize("G,Q,D,T,dtype", [(1, 4, 128, 1333, "bf16"), (2, 2, 128, 700, "fp16"),
                                           (1, 3, 64, 300, "fp16"), (1, 4, 128, 21, "bf16"),
                                           (4, 1, 128, 500, "bf16")])
def test_multi_token_decode(G, Q, D, T, dtype):
    say(f"case: multi-token decode G={G} Q={Q} D={D} T={T} {dtype}")
    rng = np.random.default_rng(400 + 10 * G + Q + T)
    ocfg = O.CacheConfig(2, 3, 3 * G, D, T + 8, 4, 40, dtype, "hybrid", (3, 2, 16), (2, 4, 3))
    k = workloads.random_raw16(rng, (2, 3, T, D), dtype, 2.0)
    v = workloads.random_raw16(rng, (2, 3, T, D), dtype)
    q = workloads.random_raw16(rng, (2, Q, 3 * G, D), dtype)
    oc = O.build_cache(k, v, ocfg)
    cache = gpu_cache(ocfg, k, v)
    want = O.decode_multi(oc, q)
    qd = to_dev(q)
    for ns in (1, 3, 16):
        out = torch.empty((2, Q, 3 * G, D), dtype=torch.float32, device=DEV)
        ws = torch.zeros(kvq.decode_multi_workspace_bytes(cache, ns, Q), dtype=torch.uint8, device=DEV)
        kvq.decode_multi(cache, qd, out, ns, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for i in range(Q):  # each query token against its own output scale
            ok, err, bound = within_tol(got[:, i], want[:, i])
            assert ok, (ns, i, err, bound)
        say(f"    n_splits={ns}: every query token within tolerance")
        if Q == 1:
            ref = gpu_decode(cache, q[:, 0], ns)
            assert np.array_equal(got[:, 0], ref)


def test_multi_token_decode_key_norm():
    # the folded key norms apply to every (query token, head) row
    say("case: multi-token decode with key normalization, G=1 Q=4")
    rng = np.random.default_rng(460)
    T, D = 900, 128
    ocfg = O.CacheConfig(2, 2, 2, D, T, 4, 40, "bf16", "hybrid", (3, 2), (2, 4), key_norm=True)
    k = outlier_keys(rng, (2, 2, T, D), "bf16")
    v = workloads.random_raw16(rng, (2, 2, T, D), "bf16")
    q = workloads.random_raw16(rng, (2, 4, 2, D), "bf16")
    oc = O.build_cache(k, v, ocfg, norm_tokens=300)
    cache = gpu_cache(ocfg, k, v, chunks=[300, T - 300])
    want = O.decode_multi(oc, q)
    out = torch.empty((2, 4, 2, D), dtype=torch.float32, device=DEV)
    ws = torch.zeros(kvq.decode_multi_workspace_bytes(cache, 6, 4), dtype=torch.uint8, device=DEV)
    kvq.decode_multi(cache, to_dev(q), out, 6, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for i in range(4):
        ok, err, bound = within_tol(got[:, i], want[:, i])
        assert ok, (i, err, bound)


def test_multi_token_decode_rejects():
    ocfg = O.CacheConfig(1, 2, 4, 64, 400, 2, 0, "bf16", "asym", (2, 2), (2, 2))
    rng = np.random.default_rng(450)
    k = workloads.random_raw16(rng, (1, 2, 300, 64), "bf16")
    cache = gpu_cache(ocfg, k, k)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    q9 = torch.zeros((1, 9, 4, 64), dtype=torch.int16, device=DEV)
    out9 = torch.zeros((1, 9, 4, 64), dtype=torch.float32, device=DEV)
    with pytest.raises(kvq.KvqError) as e:  # 2 query heads per KV head x 9 tokens > 16 rows
        kvq.decode_multi(cache, q9, out9, 2, ws)
    assert e.value.status == -5
    # n_recent = 0: after a flush the window holds fewer than Q - 1 tokens
    ocfg1 = O.CacheConfig(1, 2, 2, 64, 400, 2, 0, "bf16", "asym", (2, 2), (2, 2))
    cache1 = gpu_cache(ocfg1, k[:, :, :290], k[:, :, :290])  # body 288, window 0
    q4 = torch.zeros((1, 4, 2, 64), dtype=torch.int16, device=DEV)
    out4 = torch.zeros((1, 4, 2, 64), dtype=torch.float32, device=DEV)
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_multi(cache1, q4, out4, 2, ws)
    assert e.value.status == -5


# The 16-row tile: 5 to 16 query rows per KV head (GQA heads x query tokens) in one pass.
# Every width 2..8 and 16-bit sides on either side, windows only, several split counts.
DENSE_CASES = [
    # G, Q, D, T, dtype, quant, k_bits, v_bits
    (4, 4, 128, 1333, "bf16", "hybrid", (3, 2, 4), (2, 3, 4)),
    (4, 2, 128, 700, "fp16", "asym", (2, 4, 3), (4, 2, 2)),
    (2, 3, 64, 300, "fp16", "hybrid", (3, 16, 2), (2, 4, 16)),
    (1, 16, 128, 500, "bf16", "asym", (5, 6, 7), (8, 5, 6)),
    (4, 3, 128, 900, "bf16", "hybrid", (8, 7, 16), (7, 16, 3)),
    (4, 4, 64, 21, "fp16", "asym", (2, 3, 4), (4, 3, 2)),     # window tokens only
    (2, 8, 128, 2100, "fp16", "hybrid", (16, 3, 2), (16, 2, 5)),
]


@pytest.mark.parametrize("G,Q,D,T,dtype,quant,kb,vb", DENSE_CASES,
                         ids=[f"G{c[0]}Q{c[1]}D{c[2]}T{c[3]}-{c[5]}" for c in DENSE_CASES])
def test_multi_token_decode_16_row_tile(G, Q, D, T, dtype, quant, kb, vb):
    say(f"case: 16-row multi-token decode G={G} Q={Q} D={D} T={T} {dtype} {quant} K{kb} V{vb}")
    assert 4 < G * Q <= 16
    rng = np.random.default_rng(900 + 10 * G + Q + T)
    ocfg = O.CacheConfig(2, 3, 3 * G, D, T + 8, 4, 40, dtype, quant, kb, vb)
    k = workloads.random_raw16(rng, (2, 3, T, D), dtype, 2.0)
    v = workloads.random_raw16(rng, (2, 3, T, D), dtype)
    q = workloads.random_raw16(rng, (2, Q, 3 * G, D), dtype)
    oc = O.build_cache(k, v, ocfg)
    cache = gpu_cache(ocfg, k, v)
    want = O.decode_multi(oc, q)
    qd = to_dev(q)
    for ns in (1, 3, 16):
        out = torch.full((2, Q, 3 * G, D), float("nan"), dtype=torch.float32, device=DEV)
        ws = torch.zeros(kvq.decode_multi_workspace_bytes(cache, ns, Q), dtype=torch.uint8, device=DEV)
        kvq.decode_multi(cache, qd, out, ns, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        worst = 0.0
        for i in range(Q):  # each query token against its own output scale
            ok, err, bound = within_tol(got[:, i], want[:, i])
            worst = max(worst, err / bound)
            assert ok, (ns, i, err, bound)
        say(f"    n_splits={ns}: worst error / bound {worst:.3e}")


def test_multi_token_decode_16_row_tile_key_norm_and_paged():
    # key norms folded into all 16 rows; a paged twin gives bit-identical outputs
    say("case: 16-row multi-token decode, key normalization, contiguous and paged")
    rng = np.random.default_rng(930)
    G, Q, T, D = 4, 4, 2500, 128
    ocfg = O.CacheConfig(2, 2, 2 * G, D, T, 4, 40, "bf16", "hybrid", (3, 2), (2, 4), key_norm=True)
    k = outlier_keys(rng, (2, 2, T, D), "bf16")
    v = workloads.random_raw16(rng, (2, 2, T, D), "bf16")
    q = workloads.random_raw16(rng, (2, Q, 2 * G, D), "bf16")
    oc = O.build_cache(k, v, ocfg, norm_tokens=700)
    cache = gpu_cache(ocfg, k, v, chunks=[700, T - 700])
    paged, _ = _paged_twin(ocfg, rng)
    for a, n in ((0, 700), (700, T - 700)):
        kvq.append(paged, to_dev(k[:, :, a:a + n]), to_dev(v[:, :, a:a + n]))
    torch.cuda.synchronize()
    kvq.cache_check(paged)
    want = O.decode_multi(oc, q)
    outs = []
    for c in (cache, paged):
        out = torch.empty((2, Q, 2 * G, D), dtype=torch.float32, device=DEV)
        ws = torch.zeros(kvq.decode_multi_workspace_bytes(c, 5, Q), dtype=torch.uint8, device=DEV)
        kvq.decode_multi(c, to_dev(q), out, 5, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    for i in range(Q):
        ok, err, bound = within_tol(outs[0][:, i], want[:, i])
        assert ok, (i, err, bound)


# ------------------------------------------------------------------------------------------
# Ragged batches: rows of different lengths, each appended and decoded on its own schedule

def _ragged_input(chunks_k, chunks_v, n_max, H, D):
    """[B][H][n_max][D] inputs holding row b's chunk in its first slots; the unused slots hold
    garbage that must never be read."""
    B = len(chunks_k)
    rng = np.random.default_rng(n_max + 7 * B)
    k = rng.integers(0, 1 << 16, size=(B, H, n_max, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(B, H, n_max, D), dtype=np.uint16)
    for b in range(B):
        n = chunks_k[b].shape[1]
        k[b, :, :n] = chunks_k[b]
        v[b, :, :n] = chunks_v[b]
    return k, v


def _row_cfg(ocfg):
    return O.CacheConfig(1, ocfg.n_kv, ocfg.n_q, ocfg.head_dim, ocfg.capacity, ocfg.n_sink, ocfg.n_recent,
                         ocfg.dtype, ocfg.quant, ocfg.k_bits, ocfg.v_bits, key_norm=ocfg.key_norm)


def _check_ragged(cache, ocfg, k_rows, v_rows, lens, first, q, splits):
    outs = {}
    for ns in splits:
        out = torch.empty((ocfg.batch, ocfg.n_q, ocfg.head_dim), dtype=torch.float32, device=DEV)
        ws = torch.zeros(kvq.decode_workspace_bytes(cache, ns), dtype=torch.uint8, device=DEV)
        kvq.decode_ragged(cache, lens, to_dev(q), out, ns, ws)
        torch.cuda.synchronize()
        outs[ns] = out.cpu().numpy()
    for b in range(ocfg.batch):
        T = lens[b]
        oc = O.build_cache(k_rows[b][None, :, :T], v_rows[b][None, :, :T], _row_cfg(ocfg), norm_tokens=first[b])
        assert_regions_equal(cache, oc, rows=[0], map_bh=lambda _b, h, b=b: (b, h))
        want = O.decode(oc, q[b:b + 1])[0]
        for ns, got in outs.items():
            ok, err, bound = within_tol(got[b], want)
            assert ok, (b, T, ns, err, bound)


@pytest.mark.parametrize("key_norm,kb,vb", [(False, (3, 2), (2, 4)), (True, (3, 2), (2, 4)),
                                             (False, (5, 16), (8, 3))], ids=["plain", "key-norm", "wide"])
def test_ragged_appends_and_decode(key_norm, kb, vb):
    say(f"case: ragged appends and decode, key norm {key_norm}, K bits {kb}, V bits {vb}")
    B, H, D, G = 3, 2, 128, 2
    schedule = [[100, 0, 37], [1, 250, 64], [37, 5, 1], [0, 1, 200], [300, 33, 0]]
    totals = [sum(c[b] for c in schedule) for b in range(B)]
    ocfg = O.CacheConfig(B, H, H * G, D, 1200, 4, 40, "bf16", "hybrid", kb, vb, key_norm=key_norm)
    rng = np.random.default_rng(500 + key_norm)
    k_rows = [outlier_keys(rng, (1, H, totals[b], D), "bf16")[0] for b in range(B)]
    v_rows = [workloads.random_raw16(rng, (H, totals[b], D), "bf16") for b in range(B)]
    q = workloads.random_raw16(rng, (B, H * G, D), "bf16")
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    lens, first = [0] * B, [None] * B
    for step, n_new in enumerate(schedule):
        n_max = max(n_new)
        ck = [k_rows[b][:, lens[b]:lens[b] + n_new[b]] for b in range(B)]
        cv = [v_rows[b][:, lens[b]:lens[b] + n_new[b]] for b in range(B)]
        kin, vin = _ragged_input(ck, cv, n_max, H, D)
        kvq.append_ragged(cache, lens, n_new, to_dev(kin), to_dev(vin))
        for b in range(B):
            if first[b] is None and n_new[b] > 0:
                first[b] = n_new[b]
            lens[b] += n_new[b]
        if step in (2, 4):
            _check_ragged(cache, ocfg, k_rows, v_rows, lens, first, q, splits=(1, 5))
            say(f"    after call {step}: lengths {lens}, regions and decode match")
    kvq.cache_check(cache)


def test_ragged_serving_steps():
    # rows prefilled to different lengths, then one token per row per step: the rows flush
    # their 32-token blocks at different steps
    say("case: ragged serving steps")
    B, H, D, G = 4, 2, 64, 2
    pre = [90, 300, 150, 33]
    steps = 40
    ocfg = O.CacheConfig(B, H, H * G, D, 400, 3, 32, "fp16", "asym", (2, 4), (3, 2))
    rng = np.random.default_rng(510)
    k_rows = [workloads.random_raw16(rng, (H, pre[b] + steps, D), "fp16", 2.0) for b in range(B)]
    v_rows = [workloads.random_raw16(rng, (H, pre[b] + steps, D), "fp16") for b in range(B)]
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    lens = [0] * B
    kin, vin = _ragged_input([k[:, :p] for k, p in zip(k_rows, pre)], [v[:, :p] for v, p in zip(v_rows, pre)],
                             max(pre), H, D)
    kvq.append_ragged(cache, lens, pre, to_dev(kin), to_dev(vin))
    lens = list(pre)
    first = list(pre)
    for s_ in range(steps):
        ck = [k_rows[b][:, lens[b]:lens[b] + 1] for b in range(B)]
        cv = [v_rows[b][:, lens[b]:lens[b] + 1] for b in range(B)]
        kin, vin = _ragged_input(ck, cv, 1, H, D)
        kvq.append_ragged(cache, lens, [1] * B, to_dev(kin), to_dev(vin))
        lens = [n + 1 for n in lens]
        if s_ % 8 == 7:
            q = workloads.random_raw16(rng, (B, H * G, D), "fp16")
            _check_ragged(cache, ocfg, k_rows, v_rows, lens, first, q, splits=(3,))
            say(f"    step {s_}: lengths {lens} match")


def test_ragged_rejects():
    ocfg = O.CacheConfig(2, 1, 1, 64, 100, 2, 8, "bf16", "asym", (2,), (2,))
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    k = torch.zeros((2, 1, 4, 64), dtype=torch.int16, device=DEV)
    with pytest.raises(kvq.KvqError) as e:  # n_new above the input's slots
        kvq.append_ragged(cache, [0, 0], [5, 1], k, k)
    assert e.value.status == -1
    with pytest.raises(kvq.KvqError) as e:  # past the capacity
        kvq.append_ragged(cache, [98, 0], [4, 1], k, k)
    assert e.value.status == -3
    kvq.append_ragged(cache, [0, 0], [4, 0], k, k)
    q = torch.zeros((2, 1, 64), dtype=torch.int16, device=DEV)
    out = torch.zeros((2, 1, 64), dtype=torch.float32, device=DEV)
    ws = torch.zeros(1 << 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(kvq.KvqError) as e:  # row 1 is empty
        kvq.decode_ragged(cache, [4, 0], q, out, 1, ws)
    assert e.value.status == -1
    big = O.CacheConfig(65, 1, 1, 64, 100, 2, 8, "bf16", "asym", (2,), (2,))
    cache65 = kvq.KVCache(lib_cfg(kvq, big), device=DEV)
    k65 = torch.zeros((65, 1, 1, 64), dtype=torch.int16, device=DEV)
    with pytest.raises(kvq.KvqError) as e:  # the last row (in the second row group) past the capacity
        kvq.append_ragged(cache65, [0] * 64 + [100], [1] * 65, k65, k65)
    assert e.value.status == -3


# ------------------------------------------------------------------------- paged caches ---

def assert_paged_regions_equal(cache, oc, table, stride):
    """Gather each (row, head)'s body regions out of the pools through `table`, read them and
    the per-row regions through the cache format, and compare the logical content with the
    oracle's."""
    cfg = oc.cfg
    blob = cache.blob.cpu().numpy()
    rt = cache.region_table().astype(np.int64)
    ccfg = lib_cfg(kvq, cfg)
    for b in range(cfg.batch):
        for h in range(cfg.n_kv):
            tb = F.tile_bytes(cfg, h)
            regions = []
            for r in range(F.N_REGIONS):
                size = kvq.region_offset(ccfg, b, h, r)[1]
                if r <= 4:
                    base = int(rt[b, h, r])
                    got = np.concatenate([blob[base + int(table[b][t]) * tb[r]:][:tb[r]] for t in range(stride)])
                    regions.append(got[:size])
                else:
                    regions.append(blob[int(rt[b, h, r]):int(rt[b, h, r]) + size])
            got = F.decode_head(regions, cfg, h, oc.T)
            F.assert_content_equal(got, F.oracle_head_content(oc, b, h), f"row {b} head {h}")


@pytest.mark.parametrize("kb,vb,quant,dtype,D", [((3, 2, 4), (2, 4, 3), "hybrid", "bf16", 128),
                                                 ((16, 5, 2), (7, 16, 16), "asym", "fp16", 64)])
def test_paged_cache(kb, vb, quant, dtype, D):
    say(f"case: paged cache K bits {kb}, V bits {vb}, {quant}, {dtype}, D {D}")
    B, H, G, T = 3, len(kb), 2, 1100
    ocfg = O.CacheConfig(B, H, H * G, D, 1200, 4, 40, dtype, quant, kb, vb)
    rng = np.random.default_rng(700 + D)
    k = workloads.random_raw16(rng, (B, H, T, D), dtype, 3.0)
    v = workloads.random_raw16(rng, (B, H, T, D), dtype)
    q = workloads.random_raw16(rng, (B, H * G, D), dtype)
    oc = O.build_cache(k, v, ocfg)
    ref = gpu_cache(ocfg, k, v, chunks=[300, 1, 64, 735])
    # a pool larger than the rows need, its pages dealt to (row, tile) in a shuffled order
    stride = (O.body_len(1200, 4, 40) // 32 + 1) // 2
    n_pages = B * stride + 7
    perm = rng.permutation(n_pages)[:B * stride].astype(np.int32)
    table = perm.reshape(B, stride)
    cache = kvq.cache_init_paged(lib_cfg(kvq, ocfg), n_pages, device=DEV)
    for b in range(B):
        cache.map_pages(b, 0, table[b, :5].tolist())
        cache.map_pages(b, 5, table[b, 5:].tolist())
    pos = 0
    for n in [300, 1, 64, 735]:
        kvq.append(cache, to_dev(k[:, :, pos:pos + n]), to_dev(v[:, :, pos:pos + n]))
        pos += n
    torch.cuda.synchronize()
    kvq.cache_check(cache)
    assert_paged_regions_equal(cache, oc, table, stride)
    say("    pooled regions gathered through the page table match the oracle")
    check_decode(cache, oc, q, splits=(1, 5))
    for ns in (1, 5):
        assert np.array_equal(gpu_decode(cache, q, ns), gpu_decode(ref, q, ns)), ns
    say("    paged decode equals the contiguous cache's decode bit for bit")


def test_page_given_to_two_tiles_is_rejected():
    """kvq_cache_map_pages refuses any call after which one page would hold two tiles, within
    the call, across calls or across rows, and then writes nothing; remapping a tile, freeing a
    page and giving it to another tile is allowed."""
    ocfg = O.CacheConfig(2, 1, 1, 64, 400, 2, 32, "fp16", "asym", (2,), (2,))
    cache = kvq.cache_init_paged(lib_cfg(kvq, ocfg), 8, device=DEV)
    cache.map_pages(0, 0, [5, 7])
    cache.map_pages(0, 0, [5, 7])  # the same mapping again
    for row, first, pages in ((1, 0, [5]), (0, 2, [7]), (1, 0, [3, 3])):
        with pytest.raises(kvq.KvqError) as e:
            cache.map_pages(row, first, pages)
        assert e.value.status == -1
    cache.map_pages(1, 0, [6])  # row 1 tile 0 was left unmapped by the rejected calls
    cache.map_pages(0, 0, [2, -1])  # frees pages 5 and 7
    cache.map_pages(1, 1, [5, 7])
    with pytest.raises(kvq.KvqError) as e:
        cache.map_pages(0, 1, [6])
    assert e.value.status == -1


def test_paged_unmapped_tile_is_flagged():
    say("case: paged cache append into an unmapped tile")
    ocfg = O.CacheConfig(1, 1, 1, 64, 400, 2, 8, "bf16", "asym", (2,), (3,))
    rng = np.random.default_rng(710)
    k = workloads.random_raw16(rng, (1, 1, 300, 64), "bf16")
    v = workloads.random_raw16(rng, (1, 1, 300, 64), "bf16")
    cache = kvq.cache_init_paged(lib_cfg(kvq, ocfg), 8, device=DEV)
    cache.map_pages(0, 0, [3, 1])  # tiles 0 and 1: body tokens 0..127
    kvq.append(cache, to_dev(k[:, :, :100]), to_dev(v[:, :, :100]))
    torch.cuda.synchronize()
    kvq.cache_check(cache)  # body 64 tokens: tile 0 only
    kvq.append(cache, to_dev(k[:, :, 100:]), to_dev(v[:, :, 100:]))
    torch.cuda.synchronize()
    with pytest.raises(kvq.KvqError, match="ERR_PAGE"):
        kvq.cache_check(cache)
    with pytest.raises(kvq.KvqError, match="ERR_ARG"):
        cache.map_pages(0, 0, [8])
    with pytest.raises(kvq.KvqError, match="ERR_ARG"):
        cache.map_pages(0, (O.body_len(400, 2, 8) // 32 + 1) // 2, [0])
    with pytest.raises(kvq.KvqError, match="ERR_ARG.*two tiles"):
        cache.map_pages(0, 0, [5, 5])


def test_paged_decode_of_an_unmapped_tile_is_flagged():
    # every tile mapped and appended, then one unmapped: decode (single query and the 16-row
    # multi-token tile) still reads in bounds, and the sticky flag reports the unmapped read
    say("case: paged decode over an unmapped tile")
    ocfg = O.CacheConfig(1, 2, 8, 128, 700, 4, 40, "bf16", "asym", (3, 2), (2, 3))
    rng = np.random.default_rng(712)
    T = 600
    k = workloads.random_raw16(rng, (1, 2, T, 128), "bf16")
    v = workloads.random_raw16(rng, (1, 2, T, 128), "bf16")
    for multi in (False, True):
        cache, table = _paged_twin(ocfg, rng)
        kvq.append(cache, to_dev(k), to_dev(v))
        q = workloads.random_raw16(rng, (1, 8, 128), "bf16")
        gpu_decode(cache, q, 3)
        kvq.cache_check(cache)  # all mapped: clean
        cache.map_pages(0, 2, [-1])
        if multi:
            qm = workloads.random_raw16(rng, (1, 4, 8, 128), "bf16")
            out = torch.empty((1, 4, 8, 128), dtype=torch.float32, device=DEV)
            ws = torch.zeros(kvq.decode_multi_workspace_bytes(cache, 3, 4), dtype=torch.uint8, device=DEV)
            kvq.decode_multi(cache, to_dev(qm), out, 3, ws)
        else:
            gpu_decode(cache, q, 3)
        torch.cuda.synchronize()
        with pytest.raises(kvq.KvqError, match="ERR_PAGE"):
            kvq.cache_check(cache)


def _paged_twin(ocfg, rng, extra_pages=9):
    """A paged cache for ocfg with every tile of every row mapped to a page dealt from a pool
    in shuffled order; returns (cache, table)."""
    stride = (O.body_len(ocfg.capacity, ocfg.n_sink, ocfg.n_recent) // 32 + 1) // 2
    n_pages = ocfg.batch * stride + extra_pages
    table = rng.permutation(n_pages)[:ocfg.batch * stride].astype(np.int32).reshape(ocfg.batch, stride)
    cache = kvq.cache_init_paged(lib_cfg(kvq, ocfg), n_pages, device=DEV)
    for b in range(ocfg.batch):
        cache.map_pages(b, 0, table[b].tolist())
    return cache, table


@pytest.mark.parametrize("key_norm", [False, True], ids=["plain", "key-norm"])
def test_ragged_batch_beyond_one_row_group(key_norm):
    """Ragged calls on 150 rows (row groups of 64, 64 and 22 inside the library): contiguous and
    paged caches agree bit for bit, the logical content of rows on either side of each group
    boundary matches the oracle, and every row's decode matches the oracle's one-row cache."""
    say(f"case: ragged batch of 150 rows (three row groups), key norm {key_norm}")
    rng = np.random.default_rng(740 + key_norm)
    B, H, D = 150, 1, 64
    ocfg = O.CacheConfig(B, H, 2 * H, D, 260, 2, 32, "fp16", "hybrid", (3,), (2,), key_norm=key_norm)
    k = workloads.random_raw16(rng, (B, H, 260, D), "fp16", 2.0)
    v = workloads.random_raw16(rng, (B, H, 260, D), "fp16")
    q = workloads.random_raw16(rng, (B, 2 * H, D), "fp16")
    ref = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    paged, _ = _paged_twin(ocfg, rng)
    lens = [0] * B
    first = [int(n) for n in rng.integers(1, 200, size=B)]
    for n_new in (first, [int(n) for n in rng.integers(0, 40, size=B)]):
        n_max = max(n_new)
        kk = np.zeros((B, H, n_max, D), dtype=np.uint16)
        vv = np.zeros((B, H, n_max, D), dtype=np.uint16)
        for b in range(B):
            kk[b, :, :n_new[b]] = k[b, :, lens[b]:lens[b] + n_new[b]]
            vv[b, :, :n_new[b]] = v[b, :, lens[b]:lens[b] + n_new[b]]
        for c in (ref, paged):
            kvq.append_ragged(c, lens, n_new, to_dev(kk), to_dev(vv))
        lens = [l + n for l, n in zip(lens, n_new)]
    torch.cuda.synchronize()
    kvq.cache_check(ref)
    kvq.cache_check(paged)
    for b in (0, 63, 64, 127, 128, 149):
        oc = O.build_cache(k[b:b + 1, :, :lens[b]], v[b:b + 1, :, :lens[b]], _row_cfg(ocfg), norm_tokens=first[b])
        assert_regions_equal(ref, oc, rows=[0], map_bh=lambda _b, h, b=b: (b, h))
    for ns in (1, 3):
        outs = []
        for c in (ref, paged):
            out = torch.empty((B, 2 * H, D), dtype=torch.float32, device=DEV)
            ws = torch.zeros(kvq.decode_workspace_bytes(c, ns), dtype=torch.uint8, device=DEV)
            kvq.decode_ragged(c, lens, to_dev(q), out, ns, ws)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy().astype(np.float64))
        assert np.array_equal(outs[0], outs[1])
        worst = 0.0
        for b in range(B):
            oc = O.build_cache(k[b:b + 1, :, :lens[b]], v[b:b + 1, :, :lens[b]], _row_cfg(ocfg),
                               norm_tokens=first[b])
            ok, err, bound = within_tol(outs[0][b:b + 1], O.decode(oc, q[b:b + 1]))
            assert ok, (b, lens[b], ns, err, bound)
            worst = max(worst, err / bound)
        say(f"    {ns} splits: every row within tolerance (worst err/bound {worst:.3f})")


def test_paged_long_rows_and_every_entry_point():
    """Paged caches through every call that takes one, each checked against a contiguous twin
    (bit for bit) and the oracle: a long row (more than 64 tiles per wavefront at one split,
    so the wavefront reloads its page register), a head that is 16-bit on both sides, fused
    decode steps across a block flush, and multi-token decode."""
    say("case: paged long rows, 16-bit head, decode_step, decode_multi")
    rng = np.random.default_rng(720)
    B, H, D, T = 2, 3, 128, 20700
    kb, vb = (3, 16, 2), (2, 16, 4)
    ocfg = O.CacheConfig(B, H, H, D, T + 40, 4, 64, "bf16", "hybrid", kb, vb)
    k = workloads.random_raw16(rng, (B, H, T + 34, D), "bf16", 2.0)
    v = workloads.random_raw16(rng, (B, H, T + 34, D), "bf16")
    q = workloads.random_raw16(rng, (B, H, D), "bf16")
    ref = gpu_cache(ocfg, k[:, :, :T], v[:, :, :T], chunks=[5000, 15700])
    paged, table = _paged_twin(ocfg, rng)
    for a, n in ((0, 5000), (5000, 15700)):
        kvq.append(paged, to_dev(k[:, :, a:a + n]), to_dev(v[:, :, a:a + n]))
    torch.cuda.synchronize()
    kvq.cache_check(paged)
    oc = O.build_cache(k[:, :, :T], v[:, :, :T], ocfg)
    assert oc.body >= 20000
    assert_paged_regions_equal(paged, oc, table, table.shape[1])
    for ns in (1, 3):
        got = gpu_decode(paged, q, ns)
        assert np.array_equal(got, gpu_decode(ref, q, ns)), ns
        ok, err, bound = within_tol(got, O.decode(oc, q))
        say(f"    paged decode n_splits={ns}: max err {err:.3e} (bound {bound:.3e})")
        assert ok
    # fused decode steps: 34 one-token steps, one of which flushes a block into a page
    ws = torch.zeros(kvq.decode_workspace_bytes(ref, 2), dtype=torch.uint8, device=DEV)
    ws2 = torch.zeros_like(ws)
    for i in range(34):
        t = T + i
        qs = workloads.random_raw16(rng, (B, H, D), "bf16")
        o1 = torch.empty((B, H, D), dtype=torch.float32, device=DEV)
        o2 = torch.empty_like(o1)
        kvq.decode_step(ref, to_dev(k[:, :, t:t + 1]), to_dev(v[:, :, t:t + 1]), to_dev(qs), o1, 2, ws)
        kvq.decode_step(paged, to_dev(k[:, :, t:t + 1]), to_dev(v[:, :, t:t + 1]), to_dev(qs), o2, 2, ws2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), i
        if i in (0, 33):
            want = O.decode(O.build_cache(k[:, :, :t + 1], v[:, :, :t + 1], ocfg), qs)
            ok, err, bound = within_tol(o2.cpu().numpy().astype(np.float64), want)
            say(f"    paged decode_step {i}: max err {err:.3e} (bound {bound:.3e})")
            assert ok
    kvq.cache_check(paged)
    # multi-token decode of the last 3 tokens (G = 1, so 3 query rows per KV head)
    qm = workloads.random_raw16(rng, (B, 3, H, D), "bf16")
    outs = []
    for c in (ref, paged):
        out = torch.empty((B, 3, H, D), dtype=torch.float32, device=DEV)
        wsm = torch.zeros(kvq.decode_multi_workspace_bytes(c, 3, 3), dtype=torch.uint8, device=DEV)
        kvq.decode_multi(c, to_dev(qm), out, 3, wsm)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy().astype(np.float64))
    assert np.array_equal(outs[0], outs[1])
    want = O.decode_multi(O.build_cache(k, v, ocfg), qm)
    ok, err, bound = within_tol(outs[1], want)
    say(f"    paged decode_multi: max err {err:.3e} (bound {bound:.3e})")
    assert ok


def test_paged_ragged_rows():
    """Ragged appends and decodes on a paged cache equal those on a contiguous cache, and each
    row matches the oracle's one-row cache."""
    say("case: paged ragged rows")
    rng = np.random.default_rng(730)
    B, H, D = 3, 2, 64
    ocfg = O.CacheConfig(B, H, 2 * H, D, 1500, 2, 40, "fp16", "asym", (3, 4), (2, 3))
    n_max = 700
    k = workloads.random_raw16(rng, (B, H, 2 * n_max, D), "fp16")
    v = workloads.random_raw16(rng, (B, H, 2 * n_max, D), "fp16")
    q = workloads.random_raw16(rng, (B, 2 * H, D), "fp16")
    ref = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    paged, _ = _paged_twin(ocfg, rng)
    lens = [0] * B
    for n_new in ([700, 3, 650], [1, 697, 0]):
        for c in (ref, paged):
            kk = np.stack([k[b, :, lens[b]:lens[b] + n_max] for b in range(B)])
            vv = np.stack([v[b, :, lens[b]:lens[b] + n_max] for b in range(B)])
            kvq.append_ragged(c, lens, n_new, to_dev(np.ascontiguousarray(kk)), to_dev(np.ascontiguousarray(vv)))
        lens = [l + n for l, n in zip(lens, n_new)]
    torch.cuda.synchronize()
    kvq.cache_check(ref)
    kvq.cache_check(paged)
    outs = []
    for c in (ref, paged):
        out = torch.empty((B, 2 * H, D), dtype=torch.float32, device=DEV)
        ws = torch.zeros(kvq.decode_workspace_bytes(c, 4), dtype=torch.uint8, device=DEV)
        kvq.decode_ragged(c, lens, to_dev(q), out, 4, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy().astype(np.float64))
    assert np.array_equal(outs[0], outs[1])
    for b in range(B):
        c1 = O.CacheConfig(1, H, 2 * H, D, 1500, 2, 40, "fp16", "asym", (3, 4), (2, 3))
        oc = O.build_cache(k[b:b + 1, :, :lens[b]], v[b:b + 1, :, :lens[b]], c1)
        ok, err, bound = within_tol(outs[1][b:b + 1], O.decode(oc, q[b:b + 1]))
        say(f"    paged ragged row {b} ({lens[b]} tokens): max err {err:.3e} (bound {bound:.3e})")
        assert ok
