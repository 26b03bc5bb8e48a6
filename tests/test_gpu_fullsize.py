"""Full-size parity on the five workloads, in the launch configuration the benchmark times
(bulk prefill append, then split-K decode with the workload's split count).

The oracle recomputes sampled (row, KV head) slices one by one: their packed bytes must be
bit-exact and their decode outputs within 2e-3 * RMS. Bit allocations (and, for the prefill
workload, the calibration fit) are compared in full.
"""
import numpy as np
import pytest
import torch

import mixed_precision_quantized_kvq_amd as kvq
import workloads
from oracle import kvq_oracle as O
from tests.kvq_test_util import head_slice_cfg, lib_cfg, oracle_bits, oracle_calibration, oracle_cfg, within_tol
from tests.test_gpu_parity import DEV, assert_regions_equal, gpu_decode, say, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _bits(w):
    s = w["spec"]
    if s.alloc == "fixed":
        return tuple(s.fixed_bits), tuple(s.fixed_bits), None
    if s.alloc == "joint":
        b, _ = kvq.allocate_bits(w["alpha"], w["beta"], w["w"], s.k_total, s.b_lo, s.b_hi)
        return tuple(b), tuple(b), None
    if s.alloc == "separate":
        kb, _ = kvq.allocate_bits(w["alpha_k"], w["beta_k"], w["w_k"], s.k_total, s.b_lo, s.b_hi)
        vb, _ = kvq.allocate_bits(w["alpha_v"], w["beta_v"], w["w_v"], s.v_total, s.b_lo, s.b_hi)
        return tuple(kb), tuple(vb), None
    fits = {}
    for name, arr, axis in (("k", w["k"], kvq.AXIS_KEY), ("v", w["v"], kvq.AXIS_VALUE)):
        x = to_dev(np.ascontiguousarray(arr[0, :, :s.calib_tokens]))
        fits[name] = kvq.calibrate_fit(x, s.dtype, axis, kvq.QUANT_ASYM, 2, 8)
    kb, _ = kvq.allocate_bits(fits["k"][0], fits["k"][1], w["w_k"], s.k_total, 2, 4)
    vb, _ = kvq.allocate_bits(fits["v"][0], fits["v"][1], w["w_v"], s.v_total, 2, 4)
    return tuple(kb), tuple(vb), fits


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_full_size_sampled(name):
    _full_size_sampled(name, key_norm=False)


@pytest.mark.parametrize("name", ["qwen8b_t32k", "long_t128k"])
def test_full_size_key_norm(name):
    # the same bulk append + decode with per-channel key normalization
    _full_size_sampled(name, key_norm=True)


def _full_size_sampled(name, key_norm):
    say(f"case: full-size {name}, key normalization {key_norm}")
    w = workloads.make(name)
    s = w["spec"]
    kb, vb, fits = _bits(w)
    if fits is not None:
        ref = oracle_calibration(w)
        for c in ("k", "v"):
            for g, r in zip(fits[c], ref[c]):
                assert np.allclose(np.array(g), r, rtol=1e-13, atol=0)
        assert (kb, vb) == oracle_bits(w, alpha_k=ref["k"][0], beta_k=ref["k"][1],
                                       alpha_v=ref["v"][0], beta_v=ref["v"][1])
    else:
        assert (kb, vb) == oracle_bits(w)
    say(f"    bits K={kb} V={vb}")
    ocfg = oracle_cfg(w, kb, vb, key_norm=key_norm)
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    kd, vd = to_dev(w["k"]), to_dev(w["v"])
    kvq.append(cache, kd, vd)
    torch.cuda.synchronize()
    kvq.cache_check(cache)
    del kd, vd
    out = gpu_decode(cache, w["q"], s.n_splits)
    B, H, G = s.batch, s.n_kv, s.n_q // s.n_kv
    samples = sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 2), (0, H - 1)})
    gots, wants = [], []
    for b, h in samples:
        cfg1 = head_slice_cfg(ocfg, h)
        oc1 = O.build_cache(w["k"][b:b + 1, h:h + 1], w["v"][b:b + 1, h:h + 1], cfg1)
        assert_regions_equal(cache, oc1, map_bh=lambda _b, _h, b=b, h=h: (b, h))
        wants.append(O.decode(oc1, w["q"][b:b + 1, h * G:(h + 1) * G])[0])
        gots.append(out[b, h * G:(h + 1) * G])
        say(f"    row {b} head {h}: bytes equal")
    ok, err, bound = within_tol(np.stack(gots), np.stack(wants))
    say(f"    decode n_splits={s.n_splits}: max err {err:.3e} (bound {bound:.3e})")
    assert ok
    assert np.all(np.isfinite(out))


def test_full_size_multi_token():
    # the 7B-shaped multi-head layer: the last 4 tokens of every row decoded at once, causally,
    # in the launch configuration the benchmark times; sampled slices against the oracle
    name = "mha7b_t8k"
    say(f"case: full-size multi-token decode on {name}")
    w = workloads.make(name)
    s = w["spec"]
    kb, vb, _ = _bits(w)
    ocfg = oracle_cfg(w, kb, vb)
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    kvq.append(cache, to_dev(w["k"]), to_dev(w["v"]))
    qm = w["q_multi"]
    Q = qm.shape[1]
    out = torch.empty(qm.shape, dtype=torch.float32, device=DEV)
    ws = torch.zeros(kvq.decode_multi_workspace_bytes(cache, s.n_splits, Q), dtype=torch.uint8, device=DEV)
    kvq.decode_multi(cache, to_dev(qm), out, s.n_splits, ws)
    got = out.cpu().numpy()
    G = s.n_q // s.n_kv
    B, H = s.batch, s.n_kv
    for b, h in sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 2)}):
        oc1 = O.build_cache(w["k"][b:b + 1, h:h + 1], w["v"][b:b + 1, h:h + 1], head_slice_cfg(ocfg, h))
        want = O.decode_multi(oc1, qm[b:b + 1, :, h * G:(h + 1) * G])[0]
        for i in range(Q):
            ok, err, bound = within_tol(got[b, i, h * G:(h + 1) * G], want[i])
            assert ok, (b, h, i, err, bound)
        say(f"    row {b} head {h}: {Q} query tokens within tolerance")


def test_full_size_multi_token_gqa():
    # the 32k-token GQA workload: the last 4 tokens of every row decoded at once by its 4 query
    # heads (16 rows per KV head, the 16-row tile), in the benchmark's launch configuration;
    # sampled (row, KV head) slices against the oracle
    name = "qwen8b_t32k"
    say(f"case: full-size 4-token decode on {name}")
    w = workloads.make(name)
    s = w["spec"]
    kb, vb, _ = _bits(w)
    ocfg = oracle_cfg(w, kb, vb)
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    kvq.append(cache, to_dev(w["k"]), to_dev(w["v"]))
    Q = 4
    qm = workloads.random_raw16(np.random.default_rng(4242), (s.batch, Q, s.n_q, s.head_dim), s.dtype)
    out = torch.empty(qm.shape, dtype=torch.float32, device=DEV)
    ws = torch.zeros(kvq.decode_multi_workspace_bytes(cache, s.n_splits, Q), dtype=torch.uint8, device=DEV)
    kvq.decode_multi(cache, to_dev(qm), out, s.n_splits, ws)
    got = out.cpu().numpy()
    G = s.n_q // s.n_kv
    B, H = s.batch, s.n_kv
    for b, h in sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 2)}):
        oc1 = O.build_cache(w["k"][b:b + 1, h:h + 1], w["v"][b:b + 1, h:h + 1], head_slice_cfg(ocfg, h))
        want = O.decode_multi(oc1, qm[b:b + 1, :, h * G:(h + 1) * G])[0]
        for i in range(Q):
            ok, err, bound = within_tol(got[b, i, h * G:(h + 1) * G], want[i])
            assert ok, (b, h, i, err, bound)
        say(f"    row {b} head {h}: {Q} query tokens x {G} heads within tolerance")


def test_full_size_decode_steps():
    # the benchmark's step: prefill T - 1 tokens of the 32k workload, then one-token decode
    # steps (append + decode + merge in one call) up to and across the next block flush;
    # sampled slices against the oracle on the whole prefix after the first and the flush step
    name = "qwen8b_t32k"
    say(f"case: full-size fused decode steps on {name}")
    w = workloads.make(name)
    s = w["spec"]
    kb, vb, _ = _bits(w)
    rng = np.random.default_rng(7)
    T0 = s.tokens - 1
    n_steps = 6
    extra_k = workloads.random_raw16(rng, (s.batch, s.n_kv, n_steps - 1, s.head_dim), s.dtype)
    extra_v = workloads.random_raw16(rng, (s.batch, s.n_kv, n_steps - 1, s.head_dim), s.dtype)
    k_all = np.concatenate([w["k"], extra_k], axis=2)
    v_all = np.concatenate([w["v"], extra_v], axis=2)
    ocfg = oracle_cfg(w, kb, vb, capacity=T0 + n_steps)
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    kvq.append(cache, to_dev(np.ascontiguousarray(k_all[:, :, :T0])), to_dev(np.ascontiguousarray(v_all[:, :, :T0])))
    out = torch.empty((s.batch, s.n_q, s.head_dim), dtype=torch.float32, device=DEV)
    ws = torch.zeros(kvq.decode_workspace_bytes(cache, s.n_splits), dtype=torch.uint8, device=DEV)
    q = to_dev(w["q"])
    B, H, G = s.batch, s.n_kv, s.n_q // s.n_kv
    body = lambda t: O.body_len(t, s.n_sink, s.n_recent)
    flush_step = next(i for i in range(n_steps) if body(T0 + i + 1) > body(T0 + i))
    samples = sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 2)})
    for i in range(n_steps):
        t = T0 + i
        kvq.decode_step(cache, to_dev(np.ascontiguousarray(k_all[:, :, t:t + 1])),
                        to_dev(np.ascontiguousarray(v_all[:, :, t:t + 1])), q, out, s.n_splits, ws)
        if i not in (0, flush_step):
            continue
        got = out.cpu().numpy()
        gots, wants = [], []
        for b, h in samples:
            cfg1 = O.CacheConfig(1, 1, G, s.head_dim, t + 1, s.n_sink, s.n_recent, s.dtype, s.quant,
                                 (kb[h],), (vb[h],))
            oc1 = O.build_cache(k_all[b:b + 1, h:h + 1, :t + 1], v_all[b:b + 1, h:h + 1, :t + 1], cfg1)
            wants.append(O.decode(oc1, w["q"][b:b + 1, h * G:(h + 1) * G])[0])
            gots.append(got[b, h * G:(h + 1) * G])
        ok, err, bound = within_tol(np.stack(gots), np.stack(wants))
        say(f"    step {i} (T = {t + 1}, flush {i == flush_step}): max err {err:.3e} (bound {bound:.3e})")
        assert ok
    kvq.cache_check(cache)
