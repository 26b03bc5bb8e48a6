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
    say(f"case: full-size {name}")
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
    ocfg = oracle_cfg(w, kb, vb)
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
