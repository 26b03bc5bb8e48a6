"""Whole-model calibration and allocation on the GPU against the oracle (RateQuant page:
288 (layer, KV head) pairs of Qwen3-8B, 16 calibration sequences of 512 tokens, sections
3.3, 4.1 and W.12).

Every pair of a Qwen3-8B-shaped model is calibrated in one call per cache side. The fit
(alpha, beta, R^2) must match the oracle to 1e-13 relative, and the integer allocation over
all 288 pairs must equal the oracle's bit for bit. The reduced test checks every pair, with
16 x 16-token sequences. The full-size test (16 x 512 tokens) checks sampled pairs' fits,
and the allocation over all pairs from the library's fits.
"""
import numpy as np
import pytest
import torch

import mixed_precision_quantized_kvq_amd as kvq
import workloads
from oracle import kvq_oracle as O
from tests.test_gpu_parity import DEV, say

pytestmark = pytest.mark.gpu

BS = list(range(2, 9))


def _calibrate(m):
    s = m["spec"]
    q = kvq.QUANT_HYBRID if s.quant == "hybrid" else kvq.QUANT_ASYM
    out = {}
    for name, axis in (("k", kvq.AXIS_KEY), ("v", kvq.AXIS_VALUE)):
        x = torch.from_numpy(m[name].view(np.int16)).to(DEV)
        out[name] = kvq.calibrate_fit(x, s.dtype, axis, q, 2, 8)
        del x
    return out


def _allocate(m, fits):
    s = m["spec"]
    kb, _ = kvq.allocate_bits(fits["k"][0], fits["k"][1], m["w_k"], m["k_total"], s.b_lo, s.b_hi)
    vb, _ = kvq.allocate_bits(fits["v"][0], fits["v"][1], m["w_v"], m["v_total"], s.b_lo, s.b_hi)
    return kb, vb


def test_model_calibration_all_pairs_reduced():
    say("case: 288-pair calibration + allocation, 16 x 16 tokens per pair")
    m = workloads.make_model_calib(seq_len=16)
    s = m["spec"]
    hyb = s.quant == "hybrid"
    got = _calibrate(m)
    for name, axis in (("k", 0), ("v", 1)):
        Ds = [O.calib_distortion(m[name][p], s.dtype, axis, 2, 8, hyb) for p in range(s.pairs)]
        ref = O.fit_heads(BS, Ds)
        for g, r in zip(got[name], ref):
            assert np.allclose(np.array(g), r, rtol=1e-13, atol=0), name
    kb, vb = _allocate(m, got)
    assert kb == O.allocate_greedy(got["k"][0], got["k"][1], list(m["w_k"]), m["k_total"], s.b_lo, s.b_hi)
    assert vb == O.allocate_greedy(got["v"][0], got["v"][1], list(m["w_v"]), m["v_total"], s.b_lo, s.b_hi)
    assert sum(kb) == m["k_total"] and sum(vb) == m["v_total"]
    say(f"    K bits {[kb.count(b) for b in (2, 3, 4)]}, V bits {[vb.count(b) for b in (2, 3, 4)]}")


@pytest.mark.slow
def test_model_calibration_full_size():
    say("case: 288-pair calibration + allocation, 16 x 512 tokens per pair")
    m = workloads.make_model_calib()
    s = m["spec"]
    hyb = s.quant == "hybrid"
    got = _calibrate(m)
    kb, vb = _allocate(m, got)
    # the allocation over all pairs, from the library's own fits
    assert kb == O.allocate_greedy(got["k"][0], got["k"][1], list(m["w_k"]), m["k_total"], s.b_lo, s.b_hi)
    assert vb == O.allocate_greedy(got["v"][0], got["v"][1], list(m["w_v"]), m["v_total"], s.b_lo, s.b_hi)
    # sampled pairs: the oracle's fit of each alone (beta only where no fallback applies)
    for name, axis in (("k", 0), ("v", 1)):
        for p in (0, 1, 143, 287):
            a, b, r2, degen = O.fit_one(BS, O.calib_distortion(m[name][p], s.dtype, axis, 2, 8, hyb))
            ga, gb, gr = got[name][0][p], got[name][1][p], got[name][2][p]
            assert not degen
            assert np.isclose(ga, a, rtol=1e-13, atol=0) and np.isclose(gr, r2, rtol=1e-13, atol=0), (name, p)
            if r2 >= O.R2_FALLBACK:
                assert np.isclose(gb, b, rtol=1e-13, atol=0), (name, p)
            say(f"    {name} pair {p}: alpha {ga:.6g} beta {gb:.6g} R^2 {gr:.6f}")
    say(f"    K bits {[kb.count(b) for b in (2, 3, 4)]}, V bits {[vb.count(b) for b in (2, 3, 4)]}")
