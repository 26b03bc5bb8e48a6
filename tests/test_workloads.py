"""The synthetic input generators (CPU): the whole-model calibration set draws any subset of
pairs with the same bits as the full draw, and its budgets are the stated averages."""
import numpy as np

import workloads


def test_model_calib_subset_draw():
    full = workloads.make_model_calib(seq_len=4)
    sub = workloads.make_model_calib(seq_len=4, pairs=[0, 77, 287])
    s = full["spec"]
    assert full["k"].shape == (s.pairs, s.seqs * 4, s.head_dim)
    for i, p in enumerate(sub["pairs"]):
        assert np.array_equal(sub["k"][i], full["k"][p]) and np.array_equal(sub["v"][i], full["v"][p])
    assert full["k_total"] == 3 * 288 and full["v_total"] == 720
    assert np.array_equal(sub["w_k"], full["w_k"])
