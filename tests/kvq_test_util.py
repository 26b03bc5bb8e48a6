"""Helpers shared by the tests: workload -> oracle / library configs and bit allocations."""
import numpy as np

from oracle import kvq_oracle as O


def oracle_bits(w, *, alpha_k=None, beta_k=None, alpha_v=None, beta_v=None):
    """Per-KV-head (k_bits, v_bits) for a workload, allocated by the oracle."""
    s = w["spec"]
    if s.alloc == "fixed":
        return tuple(s.fixed_bits), tuple(s.fixed_bits)
    if s.alloc == "joint":
        b = O.allocate_greedy(list(w["alpha"]), list(w["beta"]), list(w["w"]), s.k_total, s.b_lo, s.b_hi)
        return tuple(b), tuple(b)
    if s.alloc == "separate":
        kb = O.allocate_greedy(list(w["alpha_k"]), list(w["beta_k"]), list(w["w_k"]), s.k_total, s.b_lo, s.b_hi)
        vb = O.allocate_greedy(list(w["alpha_v"]), list(w["beta_v"]), list(w["w_v"]), s.v_total, s.b_lo, s.b_hi)
        return tuple(kb), tuple(vb)
    if s.alloc == "calibrated":
        kb = O.allocate_greedy(list(alpha_k), list(beta_k), list(w["w_k"]), s.k_total, s.b_lo, s.b_hi)
        vb = O.allocate_greedy(list(alpha_v), list(beta_v), list(w["w_v"]), s.v_total, s.b_lo, s.b_hi)
        return tuple(kb), tuple(vb)
    raise ValueError(s.alloc)


def oracle_calibration(w):
    """(alpha, beta, r2) for keys and values from the calibration slice of a workload."""
    s = w["spec"]
    n = s.calib_tokens
    res = {}
    for name, arr, axis in (("k", w["k"], 0), ("v", w["v"], 1)):
        Ds = [O.calib_distortion(arr[0, h, :n], s.dtype, axis, 2, 8, s.quant == "hybrid")
              for h in range(s.n_kv)]
        res[name] = O.fit_heads(list(range(2, 9)), Ds)
    return res


def oracle_cfg(w, k_bits, v_bits, capacity=None, batch=None, n_kv=None, n_q=None, key_norm=False):
    s = w["spec"]
    return O.CacheConfig(batch=w["batch"] if batch is None else batch,
                         n_kv=s.n_kv if n_kv is None else n_kv,
                         n_q=s.n_q if n_q is None else n_q, head_dim=s.head_dim,
                         capacity=w["tokens"] if capacity is None else capacity,
                         n_sink=s.n_sink, n_recent=s.n_recent, dtype=s.dtype, quant=s.quant,
                         k_bits=tuple(k_bits), v_bits=tuple(v_bits), key_norm=key_norm)


def lib_cfg(kvq, ocfg):
    return kvq.Config.make(ocfg.batch, ocfg.n_kv, ocfg.n_q, ocfg.head_dim, ocfg.capacity,
                           ocfg.n_sink, ocfg.n_recent, ocfg.dtype, ocfg.quant, ocfg.k_bits,
                           ocfg.v_bits, key_norm=ocfg.key_norm)


def head_slice_cfg(ocfg, h):
    """Oracle config of a single (row, KV head) slice of ocfg."""
    G = ocfg.n_q // ocfg.n_kv
    return O.CacheConfig(batch=1, n_kv=1, n_q=G, head_dim=ocfg.head_dim, capacity=ocfg.capacity,
                         n_sink=ocfg.n_sink, n_recent=ocfg.n_recent, dtype=ocfg.dtype,
                         quant=ocfg.quant, k_bits=(ocfg.k_bits[h],), v_bits=(ocfg.v_bits[h],),
                         key_norm=ocfg.key_norm)


def within_tol(got, want, rel=2e-3):
    """max |got - want| <= rel * RMS(want); returns (ok, max_err, bound)."""
    rms = float(np.sqrt(np.mean(np.asarray(want, dtype=np.float64) ** 2)))
    err = float(np.max(np.abs(np.asarray(got, dtype=np.float64) - want)))
    return err <= rel * rms, err, rel * rms
