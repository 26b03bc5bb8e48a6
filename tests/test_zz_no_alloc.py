"""The decode entry point that allocates nothing (static device scratch), against the one that
takes a caller workspace, through the C ABI: bit-identical outputs on two calls in a row, the
second on a smaller cache, and a clear error for partials larger than the scratch."""
import numpy as np
import pytest
import torch

import mixed_precision_quantized_kvq_amd as kvq
import workloads
from oracle import kvq_oracle as O
from tests.kvq_test_util import lib_cfg, within_tol

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def _case(seed, B, H, G, D, T, quant, dtype, kb, vb):
    rng = np.random.default_rng(seed)
    ocfg = O.CacheConfig(B, H, H * G, D, T + 8, 4, 64, dtype, quant, kb, vb)
    k = workloads.random_raw16(rng, (B, H, T, D), dtype, 2.0)
    v = workloads.random_raw16(rng, (B, H, T, D), dtype)
    q = workloads.random_raw16(rng, (B, H * G, D), dtype)
    cache = kvq.KVCache(lib_cfg(kvq, ocfg), device=DEV)
    kvq.append(cache, _to_dev(k), _to_dev(v))
    return ocfg, cache, k, v, q


def test_noalloc_decode_equals_workspace_decode():
    cases = [(800, 4, 8, 4, 128, 5000, "hybrid", "bf16", (2, 3, 4, 3, 2, 4, 3, 2), (2,) * 8, 16),
             (801, 1, 2, 2, 64, 700, "asym", "fp16", (3, 16), (4, 2), 3)]
    for seed, B, H, G, D, T, quant, dtype, kb, vb, ns in cases:
        print(f"case: B={B} H={H} G={G} D={D} T={T} n_splits={ns}", flush=True)
        ocfg, cache, k, v, q = _case(seed, B, H, G, D, T, quant, dtype, kb, vb)
        qd = _to_dev(q)
        out_ws = torch.empty((B, H * G, D), dtype=torch.float32, device=DEV)
        ws = torch.zeros(kvq.decode_workspace_bytes(cache, ns), dtype=torch.uint8, device=DEV)
        kvq.decode_attention(cache, qd, out_ws, ns, ws)
        out_na = torch.full_like(out_ws, float("nan"))
        kvq.decode_attention_noalloc(cache, qd, out_na, ns)
        torch.cuda.synchronize()
        assert torch.equal(out_ws, out_na)
        oc = O.build_cache(k, v, ocfg)
        ok, err, bound = within_tol(out_na.cpu().numpy().astype(np.float64), O.decode(oc, q))
        print(f"    max err {err:.3e} (bound {bound:.3e})", flush=True)
        assert ok


def test_noalloc_decode_rejects_partials_larger_than_the_scratch():
    ocfg, cache, _, _, q = _case(802, 4, 8, 4, 128, 300, "asym", "bf16", (2,) * 8, (2,) * 8)
    assert kvq.decode_workspace_bytes(cache, 256) > 4 << 20
    out = torch.zeros((4, 32, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(kvq.KvqError, match="ERR_ARG.*static scratch"):
        kvq.decode_attention_noalloc(cache, _to_dev(q), out, 256)
    torch.cuda.synchronize()
    assert not out.any()  # nothing was enqueued
