"""Benchmark: decode attention over the packed mixed-precision KV cache on one MI355X.

Workload: qwen8b_t32k — batch 4, 32 query / 8 KV heads, head_dim 128, 32768-token context,
bf16 inputs, K at 3.0 / V at 2.0 average bits allocated per KV head by reverse waterfilling,
hybrid symmetric/asymmetric groups, 4 sink + 128 recent 16-bit tokens, 16 split-K chunks.

A timed step is one decode step of every row: append the step's new key/value token
(quantizing a 32-token block whenever one leaves the recent window), split-K fused-dequant
decode attention over the whole cache, and the log-sum-exp merge. Calibration, fit and bit
allocation run once per model before decoding (the method's offline stage) and are reported
separately. Several cache instances (together > 512 MB) are rotated so the 256 MB Infinity
Cache cannot serve the reads: every decode reads its cache from HBM.

Prints one JSON line. `value` = KV tokens x KV heads attended per second.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "qwen8b_t32k"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--instances", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def decode_bytes(spec, k_bits, v_bits, T, n_splits):
    """Algorithmic HBM bytes of one decode launch: packed codes + fp16 (s, z) of every body
    token, 16-bit sink/window rows, the queries, and the split partials written."""
    D = spec.head_dim
    body = 32 * max(0, (T - spec.n_sink - spec.n_recent) // 32)
    win = T - body
    per_head = 0
    for kb, vb in zip(k_bits, v_bits):
        per_tok = D * kb // 8 + D * vb // 8 + (D // 32) * 4 + D * 4 // 32
        per_head += body * per_tok + win * D * 4
    rows = spec.batch * spec.n_q
    q = rows * D * 2
    partials = n_splits * rows * (D + 2) * 4
    return spec.batch * per_head + q + partials


def cpu_baseline(w, k_bits, v_bits, seconds):
    """Oracle decode timed on the host: the float64 oracle over a sample of (row, KV head)
    slices of the same workload, BLAS limited to one thread."""
    from threadpoolctl import threadpool_limits

    from oracle import kvq_oracle as O
    s = w["spec"]
    G = s.n_q // s.n_kv
    pairs = [(b, h) for b in range(s.batch) for h in range(s.n_kv)][::4]
    caches = []
    for b, h in pairs:
        cfg1 = O.CacheConfig(1, 1, G, s.head_dim, w["tokens"], s.n_sink, s.n_recent, s.dtype,
                             s.quant, (k_bits[h],), (v_bits[h],))
        caches.append((O.build_cache(w["k"][b:b + 1, h:h + 1], w["v"][b:b + 1, h:h + 1], cfg1),
                       w["q"][b:b + 1, h * G:(h + 1) * G]))
    done = 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        while True:
            for oc, q in caches:
                O.decode(oc, q)
                done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": done * w["tokens"] / el, "unit": "KV tokens*heads/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{len(pairs)} of {s.batch * s.n_kv} (row, KV head) slices of {WORKLOAD}, "
                      f"{done} float64 decodes in {el:.1f} s (unpack codes, dequantize, attention)"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (the decode path has no multi-GPU "
              "stage); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import mixed_precision_quantized_kvq_amd as kvq
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.make(WORKLOAD)
    s = w["spec"]
    B, H, Hq, D = s.batch, s.n_kv, s.n_q, s.head_dim

    # ---- offline stage: bit allocation (host) and a calibration pass of the same shape as
    # the prefill workload's (8 heads x 512 tokens x 128)
    t0 = time.perf_counter()
    k_bits, _ = kvq.allocate_bits(w["alpha_k"], w["beta_k"], w["w_k"], s.k_total, s.b_lo, s.b_hi)
    v_bits, _ = kvq.allocate_bits(w["alpha_v"], w["beta_v"], w["w_v"], s.v_total, s.b_lo, s.b_hi)
    alloc_us = (time.perf_counter() - t0) * 1e6 / 2
    cw = workloads.make("prefill_t4k", tokens=512, batch=1)
    xk = torch.from_numpy(cw["k"][0].view(np.int16)).to(dev)
    xv = torch.from_numpy(cw["v"][0].view(np.int16)).to(dev)
    kvq.calibrate_fit(xk, "bf16", kvq.AXIS_KEY)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    kvq.calibrate_fit(xk, "bf16", kvq.AXIS_KEY)
    kvq.calibrate_fit(xv, "bf16", kvq.AXIS_VALUE)
    calib_ms = (time.perf_counter() - t0) * 1e3

    # ---- caches: prefill T-1 tokens into each instance, then one token per step
    T0 = s.tokens - 1
    steps_per_inst = (args.steps + args.warmup + args.instances - 1) // args.instances + 1
    capacity = T0 + steps_per_inst + 64
    cfg = kvq.Config.make(B, H, Hq, D, capacity, s.n_sink, s.n_recent, s.dtype, s.quant, k_bits, v_bits)
    kd = torch.from_numpy(w["k"][:, :, :T0].view(np.int16)).to(dev)
    vd = torch.from_numpy(w["v"][:, :, :T0].view(np.int16)).to(dev)
    caches = []
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    prefill_ms = []
    for _ in range(args.instances):
        c = kvq.KVCache(cfg, device=dev)
        ev0.record()
        kvq.append(c, kd, vd)
        ev1.record()
        torch.cuda.synchronize()
        prefill_ms.append(ev0.elapsed_time(ev1))
        kvq.cache_check(c)
        caches.append(c)
    del kd, vd
    cache_mb = kvq.cache_bytes(cfg) / 1e6
    rng = np.random.default_rng(1)
    n_new = 8
    newk = [torch.from_numpy(workloads.random_raw16(rng, (B, H, 1, D), s.dtype).view(np.int16)).to(dev)
            for _ in range(n_new)]
    newv = [torch.from_numpy(workloads.random_raw16(rng, (B, H, 1, D), s.dtype).view(np.int16)).to(dev)
            for _ in range(n_new)]
    q = torch.from_numpy(w["q"].view(np.int16)).to(dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.zeros(kvq.decode_workspace_bytes(caches[0], s.n_splits) * 2, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, evs=None):
        # one decode step = append the new token + split-K decode + merge (the two launches of
        # decode_attention, called apart so that events bracket the split-K kernel alone)
        c = caches[i % len(caches)]
        kvq.append(c, newk[i % n_new], newv[i % n_new], stream=stream)
        if evs is not None:
            evs[0].record(stream)
        kvq.decode_splitk(c, q, s.n_splits, ws, stream=stream)
        if evs is not None:
            evs[1].record(stream)
        kvq.decode_merge(c, out, s.n_splits, ws, stream=stream)
        return c.len

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    toks = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        toks += step(args.warmup + i, evs[i]) * B * H
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    for c in caches:
        kvq.cache_check(c)
    dec_ms = [a.elapsed_time(b) for a, b in evs]
    dec_us = float(np.mean(dec_ms)) * 1e3
    T_mean = toks / (args.steps * B * H)
    nbytes = decode_bytes(s, k_bits, v_bits, int(round(T_mean)), s.n_splits)
    achieved = nbytes / (dec_us * 1e-6) / 1e9
    res = {
        "metric": "decode-attention KV tokens*heads/s over the packed mixed-precision cache",
        "value": toks / el,
        "unit": "KV tokens*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": el * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) keys with log-normal(0,0.5) channel scales, N(0,1) values)",
        "config": {"workload": WORKLOAD, "batch": B, "kv_heads": H, "q_heads": Hq, "head_dim": D,
                   "context_mean": T_mean, "k_bits": k_bits, "v_bits": v_bits, "quant": s.quant,
                   "n_sinks": s.n_sink, "n_recent": s.n_recent, "n_splits": s.n_splits,
                   "cache_instances": args.instances, "cache_mb_each": round(cache_mb, 1),
                   "step": "append 1 token + split-K decode + LSE merge"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "decode_kernel (split-K fused-dequant decode), HIP events around each launch",
                     "bytes_per_launch": nbytes, "avg_us": dec_us},
        "offline": {"allocate_bits_us": alloc_us, "calibrate_fit_ms_k_plus_v": calib_ms,
                    "prefill_append_ms": float(np.median(prefill_ms)),
                    "prefill_append_gbs": (B * H * T0 * D * 4) / (float(np.median(prefill_ms)) * 1e-3) / 1e9},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, k_bits, v_bits, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
