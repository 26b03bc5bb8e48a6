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
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the decode timings of the other full-size workloads and the prefill ingest")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run only the launches the HBM-counter passes measure: a 256 MiB "
                         "elementwise copy (counter calibration), then 30 decode launches")
    ap.add_argument("--probe", choices=("decode", "step", "append", "calib"),
                    help="run only one kind of launch for a profiler pass, after the same 256 MiB "
                         "copy: 30 split-K decode launches of --workload (rotating caches), 4 "
                         "prefill appends of prefill_t4k, or 3 whole-model calibrations (K and V)")
    ap.add_argument("--workload", default=WORKLOAD, help="decode workload of --probe decode")
    return ap.parse_args()


def _copy_probe():
    """torch.add over 64 Mi int32 (256 MiB read + 256 MiB written, a plain copy of known size)
    10 times: the counter calibration of every profiler pass."""
    import torch
    dev = torch.device("cuda:0")
    n = 64 << 20
    src = torch.arange(n, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(10):
        torch.add(src, 1, out=dst)
    torch.cuda.synchronize()


def probe(kind, workload):
    """The launches behind a committed profiler summary: the copy, then one kind of launch.
    decode: 30 split-K decode launches of `workload` over rotating full-size caches (5, or 3
    for the 128k-token context); step: 64 decode steps (append one token + split-K decode +
    merge) over the same rotating caches; append: 4 appends of the whole 16 x 4096-token
    prefill into fresh caches; calib: 3 calibrations + fits of the 288-pair whole-model set, K
    and V."""
    import torch

    import mixed_precision_quantized_kvq_amd as kvq
    import workloads
    dev = torch.device("cuda:0")
    _copy_probe()
    if kind in ("decode", "step"):
        w = workloads.make(workload)
        s = w["spec"]
        kb, vb = workload_bits(kvq, w)
        # decode: full caches; step: one token short, with room for the appended ones
        T0 = s.tokens if kind == "decode" else s.tokens - 1
        cfg = kvq.Config.make(s.batch, s.n_kv, s.n_q, s.head_dim, T0 + (0 if kind == "decode" else 64), s.n_sink,
                              s.n_recent, s.dtype, s.quant, kb, vb)
        kd = torch.from_numpy(np.ascontiguousarray(w["k"][:, :, :T0]).view(np.int16)).to(dev)
        vd = torch.from_numpy(np.ascontiguousarray(w["v"][:, :, :T0]).view(np.int16)).to(dev)
        n_inst = 3 if s.tokens > 65536 else 5
        caches = []
        for _ in range(n_inst):
            c = kvq.KVCache(cfg, device=dev)
            kvq.append(c, kd, vd)
            caches.append(c)
        del kd, vd
        q = torch.from_numpy(w["q"].view(np.int16)).to(dev)
        ws = torch.zeros(kvq.decode_workspace_bytes(caches[0], s.n_splits) * 2, dtype=torch.uint8, device=dev)
        if kind == "decode":
            for i in range(30):
                kvq.decode_splitk(caches[i % n_inst], q, s.n_splits, ws)
        else:
            rng = np.random.default_rng(1)
            shape = (s.batch, s.n_kv, 1, s.head_dim)
            newk = torch.from_numpy(workloads.random_raw16(rng, shape, s.dtype).view(np.int16)).to(dev)
            newv = torch.from_numpy(workloads.random_raw16(rng, shape, s.dtype).view(np.int16)).to(dev)
            out = torch.empty((s.batch, s.n_q, s.head_dim), dtype=torch.float32, device=dev)
            for i in range(64):
                kvq.decode_step(caches[i % n_inst], newk, newv, q, out, s.n_splits, ws)
    elif kind == "append":
        w = workloads.make("prefill_t4k")
        s = w["spec"]
        xk = torch.from_numpy(np.ascontiguousarray(w["k"][0, :, :s.calib_tokens]).view(np.int16)).to(dev)
        xv = torch.from_numpy(np.ascontiguousarray(w["v"][0, :, :s.calib_tokens]).view(np.int16)).to(dev)
        kb, vb = workload_bits(kvq, w, xk, xv)
        cfg = kvq.Config.make(s.batch, s.n_kv, s.n_q, s.head_dim, s.tokens, s.n_sink, s.n_recent, s.dtype,
                              s.quant, kb, vb)
        kd = torch.from_numpy(w["k"].view(np.int16)).to(dev)
        vd = torch.from_numpy(w["v"].view(np.int16)).to(dev)
        for _ in range(4):
            c = kvq.KVCache(cfg, device=dev)
            kvq.append(c, kd, vd)
            torch.cuda.synchronize()
            kvq.cache_check(c)
            del c
    else:
        m = workloads.make_model_calib()
        s = m["spec"]
        xk = torch.from_numpy(m["k"].view(np.int16)).to(dev)
        xv = torch.from_numpy(m["v"].view(np.int16)).to(dev)
        ws = torch.empty(kvq.calibrate_workspace_bytes(s.pairs, s.tokens, s.head_dim, 2, 8), dtype=torch.uint8,
                         device=dev)
        q = kvq.QUANT_HYBRID if s.quant == "hybrid" else kvq.QUANT_ASYM
        for _ in range(3):
            kvq.calibrate_fit(xk, s.dtype, kvq.AXIS_KEY, q, 2, 8, workspace=ws)
            kvq.calibrate_fit(xv, s.dtype, kvq.AXIS_VALUE, q, 2, 8, workspace=ws)
    torch.cuda.synchronize()
    print(f"probe {kind} done", flush=True)


def traffic_probe():
    """The launches behind the committed FETCH_SIZE / WRITE_SIZE summary of the headline
    decode: the copy, then 30 split-K decode launches of qwen8b_t32k over 5 rotating caches."""
    probe("decode", WORKLOAD)


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


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "decode_kernel_qwen8b_t32k_traffic.txt")
KERNEL_SRCS = [os.path.join(os.path.dirname(os.path.abspath(__file__)), "mixed_precision_quantized_kvq_amd", f)
               for f in ("csrc/decode.hip", "csrc/code_plans.h", "csrc/kvq_internal.h", "build.py")]


def kernel_sources_sha256():
    """sha256 over the decode kernel's sources, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode launch from the committed FETCH_SIZE + WRITE_SIZE summary, or None
    when that summary was taken on another version of the kernel sources (sha256 mismatch)."""
    try:
        fields = dict(l.split("=", 1) for l in open(TRAFFIC_FILE).read().split()
                      if "=" in l and not l.startswith("#"))
        if fields.get("decode_sources_sha256") != kernel_sources_sha256():
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _host_cpu():
    """CPU model name and the cores this process may run on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return model, avail, os.cpu_count() or avail


def _oracle_units(w, k_bits, v_bits, pairs):
    from oracle import kvq_oracle as O
    s = w["spec"]
    G = s.n_q // s.n_kv
    units = []
    for b, h in pairs:
        cfg1 = O.CacheConfig(1, 1, G, s.head_dim, w["tokens"], s.n_sink, s.n_recent, s.dtype,
                             s.quant, (k_bits[h],), (v_bits[h],))
        units.append((O.build_cache(w["k"][b:b + 1, h:h + 1], w["v"][b:b + 1, h:h + 1], cfg1),
                      w["q"][b:b + 1, h * G:(h + 1) * G]))
    return units


def _oracle_worker(args):
    """One process of the all-cores leg: decode its (row, KV head) units, built by the parent,
    until `seconds` pass (one BLAS thread); returns (decodes done, elapsed)."""
    units, seconds = args
    from threadpoolctl import threadpool_limits

    from oracle import kvq_oracle as O
    done = 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        while True:
            for oc, q in units:
                O.decode(oc, q)
                done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return done, el


def cpu_baseline(w, k_bits, v_bits, seconds):
    """The float64 oracle's decode timed on the host, over (row, KV head) units of the same
    workload (each unit's cache built beforehand, outside the timing): first on one core (one
    process, one BLAS thread), then on every available core up to 16 (one process per core,
    each decoding its own units with one BLAS thread). The oracle holds its codes unpacked,
    so a decode is dequantization plus float64 attention."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits

    from oracle import kvq_oracle as O
    s = w["spec"]
    model, avail, n_cpu = _host_cpu()
    pairs = [(b, h) for b in range(s.batch) for h in range(s.n_kv)]
    all_units = _oracle_units(w, k_bits, v_bits, pairs)
    one = all_units[::4]
    done = 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        while True:
            for oc, q in one:
                O.decode(oc, q)
                done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    res = {"value": done * w["tokens"] / el, "unit": "KV tokens*heads/s", "cores": 1, "kind": "oracle",
           "sample": f"{len(one)} of {len(pairs)} (row, KV head) units of {WORKLOAD}, {done} float64 decodes "
                     f"in {el:.1f} s on one core (dequantize + attention; codes held unpacked)",
           "host_cpu": model, "host_cpus_available": avail, "host_cpus_total": n_cpu}
    n_proc = max(1, min(16, avail, len(all_units)))
    if n_proc > 1:
        per = [all_units[i::n_proc] for i in range(n_proc)]
        with mp.get_context("spawn").Pool(n_proc) as pool:
            out = pool.map(_oracle_worker, [(u, seconds) for u in per])
        res["all_cores"] = {
            "value": sum(d * w["tokens"] / e for d, e in out), "unit": "KV tokens*heads/s", "cores": n_proc,
            "sample": f"all {len(pairs)} (row, KV head) units over {n_proc} processes, "
                      f"{sum(d for d, _ in out)} float64 decodes in {max(e for _, e in out):.1f} s"}
    return res


def workload_bits(kvq, w, xk=None, xv=None):
    """Per-KV-head (K, V) widths of a workload: fixed, one joint or two separate allocations,
    or calibration (on device) followed by allocation."""
    s = w["spec"]
    if s.alloc == "fixed":
        return list(s.fixed_bits), list(s.fixed_bits)
    if s.alloc == "joint":
        b, _ = kvq.allocate_bits(w["alpha"], w["beta"], w["w"], s.k_total, s.b_lo, s.b_hi)
        return list(b), list(b)
    if s.alloc == "separate":
        kb, _ = kvq.allocate_bits(w["alpha_k"], w["beta_k"], w["w_k"], s.k_total, s.b_lo, s.b_hi)
        vb, _ = kvq.allocate_bits(w["alpha_v"], w["beta_v"], w["w_v"], s.v_total, s.b_lo, s.b_hi)
        return list(kb), list(vb)
    fk = kvq.calibrate_fit(xk, s.dtype, kvq.AXIS_KEY, kvq.QUANT_ASYM, 2, 8)
    fv = kvq.calibrate_fit(xv, s.dtype, kvq.AXIS_VALUE, kvq.QUANT_ASYM, 2, 8)
    kb, _ = kvq.allocate_bits(fk[0], fk[1], w["w_k"], s.k_total, s.b_lo, s.b_hi)
    vb, _ = kvq.allocate_bits(fv[0], fv[1], w["w_v"], s.v_total, s.b_lo, s.b_hi)
    return list(kb), list(vb)


def other_configs():
    """The other full-size workloads, one GPU: split-K decode time (and split-K + merge time) of
    the 8k-token Llama-shaped layer, of the 128k-token context and of the 32k-token workload with
    per-channel key normalization (caches rotated so their reads come from HBM, launches back to
    back behind a spin kernel, HIP events on the launch stream), decode + merge of one and of several query
    tokens per row on the multi-head 7B-shaped layer and on the 32k-token GQA workload, a ragged serving step (rows of 32767,
    28000, 20000 and 12000 tokens; host loop, append + decode + merge), and the ingest rate of the 16 x
    4096-token prefill (calibration, allocation, then one append of every token), with and
    without key normalization."""
    import torch

    import mixed_precision_quantized_kvq_amd as kvq
    import workloads
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    res = {}
    for name, n_inst, key_norm in (("llama8b_t8k", 5, False), ("long_t128k", 3, False),
                                   ("qwen8b_t32k", 5, True)):
        w = workloads.make(name)
        s = w["spec"]
        kb, vb = workload_bits(kvq, w)
        cfg = kvq.Config.make(s.batch, s.n_kv, s.n_q, s.head_dim, s.tokens, s.n_sink, s.n_recent, s.dtype,
                              s.quant, kb, vb, key_norm=key_norm)
        kd = torch.from_numpy(w["k"].view(np.int16)).to(dev)
        vd = torch.from_numpy(w["v"].view(np.int16)).to(dev)
        caches = []
        for _ in range(n_inst):
            c = kvq.KVCache(cfg, device=dev)
            kvq.append(c, kd, vd)
            caches.append(c)
        del kd, vd
        q = torch.from_numpy(w["q"].view(np.int16)).to(dev)
        ws = torch.zeros(kvq.decode_workspace_bytes(caches[0], s.n_splits), dtype=torch.uint8, device=dev)
        for i in range(10):
            kvq.decode_splitk(caches[i % n_inst], q, s.n_splits, ws, stream=stream)
        t_us = []
        for _ in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(20_000_000)
            e0.record(stream)
            for i in range(50):
                kvq.decode_splitk(caches[i % n_inst], q, s.n_splits, ws, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            t_us.append(e0.elapsed_time(e1) * 1e3 / 50)
        us = float(np.median(t_us))
        # the whole call: split-K launch and merge launch, same method
        out = torch.empty((s.batch, s.n_q, s.head_dim), dtype=torch.float32, device=dev)
        t_us = []
        for _ in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(20_000_000)
            e0.record(stream)
            for i in range(50):
                kvq.decode_attention(caches[i % n_inst], q, out, s.n_splits, ws, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            t_us.append(e0.elapsed_time(e1) * 1e3 / 50)
        us_merge = float(np.median(t_us))
        nbytes = decode_bytes(s, kb, vb, s.tokens, s.n_splits)
        res[name + ("_key_norm" if key_norm else "")] = {"decode_us": us, "decode_merge_us": us_merge,
                     "bytes_per_launch": nbytes, "achieved_gbs": nbytes / (us * 1e-6) / 1e9,
                     "frac_of_8tbs": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "k_bits": kb, "v_bits": vb,
                     "n_splits": s.n_splits, "kv_tokens_heads_per_s": s.batch * s.n_kv * s.tokens / (us * 1e-6)}
        del caches, ws, q, out
        torch.cuda.empty_cache()
    # the 32k-token workload on paged caches: 64-token pages dealt to (row, tile) from a pool
    # in a shuffled order, one permutation per cache instance
    w = workloads.make("qwen8b_t32k")
    s = w["spec"]
    kb, vb = workload_bits(kvq, w)
    cfg = kvq.Config.make(s.batch, s.n_kv, s.n_q, s.head_dim, s.tokens, s.n_sink, s.n_recent, s.dtype, s.quant,
                          kb, vb)
    stride = (32 * max(0, (s.tokens - s.n_sink - s.n_recent) // 32) // 32 + 1) // 2
    n_pages = s.batch * stride + 64
    kd = torch.from_numpy(w["k"].view(np.int16)).to(dev)
    vd = torch.from_numpy(w["v"].view(np.int16)).to(dev)
    rng = np.random.default_rng(2)
    caches = []
    for _ in range(5):
        c = kvq.cache_init_paged(cfg, n_pages, device=dev)
        perm = rng.permutation(n_pages)[:s.batch * stride].reshape(s.batch, stride)
        for b in range(s.batch):
            c.map_pages(b, 0, perm[b].tolist())
        kvq.append(c, kd, vd)
        caches.append(c)
    torch.cuda.synchronize()
    for c in caches:
        kvq.cache_check(c)
    del kd, vd
    q = torch.from_numpy(w["q"].view(np.int16)).to(dev)
    ws = torch.zeros(kvq.decode_workspace_bytes(caches[0], s.n_splits), dtype=torch.uint8, device=dev)
    for i in range(10):
        kvq.decode_splitk(caches[i % 5], q, s.n_splits, ws, stream=stream)
    t_us = []
    for _ in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(20_000_000)
        e0.record(stream)
        for i in range(50):
            kvq.decode_splitk(caches[i % 5], q, s.n_splits, ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        t_us.append(e0.elapsed_time(e1) * 1e3 / 50)
    us = float(np.median(t_us))
    nbytes = decode_bytes(s, kb, vb, s.tokens, s.n_splits)
    res["qwen8b_t32k_paged"] = {"decode_us": us, "bytes_per_launch": nbytes, "achieved_gbs": nbytes / (us * 1e-6) / 1e9,
                                "frac_of_8tbs": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "n_pages": n_pages,
                                "page_tokens": 64, "n_splits": s.n_splits,
                                "kv_tokens_heads_per_s": s.batch * s.n_kv * s.tokens / (us * 1e-6)}
    del caches, ws, q
    torch.cuda.empty_cache()
    # multi-token decode (decode + merge launches): the last Q tokens of every row at once.
    # The multi-head 7B-shaped layer has 1 query head per KV head (Q = 4: 4 query rows per KV
    # head, the single-query kernel's tile); the 32k-token GQA workload has 4 (Q = 2, 4: 8 and
    # 16 rows, the 16-row tile), against one query token per row
    for name, qs in (("mha7b_t8k", (1, 4)), ("qwen8b_t32k", (1, 2, 4))):
        w = workloads.make(name)
        s = w["spec"]
        kb, vb = workload_bits(kvq, w)
        cfg = kvq.Config.make(s.batch, s.n_kv, s.n_q, s.head_dim, s.tokens, s.n_sink, s.n_recent, s.dtype, s.quant,
                              kb, vb)
        kd = torch.from_numpy(w["k"].view(np.int16)).to(dev)
        vd = torch.from_numpy(w["v"].view(np.int16)).to(dev)
        caches = []
        for _ in range(5):
            c = kvq.KVCache(cfg, device=dev)
            kvq.append(c, kd, vd)
            caches.append(c)
        del kd, vd
        qsrc = w["q_multi"] if "q_multi" in w else workloads.random_raw16(
            np.random.default_rng(4242), (s.batch, 4, s.n_q, s.head_dim), s.dtype)
        qm = torch.from_numpy(qsrc.view(np.int16)).to(dev)
        nbytes = decode_bytes(s, kb, vb, s.tokens, s.n_splits)
        multi = {"k_bits": kb, "v_bits": vb, "n_splits": s.n_splits, "query_heads_per_kv_head": s.n_q // s.n_kv,
                 "bytes_per_launch_q1": nbytes}
        for Q in qs:
            q = qm[:, 4 - Q:].contiguous()
            out = torch.empty(q.shape, dtype=torch.float32, device=dev)
            ws = torch.zeros(kvq.decode_multi_workspace_bytes(caches[0], s.n_splits, Q), dtype=torch.uint8,
                             device=dev)
            for i in range(10):
                kvq.decode_multi(caches[i % 5], q, out, s.n_splits, ws, stream=stream)
            t_us = []
            for _ in range(4):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(20_000_000)
                e0.record(stream)
                for i in range(50):
                    kvq.decode_multi(caches[i % 5], q, out, s.n_splits, ws, stream=stream)
                e1.record(stream)
                torch.cuda.synchronize()
                t_us.append(e0.elapsed_time(e1) * 1e3 / 50)
            us = float(np.median(t_us))
            multi[f"q{Q}_us"] = us
            multi[f"q{Q}_query_tokens_per_s"] = s.batch * Q / (us * 1e-6)
            multi[f"q{Q}_frac_of_8tbs"] = nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS
        res[name + "_multi_token"] = multi
        del caches, qm
        torch.cuda.empty_cache()
    # ragged serving step on the 32k-token workload: the four rows hold 32767, 28000, 20000 and
    # 12000 tokens; one step appends one token to every row and decodes one query per row
    w = workloads.make("qwen8b_t32k")
    s = w["spec"]
    kb, vb = workload_bits(kvq, w)
    cfg = kvq.Config.make(s.batch, s.n_kv, s.n_q, s.head_dim, s.tokens + 256, s.n_sink, s.n_recent, s.dtype,
                          s.quant, kb, vb)
    lens0 = [32767, 28000, 20000, 12000]
    kd = torch.from_numpy(w["k"][:, :, :max(lens0)].view(np.int16)).to(dev)
    vd = torch.from_numpy(w["v"][:, :, :max(lens0)].view(np.int16)).to(dev)
    rcaches = []
    for _ in range(3):
        c = kvq.KVCache(cfg, device=dev)
        kvq.append_ragged(c, [0] * s.batch, lens0, kd, vd)
        rcaches.append(c)
    k1 = torch.from_numpy(np.ascontiguousarray(w["k"][:, :, -1:]).view(np.int16)).to(dev)
    v1 = torch.from_numpy(np.ascontiguousarray(w["v"][:, :, -1:]).view(np.int16)).to(dev)
    q = torch.from_numpy(w["q"].view(np.int16)).to(dev)
    out = torch.empty((s.batch, s.n_q, s.head_dim), dtype=torch.float32, device=dev)
    ws = torch.zeros(kvq.decode_workspace_bytes(rcaches[0], s.n_splits), dtype=torch.uint8, device=dev)
    lens = [list(lens0) for _ in rcaches]
    n_steps = 60
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)
    e0.record(stream)
    for i in range(n_steps):
        c, L = rcaches[i % 3], lens[i % 3]
        kvq.append_ragged(c, L, [1] * s.batch, k1, v1, stream=stream)
        for b in range(s.batch):
            L[b] += 1
        kvq.decode_ragged(c, L, q, out, s.n_splits, ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3 / n_steps
    tok = sum(lens0) + s.batch * n_steps // 2
    res["qwen8b_t32k_ragged_step"] = {"row_lengths": lens0, "step_us": step_us,
                                      "kv_tokens_heads_per_s": tok * s.n_kv / (step_us * 1e-6),
                                      "step": "append_ragged 1 token per row + decode_ragged + merge"}
    del rcaches, kd, vd
    torch.cuda.empty_cache()
    # prefill ingest
    w = workloads.make("prefill_t4k")
    s = w["spec"]
    xk = torch.from_numpy(np.ascontiguousarray(w["k"][0, :, :s.calib_tokens]).view(np.int16)).to(dev)
    xv = torch.from_numpy(np.ascontiguousarray(w["v"][0, :, :s.calib_tokens]).view(np.int16)).to(dev)
    kb, vb = workload_bits(kvq, w, xk, xv)
    kd = torch.from_numpy(w["k"].view(np.int16)).to(dev)
    vd = torch.from_numpy(w["v"].view(np.int16)).to(dev)
    for key_norm in (False, True):
        cfg = kvq.Config.make(s.batch, s.n_kv, s.n_q, s.head_dim, s.tokens, s.n_sink, s.n_recent, s.dtype,
                              s.quant, kb, vb, key_norm=key_norm)
        ms = []
        for _ in range(4):
            c = kvq.KVCache(cfg, device=dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            # the launches queue behind a spin kernel, so the events time the GPU's work and
            # not the host's launch latency
            torch.cuda._sleep(5_000_000)
            e0.record(stream)
            kvq.append(c, kd, vd, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            kvq.cache_check(c)
            ms.append(e0.elapsed_time(e1))
            del c
        in_bytes = 2 * kd.numel() * 2
        t = float(np.median(ms[1:]))
        res["prefill_t4k" + ("_key_norm" if key_norm else "")] = {
            "append_ms": t, "input_bytes": in_bytes, "ingest_gbs": in_bytes / (t * 1e-3) / 1e9,
            "tokens_per_s": s.batch * s.tokens / (t * 1e-3), "k_bits": kb, "v_bits": vb}
    return res


def model_calibration():
    """Whole-model offline stage on one GPU: calibration + fit of every (layer, KV head) pair
    of a Qwen3-8B-shaped model (36 x 8 = 288 pairs, 16 x 512 tokens each, keys and values
    separately, widths 2..8), then the K and V bit allocations over all 288 pairs. Inputs are
    resident on the GPU; each call blocks until its result is on the host."""
    import torch

    import mixed_precision_quantized_kvq_amd as kvq
    import workloads
    dev = torch.device("cuda:0")
    m = workloads.make_model_calib()
    s = m["spec"]
    P, T, D = s.pairs, s.tokens, s.head_dim
    xk = torch.from_numpy(m["k"].view(np.int16)).to(dev)
    xv = torch.from_numpy(m["v"].view(np.int16)).to(dev)
    del m["k"], m["v"]
    ws = torch.empty(kvq.calibrate_workspace_bytes(P, T, D, 2, 8), dtype=torch.uint8, device=dev)
    q = kvq.QUANT_HYBRID if s.quant == "hybrid" else kvq.QUANT_ASYM
    kvq.calibrate_fit(xk, s.dtype, kvq.AXIS_KEY, q, 2, 8, workspace=ws)  # warm-up
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        ak, bk, _ = kvq.calibrate_fit(xk, s.dtype, kvq.AXIS_KEY, q, 2, 8, workspace=ws)
        t1 = time.perf_counter()
        av, bv, _ = kvq.calibrate_fit(xv, s.dtype, kvq.AXIS_VALUE, q, 2, 8, workspace=ws)
        t2 = time.perf_counter()
        kb, _ = kvq.allocate_bits(ak, bk, m["w_k"], m["k_total"], s.b_lo, s.b_hi)
        vb, _ = kvq.allocate_bits(av, bv, m["w_v"], m["v_total"], s.b_lo, s.b_hi)
        t3 = time.perf_counter()
        runs.append((t1 - t0, t2 - t1, t3 - t2, t3 - t0))
    ck, cv, al, tot = (float(np.median([r[i] for r in runs])) * 1e3 for i in range(4))
    in_bytes = 2 * P * T * D * 2
    return {"workload": s.name, "pairs": P, "tokens_per_pair": T, "head_dim": D, "widths": "2..8",
            "calibrate_k_ms": ck, "calibrate_v_ms": cv, "allocate_k_plus_v_ms": al, "total_ms": tot,
            "input_bytes": in_bytes, "input_gbs": in_bytes / ((ck + cv) * 1e-3) / 1e9,
            "k_bits_count": {b: kb.count(b) for b in (2, 3, 4)},
            "v_bits_count": {b: vb.count(b) for b in (2, 3, 4)}}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (the decode path has no multi-GPU "
              "stage); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.traffic_probe:
        traffic_probe()
        return
    if args.probe:
        probe(args.probe, args.workload)
        return
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
    steps_per_inst = (args.steps + args.warmup + 160 + args.instances - 1) // args.instances + 1
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

    def step(i):
        # one decode step = append the new token + split-K decode + merge, in one call (the
        # split-K launch attends to the new token from the inputs, the merge launch stores it
        # in the recent window; a 32-token block leaving the window is quantized first)
        c = caches[i % len(caches)]
        kvq.decode_step(c, newk[i % n_new], newv[i % n_new], q, out, s.n_splits, ws, stream=stream)
        return c.len

    for i in range(args.warmup):
        step(i)
    toks = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        toks += step(args.warmup + i) * B * H
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    done = args.warmup + args.steps
    T_mean = toks / (args.steps * B * H)

    # ---- GPU time of a step without host gaps: steps queued behind a spin kernel, events on
    # the launch stream around the batch (a 160-step batch holds the 5 flushes per 160 steps
    # that the rotation over 5 caches gives)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_gpu_steps = 160
    torch.cuda._sleep(50_000_000)
    e0.record(stream)
    for i in range(n_gpu_steps):
        step(done + i)
    e1.record(stream)
    torch.cuda.synchronize()
    step_gpu_us = e0.elapsed_time(e1) * 1e3 / n_gpu_steps
    for c in caches:
        kvq.cache_check(c)

    # ---- the split-K kernel alone, for the roofline: launches queued back to back behind a
    # spin kernel (so the host is ahead and no launch gap enters the events), rotating over
    # the cache instances; events on the launch stream bracket each batch
    n_batch, per_batch = 4, 50
    t_us = []
    for _ in range(n_batch):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(20_000_000)
        e0.record(stream)
        for i in range(per_batch):
            kvq.decode_splitk(caches[i % len(caches)], q, s.n_splits, ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        t_us.append(e0.elapsed_time(e1) * 1e3 / per_batch)
    dec_us = float(np.median(t_us))
    T_now = int(round(np.mean([c.len for c in caches])))
    nbytes = decode_bytes(s, k_bits, v_bits, T_now, s.n_splits)
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
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "decode_kernel (split-K fused-dequant decode), HIP events around "
                               f"{n_batch}x{per_batch} back-to-back launches",
                     "bytes_per_launch": nbytes, "avg_us": dec_us, "context": T_now},
        "step_gpu_us": step_gpu_us,
        "offline": {"allocate_bits_us": alloc_us, "calibrate_fit_ms_k_plus_v": calib_ms,
                    # the whole-prefill append that builds each timed cache (hybrid groups)
                    "cache_build_append_ms": float(np.median(prefill_ms)),
                    "cache_build_ingest_gbs": (B * H * T0 * D * 4) / (float(np.median(prefill_ms)) * 1e-3) / 1e9},
    }
    if not args.no_other_configs:
        res["other_configs"] = other_configs()
        res["offline"]["model_calibrate_allocate"] = model_calibration()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, k_bits, v_bits, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
