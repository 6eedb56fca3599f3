#!/usr/bin/env python3
"""Throughput of the product-VQ encode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

A step is one call of the whole hot path (``vq_encode`` through the C ABI)
over one batch of synthetic input.  The default workload is the Falcon3-7B
key-cache shape of the VeloxQuant-MLX post "I Wrote a Metal Kernel to Stop My
Mac From OOMing" (section "What quantize_vq Was Doing Wrong": 4096 tokens x 4
KV heads x head_dim 256, sub_dim 4 -> 1,048,576 sub-vectors, 256 centroids),
with seeded per-channel-scaled Gaussian keys and outlier channels.  Inputs are
resident in HBM before the timed region starts.

Printed: one JSON line.  Headline: sub-vectors/s over the timed region (W
untimed warmup steps, then K steps between synchronisations) and the encode
kernel's roofline position: algorithmic fp32 flops per launch divided by the
launch's average duration (HIP events on the launch stream) against the
MI355X fp32 vector peak.  The flops are those of the direct form, 3 * sub_dim
* n_centroids per sub-vector (a subtraction, a multiply and an add per
component per centroid).  The kernel does not execute them: it bounds the
distances on the matrix cores and recomputes a few candidates exactly, so the
figure is a direct-form-equivalent rate, which can exceed the vector peak on
large codebooks.  What binds the kernel is read from rocprofv3 counters
committed under profiles/ and reported next to it (``utilization``: VALU
issue busy, matrix-core busy, shader clock), as is the HBM traffic.

``cpu_baseline`` is the CPU oracle on the host: on all host threads (the
headline baseline, ``cores`` = threads used) and on one core, with the CPU
model.  Its all-thread run covers every row of the Falcon-shape workload and
supplies the parity sample.

``--configs`` adds the other encode workloads as rows (default all four):
  config1  tiny: 2,048 sub-vectors, 256 centroids of sub_dim 8 (launch-bound)
  config2  Llama-3.1-8B keys: 524,288 sub-vectors, sub_dim 8
  config4  full batched cache: 33,554,432 sub-vectors, 256 codebook slots
  config5  large codebook: 1,048,576 bf16 sub-vectors, 4,096 centroids
``--rows`` adds the steps adjacent to the encode:
  fused  ``vq_encode_packed``: per-channel smoothing + 8-bit packed codes on
         the smoothed Falcon3-7B-shape cache.
  attention  ``vq_attention_decode``: one decode step of Falcon3-7B (32
         sequences, 12 query / 4 KV heads, head_dim 256, lengths U[2048,
         4096]) over 8-bit key/value codes; HBM roofline on the algorithmic
         bytes (attended codes, queries, outputs, codebooks, factors).
  kmeans  ``vq_kmeans``: 5 Lloyd iterations per call on the Falcon3-7B keys
         (1,048,576 sub-vectors, 256 centroids, sub_dim 4); fp32 vector
         roofline on the assignment's algorithmic flops.
  kmeans_bf16  the same on the large-codebook workload (1,048,576 bf16
         sub-vectors, 4,096 centroids of sub_dim 8).
Every row is timed after a short GPU warm-up: its launches are enqueued
behind a short spin kernel, so the events measure the launches back to back
(``kernel_ms_per_launch``) however fast the host enqueues; ``host_ms_per_call``
is the wall time per call of the same loop.  ``--only ROW`` runs one row
alone (for profiling its kernel).  ``--ab PKG_A PKG_B --ab-row ROW`` compares
two builds of the library on one row in the same process, in alternating
rounds of launches (package directories: this one, and a copy built from
another revision).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP32_VECTOR_PEAK_TFLOPS = 157.3   # MI355X published fp32 vector peak (2.4 GHz)
PEAK_CLOCK_GHZ = 2.4
HBM_PEAK_GBS = 8000.0             # MI355X published HBM3E bandwidth
# Pages' own figure for the same workload, on an Apple-Silicon GPU (context):
# 1,048,576 sub-vectors in 7.98 ms (post's "The Numbers" throughput table).
PAGES_FALCON_SUBVEC_PER_S = 1048576 / 7.98e-3
KMEANS_ITERATIONS = 5
KERNEL_SOURCES = os.path.join(ROOT, "product_vq_kv_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# profile summary name of each encode workload
CONFIG_TAGS = {1: "encode_tiny", 2: "encode_llama8b", 3: "encode_falcon3", 4: "encode_full_cache",
               5: "encode_large_codebook"}
ROW_TAGS = {"fused": "encode_fused_falcon3", "attention": "attention_falcon3_decode",
            "kmeans": "kmeans_falcon3", "kmeans_bf16": "kmeans_bf16_large_codebook"}
# sequence counts of the attention row with a profile of their own (the
# streaming form runs at 128)
ATTENTION_BATCH_TAGS = {128: "attention_falcon3_decode_b128"}
# rows of each config the oracle checks in the bench (the tests check all)
PARITY_ROWS = {1: 2048, 2: 1 << 18, 4: 1 << 18, 5: 1 << 14}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# The sources each profiled kernel is built from: a counter summary stays
# valid while these files are unchanged.
ENCODE_SOURCES = ("vq_encode_mfma.hip", "vq_codes.h")
ATTENTION_SOURCES = ("vq_attention.hip",)
KMEANS_SOURCES = ("vq_encode_mfma.hip", "vq_codes.h", "vq_kmeans.hip")


def kernel_source_hash(names=ENCODE_SOURCES) -> str:
    """Hash of the named library sources (a change invalidates counter
    figures taken on an earlier build of that kernel)."""
    h = hashlib.sha256()
    for name in sorted(names):
        with open(os.path.join(KERNEL_SOURCES, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _summary_json(path: str):
    """The JSON line of a committed counter summary, or None when there is
    none or the kernel's sources changed since it was taken."""
    try:
        with open(path) as f:
            rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
        t = json.loads(rows[-1])
        names = tuple(t["kernel_sources"])
    except (OSError, ValueError, IndexError, KeyError, TypeError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash(names):
        return None
    return t


def traffic_bytes_per_launch(tag: str):
    """HBM bytes per launch from profiles/<tag>_traffic.txt (None if stale)."""
    t = _summary_json(os.path.join(PROFILES, f"{tag}_traffic.txt"))
    return None if t is None else t.get("hbm_bytes_per_launch")


def utilization(tag: str, launch_s: float):
    """Counter-derived busy fractions from profiles/<tag>_counters.txt (None
    if stale), and the shader clock of this run: the busy shader cycles per
    launch the counters measured (the kernel is compute-bound, so its cycle
    count does not depend on the clock) over the launch time measured here."""
    t = _summary_json(os.path.join(PROFILES, f"{tag}_counters.txt"))
    if t is None:
        return None
    keep = ("valu_busy", "mfma_busy", "valu_insts_per_wave", "lds_conflict_cycles_per_inst",
            "busy_cycles_per_launch")
    out = {k: t[k] for k in keep if k in t}
    if t.get("busy_cycles_per_launch"):
        out["sclk_ghz"] = t["busy_cycles_per_launch"] / launch_s / 1e9
        out["peak_tflops_at_sclk"] = FP32_VECTOR_PEAK_TFLOPS * out["sclk_ghz"] / PEAK_CLOCK_GHZ
    out["source"] = f"profiles/{tag}_counters.txt"
    return out


def kernel_counters(tag: str):
    """Counter-derived figures of the dominant kernel of a multi-launch row
    from profiles/<tag>_counters.txt (None if stale): busy fractions and
    instructions per wave, no clock (the row's time spans several launches)."""
    t = _summary_json(os.path.join(PROFILES, f"{tag}_counters.txt"))
    if t is None:
        return None
    c = t.get("counters", {})
    waves = t.get("waves") or 1.0
    out = {k: t[k] for k in ("kernel", "valu_busy", "mfma_busy", "valu_insts_per_wave",
                             "mfma_insts_per_wave", "lds_conflict_cycles_per_inst") if k in t}
    if "SQ_INSTS_LDS" in c:
        out["lds_insts_per_wave"] = c["SQ_INSTS_LDS"] / waves
    out["source"] = f"profiles/{tag}_counters.txt"
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Threads the host grants this process (the GPU machine sets OMP_NUM_THREADS
    to its CPU share)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return len(os.sched_getaffinity(0))


def cpu_baseline(wl, rows_one: int, rows_all: int):
    """The oracle on one core and on all host threads (same single-threaded C
    routine per slice; results do not depend on the slicing).  Returns the
    all-thread indices and the baseline object."""
    import numpy as np
    import oracle
    threads = host_threads()
    rows_one = min(rows_one, wl.n)
    rows_all = min(rows_all, wl.n)
    t0 = time.perf_counter()
    oracle.encode(np.ascontiguousarray(wl.x[:rows_one]), wl.codebook, wl.sub_dim,
                  wl.n_centroids, wl.dtype, threads=1)
    dt1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    idx = oracle.encode(np.ascontiguousarray(wl.x[:rows_all]), wl.codebook, wl.sub_dim,
                        wl.n_centroids, wl.dtype, threads=threads)
    dta = time.perf_counter() - t0
    model = cpu_model()
    return idx, dict(
        value=rows_all / dta, unit="sub-vectors/s", cores=threads, kind="oracle",
        sample=f"first {rows_all} of {wl.n} sub-vectors of the same workload, {threads} threads "
               f"slicing the rows, {dta:.1f} s",
        cpu_model=model, host_cpus_visible=len(os.sched_getaffinity(0)),
        one_core=dict(value=rows_one / dt1, unit="sub-vectors/s", cores=1,
                      sample=f"first {rows_one} sub-vectors, one thread, {dt1:.1f} s"))


def copy_calibration(torch, dev) -> None:
    """Plain copy of 256 MiB, five times: the counter scale reference."""
    src = torch.empty(1 << 26, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: 5 x 268435456-byte device copies")


def time_row(fn, steps: int, stream, warm_s: float = 0.05):
    """(host seconds per call, GPU seconds per launch) over `steps` calls.

    A warm-up of `warm_s` seconds of calls first (the shader clock drops
    while the GPU idles, e.g. during the CPU baseline).  The timed launches
    are enqueued behind a spin kernel, so the events bracket them back to
    back even when the host enqueues more slowly than the GPU runs them."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    # long enough for the host to enqueue every launch first (~25 us per call)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(2.0e9 * max(0.01, 25e-6 * steps)))
    e0.record(stream)
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    host = (time.perf_counter() - t0) / steps
    e1.record(stream)
    torch.cuda.synchronize()
    return host, e0.elapsed_time(e1) / 1e3 / steps


def encode_roofline(wl, launch_s: float, tag: str):
    flops = 3.0 * wl.sub_dim * wl.n_centroids * wl.n
    achieved = flops / launch_s / 1e12
    return {"bound": "alu", "achieved": achieved, "peak": FP32_VECTOR_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / FP32_VECTOR_PEAK_TFLOPS,
            "traffic": traffic_bytes_per_launch(tag)}


def encode_bytes(wl) -> float:
    """Algorithmic HBM bytes of one encode launch: keys, indices, codebooks."""
    return wl.n * (2 * wl.sub_dim + 4) + wl.n_codebooks * wl.n_centroids * wl.sub_dim * 2


def leg_config(cfg: int):
    def leg(args, dev, stream):
        import numpy as np
        import torch
        import workloads as W
        import product_vq_kv_amd as vq
        from tests import parity
        wl = W.config(cfg)
        log(f"row config{cfg}: {wl.name} (n={wl.n})")
        tdt = torch.float16 if wl.dtype == W.F16 else torch.bfloat16
        x = torch.from_numpy(wl.x.view(np.int16)).view(tdt).to(dev)
        cb = torch.from_numpy(wl.codebook.view(np.int16)).view(tdt).to(dev)
        out = torch.empty(wl.n, dtype=torch.uint32, device=dev)
        call = (x.data_ptr(), cb.data_ptr(), wl.n, wl.sub_dim, wl.n_centroids, wl.dtype,
                wl.codebook_stride, wl.n_codebooks, wl.group_len, None, out.data_ptr(),
                stream.cuda_stream)
        steps = max(args.steps, 20)
        host, launch_s = time_row(lambda: vq.encode_raw(*call), steps, stream)
        parity_sample = None
        if args.cpu_sample > 0:
            got = out.cpu().numpy().view(np.uint32)
            k = min(PARITY_ROWS.get(cfg, 1 << 16), wl.n)
            rows = np.sort(np.random.default_rng(cfg).choice(wl.n, size=k, replace=False))
            ref = parity.oracle_indices(wl, rows, threads=host_threads())
            parity_sample = dict(rows=int(k), equal=int(np.sum(ref == got[rows])),
                                 threads=host_threads())
        tag = CONFIG_TAGS[cfg]
        gbs = encode_bytes(wl) / launch_s / 1e9
        return {
            "workload": wl.name,
            "value": wl.n / launch_s,
            "unit": "sub-vectors/s",
            "kernel_ms_per_launch": launch_s * 1e3,
            "host_ms_per_call": host * 1e3,
            "launches": steps,
            "roofline": encode_roofline(wl, launch_s, tag),
            "utilization": utilization(tag, launch_s),
            "algorithmic_gb_per_s": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS,
            "parity_sample": parity_sample,
        }
    return leg


def leg_fused(args, dev, stream):
    """Smoothed keys, 8-bit codes (vq_encode_packed) on the Falcon3-7B shape."""
    import numpy as np
    import torch
    import workloads as W
    import product_vq_kv_amd as vq
    wl = W.falcon_smoothed()
    log(f"row fused: {wl.name} (n={wl.n})")
    x = torch.from_numpy(wl.x.view(np.int16)).view(torch.float16).to(dev)
    cb = torch.from_numpy(wl.codebook.view(np.int16)).view(torch.float16).to(dev)
    sc = torch.from_numpy(wl.channel_scale[0]).to(dev)
    bits = 8
    out = torch.empty(vq.packed_bytes(wl.n, bits), dtype=torch.uint8, device=dev)
    call = (x.data_ptr(), cb.data_ptr(), wl.n, wl.sub_dim, wl.n_centroids, wl.dtype,
            wl.codebook_stride, wl.n_codebooks, wl.group_len, None, sc.data_ptr(), wl.head_dim,
            0, bits, out.data_ptr(), stream.cuda_stream)
    steps = max(args.steps, 20)
    host, launch_s = time_row(lambda: vq.encode_packed_raw(*call), steps, stream)
    flops = 3.0 * wl.sub_dim * wl.n_centroids * wl.n
    algo_bytes = wl.n * (2 * wl.sub_dim + bits / 8) + wl.n_centroids * wl.sub_dim * 2 + wl.head_dim * 4
    achieved = flops / launch_s / 1e12
    parity = None
    if args.cpu_sample > 0:
        import oracle
        rows = min(args.cpu_sample // 4, wl.n)
        ref = oracle.encode_packed(wl.x[:rows], wl.codebook, wl.sub_dim, wl.n_centroids, wl.dtype,
                                   code_bits=bits, threads=host_threads(), **wl.packed_kwargs())
        got = out.cpu().numpy()[:ref.size]
        parity = dict(rows=int(rows), equal=int(np.sum(ref == got)))
    tag = ROW_TAGS["fused"]
    return {
        "workload": wl.name + ", 8-bit codes",
        "value": wl.n / launch_s,
        "unit": "sub-vectors/s",
        "kernel_ms_per_launch": launch_s * 1e3,
        "host_ms_per_call": host * 1e3,
        "launches": steps,
        "roofline": {"bound": "alu", "achieved": achieved, "peak": FP32_VECTOR_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / FP32_VECTOR_PEAK_TFLOPS,
                     "traffic": traffic_bytes_per_launch(tag)},
        "utilization": utilization(tag, launch_s),
        "algorithmic_gb_per_s": algo_bytes / launch_s / 1e9,
        "parity_sample": parity,
    }


def attention_call(wl, dev, stream):
    """Device buffers and the C-ABI argument tuple of one decode-attention call."""
    import numpy as np
    import torch
    import workloads as W
    import product_vq_kv_amd as vq
    B, Hq, Hkv, D, S = wl.shape

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).to(dev)

    keep = dict(q=bits(wl.q), kcb=bits(wl.k_codebook), vcb=bits(wl.v_codebook),
                kc=torch.from_numpy(wl.k_codes).to(dev), vc=torch.from_numpy(wl.v_codes).to(dev),
                ks=torch.from_numpy(wl.k_scale).to(dev), kl=torch.from_numpy(wl.kv_len).to(dev),
                out=torch.empty((B, Hq, D), dtype=torch.float32, device=dev))
    wsb = vq.attention_workspace_bytes(B, Hq, D, S)
    keep["ws"] = torch.empty(wsb, dtype=torch.uint8, device=dev)
    sdk, sdv = D // wl.k_codes.shape[3], D // wl.v_codes.shape[3]
    n_c = wl.k_codebook.shape[1]
    call = (keep["q"].data_ptr(), keep["kc"].data_ptr(), keep["vc"].data_ptr(),
            keep["kcb"].data_ptr(), keep["vcb"].data_ptr(), keep["ks"].data_ptr(),
            keep["kl"].data_ptr(), B, Hq, Hkv, D, S, sdk, sdv, n_c, W.F16, 0, 1.0 / D ** 0.5,
            keep["out"].data_ptr(), keep["ws"].data_ptr(), wsb, stream.cuda_stream)
    toks = int(np.sum(wl.kv_len)) * Hkv
    algo_bytes = (toks * (D // sdk + D // sdv) + B * Hq * D * (2 + 4)
                  + Hkv * n_c * (sdk + sdv) * 2 + Hkv * D * 4)
    return keep, call, algo_bytes


def leg_attention(args, dev, stream):
    """One decode-attention step over the VQ-coded Falcon3-7B cache, plus the
    same step at 64 and 128 sequences (the rate as the batch grows)."""
    import numpy as np
    import workloads as W
    import product_vq_kv_amd as vq
    wl = W.falcon_decode_attention()
    log(f"row attention: {wl.name}")
    B, Hq, Hkv, D, S = wl.shape
    keep, call, algo_bytes = attention_call(wl, dev, stream)
    steps = max(args.steps, 20)
    host, launch_s = time_row(lambda: vq.attention_decode_raw(*call), steps, stream)
    achieved = algo_bytes / launch_s / 1e9
    parity = None
    if args.cpu_sample > 0:
        from oracle import attention as A
        nb = 4
        ref = A.decode_attention(wl.q[:nb], wl.k_codes[:nb], wl.v_codes[:nb], wl.k_codebook,
                                 wl.v_codebook, wl.dtype, k_scale=wl.k_scale,
                                 kv_len=wl.kv_len[:nb])
        got = keep["out"].cpu().numpy()[:nb].astype(np.float64)
        parity = dict(sequences=nb, max_abs_err=float(np.max(np.abs(got - ref))),
                      max_abs_ref=float(np.max(np.abs(ref))))
    batches = {}
    for nb in [int(b) for b in args.attention_batches.split(",") if b]:
        wlb = W.falcon_decode_attention(B=nb)
        _, callb, bytes_b = attention_call(wlb, dev, stream)
        _, ls = time_row(lambda: vq.attention_decode_raw(*callb), steps, stream, warm_s=0.02)
        batches[str(nb)] = dict(kernel_ms_per_launch=ls * 1e3,
                                algorithmic_gb_per_s=bytes_b / ls / 1e9,
                                frac=bytes_b / ls / 1e9 / HBM_PEAK_GBS,
                                algorithmic_bytes_per_launch=bytes_b)
        if nb in ATTENTION_BATCH_TAGS:
            batches[str(nb)]["traffic"] = traffic_bytes_per_launch(ATTENTION_BATCH_TAGS[nb])
            batches[str(nb)]["partial_kernel_counters"] = kernel_counters(ATTENTION_BATCH_TAGS[nb])
    tag = ROW_TAGS["attention"]
    return {
        "workload": wl.name,
        "value": B / launch_s,
        "unit": "decode steps (sequences) / s",
        "kernel_ms_per_launch": launch_s * 1e3,
        "host_ms_per_call": host * 1e3,
        "launches": steps,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_bytes_per_launch(tag)},
        "partial_kernel_counters": kernel_counters(tag),
        "algorithmic_bytes_per_launch": algo_bytes,
        "tokens_attended_per_launch": int(np.sum(wl.kv_len)) * Hq,
        "by_batch": batches,
        "parity_sample": parity,
    }


def leg_kmeans(args, dev, stream, cfg: int = 3, tag: str = "kmeans"):
    """K-means calibration (Lloyd) on the Falcon3-7B keys (fp16), or on the
    large-codebook workload (bf16, 4,096 centroids; its parity is checked by
    the GPU tests, the oracle being too slow for a bench sample)."""
    import numpy as np
    import torch
    import workloads as W
    import product_vq_kv_amd as vq
    wl = W.config(cfg)
    log(f"row {tag}: {wl.name}, {KMEANS_ITERATIONS} iterations per call")
    tdt = torch.float16 if wl.dtype == W.F16 else torch.bfloat16
    x = torch.from_numpy(wl.x.view(np.int16)).view(tdt).to(dev)
    cb0 = torch.from_numpy(wl.codebook.view(np.int16)).view(tdt).to(dev)
    cb = cb0.clone()
    idx = torch.empty(wl.n, dtype=torch.uint32, device=dev)
    wsb = vq.kmeans_workspace_bytes(wl.sub_dim, wl.n_centroids, 1, wl.dtype)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    call = (x.data_ptr(), cb.data_ptr(), wl.n, wl.sub_dim, wl.n_centroids, wl.dtype,
            wl.codebook_stride, 1, wl.group_len, None, KMEANS_ITERATIONS, idx.data_ptr(),
            ws.data_ptr(), wsb, stream.cuda_stream)
    steps = max(args.steps, 20)
    host, launch_s = time_row(lambda: vq.kmeans_raw(*call), steps, stream)
    it_s = launch_s / KMEANS_ITERATIONS
    flops = 3.0 * wl.sub_dim * wl.n_centroids * wl.n
    achieved = flops / it_s / 1e12
    parity = None
    if args.cpu_sample > 0 and wl.n_centroids <= 256:
        # from the initial codebook, one call of the library against the oracle
        from oracle import kmeans as K
        cb.copy_(cb0)
        vq.kmeans_raw(*call)
        torch.cuda.synchronize()
        want_cb, want_idx, _ = K.kmeans(wl.x, wl.codebook, wl.sub_dim, wl.n_centroids,
                                        KMEANS_ITERATIONS, threads=host_threads())
        got_cb = cb.view(torch.int16).cpu().numpy().view(np.uint16)
        parity = dict(iterations=KMEANS_ITERATIONS,
                      codebook_equal=int(np.sum(got_cb == want_cb)), codebook_size=int(want_cb.size),
                      assignment_equal=int(np.sum(idx.cpu().numpy().view(np.uint32) == want_idx)),
                      rows=int(wl.n))
    tag = ROW_TAGS[tag]
    return {
        "workload": wl.name + f", Lloyd x{KMEANS_ITERATIONS} per call",
        "value": wl.n * KMEANS_ITERATIONS / launch_s,
        "unit": "sub-vector-iterations/s",
        "kernel_ms_per_launch": launch_s * 1e3,
        "host_ms_per_call": host * 1e3,
        "ms_per_iteration": it_s * 1e3,
        "launches": steps,
        "roofline": {"bound": "alu", "achieved": achieved, "peak": FP32_VECTOR_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / FP32_VECTOR_PEAK_TFLOPS,
                     "traffic": traffic_bytes_per_launch(tag)},
        "parity_sample": parity,
    }


ROW_LEGS = {"fused": leg_fused, "attention": leg_attention, "kmeans": leg_kmeans,
            "kmeans_bf16": lambda args, dev, stream: leg_kmeans(args, dev, stream, 5,
                                                                "kmeans_bf16")}
ROW_LEGS.update({f"config{c}": leg_config(c) for c in (1, 2, 4, 5)})


def load_binding(pkg_dir: str, name: str):
    """The binding module of another build of the library: `pkg_dir` holds a
    package's __init__.py and the libvq.so built beside it."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(name, os.path.join(pkg_dir, "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def ab_compare(args, dev, stream) -> dict:
    """Same-process A/B of two library builds on one row: both are loaded, and
    rounds of `ab_steps` launches alternate between them (A then B, then B
    then A, ...), so clock drift between runs does not enter the comparison."""
    import statistics
    import numpy as np
    import torch
    import workloads as W
    mods = [load_binding(os.path.abspath(d), f"_vq_ab{i}") for i, d in enumerate(args.ab)]
    keep = []
    cases = []  # (label, [launch function per build])
    row = args.ab_row
    if row == "attention":
        for nb in [int(b) for b in (args.attention_batches or "32").split(",") if b]:
            wl = W.falcon_decode_attention(B=nb)
            k, call, _ = attention_call(wl, dev, stream)
            keep.append(k)
            cases.append((f"{nb} sequences",
                          [lambda m=m, c=call: m.attention_decode_raw(*c) for m in mods]))
    elif row.startswith("config"):
        wl = W.config(int(row[len("config"):]))
        tdt = torch.float16 if wl.dtype == W.F16 else torch.bfloat16
        x = torch.from_numpy(wl.x.view(np.int16)).view(tdt).to(dev)
        cb = torch.from_numpy(wl.codebook.view(np.int16)).view(tdt).to(dev)
        out = torch.empty(wl.n, dtype=torch.uint32, device=dev)
        keep.append((x, cb, out))
        call = (x.data_ptr(), cb.data_ptr(), wl.n, wl.sub_dim, wl.n_centroids, wl.dtype,
                wl.codebook_stride, wl.n_codebooks, wl.group_len, None, out.data_ptr(),
                stream.cuda_stream)
        cases.append((wl.name, [lambda m=m: m.encode_raw(*call) for m in mods]))
    elif row == "fused":
        wl = W.falcon_smoothed()
        x = torch.from_numpy(wl.x.view(np.int16)).view(torch.float16).to(dev)
        cb = torch.from_numpy(wl.codebook.view(np.int16)).view(torch.float16).to(dev)
        sc = torch.from_numpy(wl.channel_scale[0]).to(dev)
        out = torch.empty(mods[0].packed_bytes(wl.n, 8), dtype=torch.uint8, device=dev)
        keep.append((x, cb, sc, out))
        call = (x.data_ptr(), cb.data_ptr(), wl.n, wl.sub_dim, wl.n_centroids, wl.dtype,
                wl.codebook_stride, wl.n_codebooks, wl.group_len, None, sc.data_ptr(), wl.head_dim,
                0, 8, out.data_ptr(), stream.cuda_stream)
        cases.append((wl.name + ", 8-bit codes", [lambda m=m: m.encode_packed_raw(*call) for m in mods]))
    elif row in ("kmeans", "kmeans_bf16"):
        wl = W.config(3 if row == "kmeans" else 5)
        tdt = torch.float16 if wl.dtype == W.F16 else torch.bfloat16
        x = torch.from_numpy(wl.x.view(np.int16)).view(tdt).to(dev)
        keep.append(x)
        fns = []
        for m in mods:  # each build with its own codebook copy and workspace size
            cb = torch.from_numpy(wl.codebook.view(np.int16)).view(tdt).to(dev)
            idx = torch.empty(wl.n, dtype=torch.uint32, device=dev)
            wsb = m.kmeans_workspace_bytes(wl.sub_dim, wl.n_centroids, 1, wl.dtype)
            ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
            keep.append((cb, idx, ws))
            c = (x.data_ptr(), cb.data_ptr(), wl.n, wl.sub_dim, wl.n_centroids, wl.dtype,
                 wl.codebook_stride, 1, wl.group_len, None, KMEANS_ITERATIONS, idx.data_ptr(),
                 ws.data_ptr(), wsb, stream.cuda_stream)
            fns.append(lambda m=m, c=c: m.kmeans_raw(*c))
        cases.append((wl.name + f", Lloyd x{KMEANS_ITERATIONS}", fns))
    else:
        raise SystemExit(f"--ab-row {row!r}: one of attention, config1..config5, fused, kmeans, kmeans_bf16")
    res = {}
    for label, fns in cases:
        t = [[], []]
        for r in range(args.ab_rounds):
            for i in ((0, 1) if r % 2 == 0 else (1, 0)):
                _, sec = time_row(fns[i], args.ab_steps, stream, warm_s=0.02)
                t[i].append(sec * 1e6)
        med = [statistics.median(v) for v in t]
        res[label] = {"A_us": med[0], "B_us": med[1], "B_over_A": med[1] / med[0],
                      "rounds_B_faster": sum(1 for a, b in zip(t[0], t[1]) if b < a),
                      "rounds": args.ab_rounds}
        log(f"ab {row} {label}: A {med[0]:.3f} us, B {med[1]:.3f} us, B/A {med[1] / med[0]:.4f}")
    return {"ab": {"row": row, "A": args.ab[0], "B": args.ab[1], "cases": res}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--cpu-sample", type=int, default=1 << 19,
                    help="rows the CPU oracle encodes on one core (0 = no CPU work at all)")
    ap.add_argument("--cpu-sample-all", type=int, default=1 << 22,
                    help="rows the CPU oracle encodes on all host threads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (counter scaling)")
    ap.add_argument("--configs", default="config1,config2,config4,config5",
                    help="comma-separated encode workloads to add as rows ('' = none)")
    ap.add_argument("--rows", default="fused,attention,kmeans,kmeans_bf16",
                    help="comma-separated adjacent rows to time after the headline ('' = none)")
    ap.add_argument("--attention-batches", default="64,128",
                    help="extra sequence counts the attention row is timed at ('' = none)")
    ap.add_argument("--only", choices=sorted(ROW_LEGS), default=None,
                    help="run only this row's leg and print its object")
    ap.add_argument("--ab", nargs=2, metavar=("PKG_A", "PKG_B"), default=None,
                    help="same-process A/B of two builds of the library (each a package "
                         "directory: __init__.py and the libvq.so built beside it) on --ab-row")
    ap.add_argument("--ab-row", default="config3",
                    help="attention (at --attention-batches, default 32), config1..config5, "
                         "fused, kmeans or kmeans_bf16")
    ap.add_argument("--ab-rounds", type=int, default=10)
    ap.add_argument("--ab-steps", type=int, default=300)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the encode step needs no exchange between "
              "GPUs, and this build runs on a single MI355X (see the sharding note in the "
              "design document).", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (there is no CPU path)", file=sys.stderr)
        return 2
    import product_vq_kv_amd as vq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.ab:
        print(json.dumps(ab_compare(args, dev, torch.cuda.current_stream(dev))), flush=True)
        return 0
    if args.only:
        res = ROW_LEGS[args.only](args, dev, torch.cuda.current_stream(dev))
        if args.copy_calibration:
            copy_calibration(torch, dev)
        print(json.dumps({args.only: res}), flush=True)
        return 0
    wl = W.config(args.config)
    log(f"workload: {wl.name} (n={wl.n})")
    tdt = torch.float16 if wl.dtype == W.F16 else torch.bfloat16
    x = torch.from_numpy(wl.x.view(np.int16)).view(tdt).to(dev)
    cb = torch.from_numpy(wl.codebook.view(np.int16)).view(tdt).to(dev)
    out = torch.empty(wl.n, dtype=torch.uint32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    call = (x.data_ptr(), cb.data_ptr(), wl.n, wl.sub_dim, wl.n_centroids, wl.dtype,
            wl.codebook_stride, wl.n_codebooks, wl.group_len, None, out.data_ptr(), sptr)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        vq.encode_raw(*call)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        vq.encode_raw(*call)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    log(f"timed {args.steps} steps: wall {wall * 1e3:.2f} ms, events {gpu_ms:.2f} ms")

    if args.copy_calibration:
        copy_calibration(torch, dev)

    ms_per_step = wall * 1e3 / args.steps
    launch_s = gpu_ms / 1e3 / args.steps
    algo_bytes = encode_bytes(wl)
    value = wl.n / (ms_per_step / 1e3)
    tag = CONFIG_TAGS[args.config]

    gpu_idx = out.cpu().numpy().view(np.uint32)
    cpu = None
    parity_sample = None
    if args.cpu_sample > 0:
        log(f"cpu baseline: oracle on {min(args.cpu_sample, wl.n)} rows on one core, "
            f"{min(args.cpu_sample_all, wl.n)} rows on {host_threads()} threads")
        ref, cpu = cpu_baseline(wl, args.cpu_sample, args.cpu_sample_all)
        parity_sample = dict(rows=int(ref.size), equal=int(np.sum(ref == gpu_idx[:ref.size])))

    cfg = dict(workload=wl.name, n_subvectors=wl.n, sub_dim=wl.sub_dim,
               n_centroids=wl.n_centroids, element="fp16" if wl.dtype == W.F16 else "bf16",
               n_codebooks=wl.n_codebooks, **{k: v for k, v in wl.meta.items()
                                               if isinstance(v, (int, float, str))})
    util = utilization(tag, launch_s)
    line = {
        "metric": "sub-vectors encoded/sec and % fp32 VALU peak (Falcon3-7B shape, 1 GPU)",
        "value": value,
        "unit": "sub-vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (value / PAGES_FALCON_SUBVEC_PER_S) if args.config == 3 else None,
        "dtype": "f32",
        "data": "synthetic (seeded; per-channel LogNormal-scaled Gaussian keys, outlier channels)",
        "config": cfg,
        "roofline": encode_roofline(wl, launch_s, tag),
        "roofline_note": ("achieved = direct-form-equivalent fp32 flops (3 * sub_dim * "
                          "n_centroids per sub-vector) / kernel time; the kernel executes a "
                          "matrix-core bound plus an exact recompute of few candidates, and "
                          "what binds it is in 'utilization'"),
        "utilization": util,
        "cpu_baseline": cpu,
        "vs_cpu_oracle": (value / cpu["value"]) if cpu else None,
        "kernel_ms_per_launch": launch_s * 1e3,
        "algorithmic_gb_per_s": algo_bytes / launch_s / 1e9,
        "hbm_frac": algo_bytes / launch_s / 1e9 / HBM_PEAK_GBS,
        "parity_sample": parity_sample,
        "vs_baseline_note": ("pages' Apple-Silicon Metal kernel on the same shape, 1,048,576 "
                             "sub-vectors in 7.98 ms (context only, another machine)"),
    }
    rows = [r for r in (args.configs.split(",") + args.rows.split(",")) if r]
    if rows:
        line["rows"] = {}
        for r in rows:
            line["rows"][r] = ROW_LEGS[r](args, dev, stream)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
