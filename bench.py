#!/usr/bin/env python3
"""Benchmark: decoded BF16 GB/s of the HIP decode path on one MI355X, its
fraction of the HBM roofline, and compressed bits/weight against the
empirical conditional entropy.

A step is one decode of the whole workload (bs_decode_async over every
record: the rANS decode kernel plus the verbatim residual copy), with the
containers already resident in HBM and the output buffer preallocated.
The default workload is the largest: the synthetic 27.7B-weight checkpoint
(1,199 tensors in 84 layer containers plus one of trailing vectors, about
36 GB compressed, all resident), decoded layer by layer into one reused
buffer; every layer is compared with its original bytes on the device before
and after the timing, and the CPU oracle decodes a chunk of every tensor
(and more, within its time budget), each compared with the original words.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1|2|3|4|5] [--cold]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth, GB/s


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def copy_ceiling(n: int = 1 << 30, reps: int = 20) -> float:
    """GB/s (bytes read + written) of a plain device copy of n bytes."""
    import torch
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * n / ms / 1e6


def cold_flush(buf) -> None:
    """Leave the GPU caches cold and clean before a timed launch: write a
    1 GiB buffer (evicting what the launch would find cached), then read it
    back, so that the dirty lines of the write are written back here and not
    during the timed launch.  Enqueued on the current stream without a host
    synchronisation: the timed launch queues behind it, so the GPU is busy up
    to the launch and no host launch latency enters the launch's events."""
    import torch
    buf.fill_(1)
    buf.sum(dtype=torch.int64)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 20 for the checkpoint, 200 for the other workloads)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None, choices=["1", "2", "3", "4", "5"],
                    help="workload (default: 5, the checkpoint; 2, the 4096x4096 matrix, with --gemv, and for the "
                         "products in --fixed)")
    ap.add_argument("--cold", action="store_true", help="write and read back a 1 GiB buffer before each timed decode (not in the timing): cold, clean caches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the oracle baseline")
    ap.add_argument("--cfg5-layers", type=int, default=84, help="config 5: layers to build (84 = full checkpoint)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB a few times (to scale HBM byte counters)")
    ap.add_argument("--lanes", type=int, default=None, help="override the lanes per chunk of the workload")
    ap.add_argument("--chunk-weights", type=int, default=None, help="override the weights per chunk")
    ap.add_argument("--stream-lanes", type=int, default=None, help="override the lanes per word stream")
    ap.add_argument("--m-s", type=int, default=None, help="override the (sign, exponent) table precision")
    ap.add_argument("--m-f", type=int, default=None, help="override the fraction table precision")
    ap.add_argument("--layout", type=int, default=None, choices=[1, 2, 3],
                    help="override the record layout (2: one renormalisation per weight; 3: the same with s and "
                         "the fraction's high bits one joint symbol)")
    ap.add_argument("--gemv", action="store_true",
                    help="time the fused decode and matrix-vector product (bs_gemv_async) of the 4096x4096 "
                         "workload against decode-then-GEMV and a GEMV on the uncompressed matrix")
    ap.add_argument("--fixed", action="store_true",
                    help="time the decode of the fixed-width lane-stream form (bs_fixed_decode_async) derived from "
                         "the workload's container, against the rANS decode of the same container")
    ap.add_argument("--encode", action="store_true",
                    help="time the GPU encoder (bs_encode_device_*) on the workload against the host encoder")
    ap.add_argument("--stream", action="store_true",
                    help="stream the checkpoint's layers from pinned host memory under a device budget "
                         "(bs_streamer_*), against copying the uncompressed layers")
    ap.add_argument("--stream-layers", type=int, default=12, help="--stream: layers of the checkpoint to build")
    ap.add_argument("--stream-slots", type=int, default=3, help="--stream: decoded layers the budget holds")
    a = ap.parse_args()
    if a.config is None:
        a.config = "2" if a.gemv else "5"
    if a.steps is None:
        a.steps = 20 if a.config == "5" and not (a.gemv or a.fixed or a.encode or a.stream) else 200
    return a


TRAFFIC_SOURCES = {"decode_kernel": ("bs_decode.hip", "bs_decode_common.h", "bs_device.h"),
                   "decode2_kernel": ("bs_decode2.hip", "bs_decode_common.h", "bs_device.h"),
                   "decode3_kernel": ("bs_decode2.hip", "bs_decode_common.h", "bs_device.h"),
                   "fixed": ("bs_fixed.hip", "bs_fixed_device.h")}


def kernel_source_sha256(kind: str) -> str:
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    return hashlib.sha256(b"".join(open(os.path.join(root, "lossless_entropy_coding_amd", "csrc", n), "rb").read()
                                   for n in TRAFFIC_SOURCES[kind])).hexdigest()


def measured_traffic(key: str, kind: str = "decode_kernel"):
    """HBM bytes per launch of a kernel on a workload, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE passes (scaled by a plain-copy
    calibration), or None when there is no pass for this workload or the
    kernel's source has changed since the counters were taken."""
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(root, "profiles", "hbm_traffic.json")) as f:
            rec = json.load(f)
        sha = kernel_source_sha256(kind)
    except OSError:
        return None
    w = rec.get("workloads", {}).get(key)
    if w is None or w.get("kernel_source_sha256") != sha:
        return None
    return int(w["traffic_bytes"])


def model_build_rate(job):
    """bs_build_tables (the HIP histogram pass + host quantisation) on the
    workload's first BF16 tensor (the checkpoint: its first layer's largest),
    already in HBM: wall time per call."""
    import torch
    from lossless_entropy_coding_amd import codec
    if getattr(job, "model_sample", None) is not None:
        # the checkpoint: the first layer's largest tensor
        words = job.model_sample.view(torch.int16).reshape(-1)
        n = words.numel()
    else:
        if not hasattr(job, "ref") or not hasattr(job, "plan"):
            return None
        ri = codec.record_info(job.plan.host, 0) if job.plan.host is not None else None
        if ri is None or ri.kind != 1 or ri.n == 0:
            return None
        words = job.ref[ri.out_offset: ri.out_offset + 2 * ri.n].view(torch.int16)
        n = ri.n
    if getattr(job, "layout", 1) == 3:
        p = codec.params3(chunk_weights=job.chunk_weights, lanes=job.lanes, m_s=job.m_s, stream_lanes=job.stream_lanes)
    elif getattr(job, "layout", 1) == 2:
        p = codec.params2(chunk_weights=job.chunk_weights, lanes=job.lanes, m_s=job.m_s, stream_lanes=job.stream_lanes)
    else:
        p = codec.params(chunk_weights=job.chunk_weights, lanes=job.lanes, m_s=job.m_s, m_f=job.m_f,
                         stream_lanes=job.stream_lanes)
    codec.build_tables(words, p)          # warm-up
    best = float("inf")
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        codec.build_tables(words, p)
        best = min(best, time.perf_counter() - t0)
    return {"weights": int(n), "ms": round(best * 1e3, 3), "read_GB_s": round(2 * n / best / 1e9, 1),
            "what": "bs_build_tables wall time: one HIP histogram pass, the counts read back, host quantisation"}


def _oracle_sources(job):
    """(host container, device original bytes) pairs the oracle decodes from:
    every layer of the checkpoint, else the job's one container."""
    import torch
    if hasattr(job, "oracle_samples"):
        return [(dev.cpu().numpy(), ref) for dev, ref in job.oracle_samples()]
    return [(np.frombuffer(job.enc.container, np.uint8), job.ref)]


def cpu_baseline(job, seconds: float):
    """The CPU oracle (plain scalar C, not tuned) decoding the same
    containers on the host, every decoded chunk compared with the original
    words.  The tasks are the chunks of every BF16 record: first one chunk of
    every tensor (a parity pass over all of them), then further chunks spread
    over the records.  Two legs: one thread for a third of the budget, then a
    pool of host threads (the process's CPU share) that take tasks in turn,
    one scalar call per chunk, for the rest of the budget, and at least
    through the parity pass.  Returns the pool's decoded BF16 GB/s with the
    one-thread figure beside it; exits non-zero on any mismatch."""
    import threading
    import torch
    from oracle import oracle as O
    from lossless_entropy_coding_amd import checkpoint, codec
    sources = _oracle_sources(job)
    first, rest = [], []
    for si, (c, _) in enumerate(sources):
        info = codec.container_info(c)
        for i in range(info.n_records):
            ri = codec.record_info(c, i)
            if ri.kind != 1 or ri.n_chunks == 0:
                continue
            first.append((si, i, 0, int(ri.out_offset), int(ri.chunk_weights)))
            # the rest of the record's chunks, strided so that a prefix of the
            # list samples the whole record
            order = list(range(1, ri.n_chunks))
            step = max(1, len(order) // 7)
            order = order[::step] + [ch for ch in order if (ch - 1) % step]
            rest += [(r, si, i, ch, int(ri.out_offset), int(ri.chunk_weights)) for r, ch in enumerate(order)]
    # interleave the records' further chunks so that any prefix spans them all
    rest.sort(key=lambda t: t[:3])
    tasks = first + [t[1:] for t in rest]
    mismatches = []

    def run_task(k):
        si, i, ch, off, W = tasks[k]
        c, ref = sources[si]
        w = O.decode_chunk(c, i, ch)     # the C call releases the GIL
        a = off + 2 * ch * W
        want = ref[a: a + 2 * w.size].cpu().numpy().view(np.uint16)
        if not np.array_equal(w, want):
            mismatches.append((si, i, ch))
        return 2 * w.size

    def leg(threads: int, budget: float, at_least: int):
        nxt, decoded, lock = [0], [0], threading.Lock()
        t0 = time.perf_counter()

        def work():
            while True:
                with lock:
                    k = nxt[0]
                    if k >= len(tasks) or (k >= at_least and time.perf_counter() - t0 > budget):
                        return
                    nxt[0] += 1
                b = run_task(k)
                with lock:
                    decoded[0] += b
        pool = [threading.Thread(target=work) for _ in range(threads)]
        for th in pool:
            th.start()
        for th in pool:
            th.join()
        return decoded[0], time.perf_counter() - t0, min(nxt[0], len(tasks))

    d1, t1, n1 = leg(1, seconds / 3, 1)
    cores = checkpoint.host_threads()
    dT, tT, nT = leg(cores, 2 * seconds / 3, len(first))
    log(f"cpu baseline: 1 thread {d1 / 1e6:.1f} MB in {t1:.1f}s; {cores} threads {dT / 1e6:.1f} MB in {tT:.1f}s; "
        f"{nT} chunks checked, {len(mismatches)} mismatches")
    if mismatches:
        log("ORACLE MISMATCH", mismatches[:5])
        sys.exit(1)
    n_tensors = len(first)
    return {"value": round(dT / tT / 1e9, 5), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{nT} of {len(tasks)} chunks ({dT / 2:.0f} weights): one chunk of each of the {n_tensors} "
                      f"BF16 tensors, then chunks spread over every record; {cores} threads, one chunk per call; "
                      f"every chunk equal to the original words",
            "affinity_cores": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count(),
            "chunks_checked": nT, "tensors_checked": n_tensors, "mismatches": 0,
            "single_thread": {"value": round(d1 / t1 / 1e9, 5), "chunks": n1, "seconds": round(t1, 2)},
            "seconds": round(t1 + tT, 2)}


def gemv_bench(a):
    """Fused decode and GEMV on the 4096x4096 workload (y = W x, x BF16, y fp32)
    against (1) bs_decode_async then torch.mv on the decoded BF16 matrix and
    (2) torch.mv on the uncompressed BF16 matrix resident in HBM."""
    import torch
    from lossless_entropy_coding_amd import workloads
    enc = workloads.encode_config(a.config, device="cpu", keep_reference=False, keep_device_reference=True,
                                  lanes=a.lanes, chunk_weights=a.chunk_weights, stream_lanes=a.stream_lanes,
                                  m_s=a.m_s, m_f=a.m_f, layout=a.layout)
    assert a.config == "2", "the fused product is timed on the 4096x4096 workload"
    rows = cols = 4096
    job = workloads.DecodeJob(enc)
    W = job.ref[: 2 * rows * cols].view(torch.bfloat16).reshape(rows, cols)
    g = torch.Generator(device="cpu").manual_seed(1)
    x = torch.randn(cols, generator=g).to(torch.bfloat16).cuda()
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fused = job.plan.bound_gemv(y, x.view(torch.int16), rows, cols, stream=stream)
    dec = job.fast_decoder(stream)
    Wd = job.out[: 2 * rows * cols].view(torch.bfloat16).reshape(rows, cols)

    def two_step():
        dec()
        torch.mv(Wd, x)

    def plain():
        torch.mv(W, x)

    def timed(fn):
        for _ in range(a.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(a.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / a.steps     # us per call

    t_fused, t_two, t_plain = timed(fused), timed(two_step), timed(plain)
    fused()
    torch.cuda.synchronize()
    ref = (W.float() @ x.float())
    err = float((y - ref).abs().max() / ref.abs().max())
    comp = int(job.read_bytes)
    line = {"metric": "fused decode + GEMV (4096x4096 BF16 weights, batch 1)", "unit": "us per product",
            "fused_us": round(t_fused, 2), "decode_then_gemv_us": round(t_two, 2), "plain_bf16_gemv_us": round(t_plain, 2),
            "fused_weight_bytes_read": comp, "plain_weight_bytes_read": 2 * rows * cols,
            "fused_GB_s_of_compressed_weights": round(comp / t_fused / 1e3, 1),
            "plain_GB_s_of_bf16_weights": round(2 * rows * cols / t_plain / 1e3, 1),
            "max_rel_diff_vs_fp32_product": err, "steps": a.steps, "data": "synthetic",
            "config": {"workload": job.name, "lanes": job.lanes, "stream_lanes": job.stream_lanes,
                       "chunk_weights": job.chunk_weights, "layout": job.layout}}
    print(json.dumps(line))


def fixed_bench(a):
    """The fixed-width lane-stream form of every BF16 record of the workload,
    derived on the GPU (bs_fixed_encode_device) from the GPU decode of the
    canonical container, then decoded by bs_fixed_decode_async (one tensor) or
    bs_fixed_decode_many_async (up to 16 tensors per launch; the same tensors
    in one launch each are timed beside it).  Reports decoded GB/s, the kernel's HBM roofline fraction and
    bits/weight, next to the rANS decode of the same container, and the
    transcoding time on the GPU and with the host transcoder (whose bytes must
    be the same)."""
    import torch
    from lossless_entropy_coding_amd import _lib as L
    from lossless_entropy_coding_amd import codec, workloads
    gen_dev = "cuda" if a.config == "4" else "cpu"
    enc = workloads.encode_config(a.config, device=gen_dev, keep_reference=False, keep_device_reference=True,
                                  lanes=a.lanes, chunk_weights=a.chunk_weights, stream_lanes=a.stream_lanes,
                                  m_s=a.m_s, m_f=a.m_f)
    job = workloads.DecodeJob(enc)
    stream = torch.cuda.current_stream()
    job.decode(stream)
    torch.cuda.synchronize()
    ok, detail = job.verify()
    assert ok, detail
    # derive the fixed form of each BF16 record from the decoded canonical container, on the GPU
    decs = []
    for i in range(job.plan.n_records):
        ri = codec.record_info(enc.container, i)
        if ri.kind == L.KIND_BF16:
            decs.append((ri, codec.record_output(job.out, job.plan, i).view(torch.int16)))
    codec.fixed_encode_device(decs[0][1][:4096])          # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    blobs = [codec.fixed_encode_device(d) for _, d in decs]
    torch.cuda.synchronize()
    t_transcode_gpu = time.perf_counter() - t0
    t0 = time.perf_counter()
    host_blobs = [codec.fixed_encode(d.cpu().numpy().view(np.uint16)) for _, d in decs]
    t_transcode = time.perf_counter() - t0
    if any(b.cpu().numpy().tobytes() != h for b, h in zip(blobs, host_blobs)):
        log("GPU AND HOST TRANSCODERS DISAGREE")
        sys.exit(1)
    plans = [codec.FixedPlan(b) for b in blobs]
    outs = [torch.empty(max(ri.n, 8), dtype=torch.int16, device="cuda") for ri, _ in decs]
    refs = [d for _, d in decs]
    n = sum(p.n for p in plans)
    blob_bytes = sum(p.bytes for p in plans)
    # one launch for a single tensor; several tensors in launches of up to
    # FIXED_MANY_MAX blobs each (bs_fixed_decode_many_async)
    groups = [list(range(i, min(i + L.FIXED_MANY_MAX, len(plans)))) for i in range(0, len(plans), L.FIXED_MANY_MAX)]
    many = len(plans) > 1
    if many:
        steps = [codec.bound_fixed_decode_many([plans[i] for i in g], [outs[i] for i in g], stream=stream)
                 for g in groups]
    else:
        steps = [plans[0].bound_decode(outs[0], status=False, stream=stream)]
    per_tensor = [p.bound_decode(o, status=False, stream=stream) for p, o in zip(plans, outs)]

    def step():
        for s_ in steps:
            s_()

    def step_per_tensor():
        for s_ in per_tensor:
            s_()

    def check():
        for o in outs:
            o.fill_(-1)
        if many:
            for g in groups:
                codec.fixed_decode_many([plans[i] for i in g], [outs[i] for i in g], stream=stream)
        else:
            plans[0].decode_into(outs[0], stream=stream)
        torch.cuda.synchronize()
        for p, o, r in zip(plans, outs, refs):
            if not torch.equal(o[: p.n], r) or int(p.status[: p.info.n_blocks].abs().sum()) != 0:
                log("FIXED DECODE MISMATCH")
                sys.exit(1)

    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if a.cold else None

    def timed(fn):
        for _ in range(a.warmup):
            fn()
        torch.cuda.synchronize()
        if flush is not None:
            # cold caches: a 1 GiB write and read-back before each step, outside the timing
            # (device time only: the flushes run between the launches)
            dev_s_ = 0.0
            for _ in range(a.steps):
                cold_flush(flush)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                dev_s_ += e0.elapsed_time(e1) * 1e-3
            return dev_s_ / a.steps, dev_s_ / a.steps
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_s = time.perf_counter()
        e0.record(stream)
        for _ in range(a.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t_s) / a.steps, e0.elapsed_time(e1) * 1e-3 / a.steps

    check()
    wall, dev_s = timed(step)
    check()
    per_tensor_launches = None
    if many:
        pt_wall, pt_dev = timed(step_per_tensor)
        per_tensor_launches = {"launches": len(plans), "value": round(2 * n / pt_wall / 1e9, 2),
                               "avg_step_ms": round(pt_dev * 1e3, 4)}
    rans_wall, rans_dev = timed(job.fast_decoder(stream))
    alg = blob_bytes + 2 * n
    achieved = alg / dev_s / 1e9          # algorithmic bytes over the launches' device time
    gemv = None
    if a.config == "2":
        # y = W x on the 4096 x 4096 matrix: fused on the fixed form, fused on the
        # rANS container, and torch.mv on the uncompressed matrix
        rows = cols = 4096
        g = torch.Generator(device="cpu").manual_seed(1)
        x = torch.randn(cols, generator=g).to(torch.bfloat16).cuda()
        y = torch.empty(rows, dtype=torch.float32, device="cuda")
        W = refs[0].view(torch.bfloat16).reshape(rows, cols)
        fx = plans[0].bound_gemv(y, x.view(torch.int16), rows, cols, stream=stream)
        rx = job.plan.bound_gemv(y, x.view(torch.int16), rows, cols, stream=stream)
        _, t_fixed = timed(fx)
        _, t_rans = timed(rx)
        _, t_plain = timed(lambda: torch.mv(W, x))
        fx()
        torch.cuda.synchronize()
        ref = W.float() @ x.float()
        gemv = {"fixed_fused_us": round(t_fixed * 1e6, 2), "rans_fused_us": round(t_rans * 1e6, 2),
                "plain_bf16_gemv_us": round(t_plain * 1e6, 2),
                "fixed_fused_GB_s_of_blob": round(plans[0].bytes / t_fixed / 1e9, 1),
                "max_rel_diff_vs_fp32_product": float((y - ref).abs().max() / ref.abs().max())}
        # Y = X W^T for batches of 16 and 64 on the matrix cores, against the BLAS product
        # on the uncompressed matrix and decode-then-BLAS
        Wd = outs[0][: rows * cols].view(torch.bfloat16).reshape(rows, cols)
        gemm = {}
        for batch in (16, 32, 64):
            X = torch.randn(batch, cols, generator=g).to(torch.bfloat16).cuda()
            Y = torch.empty(batch, rows, dtype=torch.float32, device="cuda")
            R = (X.float() @ W.float().t())
            # the library's choice (a workspace where bs_fixed_gemm_work_bytes asks for
            # one), and both forms forced: 16 rows per workgroup, and the split product
            # (32 rows, two workgroups per group of rows, then the sums' addition) with
            # a workspace of its size
            wsplit = torch.empty(4 * batch * rows, dtype=torch.uint8, device="cuda")
            forms = {"fixed_fused_us": "auto", "fixed_fused_16row_us": None, "fixed_fused_split_us": wsplit}
            rec, diffs = {}, {}
            for key, work in forms.items():
                fg = plans[0].bound_gemm(Y, X.view(torch.int16), rows, cols, stream=stream, work=work)
                _, t_fg = timed(fg)
                Y.fill_(float("nan"))
                fg()
                torch.cuda.synchronize()
                rec[key] = round(t_fg * 1e6, 2)
                diffs[key] = float((Y - R).abs().max() / R.abs().max())
            _, t_pg = timed(lambda: torch.matmul(X, W.t()))
            dec0 = steps[0]
            _, t_dg = timed(lambda: (dec0(), torch.matmul(X, Wd.t())))
            gemm[f"batch_{batch}"] = dict(rec, **{
                "split_chosen": int(L.lib().bs_fixed_gemm_work_bytes(rows, cols, batch)) > 0,
                "plain_bf16_gemm_us": round(t_pg * 1e6, 2), "decode_then_gemm_us": round(t_dg * 1e6, 2),
                "fixed_fused_TFLOP_s": round(2 * batch * rows * cols / (rec["fixed_fused_us"] * 1e-6) / 1e12, 2),
                "max_rel_diff_vs_fp32_product": max(diffs.values())})
        gemv["gemm"] = gemm
    line = {"metric": "fixed-width lane-stream decode: decoded BF16 GB/s on 1 MI355X (% HBM roofline) + bits/weight",
            "value": round(2 * n / wall / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
            "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True, "dtype": "u32", "data": "synthetic",
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "kernel": "fixed_decode_many_kernel" if many else "fixed_decode_kernel",
                         "traffic": measured_traffic(f"fixed|{job.name}", "fixed"),
                         "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                         "alg_bytes_per_step": alg, "launches_per_step": len(steps),
                         "avg_step_ms": round(dev_s * 1e3, 4)},
            "bits_per_weight": round(8 * blob_bytes / n, 4), "per_tensor_launches": per_tensor_launches,
            "rans": {"value": round(2 * n / rans_wall / 1e9, 2), "avg_step_ms": round(rans_dev * 1e3, 4),
                     "bits_per_weight": round(job.bits_per_weight, 4)},
            "transcode_s_gpu": round(t_transcode_gpu, 4), "transcode_s_host": round(t_transcode, 2),
            "transcode_note": "GPU: device words to device blob, including the blob's read-back-free layout; host: "
                              "from host words (the copy to the host not included)", "gemv": gemv,
            "config": {"workload": job.name, "bf16_weights": n, "tensors": len(plans),
                       "escapes": sum(p.info.n_esc for p in plans), "cold_cache": bool(a.cold)}}
    print(json.dumps(line))


def fixed_checkpoint_bench(a):
    """The fixed-width form of the synthetic checkpoint (84 layers of 14
    tensors + 23 trailing vectors, 27.7B weights): each tensor generated on
    the GPU and transcoded there (bs_fixed_encode_device), every blob kept
    resident; a step decodes every layer in turn into one reused buffer, a
    layer's tensors in one bs_fixed_decode_many_async launch (at most 16 per
    launch)."""
    import torch
    from lossless_entropy_coding_amd import _lib as L
    from lossless_entropy_coding_amd import codec, synth
    layout = synth.cfg5_layout(layers=a.cfg5_layers)
    n_layers = a.cfg5_layers
    t0 = time.time()
    layers, out_words, n, blob_bytes, escapes = [], 0, 0, 0, 0
    for li in range(n_layers + 1):
        wl = synth.cfg5_layer(li, device="cuda", layout=layout)
        plans, offs, off = [], [], 0
        for it in wl.items:
            w = synth.as_words(it.tensor)
            plans.append(codec.FixedPlan(codec.fixed_encode_device(w)))
            offs.append(off)
            off += (w.numel() + 127) // 128 * 128          # 256-B aligned, as in the container layout
            n += w.numel()
        blob_bytes += sum(p.bytes for p in plans)
        escapes += sum(p.info.n_esc for p in plans)
        out_words = max(out_words, off)
        layers.append((plans, offs))
        del wl
        if li % 12 == 0 or li == n_layers:
            log(f"fixed checkpoint: layer {li + 1}/{n_layers + 1} transcoded and resident "
                f"({blob_bytes / 1e9:.2f} GB, {time.time() - t0:.0f}s)")
    out = torch.empty(max(out_words, 8), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    calls = []
    for plans, offs in layers:
        for g in range(0, len(plans), L.FIXED_MANY_MAX):
            ps = plans[g: g + L.FIXED_MANY_MAX]
            os_ = offs[g: g + L.FIXED_MANY_MAX]
            calls.append(codec.bound_fixed_decode_many(ps, [out[o: o + p.n] for p, o in zip(ps, os_)], stream=stream))

    def step():
        for c in calls:
            c()

    def check(li):
        # decode layer li alone (with status), compare every tensor with its regenerated words
        plans, offs = layers[li]
        for g in range(0, len(plans), L.FIXED_MANY_MAX):
            ps, os_ = plans[g: g + L.FIXED_MANY_MAX], offs[g: g + L.FIXED_MANY_MAX]
            codec.fixed_decode_many(ps, [out[o: o + p.n] for p, o in zip(ps, os_)], stream=stream)
        wl = synth.cfg5_layer(li, device="cuda", layout=layout)
        torch.cuda.synchronize()
        for it, p, o in zip(wl.items, plans, offs):
            if not torch.equal(out[o: o + p.n], synth.as_words(it.tensor)) or (p.block_status() != 0).any():
                log("FIXED CHECKPOINT DECODE MISMATCH in layer", li, it.name)
                sys.exit(1)

    for li in range(n_layers + 1):
        check(li)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_s = time.perf_counter()
    e0.record(stream)
    for _ in range(a.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t_s) / a.steps
    dev_s = e0.elapsed_time(e1) * 1e-3 / a.steps
    for li in (0, n_layers // 2, n_layers):
        check(li)
    alg = blob_bytes + 2 * n
    achieved = alg / dev_s / 1e9
    line = {"metric": "fixed-width lane-stream decode: decoded BF16 GB/s on 1 MI355X (% HBM roofline) + bits/weight",
            "value": round(2 * n / wall / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
            "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True, "dtype": "u32", "data": "synthetic",
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "kernel": "fixed_decode_many_kernel",
                         "traffic": None, "alg_bytes_per_step": alg, "launches_per_step": len(calls),
                         "avg_step_ms": round(dev_s * 1e3, 4)},
            "bits_per_weight": round(8 * blob_bytes / n, 4),
            "config": {"workload": f"cfg5_checkpoint_{n_layers}layers_fixed", "bf16_weights": n,
                       "tensors": sum(len(p) for p, _ in layers), "escapes": escapes,
                       "resident_blob_bytes": blob_bytes, "layer_buffer_bytes": 2 * out_words,
                       "note": "every layer decoded into one reused buffer; all layers checked word for word "
                               "against their regenerated tensors before the timing, three after"}}
    print(json.dumps(line))


def encode_bench(a):
    """The workload's tensors encoded on the GPU (models from the HIP
    histogram, streams coded on the device, container written to device
    memory), end to end from device-resident words, against the host encoder
    (host models, all host threads) from host-resident words.  Both produce the
    same bytes; the check is part of the run."""
    import hashlib
    import torch
    from lossless_entropy_coding_amd import codec, synth, workloads
    wl = workloads.CONFIG_BUILDERS[a.config]("cuda")
    layout = a.layout or wl.layout
    p = codec.params(chunk_weights=a.chunk_weights or wl.chunk_weights, lanes=a.lanes or wl.lanes,
                     stream_lanes=a.stream_lanes if a.stream_lanes is not None else wl.stream_lanes,
                     m_s=11 if layout >= 2 else 12, m_f={1: 10, 2: 5, 3: codec.JOINT_BITS}[layout],
                     max_tables=31 if layout == 2 else 6, layout=layout)
    dev, host, digests = [], [], []
    n_bf16 = 0
    for it in wl.items:
        if it.kind == "bf16":
            t = synth.as_words(it.tensor).contiguous()
            dev.append(("bf16", t))
            h = t.cpu().numpy().view(np.uint16)
            host.append(codec.bf16(h))
            n_bf16 += t.numel()
        else:
            t = it.tensor.contiguous().view(torch.uint8).reshape(-1)
            dev.append(("raw", t))
            h = t.cpu().numpy()
            host.append(codec.raw(h))
        digests.append(hashlib.sha256(h.tobytes()).digest())
    torch.cuda.synchronize()
    codec.encode_device(dev[:1], p, digests=digests[:1])           # warm-up (module load, first launches)
    torch.cuda.synchronize()
    gpu_s = []
    for _ in range(max(1, a.steps)):
        t0 = time.perf_counter()
        dc = codec.encode_device(dev, p, digests=digests)
        torch.cuda.synchronize()
        gpu_s.append(time.perf_counter() - t0)
    t0 = time.perf_counter()
    hc = codec.encode(host, p)
    host_s = time.perf_counter() - t0
    same = dc.cpu().numpy().tobytes() == hc
    if not same:
        log("DEVICE CONTAINER DIFFERS FROM THE HOST ENCODER'S")
        sys.exit(1)
    gs = min(gpu_s)
    line = {"metric": "GPU encoder: BF16 GB/s encoded (device words to device container)",
            "value": round(2 * n_bf16 / gs / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
            "s_per_encode": round(gs, 4), "higher_is_better": True, "data": "synthetic",
            "host_encoder_GB_s": round(2 * n_bf16 / host_s / 1e9, 3), "host_encoder_s": round(host_s, 3),
            "host_threads": os.cpu_count(), "speedup_vs_host": round(host_s / gs, 1),
            "identical_bytes": same, "container_bytes": len(hc),
            "config": {"workload": wl.name, "bf16_weights": n_bf16, "chunk_weights": p.chunk_weights, "lanes": p.lanes,
                       "stream_lanes": p.stream_lanes, "layout": p.layout}}
    print(json.dumps(line))


def stream_bench(a):
    """Layer streaming: the first --stream-layers layers of the synthetic
    checkpoint (configuration 5's layer layout) are encoded, their containers
    handed to a streamer (pinned host memory, a budget of --stream-slots
    decoded layers plus two staging buffers), and one pass over the layers is
    timed: acquire layer i, prefetch layer i + 1, release layer i.  The copy
    of the next layer overlaps the decode of the current one.  The same pass
    with the uncompressed layers (pinned host -> device copies of the BF16
    bytes) is timed for comparison; both rates include the PCIe transfer."""
    import torch
    from lossless_entropy_coding_amd import codec, synth, workloads
    layout = synth.cfg5_layout(layers=84)
    containers, refs = [], []
    t0 = time.time()
    for layer in range(a.stream_layers):
        # the checkpoint's chunk shape and record layout (layout 2: K 256 in
        # streams of 128)
        wl = synth.cfg5_layer(layer, device="cuda", chunk_weights=65536, lanes=256, layout=layout)
        wl.stream_lanes, wl.layout, wl.m_s, wl.m_f = 128, 2, 11, 5
        enc = workloads.encode_workload(wl, device="cuda", keep_reference=False, keep_device_reference=True)
        containers.append(enc.container)
        refs.append(enc.reference_device)
        del wl
    log(f"stream: {len(containers)} layers encoded in {time.time() - t0:.0f}s, "
        f"{sum(map(len, containers)) / 1e9:.2f} GB compressed")
    stream = torch.cuda.current_stream()
    slot = max(r.numel() for r in refs)
    slot = (slot + 255) // 256 * 256
    staging = (max(map(len, containers)) + 255) // 256 * 256
    budget = 2 * staging + a.stream_slots * slot
    s = codec.Streamer(containers, budget)
    torch.cuda.synchronize()

    def one_pass():
        n = len(containers)
        s.prefetch(0, stream=stream)
        for i in range(n):
            s.acquire_ptr(i, stream=stream)
            if i + 1 < n:
                s.prefetch(i + 1, stream=stream)
            s.release(i, stream=stream)

    def timed(fn):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_s = time.perf_counter()
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t_s, e0.elapsed_time(e1) * 1e-3

    # warm-up pass, then check every layer against its original bytes
    one_pass()
    for i, ref in enumerate(refs):
        v = s.acquire(i, stream=stream)
        ok = torch.equal(v[: ref.numel()], ref)
        s.release(i, stream=stream)
        if not ok:
            log(f"STREAMED LAYER {i} MISMATCH")
            sys.exit(1)
    before = s.stats()
    walls = [timed(one_pass)[0] for _ in range(max(1, a.steps))]
    after = s.stats()
    wall = min(walls)
    decoded = sum(r.numel() for r in refs)
    compressed = sum(map(len, containers))
    # the uncompressed layers streamed the same way: pinned host -> one device buffer per slot
    host = [r.cpu().pin_memory() for r in refs]
    dev = [torch.empty(slot, dtype=torch.uint8, device="cuda") for _ in range(a.stream_slots)]

    def raw_pass():
        for i, h in enumerate(host):
            dev[i % len(dev)][: h.numel()].copy_(h, non_blocking=True)

    raw_pass()
    raw_wall = min(timed(raw_pass)[0] for _ in range(max(1, a.steps)))
    line = {"metric": "layer streaming from pinned host memory: decoded BF16 GB/s delivered (PCIe-inclusive)",
            "value": round(decoded / wall / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
            "ms_per_pass": round(wall * 1e3, 2), "higher_is_better": True, "data": "synthetic",
            "uncompressed_copy_GB_s": round(decoded / raw_wall / 1e9, 2),
            "uncompressed_ms_per_pass": round(raw_wall * 1e3, 2),
            "speedup_vs_uncompressed": round(raw_wall / wall, 3),
            "compressed_h2d_GB_s": round(compressed / wall / 1e9, 2),
            "bits_per_weight": round(8 * compressed / (decoded / 2), 4),
            "streamer": {"slots": after["n_slots"], "slot_bytes": after["slot_bytes"],
                         "staging_bytes": after["staging_bytes"], "plan_bytes": after["plan_bytes"],
                         "vram_budget": budget, "misses_per_pass": (after["misses"] - before["misses"]) // len(walls),
                         "hits_per_pass": (after["hits"] - before["hits"]) // len(walls)},
            "config": {"workload": f"cfg5_checkpoint_first_{len(containers)}_layers", "bf16_bytes": decoded,
                       "container_bytes": compressed, "layout": 2}}
    print(json.dumps(line))


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only: the library decodes on one MI355X and has no multi-GPU "
              f"path (asked for --gpus {a.gpus}). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    from lossless_entropy_coding_amd import _lib as L
    from lossless_entropy_coding_amd import codec, synth, workloads

    assert torch.cuda.is_available(), "no GPU visible"
    if a.calibrate_copy:
        n = a.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

        def timed(fn, reps=20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps
        # the bandwidth plain streams reach on this GPU: a copy (as much read
        # as written) and a fill (written only), HIP events around 20 of each
        t_copy = timed(lambda: dst.copy_(src))
        t_fill = timed(lambda: dst.fill_(3))
        print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                          "copies": 5, "copy_ms": round(t_copy, 4), "copy_GB_s": round(2 * n / t_copy / 1e6, 1),
                          "fill_ms": round(t_fill, 4), "fill_GB_s": round(n / t_fill / 1e6, 1),
                          "copy_frac_of_8TB_s": round(2 * n / t_copy / 1e6 / 8000, 4),
                          "fill_frac_of_8TB_s": round(n / t_fill / 1e6 / 8000, 4)}))
        return
    L.lib()   # fails loudly if the HIP library is missing
    if a.gemv:
        if a.cold:
            print("--cold is not supported with --gemv (its timer runs back to back)", file=sys.stderr)
            sys.exit(2)
        gemv_bench(a)
        return
    if a.fixed:
        if a.config == "5":
            fixed_checkpoint_bench(a)
        else:
            fixed_bench(a)
        return
    if a.stream:
        stream_bench(a)
        return
    if a.encode:
        encode_bench(a)
        return
    dev = "cuda"
    t0 = time.time()
    if a.config == "5":
        from lossless_entropy_coding_amd import checkpoint
        over = {k: v for k, v in (("m_s", a.m_s), ("m_f", a.m_f), ("lanes", a.lanes), ("chunk_weights", a.chunk_weights),
                                  ("stream_lanes", a.stream_lanes), ("layout", a.layout)) if v}
        job = checkpoint.build_job(layers=a.cfg5_layers, log=log, **over)
    else:
        gen_dev = "cuda" if a.config == "4" else "cpu"
        enc = workloads.encode_config(a.config, device=gen_dev, keep_reference=False, keep_device_reference=True,
                                      lanes=a.lanes, chunk_weights=a.chunk_weights, stream_lanes=a.stream_lanes,
                                      m_s=a.m_s, m_f=a.m_f, layout=a.layout)
        job = workloads.DecodeJob(enc)
    log(f"workload {job.name}: {job.n_weights} BF16 weights, container {job.container_bytes / 1e6:.1f} MB, "
        f"built in {time.time() - t0:.1f}s")

    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if a.cold else None

    step = job.fast_decoder(stream) if hasattr(job, "fast_decoder") else (lambda: job.decode(stream))

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    # correctness of the measured configuration: status + device compare against the original bits
    ok, detail = job.verify()
    if not ok:
        log("VERIFY FAILED", detail)
        sys.exit(1)

    torch.cuda.synchronize()
    if flush is None:
        # back-to-back steps; HIP events on the launch stream bracket the whole
        # timed region, so the per-launch average includes no host gaps
        e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_start = time.perf_counter()
        e_start.record(stream)
        for _ in range(a.steps):
            step()
        e_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        avg_ms = e_start.elapsed_time(e_end) / a.steps
    else:
        # cold caches: a 1 GiB write and read-back between steps, outside the
        # timing; the value is then from device time (the flushes run between
        # the launches, so host time would count them)
        dev_ms = 0.0
        for _ in range(a.steps):
            cold_flush(flush)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            dev_ms += e0.elapsed_time(e1)
        avg_ms = dev_ms / a.steps
        wall = dev_ms * 1e-3
    ok, detail = job.verify()
    if not ok:
        log("VERIFY FAILED after timing", detail)
        sys.exit(1)

    out_bytes = 2 * job.n_weights + job.raw_bytes
    value = job.n_weights * 2 * a.steps / wall / 1e9          # decoded BF16 GB/s, whole job
    # algorithmic bytes per decode: the container bytes that are read (BF16
    # records: tables, index, states, words; verbatim spans) + the bytes written
    alg_bytes = job.read_bytes + out_bytes
    achieved = alg_bytes / (avg_ms * 1e-3) / 1e9
    layout = getattr(job, "layout", 1)
    traffic = measured_traffic(f"{job.name}|W={job.chunk_weights}|K={job.lanes}|P={job.stream_lanes}|L={layout}",
                               {2: "decode2_kernel", 3: "decode3_kernel"}.get(layout, "decode_kernel"))
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "kernel": job.kernel_name if hasattr(job, "kernel_name") else "decode_kernel",
                "alg_bytes_per_launch": alg_bytes, "avg_launch_ms": round(avg_ms, 4)}
    # context, measured after the timed region: what a plain 1 GiB device
    # copy (as many bytes read as written) reaches on this GPU
    copy_gbs = copy_ceiling()
    roofline["copy_ceiling"] = {"GB_s": round(copy_gbs, 1), "frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
                                "decode_vs_copy": round(achieved / copy_gbs, 4),
                                "what": "torch copy_ of 1 GiB, HIP events around 20 copies"}

    model = model_build_rate(job)

    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(job, a.cpu_seconds)

    line = {
        "metric": "decoded BF16 GB/s on 1 MI355X (% HBM roofline) + compressed bits/weight",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(wall / a.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": job.name, "bf16_weights": job.n_weights, "raw_bytes": job.raw_bytes,
                   "chunk_weights": job.chunk_weights, "lanes": job.lanes, "stream_lanes": job.stream_lanes,
                   "m_s": job.m_s, "m_f": job.m_f, "layout": getattr(job, "layout", 1),
                   "bits_per_weight": round(job.bits_per_weight, 5), "entropy_bits": round(job.entropy_bits, 5),
                   "bits_over_entropy_pct": round(100 * (job.bits_per_weight / job.entropy_bits - 1), 3),
                   "cold_cache": bool(a.cold), "parallelism": "single GPU",
                   "tensors": getattr(job, "n_tensors", None), "container_bytes": job.container_bytes,
                   # bits per weight by part of the BF16 records (bs_container_sizes_get); they sum to bits_per_weight
                   "bits_per_weight_parts": codec.size_breakdown_bits_per_weight(job.sizes)},
        "roofline": roofline,
        "model_build": model,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
