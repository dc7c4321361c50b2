"""The synthetic ~27.7B-weight checkpoint, compressed layer by layer and
decoded layer by layer into one reused HBM buffer.

The pages report their codec on a 27.8B-weight BF16 checkpoint of 1,199
tensors [Qwen3.8-27B-BF16-NVLC-Lossless model card, metrics table]; the
stand-in here has the same tensor count and a layer layout of the same
sizes, with per-tensor scales drawn log-uniformly.  Each layer (plus the
trailing vectors) is one container; all containers stay resident in HBM
(about 36 GB of the 288 GB) and a decode step walks the layers in order,
decoding each into the same output buffer, as a loader that materialises
one layer at a time would.

The tensors are generated on the GPU and encoded there (bs_encode_device_*,
whose containers equal the host encoder's byte for byte), so the whole
checkpoint is built in seconds.  Each layer's original bytes stay resident
too (laid out as its decode), so that every layer's decode can be compared
with them on the device.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import time

import numpy as np
import torch

from . import _lib as L
from . import codec, synth, workloads


def _digest(t: torch.Tensor) -> bytes:
    # hashlib releases the GIL on large buffers, so a thread pool hashes in parallel
    return hashlib.sha256(t.cpu().numpy().tobytes()).digest()


def host_threads() -> int:
    """Host worker threads: the process's CPU share (OMP_NUM_THREADS when it
    is set, as on a GPU machine shared by several jobs), at most the cores the
    process may run on."""
    cores = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(cores, int(env))) if env.isdigit() and int(env) > 0 else cores


class CheckpointJob:
    """One Plan per layer container; decode() decodes every layer in order."""

    def __init__(self, layers: int = 84, chunk_weights: int | None = None, lanes: int | None = None, log=print,
                 device: str = "cuda", m_s: int | None = None, m_f: int | None = None,
                 stream_lanes: int | None = None, layout: int = 3):
        tensors = synth.cfg5_layout(layers=layers)
        # chunk shape: layout 3 takes chunks of 32,768 weights with K = 128
        # lanes in one stream (256 weights per lane, as K = 256 over 65,536
        # weights, at twice the decode units: a layer's units then divide
        # evenly over a workgroup's waves); layout 2 K = 256 in streams of 128
        # over 65,536 weights; layout 1 512 lanes in streams of 256
        if chunk_weights is None:
            chunk_weights = 32768 if layout == 3 else 65536
        if lanes is None:
            lanes = 128 if layout == 3 else 256 if layout == 2 else 512
        if stream_lanes is None:
            stream_lanes = 128 if layout >= 2 else 256
        self.name = "cfg5_checkpoint_%dlayers_%dtensors" % (layers, len(tensors))
        self.chunk_weights, self.lanes, self.stream_lanes = chunk_weights, lanes, stream_lanes or lanes
        # record layout 2 codes the fraction's high three bits at M_h = 16 - M_s,
        # layout 3 the joint (s, h) symbol at 13 bits
        if m_s is None:
            m_s = 11 if layout >= 2 else 12
        if m_f is None:
            m_f = {1: 10, 2: 16 - m_s, 3: codec.JOINT_BITS}[layout]
        self.m_s, self.m_f, self.layout = m_s, m_f, layout
        self.lanes_per_thread = max(1, self.stream_lanes // 64)
        # one mixed launch per layer: matrices (several lanes per thread) and vectors (one)
        variant = 0 if self.lanes_per_thread <= 2 else 3
        if layout >= 2:
            self.kernel_name = "decode%d_kernel<%d>" % (layout, variant)
        else:
            self.kernel_name = "decode_kernel<%d, %s>" % (variant, "true" if m_s <= 11 and m_f <= 9 else "false")
        self.plans, self.refs = [], []
        self.model_sample = None
        self.n_weights = self.raw_bytes = self.read_bytes = self.container_bytes = 0
        self.sizes = {}
        self.n_tensors = 0
        bits = ent = 0.0
        if layout == 3:
            p = codec.params3(chunk_weights=chunk_weights, lanes=lanes, m_s=m_s, stream_lanes=stream_lanes)
        elif layout == 2:
            p = codec.params2(chunk_weights=chunk_weights, lanes=lanes, m_s=m_s, stream_lanes=stream_lanes)
        else:
            p = codec.params(chunk_weights=chunk_weights, lanes=lanes, m_s=m_s, m_f=m_f, stream_lanes=stream_lanes)
        self.params = p
        pool = cf.ThreadPoolExecutor(max_workers=host_threads())
        t0 = time.time()
        out_max = 16
        for layer in range(layers + 1):
            wl = synth.cfg5_layer(layer, device=device, chunk_weights=chunk_weights, lanes=lanes, layout=tensors)
            words = [synth.as_words(it.tensor) for it in wl.items]
            if layer == 0:
                # the first layer's largest tensor, kept to time the model build
                self.model_sample = max(words, key=lambda t: t.numel())
            digests = list(pool.map(_digest, words))
            dev = codec.encode_device([("bf16", w) for w in words], p, digests=digests)
            host = dev.cpu().numpy().tobytes()
            plan = codec.Plan(host, device, dev=dev)
            info = plan.info
            # the layer's original bytes at their output offsets (the gaps are zero, like the decode's)
            ref = torch.zeros(max(plan.out_bytes(), 16), dtype=torch.uint8, device=device)
            for i, w in enumerate(words):
                ri = codec.record_info(host, i)
                ref[ri.out_offset: ri.out_offset + 2 * w.numel()] = w.view(torch.uint8)
                ent += workloads.word_entropy_bits(w) * w.numel()
            self.n_tensors += len(words)
            self.n_weights += int(info.bf16_weights)
            self.raw_bytes += int(info.raw_bytes)
            self.read_bytes += int(info.bf16_bytes) + int(info.raw_bytes)
            self.container_bytes += len(host)
            bits += 8.0 * info.bf16_bytes
            for k, v in codec.container_sizes(host).items():       # where the BF16 bits go
                self.sizes[k] = self.sizes.get(k, 0) + v
            out_max = max(out_max, plan.out_bytes())
            self.plans.append(plan)
            self.refs.append(ref)
            plan.host = None          # the host copy is not needed once the plan is built
            del wl, words, host
            if log and (layer % 8 == 0 or layer == layers):
                log(f"checkpoint: layer {layer + 1}/{layers + 1} encoded on the GPU and resident "
                    f"({self.container_bytes / 1e9:.2f} GB compressed, {time.time() - t0:.0f}s)")
        pool.shutdown()
        self.bits_per_weight = bits / self.n_weights
        self.entropy_bits = ent / self.n_weights
        self.out = torch.zeros(out_max, dtype=torch.uint8, device=device)

    def decode(self, stream=None):
        for plan in self.plans:
            plan.decode_into(self.out, stream=stream)

    def fast_decoder(self, stream):
        """One callable that enqueues every layer's decode into the shared
        buffer, with the C arguments of each marshalled once."""
        calls = [plan.bound_decode(self.out, stream=stream) for plan in self.plans]

        def run():
            for c in calls:
                c()
        return run

    def verify(self):
        """Every layer decoded into the shared buffer and checked twice on the
        device: torch.equal against the layer's original bytes (independent
        of the library), and the library's per-stream status words."""
        bad = []
        for i, (plan, ref) in enumerate(zip(self.plans, self.refs)):
            plan.decode_into(self.out)
            n = ref.numel()
            same = torch.equal(self.out[:n], ref)
            rc, rep = plan.verify(self.out[:n], flags=L.VERIFY_STATUS)
            if not same or rc != L.BS_OK:
                bad.append((i, same, rc, rep))
        return not bad, bad[:3]

    def oracle_samples(self):
        """What the CPU oracle checks: the layers' containers (host copies) and
        their original bytes (device); see bench.cpu_baseline."""
        return [(plan.dev, ref) for plan, ref in zip(self.plans, self.refs)]


def build_job(layers: int = 84, log=print, **kw) -> CheckpointJob:
    return CheckpointJob(layers=layers, log=log, **kw)
