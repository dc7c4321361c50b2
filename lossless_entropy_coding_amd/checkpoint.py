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
"""
from __future__ import annotations

import math
import time

import torch

from . import _lib as L
from . import codec, synth, workloads


class CheckpointJob:
    """One Plan per layer container; decode() decodes every layer in order."""

    def __init__(self, layers: int = 84, chunk_weights: int = 65536, lanes: int = 512, log=print,
                 device: str = "cuda", keep_host_first: bool = True, m_s: int = 12, m_f: int = 10,
                 stream_lanes: int = 256):
        layout = synth.cfg5_layout(layers=layers)
        self.name = "cfg5_checkpoint_%dlayers_%dtensors" % (layers, len(layout))
        self.chunk_weights, self.lanes, self.stream_lanes = chunk_weights, lanes, stream_lanes or lanes
        self.m_s, self.m_f = m_s, m_f
        self.lanes_per_thread = max(1, self.stream_lanes // 64)
        # one mixed launch per layer: matrices (several lanes per thread) and vectors (one)
        self.kernel_name = "decode_kernel<%d, %s>" % (0 if self.lanes_per_thread <= 2 else 3,
                                                      "true" if m_s <= 11 and m_f <= 9 else "false")
        self.plans, self.refs = [], []
        self.n_weights = self.raw_bytes = self.read_bytes = self.container_bytes = 0
        bits = ent = 0.0
        self.first_container = None
        t0 = time.time()
        out_max = 16
        for layer in range(layers + 1):
            wl = synth.cfg5_layer(layer, device=device, chunk_weights=chunk_weights, lanes=lanes, layout=layout)
            wl.m_s, wl.m_f, wl.stream_lanes = m_s, m_f, stream_lanes
            enc = workloads.encode_workload(wl, device=device, keep_reference=False, keep_device_reference=True)
            plan = codec.Plan(enc.container, device)
            if layer == 0 and keep_host_first:
                self.first_container = enc.container
            info = plan.info
            self.n_weights += enc.n_weights
            self.raw_bytes += enc.raw_bytes
            self.read_bytes += int(info.bf16_bytes) + int(info.raw_bytes)
            self.container_bytes += len(enc.container)
            bits += enc.bits_per_weight * enc.n_weights
            ent += enc.entropy_bits * enc.n_weights
            out_max = max(out_max, plan.out_bytes())
            self.plans.append(plan)
            self.refs.append(enc.reference_device)
            plan.host = None          # the host copy is not needed once the plan is built
            del wl, enc
            if log and (layer % 8 == 0 or layer == layers):
                log(f"checkpoint: layer {layer + 1}/{layers + 1} encoded and resident "
                    f"({self.container_bytes / 1e9:.2f} GB compressed, {time.time() - t0:.0f}s)")
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
        """Every layer decoded into the shared buffer, checked on the device
        against its original words, with every chunk's status word."""
        bad = []
        for i, (plan, ref) in enumerate(zip(self.plans, self.refs)):
            plan.decode_into(self.out)
            n = ref.numel()
            rc, rep = plan.verify(self.out[:n], ref=ref, flags=L.VERIFY_STATUS | L.VERIFY_COMPARE)
            if rc != L.BS_OK:
                bad.append((i, rc, rep))
        return not bad, bad[:3]

    def containers(self):
        """Host containers available for the CPU baseline (the first layer)."""
        return [self.first_container] if self.first_container is not None else []


def build_job(layers: int = 84, log=print, **kw) -> CheckpointJob:
    return CheckpointJob(layers=layers, log=log, **kw)
