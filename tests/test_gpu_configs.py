"""GPU parity on the synthetic workloads at full size, in the launch
configuration the benchmark uses.

configs 1-3: the oracle decodes the whole container and the GPU output must
equal it and the original bits.  configs 4 and 5 (917M and 27.7B weights):
the GPU output is compared with the original bits on the device for every
byte (exact at any size), sha256 per tensor is checked, and the oracle
decodes a sample of chunks one by one for an independent comparison.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import entropy as E
from oracle import oracle as O
from lossless_entropy_coding_amd import _lib as L
from lossless_entropy_coding_amd import codec, synth, workloads

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("cfg", ["1", "2", "3"])
def test_small_configs_full_oracle(cfg):
    say("config", cfg)
    enc = workloads.encode_config(cfg)
    expect, st = O.decode(enc.container)
    assert all(s == 0 for s in st)
    assert expect[: len(enc.reference)] == enc.reference
    plan = codec.Plan(enc.container)
    out = plan.decode()
    rc, rep = plan.verify(out, flags=L.VERIFY_STATUS | L.VERIFY_SHA256)
    assert rc == L.BS_OK, rep
    assert out.cpu().numpy().tobytes()[: len(expect)] == expect
    # bits/weight within 1% of the empirical conditional entropy
    assert enc.bits_per_weight <= 1.01 * enc.entropy_bits, (enc.bits_per_weight, enc.entropy_bits)


@pytest.mark.slow
def test_config4_full_size():
    say("config 4 (917M weights)")
    enc = workloads.encode_config("4", device="cuda")
    plan = codec.Plan(enc.container)
    out = plan.decode()
    ref = enc.reference_device
    rc, rep = plan.verify(out, ref=ref, flags=L.VERIFY_STATUS | L.VERIFY_COMPARE)
    assert rc == L.BS_OK, rep
    assert rep["bytes_compared"] == 2 * enc.n_weights
    # oracle on sampled chunks
    ri = codec.record_info(enc.container, 0)
    rng = np.random.default_rng(0)
    host = None
    for ch in sorted(rng.choice(ri.n_chunks, 8, replace=False).tolist()) + [ri.n_chunks - 1]:
        o = O.decode_chunk(enc.container, 0, ch)
        a = ch * ri.chunk_weights
        got = out[2 * a: 2 * (a + o.size)].cpu().numpy().view(np.uint16)
        assert np.array_equal(got, o), ch
    assert enc.bits_per_weight <= 1.01 * enc.entropy_bits, (enc.bits_per_weight, enc.entropy_bits)


def test_config5_layers_into_one_buffer():
    """Config 5 in the benchmark's launch configuration, cut to its first two
    decoder layers plus the trailing vectors (the full run repeats the same
    layer shapes 84 times): every layer encoded on the GPU and resident in
    HBM, decoded in order into one reused buffer, each layer compared on the
    device with its original words (torch.equal) and through its status
    words, and chunks of every tensor of every layer against the oracle."""
    from lossless_entropy_coding_amd import checkpoint
    say("config 5, two layers + tail")
    job = checkpoint.build_job(layers=2, log=say)
    assert len(job.plans) == 3 and job.n_tensors == 2 * 14 + 23
    # a layer's 7 norm vectors are decoded in packs beside its matrices; the
    # trailing vectors alone have no large record to share the CUs with
    packs = [p.packs() for p in job.plans]
    say("packs per launch", packs)
    assert packs[0] >= 1 and packs[1] >= 1 and packs[2] == 0
    job.decode()
    torch.cuda.synchronize()
    ok, bad = job.verify()
    assert ok, bad
    rng = np.random.default_rng(5)
    for layer, (dev, ref) in enumerate(job.oracle_samples()):
        c = dev.cpu().numpy().tobytes()
        info = codec.container_info(c)
        for i in range(info.n_records):
            ri = codec.record_info(c, i)
            if ri.kind != L.KIND_BF16 or ri.n_chunks == 0:
                continue
            for ch in sorted({0, ri.n_chunks - 1, int(rng.integers(ri.n_chunks))}):
                o = O.decode_chunk(c, i, ch)
                a = ri.out_offset + 2 * ch * ri.chunk_weights
                want = ref[a: a + 2 * o.size].cpu().numpy().view(np.uint16)
                assert np.array_equal(want, o), (layer, i, ch)
    assert job.bits_per_weight <= 1.01 * job.entropy_bits, (job.bits_per_weight, job.entropy_bits)
