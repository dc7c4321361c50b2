"""GPU parity for packed small records: a decode launch that holds large
records and small ones decodes the small ones several to a workgroup, one
after another, and spreads the large records' runs over the other CUs.

The output must still be every record's original words, and the per-stream
status must still name a damaged small record [Qwen3.8-27B-BF16-NVLC-Lossless
card, metrics table: per-codec and integrated inverse verification; Gemma 2
9B Instruct -- Lossless Compressed card, "What lossless means"].  Calls go
through the C ABI (bs_encode_host, bs_plan_create, bs_plan_packs,
bs_decode_async, bs_verify); sampled chunks are checked against the oracle's
decoder.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from lossless_entropy_coding_amd import _lib as L
from lossless_entropy_coding_amd import codec

pytestmark = pytest.mark.gpu

W, K = 4096, 8
BIG = 2048 * W


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def _words(rng, n, scale):
    x = rng.standard_normal(n).astype(np.float32) * scale
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def _params(layout):
    if layout == 3:
        return codec.params3(chunk_weights=W, lanes=K, stream_lanes=K, m_s=11)
    return codec.params2(chunk_weights=W, lanes=K, stream_lanes=K, m_s=11)


def _container(layout, seed):
    """Two large records of about 2048 chunks (8-lane streams, 512 weights
    per lane) with small records between them: five of about 1000 weights
    (2 lanes of 500), one of 5 weights and an empty one."""
    rng = np.random.default_rng(seed)
    sizes = [1000, BIG, 1000, 0, 1000, BIG + 333, 999, 5, 1000]
    words = [_words(rng, n, float(rng.choice([0.004, 0.02, 0.07]))) for n in sizes]
    c = codec.encode([codec.bf16(w) for w in words], _params(layout))
    return c, words


def _expect_packs(plan, full):
    # 256 CUs: runs of 17 units over the 4,097 large units take 242
    # workgroups, and packs of 2 small records (500 + 64 lane steps each
    # against 1.5 x 2 rounds x 512 steps) take 3 more
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = plan.packs()
    say("packs", n, "CUs", cus)
    assert n >= 1
    if cus == 256 and full:
        assert n == 3


@pytest.mark.parametrize("layout", [3, 2])
def test_small_records_packed_beside_large_ones(layout):
    say("packs, layout", layout)
    c, words = _container(layout, 90 + layout)
    plan = codec.Plan(c)
    _expect_packs(plan, layout == 3)
    out = plan.decode()
    rc, rep = plan.verify(out, flags=L.VERIFY_STATUS | L.VERIFY_SHA256)
    assert rc == L.BS_OK, rep
    assert rep["chunks_bad"] == 0 and rep["records_hash_bad"] == 0
    for i, w in enumerate(words):
        got = codec.record_output(out, plan, i, 0).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, w), i
    # the oracle's decode of the small records and of sampled large chunks
    for i in (0, 2, 4, 6, 7, 8):
        assert np.array_equal(O.decode_chunk(c, i, 0), words[i]), i
    for ch in (0, 1000, 2048):
        assert np.array_equal(O.decode_chunk(c, 5, ch), words[5][ch * W:(ch + 1) * W]), ch

    # a record range with both large records and two small ones (one pack);
    # with one large record alone its runs would be single rounds, and
    # nothing would be packed
    first, count = 1, 5
    assert plan.packs(first, count) == 1
    assert plan.packs(1, 4) == 0
    sub = plan.decode(first, count)
    torch.cuda.synchronize()
    for i in range(first, first + count):
        assert torch.equal(codec.record_output(sub, plan, i, first), codec.record_output(out, plan, i, 0)), i


def test_damaged_small_record_in_a_pack_is_reported():
    say("packs, damaged small record")
    c, words = _container(3, 95)
    ri = codec.record_info(c, 4)
    assert ri.n == 1000
    b = bytearray(c)
    b[ri.rec_offset + int(ri.rec_len * 0.8)] ^= 0x3C
    plan = codec.Plan(bytes(b))
    assert plan.packs() >= 1
    out = plan.decode()
    rc, rep = plan.verify(out, flags=L.VERIFY_STATUS | L.VERIFY_SHA256)
    assert rc != L.BS_OK
    assert rep["records_hash_bad"] == 1
    for i, w in enumerate(words):
        if i == 4:
            continue
        got = codec.record_output(out, plan, i, 0).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, w), i


def test_packs_of_multi_unit_small_records_with_fifteen_waves():
    """M_s 12 leaves room for 15 rings: small records are those of at most
    15 units.  Chunks of 8192 weights over 128 lanes in 2 streams of 64:
    small records of 1 to 7 chunks (2 to 14 units, several waves each) and
    one of 300 weights (one unit) sit between three large records; on 256
    CUs they take 4 packs of 2."""
    say("packs, m_s 12, multi-unit small records")
    rng = np.random.default_rng(123)
    W2 = 8192
    big = 1400 * W2
    sizes = [5 * W2 + 17, big, 3 * W2, 2 * W2 + 1, big + 4000, 7 * W2, 300, W2, big - 77, 6 * W2 + 5]
    words = [_words(rng, n, float(rng.choice([0.004, 0.02, 0.07]))) for n in sizes]
    p = codec.params3(chunk_weights=W2, lanes=128, stream_lanes=64, m_s=12)
    c = codec.encode([codec.bf16(w) for w in words], p)
    plan = codec.Plan(c)
    assert plan.waves_per_block == 15
    n = plan.packs()
    say("packs", n)
    assert n >= 1
    out = plan.decode()
    rc, rep = plan.verify(out, flags=L.VERIFY_STATUS | L.VERIFY_SHA256)
    assert rc == L.BS_OK, rep
    for i, w in enumerate(words):
        got = codec.record_output(out, plan, i, 0).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, w), i
    for i in (0, 3, 5, 9):
        ri = codec.record_info(c, i)
        last = (ri.n - 1) // W2
        assert np.array_equal(O.decode_chunk(c, i, last), words[i][last * W2:]), i
