"""GPU parity for layout-3 records (container version 3): the HIP decode path
against the original bits and the oracle.

Layout 3 codes the sign/exponent symbol s and the fraction's high three bits
as one joint symbol per weight (one table read, one step, one
renormalisation) and keeps the low four bits in a plane; the decode must
still reproduce every BF16 word [Qwen3.8-27B-BF16-NVLC-Lossless card,
metrics table: per-codec and integrated inverse verification; Gemma 2 9B
Instruct -- Lossless Compressed card, "What lossless means"].  Every call
goes through the C ABI (bs_build_tables, bs_encode_host, bs_encode_device_*,
bs_plan_create, bs_decode_async, bs_verify) via the ctypes binding; the
containers are checked byte for byte against the oracle's encoder first.
"""
import hashlib
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from lossless_entropy_coding_amd import _lib as L
from lossless_entropy_coding_amd import codec, synth
from test_gpu_decode2 import CASES

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def _words(x) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def _oracle_bytes(container: bytes) -> bytes:
    out, st = O.decode(container)
    assert all(s == 0 for s in st)
    return out


def _encode_both(tensors_o, tensors_l, W, K, P, M_s=11):
    c = codec.encode(tensors_l, codec.params3(chunk_weights=W, lanes=K, stream_lanes=P, m_s=M_s))
    assert c == O.encode(tensors_o, W=W, K=K, P=P, M_s=M_s, M_f=13, layout=3)
    assert codec.container_info(c).version == 3
    return c


def _decode_check(c, expect):
    plan = codec.Plan(c)
    out = plan.decode()
    rc, rep = plan.verify(out, flags=L.VERIFY_STATUS | L.VERIFY_SHA256)
    assert rc == L.BS_OK, rep
    assert rep["chunks_bad"] == 0 and rep["records_hash_bad"] == 0
    assert out[: len(expect)].cpu().numpy().tobytes() == expect
    return plan, out


@pytest.mark.parametrize("name,n,scale,W,K,P,ms", CASES, ids=[c[0] for c in CASES])
def test_layout3_decode_matches_oracle_and_original(name, n, scale, W, K, P, ms):
    say("layout 3 case", name, n, W, K, P, ms)
    rng = np.random.default_rng(n + 7)
    x = rng.standard_normal(n) * scale
    x[rng.random(n) < 0.01] = 0.0
    w = _words(x)
    c = _encode_both([O.bf16(w)], [codec.bf16(w)], W, K, P, ms)
    expect = _oracle_bytes(c)
    assert expect == w.tobytes()
    _decode_check(c, expect)


def test_layout3_heavy_tails_and_many_exponents():
    # rows of very different scales: dozens of occupied (sign, exponent)
    # symbols, each with its own h distribution in the joint table
    say("layout 3, many exponents")
    rng = np.random.default_rng(21)
    rows = [rng.standard_normal(4096) * np.exp(rng.uniform(np.log(1e-4), np.log(10.0))) for _ in range(200)]
    w = _words(np.concatenate(rows))
    c = _encode_both([O.bf16(w)], [codec.bf16(w)], 65536, 128, 128, 11)
    assert codec.record_info(c, 0).n_sym >= 50
    _decode_check(c, w.tobytes())


def test_layout3_special_values_and_residual():
    say("layout 3, special values + residual")
    rng = np.random.default_rng(1)
    specials = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81, 0x0001, 0x807F, 0x0080, 0x7F7F,
                         0xFF7F], np.uint16)
    body = _words(rng.standard_normal(70000) * 0.02)
    mix = np.concatenate([body, np.tile(specials, 500)])
    rng.shuffle(mix)
    allw = synth.as_words(synth.special_words()).numpy().astype(np.uint16)   # stored verbatim (> 256 symbols)
    half = allw[(allw >> 7) < 256].copy()                                     # every pattern with sign 0: coded
    raw = np.arange(3584, dtype=np.float32).tobytes()
    t_o = [O.bf16(mix), O.raw(raw), O.bf16(allw), O.raw(b"xyz"), O.bf16(np.zeros(0, np.uint16)),
           O.bf16(np.full(77, 0x3F80, np.uint16)), O.bf16(half)]
    t_l = [codec.bf16(mix), codec.raw(raw), codec.bf16(allw), codec.raw(b"xyz"), codec.bf16(np.zeros(0, np.uint16)),
           codec.bf16(np.full(77, 0x3F80, np.uint16)), codec.bf16(half)]
    c = _encode_both(t_o, t_l, 8192, 64, 64, 11)
    expect = _oracle_bytes(c)
    plan = codec.Plan(c)
    out = plan.decode()
    rc, rep = plan.verify(out, flags=L.VERIFY_STATUS | L.VERIFY_SHA256)
    assert rc == L.BS_OK, rep
    host = out.cpu().numpy().tobytes()
    for i in range(plan.n_records):
        ri = codec.record_info(c, i)
        nb = 2 * ri.n if ri.kind == L.KIND_BF16 else ri.n
        assert host[ri.out_offset: ri.out_offset + nb] == expect[ri.out_offset: ri.out_offset + nb], i


@pytest.mark.parametrize("stream_lanes,ms", [(0, 11), (64, 11), (128, 12)])
def test_layout3_many_records_mixed_lane_classes(stream_lanes, ms):
    """Hundreds of records of ragged sizes: small records get fewer lanes
    (other lanes-per-thread instances), more records than CUs, records cut
    into several workgroup runs, a middle record range."""
    say("layout 3, many records, stream lanes", stream_lanes, "m_s", ms)
    rng = np.random.default_rng(31 + ms)
    sizes = list(rng.integers(1, 3000, 700)) + list(rng.integers(3000, 140000, 60)) + [0, 8, 131072, 262144 + 17]
    rng.shuffle(sizes)
    t_o, t_l = [], []
    for i, n in enumerate(sizes):
        w = _words(rng.standard_normal(int(n)) * float(rng.choice([0.003, 0.02, 0.08])))
        t_o.append(O.bf16(w))
        t_l.append(codec.bf16(w))
        if i % 37 == 0:
            r = rng.integers(0, 256, int(rng.integers(1, 5000)), dtype=np.uint8)
            t_o.append(O.raw(r))
            t_l.append(codec.raw(r))
    c = _encode_both(t_o, t_l, 131072, 256, stream_lanes or 256, ms)
    expect = _oracle_bytes(c)
    plan, out = _decode_check(c, expect)
    first, count = 50, 400
    sub = plan.decode(first, count)
    torch.cuda.synchronize()
    for i in range(first, first + count):
        assert torch.equal(codec.record_output(sub, plan, i, first), codec.record_output(out, plan, i, 0)), i


def test_layout3_corrupt_payload_is_reported_not_crashing():
    say("layout 3, corrupt payload")
    rng = np.random.default_rng(5)
    w = _words(rng.standard_normal(65536 * 4) * 0.02)
    c = bytearray(codec.encode([codec.bf16(w)], codec.params3(chunk_weights=65536, lanes=64)))
    ri = codec.record_info(bytes(c), 0)
    for frac in (0.2, 0.7):
        pos = ri.rec_offset + int(ri.rec_len * frac)
        c[pos] ^= 0x5A
    plan = codec.Plan(bytes(c))
    out = plan.decode()
    ref = torch.from_numpy(w.view(np.uint8).copy()).cuda()
    rc, rep = plan.verify(out, ref=ref, flags=L.VERIFY_STATUS | L.VERIFY_COMPARE | L.VERIFY_SHA256)
    assert rc in (L.BS_E_CORRUPT, L.BS_E_MISMATCH)
    assert rep["bytes_mismatched"] > 0 and rep["records_hash_bad"] == 1


def test_layout3_device_tables_match_host_tables():
    # the histogram's negative counters per (exponent, h) give the joint
    # (sign, exponent, h) counts of the device model
    say("layout 3, device histogram tables")
    rng = np.random.default_rng(6)
    for x in [rng.standard_normal(1 << 20) * 0.02, rng.standard_normal(300001) * 0.3,
              np.where(rng.random(123457) < 0.1, 0.0, rng.standard_normal(123457))]:
        w = _words(x)
        dev = torch.from_numpy(w.view(np.int16)).cuda()
        for ms in (11, 12):
            p = codec.params3(m_s=ms)
            td = codec.build_tables(dev, p).get()
            th = codec.build_tables_host(w, p).get()
            for k in ("counts_s", "q_s", "q_t"):
                assert np.array_equal(td[k], th[k]), (k, ms)
            assert td["layout"] == 3 and int(td["q_t"].sum()) == 1 << 13


CASES_ENC = [
    # (name, sizes, chunk weights, lanes, lanes per stream, M_s)
    ("l3_k64_p32_two_streams", [5000, 70001], 4096, 64, 32, 11),
    ("l3_k128_full_and_ragged", [6 * 65536, 65536 + 1025], 65536, 128, 128, 11),
    ("l3_k256_p128_ms12", [131072 + 2049 + 7], 131072, 256, 128, 12),
    ("l3_k256_p128_checkpoint_shape", [3 * 65536 + 5, 5120], 65536, 256, 128, 11),
    ("l3_k2048_p64", [2 * 131072 + 8 * 333 + 3], 131072, 2048, 64, 11),
    ("l3_k1_tiny", [1, 8, 9], 64, 1, 1, 11),
]


@pytest.mark.parametrize("name,sizes,W,K,P,ms", CASES_ENC, ids=[c[0] for c in CASES_ENC])
def test_layout3_device_container_equals_host_container(name, sizes, W, K, P, ms):
    say("layout 3 encode case", name)
    rng = np.random.default_rng(len(name) + 300)
    words = []
    for i, n in enumerate(sizes):
        x = rng.standard_normal(n) * (0.02 if i % 2 == 0 else 1.0)
        x[rng.random(n) < 0.001] *= 60.0
        x[rng.random(n) < 0.01] = 0.0
        words.append(_words(x))
    raw = rng.integers(0, 256, 777, dtype=np.uint8)
    p = codec.params3(chunk_weights=W, lanes=K, stream_lanes=P, m_s=ms)
    host = codec.encode([codec.bf16(w) for w in words] + [codec.raw(raw)], p)
    assert host == O.encode([O.bf16(w) for w in words] + [O.raw(raw)], W=W, K=K, P=P, M_s=ms, M_f=13, layout=3)
    dev_tensors = [("bf16", torch.from_numpy(w.view(np.int16).copy()).cuda()) for w in words]
    dev_tensors.append(("raw", torch.from_numpy(raw.copy()).cuda()))
    digests = [hashlib.sha256(w.tobytes()).digest() for w in words] + [None]
    dc = codec.encode_device(dev_tensors, p, digests=digests)
    torch.cuda.synchronize()
    got = dc.cpu().numpy().tobytes()
    assert len(got) == len(host)
    if got != host:
        diff = np.flatnonzero(np.frombuffer(got, np.uint8) != np.frombuffer(host, np.uint8))
        pytest.fail(f"{diff.size} bytes differ, first at {diff[:8]}")
    _decode_check(got, _oracle_bytes(host))


def test_layout3_record_with_512_lane_streams_is_refused():
    say("layout 3, 512-lane stream refused")
    w = _words(np.random.default_rng(8).standard_normal(200000) * 0.02)
    c = O.encode([O.bf16(w)], W=65536, K=512, P=512, M_s=11, M_f=13, layout=3)
    with pytest.raises(L.BSError) as e:
        codec.Plan(c)
    assert e.value.rc == L.BS_E_INVAL


@pytest.mark.parametrize("ms,waves", [(12, 15), (11, 16)])
def test_layout3_full_workgroups(ms, waves):
    # the table image (64 KiB joint part + the s part) leaves room for 16
    # rings with M_s 11 and 15 with M_s 12; 4096 decode units (chunks of
    # 16384 weights, one 256-lane stream each), so that every workgroup has
    # at least 16 units and runs all of its waves
    say("layout 3, full workgroups, m_s", ms)
    rng = np.random.default_rng(40 + ms)
    w = _words(rng.standard_normal(1 << 26).astype(np.float32) * 0.02)
    c = codec.encode([codec.bf16(w)], codec.params3(chunk_weights=16384, lanes=256, stream_lanes=256, m_s=ms))
    plan = codec.Plan(c)
    assert plan.waves_per_block == waves
    out = plan.decode()
    ref = torch.from_numpy(w.view(np.uint8).copy()).cuda()
    rc, rep = plan.verify(out, ref=ref, flags=L.VERIFY_STATUS | L.VERIFY_COMPARE | L.VERIFY_SHA256)
    assert rc == L.BS_OK, rep
    assert torch.equal(out[: ref.numel()], ref)
    # and the oracle on sampled chunks of the same container
    for ch in (0, 777, 4095):
        got = O.decode_chunk(c, 0, ch)
        assert got.size == 16384 and np.array_equal(got, w[ch * 16384: (ch + 1) * 16384])
