"""GPU parity: the HIP decode path against the original bits and the oracle.

Bit-exact equality is the bar: decoding must reproduce every BF16 word
[Qwen3.8-27B-BF16-NVLC-Lossless card, metrics table: per-codec and integrated
inverse verification; Gemma 2 9B Instruct -- Lossless Compressed card, "What
lossless means"].  Every call goes through the C ABI (bs_plan_create,
bs_decode_async, bs_verify, bs_build_tables) via the ctypes binding.
"""
import hashlib
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from lossless_entropy_coding_amd import _lib as L
from lossless_entropy_coding_amd import codec, synth

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def _words(x) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def _decode_check(container: bytes, expect: bytes, flags=L.VERIFY_STATUS | L.VERIFY_SHA256):
    plan = codec.Plan(container)
    out = plan.decode()
    rc, rep = plan.verify(out, flags=flags)
    got = out[: len(expect)].cpu().numpy().tobytes()
    return plan, out, rc, rep, got


def _expected_bytes(container: bytes) -> bytes:
    out, st = O.decode(container)
    assert all(s == 0 for s in st)
    return out


CASES = [
    # (name, n, scale, W, K, P = lanes per word stream)
    ("one_group", 8, 0.02, 64, 1, 1),
    ("ragged_k1", 1001, 0.02, 64, 1, 1),
    ("k8_ragged", 40000 + 13, 0.02, 4096, 8, 8),
    ("k32_cfg1_shape", 3 * 32768 + 777, 0.02, 32768, 32, 32),
    ("k64_full", 4 * 65536, 0.02, 65536, 64, 64),
    ("k64_ragged", 3 * 65536 + 4099, 0.05, 65536, 64, 64),
    ("k128_full", 6 * 65536, 0.02, 65536, 128, 128),
    ("k128_ragged", 2 * 65536 + 1025, 0.003, 65536, 128, 128),
    ("k256_full", 4 * 131072, 0.02, 131072, 256, 256),
    ("k256_ragged", 131072 + 2049 + 7, 0.1, 131072, 256, 256),
    ("small_k_tiny_chunks", 5000, 0.02, 512, 4, 4),
    ("k512_full", 2 * 262144, 0.02, 262144, 512, 512),
    ("k512_ragged", 262144 + 4096 * 3 + 5, 0.05, 262144, 512, 512),
    ("k512_one_chunk_short", 70001, 0.02, 262144, 512, 512),
    # chunks split into word streams, one wavefront per stream
    ("k256_p64_full", 4 * 131072, 0.02, 131072, 256, 64),
    ("k256_p64_ragged", 2 * 131072 + 8 * 100 + 3, 0.05, 131072, 256, 64),
    ("k512_p64_ragged", 262144 + 9999, 0.02, 262144, 512, 64),
    ("k256_p128", 3 * 131072 + 77, 0.02, 131072, 256, 128),
    ("k512_p256", 2 * 262144 + 11, 0.03, 262144, 512, 256),
    ("k128_p32", 3 * 65536 + 5, 0.02, 65536, 128, 32),
    ("k64_p8_small", 20000 + 3, 0.02, 8192, 64, 8),
    ("k8_p1", 4096 + 9, 0.02, 4096, 8, 1),
    ("k1024_p64", 2 * 131072 + 8 * 1000 + 5, 0.02, 131072, 1024, 64),
    ("k1024_p512", 262144 + 3, 0.03, 262144, 1024, 512),
    ("k1024_p128_short", 9000, 0.02, 131072, 1024, 128),
    ("k2048_p64", 3 * 131072 + 8 * 2000 + 3, 0.02, 131072, 2048, 64),
    ("k2048_p256_ragged", 131072 + 12345, 0.03, 131072, 2048, 256),
    ("k2048_p64_short", 20001, 0.02, 131072, 2048, 64),
]


@pytest.mark.parametrize("name,n,scale,W,K,P", CASES, ids=[c[0] for c in CASES])
def test_decode_matches_oracle_and_original(name, n, scale, W, K, P):
    say("case", name, n, W, K, P)
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n) * scale
    x[rng.random(n) < 0.01] = 0.0
    w = _words(x)
    c = codec.encode([codec.bf16(w)], codec.params(chunk_weights=W, lanes=K, stream_lanes=P))
    assert c == O.encode([O.bf16(w)], W=W, K=K, P=P)
    expect = _expected_bytes(c)
    assert expect == w.tobytes()
    plan, out, rc, rep, got = _decode_check(c, expect)
    assert got == expect
    assert rc == L.BS_OK, rep
    assert rep["chunks_bad"] == 0 and rep["records_hash_bad"] == 0


COMPACT_CASES = [
    # (name, n, scale, W, K, P, M_s, M_f): tables small enough for the compact LDS layout
    ("compact_k128", 3 * 65536 + 999, 0.02, 65536, 128, 128, 11, 9),
    ("compact_k128_p64", 2 * 65536 + 17, 0.05, 65536, 128, 64, 11, 9),
    ("compact_k256_r4", 2 * 131072 + 3, 0.02, 131072, 256, 256, 11, 9),
    ("compact_k32_small_tables", 50000 + 1, 0.02, 32768, 32, 32, 9, 8),
    ("full_k128_ms11_mf10", 2 * 65536 + 5, 0.02, 65536, 128, 128, 11, 10),
    ("k512_ms10_mf8", 262144 + 1001, 0.02, 262144, 512, 512, 10, 8),
]


@pytest.mark.parametrize("name,n,scale,W,K,P,ms,mf", COMPACT_CASES, ids=[c[0] for c in COMPACT_CASES])
def test_decode_table_precisions(name, n, scale, W, K, P, ms, mf):
    say("case", name, n, W, K, P, ms, mf)
    rng = np.random.default_rng(n + ms)
    x = rng.standard_normal(n) * scale
    x[rng.random(n) < 0.01] = 0.0
    w = _words(x)
    c = codec.encode([codec.bf16(w)], codec.params(chunk_weights=W, lanes=K, stream_lanes=P, m_s=ms, m_f=mf))
    assert c == O.encode([O.bf16(w)], W=W, K=K, P=P, M_s=ms, M_f=mf)
    expect = _expected_bytes(c)
    assert expect == w.tobytes()
    plan, out, rc, rep, got = _decode_check(c, expect)
    assert got == expect
    assert rc == L.BS_OK, rep


def test_special_values_and_residual():
    say("special values + residual")
    rng = np.random.default_rng(1)
    specials = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81, 0x0001, 0x807F, 0x0080, 0x7F7F,
                         0xFF7F], np.uint16)
    body = _words(rng.standard_normal(70000) * 0.02)
    mix = np.concatenate([body, np.tile(specials, 500)])
    rng.shuffle(mix)
    allw = synth.as_words(synth.special_words()).numpy().astype(np.uint16)   # stored verbatim (> 256 symbols)
    raw = np.arange(3584, dtype=np.float32).tobytes()
    tensors = [codec.bf16(mix), codec.raw(raw), codec.bf16(allw), codec.raw(b"xyz"), codec.bf16(np.zeros(0, np.uint16)),
               codec.bf16(np.full(77, 0x3F80, np.uint16))]
    c = codec.encode(tensors, codec.params(chunk_weights=8192, lanes=64))
    expect = _expected_bytes(c)
    plan = codec.Plan(c)
    out = plan.decode()
    rc, rep = plan.verify(out, flags=L.VERIFY_STATUS | L.VERIFY_SHA256)
    assert rc == L.BS_OK, rep
    host = out.cpu().numpy().tobytes()
    for i in range(plan.n_records):
        ri = codec.record_info(c, i)
        nb = 2 * ri.n if ri.kind == L.KIND_BF16 else ri.n
        assert host[ri.out_offset: ri.out_offset + nb] == expect[ri.out_offset: ri.out_offset + nb], i


@pytest.mark.parametrize("stream_lanes,ms,mf", [(0, 12, 10), (64, 12, 10), (0, 11, 9), (64, 11, 9)])
def test_many_records_mixed_lane_classes(stream_lanes, ms, mf):
    """Hundreds of records of ragged sizes in one container: small records get
    fewer lanes (other lanes-per-thread classes, or fewer word streams), more
    records than CUs, and records cut into several workgroup runs."""
    say("many records, mixed classes, stream lanes", stream_lanes)
    rng = np.random.default_rng(11)
    sizes = list(rng.integers(1, 3000, 700)) + list(rng.integers(3000, 140000, 60)) + [0, 8, 131072, 262144 + 17]
    rng.shuffle(sizes)
    tensors = []
    for i, n in enumerate(sizes):
        x = rng.standard_normal(int(n)) * float(rng.choice([0.003, 0.02, 0.08]))
        tensors.append(codec.bf16(_words(x)))
        if i % 37 == 0:
            tensors.append(codec.raw(rng.integers(0, 256, int(rng.integers(1, 5000)), dtype=np.uint8)))
    c = codec.encode(tensors, codec.params(chunk_weights=131072, lanes=256, stream_lanes=stream_lanes, m_s=ms, m_f=mf))
    info = codec.container_info(c)
    ris = [codec.record_info(c, i) for i in range(info.n_records)]
    bf = [ri for ri in ris if ri.kind == L.KIND_BF16 and ri.n]
    if stream_lanes:
        assert {ri.streams for ri in bf} >= {1, 2, 4}
    else:
        assert len({max(ri.lanes // 64, 1) for ri in bf}) >= 3
    expect = _expected_bytes(c)
    plan, out, rc, rep, got = _decode_check(c, expect)
    assert rc == L.BS_OK, rep
    assert got == expect
    # a middle sub-range decodes to the same bytes as in the full decode
    first, count = 50, 400
    sub = plan.decode(first, count)
    torch.cuda.synchronize()
    for i in range(first, first + count):
        assert torch.equal(codec.record_output(sub, plan, i, first), codec.record_output(out, plan, i, 0)), i


def test_record_range_and_determinism():
    say("record ranges")
    rng = np.random.default_rng(2)
    ws = [_words(rng.standard_normal(n) * s) for n, s in [(65536 * 3, 0.02), (5000, 0.01), (131072 + 99, 0.04)]]
    tensors = [codec.bf16(ws[0]), codec.raw(b"q" * 1000), codec.bf16(ws[1]), codec.bf16(ws[2])]
    c = codec.encode(tensors, codec.params(chunk_weights=65536, lanes=128))
    plan = codec.Plan(c)
    full = plan.decode()
    again = plan.decode()
    torch.cuda.synchronize()
    assert torch.equal(full, again)
    for first, count in [(0, 1), (1, 2), (2, 2), (3, 1), (0, 4)]:
        out = plan.decode(first, count)
        torch.cuda.synchronize()
        for i in range(first, first + count):
            a = codec.record_output(out, plan, i, first)
            b = codec.record_output(full, plan, i, 0)
            assert torch.equal(a, b), (first, count, i)
    rc, rep = plan.verify(plan.decode(1, 3), flags=L.VERIFY_STATUS | L.VERIFY_SHA256, first=1, count=3)
    assert rc == L.BS_OK, rep


def test_output_capacity_and_alignment_errors():
    say("capacity errors")
    w = _words(np.random.default_rng(3).standard_normal(10000) * 0.02)
    c = codec.encode([codec.bf16(w)], codec.params(chunk_weights=4096, lanes=8))
    plan = codec.Plan(c)
    small = torch.empty(100, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.BSError) as e:
        plan.decode_into(small)
    assert e.value.rc == L.BS_E_NOSPACE
    big = torch.empty(plan.out_bytes() + 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.BSError) as e:
        plan.decode_into(big[8:])
    assert e.value.rc == L.BS_E_INVAL


def test_guard_bytes_untouched():
    say("guard bytes")
    w = _words(np.random.default_rng(4).standard_normal(65536 * 2 + 333) * 0.02)
    c = codec.encode([codec.bf16(w)], codec.params(chunk_weights=65536, lanes=128))
    plan = codec.Plan(c)
    n = plan.out_bytes()
    buf = torch.full((n + 4096 + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    out = buf[4096: 4096 + n]
    plan.decode_into(out)
    torch.cuda.synchronize()
    assert bool((buf[:4096] == 0xA5).all()) and bool((buf[4096 + n:] == 0xA5).all())
    assert out.cpu().numpy().tobytes() == w.tobytes()


def test_corrupt_payload_is_reported_not_crashing():
    say("corrupt payload")
    rng = np.random.default_rng(5)
    w = _words(rng.standard_normal(65536 * 4) * 0.02)
    c = bytearray(codec.encode([codec.bf16(w)], codec.params(chunk_weights=65536, lanes=64)))
    ri = codec.record_info(bytes(c), 0)
    # flip bytes inside the payload area of the first and third chunk (past the index)
    for frac in (0.2, 0.7):
        pos = ri.rec_offset + int(ri.rec_len * frac)
        c[pos] ^= 0x5A
    plan = codec.Plan(bytes(c))
    out = plan.decode()
    ref = torch.from_numpy(w.view(np.uint8).copy()).cuda()
    rc, rep = plan.verify(out, ref=ref, flags=L.VERIFY_STATUS | L.VERIFY_COMPARE | L.VERIFY_SHA256)
    assert rc in (L.BS_E_CORRUPT, L.BS_E_MISMATCH)
    assert rep["chunks_bad"] >= 1 and rep["bytes_mismatched"] > 0 and rep["records_hash_bad"] == 1


def test_device_tables_match_host_tables():
    say("device histogram tables")
    rng = np.random.default_rng(6)
    for x in [rng.standard_normal(1 << 20) * 0.02, rng.standard_normal(300001) * 0.3,
              np.where(rng.random(123457) < 0.1, 0.0, rng.standard_normal(123457))]:
        w = _words(x)
        dev = torch.from_numpy(w.view(np.int16)).cuda()
        for off in (0, 1, 3):   # unaligned starts exercise the head/tail path
            td = codec.build_tables(dev[off:]).get()
            th = codec.build_tables_host(w[off:]).get()
            for k in ("counts_s", "q_s", "route", "q_f"):
                assert np.array_equal(td[k], th[k]), (k, off)
            assert td["n_tables"] == th["n_tables"]
            cs, cf = O.histogram(w[off:])
            assert np.array_equal(td["counts_s"], cs)


def test_device_tables_encode_same_container():
    say("encode with device tables")
    wl = synth.cfg1()
    w = synth.as_words(wl.items[0].tensor).numpy().astype(np.uint16)
    p = codec.params(chunk_weights=wl.chunk_weights, lanes=wl.lanes)
    t = codec.build_tables(torch.from_numpy(w.view(np.int16)).cuda(), p)
    c1 = codec.encode([codec.bf16(w, t)], p)
    c2 = O.encode([O.bf16(w)], W=wl.chunk_weights, K=wl.lanes)
    assert c1 == c2
