"""GPU parity for layout-2 records (container version 2): the HIP decode path
against the original bits and the oracle.

Layout 2 codes s and the fraction's high three bits with one renormalisation
per weight and keeps the low four bits in a plane; the decode must still
reproduce every BF16 word [Qwen3.8-27B-BF16-NVLC-Lossless card, metrics table:
per-codec and integrated inverse verification; Gemma 2 9B Instruct --
Lossless Compressed card, "What lossless means"].  Every call goes through
the C ABI (bs_build_tables, bs_encode_host, bs_plan_create, bs_decode_async,
bs_verify) via the ctypes binding; the containers are checked byte for byte
against the oracle's encoder first.
"""
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


def _oracle_bytes(container: bytes) -> bytes:
    out, st = O.decode(container)
    assert all(s == 0 for s in st)
    return out


def _encode_both(tensors_o, tensors_l, W, K, P, M_s=11):
    c = codec.encode(tensors_l, codec.params2(chunk_weights=W, lanes=K, stream_lanes=P, m_s=M_s))
    assert c == O.encode(tensors_o, W=W, K=K, P=P, M_s=M_s, M_f=16 - M_s, cmax=31, layout=2)
    assert codec.container_info(c).version == 2
    return c


CASES = [
    # (name, n, scale, W, K, P, M_s)
    ("one_group", 8, 0.02, 64, 1, 1, 11),
    ("ragged_k1", 1001, 0.02, 64, 1, 1, 11),
    ("k8_ragged", 40000 + 13, 0.02, 4096, 8, 8, 12),
    ("k32_cfg1_shape", 3 * 32768 + 777, 0.02, 32768, 32, 32, 11),
    ("k64_full", 4 * 65536, 0.02, 65536, 64, 64, 11),
    ("k64_ragged", 3 * 65536 + 4099, 0.05, 65536, 64, 64, 12),
    ("k128_full", 6 * 65536, 0.02, 65536, 128, 128, 11),
    ("k128_ragged", 2 * 65536 + 1025, 0.003, 65536, 128, 128, 11),
    ("k256_full", 4 * 65536, 0.02, 65536, 256, 256, 11),
    ("k256_ragged", 131072 + 2049 + 7, 0.1, 131072, 256, 256, 12),
    ("small_k_tiny_chunks", 5000, 0.02, 512, 4, 4, 11),
    ("k256_p64_full", 4 * 131072, 0.02, 131072, 256, 64, 11),
    ("k256_p64_ragged", 2 * 131072 + 8 * 100 + 3, 0.05, 131072, 256, 64, 11),
    ("k512_p256_full", 3 * 65536, 0.02, 65536, 512, 256, 11),
    ("k512_p256_ragged", 2 * 65536 + 11, 0.03, 65536, 512, 256, 12),
    ("k512_p64_ragged", 262144 + 9999, 0.02, 262144, 512, 64, 11),
    ("k256_p128", 3 * 131072 + 77, 0.02, 131072, 256, 128, 11),
    ("k128_p32", 3 * 65536 + 5, 0.02, 65536, 128, 32, 11),
    ("k64_p8_small", 20000 + 3, 0.02, 8192, 64, 8, 11),
    ("k8_p1", 4096 + 9, 0.02, 4096, 8, 1, 11),
    ("k1024_p64", 2 * 131072 + 8 * 1000 + 5, 0.02, 131072, 1024, 64, 11),
    ("k1024_p128_short", 9000, 0.02, 131072, 1024, 128, 11),
    ("k2048_p64", 3 * 131072 + 8 * 2000 + 3, 0.02, 131072, 2048, 64, 11),
    ("k2048_p256_ragged", 131072 + 12345, 0.03, 131072, 2048, 256, 12),
    ("k2048_p64_short", 20001, 0.02, 131072, 2048, 64, 11),
]


@pytest.mark.parametrize("name,n,scale,W,K,P,ms", CASES, ids=[c[0] for c in CASES])
def test_layout2_decode_matches_oracle_and_original(name, n, scale, W, K, P, ms):
    say("layout 2 case", name, n, W, K, P, ms)
    rng = np.random.default_rng(n + 7)
    x = rng.standard_normal(n) * scale
    x[rng.random(n) < 0.01] = 0.0
    w = _words(x)
    c = _encode_both([O.bf16(w)], [codec.bf16(w)], W, K, P, ms)
    expect = _oracle_bytes(c)
    assert expect == w.tobytes()
    plan = codec.Plan(c)
    out = plan.decode()
    rc, rep = plan.verify(out, flags=L.VERIFY_STATUS | L.VERIFY_SHA256)
    assert out[: len(expect)].cpu().numpy().tobytes() == expect
    assert rc == L.BS_OK, rep
    assert rep["chunks_bad"] == 0 and rep["records_hash_bad"] == 0


def test_layout2_skewed_fractions_use_coded_tables():
    # heavy-tailed rows: many exponents whose high fraction bits are skewed,
    # so the record carries many coded h tables (up to the 31 allowed)
    say("layout 2, many coded h tables")
    rng = np.random.default_rng(21)
    rows = [rng.standard_normal(4096) * np.exp(rng.uniform(np.log(1e-4), np.log(10.0))) for _ in range(200)]
    w = _words(np.concatenate(rows))
    c = _encode_both([O.bf16(w)], [codec.bf16(w)], 65536, 128, 128, 11)
    assert codec.record_info(c, 0).n_tables >= 10
    plan = codec.Plan(c)
    out = plan.decode()
    rc, rep = plan.verify(out, flags=L.VERIFY_STATUS | L.VERIFY_SHA256)
    assert rc == L.BS_OK, rep
    assert out[: 2 * w.size].cpu().numpy().tobytes() == w.tobytes()


def test_layout2_special_values_and_residual():
    say("layout 2, special values + residual")
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
def test_layout2_many_records_mixed_lane_classes(stream_lanes, ms):
    """Hundreds of records of ragged sizes: small records get fewer lanes
    (other lanes-per-thread instances, fewer word streams), more records than
    CUs, records cut into several workgroup runs, a middle record range."""
    say("layout 2, many records, stream lanes", stream_lanes, "m_s", ms)
    rng = np.random.default_rng(11 + ms)
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
    info = codec.container_info(c)
    bf = [ri for ri in (codec.record_info(c, i) for i in range(info.n_records)) if ri.kind == L.KIND_BF16 and ri.n]
    classes = {max(ri.lanes // max(ri.streams, 1) // 64, 1) for ri in bf}
    # 64 lanes per stream put every record at one lane per thread; wider
    # streams leave the small records with fewer lanes than the large ones
    assert len(classes) >= (1 if stream_lanes == 64 else 2), classes
    expect = _oracle_bytes(c)
    plan = codec.Plan(c)
    out = plan.decode()
    rc, rep = plan.verify(out, flags=L.VERIFY_STATUS | L.VERIFY_SHA256)
    assert rc == L.BS_OK, rep
    assert out[: len(expect)].cpu().numpy().tobytes() == expect
    first, count = 50, 400
    sub = plan.decode(first, count)
    torch.cuda.synchronize()
    for i in range(first, first + count):
        assert torch.equal(codec.record_output(sub, plan, i, first), codec.record_output(out, plan, i, 0)), i


def test_layout2_guard_bytes_and_repeat():
    say("layout 2, guard bytes")
    w = _words(np.random.default_rng(4).standard_normal(65536 * 2 + 333) * 0.02)
    c = codec.encode([codec.bf16(w)], codec.params2(chunk_weights=65536, lanes=128))
    plan = codec.Plan(c)
    n = plan.out_bytes()
    buf = torch.full((n + 8192,), 0xA5, dtype=torch.uint8, device="cuda")
    out = buf[4096: 4096 + n]
    for _ in range(2):
        plan.decode_into(out)
        torch.cuda.synchronize()
        assert bool((buf[:4096] == 0xA5).all()) and bool((buf[4096 + n:] == 0xA5).all())
        assert out.cpu().numpy().tobytes() == w.tobytes()


def test_layout2_corrupt_payload_is_reported_not_crashing():
    say("layout 2, corrupt payload")
    rng = np.random.default_rng(5)
    w = _words(rng.standard_normal(65536 * 4) * 0.02)
    c = bytearray(codec.encode([codec.bf16(w)], codec.params2(chunk_weights=65536, lanes=64)))
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


def test_layout2_device_tables_match_host_tables():
    say("layout 2, device histogram tables")
    rng = np.random.default_rng(6)
    for x in [rng.standard_normal(1 << 20) * 0.02, rng.standard_normal(300001) * 0.3,
              np.where(rng.random(123457) < 0.1, 0.0, rng.standard_normal(123457))]:
        w = _words(x)
        dev = torch.from_numpy(w.view(np.int16)).cuda()
        for ms in (11, 12):
            p = codec.params2(m_s=ms)
            td = codec.build_tables(dev, p).get()
            th = codec.build_tables_host(w, p).get()
            for k in ("counts_s", "q_s", "route", "q_h"):
                assert np.array_equal(td[k], th[k]), (k, ms)
            assert td["n_tables"] == th["n_tables"] and td["layout"] == 2


def test_layout2_record_with_512_lane_streams_is_refused():
    # the format allows 512-lane streams, the layout-2 kernel takes 256: the
    # plan refuses such a record before anything is decoded
    say("layout 2, 512-lane stream refused")
    w = _words(np.random.default_rng(8).standard_normal(200000) * 0.02)
    c = O.encode([O.bf16(w)], W=65536, K=512, P=512, M_s=11, M_f=5, cmax=31, layout=2)
    with pytest.raises(L.BSError) as e:
        codec.Plan(c)
    assert e.value.rc == L.BS_E_INVAL


def test_layout2_shared_routes():
    """Shared routing: exponents without a table of their own routed to a
    coded table (the route byte names it), decoded on the GPU bit for bit;
    the GPU encoder's container equals the host's with the same routes."""
    say("layout 2, shared routes")
    rng = np.random.default_rng(21)
    words = []
    # exponent 120 earns a table; 100 and 99 (rare, h mostly 0 or 7) share it;
    # 101 uses an h that table has no room for and stays flat
    for e, hs, n in ((120, [0] * 90 + [7] * 7, 200000), (100, [0, 0, 0, 7], 12), (99, [0, 7, 7], 9),
                     (101, [0, 1], 10), (121, list(range(8)), 50000)):
        for _ in range(n):
            h = hs[int(rng.integers(len(hs)))]
            words.append((int(rng.integers(2)) << 15) | (e << 7) | (h << 4) | int(rng.integers(16)))
    w = np.array(words, np.uint16)
    rng.shuffle(w)
    t = codec.build_tables_host(w, codec.params2()).get()
    assert t["n_tables"] == 1 and t["route"][120] == 1
    assert t["route"][100] == 1 and t["route"][99] == 1 and t["route"][101] == 0 and t["route"][121] == 0
    cs, cf = O.histogram(w)
    route, nt, qh = O.select_htables(cs, cf, 5, 31)
    assert route[100] == 0 and route[99] == 0            # no table of their own: routed by sharing
    c = _encode_both([O.bf16(w)], [codec.bf16(w)], 65536, 128, 128)
    plan = codec.Plan(c)
    out = plan.decode()
    torch.cuda.synchronize()
    assert out[: 2 * w.size].cpu().numpy().view(np.uint16).tolist() == w.tolist()
    assert out[: 2 * w.size].cpu().numpy().tobytes() == _oracle_bytes(c)[: 2 * w.size]
    rc, rep = plan.verify(out, flags=L.VERIFY_STATUS | L.VERIFY_SHA256)
    assert rc == L.BS_OK, rep
    dev = codec.encode_device([("bf16", torch.from_numpy(w.view(np.int16)).cuda())], codec.params2(lanes=128, stream_lanes=128))
    assert dev.cpu().numpy().tobytes() == c


def _words_31_tables(seed: int) -> np.ndarray:
    """40 exponents of 6,000 weights each, each with a different dominant h:
    more eligible h tables than the 31 a record may hold."""
    rng = np.random.default_rng(seed)
    parts = []
    for k, e in enumerate(range(90, 130)):
        p = np.full(8, 0.2 / 7)
        p[k % 8] = 0.8
        h = rng.choice(8, size=6000, p=p)
        sign = rng.integers(0, 2, 6000)
        parts.append((sign << 15) | (e << 7) | (h << 4) | rng.integers(0, 16, 6000))
    w = np.concatenate(parts).astype(np.uint16)
    rng.shuffle(w)
    return w


@pytest.mark.parametrize("ms,P", [(12, 256), (11, 256), (12, 128)])
def test_layout2_largest_table_image(ms, P):
    """31 coded h tables: the largest table image a record can have (with
    M_s = 12, 96 KiB of LDS before the rings, so a workgroup runs fewer
    waves), decoded bit for bit."""
    say("layout 2, 31 h tables, m_s", ms, "stream lanes", P)
    w = _words_31_tables(5)
    c = _encode_both([O.bf16(w)], [codec.bf16(w)], 16384, 256, P, ms)
    assert codec.record_info(c, 0).n_tables == 31
    plan = codec.Plan(c)
    for _ in range(2):
        out = plan.decode()
        rc, rep = plan.verify(out, flags=L.VERIFY_STATUS | L.VERIFY_SHA256)
        assert rc == L.BS_OK, rep
        assert out[: 2 * w.size].cpu().numpy().tobytes() == w.tobytes()


@pytest.mark.parametrize("ms,waves", [(12, 15), (11, 16)])
def test_layout2_largest_table_image_full_workgroups(ms, waves):
    """The same tables over enough chunks (about 65M weights) that every
    workgroup runs as many waves as fit after the table image: 15 with
    M_s = 12 (96 KiB of tables), 16 with M_s = 11; compared with the original
    words on the device and through the record digest."""
    say("layout 2, 31 h tables, full workgroups, m_s", ms)
    w = np.tile(_words_31_tables(5), 270)
    c = codec.encode([codec.bf16(w)], codec.params2(chunk_weights=16384, lanes=256, stream_lanes=256, m_s=ms))
    assert codec.record_info(c, 0).n_tables == 31
    plan = codec.Plan(c)
    assert plan.waves_per_block == waves
    out = plan.decode()
    rc, rep = plan.verify(out, flags=L.VERIFY_STATUS | L.VERIFY_SHA256)
    assert rc == L.BS_OK, rep
    ref = torch.from_numpy(w.view(np.int16)).cuda()
    assert torch.equal(out[: 2 * w.size].view(torch.int16), ref)
