"""Host-side parts of the HIP library against the oracle (no GPU needed).

The library's encoder, model building, container validation and sha256 are
host C++ written independently of the oracle; the container is a
deterministic encoding, so the two must agree byte for byte.
"""
import ctypes as C
import hashlib
import os
import re
import struct

import numpy as np
import pytest
import torch

from oracle import oracle as O
from lossless_entropy_coding_amd import _lib as L
from lossless_entropy_coding_amd import codec, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_declared_symbol_is_exported():
    hdr = open(os.path.join(ROOT, "include", "bs.h")).read()
    decl = set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(bs_\w+)\s*\(", hdr, re.M))
    assert len(decl) >= 20, decl
    lib = L.lib()
    missing = [n for n in decl if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding declares exactly the header's functions
    assert decl == set(L.SIGNATURES), decl ^ set(L.SIGNATURES)


def _words(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def _same(tensors_o, tensors_l, **kw):
    p = codec.params(chunk_weights=kw.get("W", 65536), lanes=kw.get("K", 64), m_s=kw.get("M_s", 12),
                     m_f=kw.get("M_f", 10), max_tables=kw.get("cmax", 6), stream_lanes=kw.get("P") or 0)
    a = O.encode(tensors_o, **kw)
    b = codec.encode(tensors_l, p)
    assert a == b
    return a


@pytest.mark.parametrize("seed,n,W,K", [(0, 100000, 4096, 8), (1, 33333, 2048, 16), (2, 8, 64, 1), (3, 0, 64, 2),
                                        (4, 70000, 65536, 128), (5, 5000, 65536, 256), (6, 262144, 131072, 256),
                                        (7, 300000, 262144, 512)])
def test_encoder_bytes_match_oracle(seed, n, W, K):
    rng = np.random.default_rng(seed)
    w = _words(rng.standard_normal(n) * rng.choice([0.004, 0.02, 0.1]))
    _same([O.bf16(w)], [codec.bf16(w)], W=W, K=K)


@pytest.mark.parametrize("seed,n,W,K,P", [(10, 100000, 4096, 8, 2), (11, 40000, 8192, 64, 16), (12, 300000, 131072, 256, 64),
                                          (13, 5000, 131072, 256, 64), (14, 70001, 65536, 128, 1), (15, 0, 64, 8, 4),
                                          (16, 262144 * 2 + 5, 262144, 512, 128), (17, 131072 * 2 + 77, 131072, 1024, 64),
                                          (18, 3000, 131072, 1024, 512), (19, 131072 * 2 + 8 * 2047 + 3, 131072, 2048, 64),
                                          (20, 5000, 131072, 2048, 512)])
def test_encoder_bytes_match_oracle_streams(seed, n, W, K, P):
    rng = np.random.default_rng(seed)
    w = _words(rng.standard_normal(n) * rng.choice([0.004, 0.02, 0.1]))
    c = _same([O.bf16(w)], [codec.bf16(w)], W=W, K=K, P=P)
    info = codec.container_info(c)
    ri = codec.record_info(c, 0)
    assert ri.streams == (ri.lanes // min(P, ri.lanes) if n else 1)
    assert info.n_streams == ri.n_chunks * ri.streams


def test_encoder_bytes_match_oracle_cfg1():
    wl = synth.cfg1()
    w = synth.as_words(wl.items[0].tensor).numpy().astype(np.uint16)
    _same([O.bf16(w)], [codec.bf16(w)], W=wl.chunk_weights, K=wl.lanes)


def test_encoder_bytes_match_oracle_mixed_records():
    rng = np.random.default_rng(9)
    a = _words(rng.standard_normal(20000) * 0.02)
    zeros = np.zeros(4096, np.uint16)
    ones = np.full(1000, 0x3F80, np.uint16)
    specials = synth.as_words(synth.special_words()).numpy().astype(np.uint16)   # > 256 symbols -> raw
    r = np.arange(3584, dtype=np.float32).tobytes()
    outl = np.where(rng.random(30000) < 0.01, 50.0, 1.0) * rng.standard_normal(30000) * 0.02
    b = _words(np.where(rng.random(30000) < 0.05, 0.0, outl))
    tens_o = [O.bf16(a), O.raw(r), O.bf16(zeros), O.bf16(ones), O.bf16(specials), O.raw(b"abc"), O.bf16(b)]
    tens_l = [codec.bf16(a), codec.raw(r), codec.bf16(zeros), codec.bf16(ones), codec.bf16(specials),
              codec.raw(b"abc"), codec.bf16(b)]
    c = _same(tens_o, tens_l, W=4096, K=32)
    info = codec.container_info(c)
    assert info.n_records == 7
    assert codec.record_info(c, 4).kind == L.KIND_RAW   # too many symbols: verbatim


def test_models_match_oracle():
    rng = np.random.default_rng(12)
    for scale in (0.003, 0.02, 0.3):
        x = rng.standard_normal(200000) * scale
        x[rng.random(x.size) < 0.02] = 0.0
        w = _words(x)
        t = codec.build_tables_host(w).get()
        cs, cf = O.histogram(w)
        assert (t["counts_s"] == cs).all()
        assert (t["q_s"] == O.normalise(cs, 12)).all()
        route, nt, qf = O.select_tables(cs, cf, 10, 6)
        assert nt == t["n_tables"] and (route == t["route"]).all() and (qf == t["q_f"]).all()


def test_sha256_matches_hashlib():
    rng = np.random.default_rng(0)
    for n in [0, 1, 55, 56, 63, 64, 65, 119, 120, 1000, 1 << 20]:
        b = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert codec.sha256(b) == hashlib.sha256(b).digest()


def test_encoder_deterministic_across_threads():
    rng = np.random.default_rng(3)
    w = _words(rng.standard_normal(500000) * 0.02)
    outs = {codec.encode([codec.bf16(w)], codec.params(chunk_weights=32768, lanes=64, threads=t)) for t in (1, 3, 8)}
    assert len(outs) == 1


def test_validation_errors():
    rng = np.random.default_rng(4)
    w = _words(rng.standard_normal(50000) * 0.02)
    c = codec.encode([codec.bf16(w)], codec.params(chunk_weights=4096, lanes=8))
    codec.container_info(c)
    bad = bytearray(c)
    bad[8:12] = struct.pack("<I", 4)
    with pytest.raises(L.BSError) as e:
        codec.container_info(bytes(bad))
    assert e.value.rc == L.BS_E_VERSION
    # version 2 names every BF16 record's layout: a version-1 record's 0 is malformed there
    bad[8:12] = struct.pack("<I", 2)
    with pytest.raises(L.BSError) as e:
        codec.container_info(bytes(bad))
    assert e.value.rc == L.BS_E_FORMAT
    with pytest.raises(L.BSError) as e:
        codec.container_info(c[:-16])
    assert e.value.rc == L.BS_E_FORMAT
    # a record running past the container end
    short = bytearray(c[:-16])
    short[24:32] = struct.pack("<Q", len(short))
    with pytest.raises(L.BSError) as e:
        codec.container_info(bytes(short))
    assert e.value.rc == L.BS_E_FORMAT
    # a chunk payload offset pointing past the record
    ri = codec.record_info(c, 0)
    body = ri.rec_offset
    n_sym = struct.unpack_from("<I", c, body + 16)[0]
    nt = c[body + 14]
    idx = body + ((((24 + 5 * n_sym + 3) // 4) * 4 + 256 * nt + 15) // 16) * 16
    bad = bytearray(c)
    bad[idx:idx + 8] = struct.pack("<Q", ri.rec_len + 4096)
    with pytest.raises(L.BSError) as e:
        codec.container_info(bytes(bad))
    assert e.value.rc == L.BS_E_FORMAT
    # frequencies that do not sum to 2^M
    bad = bytearray(c)
    q = struct.unpack_from("<H", bad, body + 26)[0]
    struct.pack_into("<H", bad, body + 26, q + 1)
    with pytest.raises(L.BSError) as e:
        codec.container_info(bytes(bad))
    assert e.value.rc == L.BS_E_FORMAT


def test_stream_table_validation():
    """The record's stream table must give ascending starts inside the chunk's
    stream area, each stream at least as long as its lanes' state bits."""
    rng = np.random.default_rng(7)
    w = _words(rng.standard_normal(4096 * 3) * 0.02)
    c = codec.encode([codec.bf16(w)], codec.params(chunk_weights=4096, lanes=64, stream_lanes=16))
    assert c == O.encode([O.bf16(w)], W=4096, K=64, P=16)
    codec.container_info(c)
    ri = codec.record_info(c, 0)
    body = ri.rec_offset
    n_sym = struct.unpack_from("<I", c, body + 16)[0]
    nt = c[body + 14]
    idx = body + ((((24 + 5 * n_sym + 3) // 4) * 4 + 256 * nt + 15) // 16) * 16
    n_chunks = struct.unpack_from("<I", c, body + 8)[0]
    stab = idx + 16 * n_chunks            # chunk 0: starts of streams 1, 2, 3
    s1, s2, s3 = struct.unpack_from("<III", c, stab)
    total = struct.unpack_from("<I", c, idx + 8)[0]
    assert 0 < s1 < s2 < s3 < total
    for vals in [(s2 + 1, s2, s3), (s1, s2, total + 1), (1, s2, s3)]:
        bad = bytearray(c)
        struct.pack_into("<III", bad, stab, *vals)
        with pytest.raises(L.BSError) as e:
            codec.container_info(bytes(bad))
        assert e.value.rc == L.BS_E_FORMAT, vals


def test_bad_params_rejected():
    w = np.zeros(100, np.uint16)
    for kw in [dict(lanes=3), dict(lanes=96), dict(lanes=1024, chunk_weights=1 << 20), dict(lanes=64, stream_lanes=128),
               dict(lanes=64, stream_lanes=48), dict(chunk_weights=100, lanes=8), dict(m_s=13), dict(m_f=6), dict(m_f=7),
               dict(max_tables=7)]:
        with pytest.raises(L.BSError) as e:
            codec.encode([codec.bf16(w)], codec.params(**kw))
        assert e.value.rc == L.BS_E_INVAL


def test_write_file_refuses_existing(tmp_path):
    p = str(tmp_path / "c.bs")
    codec.write_new(p, b"abc")
    assert open(p, "rb").read() == b"abc"
    with pytest.raises(L.BSError) as e:
        codec.write_new(p, b"xyz")
    assert e.value.rc == L.BS_E_EXISTS
    assert open(p, "rb").read() == b"abc"


# --------------------------------------------------------------------------- fixed-width lane streams
@pytest.mark.parametrize("n,kind", [(0, "gauss"), (1, "gauss"), (35, "gauss"), (2048, "gauss"), (70001, "gauss"),
                                    (3 * 2048 + 77, "uniform"), (65536, "patterns"), (5 * 2048 + 9, "wide")])
def test_fixed_encoder_matches_oracle(n, kind):
    rng = np.random.default_rng(n)
    if kind == "gauss":
        w = _words(rng.standard_normal(n) * 0.02)
    elif kind == "uniform":
        w = rng.integers(0, 1 << 16, n, dtype=np.uint16)
    elif kind == "wide":
        w = _words(rng.standard_normal(n) * np.exp(rng.standard_normal(n) * 4))
    else:
        w = np.arange(n, dtype=np.uint16)
    want = O.fixed_encode(w)
    for threads in (0, 1, 3):
        assert codec.fixed_encode(w, threads=threads) == want
    info = codec.fixed_info(want)
    assert (info.n, info.n_blocks, info.bytes) == (n, (n + 2047) // 2048, len(want))
    assert list(info.table) == list(struct.unpack_from("<16H", want, 64))


def test_fixed_info_validation():
    w = _words(np.random.default_rng(4).standard_normal(5000) * 0.02)
    blob = codec.fixed_encode(w)

    def bad(off, fmt, value):
        b = bytearray(blob)
        struct.pack_into(fmt, b, off, value)
        return bytes(b)
    for b, rc in [(b"BF16FIX0" + blob[8:], L.BS_E_FORMAT), (bad(8, "<I", 2), L.BS_E_VERSION),
                  (bad(24, "<Q", 4), L.BS_E_FORMAT), (bad(32, "<Q", 0), L.BS_E_FORMAT),
                  (bad(40, "<Q", 10 ** 6), L.BS_E_FORMAT), (bad(64, "<H", 512), L.BS_E_FORMAT),
                  (bad(94, "<H", 3), L.BS_E_FORMAT), (blob[:95], L.BS_E_FORMAT)]:
        with pytest.raises(L.BSError) as e:
            codec.fixed_info(b)
        assert e.value.rc == rc
    with pytest.raises(L.BSError) as e:                      # the whole blob must be there
        codec.fixed_info(blob[:96], blob_len=len(blob) - 16)
    assert e.value.rc == L.BS_E_FORMAT
    assert codec.fixed_info(blob[:96], blob_len=len(blob)).bytes == len(blob)


def test_fixed_decode_argument_checks_before_launch():
    import ctypes as C
    w = _words(np.random.default_rng(5).standard_normal(5000) * 0.02)
    info = codec.fixed_info(codec.fixed_encode(w))
    f = L.lib().bs_fixed_decode_async
    assert f(None, C.c_void_p(4096), C.c_void_p(4096), 10000, None, None) == L.BS_E_INVAL
    assert f(C.byref(info), C.c_void_p(4100), C.c_void_p(4096), 10000, None, None) == L.BS_E_INVAL
    assert f(C.byref(info), C.c_void_p(4096), C.c_void_p(4104), 10000, None, None) == L.BS_E_INVAL
    assert f(C.byref(info), C.c_void_p(4096), C.c_void_p(4096), 9999, None, None) == L.BS_E_NOSPACE
    forged = L.FixedInfo.from_buffer_copy(info)
    forged.n_blocks += 1
    assert f(C.byref(forged), C.c_void_p(4096), C.c_void_p(4096), 10000, None, None) == L.BS_E_INVAL
    empty = codec.fixed_info(codec.fixed_encode(np.zeros(0, np.uint16)))
    assert f(C.byref(empty), C.c_void_p(4096), None, 0, None, None) == L.BS_OK     # nothing to do


@pytest.mark.parametrize("layout,n,W,K,P", [(1, 100000, 4096, 8, 2), (2, 70001, 65536, 128, 64), (3, 300000, 131072, 256, 64),
                                             (3, 5000, 131072, 256, 0), (1, 0, 64, 8, 0), (3, 33333, 32768, 128, 128)])
def test_size_breakdown_adds_up_and_matches_the_layout(layout, n, W, K, P):
    """bs_container_sizes_get against a walk of the container written here
    from the layout bs.h documents: the fixed parts, tables, index, length
    codes and planes from the header fields, the state bits from the lanes'
    length codes read out of each payload, the words from the index's unit
    counts; the parts sum to 8 x the BF16 bytes."""
    rng = np.random.default_rng(n + W + K + layout)
    w = _words(rng.standard_normal(n) * 0.02)
    mk = {1: codec.params, 2: codec.params2, 3: codec.params3}[layout]
    p = mk(chunk_weights=W, lanes=K, stream_lanes=P)
    blob = codec.encode([codec.bf16(w), codec.raw(np.arange(77, dtype=np.uint8))], p)
    sz = codec.container_sizes(blob)
    info = codec.container_info(blob)
    parts = [v for k, v in sz.items() if k != "weights"]
    assert sz["weights"] == n and sum(parts) == 8 * info.bf16_bytes
    if n == 0:                                  # nothing is charged to BF16 weights
        assert not any(parts)
        return
    ri = codec.record_info(blob, 0)
    b = blob[ri.rec_offset: ri.rec_offset + ri.rec_len]
    n_chunks, S = ri.n_chunks, ri.streams
    K, W = ri.lanes, ri.chunk_weights          # a record smaller than a chunk gets fewer lanes
    rd = lambda o, k: int.from_bytes(b[o: o + k], "little")
    assert sz["fixed_bits"] == 8 * 24
    first = rd(index_off := sz["fixed_bits"] // 8 + sz["table_bits"] // 8, 8) if n_chunks else ri.rec_len
    assert sz["index_bits"] == 8 * (first - index_off) and first - index_off >= 16 * n_chunks + 4 * (S - 1) * n_chunks
    codes = -(-((K + 1) // 2) // 16) * 16
    assert sz["code_bits"] == 8 * codes * n_chunks
    n_c = [min(W, n - c * W) for c in range(n_chunks)]
    assert sz["plane_bits"] == (8 * sum(-(-(4 * -(-m // 8)) // 16) * 16 for m in n_c) if layout >= 2 else 0)
    lanes_per = K // S
    state = words = 0
    for c in range(n_chunks):
        po, total = rd(index_off + 16 * c, 8), rd(index_off + 16 * c + 8, 4)
        starts = [0] + [rd(index_off + 16 * n_chunks + 4 * ((S - 1) * c + j), 4) for j in range(S - 1)] + [total]
        for st in range(S):
            e = sum((b[po + l // 2] >> (4 * (l % 2))) & 15 for l in range(st * lanes_per, (st + 1) * lanes_per))
            state += 16 * lanes_per + e
            words += 16 * (starts[st + 1] - starts[st] - -(-(16 * lanes_per + e) // 16))
    assert sz["state_bits"] == state and sz["word_bits"] == words
    assert 0 <= sz["pad_bits"] < 8 * 16 * (2 * n_chunks + 1) + 16 * S * n_chunks


def test_fixed_gemm_workspace_size_and_checks_before_launch():
    """The split product's workspace: the second half's partial sums (batch x
    rows fp32), asked for only where the product has at least 8 batch rows
    and two panels; a workspace too small or misaligned is refused before any
    launch."""
    import ctypes as C
    ws = L.lib().bs_fixed_gemm_work_bytes
    assert ws(4096, 4096, 64) == 4 * 64 * 4096
    assert ws(1000, 14336, 17) == 4 * 17 * 1000
    assert ws(20, 8192, 40) == 4 * 40 * 20
    assert ws(4096, 4096, 8) == 4 * 8 * 4096
    for rows, cols, batch in [(4096, 4096, 7), (4096, 2048, 64), (4096, 4096, 65), (0, 4096, 64), (64, 3000, 64)]:
        assert ws(rows, cols, batch) == 0, (rows, cols, batch)
    w = _words(np.random.default_rng(7).standard_normal(32 * 4096) * 0.02)
    info = codec.fixed_info(codec.fixed_encode(w))
    f = L.lib().bs_fixed_gemm_async
    call = lambda wp, wb: f(C.byref(info), C.c_void_p(4096), 32, 4096, 40, C.c_void_p(4096), C.c_void_p(8192), None,
                            C.c_void_p(wp), C.c_uint64(wb), None)
    need = 4 * 40 * 32
    assert call(1 << 20, need - 1) == L.BS_E_INVAL
    assert b"needed" in L.lib().bs_last_error()
    assert call((1 << 20) + 128, need) == L.BS_E_INVAL
    assert b"aligned" in L.lib().bs_last_error()
    assert call(8192 - 256, need) == L.BS_E_INVAL            # Y is at 8192: the workspace would overlap it
    assert b"overlaps" in L.lib().bs_last_error()


def test_fixed_decode_many_argument_checks_before_launch():
    import ctypes as C
    w = _words(np.random.default_rng(6).standard_normal(5000) * 0.02)
    info = codec.fixed_info(codec.fixed_encode(w))
    empty = codec.fixed_info(codec.fixed_encode(np.zeros(0, np.uint16)))
    f = L.lib().bs_fixed_decode_many_async

    def call(infos, blobs, outs, caps, count=None):
        k = len(infos)
        ia = (L.FixedInfo * max(k, 1))(*infos)
        ba = (C.c_void_p * max(k, 1))(*blobs)
        oa = (C.c_void_p * max(k, 1))(*outs)
        ca = (C.c_uint64 * max(k, 1))(*caps)
        return f(ia, ba, oa, ca, None, k if count is None else count, None)

    assert call([], [], [], []) == L.BS_OK                                        # nothing to do
    assert call([empty, empty], [4096, 8192], [None, None], [0, 0]) == L.BS_OK
    assert call([info], [4096], [4096], [10000], count=L.FIXED_MANY_MAX + 1) == L.BS_E_INVAL
    assert f(None, None, None, None, None, 1, None) == L.BS_E_INVAL
    assert call([empty, info], [4096, 4100], [4096, 8192], [0, 10000]) == L.BS_E_INVAL   # blob alignment
    assert call([info, info], [4096, 8192], [4096, 8200], [10000, 10000]) == L.BS_E_INVAL  # output alignment
    assert call([info, info], [4096, 8192], [4096, None], [10000, 10000]) == L.BS_E_INVAL  # NULL output
    assert call([info, info], [4096, 8192], [4096, 8192], [10000, 9999]) == L.BS_E_NOSPACE
    forged = L.FixedInfo.from_buffer_copy(info)
    forged.esc_off += 4
    assert call([info, forged], [4096, 8192], [4096, 8192], [10000, 10000]) == L.BS_E_INVAL


def test_streamer_argument_checks_before_any_device_call():
    import ctypes as C
    f = L.lib().bs_streamer_create
    out = C.c_void_p()
    assert f(None, None, 0, 1 << 30, None, C.byref(out)) == L.BS_E_INVAL
    c = codec.encode([codec.bf16(_words(np.random.default_rng(1).standard_normal(5000) * 0.02))],
                     codec.params(chunk_weights=4096, lanes=8))
    bad = bytearray(c)
    bad[0] ^= 0xFF
    ptrs = (C.c_void_p * 1)(C.cast(C.c_char_p(bytes(bad)), C.c_void_p))
    lens = (C.c_uint64 * 1)(len(bad))
    assert f(ptrs, lens, 1, 1 << 30, None, C.byref(out)) == L.BS_E_FORMAT
    ptrs = (C.c_void_p * 1)(C.cast(C.c_char_p(c), C.c_void_p))
    lens = (C.c_uint64 * 1)(len(c))
    assert f(ptrs, lens, 1, 1000, None, C.byref(out)) == L.BS_E_INVAL           # budget below two slots
    assert L.lib().bs_streamer_acquire(None, 0, None, C.byref(out)) == L.BS_E_INVAL
    assert L.lib().bs_streamer_release(None, 0, None) == L.BS_E_INVAL
    assert L.lib().bs_plan_rebind(None, C.c_void_p(4096)) == L.BS_E_INVAL


def test_fixed_device_transcoder_argument_checks():
    import ctypes as C
    assert L.lib().bs_fixed_max_bytes(0) == 96
    assert L.lib().bs_fixed_max_bytes(2048) == -(-(96 + 2820 + 4096) // 16) * 16
    f = L.lib().bs_fixed_encode_device
    ln = C.c_uint64()
    assert f(C.c_void_p(4096), 10, C.c_void_p(8192), 1 << 20, None, None) == L.BS_E_INVAL          # no out_len
    assert f(C.c_void_p(4098), 10, C.c_void_p(8192), 1 << 20, C.byref(ln), None) == L.BS_E_INVAL  # misaligned
    assert f(None, 10, C.c_void_p(8192), 1 << 20, C.byref(ln), None) == L.BS_E_INVAL              # no words


# ------------------------------------------------------------------ layout 2
@pytest.mark.parametrize("seed,n,W,K,P,M_s", [(30, 100000, 4096, 8, 4, 11), (31, 33333, 65536, 128, 64, 12),
                                              (32, 8, 64, 1, 1, 11), (33, 0, 64, 2, 2, 11),
                                              (34, 300000, 131072, 2048, 64, 11), (35, 262144 * 2 + 5, 65536, 512, 256, 11),
                                              (36, 5000, 65536, 256, 256, 12), (37, 70001, 65536, 128, 128, 11)])
def test_layout2_encoder_bytes_match_oracle(seed, n, W, K, P, M_s):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n) * rng.choice([0.004, 0.02, 0.1])
    x[rng.random(n) < 0.01] = 0.0
    w = _words(x)
    a = O.encode([O.bf16(w)], W=W, K=K, M_s=M_s, M_f=16 - M_s, cmax=31, P=P, layout=2)
    b = codec.encode([codec.bf16(w)], codec.params2(chunk_weights=W, lanes=K, m_s=M_s, stream_lanes=P))
    assert a == b
    assert codec.container_info(b).version == 2 and codec.record_info(b, 0).layout == 2


def test_layout2_models_match_oracle():
    rng = np.random.default_rng(13)
    for scale in (0.003, 0.02, 0.3):
        x = rng.standard_normal(200000) * scale
        x[rng.random(x.size) < 0.02] = 0.0
        w = _words(x)
        for M_s, cmax in [(11, 31), (12, 31), (11, 3)]:
            t = codec.build_tables_host(w, codec.params2(m_s=M_s, max_tables=cmax)).get()
            cs, cf = O.histogram(w)
            assert t["layout"] == 2 and (t["q_s"] == O.normalise(cs, M_s)).all()
            route, nt, qh = O.select_htables(cs, cf, 16 - M_s, cmax)
            route = O.share_hroutes(cs, cf, qh[:nt], route, 16 - M_s)
            assert nt == t["n_tables"] and (route == t["route"]).all() and (qh[:nt] == t["q_h"]).all()


def test_layout2_mixed_records_and_raw():
    rng = np.random.default_rng(14)
    a = _words(rng.standard_normal(70000) * 0.02)
    b = np.full(5000, 0x3F80, np.uint16)
    raw = np.arange(999, dtype=np.uint8)
    o = O.encode([O.bf16(a), O.raw(raw), O.bf16(b)], W=65536, K=128, M_s=11, M_f=5, cmax=31, P=64, layout=2)
    l = codec.encode([codec.bf16(a), codec.raw(raw), codec.bf16(b)], codec.params2(lanes=128, stream_lanes=64))
    assert o == l


def test_layout2_params_rejected():
    w = np.zeros(100, np.uint16)
    for kw in [dict(m_s=10), dict(m_s=13), dict(max_tables=32)]:
        with pytest.raises(L.BSError) as e:
            codec.encode([codec.bf16(w)], codec.params2(**kw))
        assert e.value.rc == L.BS_E_INVAL
    for m_f in (4, 6):   # m_f must be 16 - m_s
        p = codec.params2(m_s=11)
        p.m_f = m_f
        with pytest.raises(L.BSError):
            codec.encode([codec.bf16(w)], p)
    p = codec.params2()
    p.layout = 3
    with pytest.raises(L.BSError):
        codec.encode([codec.bf16(w)], p)
    # a model built for one layout cannot encode the other
    t = codec.build_tables_host(_words(np.ones(64)), codec.params())
    with pytest.raises(L.BSError):
        codec.encode([codec.bf16(_words(np.ones(64)), t)], codec.params2())


def test_layout3_is_the_library_default():
    import ctypes
    p = L.Params()
    L.lib().bs_params_default(ctypes.byref(p))
    assert (p.layout, p.m_s, p.m_f, p.max_tables, p.lanes, p.chunk_weights) == (3, 11, 13, 31, 128, 65536)
    # the defaults encode as they are, and in layout 2 once m_f follows m_s
    w = _words(np.random.default_rng(2).standard_normal(70000) * 0.02)
    assert codec.container_info(codec.encode([codec.bf16(w)], p)).version == 3
    p.layout, p.m_f = 2, 16 - p.m_s
    assert codec.container_info(codec.encode([codec.bf16(w)], p)).version == 2


def test_noalloc_tables_refuses_bad_arguments_on_the_host():
    """bs_build_tables_noalloc checks its arguments before any device work
    (so this runs without a GPU): NULL tables, NULL words, and more words than
    its maximum are refused with BS_E_INVAL and a message."""
    p = codec.params2()
    into = codec.build_tables_host(np.zeros(0, np.uint16), p)
    fake = C.c_void_p(1 << 20)   # never dereferenced: every call below is refused first
    lib = L.lib()
    assert lib.bs_build_tables_noalloc(fake, 8, C.byref(p), None, None) == L.BS_E_INVAL
    assert lib.bs_build_tables_noalloc(None, 8, C.byref(p), None, into.handle) == L.BS_E_INVAL
    assert lib.bs_build_tables_noalloc(fake, L.NOALLOC_MAX_WEIGHTS + 1, C.byref(p), None, into.handle) == L.BS_E_INVAL
    assert b"maximum" in lib.bs_last_error()
    bad = codec.params2()
    bad.m_s = 13
    assert lib.bs_build_tables_noalloc(fake, 8, C.byref(bad), None, into.handle) == L.BS_E_INVAL
