"""Pins for the oracle's layout 3 (container version 3), no GPU.

Layout 3 codes, per weight of a lane's groups other than its last, the
(sign, exponent) symbol s and the fraction's high three bits h = f >> 4 as one
joint symbol t = 8 s + h with a per-tensor table of precision M_t = 13, one
coding step and one renormalisation check per weight.  As in layout 2 a
lane's last group codes s alone (precision M_s, its h values in the start
state) and the low four bits l = f & 15 sit verbatim in the chunk's plane.
The joint table is this container's own reading of the decoded symbol
selecting the fraction's distribution [Qwen3.8-27B-BF16-NVLC-Lossless card,
codec paragraph]: P(s, h) = P(s) P(h | s) with every s keeping its own h
distribution.  Reconstruction stays bit-identical [same card, metrics table:
per-codec verification].

Pins: an independent bit-insertion model of the chunk coder for power-of-two
tables (each coding step inserts the symbol's rank into the state); the
stored joint table against the normaliser applied to joint counts built here
from the words; the record header; round trips over edge shapes, precisions
and streams; corruption and format errors; the size bound.
"""
import hashlib
import struct

import numpy as np
import pytest
import torch

from oracle import entropy as E
from oracle import oracle as O

M_T = 13


def _body(c, rec=0):
    return int.from_bytes(c[64 + 96 * rec + 24: 64 + 96 * rec + 32], "little")


def _words(n, seed, std=0.02):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(max(n, 1), generator=g)[:n] * std
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _enc(tensors, **kw):
    return O.encode(tensors, layout=3, **{"M_s": 11, "M_f": M_T, **kw})


# ------------------------------------------------------------------ record header and tables
def _tables(c, rec=0):
    """(header fields, s list, q_s, joint q by t) of a layout-3 record."""
    b = c[_body(c, rec):]
    W, K, nch, M_s, M_f, nt, l2s, n_sym, layout = struct.unpack("<IIIBBBBII", b[:24])
    syms = [struct.unpack_from("<HH", b, 24 + 4 * k) for k in range(n_sym)]
    routes = list(b[24 + 4 * n_sym: 24 + 5 * n_sym])
    ft = (24 + 5 * n_sym + 3) // 4 * 4
    qt = np.zeros(512 * 8, np.int64)
    for k, (s, _) in enumerate(syms):
        qt[8 * s: 8 * s + 8] = struct.unpack_from("<8H", b, ft + 16 * k)
    return dict(W=W, K=K, chunks=nch, M_s=M_s, M_f=M_f, n_tables=nt, log2S=l2s, n_sym=n_sym, layout=layout,
                routes=routes), syms, qt


def test_header_and_version():
    w = _words(70000, 1)
    c = _enc([O.bf16(w)], W=65536, K=256, P=128)
    assert int.from_bytes(c[8:12], "little") == 3
    hd, syms, qt = _tables(c)
    assert hd["layout"] == 3 and hd["M_f"] == M_T and hd["M_s"] == 11 and hd["n_tables"] == 0
    assert hd["W"] == 65536 and hd["K"] == 256 and hd["log2S"] == 1 and hd["chunks"] == 2
    assert hd["routes"] == [0] * hd["n_sym"]
    # the s list is the occupied symbols in ascending order with q_s = normalise(counts, M_s)
    s = (w.astype(np.int64) >> 7)
    cs = np.bincount(s, minlength=512).astype(np.uint64)
    assert [x for x, _ in syms] == [int(v) for v in np.nonzero(cs)[0]]
    assert [q for _, q in syms] == [int(v) for v in O.normalise(cs, 11)[cs > 0]]


@pytest.mark.parametrize("seed,std", [(2, 0.02), (3, 0.004), (4, 0.3)])
def test_joint_table_is_the_normaliser_on_joint_counts(seed, std):
    w = _words(150000, seed, std)
    w[::97] = 0                                    # some exact zeros
    w[5::131] |= 0x8000                            # and sign flips
    c = _enc([O.bf16(w)], W=65536, K=128, P=64)
    _, _, qt = _tables(c)
    t = (w.astype(np.int64) >> 7) * 8 + ((w.astype(np.int64) >> 4) & 7)
    ct = np.bincount(t, minlength=4096).astype(np.uint64)
    want = O.normalise(ct, M_T)
    assert qt.sum() == 1 << M_T
    assert qt.tolist() == [int(v) for v in want]
    assert all(qt[ct > 0] >= 1) and all(qt[ct == 0] == 0)


# ------------------------------------------------------------------ bit-insertion model
def _stream_payloads(c, rec=0):
    """Per stream of the first chunk of a layout-3 record: (states, words)."""
    d = c[64 + 96 * rec: 64 + 96 * (rec + 1)]
    b = c[_body(c, rec):]
    W, K, nch, M_s, M_f, nt, l2s, n_sym, layout = struct.unpack("<IIIBBBBII", b[:24])
    assert layout == 3
    S = 1 << l2s
    P = K // S
    ft = (24 + 5 * n_sym + 3) // 4 * 4
    io = (ft + 16 * n_sym + 15) // 16 * 16
    po, total = struct.unpack("<QI", b[io: io + 12])
    stab = [0] + [int.from_bytes(b[io + 16 * nch + 4 * i: io + 16 * nch + 4 * i + 4], "little")
                  for i in range(S - 1)] + [total]
    n = int.from_bytes(d[8:16], "little")
    n_c = min(n, W)
    code = ((K + 1) // 2 + 15) // 16 * 16
    plane = (4 * ((n_c + 7) // 8) + 15) // 16 * 16
    area = po + code + plane
    res = []
    for st in range(S):
        u0, u1 = stab[st], stab[st + 1]
        raw = b[area + 2 * u0: area + 2 * u1]
        bits = int.from_bytes(raw, "little")
        states, off = [], 0
        for l in range(st * P, (st + 1) * P):
            e = (b[po + l // 2] >> (4 * (l % 2))) & 15
            states.append((1 << (16 + e)) | ((bits >> off) & ((1 << (16 + e)) - 1)))
            off += 16 + e
        mu = (off + 15) // 16
        ws = [int.from_bytes(raw[2 * i: 2 * i + 2], "little") for i in range(mu, u1 - u0)]
        res.append((states, ws))
    return res, K, P


def _insertion_streams(words, K, P):
    """Independent model of one chunk for power-of-two tables: 2^j occupied s
    with equal counts (q_s = 2^(11 - j) at M_s 11) and 2^k occupied t = 8 s + h
    with equal counts (q_t = 2^(13 - k)).  Coding t inserts its k-bit rank at
    bit 13 - k, coding s inserts its j-bit rank at bit 11 - j; a symbol of
    frequency q at precision M first flushes 16 bits if x >= q 2^(32 - M)."""
    s_occ = sorted(set(int(w) >> 7 for w in words))
    t_occ = sorted(set((int(w) >> 7) * 8 + ((int(w) >> 4) & 7) for w in words))
    j, k = (len(s_occ) - 1).bit_length(), (len(t_occ) - 1).bit_length()
    assert len(s_occ) == 1 << j and len(t_occ) == 1 << k
    rs = {s: i for i, s in enumerate(s_occ)}
    rt = {t: i for i, t in enumerate(t_occ)}
    n = len(words)
    groups = (n + 7) // 8
    T = (groups + K - 1) // K

    def ins(x, pos, bits, v):
        return ((x >> pos) << (pos + bits)) | (v << pos) | (x & ((1 << pos) - 1))

    def last_group(l):
        return l + K * ((groups - 1 - l) // K) if l < groups else None

    out = []
    for st in range(K // P):
        lanes = range(st * P, (st + 1) * P)
        x = {}
        for l in lanes:
            g = last_group(l)
            if g is None:
                x[l] = 1 << 16
                continue
            hs = [(int(words[i]) & 127) >> 4 for i in range(8 * g, min(8 * g + 8, n))]
            x[l] = (1 << max(16, 3 * len(hs))) + sum(v << (3 * i) for i, v in enumerate(hs))
        emitted = []
        for t in reversed(range(T)):
            for p in reversed(range(8)):
                for l in reversed(lanes):
                    i = 8 * (t * K + l) + p
                    if i >= n:
                        continue
                    w = int(words[i])
                    if i // 8 == last_group(l):
                        bits, M, rank = j, 11, rs[w >> 7]
                    else:
                        bits, M, rank = k, 13, rt[(w >> 7) * 8 + ((w >> 4) & 7)]
                    if x[l] >= 1 << (32 - bits):      # q 2^(32 - M) with q = 2^(M - bits)
                        emitted.append(x[l] & 0xFFFF)
                        x[l] >>= 16
                    x[l] = ins(x[l], M - bits, bits, rank)
        out.append(([x[l] for l in lanes], emitted[::-1]))
    return out


@pytest.mark.parametrize("j,k,n,K,P", [(1, 3, 1000, 8, 8), (2, 4, 4096, 16, 4), (0, 2, 800, 4, 2),
                                       (1, 1, 8 * 64 * 3 + 8, 64, 16), (2, 5, 64000, 64, 32), (0, 0, 96, 4, 4)])
def test_streams_equal_bit_insertion_model(j, k, n, K, P):
    # 2^j exponents, each with 2^(k-j) h values, every t equally often (n a
    # multiple of 2^k); the low bits are random
    assert k >= j and n % (1 << k) == 0
    rng = np.random.default_rng(1000 * j + 10 * k + n)
    per_s = 1 << (k - j)
    m = n >> k
    words = np.array([((100 + s) << 7) | ((3 * hh + 1) % 8 << 4) | int(rng.integers(16))
                      for s in range(1 << j) for hh in range(per_s) for _ in range(m)], np.uint16)
    rng.shuffle(words)
    c = _enc([O.bf16(words)], W=65536, K=K, P=P)
    got, K_rec, P_rec = _stream_payloads(c)
    want = _insertion_streams(words[:65536], K_rec, P_rec)
    assert got == want
    out, st = O.decode(c)
    assert st == [0] and np.frombuffer(out, np.uint16)[:n].tolist() == words.tolist()


# ------------------------------------------------------------------ round trips
def _rt(tensors, **kw):
    c = _enc(tensors, **kw)
    assert int.from_bytes(c[8:12], "little") == 3
    out, st = O.decode(c)
    assert all(s == 0 for s in st), st
    for i, t in enumerate(tensors):
        d = c[64 + 96 * i: 64 + 96 * (i + 1)]
        oo = int.from_bytes(d[16:24], "little")
        b = t.data.tobytes()
        assert out[oo: oo + len(b)] == b
        assert d[40:72] == hashlib.sha256(b).digest()
    return c


def test_every_bit_pattern_round_trips():
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(7)
    # more than 256 distinct s are stored verbatim: code each half of the s range
    for part in (w[(w >> 7) < 256], w[(w >> 7) >= 256]):
        rng.shuffle(part)
        for M_s in (11, 12):
            _rt([O.bf16(part)], W=32768, K=64, M_s=M_s, P=16)


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 63, 64, 65, 8 * 64 - 1, 8 * 64 + 1, 4096, 65535, 65536, 65537, 140000])
def test_edge_sizes(n):
    w = _words(n, n)
    for K, P in [(64, 64), (128, 32), (1, 1), (256, 128)]:
        _rt([O.bf16(w)], W=65536, K=K, P=P)


def test_streams_and_precisions():
    w = _words(200000, 3, 0.03)
    for M_s in (11, 12):
        for K, P, W in [(2048, 64, 131072), (512, 256, 65536), (256, 128, 65536), (512, 512, 65536)]:
            _rt([O.bf16(w)], W=W, K=K, M_s=M_s, P=P)


def test_mixed_records_and_zeros():
    a = _words(70000, 9)
    a[::7] = 0
    wb = np.full(5000, 0x3F80, np.uint16)
    raw = np.arange(999, dtype=np.uint8)
    _rt([O.bf16(a), O.raw(raw), O.bf16(wb), O.bf16(np.zeros(0, np.uint16))], W=65536, K=128, P=64)


def test_bad_parameters_rejected():
    w = np.full(100, 0x3F80, np.uint16)
    for kw in [dict(M_s=10), dict(M_s=13), dict(M_f=12), dict(M_f=5)]:
        with pytest.raises(O.OracleError):
            _enc([O.bf16(w)], **kw)


def test_corruption_and_format_errors():
    w = _words(40000, 5)
    c = _enc([O.bf16(w)], W=65536, K=64)
    ro = _body(c)
    bad = bytearray(c)
    bad[len(c) - 40] ^= 0x5A
    rc, out, st = O.decode_status(bytes(bad))
    assert st[0] != 0 or out[:2 * w.size] != w.tobytes()
    # layout 3 inside a version-2 container; layout word 4 or 0 in version 3
    for field, version in [(3, 2), (4, 3), (0, 3)]:
        bad = bytearray(c)
        bad[8:12] = version.to_bytes(4, "little")
        bad[ro + 20: ro + 24] = field.to_bytes(4, "little")
        rc, out, st = O.decode_status(bytes(bad))
        assert st[0] == -2, (field, version)
    # a joint table that does not sum to 2^13, and M_t other than 13
    n_sym = int.from_bytes(c[ro + 16: ro + 20], "little")
    ft = ro + (24 + 5 * n_sym + 3) // 4 * 4
    bad = bytearray(c)
    bad[ft] ^= 1
    assert O.decode_status(bytes(bad))[2][0] == -2
    bad = bytearray(c)
    bad[ro + 13] = 12
    assert O.decode_status(bytes(bad))[2][0] == -2
    # layout-2 and version-1 containers still decode
    for lay, kw in [(2, dict(M_s=11, M_f=5, cmax=31)), (1, {})]:
        c_old = O.encode([O.bf16(w)], W=65536, K=64, layout=lay, **kw)
        out, st = O.decode(c_old)
        assert st == [0] and out[:2 * w.size] == w.tobytes()


# ------------------------------------------------------------------ size
def test_size_within_one_percent_of_conditional_entropy():
    # N(0, 0.02) words, 256 lanes per chunk in streams of 128: the container
    # (tables, index, states, plane and streams included) stays within 1% of
    # H(S) + H(F | S) and above it
    w = _words(1 << 21, 11)
    hs, hf = E.conditional_entropy_bits(w)
    c = _enc([O.bf16(w)], W=65536, K=256, P=128)
    ro, rl = _body(c), int.from_bytes(c[64 + 32: 64 + 40], "little")
    bits = 8 * rl / w.size
    assert hs + hf < bits < 1.01 * (hs + hf)
