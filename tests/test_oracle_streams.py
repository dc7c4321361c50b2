"""Pins for chunks whose lanes are split into several word streams.

A chunk's K lanes form S = K/P streams of P consecutive lanes; each stream
keeps its own 16-bit word sequence, so the streams of one chunk can be
decoded independently.  This is part of the container's own layout (the
pages give no chunk layout).  The pins:
  - a hand-built two-stream container, derived field by field from the
    one-lane hand example;
  - every stream's states and words equal the explicit-schedule coder (a
    separate code path pinned by the worked examples) run on the schedule
    that the lane interleave defines, with the tables read from the record
    and each lane started from a state holding its last fractions;
  - round trips over ragged sizes and stream widths.
"""
import hashlib
import json
import os
import struct

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "container_16x_one_two_streams.json")


def _hand_two_streams():
    g = json.load(open(GOLD))
    words = np.array([int(h, 16) for h in g["weights_hex"]], np.uint16)
    body = bytearray()
    body += struct.pack("<IIIBBBBII", 16, 2, 1, 12, 10, 0, 1, 1, 0)  # W, K, chunks, M_s, M_f, tables, log2 S, n_sym, 0
    body += struct.pack("<HH", 127, 4096)                             # s-table
    body += bytes([0])                                                # route
    body += bytes(32 - len(body))                                     # pad to 32 (index offset)
    nw, units = g["n_words"], g["stream_units"]                      # per stream
    body += struct.pack("<QII", 64, 2 * units, 0)                     # chunk index: payload at 64, both streams' units
    body += struct.pack("<I", units) + bytes(12)                      # stream table: stream 1 starts at unit 4; pad
    x = g["final_state"]
    e = x.bit_length() - 17                                           # length code of both lanes
    assert e == 8
    body += bytes([e | e << 4]) + bytes(15)                           # two length codes + pad
    mant = x - (1 << (16 + e))
    mu = (16 + e + 15) // 16
    assert mu + nw == units
    for _ in range(2):                                                # stream 0, then stream 1
        body += mant.to_bytes(2 * mu, "little") + bytes(2 * nw)       # its lane's state bits, then its words
    assert len(body) == 96
    hdr = b"BF16RANS" + struct.pack("<IIQQQI", 1, 1, 64, 256, 32, 0) + bytes(20)
    d = struct.pack("<IIQQQQ", 1, 0, 16, 0, 160, 96) + hashlib.sha256(words.tobytes()).digest() + bytes(24)
    return words, g["params"], hdr + d + bytes(body)


def test_hand_built_two_stream_container_matches_encoder():
    words, p, expect = _hand_two_streams()
    got = O.encode([O.bf16(words)], W=p["W"], K=p["K"], P=p["P"], M_s=p["M_s"], M_f=p["M_f"], cmax=p["cmax"])
    assert got == expect


def test_hand_built_two_stream_container_decodes():
    words, p, c = _hand_two_streams()
    out, st = O.decode(c)
    assert st == [0]
    assert np.frombuffer(out, np.uint16).tolist() == words.tolist()
    assert O.decode_chunk(c, 0, 0).tolist() == words.tolist()


def _words(n, scale, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * scale).astype(np.float32)
    x[rng.random(n) < 0.02] = 0.0
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def _u(b, off, fmt):
    return struct.unpack_from("<" + fmt, b, off)[0]


def _record_model(c, i):
    """Read record i's shape and tables straight from the bytes."""
    d = 64 + 96 * i
    n, ro = _u(c, d + 8, "Q"), _u(c, d + 24, "Q")
    b = c[ro:]
    W, K, nch = _u(b, 0, "I"), _u(b, 4, "I"), _u(b, 8, "I")
    M_s, M_f, nt, log2S = b[12], b[13], b[14], b[15]
    n_sym = _u(b, 16, "I")
    qs = np.zeros(512, np.uint32)
    route = np.zeros(512, np.uint32)
    for k in range(n_sym):
        s, q = _u(b, 24 + 4 * k, "H"), _u(b, 26 + 4 * k, "H")
        qs[s] = q
        route[s] = b[24 + 4 * n_sym + k]
    ft = (24 + 5 * n_sym + 3) // 4 * 4
    qf = [np.full(128, 1 << (M_f - 7), np.uint32)]
    for t in range(nt):
        qf.append(np.frombuffer(b[ft + 256 * t: ft + 256 * (t + 1)], np.uint16).astype(np.uint32))
    index = (ft + 256 * nt + 15) // 16 * 16
    return dict(n=n, b=b, W=W, K=K, nch=nch, S=1 << log2S, qs=qs, route=route, qf=qf, M_s=M_s, M_f=M_f,
                index=index)


def _stream_schedule(w, n_c, K, lanes):
    """Symbols and table kinds of one stream, by sub-step: (t, p, phase) with
    phase 0 the (sign, exponent) symbol and 1 the fraction; idle = -1.  The
    lane's last group of c weights (its last macro-step) hands the fractions
    of its last min(4, c) weights to the start state: they are left out of
    the schedule and packed 7 bits each, first one lowest, under a leading
    one at bit max(16, 7m) (an empty lane starts at 2^16)."""
    groups = (n_c + 7) // 8
    T = (groups + K - 1) // K
    P = len(lanes)
    syms = np.full((T * 16, P), -1, np.int32)
    kind = np.zeros((T * 16, P), np.int32)     # 0 = s, 1 = f
    init = np.full(P, 1 << 16, np.uint32)
    raw = set()
    for i, l in enumerate(lanes):
        tl = [t for t in range(T) if 8 * (t * K + l) < n_c]
        if not tl:
            continue
        js = [8 * (tl[-1] * K + l) + p for p in range(8) if 8 * (tl[-1] * K + l) + p < n_c]
        mine = js[-min(4, len(js)):]
        x = 1 << max(16, 7 * len(mine))
        for k, j in enumerate(mine):
            x |= (int(w[j]) & 0x7F) << (7 * k)
            raw.add((i, j))
        init[i] = x
    for t in range(T):
        for p in range(8):
            for i, l in enumerate(lanes):
                j = 8 * (t * K + l) + p
                if j >= n_c:
                    continue
                syms[(t * 8 + p) * 2, i] = int(w[j]) >> 7
                if (i, j) not in raw:
                    syms[(t * 8 + p) * 2 + 1, i] = int(w[j]) & 0x7F
                kind[(t * 8 + p) * 2 + 1, i] = 1
    return syms, kind, init


@pytest.mark.parametrize("n,W,K,P", [(5000, 1024, 8, 8), (5000, 1024, 8, 2), (3005, 512, 16, 4),
                                     (4096 + 77, 4096, 64, 16), (777, 64, 1, 1), (20000, 8192, 32, 8)])
def test_stream_payload_equals_schedule_coder(n, W, K, P):
    w = _words(n, 0.03, n + K + P)
    c = O.encode([O.bf16(w)], W=W, K=K, P=P)
    m = _record_model(c, 0)
    b, K, S = m["b"], m["K"], m["S"]
    assert S == K // min(P, K)
    Ps = K // S
    tables = [O.Table(m["M_s"], m["qs"])] + [O.Table(m["M_f"], q) for q in m["qf"]]
    for ch in range(m["nch"]):
        n_c = min(m["W"], n - ch * m["W"])
        po, total = _u(b, m["index"] + 16 * ch, "Q"), _u(b, m["index"] + 16 * ch + 8, "I")
        stab = m["index"] + 16 * m["nch"] + 4 * (S - 1) * ch
        starts = [0] + [_u(b, stab + 4 * (s - 1), "I") for s in range(1, S)] + [total]
        cb = ((K + 1) // 2 + 15) // 16 * 16
        for s in range(S):
            area = po + cb + 2 * starts[s]
            units = starts[s + 1] - starts[s]
            lanes = list(range(s * Ps, (s + 1) * Ps))
            states, mu = _stream_states(b, po, area, lanes)
            stream = np.frombuffer(b[area + 2 * mu: area + 2 * units], np.uint16)
            syms, kind, init = _stream_schedule(w[ch * m["W"]:], n_c, K, lanes)
            tab_of = np.where(kind == 1, 1 + m["route"][np.clip(syms_prev(syms), 0, 511)], 0)
            st_ref, w_ref = O.sched_encode(Ps, syms, tab_of.astype(np.uint32), tables, init=init)
            assert np.array_equal(states, st_ref), (ch, s)
            assert np.array_equal(stream, w_ref), (ch, s)
        # the payload holds the codes and the stream area, padded to 16 bytes
        nxt = _u(b, m["index"] + 16 * (ch + 1), "Q") if ch + 1 < m["nch"] else len(b)
        assert nxt - po == (cb + 2 * total + 15) // 16 * 16


def _stream_states(b, po, area, lanes):
    """Final states of a stream's lanes: length codes from the chunk's nibble
    block (lane l in the low nibble of byte l/2 when l is even), state bits
    (16 + e per lane, least significant first, in lane order) from the head
    of the stream's area; and the 16-bit units those bits take."""
    codes = [(b[po + l // 2] >> (4 * (l % 2))) & 15 for l in lanes]
    mbits = 16 * len(lanes) + sum(codes)
    mu = (mbits + 15) // 16
    bits = int.from_bytes(b[area: area + 2 * mu], "little")
    states, off = [], 0
    for e in codes:
        states.append((1 << (16 + e)) | ((bits >> off) & ((1 << (16 + e)) - 1)))
        off += 16 + e
    return np.array(states, np.uint32), mu


def syms_prev(syms):
    """For every fraction cell, the (sign, exponent) symbol one sub-step
    earlier in the same lane (the symbol that routes it); other cells -1."""
    prev = np.full_like(syms, -1)
    prev[1::2] = syms[0::2]
    return prev


@pytest.mark.parametrize("P,K", [(1, 128), (2, 128), (8, 128), (64, 128), (128, 128), (512, 1024), (64, 2048),
                                 (512, 2048)])
def test_stream_roundtrip_ragged(P, K):
    W = 8 * K * 4
    rng = np.random.default_rng(P)
    for n in sorted({0, 1, 9, 8 * K - 1, 8 * K + 3, W - 1, W, W + 5, 3 * W + 11}):
        w = _words(n, float(rng.choice([0.003, 0.02, 0.1])), n + P)
        c = O.encode([O.bf16(w)], W=W, K=K, P=P)
        out, st = O.decode(c)
        assert st == [0]
        assert out[: 2 * n] == w.tobytes()


def test_bad_stream_widths_rejected():
    w = _words(100, 0.02, 0)
    for K, P in [(8, 3), (8, 16), (8, 0), (1024, 1024), (4096, 64)]:
        with pytest.raises(O.OracleError):
            O.encode([O.bf16(w)], W=64 * 8, K=K, P=P)


def test_stream_word_count_corruption_detected():
    w = _words(4096, 0.02, 3)
    c = bytearray(O.encode([O.bf16(w)], W=4096, K=8, P=2))
    m = _record_model(bytes(c), 0)
    ro = _u(c, 64 + 24, "Q")
    stab = ro + m["index"] + 16 * m["nch"]                 # stream table of chunk 0: start of stream 1
    a = _u(c, stab, "I")
    # move one word from stream 0 to stream 1: totals agree, streams do not
    struct.pack_into("<I", c, stab, a - 1)
    rc, out, st = O.decode_status(bytes(c))
    assert rc != 0 and st[0] != 0
