"""Pins for the oracle's fixed-width lane-stream form (no GPU).

The pages say only that the GPU runtime derives fixed-width, lane-oriented
streams from the canonical model once at initialisation, names them
Fixed7/Compact11 and gives their resident size (about 71% of raw BF16)
[Qwen3.8-27B-BF16-NVLC-Lossless card, runtime accounting table].  The layout
is this repository's own: an 11-bit code word per weight, a 4-bit code for
one of the tensor's 15 most frequent (sign, exponent) symbols (15 = escape,
the symbol then comes from the tensor's escape list) and the exact 7-bit
fraction; 64 lanes of 32 weights per 2048-weight block, code and fraction
planes interleaved by lane dword.  The pins:
  - two hand-built blobs whose bytes are written out below, field by field
    (fraction order, code nibbles, the table's tie rule, escapes in weight
    order, lane layout);
  - block escape offsets and sizes in closed form;
  - all 65536 BF16 patterns (every symbol equally frequent) and ragged
    random tensors round-trip, with the escape count recomputed from a numpy
    histogram;
  - corrupt headers and escape lists are rejected.
"""
import struct

import numpy as np
import pytest

from oracle import oracle as O

HDR, BLOCK_BYTES = 96, 2816
E_FORMAT, E_VERSION, E_NOSPACE, E_CORRUPT = -2, -3, -4, -7


def _header(n, n_blocks, esc_off, n_esc, table):
    h = b"BF16FIX1" + struct.pack("<IIQQQQ", 1, 0, n, n_blocks, esc_off, n_esc) + bytes(16)
    return h + struct.pack("<16H", *(list(table) + [0] * (16 - len(table))))


def test_hand_blob_three_weights():
    # 1.5 = 0x3FC0 (s 127, f 0x40); -2.75 = 0xC030 (s 384, f 0x30); 0x3F81 (s 127, f 1)
    words = np.array([0x3FC0, 0xC030, 0x3F81], np.uint16)
    blob = O.fixed_encode(words)
    block = bytearray(BLOCK_BYTES)
    block[0:4] = struct.pack("<I", 0x00000010)                 # lane 0 codes: 0, 1, 0
    # lane 0 fractions, 7 bits each from bit 0: 0x40 | 0x30 << 7 | 1 << 14
    block[1024:1028] = struct.pack("<I", 0x40 | 0x30 << 7 | 1 << 14)
    esc_off = HDR + BLOCK_BYTES + 4
    want = _header(3, 1, esc_off, 0, [127, 384]) + bytes(block) + struct.pack("<I", 0)
    want += bytes(-len(want) % 16)
    assert len(want) == 2928
    assert blob == want
    assert O.fixed_decode(blob).tolist() == words.tolist()


def test_hand_blob_escapes_and_lanes():
    # symbols 10, 20, ..., 170; 170 three times, the others twice: the table is
    # 170, then 10 .. 140 (equal counts, lower symbol first); 150 and 160 escape.
    seq = [170] + [10 * k for k in range(1, 17)] + [160 - 10 * t for t in range(16)] + [170, 170]
    assert len(seq) == 35
    words = np.array([s << 7 for s in seq], np.uint16)
    blob = O.fixed_encode(words)
    block = bytearray(BLOCK_BYTES)
    lane0 = [0x76543210, 0xFEDCBA98, 0xABCDEFFF, 0x23456789]   # weights 0-7, 8-15, 16-23, 24-31
    for k, v in enumerate(lane0):
        block[4 * 64 * k: 4 * 64 * k + 4] = struct.pack("<I", v)
    block[4:8] = struct.pack("<I", 0x00000001)                 # lane 1: 10, 170, 170
    esc_off = HDR + BLOCK_BYTES + 4
    table = [170] + [10 * k for k in range(1, 15)]
    want = _header(35, 1, esc_off, 4, table) + bytes(block) + struct.pack("<I", 0)
    want += struct.pack("<4H", 150, 160, 160, 150)             # weights 15, 16, 17, 18
    want += bytes(-len(want) % 16)
    assert blob == want
    assert O.fixed_decode(blob).tolist() == words.tolist()


@pytest.mark.parametrize("i", range(32))
def test_fraction_bit_position(i):
    # lane 5 of block 0: only its weight i has a nonzero fraction (1)
    words = np.full(2048, 0x3F80, np.uint16)
    words[32 * 5 + i] |= 1
    blob = np.frombuffer(O.fixed_encode(words), np.uint8)
    frac = blob[HDR + 1024: HDR + 2816].view("<u4").reshape(7, 64)
    bits = np.zeros((7, 64), np.uint32)
    bits[(7 * i) // 32, 5] = 1 << ((7 * i) % 32)
    assert (frac == bits).all()


def test_block_escape_offsets():
    s = (np.arange(2053) % 15) + 1
    s[[100, 700, 2000]] = [400, 401, 402]
    s[2048:] = [403, 1, 2, 404, 3]
    words = (s << 7).astype(np.uint16)
    blob = O.fixed_encode(words)
    n_esc = struct.unpack_from("<Q", blob, 40)[0]
    esc_off = struct.unpack_from("<Q", blob, 32)[0]
    assert n_esc == 5
    assert esc_off == HDR + 2 * BLOCK_BYTES + 8
    assert struct.unpack_from("<2I", blob, HDR + 2 * BLOCK_BYTES) == (0, 3)
    assert struct.unpack_from("<5H", blob, esc_off) == (400, 401, 402, 403, 404)
    assert O.fixed_decode(blob).tolist() == words.tolist()


@pytest.mark.parametrize("n", [0, 1, 2047, 2048, 2049, 3 * 2048 + 77])
def test_sizes(n):
    rng = np.random.default_rng(n)
    words = rng.integers(0, 1 << 16, n, dtype=np.uint16)
    blob = O.fixed_encode(words)
    nb = (n + 2047) // 2048
    n_esc = struct.unpack_from("<Q", blob, 40)[0]
    assert len(blob) == -(-(HDR + BLOCK_BYTES * nb + 4 * nb + 2 * n_esc) // 16) * 16
    assert O.fixed_decode(blob).tolist() == words.tolist()


def _escapes_by_histogram(words):
    s = words.astype(np.int64) >> 7
    counts = np.bincount(s, minlength=512)
    order = np.lexsort((np.arange(512), -counts))               # count descending, then symbol
    top = [int(v) for v in order[:15] if counts[v] > 0]
    return top, int(np.sum(~np.isin(s, top)))


def test_all_patterns_round_trip():
    words = np.arange(1 << 16, dtype=np.uint16)
    blob = O.fixed_encode(words)
    table = struct.unpack_from("<16H", blob, 64)
    assert list(table) == list(range(15)) + [0]                # all tied: the lowest symbols
    assert struct.unpack_from("<Q", blob, 40)[0] == 65536 - 15 * 128
    assert (O.fixed_decode(blob) == words).all()


@pytest.mark.parametrize("n,scale", [(70001, 0.02), (4096, 1.0), (123457, 1e-3)])
def test_gaussian_round_trip(n, scale):
    import torch
    rng = np.random.default_rng(n)
    x = torch.from_numpy(rng.standard_normal(n).astype(np.float32) * scale)
    words = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    blob = O.fixed_encode(words)
    top, n_esc = _escapes_by_histogram(words)
    assert list(struct.unpack_from("<15H", blob, 64))[: len(top)] == top
    assert struct.unpack_from("<Q", blob, 40)[0] == n_esc
    assert (O.fixed_decode(blob) == words).all()


def _corrupt(blob, off, fmt, value):
    b = bytearray(blob)
    struct.pack_into(fmt, b, off, value)
    return bytes(b)


def test_rejects_corrupt_blobs():
    s = (np.arange(5000) % 15) + 1
    s[[10, 3000, 4999]] = [300, 301, 302]
    blob = O.fixed_encode((s << 7).astype(np.uint16))
    esc_off = struct.unpack_from("<Q", blob, 32)[0]
    cases = [
        (bytes(b"BF16FIX2") + blob[8:], E_FORMAT),
        (_corrupt(blob, 8, "<I", 2), E_VERSION),
        (_corrupt(blob, 24, "<Q", 2), E_FORMAT),          # n_blocks != ceil(n / 2048)
        (_corrupt(blob, 32, "<Q", esc_off + 2), E_FORMAT),
        (_corrupt(blob, 40, "<Q", 2), E_CORRUPT),         # fewer escapes than codes 15
        (_corrupt(blob, 40, "<Q", 4), E_CORRUPT),         # one escape never used
        (_corrupt(blob, HDR + 3 * BLOCK_BYTES + 4, "<I", 2), E_CORRUPT),  # block 1's first
        (_corrupt(blob, esc_off, "<H", 512), E_CORRUPT),  # not a symbol
    ]
    for i, (bad, rc) in enumerate(cases):
        with pytest.raises(O.OracleError) as e:
            O.fixed_decode(bad)
        assert e.value.rc == rc, i
    with pytest.raises(O.OracleError) as e:
        O.fixed_decode(blob, cap=4999)
    assert e.value.rc == E_NOSPACE
