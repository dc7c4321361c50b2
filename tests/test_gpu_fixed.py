"""GPU parity: the fixed-width lane-stream decode against the oracle.

The form is the runtime's second device format [NVLC card, runtime
paragraphs: fixed-width, lane-oriented streams derived once from the
canonical model]; decoding it must give back every BF16 word bit for bit.
Every blob here is built by the library's host transcoder, checked byte for
byte against the oracle's encoder, and every GPU output is compared with the
oracle's decode of the same blob.  All calls go through the C ABI
(bs_fixed_info_get, bs_fixed_decode_async, bs_fixed_decode_many_async,
bs_fixed_gemv_async, bs_fixed_gemm_async, bs_fixed_encode_device).
"""
import struct
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from lossless_entropy_coding_amd import _lib as L
from lossless_entropy_coding_amd import codec, synth

pytestmark = pytest.mark.gpu

HDR, BLOCK_BYTES = 96, 2816


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def _bf16(x) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _case_words(name, n, seed):
    rng = np.random.default_rng(seed)
    if name.startswith("gauss"):
        w = rng.standard_normal(n) * 0.02
        w[rng.random(n) < 0.001] *= 100.0
        return _bf16(w)
    if name.startswith("uniform"):                       # every symbol: almost all escapes
        return rng.integers(0, 1 << 16, n, dtype=np.uint16)
    if name.startswith("wide"):                          # a wide exponent spread: many escapes per block
        return _bf16(rng.standard_normal(n) * np.exp(rng.standard_normal(n) * 4))
    if name.startswith("patterns"):
        return np.arange(1 << 16, dtype=np.uint16)
    if name.startswith("zeros"):
        return np.zeros(n, np.uint16)
    raise ValueError(name)


CASES = [
    ("gauss_1", 1), ("gauss_3", 3), ("gauss_63", 63), ("gauss_2047", 2047), ("gauss_2048", 2048),
    ("gauss_2049", 2049), ("gauss_ragged", 70001), ("gauss_many_blocks", 64 * 2048 * 5 + 1234),
    ("uniform_ragged", 3 * 2048 + 77), ("wide_ragged", 41 * 2048 + 5), ("patterns", 65536), ("zeros", 10000),
]


def _run(words):
    blob = codec.fixed_encode(words)
    assert blob == O.fixed_encode(words)                 # host transcoder = the oracle's encoder
    expect = O.fixed_decode(blob)
    assert (expect == words).all()
    plan = codec.FixedPlan(blob)
    out = plan.decode()
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    return plan, blob, expect, got


@pytest.mark.parametrize("name,n", CASES, ids=[c[0] for c in CASES])
def test_fixed_decode_matches_oracle(name, n):
    say("fixed case", name, n)
    words = _case_words(name, n, n)
    plan, blob, expect, got = _run(words)
    assert got.size == expect.size
    bad = np.flatnonzero(got != expect)
    assert bad.size == 0, (bad[:8], got[bad[:8]], expect[bad[:8]])
    assert (plan.block_status() == 0).all()


def test_fixed_decode_4096x4096_workload():
    # the 4096 x 4096 matrix workload at full size (16.8M weights, 8192 blocks)
    wl = synth.cfg2("cpu")
    words = synth.as_words(wl.items[0].tensor).numpy().view(np.uint16).reshape(-1)
    say("fixed 4096x4096", words.size)
    plan, blob, expect, got = _run(words)
    assert (got == expect).all()
    assert (plan.block_status() == 0).all()
    # a second decode into a dirty buffer, with no status array
    out = torch.full((words.size,), -1, dtype=torch.int16, device="cuda")
    plan.decode_into(out, status=False)
    torch.cuda.synchronize()
    assert (out.cpu().numpy().view(np.uint16) == expect).all()


def test_fixed_writes_nothing_past_n():
    words = _case_words("gauss", 2048 + 100, 5)
    blob = codec.fixed_encode(words)
    plan = codec.FixedPlan(blob)
    out = torch.full((4096,), 0x5A5A, dtype=torch.int16, device="cuda")
    plan.decode_into(out)
    torch.cuda.synchronize()
    h = out.cpu().numpy().view(np.uint16)
    assert (h[: words.size] == O.fixed_decode(blob)).all()
    assert (h[words.size:] == 0x5A5A).all()


MANY_SETS = {
    # every case above in one launch (blobs from 1 weight to 655K), plus an empty one
    "all_cases": [(nm, n) for nm, n in CASES] + [("zeros_empty", 0)],
    # the most a call takes, all ragged: workgroups split 16 ways
    "sixteen_ragged": [("gauss", 2048 * (3 * i + 1) + 7 * i + 1) for i in range(16)],
    # one large tensor beside tiny ones: the tiny ones still get a workgroup
    "skewed": [("gauss", 1), ("gauss", 2048 * 400 + 3), ("uniform", 5), ("wide", 2049)],
}


@pytest.mark.parametrize("set_name", list(MANY_SETS))
def test_fixed_decode_many_matches_oracle(set_name):
    say("fixed many", set_name)
    plans, outs, expects, guards = [], [], [], []
    for i, (nm, n) in enumerate(MANY_SETS[set_name]):
        words = _case_words(nm, n, 1000 + i)
        blob = codec.fixed_encode(words)
        expect = O.fixed_decode(blob)
        assert (expect == words).all()
        plans.append(codec.FixedPlan(blob))
        # 4 KiB of guard words past each output: nothing may be written there
        outs.append(torch.full((n + 2048,), 0x5A5A, dtype=torch.int16, device="cuda"))
        expects.append(expect)
    codec.fixed_decode_many(plans, outs)
    torch.cuda.synchronize()
    for plan, out, expect in zip(plans, outs, expects):
        h = out.cpu().numpy().view(np.uint16)
        bad = np.flatnonzero(h[: expect.size] != expect)
        assert bad.size == 0, (expect.size, bad[:8])
        assert (h[expect.size:] == 0x5A5A).all()
        assert (plan.block_status() == 0).all()
    # the same launch again into dirty buffers, no status: the same words
    for out in outs:
        out.fill_(-1)
    codec.fixed_decode_many(plans, outs, status=False)
    torch.cuda.synchronize()
    for out, expect in zip(outs, expects):
        assert (out.cpu().numpy().view(np.uint16)[: expect.size] == expect).all()


def test_fixed_decode_many_full_layer():
    # the Gemma-2-9B-shaped layer at full size (7 matrices, 198M weights) in
    # one launch, the configuration the fixed-width bench times: every word
    # against the source tensors, and the oracle's decode of one whole blob
    wl = synth.cfg3("cpu")
    words = [synth.as_words(it.tensor).numpy().view(np.uint16) for it in wl.items if it.kind == "bf16"]
    say("fixed many, full layer", [w.size for w in words])
    blobs = [codec.fixed_encode(w) for w in words]
    k = min(range(len(words)), key=lambda i: words[i].size)
    assert (O.fixed_decode(blobs[k]) == words[k]).all()
    plans = [codec.FixedPlan(b) for b in blobs]
    outs = [torch.empty(w.size, dtype=torch.int16, device="cuda") for w in words]
    codec.fixed_decode_many(plans, outs)
    torch.cuda.synchronize()
    for w, o, p in zip(words, outs, plans):
        assert torch.equal(o, torch.from_numpy(w.view(np.int16)).cuda())
        assert (p.block_status() == 0).all()


def test_fixed_decode_many_reports_a_corrupt_blob():
    # the status words of a corrupted blob flag its block; the others stay clean
    w0, w1 = _case_words("gauss", 3 * 2048, 1), _case_words("wide", 5 * 2048 + 9, 2)
    plans = [codec.FixedPlan(codec.fixed_encode(w0)), codec.FixedPlan(codec.fixed_encode(w1))]
    assert plans[1].info.n_esc > 0
    blob1 = codec.fixed_encode(w1)
    at = plans[1].info.esc_off - 4 * plans[1].info.n_blocks + 4 * 2   # block 2's first escape
    _corrupt_device(plans[1], at, "<I", struct.unpack_from("<I", blob1, at)[0] + 1)
    outs = [torch.empty(w.size, dtype=torch.int16, device="cuda") for w in (w0, w1)]
    codec.fixed_decode_many(plans, outs)
    torch.cuda.synchronize()
    assert (outs[0].cpu().numpy().view(np.uint16) == w0).all()
    assert (plans[0].block_status() == 0).all()
    st = plans[1].block_status()
    assert st[2] != 0


def _corrupt_device(plan, off, fmt, value):
    b = bytearray(plan.dev.cpu().numpy().tobytes())
    struct.pack_into(fmt, b, off, value)
    plan.dev.copy_(torch.frombuffer(b, dtype=torch.uint8))


def test_fixed_status_flags_corrupt_blocks():
    s = (np.arange(5 * 2048) % 15) + 1
    s[[10, 3000, 4999, 7000, 9000]] = [300, 301, 302, 303, 304]
    words = (s << 7).astype(np.uint16)
    blob = codec.fixed_encode(words)
    info = codec.fixed_info(blob)
    offs = HDR + BLOCK_BYTES * info.n_blocks
    assert struct.unpack_from("<5I", blob, offs) == (0, 1, 2, 3, 4)

    plan = codec.FixedPlan(blob)                             # block 1 starts one escape late
    _corrupt_device(plan, offs + 4, "<I", 2)
    plan.decode()
    torch.cuda.synchronize()
    assert plan.block_status().tolist() == [1, 1, 0, 0, 0]

    plan = codec.FixedPlan(blob)                             # offsets out of order
    _corrupt_device(plan, offs + 8, "<I", 0)
    plan.decode()
    torch.cuda.synchronize()
    assert plan.block_status().tolist() == [0, 3, 1, 0, 0]

    plan = codec.FixedPlan(blob)                             # block 4's escape is not a symbol
    _corrupt_device(plan, info.esc_off + 2 * 4, "<H", 600)
    out = plan.decode()
    torch.cuda.synchronize()
    assert plan.block_status().tolist() == [0, 0, 0, 0, 4]
    got = out.cpu().numpy().view(np.uint16)
    assert got[9000] == 0 and (np.delete(got, 9000) == np.delete(words, 9000)).all()


def test_fixed_argument_errors():
    words = _case_words("gauss", 5000, 9)
    blob = codec.fixed_encode(words)
    plan = codec.FixedPlan(blob)
    out = torch.empty(5000 + 16, dtype=torch.int16, device="cuda")
    with pytest.raises(L.BSError) as e:                      # misaligned output
        plan.decode_into(out[1:])
    assert e.value.rc == L.BS_E_INVAL
    with pytest.raises(L.BSError) as e:                      # too small
        plan.decode_into(out[:4999])
    assert e.value.rc == L.BS_E_NOSPACE
    plan.decode_into(out[:5000])
    torch.cuda.synchronize()
    assert (out[:5000].cpu().numpy().view(np.uint16) == words).all()


# --------------------------------------------------------------------------- fused product
def _as_f64(words: np.ndarray) -> np.ndarray:
    return (words.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


GEMV_CASES = [
    # (name, rows, cols): 4096 x 4096 (two blocks per row), ragged rows, blocks over two rows,
    # many rows per block, a single row, the smallest width, and row units of 8, 64 and 2 rows
    ("4096x4096", 4096, 4096), ("777x1024", 777, 1024), ("300x3584", 300, 3584), ("640x96", 640, 96),
    ("1x8192", 1, 8192), ("3x32", 3, 32), ("129x2080", 129, 2080), ("33x18944", 33, 18944),
    ("65x32", 65, 32), ("7x5120", 7, 5120),
]


@pytest.mark.parametrize("name,rows,cols", GEMV_CASES, ids=[c[0] for c in GEMV_CASES])
def test_fixed_gemv_matches_fp64_product_of_oracle_decode(name, rows, cols):
    """y = W x within the fp32 summation bound: along any path a product meets
    at most 32 roundings in its lane (16 dot2 steps), 6 in the wave sum, one
    per block of its row added to a wave's total (cols / 2048 + 2) and 3 where
    the four waves' totals are added, so the error of row r is at most
    (43 + cols / 2048) 2^-24 sum_c |W[r, c] x[c]|; the test allows twice that.
    A row is summed by one workgroup in a fixed order, so two runs agree bit
    for bit."""
    say("fixed gemv", name)
    rng = np.random.default_rng(rows * 31 + cols)
    w = rng.standard_normal(rows * cols) * 0.02
    w[rng.random(w.size) < 0.002] *= 80.0
    w[rng.random(w.size) < 0.01] = 0.0
    words = _bf16(w)
    blob = codec.fixed_encode(words)
    W64 = _as_f64(O.fixed_decode(blob)).reshape(rows, cols)
    xw = _bf16(rng.standard_normal(cols))
    x64 = _as_f64(xw)
    y_ref = W64 @ x64
    bound = 2 * (43 + cols / 2048) * 2.0 ** -24 * (np.abs(W64) @ np.abs(x64))
    plan = codec.FixedPlan(blob)
    x = torch.from_numpy(xw.view(np.int16).copy()).cuda()
    ys = []
    for rep in range(2):                     # y and the status words are rewritten each time
        y = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
        plan.gemv_into(y, x, rows, cols)
        torch.cuda.synchronize()
        assert (plan.block_status() == 0).all()
        ys.append(y.cpu().numpy())
        err = np.abs(ys[-1].astype(np.float64) - y_ref)
        assert np.all(err <= bound), (rep, float((err - bound).max()))
    assert ys[0].tobytes() == ys[1].tobytes()


def test_fixed_gemv_argument_errors():
    words = _case_words("gauss", 64 * 1024, 11)
    plan = codec.FixedPlan(codec.fixed_encode(words))
    x = torch.zeros(2048, dtype=torch.int16, device="cuda")
    for rows, cols in [(64, 1000), (100, 1024), (2048, 32 + 16), (0, 1024)]:
        with pytest.raises(L.BSError) as e:
            plan.gemv_into(torch.empty(max(rows, 1), dtype=torch.float32, device="cuda")[:rows],
                           torch.zeros(cols, dtype=torch.int16, device="cuda"), rows, cols)
        assert e.value.rc == L.BS_E_INVAL
    with pytest.raises(L.BSError) as e:                      # misaligned x
        plan.gemv_into(torch.empty(64, dtype=torch.float32, device="cuda"), x[1:1025], 64, 1024)
    assert e.value.rc == L.BS_E_INVAL
    y = plan.gemv(x[:1024], 64, 1024)
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0


# --------------------------------------------------------------------------- batched product (MFMA)
GEMM_CASES = [
    # (name, rows, cols, batch): one tile of 16 batch rows, two, four (and a ragged 3 -> 4), rows not a
    # multiple of 16, several column panels
    ("4096x4096_b16", 4096, 4096, 16), ("512x4096_b32", 512, 4096, 32), ("300x2048_b64", 300, 2048, 64),
    ("77x6144_b1", 77, 6144, 1), ("1000x14336_b8", 1000, 14336, 8), ("64x2048_b40", 64, 2048, 40),
]


# the split product (a workspace given): every case with at least two panels,
# and the bench's 4096x4096 shape at batch 64, 32-row groups with a ragged last
# group (1000, 77 and 20 rows), an odd number of panels (3, 7)
SPLIT_CASES = [c for c in GEMM_CASES if c[2] >= 4096] + [
    ("4096x4096_b64", 4096, 4096, 64), ("20x8192_b40", 20, 8192, 40), ("96x4096_b17", 96, 4096, 17),
]


def _split_work(rows, batch):
    """A workspace of the size bs.h gives for the split product, filled with
    NaN bit patterns (its contents must not matter)."""
    return torch.full((batch * rows,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)


CASES_BOTH = ([c + ("whole",) for c in GEMM_CASES] + [c + ("split",) for c in SPLIT_CASES]
              + [("4096x4096_b64", 4096, 4096, 64, "auto")])     # the plan's own workspace, as the bench runs it


@pytest.mark.parametrize("name,rows,cols,batch,form", CASES_BOTH, ids=[f"{c[0]}_{c[4]}" for c in CASES_BOTH])
def test_fixed_gemm_matches_fp64_product_of_oracle_decode(name, rows, cols, batch, form):
    """Y = X W^T within the fp32 summation bound.  The matrix cores add the
    exact BF16 products of a 32-column step into an fp32 accumulator (at most
    one rounding per addition: 32 per step, cols / 32 steps per wave), the
    waves' K slices are added in order (at most 15 more) and, in the split
    product, the two halves' sums once more, so an entry's error is at most
    (cols + 17) 2^-24 sum_c |W[r, c] X[b, c]|; the test allows twice that.
    Each entry is summed in one fixed order: two runs agree bit for bit (in
    the split product the second run finds the first run's sums in the
    workspace)."""
    say("fixed gemm", name, form)
    rng = np.random.default_rng(rows + cols + batch)
    w = rng.standard_normal(rows * cols) * 0.02
    w[rng.random(w.size) < 0.002] *= 80.0
    words = _bf16(w)
    blob = codec.fixed_encode(words)
    W64 = _as_f64(O.fixed_decode(blob)).reshape(rows, cols)
    xw = _bf16(rng.standard_normal(batch * cols)).reshape(batch, cols)
    X64 = _as_f64(xw)
    Y_ref = X64 @ W64.T
    bound = 2 * (cols + 17) * 2.0 ** -24 * (np.abs(X64) @ np.abs(W64).T)
    plan = codec.FixedPlan(blob)
    x = torch.from_numpy(xw.view(np.int16).copy()).cuda()
    work = {"split": lambda: _split_work(rows, batch), "whole": lambda: None, "auto": lambda: "auto"}[form]()
    ys = []
    for rep in range(2):
        y = torch.full((batch, rows), float("nan"), dtype=torch.float32, device="cuda")
        plan.gemm_into(y, x, rows, cols, work=work)
        torch.cuda.synchronize()
        assert (plan.block_status() == 0).all()
        ys.append(y.cpu().numpy())
        err = np.abs(ys[-1].astype(np.float64) - Y_ref)
        assert np.all(err <= bound), (rep, float((err - bound).max()))
    assert ys[0].tobytes() == ys[1].tobytes()


def test_fixed_gemm_argument_errors():
    words = _case_words("gauss", 64 * 2048, 12)
    plan = codec.FixedPlan(codec.fixed_encode(words))
    x = torch.zeros(4, 2048, dtype=torch.int16, device="cuda")
    y = torch.empty(4, 64, dtype=torch.float32, device="cuda")
    f = L.lib().bs_fixed_gemm_async
    import ctypes as C
    args = lambda rows, cols, batch, xp, wp=None, wb=0: (C.byref(plan.info), C.c_void_p(plan.dev.data_ptr()), rows,
                                                         cols, batch, C.c_void_p(xp), C.c_void_p(y.data_ptr()), None,
                                                         C.c_void_p(wp) if wp else None, C.c_uint64(wb), None)
    assert f(*args(128, 1024, 4, x.data_ptr())) == L.BS_E_INVAL          # cols not a multiple of 2048
    assert f(*args(32, 2048, 4, x.data_ptr())) == L.BS_E_INVAL           # rows * cols != n
    assert f(*args(64, 2048, 0, x.data_ptr())) == L.BS_E_INVAL           # batch 0
    assert f(*args(64, 2048, 65, x.data_ptr())) == L.BS_E_INVAL          # batch above 64
    assert f(*args(64, 2048, 4, x.data_ptr() + 2)) == L.BS_E_INVAL       # misaligned X
    assert f(*args(64, 2048, 4, x.data_ptr())) == L.BS_OK
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0
    # the split product's workspace: too small, misaligned; a blob of 32 x 4096
    plan2 = codec.FixedPlan(codec.fixed_encode(_case_words("gauss", 32 * 4096, 13)))
    x2 = torch.zeros(4, 4096, dtype=torch.int16, device="cuda")
    y2 = torch.full((4, 32), float("nan"), dtype=torch.float32, device="cuda")
    w2 = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    need = 4 * 4 * 32
    a2 = lambda wp, wb: (C.byref(plan2.info), C.c_void_p(plan2.dev.data_ptr()), 32, 4096, 4, C.c_void_p(x2.data_ptr()),
                         C.c_void_p(y2.data_ptr()), None, C.c_void_p(wp), C.c_uint64(wb), None)
    assert f(*a2(w2.data_ptr(), need - 4)) == L.BS_E_INVAL               # too small
    assert f(*a2(w2.data_ptr() + 16, need)) == L.BS_E_INVAL              # not 256-B aligned
    assert f(*a2(w2.data_ptr(), need)) == L.BS_OK
    torch.cuda.synchronize()
    assert float(y2.abs().max()) == 0.0


# --------------------------------------------------------------------------- built on the GPU
@pytest.mark.parametrize("name,n", CASES, ids=[c[0] for c in CASES])
def test_fixed_encode_device_equals_host_transcoder(name, n):
    """The blob built on the GPU from device words is the host transcoder's
    (and therefore the oracle's) byte for byte."""
    say("fixed device encode", name)
    words = _case_words(name, n, n)
    host = codec.fixed_encode(words)
    d = codec.fixed_encode_device(torch.from_numpy(words.view(np.int16).copy()).cuda())
    torch.cuda.synchronize()
    assert d.cpu().numpy().tobytes() == host
    plan = codec.FixedPlan(d)                      # a plan over the device blob itself
    out = plan.decode()
    torch.cuda.synchronize()
    assert (out.cpu().numpy().view(np.uint16) == words).all()


def test_fixed_encode_device_from_decoded_container():
    # derived from the canonical container: rANS decode on the GPU, then the fixed form on the GPU
    wl = synth.cfg2("cpu")
    words = synth.as_words(wl.items[0].tensor).numpy().view(np.uint16).reshape(-1)
    c = codec.encode([codec.bf16(words)], codec.params(chunk_weights=131072, lanes=2048, stream_lanes=64))
    dec = codec.Plan(c).decode()
    blob = codec.fixed_encode_device(dec[: 2 * words.size].view(torch.int16))
    torch.cuda.synchronize()
    assert blob.cpu().numpy().tobytes() == O.fixed_encode(words)


def test_fixed_encode_device_capacity():
    import ctypes as C
    words = torch.from_numpy(_case_words("uniform", 5000, 3).view(np.int16).copy()).cuda()
    need = len(codec.fixed_encode(words.cpu().numpy().view(np.uint16)))
    out = torch.empty(need, dtype=torch.uint8, device="cuda")
    ln = C.c_uint64()
    rc = L.lib().bs_fixed_encode_device(C.c_void_p(words.data_ptr()), 5000, C.c_void_p(out.data_ptr()), need - 16,
                                        C.byref(ln), None)
    assert rc == L.BS_E_NOSPACE and ln.value == need
    rc = L.lib().bs_fixed_encode_device(C.c_void_p(words.data_ptr()), 5000, C.c_void_p(out.data_ptr()), need,
                                        C.byref(ln), None)
    assert rc == L.BS_OK and ln.value == need
