"""bs_build_tables_noalloc, the model built with nothing allocated by the
library (its histogram counters in a fixed device array), against
bs_build_tables on the same words, through the C ABI: identical tables on two
calls in a row, the second on a smaller tensor (so counts left over from the
first call would show), in both record layouts, and against the host model.
"""
import ctypes as C
import sys

import numpy as np
import pytest
import torch

from lossless_entropy_coding_amd import _lib as L
from lossless_entropy_coding_amd import codec

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def _device_words(n: int, seed: int, scale: float) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal(n).astype(np.float32) * scale)
    x[torch.from_numpy(rng.random(n) < 0.01)] = 0.0
    return x.to(torch.bfloat16).view(torch.int16).to("cuda")


def _assert_same(a: dict, b: dict):
    assert a.keys() == b.keys()
    for k in a:
        if isinstance(a[k], np.ndarray):
            assert np.array_equal(a[k], b[k]), k
        else:
            assert a[k] == b[k], k


@pytest.mark.parametrize("layout", [2, 1])
def test_noalloc_tables_equal_build_tables_two_calls(layout):
    p = codec.params2(lanes=128) if layout == 2 else codec.params(m_s=12, m_f=10)
    # the object the calls write over: an empty model built once beforehand
    into = codec.build_tables_host(np.zeros(0, np.uint16), p)
    for n, seed, scale in ((3_000_017, 1 + layout, 0.02), (40_001, 7 + layout, 0.3)):
        say("noalloc tables, layout", layout, "n", n)
        w = _device_words(n, seed, scale)
        want = codec.build_tables(w, p).get()
        got = codec.build_tables_noalloc(w, into, p).get()
        torch.cuda.synchronize()
        assert got["n"] == n
        _assert_same(got, want)
        _assert_same(got, codec.build_tables_host(w.cpu().numpy().view(np.uint16), p).get())


def test_noalloc_empty_and_size_limit():
    say("noalloc tables, empty input and the size limit")
    p = codec.params2()
    into = codec.build_tables_host(np.zeros(0, np.uint16), p)
    w = _device_words(1000, 3, 0.02)
    codec.build_tables_noalloc(w, into, p)
    # an empty tensor replaces the model with the empty one
    rc = L.lib().bs_build_tables_noalloc(C.c_void_p(w.data_ptr()), 0, C.byref(p), C.c_void_p(0), into.handle)
    assert rc == L.BS_OK
    _assert_same(into.get(), codec.build_tables_host(np.zeros(0, np.uint16), p).get())
    # beyond the maximum: refused on the host before any device work
    rc = L.lib().bs_build_tables_noalloc(C.c_void_p(w.data_ptr()), L.NOALLOC_MAX_WEIGHTS + 1, C.byref(p),
                                         C.c_void_p(0), into.handle)
    assert rc == L.BS_E_INVAL
    assert b"maximum" in L.lib().bs_last_error()
