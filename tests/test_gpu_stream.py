"""GPU: layers streamed on demand under a device-memory budget.

A streamer keeps a model's layer containers in pinned host memory and decodes
a layer into one of a few device slots when it is acquired, reusing the least
recently used slot that is not acquired [Gemma 2 9B Instruct -- Lossless
Compressed card, "Low-VRAM streaming"].  Every decoded layer is compared
bit for bit with the oracle's decode of its container, and the hit, miss
and eviction counts with a plain LRU model of the same access sequence.  All
calls go through the C ABI (bs_streamer_*).
"""
import sys
from collections import OrderedDict

import numpy as np
import pytest
import torch

from oracle import oracle as O
from lossless_entropy_coding_amd import _lib as L
from lossless_entropy_coding_amd import codec

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def _bf16(x) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _layers(n, seed=0):
    containers, expect = [], []
    for i in range(n):
        rng = np.random.default_rng(seed + i)
        tensors = [codec.bf16(_bf16(rng.standard_normal(40000 + 997 * i) * 0.02)),
                   codec.bf16(_bf16(rng.standard_normal(20000) * 0.05)),
                   codec.raw(rng.integers(0, 256, 333 + i, dtype=np.uint8).tobytes())]
        c = codec.encode(tensors, codec.params(chunk_weights=16384, lanes=64))
        out, st = O.decode(c)
        assert all(v == 0 for v in st)
        ranges = []
        for r in range(3):
            ri = codec.record_info(c, r)
            ranges.append((ri.out_offset, ri.out_offset + (2 * ri.n if ri.kind == L.KIND_BF16 else ri.n)))
        containers.append(c)
        expect.append((np.frombuffer(out, np.uint8), ranges))
    return containers, expect


def _check(view: torch.Tensor, exp):
    ref, ranges = exp
    got = view.cpu().numpy()
    for a, b in ranges:
        assert (got[a:b] == ref[a:b]).all(), (a, b)


def _two_slot_budget(containers):
    probe = codec.Streamer(containers, 1 << 40)
    st = probe.stats()
    del probe
    return 2 * st["staging_bytes"] + 2 * st["slot_bytes"] + 4096


def test_lru_sequence_matches_model():
    containers, expect = _layers(5)
    s = codec.Streamer(containers, _two_slot_budget(containers))
    assert s.stats()["n_slots"] == 2
    model, hits, misses, evictions = OrderedDict(), 0, 0, 0
    for layer in [0, 1, 0, 2, 1, 3, 3, 0, 4, 4, 2, 0, 1]:
        say("stream layer", layer)
        v = s.acquire(layer)
        torch.cuda.synchronize()
        _check(v, expect[layer])
        s.release(layer)
        if layer in model:
            hits += 1
            model.move_to_end(layer)
        else:
            misses += 1
            if len(model) == 2:
                model.popitem(last=False)
                evictions += 1
            model[layer] = True
    st = s.stats()
    assert (st["hits"], st["misses"], st["evictions"]) == (hits, misses, evictions)
    assert st["h2d_bytes"] == sum(len(containers[i]) for i in [0, 1, 2, 1, 3, 0, 4, 2, 0, 1])


def test_prefetch_then_acquire_hits():
    containers, expect = _layers(4, seed=10)
    s = codec.Streamer(containers, _two_slot_budget(containers))
    torch.cuda.synchronize()
    for layer in range(4):
        s.prefetch(layer)                       # copy and decode start; nothing acquired
        v = s.acquire(layer)
        torch.cuda.synchronize()
        _check(v, expect[layer])
        s.release(layer)
    st = s.stats()
    assert st["misses"] == 4 and st["hits"] == 4


def test_all_slots_acquired_is_an_error():
    containers, expect = _layers(3, seed=20)
    s = codec.Streamer(containers, _two_slot_budget(containers))
    a = s.acquire(0)
    b = s.acquire(1)
    with pytest.raises(L.BSError) as e:
        s.acquire(2)
    assert e.value.rc == L.BS_E_NOSPACE
    torch.cuda.synchronize()
    _check(a, expect[0])
    _check(b, expect[1])
    s.release(0)
    c = s.acquire(2)                            # slot of layer 0 is reused
    torch.cuda.synchronize()
    _check(c, expect[2])
    _check(b, expect[1])
    s.release(1)
    s.release(2)
    with pytest.raises(L.BSError) as e:
        s.release(2)
    assert e.value.rc == L.BS_E_INVAL


def test_two_streams():
    containers, expect = _layers(3, seed=30)
    s = codec.Streamer(containers, _two_slot_budget(containers))
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    va = s.acquire(1, stream=sa)                # miss: decoded on sa
    vb = s.acquire(1, stream=sb)                # hit: sb waits for that decode
    with torch.cuda.stream(sb):
        copy_b = vb.clone()
    s.release(1, stream=sb)
    s.release(1, stream=sa)
    torch.cuda.synchronize()
    _check(copy_b, expect[1])
    _check(va, expect[1])
    # reuse of the slot waits for both releases
    for layer in (0, 2):
        v = s.acquire(layer, stream=sa)
        torch.cuda.synchronize()
        _check(v, expect[layer])
        s.release(layer, stream=sa)


def test_prefetched_slots_evicted_from_another_stream():
    # both slots hold layers decoded on sa and never acquired; each later
    # acquire on sb reuses one of them and must wait for sa's decode there
    containers, expect = _layers(4, seed=50)
    s = codec.Streamer(containers, _two_slot_budget(containers))
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    s.prefetch(0, stream=sa)
    s.prefetch(1, stream=sa)
    copies = {}
    for layer in (2, 3):
        v = s.acquire(layer, stream=sb)
        with torch.cuda.stream(sb):
            copies[layer] = v.clone()
        s.release(layer, stream=sb)
    torch.cuda.synchronize()
    for layer, c in copies.items():
        _check(c, expect[layer])
    st = s.stats()
    assert (st["misses"], st["evictions"]) == (4, 2)


def test_budget_and_argument_errors():
    containers, _ = _layers(2, seed=40)
    budget = _two_slot_budget(containers)
    with pytest.raises(L.BSError) as e:
        codec.Streamer(containers, budget - 8192)
    assert e.value.rc == L.BS_E_INVAL
    s = codec.Streamer(containers, budget)
    with pytest.raises(L.BSError) as e:
        s.acquire(2)
    assert e.value.rc == L.BS_E_INVAL
    bad = bytearray(containers[1])
    bad[0] ^= 0xFF
    with pytest.raises(L.BSError) as e:
        codec.Streamer([containers[0], bytes(bad)], budget)
    assert e.value.rc == L.BS_E_FORMAT
