"""Pins for the oracle's shared routing of layout-2 records (no GPU).

The pages route the fraction of each weight to a distribution chosen by the
decoded (sign, exponent) symbol and call it a soft-routed fraction
distribution [Qwen3.8-27B-BF16-NVLC-Lossless card, codec paragraph].  The
container reads "shared" as: after the coded h tables are chosen (one per
exponent that earns it), every occupied exponent without a table of its own
is routed to the table -- flat or coded -- that codes its merged h counts in
the fewest bits, counted as sum of m[h] (65536 M_h - L(q[h])) with
L(q) = floor(65536 log2 q).  A table with q = 0 for an h the exponent uses
cannot take it; ties go to the lower table id, so the flat table (id 0)
keeps an exponent unless a coded one is strictly cheaper.  Both signs of an
exponent follow.  The decoder reads route bytes as before.

Pins: hand cases with the costs worked out here (a routed exponent, an
unusable table, ties between coded tables and with the flat one, selected
exponents untouched), an independent Python statement of the rule on random
histograms, and a container whose route bytes and round trip are checked.
"""
import decimal
import functools
import struct

import numpy as np
import pytest

from oracle import oracle as O

FLAT = {5: 4, 4: 2}   # flat q_h for M_h


@functools.lru_cache(maxsize=None)
def L(q: int) -> int:
    """floor(65536 log2 q), from decimal logarithms at 60 digits."""
    decimal.getcontext().prec = 60
    v = decimal.Decimal(q).ln() / decimal.Decimal(2).ln() * 65536
    return int(v.to_integral_value(rounding=decimal.ROUND_FLOOR))


def _hist(spec):
    """spec: {exponent: (positive h counts[8], negative h counts[8])}; each h
    count is put on fraction 16 h.  Returns cs[512], cf[512 * 128]."""
    cs = np.zeros(512, np.uint64)
    cf = np.zeros((512, 128), np.uint64)
    for e, (pos, neg) in spec.items():
        for sign, counts in ((0, pos), (1, neg)):
            s = 256 * sign + e
            for h, c in enumerate(counts):
                cf[s, 16 * h] += c
                cs[s] += c
    return cs, cf.reshape(-1)


def _routes(spec, M_h=5, cmax=31):
    cs, cf = _hist(spec)
    route, nt, qh = O.select_htables(cs, cf, M_h, cmax)
    return cs, O.share_hroutes(cs, cf, qh[:nt], route, M_h), nt, qh[:nt]


def _cost(m, q, M_h):
    if any(mh and qv == 0 for mh, qv in zip(m, q)):
        return None
    return sum(mh * (65536 * M_h - L(int(qv))) for mh, qv in zip(m, q) if mh)


Z = [0] * 8
BIG = [9000, 0, 0, 0, 0, 0, 0, 700]    # exponent 120: a table of its own, q = [30, 0, ..., 0, 2]


def test_rare_exponent_routed_to_a_coded_table():
    # exponent 100: 8 weights (6 with h = 0, 2 with h = 7, one of them
    # negative) -- too few to earn a table, cheaper under exponent 120's
    cs, route, nt, qh = _routes({120: (BIG, Z), 100: ([5, 0, 0, 0, 0, 0, 0, 2], [1, 0, 0, 0, 0, 0, 0, 0])})
    assert nt == 1 and list(qh[0]) == list(O.normalise(np.array(BIG, np.uint64), 5))
    assert list(qh[0]) == [30, 0, 0, 0, 0, 0, 0, 2]
    m = [6, 0, 0, 0, 0, 0, 0, 2]
    flat, coded = _cost(m, [4] * 8, 5), _cost(m, qh[0], 5)
    assert flat == 8 * (5 * 65536 - 2 * 65536)
    assert coded == 6 * (5 * 65536 - L(30)) + 2 * (5 * 65536 - 65536) < flat
    assert route[100] == 1 and route[356] == 1
    assert route[120] == 1 and route[376] == 0          # the unoccupied sign keeps 0


def test_table_with_a_zero_for_a_used_h_cannot_take_the_exponent():
    # exponent 101 uses h = 1, where exponent 120's table has q = 0: it stays
    # flat although its h = 0 weights alone would be far cheaper there
    cs, route, nt, qh = _routes({120: (BIG, Z), 101: ([5, 1, 0, 0, 0, 0, 0, 0], Z)})
    assert qh[0][1] == 0
    assert route[101] == 0
    # with the zero ignored the coded table would have looked cheaper
    assert 5 * (5 * 65536 - L(30)) + 1 * (5 * 65536) < 6 * 3 * 65536


def test_tie_between_coded_tables_goes_to_the_lower_id():
    # exponents 120 and 122 have the same counts, hence the same table
    cs, route, nt, qh = _routes({120: (BIG, Z), 122: (BIG, Z), 100: ([6, 0, 0, 0, 0, 0, 0, 2], Z)})
    assert nt == 2 and list(qh[0]) == list(qh[1])
    assert route[120] == 1 and route[122] == 2 and route[100] == 1


def test_tie_with_the_flat_table_keeps_flat():
    # exponent 130's table is [8, 4, 4, 4, 4, 4, 4, 0]: for an exponent that
    # uses only h = 1..6 it costs exactly what the flat table costs
    even = [3200, 1600, 1600, 1600, 1600, 1600, 1600, 0]
    cs, route, nt, qh = _routes({130: (even, Z), 99: ([0, 2, 3, 0, 0, 1, 0, 0], Z)})
    assert nt == 1 and list(qh[0]) == [8, 4, 4, 4, 4, 4, 4, 0]
    assert _cost([0, 2, 3, 0, 0, 1, 0, 0], qh[0], 5) == _cost([0, 2, 3, 0, 0, 1, 0, 0], [4] * 8, 5)
    assert route[99] == 0


def test_selected_exponents_keep_their_own_tables_and_empty_ones_stay_zero():
    spec = {120: (BIG, [10, 0, 0, 0, 0, 0, 0, 1]), 122: ([100, 9000, 0, 0, 0, 0, 0, 0], Z),
            100: ([1, 0, 0, 0, 0, 0, 0, 0], Z)}
    cs, route, nt, qh = _routes(spec)
    assert nt == 2
    assert route[120] == 1 and route[376] == 1 and route[122] == 2
    assert route[100] == 1                                     # h = 0 is cheapest under table 1
    assert all(route[s] == 0 for s in range(512) if not cs[s])


def _rule(cs, cf, route, qh, M_h):
    """The routing rule restated in Python with exact integers."""
    cf = cf.reshape(512, 128)
    out = route.copy()
    for e in range(256):
        if cs[e] + cs[256 + e] == 0 or (cs[e] and route[e]) or (cs[256 + e] and route[256 + e]):
            continue
        m = [int(cf[e, 16 * h:16 * h + 16].sum() + cf[256 + e, 16 * h:16 * h + 16].sum()) for h in range(8)]
        tables = [[FLAT[M_h]] * 8] + [list(q) for q in qh]
        best, best_cost = 0, None
        for t, q in enumerate(tables):
            c = _cost(m, q, M_h)
            if c is not None and (best_cost is None or c < best_cost):
                best, best_cost = t, c
        for s in (e, 256 + e):
            if cs[s]:
                out[s] = best
    return out


def _random_case(seed):
    """Random histograms: returns (routes from the oracle, routes by the
    restated rule, routes before sharing)."""
    rng = np.random.default_rng(seed)
    M_h = 5 if seed % 3 else 4
    spec = {}
    for e in rng.choice(np.arange(90, 140), size=int(rng.integers(8, 40)), replace=False):
        n = int(rng.choice([3, 20, 300, 5000, 200000]))
        p = rng.dirichlet(np.full(8, float(rng.choice([0.3, 1.0, 20.0]))))
        pos = rng.multinomial(n, p)
        neg = rng.multinomial(int(rng.integers(0, n + 1)), p) if rng.random() < 0.7 else np.zeros(8, int)
        spec[int(e)] = (list(pos), list(neg))
    cs, cf = _hist(spec)
    route, nt, qh = O.select_htables(cs, cf, M_h, int(rng.choice([2, 5, 31])))
    return O.share_hroutes(cs, cf, qh[:nt], route, M_h), _rule(cs, cf, route, qh[:nt], M_h), route


@pytest.mark.parametrize("seed", range(12))
def test_rule_restated_on_random_histograms(seed):
    got, want, _ = _random_case(seed)
    assert np.array_equal(got, want)


def test_some_random_cases_are_rerouted():
    moved = 0
    for seed in range(12):
        got, _, before = _random_case(seed)
        moved += int((got != before).sum())
    assert moved > 0


def _route_bytes(container: bytes):
    """The first record's (s, route) pairs, read from the container bytes."""
    rec_off = struct.unpack_from("<Q", container, 64 + 24)[0]
    n_sym = struct.unpack_from("<I", container, rec_off + 16)[0]
    syms = [struct.unpack_from("<HH", container, rec_off + 24 + 4 * k)[0] for k in range(n_sym)]
    return {s: container[rec_off + 24 + 4 * n_sym + k] for k, s in enumerate(syms)}


def test_container_carries_shared_routes_and_round_trips():
    spec = {120: (BIG, [50, 0, 0, 0, 0, 0, 0, 4]), 100: ([5, 0, 0, 0, 0, 0, 0, 2], [1, 0, 0, 0, 0, 0, 0, 0]),
            101: ([5, 1, 0, 0, 0, 0, 0, 0], Z)}
    words = []
    rng = np.random.default_rng(3)
    for e, (pos, neg) in spec.items():
        for sign, counts in ((0, pos), (1, neg)):
            for h, c in enumerate(counts):
                # the low four fraction bits vary: only h is routed
                words += [(sign << 15) | (e << 7) | (h << 4) | int(rng.integers(16)) for _ in range(c)]
    w = np.array(words, np.uint16)
    rng.shuffle(w)
    c = O.encode([O.bf16(w)], W=4096, K=4, M_s=11, M_f=5, cmax=31, P=4, layout=2)
    r = _route_bytes(c)
    assert r[120] == 1 and r[376] == 1 and r[100] == 1 and r[356] == 1 and r[101] == 0
    out, st = O.decode(c)
    assert st == [0] and np.array_equal(np.frombuffer(out, np.uint16)[: w.size], w)
