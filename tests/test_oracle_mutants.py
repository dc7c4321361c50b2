"""Planted mistakes in the oracle must be caught by its pins (no GPU).

Each case copies oracle/bs_oracle.c, changes one expression the way a
plausible bug would (a dropped term, a wrong comparison, a reversed order),
compiles the copy with gcc into a temporary directory and runs the quick pin
tests against it in a child process.  The pins must fail for every mutant;
the unmodified oracle must pass the same selection.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "bs_oracle.c")
PINS = ["tests/test_oracle_coder.py", "tests/test_oracle_model.py", "tests/test_oracle_container.py",
        "tests/test_oracle_streams.py", "tests/test_oracle_fixed.py"]
SELECT = ["-m", "not slow", "-k", "not cfg1 and not cfg2 and not gaussian and not scale_invariance"]

MUTANTS = {
    "encode_drops_cum": ("*x = (*x / q) * (1u << t->M) + (*x % q) + cum;", "*x = (*x / q) * (1u << t->M) + (*x % q);"),
    "decode_drops_cum": ("*x = t->q[s] * (*x >> t->M) + slot - cum;", "*x = t->q[s] * (*x >> t->M) + slot;"),
    "flush_off_by_one": ("if ((uint64_t)*x >= x_max) {", "if ((uint64_t)*x > x_max) {"),
    "refill_off_by_one": ("if (*x < BSO_L) {\n        if (*pos >= nw)", "if (*x <= BSO_L) {\n        if (*pos >= nw)"),
    "chunk_lanes_ascending": ("for (int64_t l = (int64_t)l1 - 1; l >= (int64_t)l0; l--) {\n                    uint64_t j",
                              "for (int64_t l = (int64_t)l0; l < (int64_t)l1; l++) {\n                    uint64_t j"),
    "sched_lanes_ascending": ("for (int64_t l = (int64_t)K - 1; l >= 0 && !rc; l--) {",
                              "for (int64_t l = 0; l < (int64_t)K && !rc; l++) {"),
    "words_not_reversed": ("put16(area + 2 * (mu[st] + i), wls[st].w[wls[st].n - 1 - i]);",
                           "put16(area + 2 * (mu[st] + i), wls[st].w[i]);"),
    "state_units_floor": ("return (16ull * P + esum + 15) / 16;", "return (16ull * P + esum) / 16;"),
    "stream_table_off_by_one": ("if (st > 0) put32(b + stab_off + 4 * ((S - 1) * c + st - 1), (uint32_t)at);",
                                "if (st > 0) put32(b + stab_off + 4 * ((S - 1) * c + st - 1), (uint32_t)at + 1);"),
    "streams_swapped": ("states, &wls[st]);", "states, &wls[S - 1 - st]);"),
    "state_code_off_by_one": ("while (e < 15 && (x >> (17 + e)) != 0) e++;", "while (e < 15 && (x >> (16 + e)) != 0) e++;"),
    "state_nibbles_swapped": ("b[start + l / 2] |= (uint8_t)(state_code(states[l]) << (4 * (l % 2)));",
                              "b[start + l / 2] |= (uint8_t)(state_code(states[l]) << (4 * (1 - l % 2)));"),
    "state_bits_msb_first": ("if ((v >> i) & 1u) b[bit / 8] |= (uint8_t)(1u << (bit % 8));",
                             "if ((v >> i) & 1u) b[bit / 8] |= (uint8_t)(0x80u >> (bit % 8));"),
    "raw_fractions_not_in_state": ("for (uint32_t i = 0; i < m; i++) x |= bso_symbol_f(w[j0 + i]) << (7 * i);",
                                   "for (uint32_t i = 0; i < m; i++) x |= 0u;"),
    "raw_fractions_reversed": ("x |= bso_symbol_f(w[j0 + i]) << (7 * i);", "x |= bso_symbol_f(w[j0 + i]) << (7 * (m - 1 - i));"),
    "raw_fraction_read_shifted": ("((x[l] >> (7 * i)) & 0x7Fu)", "((x[l] >> (7 * i + 1)) & 0x7Fu)"),
    "raw_count_three": ("uint32_t m = c < 4 ? (uint32_t)c : 4u;", "uint32_t m = c < 3 ? (uint32_t)c : 3u;"),
    "raw_lead_always_16": ("return 7 * m > 16 ? 7 * m : 16;", "return 16;"),
    "raw_in_first_group": ("uint64_t g = l + (uint64_t)K * ((groups - 1 - l) / K);   /* the lane's last group */",
                           "uint64_t g = l;"),
    "stream_lanes_overlap": ("rc = chunk_decode(md, st, words, nws, n_c, K, s * P, (s + 1) * P, out);",
                             "rc = chunk_decode(md, st, words, nws, n_c, K, s * P, (s + 1) * P + (s + 1 < S), out);"),
    "phase_order_swapped": ("for (int phase = 1; phase >= 0; phase--) {", "for (int phase = 0; phase <= 1; phase++) {"),
    "sign_in_wrong_place": ("return (uint16_t)((sign << 15) | (expo << 7) | f);", "return (uint16_t)((sign << 7) | (expo << 8) | f);"),
    "normalise_tie_high_index": ("(rem[ib] == rem[ibest] && ib < ibest)", "(rem[ib] == rem[ibest] && ib > ibest)"),
    "normalise_no_floor_one": ("q[i] = (uint32_t)(v < 1 ? 1 : v);", "q[i] = (uint32_t)v;"),
    "table_always_eligible": ("eligible[k] = (256 * E > n * n + (unsigned __int128)726784 * n);", "eligible[k] = 1;"),
    "signs_not_merged": ("unsigned __int128 m = (unsigned __int128)cf[e * 128 + f] + cf[(256 + e) * 128 + f];",
                         "unsigned __int128 m = cf[e * 128 + f];"),
    "fixed_table_tie_high": ("if (!used[s] && cs[s] && (best < 0 || cs[s] > cs[best])) best = s;",
                             "if (!used[s] && cs[s] && (best < 0 || cs[s] >= cs[best])) best = s;"),
    "fixed_sixteen_codes": ("while (m < 15) {", "while (m < 16) {"),
    "fixed_nibbles_swapped": ("cw[(i % 8) / 2] |= (uint8_t)(code << (4 * (i % 2)));",
                              "cw[(i % 8) / 2] |= (uint8_t)(code << (4 * (1 - i % 2)));"),
    "fixed_lane_major_codes": ("uint8_t* cw = base + 4 * (64 * (i / 8) + l);", "uint8_t* cw = base + 4 * (4 * l + i / 8);"),
    "fixed_fraction_msb_first": ("put_bits(frac, 7ull * i, f, 7);", "put_bits(frac, 7ull * (31 - i), f, 7);"),
    "fixed_no_escape_check": ("if (e != (blk + 1 < n_blocks ? get32(b + offs + 4 * (blk + 1)) : n_esc)) return BSO_ECORRUPT;",
                              "if (0) return BSO_ECORRUPT;"),
    "shape_rounding": ("*W = (uint32_t)round_up(n ? n : 1, 8 * (uint64_t)k);", "*W = (uint32_t)round_up(n ? n : 1, 8);"),
}


def _run_pins(lib_path):
    env = dict(os.environ)
    env["BSO_ORACLE_LIB"] = lib_path
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS, *SELECT],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def _build(src_text, tmp_path, name):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src_text)
    subprocess.check_call(["gcc", "-O1", "-std=gnu11", "-fPIC", "-shared", "-o", str(so), str(c)])
    return str(so)


def test_unmodified_oracle_passes_selection(tmp_path):
    so = _build(open(SRC).read(), tmp_path, "clean")
    rc, out = _run_pins(so)
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation anchor not found: {name}"
    so = _build(text.replace(old, new, 1), tmp_path, name)
    rc, out = _run_pins(so)
    assert rc != 0, f"planted mistake {name} was not caught:\n{out}"
