"""Planted mistakes in the oracle must be caught by its pins (no GPU).

Each case copies oracle/bs_oracle.c, changes one expression the way a
plausible bug would (a dropped term, a wrong comparison, a reversed order),
compiles the copy with gcc into a temporary directory and runs the quick pin
tests against it in a child process (the cases run concurrently, each in its
own process).  The pins must fail for every mutant; the unmodified oracle
must pass the same selection.
"""
import concurrent.futures as cf
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
    "normalise_over_sum_tie_high": ("if (q[i] > 1 && (best == A || q[i] > q[best])) best = i;",
                                    "if (q[i] > 1 && (best == A || q[i] >= q[best])) best = i;"),
    "context_score_tie_high": ("(score[k] == score[best] && cand[k] < cand[best])) best = (int)k;",
                               "(score[k] == score[best] && cand[k] > cand[best])) best = (int)k;"),
    "context_candidates_32": ("#define BSO_CANDIDATES 64u", "#define BSO_CANDIDATES 32u"),
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

# planted mistakes in layout 2 (one renormalisation per weight), checked
# against the layout-2 pins only
PINS2 = ["tests/test_oracle_layout2.py", "tests/test_oracle_shared_routing.py"]
MUTANTS2 = {
    "split_pair_order_swapped": ("    code_step(x, th, h);\n    code_step(x, ts, s);", "    code_step(x, ts, s);\n    code_step(x, th, h);"),
    "split_flush_bound_s_only": ("uint64_t q = (uint64_t)ts->q[s] * th->q[h];", "uint64_t q = (uint64_t)ts->q[s] * (1u << th->M) / 8;"),
    "split_lead_always_16": ("static uint32_t split_lead(uint32_t c) { return 3 * c > 16 ? 3 * c : 16; }",
                             "static uint32_t split_lead(uint32_t c) { return 16 + 0 * c; }"),
    "split_start_h_reversed": ("x |= (bso_symbol_f(w[8 * g + i]) >> 4) << (3 * i);", "x |= (bso_symbol_f(w[8 * g + i]) >> 4) << (3 * (c - 1 - i));"),
    "split_plane_even_odd_swapped": ("static uint32_t low_bit_pos(uint32_t p) { return 16 * (p % 2) + 4 * (p / 2); }",
                                     "static uint32_t low_bit_pos(uint32_t p) { return 16 * (1 - p % 2) + 4 * (p / 2); }"),
    "split_last_group_paired": ("                if (j / 8 == g) {\n                    rc = enc_symbol(&states[l], &ts, s, wl);",
                                "                if (0) {\n                    rc = enc_symbol(&states[l], &ts, s, wl);"),
    "split_h_four_bits": ("rc = enc_pair_words(&states[l], &ts, s, &th, bso_symbol_f(w[j]) >> 4, wl);",
                          "rc = enc_pair_words(&states[l], &ts, s, &th, (bso_symbol_f(w[j]) >> 4) ^ (j & 1), wl);"),
    "split_refill_between_steps": ("                    rc = decode_step(&x[l], &ts, &s);\n                    if (!rc && j / 8 != g) {",
                                   "                    rc = decode_step(&x[l], &ts, &s);\n                    if (x[l] < BSO_L && pos < nw) x[l] = (x[l] << 16) | words[pos++];\n                    if (!rc && j / 8 != g) {"),
    "htable_threshold_zero": ("eligible[e] = saved[e] > (__int128)65536 * 64;", "eligible[e] = saved[e] > 0;"),
    "htable_tie_high": ("if (best < 0 || saved[e] > saved[best]) best = (int)e;", "if (best < 0 || saved[e] >= saved[best]) best = (int)e;"),
    "htable_signs_not_merged": ("for (uint32_t f = 16 * h; f < 16 * h + 16; f++) m[h] += cf[e * 128 + f] + cf[(256 + e) * 128 + f];",
                                "for (uint32_t f = 16 * h; f < 16 * h + 16; f++) m[h] += cf[e * 128 + f];"),
    "htable_ids_by_saving": ("        id++;\n        id_of[e] = id;\n        for (uint32_t h = 0; h < 8; h++) qh[(id - 1) * 8 + h] = qe[e][h];",
                             "        id++;\n        id_of[e] = (id % 2) ? id + 1 : id - 1;\n        for (uint32_t h = 0; h < 8; h++) qh[(id - 1) * 8 + h] = qe[e][h];"),
    "log2_square_shift": ("        r = (r * r) >> 62;", "        r = (r * r) >> 61;"),
    "log2_bit_compare": ("if (r >= ((unsigned __int128)2 << 62)) { bits |= 1; r >>= 1; }", "if (r > ((unsigned __int128)3 << 61)) { bits |= 1; r >>= 1; }"),
    "share_not_applied": ("        if (!rc && layout == 2) rc = bso_share_hroutes(cs, cf, M_f, md->n_tables, &md->qh[1][0], md->route);\n", ""),
    "share_tie_high": ("if (t == 0 || cost < best_cost) { best = t; best_cost = cost; }",
                       "if (t == 0 || cost <= best_cost) { best = t; best_cost = cost; }"),
    "share_zero_q_usable": ("if (q == 0) { usable = 0; break; }", "if (q == 0) { usable = 1; }"),
    "share_one_sign": ("        if (cs[256 + e]) route[256 + e] = best;\n", ""),
    "share_selected_too": ("if ((cs[e] && route[e]) || (cs[256 + e] && route[256 + e])) continue;   /* has its own table */",
                           "if (0) continue;"),
    "share_flat_value": ("uint32_t q = t == 0 ? (1u << (M_h - 3)) : qh[(t - 1) * 8 + h];",
                         "uint32_t q = t == 0 ? (1u << (M_h - 2)) : qh[(t - 1) * 8 + h];"),
    "share_positive_counts": ("for (uint32_t f = 16 * h; f < 16 * h + 16; f++) m[h] += cf[e * 128 + f] + cf[(256 + e) * 128 + f];\n        }\n        uint32_t best = 0;",
                              "for (uint32_t f = 16 * h; f < 16 * h + 16; f++) m[h] += cf[e * 128 + f];\n        }\n        uint32_t best = 0;"),
    "version2_accepts_layout0": ("else { if (lw < 1 || lw > (version == BSO_VERSION3 ? 3u : 2u)) return BSO_EFORMAT; md->layout = lw; }",
                                 "else { if (lw > (version == BSO_VERSION3 ? 3u : 2u)) return BSO_EFORMAT; md->layout = lw ? lw : 1; }"),
}

# planted mistakes in layout 3 (the joint (s, h) symbol), checked against the
# layout-3 pins only
PINS3 = ["tests/test_oracle_layout3.py"]
MUTANTS3 = {
    "joint_flush_uses_M_s": ("if ((uint64_t)*x >= ((uint64_t)q << (32 - BSO_MT))) {",
                             "if ((uint64_t)*x >= ((uint64_t)q << (32 - md->M_s))) {"),
    "joint_precision_12": ("#define BSO_MT         13u", "#define BSO_MT         12u"),
    "joint_counts_drop_low15": ("for (uint32_t lo = 0; lo < 16; lo++) ct[t] +=", "for (uint32_t lo = 0; lo < 15; lo++) ct[t] +="),
    "joint_counts_h_stride_8": ("ct[t] += cf[(t >> 3) * 128 + 16 * (t & 7u) + lo];", "ct[t] += cf[(t >> 3) * 128 + 8 * (t & 7u) + lo];"),
    "joint_counts_one_sign": ("for (uint32_t t = 0; !rc && t < 512 * 8; t++)", "for (uint32_t t = 0; !rc && t < 256 * 8; t++)"),
    "joint_index_h_major": ("rc = enc_joint(&states[l], md, jt, 8 * s + (bso_symbol_f(w[j]) >> 4), wl);",
                            "rc = enc_joint(&states[l], md, jt, s + 512 * (bso_symbol_f(w[j]) >> 4), wl);"),
    "joint_last_group_joint": ("                if (j / 8 == g) {\n                    rc = enc_symbol(&states[l], &ts, s, wl);",
                               "                if (j / 8 == g && md->layout != 3) {\n                    rc = enc_symbol(&states[l], &ts, s, wl);"),
    "joint_table_h_reversed": ("for (uint32_t h = 0; h < 8; h++) put16(b + ft + 16 * kk + 2 * h, md->qt[8 * sy + h]);",
                               "for (uint32_t h = 0; h < 8; h++) put16(b + ft + 16 * kk + 2 * (7 - h), md->qt[8 * sy + h]);"),
    "joint_decoded_h_shifted": ("                    h = t & 7u;", "                    h = (t >> 1) & 7u;"),
    "joint_no_sum_check": ("if (n_sym && tsum != (1ull << BSO_MT)) return BSO_EFORMAT;", "if (0) return BSO_EFORMAT;"),
    "layout3_plane_missing": ("uint64_t code_bytes = code_block_bytes(K) + (md->layout >= 2 ? plane_bytes(n_c) : 0);",
                              "uint64_t code_bytes = code_block_bytes(K) + (md->layout == 2 ? plane_bytes(n_c) : 0);"),
}


def _run_pins(lib_path, pins=PINS):
    env = dict(os.environ)
    env["BSO_ORACLE_LIB"] = lib_path
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *pins, *SELECT],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def _run_one(job, base_dir):
    """Build one oracle copy (name, source text) and run its pin selection."""
    name, text, pins = job
    d = os.path.join(base_dir, name)
    os.makedirs(d, exist_ok=True)
    c = os.path.join(d, f"{name}.c")
    so = os.path.join(d, f"{name}.so")
    with open(c, "w") as f:
        f.write(text)
    subprocess.check_call(["gcc", "-O1", "-std=gnu11", "-fPIC", "-shared", "-o", so, c])
    return _run_pins(so, pins)


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    """Every planted mistake (and the unmodified oracle, once per pin set),
    built and run concurrently: each case is an independent child process."""
    base = str(tmp_path_factory.mktemp("mutants"))
    src = open(SRC).read()
    jobs = [("clean", src, PINS), ("clean2", src, PINS2), ("clean3", src, PINS3)]
    for table, pins, tag in ((MUTANTS, PINS, "m1"), (MUTANTS2, PINS2, "m2"), (MUTANTS3, PINS3, "m3")):
        for name, (old, new) in table.items():
            assert src.count(old) >= 1, f"mutation anchor not found: {name}"
            jobs.append((f"{tag}_{name}", src.replace(old, new, 1), pins))
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(max_workers=workers) as pool:
        results = list(pool.map(lambda j: _run_one(j, base), jobs))
    return {j[0]: r for j, r in zip(jobs, results)}


def test_unmodified_oracle_passes_selection(outcomes):
    rc, out = outcomes["clean"]
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, outcomes):
    rc, out = outcomes[f"m1_{name}"]
    assert rc != 0, f"planted mistake {name} was not caught:\n{out}"


def test_unmodified_oracle_passes_layout2_selection(outcomes):
    rc, out = outcomes["clean2"]
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS2))
def test_layout2_mutant_is_caught(name, outcomes):
    rc, out = outcomes[f"m2_{name}"]
    assert rc != 0, f"planted mistake {name} was not caught:\n{out}"


def test_unmodified_oracle_passes_layout3_selection(outcomes):
    rc, out = outcomes["clean3"]
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS3))
def test_layout3_mutant_is_caught(name, outcomes):
    rc, out = outcomes[f"m3_{name}"]
    assert rc != 0, f"planted mistake {name} was not caught:\n{out}"
