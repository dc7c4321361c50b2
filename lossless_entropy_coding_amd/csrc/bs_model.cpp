// bs_model.cpp -- per-tensor model: field histograms, quantised frequency
// tables and the choice of coded fraction contexts.
//
// The pages state the model structure [Qwen3.8-27B-BF16-NVLC-Lossless card,
// codec paragraph]: a per-tensor rANS model of the joint (sign, exponent)
// symbol, and a fraction distribution selected by that symbol.  The integer
// rules for quantising counts and for choosing which contexts get their own
// fraction table are this container's definition (see bs.h).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <new>
#include <numeric>
#include <vector>

#include "bs_device.h"
#include "bs_internal.h"
#include "bs_model.h"

namespace bs {

namespace {
thread_local std::string g_err;
}

void set_error(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
}

const char* last_error() { return g_err.c_str(); }

bool params_ok(const bs_params* p) {
    if (!p) { set_error("params is NULL"); return false; }
    const uint32_t K = p->lanes;
    if (K == 0 || (K & (K - 1)) || !(K <= 64 || K == 128 || K == 256 || K == 512 || K == 1024 || K == 2048)) {
        set_error("lanes must be a power of two in 1..64, or 128, 256, 512, 1024 or 2048 (got %u)", K);
        return false;
    }
    if (p->stream_lanes && ((p->stream_lanes & (p->stream_lanes - 1)) || p->stream_lanes > K)) {
        set_error("stream_lanes must be 0 or a power of two <= lanes (got %u)", p->stream_lanes);
        return false;
    }
    if ((p->stream_lanes ? p->stream_lanes : K) > 512) {
        set_error("a word stream holds at most 512 lanes: set stream_lanes for 1024 or 2048 lanes");
        return false;
    }
    if (p->chunk_weights == 0 || p->chunk_weights % (8 * K)) {
        set_error("chunk_weights must be a positive multiple of 8*lanes (got %u)", p->chunk_weights);
        return false;
    }
    if (p->layout == 1) {
        if (p->m_s < 9 || p->m_s > 12 || p->m_f < 8 || p->m_f > 10 || p->max_tables > kMaxTables) {
            set_error("layout 1 needs 9 <= m_s <= 12, 8 <= m_f <= 10, max_tables <= %u", kMaxTables);
            return false;
        }
    } else if (p->layout == 2) {
        if (p->m_s < 11 || p->m_s > 12 || p->m_f != 16 - p->m_s || p->max_tables > kMaxHTables) {
            set_error("layout 2 needs m_s 11 or 12, m_f = 16 - m_s, max_tables <= %u", kMaxHTables);
            return false;
        }
        if ((p->stream_lanes ? p->stream_lanes : K) > 256) {
            set_error("layout 2 decodes with at most 256 lanes per word stream: set stream_lanes");
            return false;
        }
    } else if (p->layout == 3) {
        if (p->m_s < 11 || p->m_s > 12 || p->m_f != kMt) {
            set_error("layout 3 needs m_s 11 or 12 and m_f = %u (the joint table's precision)", kMt);
            return false;
        }
        if ((p->stream_lanes ? p->stream_lanes : K) > 256) {
            set_error("layout 3 decodes with at most 256 lanes per word stream: set stream_lanes");
            return false;
        }
    } else {
        set_error("layout must be 1, 2 or 3 (got %u)", p->layout);
        return false;
    }
    return true;
}

// floor(65536 log2 q) for the table rule of layout 2 (q <= 2^m_f <= 32 there).
// The double logarithm of an integer is within an ulp of the exact value, and
// no 65536 log2 q for q <= 2^16 lies that close to an integer without being
// one (q a power of two, where the logarithm is exact).
uint32_t log2_q16(uint32_t q) { return (uint32_t)std::floor(std::log2((double)q) * 65536.0); }

// counts -> frequencies summing to 2^M; integer rule documented in bs.h
bool quantise(const uint64_t* counts, uint32_t A, uint32_t M, uint32_t* q) {
    const uint64_t total = 1ull << M;
    uint64_t n = 0;
    uint32_t occupied = 0;
    for (uint32_t i = 0; i < A; i++) {
        n += counts[i];
        occupied += counts[i] != 0;
    }
    if (n == 0 || occupied > total) return false;
    // (fixed-size working arrays: the model is built without heap memory;
    // the largest alphabet is layout 3's 512 x 8 joint symbols)
    struct Rem { uint64_t rem; uint32_t idx; };
    if (A > 512 * 8) return false;
    Rem rems[512 * 8];
    uint32_t n_rem = 0;
    int64_t have = 0;
    for (uint32_t i = 0; i < A; i++) {
        if (!counts[i]) { q[i] = 0; continue; }
        const unsigned __int128 scaled = (unsigned __int128)counts[i] * total;
        const uint64_t fl = (uint64_t)(scaled / n);
        q[i] = fl ? (uint32_t)fl : 1u;
        have += q[i];
        rems[n_rem++] = {(uint64_t)(scaled % n), i};
    }
    int64_t deficit = (int64_t)total - have;
    if (deficit > 0) {
        // largest remainder first, lower index first on ties
        std::sort(rems, rems + n_rem, [](const Rem& a, const Rem& b) { return a.rem != b.rem ? a.rem > b.rem : a.idx < b.idx; });
        for (int64_t k = 0; k < deficit; k++) q[rems[(size_t)k % n_rem].idx]++;
    }
    for (; deficit < 0; deficit++) {
        uint32_t* big = nullptr;
        for (uint32_t i = 0; i < A; i++)
            if (q[i] > 1 && (!big || q[i] > *big)) big = &q[i];
        if (!big) return false;
        (*big)--;
    }
    return true;
}

// Choose the coded fraction contexts from the per-exponent merged counts.
// exp_counts[e] = cs[e] + cs[256+e]; merged[c][f] = fraction counts of the
// c-th candidate (candidates = the 64 most frequent exponents, lower e first
// on ties, in that order).
void choose_contexts(const uint64_t exp_counts[256], const uint32_t* cand, uint32_t n_cand,
                     const std::array<uint64_t, 128>* merged, uint32_t m_f, uint32_t max_tables, Model& md) {
    struct Scored { uint64_t score; uint32_t e, c; };
    Scored ok[256];
    uint32_t n_ok = 0;
    for (uint32_t c = 0; c < n_cand; c++) {
        const unsigned __int128 n = exp_counts[cand[c]];
        unsigned __int128 sq = 0;
        for (uint32_t f = 0; f < 128; f++) sq += (unsigned __int128)merged[c][f] * merged[c][f];
        const unsigned __int128 excess = 128 * sq - n * n;   // >= 0 by Cauchy-Schwarz
        if (256 * excess > n * n + (unsigned __int128)726784 * n) ok[n_ok++] = {(uint64_t)(excess / n), cand[c], c};
    }
    std::sort(ok, ok + n_ok, [](const Scored& a, const Scored& b) {
        return a.score != b.score ? a.score > b.score : a.e < b.e;
    });
    if (n_ok > max_tables) n_ok = max_tables;
    std::sort(ok, ok + n_ok, [](const Scored& a, const Scored& b) { return a.e < b.e; });
    md.n_tables = n_ok;
    std::array<uint32_t, 256> id{};
    for (uint32_t t = 0; t < n_ok; t++) {
        id[ok[t].e] = t + 1;
        quantise(merged[ok[t].c].data(), 128, m_f, md.q_f[t].data());
    }
    for (uint32_t s = 0; s < 512; s++) md.route[s] = md.counts_s[s] ? id[s & 255] : 0;
}

// Layout 2: the coded h tables.  hc[e][h] = counts of h = f >> 4 over both
// signs of exponent e.  An exponent is eligible when quantising its counts
// saves more than 64 bits against the flat table (bits counted in units of
// 2^-16 with floor(65536 log2 q)); the max_tables largest savings win (lower
// exponent on ties); ids ascend with the exponent.
void choose_htables(const std::array<std::array<uint64_t, 8>, 256>& hc, uint32_t m_h, uint32_t max_tables, Model& md) {
    struct Cand { __int128 saved; uint32_t e; std::array<uint32_t, 8> q; };
    Cand ok[256];
    uint32_t n_ok = 0;
    const int64_t flat = 65536 * (int64_t)(m_h - 3);
    for (uint32_t e = 0; e < 256; e++) {
        uint64_t n_e = 0;
        for (uint32_t h = 0; h < 8; h++) n_e += hc[e][h];
        if (!n_e) continue;
        Cand c{0, e, {}};
        quantise(hc[e].data(), 8, m_h, c.q.data());
        for (uint32_t h = 0; h < 8; h++)
            if (hc[e][h]) c.saved += (__int128)hc[e][h] * ((int64_t)log2_q16(c.q[h]) - flat);
        if (c.saved > (__int128)65536 * 64) ok[n_ok++] = c;
    }
    std::sort(ok, ok + n_ok, [](const Cand& a, const Cand& b) { return a.saved != b.saved ? a.saved > b.saved : a.e < b.e; });
    if (n_ok > max_tables) n_ok = max_tables;
    std::sort(ok, ok + n_ok, [](const Cand& a, const Cand& b) { return a.e < b.e; });
    md.n_tables = n_ok;
    std::array<uint32_t, 256> id{};
    for (uint32_t t = 0; t < n_ok; t++) {
        id[ok[t].e] = t + 1;
        md.q_h[t] = ok[t].q;
    }
    // Shared routing: an exponent without a table of its own goes to the
    // table (flat or coded) that codes its h counts in the fewest 2^-16 bits,
    // sum of m[h] (65536 M_h - floor(65536 log2 q_t[h])); a table with q = 0
    // for a used h cannot take it; the lower id wins ties, so flat stays
    // unless a coded table is strictly cheaper.
    for (uint32_t e = 0; e < 256; e++) {
        uint64_t n_e = 0;
        for (uint32_t h = 0; h < 8; h++) n_e += hc[e][h];
        if (!n_e || id[e]) continue;
        uint32_t best = 0;
        unsigned __int128 best_cost = 0;
        for (uint32_t t = 0; t <= n_ok; t++) {
            unsigned __int128 cost = 0;
            bool usable = true;
            for (uint32_t h = 0; h < 8 && usable; h++) {
                if (!hc[e][h]) continue;
                const uint32_t q = t == 0 ? 1u << (m_h - 3) : md.q_h[t - 1][h];
                if (!q) { usable = false; break; }
                cost += (unsigned __int128)hc[e][h] * (65536u * m_h - log2_q16(q));
            }
            if (usable && (t == 0 || cost < best_cost)) { best = t; best_cost = cost; }
        }
        id[e] = best;
    }
    for (uint32_t s = 0; s < 512; s++) md.route[s] = md.counts_s[s] ? id[s & 255] : 0;
}

// the occupied exponents, most frequent first (lower exponent on ties), at
// most kCandidates of them; returns their number
uint32_t candidates(const uint64_t exp_counts[256], uint32_t* es) {
    uint32_t all[256], n = 0;
    for (uint32_t e = 0; e < 256; e++)
        if (exp_counts[e]) all[n++] = e;
    std::sort(all, all + n, [&](uint32_t a, uint32_t b) { return exp_counts[a] != exp_counts[b] ? exp_counts[a] > exp_counts[b] : a < b; });
    n = std::min<uint32_t>(n, kCandidates);
    std::copy(all, all + n, es);
    return n;
}

// ct: the joint (sign, exponent, h) counts of layout 3 at 8 s + h (unused otherwise)
bool finish_model(Model& md, const bs_params* p, const uint32_t* cand, uint32_t n_cand,
                  const std::array<uint64_t, 128>* merged, const std::array<std::array<uint64_t, 8>, 256>& hc,
                  const uint64_t* ct) {
    md.m_s = p->m_s;
    md.m_f = p->m_f;
    md.layout = p->layout;
    md.n_sym = 0;
    for (uint32_t s = 0; s < 512; s++) md.n_sym += md.counts_s[s] != 0;
    md.n_tables = 0;
    md.route.fill(0);
    md.q_s.fill(0);
    if (md.n == 0) return true;
    if (!quantise(md.counts_s.data(), 512, md.m_s, md.q_s.data())) {
        set_error("cannot quantise the sign/exponent counts");
        return false;
    }
    if (md.layout == 2) {
        choose_htables(hc, md.m_f, p->max_tables, md);
        return true;
    }
    if (md.layout == 3) {
        if (!quantise(ct, 512 * 8, kMt, md.q_t.data())) {
            set_error("cannot quantise the joint (sign, exponent, h) counts");
            return false;
        }
        return true;
    }
    uint64_t ec[256];
    for (uint32_t e = 0; e < 256; e++) ec[e] = md.counts_s[e] + md.counts_s[256 + e];
    choose_contexts(ec, cand, n_cand, merged, md.m_f, p->max_tables, md);
    return true;
}

// The model of n words from the device histogram's counters: cnt[e * 128 +
// f] counts exponent e and fraction f over both signs, cnt[256 * 128 + 8 e +
// h] the negative words of exponent e with high fraction bits h.  md is
// overwritten; merged is working memory for kCandidates fraction histograms,
// ct for the 4096 joint counts.  Allocates nothing.
bs_status model_from_counts(Model& md, const bs_params* p, uint64_t n, const unsigned long long* cnt,
                            std::array<uint64_t, 128>* merged, uint64_t* ct) {
    md = Model{};
    md.n = n;
    uint32_t cand[kCandidates];
    uint32_t n_cand = 0;
    std::array<std::array<uint64_t, 8>, 256> hc{};
    for (uint32_t t = 0; t < 512 * 8; t++) ct[t] = 0;
    if (n) {
        // the (sign, exponent, h) counts: negatives counted directly,
        // positives as the sign-merged count minus the negatives; the
        // (sign, exponent) counts are their sums over h
        uint64_t ec[256], sum = 0;
        for (uint32_t x = 0; x < 256; x++) {
            uint64_t tot = 0, neg = 0;
            for (uint32_t h = 0; h < 8; h++) {
                uint64_t both = 0;
                for (uint32_t f = 16 * h; f < 16 * h + 16; f++) both += cnt[x * 128 + f];
                const uint64_t nh = cnt[256 * 128 + 8 * x + h];
                if (nh > both) { set_error("histogram counts are inconsistent"); return BS_E_HIP; }
                ct[8 * (256 + x) + h] = nh;
                ct[8 * x + h] = both - nh;
                tot += both;
                neg += nh;
            }
            md.counts_s[256 + x] = neg;
            md.counts_s[x] = tot - neg;
            ec[x] = tot;
            sum += tot;
        }
        if (sum != n) { set_error("histogram counts %llu words, not %llu", (unsigned long long)sum, (unsigned long long)n); return BS_E_HIP; }
        n_cand = candidates(ec, cand);
        for (uint32_t c = 0; c < n_cand; c++)
            for (uint32_t f = 0; f < 128; f++) merged[c][f] = cnt[cand[c] * 128 + f];
        for (uint32_t x = 0; x < 256; x++)
            for (uint32_t f = 0; f < 128; f++) hc[x][f >> 4] += cnt[x * 128 + f];
    }
    return finish_model(md, p, cand, n_cand, merged, hc, ct) ? BS_OK : BS_E_INVAL;
}

}  // namespace bs

using namespace bs;


extern "C" {

void bs_params_default(bs_params* p) {
    if (!p) return;
    p->chunk_weights = 65536;
    p->lanes = 128;
    p->m_s = 11;
    p->m_f = kMt;          // the joint table's precision
    p->max_tables = 31;    // layout 2's coded h tables (layout 3 has none)
    p->threads = 0;
    p->stream_lanes = 0;
    p->layout = 3;
}

bs_status bs_build_tables_host(const uint16_t* h, uint64_t n, const bs_params* p, bs_tables** out) {
    if (!out || (!h && n) || !params_ok(p)) {
        if (!out || (!h && n)) set_error("NULL argument");
        return BS_E_INVAL;
    }
    bs_tables* t = new (std::nothrow) bs_tables();
    if (!t) return BS_E_NOMEM;
    t->n = n;
    std::vector<uint64_t> cf(512 * 128, 0);
    for (uint64_t i = 0; i < n; i++) {
        const uint32_t w = h[i];
        t->counts_s[w >> 7]++;
        cf[w]++;  // (s, f) pair index == the word itself
    }
    uint64_t ec[256];
    for (uint32_t e = 0; e < 256; e++) ec[e] = t->counts_s[e] + t->counts_s[256 + e];
    uint32_t cand[kCandidates];
    const uint32_t n_cand = candidates(ec, cand);
    std::vector<std::array<uint64_t, 128>> merged(kCandidates);
    for (uint32_t c = 0; c < n_cand; c++)
        for (uint32_t f = 0; f < 128; f++) merged[c][f] = cf[(cand[c] << 7) | f] + cf[((256 + cand[c]) << 7) | f];
    std::array<std::array<uint64_t, 8>, 256> hc{};
    for (uint32_t e = 0; e < 256; e++)
        for (uint32_t f = 0; f < 128; f++) hc[e][f >> 4] += cf[(e << 7) | f] + cf[((256 + e) << 7) | f];
    std::vector<uint64_t> ct(512 * 8, 0);   // joint (s, h) counts: fraction counts summed over the low four bits
    for (uint32_t s = 0; s < 512; s++)
        for (uint32_t f = 0; f < 128; f++) ct[8 * s + (f >> 4)] += cf[(s << 7) | f];
    if (!finish_model(*t, p, cand, n_cand, merged.data(), hc, ct.data())) { delete t; return BS_E_INVAL; }
    *out = t;
    return BS_OK;
}

bs_status bs_build_tables(const void* d_bf16, uint64_t n, const bs_params* p, void* stream, bs_tables** out) {
    if (!out || (!d_bf16 && n) || !params_ok(p)) {
        if (!out || (!d_bf16 && n)) set_error("NULL argument");
        return BS_E_INVAL;
    }
    bs_tables* t = new (std::nothrow) bs_tables();
    if (!t) return BS_E_NOMEM;
    hipStream_t s = (hipStream_t)stream;
    unsigned long long* d_cnt = nullptr;   // kHistCounters: see model_from_counts
    std::vector<unsigned long long> cnt(kHistCounters, 0);
    std::vector<std::array<uint64_t, 128>> merged(kCandidates);
    std::vector<uint64_t> ct(512 * 8);
    bs_status rc = BS_OK;
    hipError_t e = hipMalloc(&d_cnt, kHistCounters * sizeof(unsigned long long));
    if (e == hipSuccess && n) {
        e = hipMemsetAsync(d_cnt, 0, kHistCounters * sizeof(unsigned long long), s);
        if (e == hipSuccess) e = (hipError_t)bsk_hist((const uint16_t*)d_bf16, n, d_cnt, d_cnt + 256 * 128, stream);
        if (e == hipSuccess) e = hipMemcpyAsync(cnt.data(), d_cnt, kHistCounters * 8, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
    }
    if (e != hipSuccess) {
        set_error("histogram: %s", hipGetErrorString(e));
        rc = BS_E_HIP;
    } else {
        rc = model_from_counts(*t, p, n, cnt.data(), merged.data(), ct.data());
    }
    if (d_cnt) (void)hipFree(d_cnt);
    if (rc != BS_OK) { delete t; return rc; }
    *out = t;
    return BS_OK;
}

void bs_tables_free(bs_tables* t) { delete t; }

bs_status bs_tables_get(const bs_tables* t, uint64_t* counts_s, uint32_t* q_s, uint32_t* route, uint32_t* q_f,
                        uint32_t* n_tables, uint32_t* m_s, uint32_t* m_f, uint64_t* n_weights) {
    if (!t) { set_error("NULL tables"); return BS_E_INVAL; }
    if (counts_s) memcpy(counts_s, t->counts_s.data(), 512 * 8);
    if (q_s) memcpy(q_s, t->q_s.data(), 512 * 4);
    if (route) memcpy(route, t->route.data(), 512 * 4);
    if (q_f)
        for (uint32_t k = 0; k < kMaxTables; k++) memcpy(q_f + 128 * k, t->q_f[k].data(), 128 * 4);
    if (n_tables) *n_tables = t->n_tables;
    if (m_s) *m_s = t->m_s;
    if (m_f) *m_f = t->m_f;
    if (n_weights) *n_weights = t->n;
    return BS_OK;
}

bs_status bs_tables_get_layout(const bs_tables* t, uint32_t* layout, uint32_t* q_h) {
    if (!t) { set_error("NULL tables"); return BS_E_INVAL; }
    if (layout) *layout = t->layout;
    if (q_h)
        for (uint32_t k = 0; k < kMaxHTables; k++) memcpy(q_h + 8 * k, t->q_h[k].data(), 8 * 4);
    return BS_OK;
}

bs_status bs_tables_get_joint(const bs_tables* t, uint32_t* q_t) {
    if (!t || !q_t) { set_error("NULL argument"); return BS_E_INVAL; }
    memcpy(q_t, t->q_t.data(), 512 * 8 * 4);
    return BS_OK;
}

}  // extern "C"
