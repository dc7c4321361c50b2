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
    if (p->m_s < 9 || p->m_s > 12 || p->m_f < 8 || p->m_f > 10 || p->max_tables > kMaxTables) {
        set_error("need 9 <= m_s <= 12, 8 <= m_f <= 10, max_tables <= %u", kMaxTables);
        return false;
    }
    return true;
}

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
    struct Rem { uint64_t rem; uint32_t idx; };
    std::vector<Rem> rems;
    rems.reserve(occupied);
    int64_t have = 0;
    for (uint32_t i = 0; i < A; i++) {
        if (!counts[i]) { q[i] = 0; continue; }
        const unsigned __int128 scaled = (unsigned __int128)counts[i] * total;
        const uint64_t fl = (uint64_t)(scaled / n);
        q[i] = fl ? (uint32_t)fl : 1u;
        have += q[i];
        rems.push_back({(uint64_t)(scaled % n), i});
    }
    int64_t deficit = (int64_t)total - have;
    if (deficit > 0) {
        std::stable_sort(rems.begin(), rems.end(), [](const Rem& a, const Rem& b) { return a.rem > b.rem; });
        for (int64_t k = 0; k < deficit; k++) q[rems[(size_t)k % rems.size()].idx]++;
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
void choose_contexts(const uint64_t exp_counts[256], const std::vector<uint32_t>& cand,
                     const std::vector<std::array<uint64_t, 128>>& merged, uint32_t m_f, uint32_t max_tables,
                     Model& md) {
    struct Scored { uint64_t score; uint32_t e, c; };
    std::vector<Scored> ok;
    for (uint32_t c = 0; c < cand.size(); c++) {
        const unsigned __int128 n = exp_counts[cand[c]];
        unsigned __int128 sq = 0;
        for (uint32_t f = 0; f < 128; f++) sq += (unsigned __int128)merged[c][f] * merged[c][f];
        const unsigned __int128 excess = 128 * sq - n * n;   // >= 0 by Cauchy-Schwarz
        if (256 * excess > n * n + (unsigned __int128)726784 * n) ok.push_back({(uint64_t)(excess / n), cand[c], c});
    }
    std::sort(ok.begin(), ok.end(), [](const Scored& a, const Scored& b) {
        return a.score != b.score ? a.score > b.score : a.e < b.e;
    });
    if (ok.size() > max_tables) ok.resize(max_tables);
    std::sort(ok.begin(), ok.end(), [](const Scored& a, const Scored& b) { return a.e < b.e; });
    md.n_tables = (uint32_t)ok.size();
    std::array<uint32_t, 256> id{};
    for (uint32_t t = 0; t < ok.size(); t++) {
        id[ok[t].e] = t + 1;
        quantise(merged[ok[t].c].data(), 128, m_f, md.q_f[t].data());
    }
    for (uint32_t s = 0; s < 512; s++) md.route[s] = md.counts_s[s] ? id[s & 255] : 0;
}

std::vector<uint32_t> candidates(const uint64_t exp_counts[256]) {
    std::vector<uint32_t> es;
    for (uint32_t e = 0; e < 256; e++)
        if (exp_counts[e]) es.push_back(e);
    std::stable_sort(es.begin(), es.end(), [&](uint32_t a, uint32_t b) { return exp_counts[a] > exp_counts[b]; });
    if (es.size() > kCandidates) es.resize(kCandidates);
    return es;
}

bool finish_model(Model& md, const bs_params* p, const std::vector<uint32_t>& cand,
                  const std::vector<std::array<uint64_t, 128>>& merged) {
    md.m_s = p->m_s;
    md.m_f = p->m_f;
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
    uint64_t ec[256];
    for (uint32_t e = 0; e < 256; e++) ec[e] = md.counts_s[e] + md.counts_s[256 + e];
    choose_contexts(ec, cand, merged, md.m_f, p->max_tables, md);
    return true;
}

}  // namespace bs

using namespace bs;

struct bs_tables : Model {};

extern "C" {

void bs_params_default(bs_params* p) {
    if (!p) return;
    p->chunk_weights = 65536;
    p->lanes = 128;
    p->m_s = 12;
    p->m_f = 10;
    p->max_tables = 6;
    p->threads = 0;
    p->stream_lanes = 0;
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
    const std::vector<uint32_t> cand = candidates(ec);
    std::vector<std::array<uint64_t, 128>> merged(cand.size());
    for (uint32_t c = 0; c < cand.size(); c++)
        for (uint32_t f = 0; f < 128; f++) merged[c][f] = cf[(cand[c] << 7) | f] + cf[((256 + cand[c]) << 7) | f];
    if (!finish_model(*t, p, cand, merged)) { delete t; return BS_E_INVAL; }
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
    t->n = n;
    hipStream_t s = (hipStream_t)stream;
    unsigned long long* d_cnt = nullptr;   // 256 x 128 sign-merged (exponent, fraction) counts, then 256 negative counts
    bs_status rc = BS_OK;
    std::vector<uint32_t> cand;
    std::vector<std::array<uint64_t, 128>> merged;
    constexpr size_t kCounters = 256 * 128 + 256;
    auto hip_fail = [&](hipError_t e, const char* what) {
        set_error("%s: %s", what, hipGetErrorString(e));
        rc = BS_E_HIP;
    };
    hipError_t e = hipMalloc(&d_cnt, kCounters * sizeof(unsigned long long));
    if (e != hipSuccess) { hip_fail(e, "hipMalloc"); goto done; }
    if (n) {
        std::vector<unsigned long long> cnt(kCounters);
        e = hipMemsetAsync(d_cnt, 0, kCounters * sizeof(unsigned long long), s);
        if (e == hipSuccess) e = (hipError_t)bsk_hist((const uint16_t*)d_bf16, n, d_cnt, d_cnt + 256 * 128, stream);
        if (e == hipSuccess) e = hipMemcpyAsync(cnt.data(), d_cnt, kCounters * 8, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) { hip_fail(e, "histogram"); goto done; }
        // the (sign, exponent) counts: negatives counted directly, positives
        // as the exponent's total minus its negatives
        uint64_t ec[256];
        for (uint32_t x = 0; x < 256; x++) {
            uint64_t tot = 0;
            for (uint32_t f = 0; f < 128; f++) tot += cnt[x * 128 + f];
            const uint64_t neg = cnt[256 * 128 + x];
            if (neg > tot) { set_error("histogram counts are inconsistent"); rc = BS_E_HIP; goto done; }
            t->counts_s[256 + x] = neg;
            t->counts_s[x] = tot - neg;
            ec[x] = tot;
        }
        cand = candidates(ec);
        merged.resize(cand.size());
        for (uint32_t c = 0; c < cand.size(); c++)
            for (uint32_t f = 0; f < 128; f++) merged[c][f] = cnt[cand[c] * 128 + f];
    }
    if (!finish_model(*t, p, cand, merged)) rc = BS_E_INVAL;
done:
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

}  // extern "C"
