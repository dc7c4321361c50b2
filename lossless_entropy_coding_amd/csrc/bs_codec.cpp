// bs_codec.cpp -- host encoder, container validation and the C ABI for
// encode / inspect / decode / verify.
//
// The coder [Qwen3.8-27B-BF16-NVLC-Lossless card, codec paragraph]: each BF16
// word is split into the joint (sign, exponent) symbol s = w >> 7 and the
// fraction f = w & 127; s is coded with the tensor's rANS model and f with the
// distribution that s selects; decoding recombines them bitwise.  The state
// width, renormalisation unit, interleave and byte layout are this library's
// container (bs.h).
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>
#include <sys/stat.h>

#include <algorithm>
#include <atomic>
#include <new>
#include <thread>
#include <vector>

#include "bs_device.h"
#include "bs_encode_device.h"
#include "bs_internal.h"
#include "bs_model.h"

namespace bs {
namespace {

constexpr uint32_t kL = 65536u;

// ------------------------------------------------------------------ encoder

// rANS encoder entry of one symbol: flush threshold, frequency, start
struct EncSym {
    uint64_t x_max;  // flush the low word first when x >= x_max
    uint32_t q;
    uint32_t cum;
};

struct EncModel {
    uint32_t layout;
    uint32_t m_s, m_f;                 // layout 2: m_f is M_h
    EncSym s[512];
    EncSym f[kMaxTables + 1][128];     // layout 1
    EncSym h[kMaxHTables + 1][8];      // layout 2 (x_max unused: a pair's bound is joint)
    EncSym t[512 * 8];                 // layout 3: the joint symbol 8 s + h at precision kMt
    uint8_t route[512];
};

void make_enc(const Model& md, EncModel& em) {
    em.layout = md.layout;
    em.m_s = md.m_s;
    em.m_f = md.m_f;
    uint32_t cum = 0;
    for (uint32_t s = 0; s < 512; s++) {
        em.s[s] = {(uint64_t)md.q_s[s] << (32 - md.m_s), md.q_s[s], cum};
        cum += md.q_s[s];
        em.route[s] = (uint8_t)md.route[s];
    }
    if (md.layout == 3) {
        cum = 0;
        for (uint32_t t = 0; t < 512 * 8; t++) {
            em.t[t] = {(uint64_t)md.q_t[t] << (32 - kMt), md.q_t[t], cum};
            cum += md.q_t[t];
        }
        return;
    }
    if (md.layout == 2) {
        for (uint32_t t = 0; t <= md.n_tables; t++) {
            cum = 0;
            for (uint32_t h = 0; h < 8; h++) {
                const uint32_t q = t == 0 ? (1u << (md.m_f - 3)) : md.q_h[t - 1][h];
                em.h[t][h] = {0, q, cum};
                cum += q;
            }
        }
        return;
    }
    for (uint32_t t = 0; t <= md.n_tables; t++) {
        cum = 0;
        for (uint32_t f = 0; f < 128; f++) {
            const uint32_t q = t == 0 ? (1u << (md.m_f - 7)) : md.q_f[t - 1][f];
            em.f[t][f] = {(uint64_t)q << (32 - md.m_f), q, cum};
            cum += q;
        }
    }
}

inline void put(uint32_t& x, const EncSym& e, uint32_t M, uint16_t*& sink) {
    if (x >= e.x_max) {
        *sink++ = (uint16_t)x;
        x >>= 16;
    }
    x = ((x / e.q) << M) + x % e.q + e.cum;
}

// Start states.  Lane l's last group holds c = min(8, weights left) weights;
// its last m = min(4, c) weights keep only their s symbol in the stream, and
// their 7-bit fractions are the low 7m bits of the lane's start state (the
// first of them lowest) under a leading one at bit max(16, 7m).  The decoder
// finds them in its final state.  A lane without weights starts at 2^16.
struct RawTail {
    uint64_t j0;   // chunk index of the first of the m weights
    uint32_t m;    // 0 for a lane without weights
};

inline RawTail raw_tail(uint32_t n_c, uint32_t K, uint32_t l) {
    const uint64_t groups = ((uint64_t)n_c + 7) / 8;
    if (l >= groups) return {0, 0};
    const uint64_t g = l + (uint64_t)K * ((groups - 1 - l) / K);   // the lane's last group
    const uint64_t end = std::min<uint64_t>(8 * g + 8, n_c);
    const uint32_t m = (uint32_t)std::min<uint64_t>(end - 8 * g, 4);
    return {end - m, m};
}

// Encode the lanes [l0, l1) of one chunk (n_c weights, K lanes): one word
// stream.  Sub-steps run from last to first, lanes from l1-1 down to l0
// inside each, so that the decoder reads forwards; the emitted words come out
// reversed and are turned around by the caller.  `scratch` must hold 2 * n_c
// words.  Returns the word count.
uint64_t encode_stream(const EncModel& em, const uint16_t* w, uint32_t n_c, uint32_t K, uint32_t l0, uint32_t l1,
                       uint32_t* x, uint16_t* scratch) {
    uint64_t j0[512];
    uint32_t m[512];
    for (uint32_t l = l0; l < l1; l++) {
        const RawTail rt = raw_tail(n_c, K, l);
        j0[l - l0] = rt.j0;
        m[l - l0] = rt.m;
        uint32_t v = rt.m ? 1u << std::max(16u, 7 * rt.m) : kL;
        for (uint32_t i = 0; i < rt.m; i++) v |= (w[rt.j0 + i] & 127u) << (7 * i);
        x[l] = v;
    }
    uint16_t* sink = scratch;
    const uint32_t groups = (n_c + 7) / 8;
    const uint32_t T = (groups + K - 1) / K;
    for (uint32_t t = T; t-- > 0;) {
        for (int p = 7; p >= 0; p--) {
            // fraction sub-step, then sign/exponent sub-step (reverse of decode order)
            for (uint32_t l = l1; l-- > l0;) {
                const uint64_t j = 8ull * ((uint64_t)t * K + l) + (uint64_t)p;
                if (j >= n_c || (j >= j0[l - l0] && j < j0[l - l0] + m[l - l0])) continue;
                const uint32_t v = w[j];
                put(x[l], em.f[em.route[v >> 7]][v & 127], em.m_f, sink);
            }
            for (uint32_t l = l1; l-- > l0;) {
                const uint64_t j = 8ull * ((uint64_t)t * K + l) + (uint64_t)p;
                if (j >= n_c) continue;
                put(x[l], em.s[w[j] >> 7], em.m_s, sink);
            }
        }
    }
    return (uint64_t)(sink - scratch);
}

// Layouts 2 and 3: one stream of the lanes [l0, l1) of a chunk, one
// renormalisation per weight.  Layout 2: a lane's weight outside its last
// group is the pair (s, h = f >> 4): one flush check against the joint bound
// q_s q_h 2^(32 - M_s - M_h) = q_s q_h 2^16, then h is coded, then s (the
// decoder takes s first).  Layout 3: that weight is the one joint symbol
// 8 s + h (precision kMt).  In its last group (c weights) a lane codes s
// only; the h of those weights start the lane's state: the low 3c bits under
// a leading one at bit max(16, 3c).  The low fraction bits go to the chunk's
// plane, not here.
uint64_t encode_stream2(const EncModel& em, const uint16_t* w, uint32_t n_c, uint32_t K, uint32_t l0, uint32_t l1,
                        uint32_t* x, uint16_t* scratch) {
    const uint64_t groups = ((uint64_t)n_c + 7) / 8;
    uint64_t last[512];
    for (uint32_t l = l0; l < l1; l++) {
        if (l >= groups) {
            x[l] = kL;
            last[l - l0] = UINT64_MAX;
            continue;
        }
        const uint64_t g = l + (uint64_t)K * ((groups - 1 - l) / K);
        const uint32_t c = (uint32_t)std::min<uint64_t>(8, n_c - 8 * g);
        uint32_t v = 1u << std::max(16u, 3 * c);
        for (uint32_t i = 0; i < c; i++) v |= ((w[8 * g + i] & 127u) >> 4) << (3 * i);
        x[l] = v;
        last[l - l0] = g;
    }
    uint16_t* sink = scratch;
    const uint32_t T = (uint32_t)((groups + K - 1) / K);
    for (uint32_t t = T; t-- > 0;) {
        for (int p = 7; p >= 0; p--) {
            for (uint32_t l = l1; l-- > l0;) {
                const uint64_t j = 8ull * ((uint64_t)t * K + l) + (uint64_t)p;
                if (j >= n_c) continue;
                const uint32_t v = w[j];
                const EncSym& es = em.s[v >> 7];
                if (j / 8 == last[l - l0]) {
                    put(x[l], es, em.m_s, sink);
                    continue;
                }
                if (em.layout == 3) {
                    put(x[l], em.t[8 * (v >> 7) + ((v & 127u) >> 4)], kMt, sink);
                    continue;
                }
                const EncSym& eh = em.h[em.route[v >> 7]][(v & 127u) >> 4];
                uint32_t& xl = x[l];
                if (xl >= ((uint64_t)es.q * eh.q) << (32 - em.m_s - em.m_f)) {
                    *sink++ = (uint16_t)xl;
                    xl >>= 16;
                }
                xl = ((xl / eh.q) << em.m_f) + xl % eh.q + eh.cum;
                xl = ((xl / es.q) << em.m_s) + xl % es.q + es.cum;
            }
        }
    }
    return (uint64_t)(sink - scratch);
}

void record_shape(uint64_t n, uint32_t W, uint32_t K, uint32_t& w_out, uint32_t& k_out) {
    if (n >= W) { w_out = W; k_out = K; return; }
    const uint64_t per_lane = W / K;
    uint32_t k = 1;
    while (k < K && (uint64_t)k * per_lane < n) k <<= 1;
    k_out = k;
    w_out = (uint32_t)align_up(n ? n : 1, 8ull * k);
}

// A final state x in [2^16, 2^32) is stored as its length code
// e = floor(log2 x) - 16 (a nibble per lane, in the chunk's code block) and
// its 16 + e bits below the leading one (concatenated in lane order, least
// significant bit first, at the head of its stream, padded to a 16-bit unit).
inline uint32_t state_code(uint32_t x) { return 31u - (uint32_t)__builtin_clz(x) - 16u; }
inline uint64_t code_bytes(uint32_t K) { return align_up((K + 1ull) / 2, 16); }
// 16-bit units of the state bits of P lanes whose codes sum to esum
inline uint64_t state_units(uint32_t P, uint64_t esum) { return (16ull * P + esum + 15) / 16; }

struct ChunkOut {
    std::vector<uint32_t> states;
    std::vector<uint32_t> plane;                // layout 2: the low fraction bits, a u32 per group
    std::vector<std::vector<uint16_t>> words;   // per stream, decode order
    std::vector<uint64_t> mu;                   // per stream, units of its state bits
    uint64_t units(uint32_t st) const { return mu[st] + words[st].size(); }
    uint64_t total() const {
        uint64_t t = 0;
        for (uint32_t st = 0; st < words.size(); st++) t += units(st);
        return t;
    }
};

// chunk payload bytes: the length codes padded to 16 bytes, then the streams
// back to back (state bits, then words), the whole padded to 16 bytes
uint64_t payload_bytes(const ChunkOut& co, uint32_t K) {
    return align_up(code_bytes(K) + 4 * co.plane.size() + 2 * co.total(), 16);
}

struct EncRecord {
    uint32_t kind = 0;
    uint64_t n = 0;
    const uint8_t* data = nullptr;
    uint8_t sha[32];
    const Model* md = nullptr;
    Model owned;
    EncModel em;
    uint32_t W = 0, K = 0, S = 1, n_chunks = 0;
    std::vector<ChunkOut> chunks;
    std::vector<uint8_t> head;   // fixed part, tables, chunk index and stream table (the last two filled at assembly)
    uint64_t index_off = 0;
    uint64_t stab_off = 0;       // stream table: per chunk, the start unit of streams 1 .. S-1
};

void build_head(EncRecord& r) {
    const Model& md = *r.md;
    const uint64_t stab = 24;
    const uint64_t route_off = stab + 4ull * md.n_sym;
    const uint64_t ftab = align_up(route_off + md.n_sym, 4);
    const uint64_t tab_end = md.layout == 3 ? ftab + 16ull * md.n_sym : ftab + (md.layout == 2 ? 8ull : 256ull) * md.n_tables;
    r.index_off = align_up(tab_end, 16);
    r.stab_off = r.index_off + 16ull * r.n_chunks;
    r.head.assign(align_up(r.stab_off + 4ull * (r.S - 1) * r.n_chunks, 16), 0);
    uint8_t* b = r.head.data();
    wr32(b + 0, r.W);
    wr32(b + 4, r.K);
    wr32(b + 8, r.n_chunks);
    b[12] = (uint8_t)md.m_s;
    b[13] = (uint8_t)md.m_f;
    b[14] = (uint8_t)md.n_tables;
    uint32_t log2s = 0;
    while ((1u << log2s) < r.S) log2s++;
    b[15] = (uint8_t)log2s;
    wr32(b + 16, md.n_sym);
    wr32(b + 20, md.layout == 1 ? 0u : md.layout);   // version 1 (layout 1 only) keeps 0 here
    uint32_t k = 0;
    for (uint32_t s = 0; s < 512; s++) {
        if (!md.counts_s[s]) continue;
        wr16(b + stab + 4 * k, s);
        wr16(b + stab + 4 * k + 2, md.q_s[s]);
        b[route_off + k] = (uint8_t)md.route[s];
        // layout 3: the eight joint frequencies of s, in the order of the s list
        if (md.layout == 3)
            for (uint32_t h = 0; h < 8; h++) wr16(b + ftab + 16 * k + 2 * h, md.q_t[8 * s + h]);
        k++;
    }
    for (uint32_t t = 0; t < md.n_tables; t++) {
        if (md.layout == 2) {
            for (uint32_t h = 0; h < 8; h++) b[ftab + 8 * t + h] = (uint8_t)md.q_h[t][h];
        } else {
            for (uint32_t f = 0; f < 128; f++) wr16(b + ftab + 256 * t + 2 * f, md.q_f[t][f]);
        }
    }
}

}  // namespace

// ------------------------------------------------------------------ validation

bs_status parse_container(const uint8_t* h, uint64_t len, Container& c) {
    if (!h || len < kHeaderBytes || memcmp(h, kMagic, 8) != 0) {
        set_error("not a BF16RANS container");
        return BS_E_FORMAT;
    }
    const uint32_t version = rd32(h + 8);
    if (version != kVersion && version != kVersion2 && version != kVersion3) {
        set_error("container version %u is not supported (this library reads versions %u to %u)", version, kVersion,
                  kVersion3);
        return BS_E_VERSION;
    }
    c.n_records = rd32(h + 12);
    const uint64_t dir = rd64(h + 16);
    c.total_len = rd64(h + 24);
    c.out_len = rd64(h + 32);
    if (c.total_len != len) { set_error("length %llu differs from the header's %llu", (unsigned long long)len, (unsigned long long)c.total_len); return BS_E_FORMAT; }
    if (dir < kHeaderBytes || dir > len || (len - dir) / kDirEntryBytes < c.n_records) {
        set_error("directory out of bounds");
        return BS_E_FORMAT;
    }
    c.recs.assign(c.n_records, Record());
    c.n_chunks = 0;
    c.n_streams = 0;
    uint64_t out_end = 0;
    for (uint32_t i = 0; i < c.n_records; i++) {
        const uint8_t* d = h + dir + kDirEntryBytes * i;
        Record& r = c.recs[i];
        r.kind = rd32(d);
        r.n = rd64(d + 8);
        r.out_offset = rd64(d + 16);
        r.rec_offset = rd64(d + 24);
        r.rec_len = rd64(d + 32);
        memcpy(r.sha, d + 40, 32);
        if (r.rec_offset > len || r.rec_len > len - r.rec_offset) { set_error("record %u out of bounds", i); return BS_E_FORMAT; }
        if (r.kind != BS_KIND_BF16 && r.kind != BS_KIND_RAW) { set_error("record %u has unknown kind %u", i, r.kind); return BS_E_FORMAT; }
        if (r.n > (1ull << 56) || r.out_offset > (1ull << 60)) { set_error("record %u size out of range", i); return BS_E_FORMAT; }
        out_end = std::max(out_end, r.out_offset + r.out_bytes());
        if (r.kind == BS_KIND_RAW) {
            if (r.rec_len < r.n) { set_error("raw record %u shorter than its size", i); return BS_E_FORMAT; }
            continue;
        }
        if (r.out_offset % 16) { set_error("BF16 record %u output offset not 16-aligned", i); return BS_E_FORMAT; }
        if (r.rec_offset % 16) { set_error("BF16 record %u not 16-aligned", i); return BS_E_FORMAT; }
        const uint8_t* b = h + r.rec_offset;
        if (r.rec_len < 24) { set_error("record %u truncated", i); return BS_E_FORMAT; }
        r.W = rd32(b);
        r.K = rd32(b + 4);
        r.n_chunks = rd32(b + 8);
        r.m_s = b[12];
        r.m_f = b[13];
        r.n_tables = b[14];
        r.n_sym = rd32(b + 16);
        // version 1: the word at +20 is 0 (layout 1); versions 2 and 3 name
        // the layout there (1 or 2; version 3 also 3)
        const uint32_t lw = rd32(b + 20);
        if (version == kVersion ? lw != 0 : (lw < 1 || lw > (version == kVersion3 ? 3u : 2u))) {
            set_error("record %u: bad layout word %u", i, lw);
            return BS_E_FORMAT;
        }
        r.layout = version == kVersion ? 1 : lw;
        const uint32_t K = r.K;
        if (b[15] > 9 || (1u << b[15]) > K) { set_error("record %u: bad stream count", i); return BS_E_FORMAT; }
        r.S = 1u << b[15];
        if (K == 0 || (K & (K - 1)) || !(K <= 64 || K == 128 || K == 256 || K == 512 || K == 1024 || K == 2048) || r.W == 0 ||
            r.W % (8 * K) || K / r.S > 512) {
            set_error("record %u: bad chunk shape W=%u K=%u", i, r.W, K);
            return BS_E_FORMAT;
        }
        if (r.layout == 1   ? (r.m_s < 9 || r.m_s > 12 || r.m_f < 8 || r.m_f > 10 || r.n_tables > kMaxTables)
            : r.layout == 2 ? (r.m_s < 11 || r.m_s > 12 || r.m_f != 16 - r.m_s || r.n_tables > kMaxHTables)
                            : (r.m_s < 11 || r.m_s > 12 || r.m_f != kMt || r.n_tables != 0)) {
            set_error("record %u: bad table parameters", i);
            return BS_E_FORMAT;
        }
        if ((uint64_t)r.n_chunks != (r.n + r.W - 1) / r.W) { set_error("record %u: chunk count mismatch", i); return BS_E_FORMAT; }
        if (r.n_sym > kMaxSyms || (r.n_sym == 0) != (r.n == 0)) { set_error("record %u: bad symbol count", i); return BS_E_FORMAT; }
        r.stab_off = 24;
        r.route_off = 24 + 4 * r.n_sym;
        r.ftab_off = (uint32_t)align_up(r.route_off + r.n_sym, 4);
        r.index_off = align_up(r.layout == 3 ? r.ftab_off + 16ull * r.n_sym : r.ftab_off + (r.layout == 2 ? 8ull : 256ull) * r.n_tables, 16);
        if (r.index_off + 16ull * r.n_chunks + 4ull * (r.S - 1) * r.n_chunks > r.rec_len) {
            set_error("record %u: chunk index or stream table out of bounds", i);
            return BS_E_FORMAT;
        }
        uint64_t sum = 0;
        int last = -1;
        for (uint32_t k = 0; k < r.n_sym; k++) {
            const uint32_t s = rd16(b + r.stab_off + 4 * k), q = rd16(b + r.stab_off + 4 * k + 2);
            if ((int)s <= last || s >= 512 || q == 0 || b[r.route_off + k] > r.n_tables) {
                set_error("record %u: bad sign/exponent table", i);
                return BS_E_FORMAT;
            }
            last = (int)s;
            sum += q;
        }
        if (r.n_sym && sum != (1ull << r.m_s)) { set_error("record %u: sign/exponent frequencies do not sum to 2^%u", i, r.m_s); return BS_E_FORMAT; }
        if (r.layout == 3) {
            uint64_t ts = 0;
            for (uint32_t k = 0; k < 8 * r.n_sym; k++) ts += rd16(b + r.ftab_off + 2 * k);
            if (r.n_sym && ts != (1ull << kMt)) { set_error("record %u: joint frequencies do not sum to 2^%u", i, kMt); return BS_E_FORMAT; }
        }
        for (uint32_t t = 0; t < r.n_tables; t++) {
            uint64_t fs = 0;
            if (r.layout == 2) {
                for (uint32_t h = 0; h < 8; h++) fs += b[r.ftab_off + 8 * t + h];
            } else {
                for (uint32_t f = 0; f < 128; f++) fs += rd16(b + r.ftab_off + 256 * t + 2 * f);
            }
            if (fs != (1ull << r.m_f)) { set_error("record %u: fraction table %u does not sum to 2^%u", i, t + 1, r.m_f); return BS_E_FORMAT; }
        }
        const uint32_t P = K / r.S;
        const uint8_t* stab = b + r.index_off + 16ull * r.n_chunks;
        for (uint32_t ch = 0; ch < r.n_chunks; ch++) {
            const uint8_t* e = b + r.index_off + 16ull * ch;
            const uint64_t po = rd64(e);
            const uint64_t total = rd32(e + 8);
            // layouts 2 and 3: the plane of low fraction bits sits between the codes and the streams
            const uint64_t n_c = std::min<uint64_t>(r.W, r.n - (uint64_t)ch * r.W);
            const uint64_t cbytes = code_bytes(K) + (r.layout >= 2 ? plane_bytes(n_c) : 0);
            // the payload (codes and stream area, padded to 16 bytes) within
            // the record; the streams' starts ascend within the area and each
            // stream holds at least its state bits
            bool ok = po % 16 == 0 && po <= r.rec_len && align_up(cbytes + 2 * total, 16) <= r.rec_len - po;
            for (uint32_t st = 0; ok && st < r.S; st++) {
                const uint64_t from = st ? rd32(stab + 4ull * ((r.S - 1) * ch + st - 1)) : 0;
                const uint64_t to = st + 1 < r.S ? rd32(stab + 4ull * ((r.S - 1) * ch + st)) : total;
                uint64_t esum = 0;
                for (uint32_t l = st * P; l < (st + 1) * P; l++) esum += (b[po + l / 2] >> (4 * (l % 2))) & 15u;
                ok = from <= to && to <= total && state_units(P, esum) <= to - from;
            }
            if (!ok) {
                set_error("record %u chunk %u: payload out of bounds", i, ch);
                return BS_E_FORMAT;
            }
        }
        r.chunk_base = c.n_chunks;
        c.n_chunks += r.n_chunks;
        r.stream_base = c.n_streams;
        c.n_streams += (uint64_t)r.n_chunks * r.S;
    }
    if (out_end > c.out_len) { set_error("records extend past the declared output length"); return BS_E_FORMAT; }
    return BS_OK;
}

}  // namespace bs

using namespace bs;

extern "C" {

bs_status bs_encode_host(const bs_tensor* tensors, uint32_t n_tensors, const bs_params* p, bs_blob** out) {
    if (!out || (!tensors && n_tensors)) { set_error("NULL argument"); return BS_E_INVAL; }
    if (!params_ok(p)) return BS_E_INVAL;
    std::vector<EncRecord> recs(n_tensors);
    try {
        // models and record shapes
        for (uint32_t i = 0; i < n_tensors; i++) {
            const bs_tensor& t = tensors[i];
            EncRecord& r = recs[i];
            r.kind = t.kind;
            r.n = t.n;
            r.data = (const uint8_t*)t.h_data;
            if ((t.kind != BS_KIND_BF16 && t.kind != BS_KIND_RAW) || (!t.h_data && t.n)) {
                set_error("tensor %u: bad kind or NULL data", i);
                return BS_E_INVAL;
            }
            if (t.kind == BS_KIND_RAW) continue;
            if (t.tables) {
                if (t.tables->n != t.n || t.tables->m_s != p->m_s || t.tables->m_f != p->m_f ||
                    t.tables->layout != p->layout) {
                    set_error("tensor %u: model was built for other data or parameters", i);
                    return BS_E_INVAL;
                }
                r.md = t.tables;
            } else {
                bs_tables* tb = nullptr;
                bs_status rc = bs_build_tables_host((const uint16_t*)t.h_data, t.n, p, &tb);
                if (rc) return rc;
                r.owned = *tb;
                bs_tables_free(tb);
                r.md = &r.owned;
            }
            if (r.md->n_sym > kMaxSyms) {   // too many distinct symbols: keep the bytes verbatim
                r.kind = BS_KIND_RAW;
                r.n = 2 * t.n;
                continue;
            }
            record_shape(t.n, p->chunk_weights, p->lanes, r.W, r.K);
            const uint32_t P = p->stream_lanes ? std::min(p->stream_lanes, r.K) : r.K;
            r.S = r.K / P;
            r.n_chunks = (uint32_t)(t.n ? (t.n + r.W - 1) / r.W : 0);
            make_enc(*r.md, r.em);
            build_head(r);
            r.chunks.resize(r.n_chunks);
        }
        // digests and chunks, in parallel
        struct Job { uint32_t rec; int32_t chunk; };  // chunk = -1: digest
        std::vector<Job> jobs;
        for (uint32_t i = 0; i < n_tensors; i++) {
            if (tensors[i].sha256) memcpy(recs[i].sha, tensors[i].sha256, 32);
            else jobs.push_back({i, -1});
            for (uint32_t ch = 0; ch < recs[i].n_chunks; ch++) jobs.push_back({i, (int32_t)ch});
        }
        const uint32_t threads = pick_threads(p->threads);
        parallel_for(jobs.size(), threads, [&](uint64_t k) {
            thread_local std::vector<uint16_t> buf;
            const Job& jb = jobs[k];
            EncRecord& r = recs[jb.rec];
            if (jb.chunk < 0) {
                sha256(r.data, r.kind == BS_KIND_BF16 ? 2 * r.n : r.n, r.sha);
                return;
            }
            const uint64_t c0 = (uint64_t)jb.chunk * r.W;
            const uint32_t n_c = (uint32_t)std::min<uint64_t>(r.W, r.n - c0);
            if (buf.size() < 2ull * n_c) buf.resize(2ull * n_c);
            ChunkOut& co = r.chunks[jb.chunk];
            co.states.resize(r.K);
            co.words.resize(r.S);
            const uint32_t P = r.K / r.S;
            co.mu.resize(r.S);
            const uint16_t* wc = (const uint16_t*)r.data + c0;
            if (r.em.layout >= 2) {
                // the plane of low fraction bits, padded to 16 bytes
                co.plane.assign(align_up((n_c + 7) / 8, 4), 0u);
                for (uint32_t j = 0; j < n_c; j++) co.plane[j / 8] |= (wc[j] & 15u) << low_bit_pos(j % 8);
            }
            for (uint32_t st = 0; st < r.S; st++) {
                const uint64_t nw = r.em.layout >= 2
                                        ? encode_stream2(r.em, wc, n_c, r.K, st * P, (st + 1) * P, co.states.data(), buf.data())
                                        : encode_stream(r.em, wc, n_c, r.K, st * P, (st + 1) * P, co.states.data(), buf.data());
                std::vector<uint16_t>& v = co.words[st];
                v.resize(nw);
                for (uint64_t i = 0; i < nw; i++) v[i] = buf[nw - 1 - i];
                uint64_t esum = 0;
                for (uint32_t l = st * P; l < (st + 1) * P; l++) esum += state_code(co.states[l]);
                co.mu[st] = state_units(P, esum);
            }
        });
        // layout
        uint64_t pos = align_up(kHeaderBytes + kDirEntryBytes * n_tensors, 16);
        std::vector<uint64_t> rec_off(n_tensors), rec_len(n_tensors), out_off(n_tensors);
        uint64_t out_pos = 0, out_end = 0;
        for (uint32_t i = 0; i < n_tensors; i++) {
            EncRecord& r = recs[i];
            rec_off[i] = pos;
            uint64_t len = 0;
            if (r.kind == BS_KIND_RAW) {
                len = r.n;
            } else {
                len = r.head.size();
                for (uint32_t ch = 0; ch < r.n_chunks; ch++) {
                    const ChunkOut& co = r.chunks[ch];
                    wr64(r.head.data() + r.index_off + 16ull * ch, len);
                    wr32(r.head.data() + r.index_off + 16ull * ch + 8, (uint32_t)co.total());
                    uint64_t at = 0;
                    for (uint32_t st = 0; st < r.S; st++) {
                        if (st) wr32(r.head.data() + r.stab_off + 4ull * ((r.S - 1) * ch + st - 1), (uint32_t)at);
                        at += co.units(st);
                    }
                    len += payload_bytes(co, r.K);
                }
            }
            rec_len[i] = len;
            pos = align_up(pos + len, 16);
            out_off[i] = out_pos;
            const uint64_t ob = r.kind == BS_KIND_BF16 ? 2 * r.n : r.n;
            out_end = out_pos + ob;
            out_pos = align_up(out_pos + ob, kOutAlign);
        }
        bs_blob* blob = new bs_blob();
        blob->bytes.assign(pos, 0);
        uint8_t* c = blob->bytes.data();
        memcpy(c, kMagic, 8);
        wr32(c + 8, p->layout == 1 ? kVersion : p->layout == 2 ? kVersion2 : kVersion3);
        wr32(c + 12, n_tensors);
        wr64(c + 16, kHeaderBytes);
        wr64(c + 24, pos);
        wr64(c + 32, n_tensors ? out_end : 0);
        for (uint32_t i = 0; i < n_tensors; i++) {
            EncRecord& r = recs[i];
            uint8_t* d = c + kHeaderBytes + kDirEntryBytes * i;
            wr32(d, r.kind);
            wr64(d + 8, r.n);
            wr64(d + 16, out_off[i]);
            wr64(d + 24, rec_off[i]);
            wr64(d + 32, rec_len[i]);
            memcpy(d + 40, r.sha, 32);
            uint8_t* b = c + rec_off[i];
            if (r.kind == BS_KIND_RAW) {
                if (r.n) memcpy(b, r.data, r.n);
                continue;
            }
            memcpy(b, r.head.data(), r.head.size());
            const uint64_t sb = code_bytes(r.K);
            const uint32_t P = r.K / r.S;
            for (uint32_t ch = 0; ch < r.n_chunks; ch++) {
                const ChunkOut& co = r.chunks[ch];
                uint8_t* pp = b + rd64(r.head.data() + r.index_off + 16ull * ch);
                // length codes, then each stream: its lanes' state bits, then
                // its words (the buffer is zero-filled)
                for (uint32_t l = 0; l < r.K; l++) pp[l / 2] |= (uint8_t)(state_code(co.states[l]) << (4 * (l % 2)));
                for (uint64_t g = 0; g < co.plane.size(); g++) wr32(pp + sb + 4 * g, co.plane[g]);
                uint8_t* area = pp + sb + 4 * co.plane.size();
                for (uint32_t st = 0; st < r.S; st++) {
                    uint64_t moff = 0;
                    for (uint32_t l = st * P; l < (st + 1) * P; l++) {
                        const uint32_t x = co.states[l], len = 16 + state_code(x);
                        const uint64_t v = (uint64_t)(x - (1u << len)) << (moff % 8);
                        for (uint32_t k = 0; k * 8 < (moff % 8) + len; k++) area[moff / 8 + k] |= (uint8_t)(v >> (8 * k));
                        moff += len;
                    }
                    uint8_t* wp = area + 2 * co.mu[st];
                    for (uint64_t k = 0; k < co.words[st].size(); k++) wr16(wp + 2 * k, co.words[st][k]);
                    area += 2 * co.units(st);
                }
            }
        }
        // the decoded extent ends with the last record (the last record may not be the largest offset)
        uint64_t ext = 0;
        for (uint32_t i = 0; i < n_tensors; i++)
            ext = std::max(ext, out_off[i] + (recs[i].kind == BS_KIND_BF16 ? 2 * recs[i].n : recs[i].n));
        wr64(c + 32, ext);
        *out = blob;
    } catch (const std::bad_alloc&) {
        set_error("out of host memory");
        return BS_E_NOMEM;
    }
    return BS_OK;
}

const void* bs_blob_data(const bs_blob* b) { return b ? b->bytes.data() : nullptr; }
uint64_t bs_blob_size(const bs_blob* b) { return b ? b->bytes.size() : 0; }
void bs_blob_free(bs_blob* b) { delete b; }

bs_status bs_container_info_get(const void* h, uint64_t len, bs_container_info* info) {
    if (!info) { set_error("NULL info"); return BS_E_INVAL; }
    Container c;
    bs_status rc = parse_container((const uint8_t*)h, len, c);
    if (rc) return rc;
    memset(info, 0, sizeof(*info));
    info->version = rd32((const uint8_t*)h + 8);
    info->n_records = c.n_records;
    info->total_len = c.total_len;
    info->out_len = c.out_len;
    info->n_chunks = c.n_chunks;
    info->n_streams = c.n_streams;
    // bytes charged to BF16 records: everything except the verbatim records
    // and their directory entries (header and padding go to the BF16 side)
    uint64_t raw = 0, n_raw = 0;
    for (const Record& r : c.recs) {
        if (r.kind == BS_KIND_BF16) info->bf16_weights += r.n;
        else { raw += r.rec_len; n_raw++; }
    }
    info->raw_bytes = raw;
    info->bf16_bytes = info->bf16_weights ? len - raw - kDirEntryBytes * n_raw : 0;
    return BS_OK;
}

bs_status bs_record_info_get(const void* h, uint64_t len, uint32_t index, bs_record_info* info) {
    if (!info) { set_error("NULL info"); return BS_E_INVAL; }
    Container c;
    bs_status rc = parse_container((const uint8_t*)h, len, c);
    if (rc) return rc;
    if (index >= c.n_records) { set_error("record %u out of range", index); return BS_E_INVAL; }
    const Record& r = c.recs[index];
    memset(info, 0, sizeof(*info));
    info->kind = r.kind;
    info->chunk_weights = r.W;
    info->lanes = r.K;
    info->n_chunks = r.n_chunks;
    info->m_s = r.m_s;
    info->m_f = r.m_f;
    info->n_tables = r.n_tables;
    info->n_sym = r.n_sym;
    info->n = r.n;
    info->out_offset = r.out_offset;
    info->rec_offset = r.rec_offset;
    info->rec_len = r.rec_len;
    info->chunk_base = r.chunk_base;
    info->layout = r.kind == BS_KIND_BF16 ? r.layout : 0;
    memcpy(info->sha256, r.sha, 32);
    info->stream_base = r.stream_base;
    info->streams = r.S;
    return BS_OK;
}

bs_status bs_container_sizes_get(const void* hv, uint64_t len, bs_size_breakdown* out) {
    if (!out) { set_error("NULL breakdown"); return BS_E_INVAL; }
    Container c;
    bs_status rc = parse_container((const uint8_t*)hv, len, c);
    if (rc) return rc;
    memset(out, 0, sizeof(*out));
    const uint8_t* h = (const uint8_t*)hv;
    uint64_t raw = 0, n_raw = 0, bf16_len = 0;
    for (const Record& r : c.recs) {
        if (r.kind != BS_KIND_BF16) {
            raw += r.rec_len;
            n_raw++;
            continue;
        }
        out->weights += r.n;
        bf16_len += r.rec_len;
        const uint8_t* b = h + r.rec_offset;
        out->fixed_bits += 8 * 24;
        out->table_bits += 8 * (r.index_off - 24);
        // the chunk index and stream table, with the padding up to the first payload
        const uint64_t first = r.n_chunks ? rd64(b + r.index_off) : r.rec_len;
        out->index_bits += 8 * (first - r.index_off);
        const uint32_t P = r.K / r.S;
        const uint8_t* stab = b + r.index_off + 16ull * r.n_chunks;
        uint64_t used = 8 * first;
        for (uint32_t ch = 0; ch < r.n_chunks; ch++) {
            const uint8_t* e = b + r.index_off + 16ull * ch;
            const uint64_t po = rd64(e), total = rd32(e + 8);
            const uint64_t n_c = std::min<uint64_t>(r.W, r.n - (uint64_t)ch * r.W);
            out->code_bits += 8 * code_bytes(r.K);
            used += 8 * code_bytes(r.K);
            if (r.layout >= 2) {
                out->plane_bits += 8 * plane_bytes(n_c);
                used += 8 * plane_bytes(n_c);
            }
            for (uint32_t st = 0; st < r.S; st++) {
                const uint64_t from = st ? rd32(stab + 4ull * ((r.S - 1) * ch + st - 1)) : 0;
                const uint64_t to = st + 1 < r.S ? rd32(stab + 4ull * ((r.S - 1) * ch + st)) : total;
                uint64_t esum = 0;
                for (uint32_t l = st * P; l < (st + 1) * P; l++) esum += (b[po + l / 2] >> (4 * (l % 2))) & 15u;
                const uint64_t sbits = 16ull * P + esum;
                out->state_bits += sbits;
                out->word_bits += 16 * (to - from - state_units(P, esum));
                used += sbits + 16 * (to - from - state_units(P, esum));
            }
        }
        out->pad_bits += 8 * r.rec_len - used;
    }
    if (out->weights == 0) {      // nothing is charged to BF16 weights (bs_container_info's bf16_bytes is 0)
        memset(out, 0, sizeof(*out));
        return BS_OK;
    }
    out->container_bits = 8 * (len - raw - kDirEntryBytes * n_raw - bf16_len);
    return BS_OK;
}

void bs_sha256(const void* h, uint64_t n, uint8_t out[32]) { sha256(h, n, out); }

bs_status bs_write_file_new(const char* path, const void* h, uint64_t n) {
    if (!path || (!h && n)) { set_error("NULL argument"); return BS_E_INVAL; }
    FILE* f = fopen(path, "wbx");   // 'x': fail if the file exists
    if (!f) {
        struct stat st;
        if (stat(path, &st) == 0) { set_error("%s already exists", path); return BS_E_EXISTS; }
        set_error("cannot create %s", path);
        return BS_E_INVAL;
    }
    const size_t w = n ? fwrite(h, 1, n, f) : 0;
    const int cl = fclose(f);
    if (w != n || cl != 0) { set_error("short write to %s", path); return BS_E_INVAL; }
    return BS_OK;
}

const char* bs_strerror(bs_status s) {
    switch (s) {
        case BS_OK: return "ok";
        case BS_E_INVAL: return "invalid argument";
        case BS_E_FORMAT: return "malformed container";
        case BS_E_VERSION: return "unsupported container version";
        case BS_E_NOSPACE: return "output buffer too small";
        case BS_E_NOMEM: return "out of memory";
        case BS_E_HIP: return "HIP runtime error";
        case BS_E_CORRUPT: return "corrupt data";
        case BS_E_MISMATCH: return "decoded bytes differ from the reference";
        case BS_E_EXISTS: return "output already exists";
    }
    return "unknown status";
}

const char* bs_last_error(void) { return last_error(); }
const char* bs_version(void) { return "bs 1.2 (container versions 1, 2 and 3, gfx950)"; }

}  // extern "C"

// ------------------------------------------------------------------ GPU encoder
//
// The same container as bs_encode_host, built from tensors in device memory:
// the models come from the HIP histogram (bs_build_tables) unless given, each
// record's streams are coded by encode_kernel into scratch, the host reads
// back the streams' word and state-bit counts and lays the container out
// exactly as the host encoder does, and assemble_kernel writes the payloads.

struct bs_dencoder {
    struct Rec {
        uint32_t kind = 0;
        uint64_t n = 0;                 // weights (BF16) or bytes (RAW)
        const uint8_t* d_data = nullptr;
        uint8_t sha[32];
        bs::Model model;
        bs::EncModel em;
        uint32_t W = 0, K = 0, S = 1, P = 1, n_chunks = 0;
        std::vector<uint8_t> head;
        uint64_t index_off = 0, stab_off = 0;
        uint64_t rec_off = 0, rec_len = 0, out_off = 0;
        uint64_t o_words = 0, o_states = 0, o_counts = 0, o_tab = 0, o_chunk = 0, o_start = 0, o_mu = 0;
        std::vector<uint64_t> chunk_off;
        std::vector<uint32_t> unit_start, unit_mu, counts;
    };
    std::vector<Rec> recs;
    std::vector<uint8_t> top;           // header and directory
    uint8_t* d_scratch = nullptr;
    uint64_t total_len = 0;
    hipEvent_t done = nullptr;
};

namespace {

bs_status denc_hip(hipError_t e, const char* what) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return e == hipErrorOutOfMemory ? BS_E_NOMEM : BS_E_HIP;
}

void fill_enc_tab(const bs::EncModel& em, bsd::EncTabDev& t) {
    memset(&t, 0, sizeof t);
    for (uint32_t s = 0; s < 512; s++) {
        t.s_qc[s] = em.s[s].q | em.s[s].cum << 16;
        t.route[s] = em.route[s];
    }
    if (em.layout == 3) {
        for (uint32_t k = 0; k < 512 * 8; k++) t.t_qc[k] = em.t[k].q | em.t[k].cum << 16;
        return;
    }
    if (em.layout == 2) {
        for (uint32_t k = 0; k <= bs::kMaxHTables; k++)
            for (uint32_t h = 0; h < 8; h++) t.h_qc[k * 8 + h] = em.h[k][h].q | em.h[k][h].cum << 16;
        return;
    }
    for (uint32_t k = 0; k <= bs::kMaxTables; k++)
        for (uint32_t f = 0; f < 128; f++) t.f_qc[k * 128 + f] = em.f[k][f].q | em.f[k][f].cum << 16;
}

bsd::EncArgs enc_args(const bs_dencoder* e, const bs_dencoder::Rec& r) {
    bsd::EncArgs a;
    memset(&a, 0, sizeof a);
    a.w = (const uint16_t*)r.d_data;
    a.n = r.n;
    a.W = r.W; a.K = r.K; a.S = r.S; a.P = r.P;
    a.n_chunks = r.n_chunks; a.m_s = r.em.m_s; a.m_f = r.em.m_f;
    a.layout = r.em.layout;
    a.tab = (const bsd::EncTabDev*)(e->d_scratch + r.o_tab);
    a.words = (uint16_t*)(e->d_scratch + r.o_words);
    a.states = (uint32_t*)(e->d_scratch + r.o_states);
    a.counts = (uint32_t*)(e->d_scratch + r.o_counts);
    a.chunk_off = (const uint64_t*)(e->d_scratch + r.o_chunk);
    a.unit_start = (const uint32_t*)(e->d_scratch + r.o_start);
    a.unit_mu = (const uint32_t*)(e->d_scratch + r.o_mu);
    return a;
}

}  // namespace

extern "C" {

bs_status bs_encode_device_begin(const bs_dtensor* tensors, uint32_t n_tensors, const bs_params* p, void* stream,
                                 bs_dencoder** out) {
    if (!out || (!tensors && n_tensors)) { set_error("NULL argument"); return BS_E_INVAL; }
    *out = nullptr;
    if (!params_ok(p)) return BS_E_INVAL;
    hipStream_t hs = (hipStream_t)stream;
    bs_dencoder* e = new (std::nothrow) bs_dencoder();
    if (!e) return BS_E_NOMEM;
    auto fail = [&](bs_status rc) { bs_encode_device_free(e); return rc; };
    try {
        e->recs.resize(n_tensors);
        uint64_t scratch = 0;
        auto take = [&](uint64_t bytes) { const uint64_t o = scratch; scratch = align_up(scratch + bytes, 256); return o; };
        for (uint32_t i = 0; i < n_tensors; i++) {
            const bs_dtensor& t = tensors[i];
            bs_dencoder::Rec& r = e->recs[i];
            r.kind = t.kind;
            r.n = t.n;
            r.d_data = (const uint8_t*)t.d_data;
            if ((t.kind != BS_KIND_BF16 && t.kind != BS_KIND_RAW) || (!t.d_data && t.n)) {
                set_error("tensor %u: bad kind or NULL data", i);
                return fail(BS_E_INVAL);
            }
            if (t.kind == BS_KIND_BF16 && ((uintptr_t)t.d_data & 15)) {
                set_error("tensor %u: BF16 data must be 16-B aligned", i);
                return fail(BS_E_INVAL);
            }
            const uint64_t nbytes = t.kind == BS_KIND_BF16 ? 2 * t.n : t.n;
            if (t.sha256) {
                memcpy(r.sha, t.sha256, 32);
            } else {                     // digest of a host copy (slow path)
                std::vector<uint8_t> h(nbytes);
                hipError_t he = nbytes ? hipMemcpy(h.data(), t.d_data, nbytes, hipMemcpyDeviceToHost) : hipSuccess;
                if (he != hipSuccess) return fail(denc_hip(he, "digest copy"));
                sha256(h.data(), nbytes, r.sha);
            }
            if (t.kind == BS_KIND_RAW) continue;
            if (t.tables) {
                if (t.tables->n != t.n || t.tables->m_s != p->m_s || t.tables->m_f != p->m_f ||
                    t.tables->layout != p->layout) {
                    set_error("tensor %u: model was built for other data or parameters", i);
                    return fail(BS_E_INVAL);
                }
                r.model = *t.tables;
            } else {
                bs_tables* tb = nullptr;
                const bs_status rc = bs_build_tables(t.d_data, t.n, p, stream, &tb);
                if (rc) return fail(rc);
                r.model = *tb;
                bs_tables_free(tb);
            }
            if (r.model.n_sym > kMaxSyms) {      // stored verbatim, as the host encoder does
                r.kind = BS_KIND_RAW;
                r.n = 2 * t.n;
                continue;
            }
            record_shape(t.n, p->chunk_weights, p->lanes, r.W, r.K);
            r.P = p->stream_lanes ? std::min(p->stream_lanes, r.K) : r.K;
            r.S = r.K / r.P;
            r.n_chunks = (uint32_t)(t.n ? (t.n + r.W - 1) / r.W : 0);
            make_enc(r.model, r.em);
            EncRecord er;                         // the record head, as the host encoder builds it
            er.md = &r.model;
            er.W = r.W; er.K = r.K; er.S = r.S; er.n_chunks = r.n_chunks;
            build_head(er);
            r.head = std::move(er.head);
            r.index_off = er.index_off;
            r.stab_off = er.stab_off;
            const uint64_t units = (uint64_t)r.n_chunks * r.S;
            r.o_words = take(4ull * r.W * r.n_chunks);
            r.o_states = take(4ull * r.K * r.n_chunks);
            r.o_counts = take(8 * units);
            r.o_tab = take(sizeof(bsd::EncTabDev));
            r.o_chunk = take(8ull * r.n_chunks);
            r.o_start = take(4 * units);
            r.o_mu = take(4 * units);
        }
        hipError_t he = hipMalloc(&e->d_scratch, std::max<uint64_t>(scratch, 256));
        if (he != hipSuccess) return fail(denc_hip(he, "encoder scratch"));
        he = hipEventCreateWithFlags(&e->done, hipEventDisableTiming);
        if (he != hipSuccess) return fail(denc_hip(he, "encoder event"));
        // code every stream
        std::vector<bsd::EncTabDev> tabs(n_tensors);
        for (uint32_t i = 0; i < n_tensors; i++) {
            bs_dencoder::Rec& r = e->recs[i];
            if (r.kind != BS_KIND_BF16 || r.n_chunks == 0) continue;
            fill_enc_tab(r.em, tabs[i]);
            he = hipMemcpyAsync(e->d_scratch + r.o_tab, &tabs[i], sizeof(bsd::EncTabDev), hipMemcpyHostToDevice, hs);
            if (he != hipSuccess) return fail(denc_hip(he, "encoder tables"));
            const bsd::EncArgs a = enc_args(e, r);
            const int ke = bsk_encode(&a, std::max<uint32_t>(1, r.P / 64), stream);
            if (ke) return fail(denc_hip((hipError_t)ke, "encode launch"));
            r.counts.resize(2ull * r.n_chunks * r.S);
            he = hipMemcpyAsync(r.counts.data(), e->d_scratch + r.o_counts, 4 * r.counts.size(), hipMemcpyDeviceToHost, hs);
            if (he != hipSuccess) return fail(denc_hip(he, "encoder counts"));
        }
        he = hipStreamSynchronize(hs);
        if (he != hipSuccess) return fail(denc_hip(he, "encode"));
        // layout, as bs_encode_host lays the container out
        uint64_t pos = align_up(kHeaderBytes + kDirEntryBytes * n_tensors, 16), out_pos = 0, ext = 0;
        for (uint32_t i = 0; i < n_tensors; i++) {
            bs_dencoder::Rec& r = e->recs[i];
            r.rec_off = pos;
            uint64_t len = 0;
            if (r.kind == BS_KIND_RAW) {
                len = r.n;
            } else {
                len = r.head.size();
                r.chunk_off.resize(r.n_chunks);
                r.unit_start.resize((uint64_t)r.n_chunks * r.S);
                r.unit_mu.resize((uint64_t)r.n_chunks * r.S);
                for (uint32_t ch = 0; ch < r.n_chunks; ch++) {
                    uint64_t at = 0;
                    for (uint32_t st = 0; st < r.S; st++) {
                        const uint64_t u = (uint64_t)ch * r.S + st;
                        const uint64_t mu = state_units(r.P, r.counts[2 * u + 1]);
                        if (st) wr32(r.head.data() + r.stab_off + 4ull * ((r.S - 1) * ch + st - 1), (uint32_t)at);
                        r.unit_start[u] = (uint32_t)at;
                        r.unit_mu[u] = (uint32_t)mu;
                        at += mu + r.counts[2 * u];
                    }
                    wr64(r.head.data() + r.index_off + 16ull * ch, len);
                    wr32(r.head.data() + r.index_off + 16ull * ch + 8, (uint32_t)at);
                    r.chunk_off[ch] = len;
                    const uint64_t n_c = std::min<uint64_t>(r.W, r.n - (uint64_t)ch * r.W);
                    len += align_up(code_bytes(r.K) + (r.em.layout >= 2 ? plane_bytes(n_c) : 0) + 2 * at, 16);
                }
            }
            r.rec_len = len;
            pos = align_up(pos + len, 16);
            r.out_off = out_pos;
            const uint64_t ob = r.kind == BS_KIND_BF16 ? 2 * r.n : r.n;
            ext = std::max(ext, out_pos + ob);
            out_pos = align_up(out_pos + ob, kOutAlign);
        }
        e->total_len = pos;
        e->top.assign(align_up(kHeaderBytes + kDirEntryBytes * n_tensors, 16), 0);
        uint8_t* c = e->top.data();
        memcpy(c, kMagic, 8);
        wr32(c + 8, p->layout == 1 ? kVersion : p->layout == 2 ? kVersion2 : kVersion3);
        wr32(c + 12, n_tensors);
        wr64(c + 16, kHeaderBytes);
        wr64(c + 24, pos);
        wr64(c + 32, n_tensors ? ext : 0);
        for (uint32_t i = 0; i < n_tensors; i++) {
            const bs_dencoder::Rec& r = e->recs[i];
            uint8_t* d = c + kHeaderBytes + kDirEntryBytes * i;
            wr32(d, r.kind);
            wr64(d + 8, r.n);
            wr64(d + 16, r.out_off);
            wr64(d + 24, r.rec_off);
            wr64(d + 32, r.rec_len);
            memcpy(d + 40, r.sha, 32);
        }
    } catch (const std::bad_alloc&) {
        set_error("out of host memory");
        return fail(BS_E_NOMEM);
    }
    *out = e;
    return BS_OK;
}

uint64_t bs_encode_device_size(const bs_dencoder* e) { return e ? e->total_len : 0; }

bs_status bs_encode_device_finish(bs_dencoder* e, void* d_out, uint64_t capacity, void* stream) {
    if (!e || !d_out) { set_error("NULL argument"); return BS_E_INVAL; }
    if ((uintptr_t)d_out & 15) { set_error("output must be 16-B aligned"); return BS_E_INVAL; }
    if (capacity < e->total_len) { set_error("capacity %llu < %llu", (unsigned long long)capacity, (unsigned long long)e->total_len); return BS_E_NOSPACE; }
    hipStream_t hs = (hipStream_t)stream;
    uint8_t* o = (uint8_t*)d_out;
    int ke = bsk_zero(o, e->total_len, stream);
    if (ke) return denc_hip((hipError_t)ke, "encoder zero fill");
    hipError_t he = hipMemcpyAsync(o, e->top.data(), e->top.size(), hipMemcpyHostToDevice, hs);
    for (bs_dencoder::Rec& r : e->recs) {
        if (he != hipSuccess) break;
        if (r.kind == BS_KIND_RAW) {
            if (r.n) he = hipMemcpyAsync(o + r.rec_off, r.d_data, r.n, hipMemcpyDeviceToDevice, hs);
            continue;
        }
        he = hipMemcpyAsync(o + r.rec_off, r.head.data(), r.head.size(), hipMemcpyHostToDevice, hs);
        if (he == hipSuccess && r.n_chunks)
            he = hipMemcpyAsync(e->d_scratch + r.o_chunk, r.chunk_off.data(), 8ull * r.n_chunks, hipMemcpyHostToDevice, hs);
        if (he == hipSuccess && r.n_chunks)
            he = hipMemcpyAsync(e->d_scratch + r.o_start, r.unit_start.data(), 4 * r.unit_start.size(), hipMemcpyHostToDevice, hs);
        if (he == hipSuccess && r.n_chunks)
            he = hipMemcpyAsync(e->d_scratch + r.o_mu, r.unit_mu.data(), 4 * r.unit_mu.size(), hipMemcpyHostToDevice, hs);
        if (he != hipSuccess) break;
        bsd::EncArgs a = enc_args(e, r);
        a.out = o + r.rec_off;
        ke = bsk_assemble(&a, stream);
        if (ke) return denc_hip((hipError_t)ke, "assemble launch");
    }
    if (he == hipSuccess) he = hipEventRecord(e->done, hs);
    if (he != hipSuccess) return denc_hip(he, "encoder finish");
    return BS_OK;
}

void bs_encode_device_free(bs_dencoder* e) {
    if (!e) return;
    if (e->done) {
        (void)hipEventSynchronize(e->done);      // the host buffers of finish's copies
        (void)hipEventDestroy(e->done);
    }
    if (e->d_scratch) {
        (void)hipDeviceSynchronize();
        (void)hipFree(e->d_scratch);
    }
    delete e;
}

}  // extern "C"
