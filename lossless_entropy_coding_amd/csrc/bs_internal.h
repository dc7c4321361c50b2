// bs_internal.h -- host-side internals of the codec library (not public).
#pragma once
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <string>
#include <thread>
#include <vector>

#include "bs.h"

namespace bs {

// container constants (the layout is documented in bs.h)
constexpr char kMagic[8] = {'B', 'F', '1', '6', 'R', 'A', 'N', 'S'};
constexpr uint32_t kVersion = 1;           // containers of layout-1 records
constexpr uint32_t kVersion2 = 2;          // containers that name each record's layout (1 or 2)
constexpr uint32_t kVersion3 = 3;          // the same with layout 3 allowed (1, 2 or 3)
constexpr uint64_t kHeaderBytes = 64;
constexpr uint64_t kDirEntryBytes = 96;
constexpr uint64_t kOutAlign = 256;
constexpr uint32_t kCandidates = 64;        // exponents whose fraction counts are gathered
constexpr uint32_t kMaxTables = 6;
constexpr uint32_t kMaxHTables = 31;       // coded h tables of a layout-2 record
constexpr uint32_t kMt = 13;               // precision of a layout-3 record's joint (s, h) table
constexpr uint32_t kMaxSyms = 256;

void set_error(const char* fmt, ...);
void sha256(const void* data, uint64_t n, uint8_t out[32]);

inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// host worker threads: `req`, or the hardware's count when 0
inline uint32_t pick_threads(uint32_t req) {
    uint32_t hw = std::thread::hardware_concurrency();
    if (!hw) hw = 4;
    return req ? req : hw;
}

// fn(i) for i in [0, n) on up to `threads` threads (the caller's included),
// items handed out one at a time
template <class F>
void parallel_for(uint64_t n, uint32_t threads, F&& fn) {
    std::atomic<uint64_t> next{0};
    auto body = [&]() {
        for (;;) {
            uint64_t i = next.fetch_add(1);
            if (i >= n) return;
            fn(i);
        }
    };
    const uint32_t nt = (uint32_t)std::min<uint64_t>(threads, std::max<uint64_t>(n, 1));
    std::vector<std::thread> pool;
    for (uint32_t k = 1; k < nt; k++) pool.emplace_back(body);
    body();
    for (auto& th : pool) th.join();
}

// little-endian field access
inline uint32_t rd16(const uint8_t* p) { return (uint32_t)p[0] | (uint32_t)p[1] << 8; }
inline uint32_t rd32(const uint8_t* p) { return rd16(p) | rd16(p + 2) << 16; }
inline uint64_t rd64(const uint8_t* p) { return (uint64_t)rd32(p) | (uint64_t)rd32(p + 4) << 32; }
inline void wr16(uint8_t* p, uint32_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
inline void wr32(uint8_t* p, uint32_t v) { wr16(p, v & 0xFFFF); wr16(p + 2, v >> 16); }
inline void wr64(uint8_t* p, uint64_t v) { wr32(p, (uint32_t)v); wr32(p + 4, (uint32_t)(v >> 32)); }

// Parsed view of one record (host side).
struct Record {
    uint32_t kind = 0;
    uint64_t n = 0, out_offset = 0, rec_offset = 0, rec_len = 0;
    uint8_t sha[32] = {0};
    // BF16 records
    uint32_t W = 0, K = 0, n_chunks = 0, m_s = 0, m_f = 0, n_tables = 0, n_sym = 0;
    uint32_t layout = 1;            // 2: s and h = f >> 4 coded, l = f & 15 in a plane (m_f holds M_h)
    uint32_t S = 1;                 // word streams per chunk (K / S lanes each)
    uint32_t stab_off = 0, route_off = 0, ftab_off = 0;
    uint64_t index_off = 0;
    uint64_t chunk_base = 0;
    uint64_t stream_base = 0;       // status index of the first stream
    uint64_t out_bytes() const { return kind == BS_KIND_BF16 ? 2 * n : n; }
};

struct Container {
    uint32_t n_records = 0;
    uint64_t total_len = 0, out_len = 0, n_chunks = 0, n_streams = 0;
    std::vector<Record> recs;
};

// Plan facts for other parts of the library (bs_plan.cpp).
uint64_t plan_device_bytes(const bs_plan* plan);   // device memory the plan allocated
uint64_t plan_status_words(const bs_plan* plan);   // status words a full decode writes
uint32_t plan_records(const bs_plan* plan);

// Validate h (len bytes) completely (header, directory, tables, chunk index
// and payload bounds) and fill c.  Returns BS_OK or an error with a message.
bs_status parse_container(const uint8_t* h, uint64_t len, Container& c);

}  // namespace bs

// Layout 2: bytes of a chunk's plane of low fraction bits (a u32 per group of
// 8 weights, padded to 16 B), and the bit of position p's low bits in it.
inline uint64_t plane_bytes(uint64_t n_c) { return bs::align_up(4 * ((n_c + 7) / 8), 16); }
inline uint32_t low_bit_pos(uint32_t p) { return 16 * (p & 1) + 4 * (p >> 1); }

// the library's opaque byte buffer
struct bs_blob {
    std::vector<uint8_t> bytes;
};
