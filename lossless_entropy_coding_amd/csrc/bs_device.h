// bs_device.h -- structures shared by the host side of the library and its
// HIP kernels (gfx950).  Not part of the public C ABI.
#pragma once
#include <stdint.h>

namespace bsd {

constexpr uint32_t kStateLow = 65536u;      // lower end of the rANS state interval
constexpr uint32_t kMaxTables = 6;          // coded fraction tables per record
constexpr uint32_t kMaxSyms = 256;          // occupied (sign, exponent) symbols per BF16 record

// LDS layout of one decode workgroup (bytes).
//   [0, 32 KiB)            s lookup table: 2^M_s entries of 8 B (M_s <= 12)
//   [32 KiB, 88 KiB)       fraction lookup tables: page t (8 KiB) = table t,
//                          t = 0 flat, 1..6 coded; 2^M_f entries of 8 B (M_f <= 10)
//   [88 KiB, ...)          one stream ring per wave
constexpr uint32_t kSlutOff = 0;
constexpr uint32_t kFlutOff = 32768;
constexpr uint32_t kFPage = 8192;
constexpr uint32_t kFPageShift = 13;
constexpr uint32_t kLutLds = kFlutOff + (kMaxTables + 1) * kFPage;   // 90112
constexpr uint32_t kRingMirror = 64;        // copy of the ring's first 64 words after its end
constexpr uint32_t kMaxWaves = 16;

// ring size (16-bit words, a power of two), ring bytes and the workgroup cap
// for R lanes per thread: 2048 words and 16 waves up to R = 4; 4096 words and
// 8 waves for R = 8 (it consumes up to 1024 words per weight position)
constexpr uint32_t ring_words(uint32_t R) { return R >= 8 ? 4096u : 2048u; }
constexpr uint32_t ring_bytes(uint32_t R) { return (ring_words(R) + kRingMirror) * 2u; }
constexpr uint32_t max_waves(uint32_t R) { return R >= 8 ? 8u : 16u; }

// Device lookup-table image of one record (built once per plan):
//   s part: 2^M_s x {A, B}
//     A = q_s | (page << 24), page = LDS address of the routed fraction table >> 11
//     B = s | (slot - cum_s) << 20
//   f part: (n_tables + 1) pages of 8 KiB, each 2^M_f x {F0, F1}
//     F0 = q_f | f << 25, F1 = slot - cum_f
struct RecDev {
    uint64_t body;          // byte offset of the record body in the container
    uint64_t index_off;     // byte offset of the chunk index from the body start
    uint64_t out_off;       // byte offset of the record in the full output
    uint64_t n;             // BF16 weights
    uint64_t lut_off;       // byte offset of the record's lookup-table image
    uint32_t W, K;          // weights per chunk, lanes
    uint32_t n_chunks;
    uint32_t status_base;   // status index of the first chunk's first stream
    uint32_t m_s, m_f;
    uint32_t n_tables;
    uint32_t lanes_per_thread;  // R = 1, 2, 4 or 8 (lanes per stream / 64, at least 1)
    uint32_t streams_log2;  // word streams per chunk = 2^streams_log2
    uint32_t P;             // lanes per stream (K >> streams_log2)
    uint32_t n_sym;
    uint32_t stab_off;      // byte offset (from body) of the s-table
    uint32_t route_off;     // byte offset (from body) of the route bytes
    uint32_t ftab_off;      // byte offset (from body) of the fraction tables
};

// One launch class of a plan (lanes per thread 1, 2 or 4; or 8): its BF16 records in container order
// and the running count of decode units (chunk streams) before each (n + 1
// entries).  Unit u of a record is stream u mod S of chunk u / S.
struct ClassDev {
    const uint32_t* recs;   // RecDev index of each record of the class
    const uint32_t* start;  // first class-wide unit of each record; start[n] = total
};

struct RawDev {
    uint64_t src;           // byte offset in the container
    uint64_t dst;           // byte offset in the full output
    uint64_t n;             // bytes
};

struct DecodeArgs {
    const uint8_t* container;
    const RecDev* recs;
    ClassDev cls;
    const uint8_t* luts;
    uint8_t* out;
    uint32_t* status;
    uint64_t out_base;      // output offset that maps to out[0]
    uint32_t i0, i1;        // class entries of the decoded records
    uint32_t run;           // units per workgroup (a run inside one record)
    uint32_t waves;         // waves per workgroup (rings allocated)
};

}  // namespace bsd

// Launchers (bs_kernels.hip).  All return a hipError_t as int.
extern "C" {
int bsk_hist_s(const uint16_t* d_w, uint64_t n, unsigned long long* d_cs, void* stream);
int bsk_hist_f(const uint16_t* d_w, uint64_t n, const int16_t* d_cand, unsigned long long* d_cf, void* stream);
int bsk_build_luts(const uint8_t* d_container, const bsd::RecDev* d_recs, uint32_t n_recs, uint8_t* d_luts,
                   void* stream);
// variant 1, 2, 4 or 8: every record of the launch has that many lanes per
// thread; variant 0: a mix of 1, 2 and 4
int bsk_decode(const bsd::DecodeArgs* args, uint32_t n_groups, uint32_t variant, void* stream);
int bsk_raw_copy(const uint8_t* d_container, const bsd::RawDev* d_raw, uint32_t n_raw, uint8_t* d_out,
                 uint64_t out_base, void* stream);
int bsk_compare(const uint8_t* a, const uint8_t* b, uint64_t n, unsigned long long* d_result /*2*/, void* stream);
int bsk_device_cus(int* cus);
}
