// bs_device.h -- structures shared by the host side of the library and its
// HIP kernels (gfx950).  Not part of the public C ABI.
#pragma once
#include <stdint.h>

namespace bsd {

constexpr uint32_t kStateLow = 65536u;      // lower end of the rANS state interval
constexpr uint32_t kMaxTables = 6;          // coded fraction tables per record
constexpr uint32_t kMaxHTablesDev = 31;     // coded h tables per layout-2 record
constexpr uint32_t kMaxSyms = 256;          // occupied (sign, exponent) symbols per BF16 record

// Two LDS layouts of a decode workgroup (bytes):
//   full    (M_s <= 12, M_f <= 10): s lookup table, 2^M_s entries of 8 B, at 0
//           (32 KiB); fraction lookup tables in pages of 8 KiB from 32 KiB
//           (page t = table t, t = 0 flat, 1..6 coded; 2^M_f entries of 8 B);
//           then one stream ring per wave, 2048 words (4096 for eight lanes
//           per thread).  One 16-wave workgroup fills a CU's LDS.
//   compact (M_s <= 11, M_f <= 9): the s table in 16 KiB, pages of 4 KiB from
//           16 KiB, rings of 1024 words: 79,872 B, so that two 16-wave
//           workgroups share a CU.
constexpr uint32_t kRingMirror = 64;        // copy of the ring's first 64 words after its end
constexpr uint32_t kMaxWaves = 16;
constexpr uint32_t slut_bytes(bool compact) { return compact ? 16384u : 32768u; }
constexpr uint32_t fpage_bytes(bool compact) { return compact ? 4096u : 8192u; }
constexpr uint32_t lut_lds(bool compact) { return slut_bytes(compact) + (kMaxTables + 1) * fpage_bytes(compact); }

// ring size (16-bit words, a power of two), ring bytes and the workgroup cap
// for R lanes per thread.  A position consumes at most 2 * 64 * R words, and
// the ring is topped up to at least half full every top_up_every(R) positions,
// so it needs at least 256 * R words times that.  Checking less often than
// every position keeps the top-up (which waits for its prefetch) away from
// the positions right after an output store: on this hardware a wait for a
// load also waits for the stores issued after it.
constexpr uint32_t ring_words(uint32_t R, bool compact) { return compact ? 1024u : (R >= 8 ? 4096u : 2048u); }
constexpr uint32_t top_up_every(uint32_t R, bool compact) { return ring_words(R, compact) / (256u * R); }
constexpr uint32_t ring_bytes(uint32_t R, bool compact) { return (ring_words(R, compact) + kRingMirror) * 2u; }
constexpr uint32_t max_waves(uint32_t R) { return R >= 8 ? 8u : 16u; }
static_assert(top_up_every(4, true) >= 1 && top_up_every(4, false) >= 1 && top_up_every(8, false) >= 1 &&
              top_up_every(1, false) == 8 && top_up_every(1, true) == 4, "ring too small for one position");
static_assert(lut_lds(true) + 16 * ring_bytes(4, true) + 8 <= 81920, "compact layout must fit twice in 160 KiB");
static_assert(lut_lds(false) + 16 * ring_bytes(4, false) + 8 <= 163840, "full layout must fit in 160 KiB");
static_assert(lut_lds(false) + 8 * ring_bytes(8, false) + 8 <= 163840, "full layout must fit in 160 KiB");

// Layout 2 lookup-table image of one record (built once per plan), copied
// as it is to the start of the workgroup's LDS:
//   s part at 0: 2^M_s x 8 B {A, B}, A = q_s | P << 24 with P the LDS
//     address of the h page of route[s] divided by 2048, B = s | (slot -
//     cum_s) << 16 (s below bit 9, so the output word s << 7 | h << 4 comes
//     from one funnel shift of B and the h entry)
//   h part at 8 * 2^M_s: (n_tables + 1) pages of 2 KiB (page 0 flat).  A
//     page is indexed by the low 8 bits i of the state after the s step (not
//     by the M_h-bit slot alone): entry i = {q_h << (8 - M_h) | h << 29,
//     q_h * (i >> M_h) + (i mod 2^M_h) - cum_h} for the h whose interval holds
//     the slot i mod 2^M_h.  Then x -> q_h (x >> M_h) + slot - cum_h becomes
//     x -> (x >> 8) * (q_h << (8 - M_h)) + entry, whose operands fit the
//     24-bit multiply (x >> 8 < 2^24, q_h << (8 - M_h) <= 256), while x >> M_h
//     itself can need 27 bits: the state is not renormalised between s and h.
//   the waves' stream rings after the h part.
// The h entry of state x after the s step sits at LDS address
// ((A >> 16) + (x mod 256)) * 8.
constexpr uint32_t kHPageBytes = 2048;
constexpr uint32_t kLds2 = 163840 - 16;    // a layout-2 workgroup's LDS (the rest: two words of record lookup)
constexpr uint32_t l2_ring_base(uint32_t m_s, uint32_t n_tables) { return (8u << m_s) + (n_tables + 1) * kHPageBytes; }
// waves of a layout-2 workgroup whose records' rings start at `ring_base` at most
constexpr uint32_t l2_max_waves(uint32_t ring_base) {
    return ring_base >= kLds2 ? 0u : ((kLds2 - ring_base) / ring_bytes(4, false) < kMaxWaves ? (kLds2 - ring_base) / ring_bytes(4, false) : kMaxWaves);
}
static_assert(l2_max_waves(l2_ring_base(12, kMaxHTablesDev)) == 15 && l2_max_waves(l2_ring_base(11, kMaxHTablesDev)) == 16,
              "layout-2 workgroup sizes");

// Layout-3 lookup-table image (LDS of a workgroup, in this order):
//   joint part at 0: 2^13 x 8-byte entries, entry i for state slot i (the
//     state's low 13 bits) of the joint symbol t = 8 s + h with
//     cum_t <= i < cum_t + q_t:
//       {A = q_t, B = (s << 7 | h << 4) | (i - cum_t) << 16}
//     so one step is x -> q_t (x >> 13) + (B >> 16), and the low half of B is
//     the output word's high twelve bits; its address (x mod 2^13) * 8 is the
//     low 16 bits of x << 3.
//   s part at 65536: 2^M_s entries {q_s, s | (slot - cum_s) << 16} for the
//     lanes' last groups (s alone), as layout 2's s part without a page;
//   the waves' stream rings after it.
constexpr uint32_t kJointBits = 13;
constexpr uint32_t kJointBytes = 8u << kJointBits;
constexpr uint32_t l3_ring_base(uint32_t m_s) { return kJointBytes + (8u << m_s); }
static_assert(l2_max_waves(l3_ring_base(11)) == 16 && l2_max_waves(l3_ring_base(12)) == 15, "layout-3 workgroup sizes");

// Device lookup-table image of one record (built once per plan):
//   s part: 2^M_s x {A, B}
//     A = q_s | (page << 24), page = LDS address of the routed fraction table >> 11
//     (in the record's LDS layout)
//     B = s | (slot - cum_s) << 20
//   f part: (n_tables + 1) pages of fpage_bytes(compact), each 2^M_f x {F0, F1}
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
    uint32_t compact;       // 1: compact LDS layout (M_s <= 11, M_f <= 9, R <= 4)
    uint32_t n_sym;
    uint32_t stab_off;      // byte offset (from body) of the s-table
    uint32_t route_off;     // byte offset (from body) of the route bytes
    uint32_t ftab_off;      // byte offset (from body) of the fraction tables (layout 2: the h tables)
    uint32_t layout;        // 1; 2: s and h = f >> 4 coded (m_f holds M_h), l = f & 15 in a plane;
                            // 3: as 2 with s and h one joint symbol (m_f holds M_t = 13)
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
    // layouts 2 and 3: records of 1..small_units units are not cut into runs
    // but decoded `pack` to a workgroup, one after another, by the workgroups
    // after the runs' (small_units = 0: none)
    uint32_t small_units;
    uint32_t pack;
    RecDev one;             // the record itself when the launch has one (i1 = i0 + 1)
    // fused product with a vector (the kernel instances with V set): the
    // record is a row-major matrix of gcols columns; y[r] += sum over c of
    // W[r, c] x[c], accumulated in fp32 (y zeroed before the launch)
    const uint16_t* gx;     // x: gcols BF16 words, 16-B aligned
    float* gy;              // y: n / gcols floats
    uint64_t gcols;         // a multiple of 8, at least 512
};

}  // namespace bsd

// Launchers (bs_kernels.hip).  All return a hipError_t as int.
extern "C" {
// d_cf: 256 x 128 counters (exponent, fraction; both signs), d_cneg: 256 x 8
// counters (negative words per exponent e and high fraction bits h, at
// 8 e + h); both zeroed by the caller
int bsk_hist(const uint16_t* d_w, uint64_t n, unsigned long long* d_cf, unsigned long long* d_cneg, void* stream);
int bsk_build_luts(const uint8_t* d_container, const bsd::RecDev* d_recs, uint32_t n_recs, uint8_t* d_luts,
                   void* stream);
// variant 1, 2, 4 or 8: every record of the launch has that many lanes per
// thread; variant 0: a mix of 1 and 2; variant 3: a mix of 1, 2 and 4.
// compact: the records use the compact LDS layout (not with variant 8).
int bsk_decode(const bsd::DecodeArgs* args, uint32_t n_groups, uint32_t variant, bool compact, void* stream);
// layout-2 records: variant 1, 2 or 4 (every record of the launch has that
// many lanes per thread), 0 (a mix of 1 and 2) or 3 (a mix with 4)
int bsk_decode2(const bsd::DecodeArgs* args, uint32_t n_groups, uint32_t variant, void* stream);
// the same for layout-3 records
int bsk_decode3(const bsd::DecodeArgs* args, uint32_t n_groups, uint32_t variant, void* stream);
// the fused matrix-vector product of one record (full layout, variant 1, 2 or 4), y zeroed first
int bsk_gemv(const bsd::DecodeArgs* args, uint32_t n_groups, uint32_t variant, uint64_t rows, void* stream);
// the same for a layout-2 record, and for a layout-3 record
int bsk_gemv2(const bsd::DecodeArgs* args, uint32_t n_groups, uint32_t variant, uint64_t rows, void* stream);
int bsk_gemv3(const bsd::DecodeArgs* args, uint32_t n_groups, uint32_t variant, uint64_t rows, void* stream);
// fill n floats at y with 0 (a kernel, so that the work stays capturable)
int bsk_zero_f32(float* y, uint64_t n, void* stream);
int bsk_raw_copy(const uint8_t* d_container, const bsd::RawDev* d_raw, uint32_t n_raw, uint8_t* d_out,
                 uint64_t out_base, void* stream);
int bsk_compare(const uint8_t* a, const uint8_t* b, uint64_t n, unsigned long long* d_result /*2*/, void* stream);
int bsk_device_cus(int* cus);
}
