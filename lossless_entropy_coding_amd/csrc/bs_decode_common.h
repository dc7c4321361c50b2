// bs_decode_common.h -- device pieces shared by the decode kernels of both
// record layouts (gfx950): the per-wave LDS ring of stream words, the
// wavefront refill, and opening a decode unit (one word stream of a chunk).
// Not part of the public C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bs_device.h"
#include "bs_wave.h"

namespace bsd {

typedef unsigned int v4o __attribute__((ext_vector_type(4)));   // 16 output bytes

// ------------------------------------------------------------------ decode

// Ring loads go through a buffer resource (gfx9 descriptor: raw 32-bit
// elements, no stride) whose base is the current stream position and whose
// size is what is left of the chunk's word area: the hardware range check
// returns zeros past the chunk's end, so the read-ahead never touches memory
// outside it.  The per-lane offset is a loop-invariant VGPR, so an in-flight
// load never pins a register that the loop overwrites.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const uint8_t* words, uint32_t bytes, uint32_t from) {
    // every input is wave-uniform; readfirstlane keeps the descriptor in SGPRs
    const uint64_t a = (uint64_t)(uintptr_t)(words + from);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t left = __builtin_amdgcn_readfirstlane(bytes > from ? bytes - from : 0u);
    const uint8_t* base = (const uint8_t*)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)left, 0x00020000);
}

__device__ __forceinline__ uint4 load_piece(__amdgpu_buffer_rsrc_t rs, uint32_t lane_off) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)lane_off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Per-wave ring of stream words in LDS: RW words (1024 to 4096, by lanes per
// thread and layout; topped up every RW / (256 R) positions) plus a 64-word
// copy of its head after its end, so that a
// refill of up to 64 consecutive words never wraps.  Words are refilled RW/2
// at a time (RW/1024 16-B pieces per lane), loaded one refill ahead.
template <uint32_t RW>
struct Ring {
    static constexpr uint32_t kPieces = RW / 1024;   // 16-B pieces per lane per refill
    uint16_t* base;       // LDS ring of this wave
    uint4 pf[kPieces];    // the next RW/2 words, in flight
    uint32_t fill;        // stream words written into the ring so far
    const uint8_t* words; // the chunk's word area (uniform)
    uint32_t bytes;       // its size, a multiple of 16
    uint32_t lane;
};

// Start the ring: issue the loads of the first RW/2 words (into `first`) and
// of the RW/2 after them (the prefetch); ring_commit writes `first` into LDS.
template <uint32_t RW>
__device__ __forceinline__ void ring_issue(Ring<RW>& g, uint32_t lane, uint4 (&first)[Ring<RW>::kPieces]) {
    g.lane = lane;
    const __amdgpu_buffer_rsrc_t rs = stream_rsrc(g.words, g.bytes, 0);
#pragma unroll
    for (uint32_t k = 0; k < Ring<RW>::kPieces; k++) first[k] = load_piece(rs, 16 * (64 * k + lane));
#pragma unroll
    for (uint32_t k = 0; k < Ring<RW>::kPieces; k++) g.pf[k] = load_piece(rs, 16 * (64 * (Ring<RW>::kPieces + k) + lane));
    g.fill = RW / 2;
}

template <uint32_t RW>
__device__ __forceinline__ void ring_commit(Ring<RW>& g, const uint4 (&first)[Ring<RW>::kPieces]) {
    uint4* r4 = (uint4*)g.base;
#pragma unroll
    for (uint32_t k = 0; k < Ring<RW>::kPieces; k++) r4[64 * k + g.lane] = first[k];
    if (g.lane < kRingMirror / 8) r4[RW / 8 + g.lane] = first[0];
}

// keep at least RW/2 words ahead of `pos` in the ring (uniform branch)
template <uint32_t RW>
__device__ __forceinline__ void ring_top_up(Ring<RW>& g, uint32_t pos) {
    if (g.fill - pos < RW / 2) {
        uint4* r4 = (uint4*)g.base;
        const uint32_t ro = (g.fill & (RW - 1)) >> 3;
#pragma unroll
        for (uint32_t k = 0; k < Ring<RW>::kPieces; k++) r4[ro + 64 * k + g.lane] = g.pf[k];
        if (ro == 0 && g.lane < kRingMirror / 8) r4[RW / 8 + g.lane] = g.pf[0];
        const __amdgpu_buffer_rsrc_t rs = stream_rsrc(g.words, g.bytes, 2 * g.fill);
#pragma unroll
        for (uint32_t k = 0; k < Ring<RW>::kPieces; k++)
            g.pf[k] = load_piece(rs, 16 * (64 * (Ring<RW>::kPieces + k) + g.lane));
        g.fill += RW / 2;
    }
}

// Renormalise the R groups of 64 lanes of one sub-step: lanes whose state
// fell below 2^16 take the next stream words, group 0 first and ascending lane
// order inside a group (a prefix count over the ballot).  Every lane reads
// its candidate word (always a valid ring index) and keeps it only if it
// needed one, so the R ring reads are in flight together.
template <int R, uint32_t RW>
__device__ __forceinline__ void refill_all(uint32_t (&x)[R], const bool (&active)[R], const Ring<RW>& g, uint32_t& pos) {
    uint32_t sel[R], w[R];
#pragma unroll
    for (int q = 0; q < R; q++) {
        const bool need = active[q] && x[q] < kStateLow;
        const uint64_t m = __builtin_amdgcn_ballot_w64(need);
        const uint32_t pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        // byte selector of the merge, chosen while the word is in flight:
        // (x << 16) | w for a refill, x unchanged otherwise
        sel[q] = need ? 0x05040100u : 0x07060504u;
        w[q] = g.base[(pos & (RW - 1)) + pre];
        pos += (uint32_t)__builtin_popcountll(m);
    }
#pragma unroll
    for (int q = 0; q < R; q++) x[q] = __builtin_amdgcn_perm(x[q], w[q], sel[q]);
}

// Waves that share a SIMD issue oldest first, so when a workgroup's waves all
// start together its youngest waves finish well after the oldest.  Giving the
// four waves of a SIMD the four issue priorities in turn, one macro-step each,
// lets them progress evenly.  That only pays when every wave has a single
// unit (the kernel then ends with the slowest wave); with several units per
// wave the default order is faster overall.
__device__ __forceinline__ void rotate_priority(uint32_t k) {
    switch (k & 3) {
        case 0: __builtin_amdgcn_s_setprio(0); break;
        case 1: __builtin_amdgcn_s_setprio(1); break;
        case 2: __builtin_amdgcn_s_setprio(2); break;
        default: __builtin_amdgcn_s_setprio(3); break;
    }
}

// inclusive prefix sum of v over the wave's lanes
__device__ __forceinline__ uint32_t wave_scan(uint32_t v) {
    const uint32_t lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t u = __shfl_up(v, d, 64);
        if (lane >= (uint32_t)d) v += u;
    }
    return v;
}

// One decode unit of a record: word stream st = u mod S of chunk ch = u / S,
// whose P lanes are lanes [st * P, st * P + P) of the chunk.  unit_open
// reads the chunk's index entry, the lanes' start states and the head of the
// stream into the wave's ring; unit_decode then decodes the unit (it needs
// the lookup tables in LDS).
template <int R, bool C>
struct Unit {
    const uint8_t* payload;        // the chunk's payload (length codes first)
    uint32_t x[R];                 // lane states
    Ring<ring_words(R, C)> g;
    uint32_t pos;                  // ring read position (stream words, from the 16-byte boundary)
    uint32_t skip;                 // ring units before the stream's first word (what precedes it, its state bits)
    uint32_t nw;                   // this stream's words
    uint32_t ch, st, n_c;          // chunk, stream, weights in the chunk
    uint32_t unit;
};

// L2: the record has layout 2, whose chunk payload holds the plane of low
// fraction bits between the length codes and the stream area; rb: LDS byte
// offset of the first wave's ring (after the lookup tables, uniform).
template <int R, bool C, bool L2>
__device__ __forceinline__ void unit_open(const DecodeArgs& a, const RecDev& r, uint32_t unit, uint32_t wave, uint8_t* lds,
                                          uint32_t rb, Unit<R, C>& u) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t ch = unit >> r.streams_log2;
    const uint32_t st = unit & ((1u << r.streams_log2) - 1);
    const uint32_t S = 1u << r.streams_log2;
    const uint8_t* body = a.container + r.body;
    // first read: the chunk's index entry (payload offset, 16-bit units of
    // its stream area) and, with several streams, the stream's start and end
    // units from the record's stream table
    const uint8_t* ent = body + r.index_off + 16ull * ch;
    const uint32_t* stab = (const uint32_t*)(body + r.index_off + 16ull * r.n_chunks) + (uint64_t)(S - 1) * ch;
    const uint64_t poff = *(const uint64_t*)ent;
    const uint32_t total = *(const uint32_t*)(ent + 8);
    uint32_t from = st ? stab[st - 1] : 0u;
    uint32_t to = st + 1 < S ? stab[st] : total;
    // (all wave-uniform; readfirstlane keeps the stream position and what
    // derives from it in scalar registers)
    const uint8_t* payload = body + (((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(poff >> 32)) << 32) |
                                     __builtin_amdgcn_readfirstlane((uint32_t)poff));
    from = __builtin_amdgcn_readfirstlane(from);
    to = __builtin_amdgcn_readfirstlane(to);
    const uint32_t K = r.K, P = r.P, LB = st * P;
    const uint64_t n_left = r.n - (uint64_t)ch * r.W;
    const uint32_t n_c = (uint32_t)(n_left < r.W ? n_left : r.W);
    // payload: the K lanes' length codes (a nibble each, padded to 16 bytes),
    // then the streams back to back, each its lanes' state bits (padded to a
    // 16-bit unit) and then its words.  Ring loads start at the 16-byte
    // boundary at or below the stream and may run to the boundary at or above
    // its end, which the payload's own padding covers; the first `skip` units
    // loaded belong to what comes before.
    const uint32_t code_bytes = (((K + 1) / 2 + 15) & ~15u) + (L2 ? ((4 * ((n_c + 7) / 8) + 15) & ~15u) : 0u);
    const uint32_t aoff = code_bytes + 2 * from;
    const uint32_t w16 = aoff & ~15u;
    const uint32_t skip = (aoff - w16) / 2;
    const uint32_t aend16 = (code_bytes + 2 * to + 15) & ~15u;

    // second read: the head of the stream into the ring, and the lanes'
    // length codes
    constexpr uint32_t RW = ring_words(R, C);
    Ring<RW>& g = u.g;
    g.base = (uint16_t*)(lds + rb + wave * ring_bytes(R, C));
    g.words = payload + w16;
    g.bytes = aend16 - w16;
    uint4 first[Ring<RW>::kPieces];
    ring_issue(g, lane, first);
    uint32_t e[R];
#pragma unroll
    for (int q = 0; q < R; q++) {
        const uint32_t l = 64 * q + lane, gl = LB + l;
        e[q] = l < P ? (payload[gl >> 1] >> (4 * (gl & 1))) & 15u : 0u;
    }
    ring_commit(g, first);

    // The state bits sit at the head of the stream, which is in the ring's
    // first half (at most 31 bits for each of up to 512 lanes, after at most
    // 7 skipped units): lane l's 16 + e bits start 16 l plus the codes of the
    // lanes before it into the stream, and a state is 1 << (16 + e) plus them.
    uint32_t (&x)[R] = u.x;
    uint32_t before = 0;
#pragma unroll
    for (int q = 0; q < R; q++) {
        const uint32_t l = 64 * q + lane;
        const uint32_t incl = wave_scan(e[q]);
        const uint32_t bit = 16 * l + before + (incl - e[q]);
        const uint32_t len = 16 + e[q];
        const uint32_t wi = skip + (bit >> 4), sh = bit & 15;
        const uint32_t w0 = g.base[wi], w1 = g.base[wi + 1], w2 = g.base[wi + 2];
        const uint32_t bits = __builtin_amdgcn_alignbit(w2, w0 | (w1 << 16), sh) & ((1u << len) - 1u);
        x[q] = l < P ? (1u << len) | bits : kStateLow;
        before += __builtin_amdgcn_readlane(incl, 63);
    }
    // units of state bits: 16 P plus the codes, rounded up
    const uint32_t mu = (16 * P + before + 15) / 16;
    __builtin_amdgcn_s_waitcnt(0);
    u.pos = skip + mu;
    u.skip = skip + mu;
    u.nw = to - from - mu;
    u.ch = ch;
    u.st = st;
    u.n_c = n_c;
    u.unit = unit;
    u.payload = payload;
}

// ------------------------------------------------------------------ fused product

// The fused product's epilogue for one group of 8 weights per lane (cnt of
// them present).  The wave's groups are 512 consecutive record elements from
// (row0, c0), 8 per lane in lane order, so with gcols >= 512 they span at most
// two matrix rows.  Each lane takes the dot product of its weights with the
// matching x (packed BF16 pairs, v_dot2 with fp32 accumulation), the wave
// sums the products per row (DPP steps, no LDS), and lane 0 adds the sums
// into y.
__device__ __forceinline__ void gemv_group(const DecodeArgs& a, const uint32_t (&o)[4], uint32_t cnt, uint64_t row0,
                                           uint32_t c0, uint32_t lane) {
    const uint32_t cols = (uint32_t)a.gcols;
    const uint32_t c = c0 + 8 * lane;
    const bool wrap = c >= cols;
    const uint32_t col = wrap ? c - cols : c;
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u xv = *(const v4u*)(a.gx + col);
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        // weights 2k and 2k + 1 of the group, the upper one dropped when absent
        const uint32_t w = 2 * k + 1 < (int)cnt ? o[k] : 2 * k < (int)cnt ? (o[k] & 0xFFFFu) : 0u;
        sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, xw[k]), sum,
                                              false);
    }
    const float s0 = wave_sum_dpp(wrap ? 0.f : sum);
    const float s1 = wave_sum_dpp(wrap ? sum : 0.f);
    const uint64_t wrapped = __builtin_amdgcn_ballot_w64(wrap && cnt > 0);
    const uint64_t here = __builtin_amdgcn_ballot_w64(!wrap && cnt > 0);
    if (lane == 0) {
        if (here) __hip_atomic_fetch_add(a.gy + row0, s0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (wrapped) __hip_atomic_fetch_add(a.gy + row0 + 1, s1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Matrix position (row, column) of a group start, advanced by whole groups
// without dividing (uniform values, kept in scalar registers).
struct MatPos {
    uint64_t row;
    uint32_t col;
    __device__ __forceinline__ void advance(uint32_t by, uint32_t cols) {
        col += by;
        while (col >= cols) { col -= cols; row++; }
    }
};

// the product of one group per lane group q of the macro-step that starts at p
template <int R>
__device__ __forceinline__ void gemv_step(const DecodeArgs& a, const uint32_t (&o)[R][4], const int32_t* cnt,
                                          MatPos p, uint32_t lane) {
    const uint32_t cols = (uint32_t)a.gcols;
#pragma unroll
    for (int q = 0; q < R; q++) {
        gemv_group(a, o[q], cnt ? (uint32_t)cnt[q] : 8u, p.row, p.col, lane);
        p.advance(512, cols);
    }
}

}  // namespace bsd
