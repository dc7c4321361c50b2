// bs_decode2.hip -- the decode kernel (gfx950) for records of layouts 2 and 3.
//
// What is decoded [Qwen3.8-27B-BF16-NVLC-Lossless model card, codec
// paragraph]: each BF16 word w = s << 7 | f; the joint (sign, exponent)
// symbol s is rANS-coded with a per-tensor model and selects the
// distribution of the fraction.  In layout 2 the fraction f = h << 4 | l is
// split: its high three bits h are coded with the distribution s selects,
// its low four bits l sit verbatim in a plane of the chunk.  Per weight a
// lane decodes s, then h, from its 32-bit state, and only then renormalises:
// the two steps use at most 16 bits of the state (M_s + M_h = 16), so one
// 16-bit word restores it.
//
// One wavefront decodes one word stream of a chunk, as in layout 1: lane
// states in VGPRs, the record's tables in LDS, a per-wave LDS ring of stream
// words, one refill per weight addressed by a wavefront prefix count, the
// plane read one 32-bit word per lane and group, 128-bit output stores.  The
// instances with V set are the fused matrix-vector product: each group of 8
// decoded weights goes into a dot product with x instead of memory.
//
// Layout 3 (the instances with J set) decodes s and h as one joint symbol:
// one table read and one step per weight instead of two, whose entry also
// holds the output word's high twelve bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "bs_decode_common.h"
#include "bs_device.h"

using namespace bsd;

namespace {

// LDS of a workgroup (bytes): the record's table image as built (s table
// of 2^M_s 8-byte entries at 0, then its 2 KiB h pages, each indexed by the
// state's low 8 bits), then one stream ring per wave.  The image's size
// depends on M_s and the number of h tables, so the rings start at a
// per-record offset and the launch takes as many waves as fit.
struct Model2 {
    uint32_t m_s;
    uint32_t smask;    // 2^M_s - 1
};

// s entry {A = q_s | P << 24, B = s | (slot - cum_s) << 16}
__device__ __forceinline__ uint2 s_entry(const uint8_t* lds, uint32_t x, const Model2& md) {
    return *(const uint2*)(lds + ((x & md.smask) << 3));
}

// the s step: q_s (x >> M_s) + slot - cum_s
__device__ __forceinline__ uint32_t s_step(uint32_t x, uint2 e, const Model2& md) {
    return __umul24(x >> md.m_s, e.x) + (e.y >> 16);
}

// the h entry of state x (after the s step) in the page that e names: index
// (A >> 16) + (x mod 256), taken in one add whose operand selects pick the
// high half of A and the low byte of x (an ALU instruction only)
__device__ __forceinline__ uint2 h_entry(const uint8_t* lds, uint2 e, uint32_t x) {
    uint32_t i;
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:BYTE_0"
        : "=v"(i) : "v"(e.x), "v"(x));
    return *(const uint2*)(lds + (i << 3));
}

// the h step on the state after the s step: q_h (x >> M_h) + slot - cum_h,
// taken as (x >> 8) (q_h << (8 - M_h)) + entry so that both multiply
// operands fit 24 bits
__device__ __forceinline__ uint32_t h_step(uint32_t x, uint2 f) { return __umul24(x >> 8, f.x) + f.y; }

// Layout 3: the joint entry of state x, at LDS address (x mod 2^13) * 8,
// which is the low half of x << 3: one shift whose result keeps its low 16
// bits (an ALU instruction only).
__device__ __forceinline__ uint2 joint_entry(const uint8_t* lds, uint32_t x) {
    uint32_t a;
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD"
        : "=v"(a) : "v"(x));
    return *(const uint2*)(lds + a);
}

// the joint step: q_t (x >> 13) + slot - cum_t
__device__ __forceinline__ uint32_t joint_step(uint32_t x, uint2 e) { return __umul24(x >> kJointBits, e.x) + (e.y >> 16); }

// One group of 8 weights per lane group q, each the pair (s, h) (J: the
// joint symbol), with one renormalisation per weight.  o receives the words'
// high twelve bits, weight p at 16-bit half p of the four dwords.
template <int R, uint32_t RW, bool J>
__device__ __forceinline__ void group_pairs(uint32_t (&x)[R], uint32_t (&o)[R][4], const uint8_t* lds, const Model2& md,
                                            Ring<RW>& g, uint32_t& pos, const bool (&on)[R]) {
#pragma unroll
    for (int p = 0; p < 8; p++) {
        if (p % top_up_every(R, false) == 0) ring_top_up(g, pos);
        uint32_t w[R];
        if (J) {
            uint2 e[R];
#pragma unroll
            for (int q = 0; q < R; q++) e[q] = joint_entry(lds, x[q]);
#pragma unroll
            for (int q = 0; q < R; q++) {
                x[q] = joint_step(x[q], e[q]);
                w[q] = e[q].y;   // low half: s << 7 | h << 4
            }
        } else {
            uint2 e[R];
#pragma unroll
            for (int q = 0; q < R; q++) e[q] = s_entry(lds, x[q], md);
#pragma unroll
            for (int q = 0; q < R; q++) x[q] = s_step(x[q], e[q], md);
            uint2 f[R];
#pragma unroll
            for (int q = 0; q < R; q++) f[q] = h_entry(lds, e[q], x[q]);
#pragma unroll
            for (int q = 0; q < R; q++) {
                x[q] = h_step(x[q], f[q]);
                // low half: (s << 7) | (f.x >> 25), and f.x >> 25 = h << 4
                w[q] = __builtin_amdgcn_alignbit(e[q].y, f[q].x, 25);
            }
        }
        refill_all<R, RW>(x, on, g, pos);
#pragma unroll
        for (int q = 0; q < R; q++) {
            if (p & 1) o[q][p >> 1] = __builtin_amdgcn_perm(w[q], o[q][p >> 1], 0x05040100u);
            else o[q][p >> 1] = w[q];
            asm volatile("" : "+v"(o[q][p >> 1]));
        }
    }
}

// The plane's low bits of one group into its four output dwords: position p
// sits at bit 16 (p mod 2) + 4 (p div 2) of the plane word, and at bits 0..3
// of its 16-bit half in the output.
__device__ __forceinline__ void add_low_bits(uint32_t (&o)[4], uint32_t d) {
#pragma unroll
    for (int k = 0; k < 4; k++) o[k] |= (d >> (4 * k)) & 0x000F000Fu;
}

// status of one stream: every lane back at its start state (the leading one
// at bit max(16, 3c) over the h of its last group's c weights; 2^16 for a
// lane without weights), and exactly the stream's words consumed
__device__ __forceinline__ bool lane_bad(uint32_t x, bool has, uint32_t c) {
    const uint32_t lead = 3 * c > 16 ? 3 * c : 16u;
    return has ? ((x >> lead) != 1u || ((x - (1u << lead)) >> (3 * c)) != 0u) : x != kStateLow;
}

template <int R, bool V, bool J>
__device__ __forceinline__ void unit_decode2(const DecodeArgs& a, const RecDev& r, const uint8_t* lds, Unit<R, false>& u,
                                             bool fair) {
    // the s entries of the lanes' last groups: at 0 in layout 2, after the
    // joint entries in layout 3
    const uint8_t* lds_s = J ? lds + kJointBytes : lds;
    const uint32_t lane = threadIdx.x & 63;
    constexpr uint32_t RW = ring_words(R, false);
    Ring<RW>& g = u.g;
    uint32_t (&x)[R] = u.x;
    const uint32_t K = r.K, P = r.P, LB = u.st * P;
    const uint32_t n_c = u.n_c, ch = u.ch, unit = u.unit, nw = u.nw, skip = u.skip;
    const Model2 md{r.m_s, (1u << r.m_s) - 1};
    uint32_t pos = u.pos;
    uint8_t* out = a.out + (r.out_off - a.out_base) + 2ull * ch * r.W;
    // the fused product: matrix position of the stream's first group
    MatPos mpos{0, 0};
    if (V) {
        const uint64_t e = (uint64_t)ch * r.W + 8ull * LB;
        const uint64_t row = e / a.gcols;
        mpos.row = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(row >> 32)) << 32) |
                   __builtin_amdgcn_readfirstlane((uint32_t)row);
        mpos.col = __builtin_amdgcn_readfirstlane((uint32_t)(e - row * a.gcols));
    }

    // the plane of low bits: one 32-bit word per group, group t K + l for
    // lane l at macro-step t; loads past its end return 0
    const uint32_t groups = (n_c + 7) / 8;
    const uint32_t code_bytes = ((K + 1) / 2 + 15) & ~15u;
    const __amdgpu_buffer_rsrc_t plane = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(u.payload + code_bytes), (short)0, (int)((4 * groups + 15) & ~15u), 0x00020000);
    const uint32_t T = (groups + K - 1) / K;
    // A stream narrower than the wave (P < 64, one lane per thread) takes the
    // unrolled path too: lanes [P, 64) step on an idle state, never refill
    // and store nothing, and are put back to the idle state after it.
    const bool part = R == 1 && !V && P < 64;
    bool on[R];
#pragma unroll
    for (int q = 0; q < R; q++) on[q] = !part || lane < P;
    // full macro-steps: every lane has 8 weights and none is in its last group
    const uint32_t T_full = (P % 64 == 0 || part) ? n_c / (8 * K) : 0;
    // a whole chunk: the last macro-step is every lane's last group, of 8 weights
    const bool whole = T_full != 0 && T_full == T;
    const uint32_t T_main = T_full ? T_full - 1 : 0;

    const uint32_t prio0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);

    uint32_t d[R];
#pragma unroll
    for (int q = 0; q < R; q++) d[q] = __builtin_amdgcn_raw_buffer_load_b32(plane, 4 * (LB + 64 * q + lane), 0, 0);
    for (uint32_t t = 0; t < T_main; t++) {
        if (fair) rotate_priority(prio0 + t);
        uint32_t dn[R];
#pragma unroll
        for (int q = 0; q < R; q++)
            dn[q] = __builtin_amdgcn_raw_buffer_load_b32(plane, 4 * ((t + 1) * K + LB + 64 * q + lane), 0, 0);
        uint32_t o[R][4];
        group_pairs<R, RW, J>(x, o, lds, md, g, pos, on);
#pragma unroll
        for (int q = 0; q < R; q++) {
            add_low_bits(o[q], d[q]);
            if (!V && on[q]) {
                v4o* op = (v4o*)out + (uint64_t)t * K + LB + 64 * q + lane;
                __builtin_nontemporal_store(v4o{o[q][0], o[q][1], o[q][2], o[q][3]}, op);
            }
            d[q] = dn[q];
        }
        if (V) {
            gemv_step<R>(a, o, nullptr, mpos, lane);
            mpos.advance(8 * K, (uint32_t)a.gcols);
        }
    }
    if (whole) {
        // the last macro-step: every lane's last group, 8 weights of s alone;
        // their h come back from the state each lane ends in
        if (fair) rotate_priority(prio0 + T_main);
        uint32_t o[R][4];
#pragma unroll
        for (int p = 0; p < 8; p++) {
            if (p % top_up_every(R, false) == 0) ring_top_up(g, pos);
            uint2 e[R];
#pragma unroll
            for (int q = 0; q < R; q++) e[q] = s_entry(lds_s, x[q], md);
#pragma unroll
            for (int q = 0; q < R; q++) x[q] = s_step(x[q], e[q], md);
            refill_all<R, RW>(x, on, g, pos);
#pragma unroll
            for (int q = 0; q < R; q++) {
                const uint32_t w = e[q].y << 7;   // low half s << 7
                if (p & 1) o[q][p >> 1] = __builtin_amdgcn_perm(w, o[q][p >> 1], 0x05040100u);
                else o[q][p >> 1] = w;
            }
        }
        bool bad = false;
#pragma unroll
        for (int q = 0; q < R; q++) {
#pragma unroll
            for (int k = 0; k < 4; k++)
                o[q][k] |= ((x[q] >> (6 * k)) & 7u) << 4 | ((x[q] >> (6 * k + 3)) & 7u) << 20;
            add_low_bits(o[q], d[q]);
            if (!V && on[q]) {
                v4o* op = (v4o*)out + (uint64_t)T_main * K + LB + 64 * q + lane;
                __builtin_nontemporal_store(v4o{o[q][0], o[q][1], o[q][2], o[q][3]}, op);
            }
            if (on[q]) bad |= lane_bad(x[q], true, 8);
        }
        if (V) gemv_step<R>(a, o, nullptr, mpos, lane);
        const uint64_t badm = __builtin_amdgcn_ballot_w64(bad);
        if (lane == 0) a.status[r.status_base + unit] = (badm ? 1u : 0u) | (pos - skip != nw ? 2u : 0u);
        return;
    }

    // remaining macro-steps (partial chunks, lanes' last groups, fewer than
    // 64 lanes in the fused product): a lane takes part while it has weights;
    // in its last group it decodes s alone.  One position per iteration; each
    // lane's eight output words move through a 128-bit shift register.
#pragma unroll
    for (int q = 0; q < R; q++)
        if (!on[q]) x[q] = kStateLow;
    bool has[R];
    uint32_t clast[R];
#pragma unroll
    for (int q = 0; q < R; q++) {
        has[q] = 64 * q + lane < P && 8ull * (LB + 64 * q + lane) < n_c;
        clast[q] = 0;
    }
    for (uint32_t t = T_main; t < T; t++) {
        if (fair) rotate_priority(prio0 + t);
        int32_t cnt[R];
        bool fin[R];
        uint32_t o[R][4], dt[R];
#pragma unroll
        for (int q = 0; q < R; q++) {
            const uint32_t l = 64 * q + lane;
            const int64_t left = (int64_t)n_c - 8 * ((int64_t)t * K + LB + l);
            cnt[q] = l < P ? (int32_t)(left < 0 ? 0 : (left > 8 ? 8 : left)) : 0;
            fin[q] = cnt[q] > 0 && left - 8 * (int64_t)K <= 0;
            if (fin[q]) clast[q] = (uint32_t)cnt[q];
            dt[q] = t == T_main ? d[q] : __builtin_amdgcn_raw_buffer_load_b32(plane, 4 * (t * K + LB + l), 0, 0);
#pragma unroll
            for (int k = 0; k < 4; k++) o[q][k] = 0;
        }
#pragma unroll 1
        for (int p = 0; p < 8; p++) {
            if (p % top_up_every(R, false) == 0) ring_top_up(g, pos);
            bool act[R];
#pragma unroll
            for (int q = 0; q < R; q++) {
                act[q] = p < cnt[q];
                uint32_t xs = x[q];
                const uint2 e = s_entry(lds_s, xs, md);
                xs = s_step(xs, e, md);
                uint32_t xh, wh;
                if (J) {
                    const uint2 ej = joint_entry(lds, x[q]);
                    xh = joint_step(x[q], ej);
                    wh = ej.y;
                } else {
                    xh = xs;
                    const uint2 f = h_entry(lds, e, xh);
                    xh = h_step(xh, f);
                    wh = __builtin_amdgcn_alignbit(e.y, f.x, 25);
                }
                const uint32_t w = fin[q] ? e.y << 7 : wh;
                if (act[q]) x[q] = fin[q] ? xs : xh;
                // shift the 128-bit register right by 16 and insert w on top
                o[q][0] = __builtin_amdgcn_alignbit(o[q][1], o[q][0], 16);
                o[q][1] = __builtin_amdgcn_alignbit(o[q][2], o[q][1], 16);
                o[q][2] = __builtin_amdgcn_alignbit(o[q][3], o[q][2], 16);
                o[q][3] = __builtin_amdgcn_alignbit(w, o[q][3], 16);
            }
            refill_all<R, RW>(x, act, g, pos);
        }
#pragma unroll
        for (int q = 0; q < R; q++) {
            // after its last group a lane is back at its start state, whose
            // low 3c bits are the h of that group's weights
            if (fin[q]) {
#pragma unroll
                for (int k = 0; k < 8; k++)
                    if (k < cnt[q]) o[q][k >> 1] |= ((x[q] >> (3 * k)) & 7u) << (4 + 16 * (k & 1));
            }
            add_low_bits(o[q], dt[q]);
            const uint64_t g16 = (uint64_t)t * K + LB + 64 * q + lane;
            if (V) {
                // below, after the R groups
            } else if (cnt[q] == 8) {
                __builtin_nontemporal_store(v4o{o[q][0], o[q][1], o[q][2], o[q][3]}, (v4o*)out + g16);
            } else if (cnt[q] > 0) {
                uint16_t* o16 = (uint16_t*)out + 8 * g16;
#pragma unroll
                for (int k = 0; k < 8; k++)
                    if (k < cnt[q]) o16[k] = (uint16_t)(o[q][k >> 1] >> (16 * (k & 1)));
            }
        }
        if (V) {
            gemv_step<R>(a, o, cnt, mpos, lane);
            mpos.advance(8 * K, (uint32_t)a.gcols);
        }
    }
    bool bad = false;
#pragma unroll
    for (int q = 0; q < R; q++) bad |= lane_bad(x[q], has[q], clast[q]);
    const uint64_t badm = __builtin_amdgcn_ballot_w64(bad);
    if (lane == 0) a.status[r.status_base + unit] = (badm ? 1u : 0u) | (pos - skip != nw ? 2u : 0u);
}

// Stage one record's table image into LDS (all threads of the workgroup),
// as it is.  Each thread moves up to
// kStage2 16-byte pieces per round trip; the first batch's loads are issued
// before a wave opens its first unit, so that the two overlap.
constexpr int kStage2 = 8;

template <int R, bool V, bool J>
__device__ __forceinline__ void run_units2(const DecodeArgs& a, const RecDev& r, uint32_t u0, uint32_t u1, uint32_t wave,
                                           uint8_t* lds) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u* src = (const v4u*)(a.luts + r.lut_off);
    const uint32_t rb = J ? l3_ring_base(r.m_s) : l2_ring_base(r.m_s, r.n_tables);
    const uint32_t n16 = rb / 16;
    const uint32_t step = kStage2 * blockDim.x;
    v4u* dst = (v4u*)lds;
    v4u sv[kStage2];
#pragma unroll
    for (int k = 0; k < kStage2; k++) {
        const uint32_t i = threadIdx.x + k * blockDim.x;
        if (i < n16) sv[k] = src[i];
    }
    Unit<R, false> un;
    uint32_t u = u0 + wave;
    if (u < u1) unit_open<R, false, true>(a, r, u, wave, lds, rb, un);
#pragma unroll
    for (int k = 0; k < kStage2; k++) {
        const uint32_t i = threadIdx.x + k * blockDim.x;
        if (i < n16) dst[i] = sv[k];
    }
    for (uint32_t base = threadIdx.x + step; base < n16; base += step) {
        v4u t[kStage2];
#pragma unroll
        for (int k = 0; k < kStage2; k++) {
            const uint32_t i = base + k * blockDim.x;
            if (i < n16) t[k] = src[i];
        }
#pragma unroll
        for (int k = 0; k < kStage2; k++) {
            const uint32_t i = base + k * blockDim.x;
            if (i < n16) dst[i] = t[k];
        }
    }
    __syncthreads();
    for (; u < u1; u += a.waves) {
        if (u != u0 + wave) unit_open<R, false, true>(a, r, u, wave, lds, rb, un);
        unit_decode2<R, V, J>(a, r, lds, un, u1 - u0 <= a.waves);
    }
}

template <int G, bool V, bool J>
__device__ __forceinline__ void run_record2(const DecodeArgs& a, const RecDev& r, uint32_t u0, uint32_t wave, uint8_t* lds) {
    const uint32_t u1 = min(r.n_chunks << r.streams_log2, u0 + a.run);
    if (G == 1 || G == 2 || G == 4) {
        constexpr int R = (G == 1 || G == 2 || G == 4) ? G : 1;
        run_units2<R, V, J>(a, r, u0, u1, wave, lds);
    } else if (r.lanes_per_thread == 1) {
        run_units2<1, V, J>(a, r, u0, u1, wave, lds);
    } else if (G == 0 || r.lanes_per_thread == 2) {
        run_units2<2, V, J>(a, r, u0, u1, wave, lds);
    } else {
        run_units2<4, V, J>(a, r, u0, u1, wave, lds);
    }
}

// A pack: the small records (1..small_units units) of the launch whose rank
// among them is in [p * pack, p * pack + pack), each decoded with all its
// units at once after its table image is staged; the workgroup waits for one
// record's waves before it stages the next image over it.
template <int G, bool V, bool J>
__device__ __forceinline__ void run_pack(const DecodeArgs& a, uint32_t p, uint32_t wave, uint8_t* lds) {
    const uint32_t first = p * a.pack, last = first + a.pack;
    uint32_t rank = 0;
    for (uint32_t e = a.i0; e < a.i1 && rank < last; e++) {
        const uint32_t n_units = a.cls.start[e + 1] - a.cls.start[e];
        if (n_units == 0 || n_units > a.small_units) continue;
        if (rank++ < first) continue;
        const RecDev r = a.recs[a.cls.recs[e]];
        run_record2<G, V, J>(a, r, 0, wave, lds);
        __syncthreads();
    }
}

// Workgroup b decodes one run of units inside one record, as the layout-1
// kernel does (record lookup by a prefix sum over the records' run counts
// when the launch has several), or, past the runs, one pack of small records.
// G: the lanes per thread of every record (1, 2 or 4), 0 for a mix of 1 and
// 2, 3 for a mix that includes 4.  V: the fused product (one record, G = 1,
// 2 or 4).  J: layout-3 records.
template <int G, bool V, bool J>
__device__ __forceinline__ void decode_body(const DecodeArgs& a) {
    __shared__ __align__(16) uint8_t lds[kLds2];
    __shared__ uint32_t pick[2];
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t b = blockIdx.x;
    if (a.i1 - a.i0 == 1) {
        const uint32_t u0 = b * a.run;
        if (u0 >= (a.one.n_chunks << a.one.streams_log2)) return;
        run_record2<G, V, J>(a, a.one, u0, wave, lds);
        return;
    }
    constexpr uint32_t kPacked = UINT32_MAX - 1;
    if (wave == 0) {
        const uint32_t lane = threadIdx.x & 63;
        uint32_t carry = 0, e = UINT32_MAX, j = 0;
        for (uint32_t base = a.i0; base < a.i1; base += 64) {
            const uint32_t i = base + lane;
            uint32_t k = 0;
            if (i < a.i1) {
                const uint32_t n_units = a.cls.start[i + 1] - a.cls.start[i];
                // small records are in packs, not runs
                k = n_units <= a.small_units ? 0u : (n_units + a.run - 1) / a.run;
            }
            const uint32_t incl = wave_scan(k);
            const uint32_t excl = carry + incl - k;
            const unsigned long long hit = __ballot(k != 0 && excl <= b && b < excl + k);
            if (hit) {
                const int src = __ffsll(hit) - 1;
                e = __shfl(i, src, 64);
                j = b - __shfl(excl, src, 64);
                break;
            }
            carry += __shfl(incl, 63, 64);
        }
        // past the runs: pack b - (run count)
        if (e == UINT32_MAX && a.pack) { e = kPacked; j = b - carry; }
        if (lane == 0) { pick[0] = e; pick[1] = j; }
    }
    __syncthreads();
    const uint32_t e = __builtin_amdgcn_readfirstlane(pick[0]);
    if (e == UINT32_MAX) return;
    if (e == kPacked) {
        run_pack<G, V, J>(a, __builtin_amdgcn_readfirstlane(pick[1]), wave, lds);
        return;
    }
    const RecDev r = a.recs[a.cls.recs[e]];
    run_record2<G, V, J>(a, r, __builtin_amdgcn_readfirstlane(pick[1]) * a.run, wave, lds);
}

// the kernels: layout 2 (decode2_kernel) and layout 3 (decode3_kernel)
template <int G, bool V = false>
__global__ __launch_bounds__(1024) void decode2_kernel(const DecodeArgs a) { decode_body<G, V, false>(a); }

template <int G, bool V = false>
__global__ __launch_bounds__(1024) void decode3_kernel(const DecodeArgs a) { decode_body<G, V, true>(a); }

// the decode of a launch's records (J: layout 3) with the instance for its
// lanes per thread
template <int G, bool V, bool J>
void launch_one(dim3 grid, dim3 block, hipStream_t st, const DecodeArgs* args) {
    if (J) hipLaunchKernelGGL((decode3_kernel<G, V>), grid, block, 0, st, *args);
    else hipLaunchKernelGGL((decode2_kernel<G, V>), grid, block, 0, st, *args);
}

template <bool J>
int launch_decode2(const DecodeArgs* args, uint32_t n_groups, uint32_t variant, void* stream) {
    if (n_groups == 0) return 0;
    const dim3 grid(n_groups), block(64 * args->waves);
    hipStream_t st = (hipStream_t)stream;
    if (args->waves == 0 || args->waves > 16) return (int)hipErrorInvalidValue;
    switch (variant) {
        case 0: launch_one<0, false, J>(grid, block, st, args); break;
        case 3: launch_one<3, false, J>(grid, block, st, args); break;
        case 1: launch_one<1, false, J>(grid, block, st, args); break;
        case 2: launch_one<2, false, J>(grid, block, st, args); break;
        case 4: launch_one<4, false, J>(grid, block, st, args); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

// the fused product of one record: y zeroed, then the decode with V set
template <bool J>
int launch_gemv2(const DecodeArgs* args, uint32_t n_groups, uint32_t variant, uint64_t rows, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (rows) {
        const int e = bsk_zero_f32(args->gy, rows, stream);
        if (e) return e;
    }
    if (n_groups == 0) return (int)hipGetLastError();
    const dim3 grid(n_groups), block(64 * args->waves);
    if (args->waves == 0 || args->waves > 16) return (int)hipErrorInvalidValue;
    switch (variant) {
        case 1: launch_one<1, true, J>(grid, block, st, args); break;
        case 2: launch_one<2, true, J>(grid, block, st, args); break;
        case 4: launch_one<4, true, J>(grid, block, st, args); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

}  // namespace

extern "C" {

int bsk_decode2(const DecodeArgs* args, uint32_t n_groups, uint32_t variant, void* stream) {
    return launch_decode2<false>(args, n_groups, variant, stream);
}

int bsk_decode3(const DecodeArgs* args, uint32_t n_groups, uint32_t variant, void* stream) {
    return launch_decode2<true>(args, n_groups, variant, stream);
}

int bsk_gemv2(const DecodeArgs* args, uint32_t n_groups, uint32_t variant, uint64_t rows, void* stream) {
    return launch_gemv2<false>(args, n_groups, variant, rows, stream);
}

int bsk_gemv3(const DecodeArgs* args, uint32_t n_groups, uint32_t variant, uint64_t rows, void* stream) {
    return launch_gemv2<true>(args, n_groups, variant, rows, stream);
}

}  // extern "C"
