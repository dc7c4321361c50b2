// bs_decode.hip -- the decode kernel (gfx950) of the lossless BF16 weight codec.
//
// What is decoded [Qwen3.8-27B-BF16-NVLC-Lossless model card, codec
// paragraph]: each BF16 word w = s << 7 | f, where the joint (sign, exponent)
// symbol s is rANS-coded with a per-tensor model and the fraction f with the
// distribution selected by s.
//
// One wavefront decodes one word stream of a chunk: lane states in VGPRs,
// lookup tables in LDS, a per-wave LDS ring of stream words filled with
// coalesced 16-B loads, refills addressed by a wavefront prefix count over the
// lanes that need a word, 128-bit output stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "bs_decode_common.h"
#include "bs_device.h"
#include "bs_wave.h"

using namespace bsd;

namespace {

struct Model {
    const uint8_t* lds;
    uint32_t m_s, m_f;
    uint32_t smask8;      // (2^m_s - 1) << 3
    uint32_t fmask8;      // (2^m_f - 1) << 3
};

// decode the s symbol of one weight for one lane; returns the s-entry
__device__ __forceinline__ uint2 step_s(uint32_t& x, const Model& md) {
    const uint2 e = *(const uint2*)(md.lds + ((x << 3) & md.smask8));
    x = __umul24(x >> md.m_s, e.x) + (e.y >> 20);
    return e;
}

// decode the fraction with the table the s-entry routes to; returns w (low 16 bits)
__device__ __forceinline__ uint32_t step_f(uint32_t& x, const uint2 se, const Model& md) {
    // the s-entry's top byte is the fraction table's LDS address >> 11, and
    // its low 24 bits hold q_s <= 4096, so se.x >> 13 is that address exactly
    const uint32_t addr = ((x << 3) & md.fmask8) | (se.x >> 13);
    const uint2 e = *(const uint2*)(md.lds + addr);
    x = __umul24(x >> md.m_f, e.x) + e.y;
    return __builtin_amdgcn_alignbit(se.y, e.x, 25);
}

template <int R, bool C, bool V>
__device__ __forceinline__ void unit_decode(const DecodeArgs& a, const RecDev& r, uint8_t* lds, Unit<R, C>& u,
                                            bool fair) {
    const uint32_t lane = threadIdx.x & 63;
    constexpr uint32_t RW = ring_words(R, C);
    Ring<RW>& g = u.g;
    uint32_t (&x)[R] = u.x;
    const uint32_t K = r.K, P = r.P, LB = u.st * P;
    const uint32_t n_c = u.n_c, ch = u.ch, unit = u.unit, nw = u.nw, skip = u.skip;
    const Model md{lds, r.m_s, r.m_f, ((1u << r.m_s) - 1) << 3, ((1u << r.m_f) - 1) << 3};

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

    const uint32_t groups = (n_c + 7) / 8;
    const uint32_t T = (groups + K - 1) / K;
    // macro-steps in which every lane decodes 8 weights and none of them is in
    // the lane's last group (whose last weights keep their fractions in the
    // lane's start state, not in the stream): all full macro-steps but the last
    const uint32_t T_full = (P % 64 == 0) ? n_c / (8 * K) : 0;
    // A whole chunk of full waves: every lane's last group is the last
    // macro-step and holds 8 weights, so positions 4..7 of that macro-step
    // carry only s for every lane, and the main loop runs it too (for one
    // lane per thread, whose chunks are a few macro-steps long; the wider
    // instances keep a main loop without the extra case, which measured
    // faster for them).
    const bool whole = R == 1 && T_full != 0 && T_full == T;
    const uint32_t T_main = whole ? T_full : (T_full ? T_full - 1 : 0);

    bool all_on[R];
#pragma unroll
    for (int q = 0; q < R; q++) all_on[q] = true;

    // full macro-steps: every lane decodes 8 weights, one 128-bit store per lane group
    const uint32_t prio0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);   // wave / 4: rank on its SIMD
    for (uint32_t t = 0; t < T_main; t++) {
        if (fair) rotate_priority(prio0 + t);
        const bool last = whole && t + 1 == T_main;   // uniform
        uint32_t o[R][4];
#pragma unroll
        for (int p = 0; p < 8; p++) {
            if (p % top_up_every(R, C) == 0) ring_top_up(g, pos);
            uint2 se[R];
#pragma unroll
            for (int q = 0; q < R; q++) se[q] = step_s(x[q], md);
            refill_all<R, RW>(x, all_on, g, pos);
            uint32_t wv[R];
            if (p >= 4 && last) {
#pragma unroll
                for (int q = 0; q < R; q++) wv[q] = se[q].y << 7;   // s alone; the fraction is in the final state
            } else {
#pragma unroll
                for (int q = 0; q < R; q++) wv[q] = step_f(x[q], se[q], md);
                refill_all<R, RW>(x, all_on, g, pos);
            }
#pragma unroll
            for (int q = 0; q < R; q++) {
                if (p & 1) o[q][p >> 1] = __builtin_amdgcn_perm(wv[q], o[q][p >> 1], 0x05040100u);
                else o[q][p >> 1] = wv[q];
                // pack now: keeps the table entries of earlier positions dead
                // (otherwise the compiler sinks the packing to the store and
                // keeps 8 positions of entries live)
                asm volatile("" : "+v"(o[q][p >> 1]));
            }
        }
#pragma unroll
        for (int q = 0; q < R; q++) {
            if (last) {
                // every lane is back at its start state 2^28 plus four fractions
                o[q][2] |= (x[q] & 127u) | ((x[q] >> 7) & 127u) << 16;
                o[q][3] |= ((x[q] >> 14) & 127u) | ((x[q] >> 21) & 127u) << 16;
            }
            if (!V) {
                // non-temporal: the output is not read again by this kernel
                v4o* op = (v4o*)out + (uint64_t)t * K + LB + 64 * q + lane;
                __builtin_nontemporal_store(v4o{o[q][0], o[q][1], o[q][2], o[q][3]}, op);
            }
        }
        if (V) {
            gemv_step<R>(a, o, nullptr, mpos, lane);
            mpos.advance(8 * K, (uint32_t)a.gcols);
        }
    }
    if (whole) {
        bool bad = false;
#pragma unroll
        for (int q = 0; q < R; q++) bad |= (x[q] >> 28) != 1u;
        const uint64_t badm = __builtin_amdgcn_ballot_w64(bad);
        if (lane == 0) a.status[r.status_base + unit] = (badm ? 1u : 0u) | (pos - skip != nw ? 2u : 0u);
        return;
    }

    // remaining macro-steps (a lane's last group, partial groups, or fewer
    // than 64 lanes): lanes take part while they still have weights.  In its
    // last group of c weights a lane decodes only the s symbol of the last
    // m = min(4, c); their fractions are the low 7m bits of the state the lane
    // ends in, under a leading one at bit max(16, 7m).  One position per
    // iteration; each lane's eight output words move through a 128-bit shift
    // register.
    bool has[R];     // the lane has any weight in this chunk
    uint32_t mraw[R];
#pragma unroll
    for (int q = 0; q < R; q++) {
        has[q] = 64 * q + lane < P && 8ull * (LB + 64 * q + lane) < n_c;
        mraw[q] = 0;
    }
    for (uint32_t t = T_main; t < T; t++) {
        if (fair) rotate_priority(prio0 + t);
        int32_t cnt[R], raw0[R];
        bool fin[R];
        uint32_t o[R][4];
#pragma unroll
        for (int q = 0; q < R; q++) {
            const uint32_t l = 64 * q + lane;
            const int64_t left = (int64_t)n_c - 8 * ((int64_t)t * K + LB + l);
            cnt[q] = l < P ? (int32_t)(left < 0 ? 0 : (left > 8 ? 8 : left)) : 0;
            // the lane's last group is in this macro-step when the next one
            // has none of its weights
            fin[q] = cnt[q] > 0 && left - 8 * (int64_t)K <= 0;
            if (fin[q]) mraw[q] = cnt[q] < 4 ? (uint32_t)cnt[q] : 4u;
            raw0[q] = fin[q] ? cnt[q] - (int32_t)mraw[q] : 8;
#pragma unroll
            for (int k = 0; k < 4; k++) o[q][k] = 0;
        }
#pragma unroll 1
        for (int p = 0; p < 8; p++) {
            if (p % top_up_every(R, C) == 0) ring_top_up(g, pos);
            bool act_s[R], act_f[R];
            uint2 se[R];
#pragma unroll
            for (int q = 0; q < R; q++) {
                act_s[q] = p < cnt[q];
                act_f[q] = p < cnt[q] && p < raw0[q];
                uint32_t xs = x[q];
                se[q] = step_s(xs, md);
                if (act_s[q]) x[q] = xs;
            }
            refill_all<R, RW>(x, act_s, g, pos);
#pragma unroll
            for (int q = 0; q < R; q++) {
                uint32_t xs = x[q];
                uint32_t w = step_f(xs, se[q], md);
                if (act_f[q]) x[q] = xs;
                if (p >= raw0[q]) w = se[q].y << 7;   // s alone; the fraction comes from the final state
                // shift the 128-bit register right by 16 and insert w on top
                o[q][0] = __builtin_amdgcn_alignbit(o[q][1], o[q][0], 16);
                o[q][1] = __builtin_amdgcn_alignbit(o[q][2], o[q][1], 16);
                o[q][2] = __builtin_amdgcn_alignbit(o[q][3], o[q][2], 16);
                o[q][3] = __builtin_amdgcn_alignbit(w, o[q][3], 16);
            }
            refill_all<R, RW>(x, act_f, g, pos);
        }
#pragma unroll
        for (int q = 0; q < R; q++) {
            // after its last group a lane is back at its start state: put the
            // fractions it holds into the words of the group's last weights
            if (fin[q]) {
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    const int32_t i = k - raw0[q];
                    if (i >= 0 && k < cnt[q]) o[q][k >> 1] |= ((x[q] >> (7 * i)) & 127u) << (16 * (k & 1));
                }
            }
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

    // a stream is whole when every lane ends at the state its encoder
    // started from (the leading one over its m fractions and nothing else;
    // 2^16 for a lane without weights) and exactly the stream's words were
    // consumed
    bool bad = false;
#pragma unroll
    for (int q = 0; q < R; q++) {
        const uint32_t lead = mraw[q] > 2 ? 7 * mraw[q] : 16u;
        bad |= has[q] ? ((x[q] >> lead) != 1u || ((x[q] - (1u << lead)) >> (7 * mraw[q])) != 0u) : x[q] != kStateLow;
    }
    const uint64_t badm = __builtin_amdgcn_ballot_w64(bad);
    if (lane == 0) a.status[r.status_base + unit] = (badm ? 1u : 0u) | (pos - skip != nw ? 2u : 0u);
}

// Stage one record's lookup tables into LDS (all threads of the workgroup):
// the image's s part goes to the start of the LDS tables and its fraction
// pages after the s region.  Each thread moves up to kStageBatch 16-byte
// pieces per round trip, so that a 16-wave workgroup copies the largest image
// in one; the first batch's loads are issued before a wave opens its first
// unit, so that the two overlap.
constexpr int kStageBatch = 8;

// LDS piece of image piece i
__device__ __forceinline__ uint32_t stage_slot(uint32_t i, uint32_t ns16, uint32_t gap16) {
    return i < ns16 ? i : i + gap16;
}

// The units [u0, u1) of one record, taken by the workgroup's waves in turn.
// Every wave takes part in the staging and the barrier after it.
template <int R, bool C, bool V>
__device__ __forceinline__ void run_units(const DecodeArgs& a, const RecDev& r, uint32_t u0, uint32_t u1,
                                          uint32_t wave, uint8_t* lds) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));   // plain vector: stays in registers
    const v4u* src = (const v4u*)(a.luts + r.lut_off);
    const uint32_t ns16 = (8u << r.m_s) / 16;
    const uint32_t n16 = ns16 + (r.n_tables + 1) * (fpage_bytes(C) / 16);
    const uint32_t gap16 = slut_bytes(C) / 16 - ns16;
    const uint32_t step = kStageBatch * blockDim.x;
    v4u* d = (v4u*)lds;
    v4u sv[kStageBatch];
#pragma unroll
    for (int k = 0; k < kStageBatch; k++) {
        const uint32_t i = threadIdx.x + k * blockDim.x;
        if (i < n16) sv[k] = src[i];
    }
    Unit<R, C> un;
    uint32_t u = u0 + wave;
    if (u < u1) unit_open<R, C, false>(a, r, u, wave, lds, lut_lds(C), un);
#pragma unroll
    for (int k = 0; k < kStageBatch; k++) {
        const uint32_t i = threadIdx.x + k * blockDim.x;
        if (i < n16) d[stage_slot(i, ns16, gap16)] = sv[k];
    }
    for (uint32_t base = threadIdx.x + step; base < n16; base += step) {
        v4u t[kStageBatch];
#pragma unroll
        for (int k = 0; k < kStageBatch; k++) {
            const uint32_t i = base + k * blockDim.x;
            if (i < n16) t[k] = src[i];
        }
#pragma unroll
        for (int k = 0; k < kStageBatch; k++) {
            const uint32_t i = base + k * blockDim.x;
            if (i < n16) d[stage_slot(i, ns16, gap16)] = t[k];
        }
    }
    __syncthreads();
    for (; u < u1; u += a.waves) {
        if (u != u0 + wave) unit_open<R, C, false>(a, r, u, wave, lds, lut_lds(C), un);
        unit_decode<R, C, V>(a, r, lds, un, u1 - u0 <= a.waves);
    }
}

// The run of units starting at u0 of record r, with the lane width that the
// kernel instance G fixes or, for a mixed instance, the record's own.
template <int G, bool C, bool V>
__device__ __forceinline__ void run_record(const DecodeArgs& a, const RecDev& r, uint32_t u0, uint32_t wave,
                                           uint8_t* lds) {
    const uint32_t u1 = min(r.n_chunks << r.streams_log2, u0 + a.run);
    if (G == 1 || G == 2 || G == 4 || G == 8) {
        constexpr int R = (G == 1 || G == 2 || G == 4 || G == 8) ? G : 1;
        run_units<R, C, V>(a, r, u0, u1, wave, lds);
    } else if (r.lanes_per_thread == 1) {
        run_units<1, C, V>(a, r, u0, u1, wave, lds);
    } else if (G == 0 || r.lanes_per_thread == 2) {
        run_units<2, C, V>(a, r, u0, u1, wave, lds);
    } else {
        run_units<4, C, V>(a, r, u0, u1, wave, lds);
    }
}

// Workgroup b of a launch decodes one run of units (chunk streams) inside one
// record: each record r of the class entries [i0, i1) is cut into
// ceil(units_r / run) runs of `run` units (the last one shorter), and the runs
// are numbered in record order.  With one record the run is b; otherwise
// wave 0 finds b's record with a prefix sum over the records' run counts.
// The record's lookup tables are staged into LDS once and the waves then take
// the run's units in turn.
// One launch covers every record with 1, 2 or 4 lanes per thread (16-wave
// workgroups), so that small tensors decode alongside large ones: G is that
// lane width when all the launch's records share it, 0 for a mix of 1 and 2,
// or 3 for a mix that includes 4 (the width is then picked per workgroup; the
// narrower mix keeps the register count low enough for two workgroups per CU
// in the compact layout).  Records with eight lanes per thread (G = 8:
// 8 waves, 4096-word rings) have a launch of their own.
template <int G, bool C, bool V = false>
__global__ __launch_bounds__(G == 8 ? 512 : 1024) void decode_kernel(const DecodeArgs a) {
    // static allocation: the LDS base is a compile-time constant, so table and
    // ring addresses fold into the instructions' offsets
    constexpr uint32_t RMAX = G == 8 ? 8 : 1;   // ring size: one for 1, 2 and 4 lanes per thread, one for 8
    __shared__ __align__(16) uint8_t lds[lut_lds(C) + max_waves(RMAX) * ring_bytes(RMAX, C)];
    __shared__ uint32_t pick[2];
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t b = blockIdx.x;
    if (a.i1 - a.i0 == 1) {
        // one record, passed by value: no lookup before the tables
        const uint32_t u0 = b * a.run;
        if (u0 >= (a.one.n_chunks << a.one.streams_log2)) return;   // uniform over the workgroup
        run_record<G, C, V>(a, a.one, u0, wave, lds);
        return;
    }
    if (wave == 0) {
        const uint32_t lane = threadIdx.x & 63;
        uint32_t carry = 0, e = UINT32_MAX, j = 0;
        for (uint32_t base = a.i0; base < a.i1; base += 64) {
            const uint32_t i = base + lane;
            uint32_t k = 0;
            if (i < a.i1) k = (a.cls.start[i + 1] - a.cls.start[i] + a.run - 1) / a.run;
            uint32_t incl = k;
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t v = __shfl_up(incl, d, 64);
                if (lane >= (uint32_t)d) incl += v;
            }
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
        if (lane == 0) { pick[0] = e; pick[1] = j; }
    }
    __syncthreads();
    // the picked run is the same for every wave: keep it in scalar registers
    const uint32_t e = __builtin_amdgcn_readfirstlane(pick[0]);
    if (e == UINT32_MAX) return;   // no run for this workgroup (launch larger than the runs)
    const RecDev r = a.recs[a.cls.recs[e]];
    run_record<G, C, V>(a, r, __builtin_amdgcn_readfirstlane(pick[1]) * a.run, wave, lds);
}

// y = 0 before a fused product (a plain fill kernel, so that the enqueued
// work stays capturable)
__global__ void zero_f32_kernel(float* y, uint64_t n) {
    for (uint64_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += 256ull * gridDim.x) y[i] = 0.f;
}

}  // namespace

extern "C" {

int bsk_zero_f32(float* y, uint64_t n, void* stream) {
    if (n == 0) return 0;
    hipLaunchKernelGGL(zero_f32_kernel, dim3((uint32_t)std::min<uint64_t>((n + 255) / 256, 65535)), dim3(256), 0,
                       (hipStream_t)stream, y, n);
    return (int)hipGetLastError();
}

int bsk_decode(const DecodeArgs* args, uint32_t n_groups, uint32_t variant, bool compact, void* stream) {
    if (n_groups == 0) return 0;
    const dim3 grid(n_groups), block(64 * args->waves);
    hipStream_t st = (hipStream_t)stream;
    if (args->waves == 0 || args->waves > max_waves(variant == 8 ? 8 : 1)) return (int)hipErrorInvalidValue;
    if (compact) {
        switch (variant) {
            case 0: hipLaunchKernelGGL((decode_kernel<0, true>), grid, block, 0, st, *args); break;
            case 3: hipLaunchKernelGGL((decode_kernel<3, true>), grid, block, 0, st, *args); break;
            case 1: hipLaunchKernelGGL((decode_kernel<1, true>), grid, block, 0, st, *args); break;
            case 2: hipLaunchKernelGGL((decode_kernel<2, true>), grid, block, 0, st, *args); break;
            case 4: hipLaunchKernelGGL((decode_kernel<4, true>), grid, block, 0, st, *args); break;
            default: return (int)hipErrorInvalidValue;
        }
    } else {
        switch (variant) {
            case 0: hipLaunchKernelGGL((decode_kernel<0, false>), grid, block, 0, st, *args); break;
            case 3: hipLaunchKernelGGL((decode_kernel<3, false>), grid, block, 0, st, *args); break;
            case 1: hipLaunchKernelGGL((decode_kernel<1, false>), grid, block, 0, st, *args); break;
            case 2: hipLaunchKernelGGL((decode_kernel<2, false>), grid, block, 0, st, *args); break;
            case 4: hipLaunchKernelGGL((decode_kernel<4, false>), grid, block, 0, st, *args); break;
            case 8: hipLaunchKernelGGL((decode_kernel<8, false>), grid, block, 0, st, *args); break;
            default: return (int)hipErrorInvalidValue;
        }
    }
    return (int)hipGetLastError();
}

int bsk_gemv(const DecodeArgs* args, uint32_t n_groups, uint32_t variant, uint64_t rows, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (rows) {
        const int e = bsk_zero_f32(args->gy, rows, stream);
        if (e) return e;
    }
    if (n_groups == 0) return (int)hipGetLastError();
    const dim3 grid(n_groups), block(64 * args->waves);
    if (args->waves == 0 || args->waves > max_waves(1)) return (int)hipErrorInvalidValue;
    switch (variant) {
        case 1: hipLaunchKernelGGL((decode_kernel<1, false, true>), grid, block, 0, st, *args); break;
        case 2: hipLaunchKernelGGL((decode_kernel<2, false, true>), grid, block, 0, st, *args); break;
        case 4: hipLaunchKernelGGL((decode_kernel<4, false, true>), grid, block, 0, st, *args); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

}  // extern "C"
