// bs_encode.hip -- the GPU encoder's kernels (gfx950).
//
// The same container as the host encoder, byte for byte [Qwen3.8-27B-BF16-
// NVLC-Lossless model card, codec paragraph: the joint (sign, exponent)
// symbol is rANS-coded with a per-tensor model and selects the fraction's
// distribution; the chunk, lane and stream layout is this library's own and
// is given in bs.h].
//
// encode_kernel: one wavefront per word stream (P lanes of one chunk, R lanes
// per thread).  It runs the decode order backwards: macro-steps, positions
// and fields from last to first (fraction before sign/exponent), lanes from
// last to first inside each sub-step.  A lane that must flush before coding
// its symbol writes its low 16 bits; the flushing lanes of a sub-step take
// consecutive slots in that lane order (a ballot and a popcount of the
// higher lanes), so each stream's words come out in exactly the reverse of
// the order its decoder reads them.  Each lane starts from the state that
// carries its last fractions and ends in its final state.
//
// assemble_kernel: one wavefront per stream writes, at the offsets the host
// computed from the streams' word and state-bit counts, the chunk's length
// codes (stream 0's wave), the stream's state bits (packed in LDS) and its
// words in decode order.  The container is zero-filled first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "bs_device.h"
#include "bs_encode_device.h"

using namespace bsd;

namespace {

constexpr uint32_t kEncWaves = 4;

// code one symbol (q | cum << 16 in qc) into x; a flushing lane writes its low
// word at slot base + (flushing lanes above it); base advances for the wave
__device__ __forceinline__ void put_symbol(bool act, uint32_t& x, uint32_t qc, uint32_t M, uint16_t* sink,
                                           uint32_t& base, uint32_t lane) {
    const uint32_t q = qc & 0xFFFFu, cum = qc >> 16;
    const bool flush = act && (x >> (32 - M)) >= q;
    const uint64_t b = __builtin_amdgcn_ballot_w64(flush);
    if (flush) {
        const uint32_t above = (uint32_t)__builtin_popcountll(lane == 63 ? 0ull : b >> (lane + 1));
        sink[base + above] = (uint16_t)x;
        x >>= 16;
    }
    base += (uint32_t)__builtin_popcountll(b);
    if (act) x = ((x / q) << M) + x % q + cum;
}

template <int R>
__global__ __launch_bounds__(64 * kEncWaves) void encode_kernel(EncArgs a) {
    __shared__ uint32_t s_qc[512];
    __shared__ uint32_t f_qc[(kMaxTables + 1) * 128];
    __shared__ uint8_t route[512];
    for (uint32_t i = threadIdx.x; i < 512; i += 64 * kEncWaves) {
        s_qc[i] = a.tab->s_qc[i];
        route[i] = a.tab->route[i];
    }
    for (uint32_t i = threadIdx.x; i < (kMaxTables + 1) * 128; i += 64 * kEncWaves) f_qc[i] = a.tab->f_qc[i];
    __syncthreads();

    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t u = (uint64_t)blockIdx.x * kEncWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (u >= (uint64_t)a.n_chunks * a.S) return;
    const uint32_t c = (uint32_t)(u / a.S), st = (uint32_t)(u % a.S);
    const uint64_t c0 = (uint64_t)c * a.W;
    const uint32_t n_c = (uint32_t)std::min<uint64_t>(a.W, a.n - c0);
    const uint16_t* w = a.w + c0;
    const uint32_t K = a.K, l0 = st * a.P;
    const uint32_t groups = (n_c + 7) / 8, T = (groups + K - 1) / K;

    // start states: a lane's last group holds cnt = min(8, left) weights, and
    // the fractions of its last m = min(4, cnt) sit under a leading one at bit
    // max(16, 7m); a lane without weights starts at 2^16
    uint32_t x[R], rj0[R], rm[R];
    bool lv[R];
#pragma unroll
    for (int q = 0; q < R; q++) {
        const uint32_t l = l0 + 64 * q + lane;
        lv[q] = 64 * q + lane < a.P;
        rj0[q] = 0;
        rm[q] = 0;
        x[q] = 65536u;
        if (lv[q] && l < groups) {
            const uint32_t g = l + K * ((groups - 1 - l) / K);
            const uint32_t end = std::min(8 * g + 8, n_c);
            rm[q] = std::min(end - 8 * g, 4u);
            rj0[q] = end - rm[q];
            uint32_t v = 1u << std::max(16u, 7 * rm[q]);
            for (uint32_t i = 0; i < rm[q]; i++) v |= (uint32_t)(w[rj0[q] + i] & 127u) << (7 * i);
            x[q] = v;
        }
    }
    uint16_t* sink = a.words + u * 2ull * (a.W / a.S);
    uint32_t base = 0;
    for (int t = (int)T - 1; t >= 0; t--) {
        uint32_t gw[R][4];
        uint32_t gj[R];
#pragma unroll
        for (int q = 0; q < R; q++) {
            const uint32_t g = (uint32_t)t * K + l0 + 64 * q + lane;
            gj[q] = 8 * g;
            gw[q][0] = gw[q][1] = gw[q][2] = gw[q][3] = 0;
            if (lv[q] && g < groups) {
                if (8 * g + 8 <= n_c) {
                    const uint4 v = *(const uint4*)(w + 8 * g);
                    gw[q][0] = v.x; gw[q][1] = v.y; gw[q][2] = v.z; gw[q][3] = v.w;
                } else {
                    for (uint32_t i = 0; 8 * g + i < n_c; i++) gw[q][i >> 1] |= (uint32_t)w[8 * g + i] << (16 * (i & 1));
                }
            }
        }
#pragma unroll 1
        for (int p = 7; p >= 0; p--) {
#pragma unroll
            for (int q = R - 1; q >= 0; q--) {        // fraction sub-step
                const uint32_t j = gj[q] + p;
                const bool act = lv[q] && j < n_c && !(j >= rj0[q] && j < rj0[q] + rm[q]);
                const uint32_t v = (gw[q][p >> 1] >> (16 * (p & 1))) & 0xFFFFu;
                put_symbol(act, x[q], f_qc[route[v >> 7] * 128u + (v & 127u)], a.m_f, sink, base, lane);
            }
#pragma unroll
            for (int q = R - 1; q >= 0; q--) {        // sign/exponent sub-step
                const uint32_t j = gj[q] + p;
                const bool act = lv[q] && j < n_c;
                const uint32_t v = (gw[q][p >> 1] >> (16 * (p & 1))) & 0xFFFFu;
                put_symbol(act, x[q], s_qc[v >> 7], a.m_s, sink, base, lane);
            }
        }
    }
    uint32_t esum = 0;
#pragma unroll
    for (int q = 0; q < R; q++) {
        if (lv[q]) {
            a.states[(uint64_t)c * K + l0 + 64 * q + lane] = x[q];
            esum += 31u - (uint32_t)__builtin_clz(x[q]) - 16u;
        }
    }
    for (int off = 32; off; off >>= 1) esum += __shfl_xor(esum, off);
    if (lane == 0) {
        a.counts[2 * u] = base;
        a.counts[2 * u + 1] = esum;
    }
}

// Layout 2: code the weight of one sub-step for a lane: outside its last
// group the pair (h first, then s; the decoder takes s first) with one flush
// check against the joint bound q_s q_h 2^(32 - M_s - M_h), inside it s alone
// (bound q_s 2^(32 - M_s)).  Flushing lanes take word slots as in put_symbol.
__device__ __forceinline__ void put_weight2(bool act, bool pair, uint32_t& x, uint32_t sqc, uint32_t hqc, uint32_t m_s,
                                           uint32_t m_h, uint16_t* sink, uint32_t& base, uint32_t lane) {
    const uint32_t qs = sqc & 0xFFFFu, cs = sqc >> 16, qh = hqc & 0xFFFFu, ch = hqc >> 16;
    const bool flush = act && (pair ? (x >> (32 - m_s - m_h)) >= qs * qh : (x >> (32 - m_s)) >= qs);
    const uint64_t b = __builtin_amdgcn_ballot_w64(flush);
    if (flush) {
        const uint32_t above = (uint32_t)__builtin_popcountll(lane == 63 ? 0ull : b >> (lane + 1));
        sink[base + above] = (uint16_t)x;
        x >>= 16;
    }
    base += (uint32_t)__builtin_popcountll(b);
    if (act) {
        if (pair) x = ((x / qh) << m_h) + x % qh + ch;
        x = ((x / qs) << m_s) + x % qs + cs;
    }
}

// Layout 3: the same sub-step, with the joint symbol 8 s + h outside the
// last group (one flush check against q_t 2^(32 - 13), one coding step).
__device__ __forceinline__ void put_weight3(bool act, bool joint, uint32_t& x, uint32_t sqc, uint32_t tqc, uint32_t m_s,
                                           uint16_t* sink, uint32_t& base, uint32_t lane) {
    const uint32_t q = joint ? tqc & 0xFFFFu : sqc & 0xFFFFu, cum = joint ? tqc >> 16 : sqc >> 16;
    const uint32_t m = joint ? kJointBits : m_s;
    const bool flush = act && (x >> (32 - m)) >= q;
    const uint64_t b = __builtin_amdgcn_ballot_w64(flush);
    if (flush) {
        const uint32_t above = (uint32_t)__builtin_popcountll(lane == 63 ? 0ull : b >> (lane + 1));
        sink[base + above] = (uint16_t)x;
        x >>= 16;
    }
    base += (uint32_t)__builtin_popcountll(b);
    if (act) x = ((x / q) << m) + x % q + cum;
}

// Layouts 2 and 3 (J): one wavefront per word stream, one sub-step per
// weight, run backwards.  A lane's start state carries the h of its last
// group's c weights (the low 3c bits under a leading one at bit max(16, 3c)).
template <int R, bool J>
__global__ __launch_bounds__(64 * kEncWaves) void encode2_kernel(EncArgs a) {
    constexpr uint32_t NH = J ? 512 * 8 : (kMaxHTablesDev + 1) * 8;
    __shared__ uint32_t s_qc[512];
    __shared__ uint32_t h_qc[NH];   // J: the joint table's q | cum << 16
    __shared__ uint8_t route[512];
    for (uint32_t i = threadIdx.x; i < 512; i += 64 * kEncWaves) {
        s_qc[i] = a.tab->s_qc[i];
        route[i] = a.tab->route[i];
    }
    for (uint32_t i = threadIdx.x; i < NH; i += 64 * kEncWaves) h_qc[i] = J ? a.tab->t_qc[i] : a.tab->h_qc[i];
    __syncthreads();

    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t u = (uint64_t)blockIdx.x * kEncWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (u >= (uint64_t)a.n_chunks * a.S) return;
    const uint32_t c = (uint32_t)(u / a.S), st = (uint32_t)(u % a.S);
    const uint64_t c0 = (uint64_t)c * a.W;
    const uint32_t n_c = (uint32_t)std::min<uint64_t>(a.W, a.n - c0);
    const uint16_t* w = a.w + c0;
    const uint32_t K = a.K, l0 = st * a.P;
    const uint32_t groups = (n_c + 7) / 8, T = (groups + K - 1) / K;

    uint32_t x[R], glast[R];
    bool lv[R];
#pragma unroll
    for (int q = 0; q < R; q++) {
        const uint32_t l = l0 + 64 * q + lane;
        lv[q] = 64 * q + lane < a.P;
        x[q] = 65536u;
        glast[q] = UINT32_MAX;
        if (lv[q] && l < groups) {
            const uint32_t g = l + K * ((groups - 1 - l) / K);
            const uint32_t cnt = std::min(n_c - 8 * g, 8u);
            uint32_t v = 1u << std::max(16u, 3 * cnt);
            for (uint32_t i = 0; i < cnt; i++) v |= (uint32_t)((w[8 * g + i] & 127u) >> 4) << (3 * i);
            x[q] = v;
            glast[q] = g;
        }
    }
    uint16_t* sink = a.words + u * 2ull * (a.W / a.S);
    uint32_t base = 0;
    for (int t = (int)T - 1; t >= 0; t--) {
        uint32_t gw[R][4];
        uint32_t g[R];
#pragma unroll
        for (int q = 0; q < R; q++) {
            g[q] = (uint32_t)t * K + l0 + 64 * q + lane;
            gw[q][0] = gw[q][1] = gw[q][2] = gw[q][3] = 0;
            if (lv[q] && g[q] < groups) {
                if (8 * g[q] + 8 <= n_c) {
                    const uint4 v = *(const uint4*)(w + 8 * g[q]);
                    gw[q][0] = v.x; gw[q][1] = v.y; gw[q][2] = v.z; gw[q][3] = v.w;
                } else {
                    for (uint32_t i = 0; 8 * g[q] + i < n_c; i++) gw[q][i >> 1] |= (uint32_t)w[8 * g[q] + i] << (16 * (i & 1));
                }
            }
        }
#pragma unroll 1
        for (int p = 7; p >= 0; p--) {
#pragma unroll
            for (int q = R - 1; q >= 0; q--) {
                const uint32_t j = 8 * g[q] + p;
                const bool act = lv[q] && j < n_c;
                const uint32_t v = (gw[q][p >> 1] >> (16 * (p & 1))) & 0xFFFFu;
                if (J)
                    put_weight3(act, g[q] != glast[q], x[q], s_qc[v >> 7], h_qc[8u * (v >> 7) + ((v & 127u) >> 4)], a.m_s,
                                sink, base, lane);
                else
                    put_weight2(act, g[q] != glast[q], x[q], s_qc[v >> 7], h_qc[route[v >> 7] * 8u + ((v & 127u) >> 4)],
                                a.m_s, a.m_f, sink, base, lane);
            }
        }
    }
    uint32_t esum = 0;
#pragma unroll
    for (int q = 0; q < R; q++) {
        if (lv[q]) {
            a.states[(uint64_t)c * K + l0 + 64 * q + lane] = x[q];
            esum += 31u - (uint32_t)__builtin_clz(x[q]) - 16u;
        }
    }
    for (int off = 32; off; off >>= 1) esum += __shfl_xor(esum, off);
    if (lane == 0) {
        a.counts[2 * u] = base;
        a.counts[2 * u + 1] = esum;
    }
}

__global__ __launch_bounds__(64 * kEncWaves) void assemble_kernel(EncArgs a) {
    __shared__ uint32_t bits[kEncWaves][512];   // a stream's state bits: at most 512 lanes x 31 bits
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint64_t u = (uint64_t)blockIdx.x * kEncWaves + __builtin_amdgcn_readfirstlane(wave);
    if (u >= (uint64_t)a.n_chunks * a.S) return;
    const uint32_t c = (uint32_t)(u / a.S), st = (uint32_t)(u % a.S);
    const uint32_t K = a.K, P = a.P, l0 = st * P;
    uint8_t* pay = a.out + a.chunk_off[c];
    const uint32_t* xs = a.states + (uint64_t)c * K;
    // the chunk's length codes, a nibble per lane (lane l low in byte l / 2 when l is even)
    if (st == 0) {
        for (uint32_t b = lane; b < (K + 1) / 2; b += 64) {
            uint32_t v = 31u - (uint32_t)__builtin_clz(xs[2 * b]) - 16u;
            if (2 * b + 1 < K) v |= (31u - (uint32_t)__builtin_clz(xs[2 * b + 1]) - 16u) << 4;
            pay[b] = (uint8_t)v;
        }
    }
    const uint64_t code_bytes = ((K + 1ull) / 2 + 15) / 16 * 16;
    uint64_t plane = 0;
    if (a.layout >= 2) {
        // layouts 2 and 3: the plane of low fraction bits between the codes and the
        // streams; this stream's wave writes its lanes' groups (position p of
        // a group at bit 16 (p mod 2) + 4 (p div 2) of the group's word)
        const uint64_t c0 = (uint64_t)c * a.W;
        const uint32_t n_c = (uint32_t)std::min<uint64_t>(a.W, a.n - c0);
        const uint32_t groups = (n_c + 7) / 8;
        plane = (4ull * groups + 15) / 16 * 16;
        uint32_t* pw = (uint32_t*)(pay + code_bytes);
        for (uint32_t t = 0; (uint64_t)t * K < groups; t++) {
            for (uint32_t l = lane; l < P; l += 64) {
                const uint32_t gg = t * K + l0 + l;
                if (gg >= groups) continue;
                uint32_t v = 0;
                for (uint32_t i = 0; i < 8 && 8 * gg + i < n_c; i++)
                    v |= (uint32_t)(a.w[c0 + 8 * gg + i] & 15u) << (16 * (i & 1) + 4 * (i >> 1));
                pw[gg] = v;
            }
        }
    }
    uint16_t* area = (uint16_t*)(pay + code_bytes + plane);
    uint16_t* dst = area + a.unit_start[u];
    // state bits: each lane's 16 + e bits below its leading one, in lane order from bit 0
    uint32_t* bb = bits[wave];
    for (uint32_t i = lane; i < 512; i += 64) bb[i] = 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    uint32_t off = 0;
    for (uint32_t q = 0; 64 * q < P; q++) {
        const bool has = 64 * q + lane < P;
        const uint32_t xv = has ? xs[l0 + 64 * q + lane] : 65536u;
        const uint32_t len = has ? 16u + (31u - (uint32_t)__builtin_clz(xv) - 16u) : 0u;
        // exclusive prefix of len over the wave
        uint32_t incl = len;
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t o = __shfl_up(incl, d);
            if (lane >= (uint32_t)d) incl += o;
        }
        const uint32_t at = off + incl - len;
        if (has) {
            const uint32_t v = xv - (1u << len);
            atomicOr(bb + (at >> 5), v << (at & 31));
            if ((at & 31) + len > 32) atomicOr(bb + (at >> 5) + 1, v >> (32 - (at & 31)));
        }
        off += __shfl(incl, 63);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const uint32_t mu = a.unit_mu[u];
    for (uint32_t k = lane; k < mu; k += 64) dst[k] = (uint16_t)(bb[k >> 1] >> (16 * (k & 1)));
    // words, in decode order
    const uint32_t nw = a.counts[2 * u];
    const uint16_t* src = a.words + u * 2ull * (a.W / a.S);
    for (uint32_t k = lane; k < nw; k += 64) dst[mu + k] = src[nw - 1 - k];
}

__global__ void zero_kernel(uint4* d, uint64_t n16, uint8_t* tail, uint32_t n_tail) {
    for (uint64_t i = blockIdx.x * 256ull + threadIdx.x; i < n16; i += 256ull * gridDim.x) d[i] = make_uint4(0, 0, 0, 0);
    if (blockIdx.x == 0 && threadIdx.x < n_tail) tail[threadIdx.x] = 0;
}

}  // namespace

extern "C" {

int bsk_encode(const EncArgs* args, uint32_t R, void* stream) {
    const uint64_t units = (uint64_t)args->n_chunks * args->S;
    if (units == 0) return 0;
    const dim3 grid((uint32_t)((units + kEncWaves - 1) / kEncWaves)), block(64 * kEncWaves);
    hipStream_t st = (hipStream_t)stream;
    if (args->layout == 2 || args->layout == 3) {
        const uint32_t v = R | (args->layout == 3 ? 8u : 0u);
        switch (v) {
            case 1: hipLaunchKernelGGL((encode2_kernel<1, false>), grid, block, 0, st, *args); break;
            case 2: hipLaunchKernelGGL((encode2_kernel<2, false>), grid, block, 0, st, *args); break;
            case 4: hipLaunchKernelGGL((encode2_kernel<4, false>), grid, block, 0, st, *args); break;
            case 9: hipLaunchKernelGGL((encode2_kernel<1, true>), grid, block, 0, st, *args); break;
            case 10: hipLaunchKernelGGL((encode2_kernel<2, true>), grid, block, 0, st, *args); break;
            case 12: hipLaunchKernelGGL((encode2_kernel<4, true>), grid, block, 0, st, *args); break;
            default: return (int)hipErrorInvalidValue;
        }
        return (int)hipGetLastError();
    }
    switch (R) {
        case 1: hipLaunchKernelGGL(encode_kernel<1>, grid, block, 0, st, *args); break;
        case 2: hipLaunchKernelGGL(encode_kernel<2>, grid, block, 0, st, *args); break;
        case 4: hipLaunchKernelGGL(encode_kernel<4>, grid, block, 0, st, *args); break;
        case 8: hipLaunchKernelGGL(encode_kernel<8>, grid, block, 0, st, *args); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

int bsk_assemble(const EncArgs* args, void* stream) {
    const uint64_t units = (uint64_t)args->n_chunks * args->S;
    if (units == 0) return 0;
    hipLaunchKernelGGL(assemble_kernel, dim3((uint32_t)((units + kEncWaves - 1) / kEncWaves)), dim3(64 * kEncWaves), 0,
                       (hipStream_t)stream, *args);
    return (int)hipGetLastError();
}

int bsk_zero(void* d, uint64_t n, void* stream) {
    if (n == 0) return 0;
    const uint64_t n16 = ((uintptr_t)d & 15) ? 0 : n / 16;
    const uint32_t n_tail = (uint32_t)(n - 16 * n16);
    if (n_tail > 256) return (int)hipErrorInvalidValue;   // d must be 16-B aligned
    const uint32_t g = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>((n16 + 255) / 256, 65536));
    hipLaunchKernelGGL(zero_kernel, dim3(g), dim3(256), 0, (hipStream_t)stream, (uint4*)d, n16,
                       (uint8_t*)d + 16 * n16, n_tail);
    return (int)hipGetLastError();
}

}  // extern "C"
