// bs_fixed.hip -- decode of the fixed-width lane-stream form (gfx950).
//
// The form keeps every weight as an 11-bit code word (a 4-bit symbol code,
// 15 = escape, and the exact 7-bit fraction) in 2048-weight blocks of 64
// lanes [NVLC card, runtime paragraphs: the GPU runtime decodes fixed-width,
// lane-oriented streams derived once from the canonical model; the layout is
// the library's own and is given in bs.h].  Nothing in a block depends on
// another block, so the decode is a plain data-parallel pass:
//   - one wavefront takes a block: each lane loads its 4 code dwords and 7
//     fraction dwords, every load instruction covering 256 contiguous bytes;
//   - a 256-entry LDS table maps a code byte (two weights) to both symbols
//     already in place (s << 7 in each 16-bit half; code 15 gives 0), and the
//     two fractions are inserted with a shift and masks;
//   - the lane's 16 output dwords go to a per-wave LDS block (its four 16-B
//     pieces rotated by lane pair, so the writes of a wave spread over all
//     banks), escaped symbols are OR-ed in there, and the block leaves LDS as
//     16-B stores that cover 1 KiB of contiguous output per instruction;
//   - escapes: the block's range of the escape list (from the per-block
//     offsets) is staged in LDS while the planes load; a lane's escapes
//     start at the wave's exclusive prefix of its escape count, and an
//     escape's rank among the lane's follows from the codes below it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "bs_device.h"

using namespace bsd;

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// bit 4 i set iff nibble i of x is 15
__device__ __forceinline__ uint32_t nibbles_15(uint32_t x) {
    uint32_t y = x & (x >> 1);
    y &= y >> 2;
    return y & 0x11111111u;
}

// exclusive prefix over the wave of v (0..32), and the wave total
__device__ __forceinline__ uint32_t wave_prefix(uint32_t v, uint32_t& total) {
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int b = 0; b < 6; b++) {
        const uint64_t m = __builtin_amdgcn_ballot_w64((v >> b) & 1u);
        pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
        tot += (uint32_t)__builtin_popcountll(m) << b;
    }
    total = tot;
    return pre;
}

// orders this wave's LDS accesses around a hand-over between its lanes (the
// LDS executes a wave's instructions in order, so no wait is needed)
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

__global__ __launch_bounds__(64 * kFixWaves) void fixed_decode_kernel(FixedArgs a) {
    __shared__ uint32_t lut[256];
    __shared__ __attribute__((aligned(16))) uint32_t stage[kFixWaves][kFixBlockW / 2];
    __shared__ uint16_t escl[kFixWaves][kFixEscLds];

    const uint32_t t = threadIdx.x, lane = t & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);
    {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (uint32_t k = 0; k < 15; k++) {
            const uint32_t sym = (a.tab[k >> 1] >> (16 * (k & 1))) & 511u;
            lo = (t & 15u) == k ? sym : lo;
            hi = (t >> 4) == k ? sym : hi;
        }
        lut[t] = (lo << 7) | (hi << 23);
    }
    __syncthreads();

    uint32_t* st = stage[wave];
    uint16_t* el = escl[wave];
    const uint32_t* offs = (const uint32_t*)(a.blob + kFixHeader + (uint64_t)kFixBlockBytes * a.n_blocks);
    const uint16_t* esc = (const uint16_t*)(a.blob + a.esc_off);
    const uint32_t rot = lane >> 1;

    for (uint64_t blk = (uint64_t)blockIdx.x * kFixWaves + wave; blk < a.n_blocks;
         blk += (uint64_t)gridDim.x * kFixWaves) {
        const uint32_t* plane = (const uint32_t*)(a.blob + kFixHeader + (uint64_t)kFixBlockBytes * blk) + lane;
        uint32_t c[4], f[7];
#pragma unroll
        for (int k = 0; k < 4; k++) c[k] = plane[64 * k];
#pragma unroll
        for (int k = 0; k < 7; k++) f[k] = plane[256 + 64 * k];

        // the block's escape range, staged in LDS (its first kFixEscLds)
        const uint64_t e0 = offs[blk];
        const uint64_t e1 = blk + 1 < a.n_blocks ? (uint64_t)offs[blk + 1] : a.n_esc;
        uint32_t bad = 0;
        uint32_t cnt = 0;
        if (e0 <= e1 && e1 <= a.n_esc) cnt = (uint32_t)std::min<uint64_t>(e1 - e0, kFixBlockW + 1);
        else bad |= 2u;
        const uint16_t* eb = esc + (bad ? 0 : e0);
        const uint32_t lim = std::min<uint32_t>(cnt, kFixEscLds);
        uint32_t ev[kFixEscLds / 64];
#pragma unroll
        for (uint32_t u = 0; u < kFixEscLds / 64; u++) {
            ev[u] = 0;
            if (64 * u < lim && lane + 64 * u < lim) ev[u] = eb[lane + 64 * u];
        }

        // escapes in the lane's codes: bit 4 i + k of m <-> weight 8 k + i of the lane
        const uint32_t m = nibbles_15(c[0]) | nibbles_15(c[1]) << 1 | nibbles_15(c[2]) << 2 | nibbles_15(c[3]) << 3;
        uint32_t total;
        const uint32_t pre = wave_prefix((uint32_t)__builtin_popcount(m), total);
        if (total != cnt) bad |= 1u;

        // symbols and fractions, two weights per dword
        uint32_t o[16];
#pragma unroll
        for (int p = 0; p < 16; p++) {
            const uint32_t sy = lut[(c[p >> 2] >> (8 * (p & 3))) & 0xFFu];
            const int q = (14 * p) >> 5, r = (14 * p) & 31;
            const uint32_t w = r <= 18 ? f[q] >> r : __builtin_amdgcn_alignbit(f[q + 1], f[q], r);
            o[p] = sy | (w & 0x7Fu) | ((w << 9) & 0x7F0000u);
        }
#pragma unroll
        for (int u = 0; u < kFixEscLds / 64; u++)
            if (64 * u < lim && lane + 64 * u < lim) el[lane + 64 * u] = (uint16_t)ev[u];
#pragma unroll
        for (uint32_t k = 0; k < 4; k++)
            *(v4u*)(st + 16 * lane + 4 * ((k + rot) & 3u)) = v4u{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
        wave_lds_fence();

        // escaped symbols: the rank of an escape among the lane's is the count
        // of the lane's escapes at lower weights
        for (uint32_t left = m; left;) {
            const uint32_t b = __builtin_ctz(left);
            left &= left - 1;
            const uint32_t k = b & 3u, i = b >> 2;
            const uint32_t km = 0x11111111u << k;
            const uint32_t below = (km - 0x11111111u) | (km & ((1u << (4 * i)) - 1u));
            const uint32_t r = pre + (uint32_t)__builtin_popcount(m & below);
            uint32_t s = 0;
            if (r < lim) s = el[r];
            else if (r < cnt) s = eb[r];
            if (r >= cnt) bad |= 1u;
            if (s > 511u) { bad |= 4u; s = 0; }
            atomicOr(st + 16 * lane + 4 * ((k + rot) & 3u) + (i >> 1), s << (7 + 16 * (i & 1u)));
        }
        wave_lds_fence();

        // out: 16-B pieces in order, 1 KiB per store instruction; the last,
        // partial block word by word
        uint16_t* ob = a.out + blk * kFixBlockW;
        const uint64_t left_w = a.n - blk * kFixBlockW;
        if (left_w >= kFixBlockW) {
#pragma unroll
            for (uint32_t u = 0; u < 4; u++) {
                const uint32_t cc = 64 * u + lane, L = cc >> 2, pc = cc & 3u;
                *(v4u*)(ob + 8 * cc) = *(const v4u*)(st + 16 * L + 4 * ((pc + (L >> 1)) & 3u));
            }
        } else {
            const uint16_t* st16 = (const uint16_t*)st;
            for (uint32_t e = lane; e < (uint32_t)left_w; e += 64) {
                const uint32_t L = e >> 5, wi = e & 31u;
                ob[e] = st16[32 * L + 8 * (((wi >> 3) + (L >> 1)) & 3u) + (wi & 7u)];
            }
        }
        if (a.status) {
            uint32_t any = 0;
#pragma unroll
            for (uint32_t bit = 0; bit < 3; bit++)
                if (__builtin_amdgcn_ballot_w64((bad >> bit) & 1u)) any |= 1u << bit;
            if (lane == 0) a.status[blk] = any;
        }
        wave_lds_fence();
    }
}

}  // namespace

extern "C" int bsk_fixed_decode(const FixedArgs* args, uint32_t n_groups, void* stream) {
    if (n_groups == 0 || args->n_blocks == 0) return 0;
    hipLaunchKernelGGL(fixed_decode_kernel, dim3(n_groups), dim3(64 * kFixWaves), 0, (hipStream_t)stream, *args);
    return (int)hipGetLastError();
}
