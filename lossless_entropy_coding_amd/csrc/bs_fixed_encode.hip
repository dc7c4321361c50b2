// bs_fixed_encode.hip -- the fixed-width lane-stream form built on the GPU
// (gfx950) from BF16 words in device memory.
//
// The form is derived from the canonical model's decoded weights once, at
// initialisation [NVLC card, runtime paragraphs]; its layout is in bs.h and
// is the same bytes the host transcoder writes.  Three passes:
//   sym_count_kernel   the (sign, exponent) symbol counts (LDS-privatised
//                      counters, one 64-bit add per bin per workgroup);
//   block_esc_kernel   escapes per 2048-weight block, given the host's code
//                      of each symbol;
//   pack_kernel        one wave per block writes the code and fraction planes
//                      (each store instruction covers 256 contiguous bytes)
//                      and scatters the block's escaped symbols at the
//                      block's first escape plus the wave prefix of the
//                      lanes' escape counts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "bs_device.h"
#include "bs_fixed_device.h"

using namespace bsd;

namespace {

// Eight interleaved copies of the 512 counters (copy k of bin b at 8 b + k;
// lane l adds to copy l mod 8): the few hot symbols of a weight tensor then
// spread over eight LDS banks instead of queueing on one.  Words are read 8
// at a time (16-B loads; the words are 16-B aligned), the ragged tail one by
// one.
constexpr uint32_t kCountCopies = 8;

__global__ __launch_bounds__(256) void sym_count_kernel(const uint16_t* w, uint64_t n, unsigned long long* counts) {
    __shared__ uint32_t c[512 * kCountCopies];
    for (uint32_t i = threadIdx.x; i < 512 * kCountCopies; i += 256) c[i] = 0;
    __syncthreads();
    uint32_t* mine = c + (threadIdx.x & (kCountCopies - 1));
    const uint64_t n8 = n / 8, stride = 256ull * gridDim.x;
    const uint4* w8 = (const uint4*)w;
    for (uint64_t j = blockIdx.x * 256ull + threadIdx.x; j < n8; j += stride) {
        const uint4 v = w8[j];
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            atomicAdd(mine + kCountCopies * ((d[k] >> 7) & 511u), 1u);   // low word's symbol
            atomicAdd(mine + kCountCopies * (d[k] >> 23), 1u);            // high word's symbol
        }
    }
    for (uint64_t j = 8 * n8 + blockIdx.x * 256ull + threadIdx.x; j < n; j += stride)
        atomicAdd(mine + kCountCopies * (w[j] >> 7), 1u);
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < 512; i += 256) {
        uint32_t t = 0;
#pragma unroll
        for (uint32_t k = 0; k < kCountCopies; k++) t += c[kCountCopies * i + k];
        if (t) atomicAdd(counts + i, (unsigned long long)t);
    }
}

// escapes of each block (code 15 <-> code_of[s] == 15)
__global__ __launch_bounds__(256) void block_esc_kernel(const uint16_t* w, uint64_t n, const uint8_t* code_of,
                                                        uint64_t n_blocks, uint32_t* esc) {
    __shared__ uint8_t cmap[512];
    for (uint32_t i = threadIdx.x; i < 512; i += 256) cmap[i] = code_of[i];
    __syncthreads();
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t blk = blockIdx.x * 4ull + (threadIdx.x >> 6);
    if (blk >= n_blocks) return;
    uint32_t cnt = 0;
#pragma unroll
    for (uint32_t i = 0; i < 4; i++) {
        // lane l takes words 8 l .. 8 l + 7 of each 512-word quarter: one
        // 16-B load (the words are 16-B aligned), 1 KiB per load instruction
        const uint64_t j = blk * kFixBlockW + 512ull * i + 8ull * lane;
        if (j + 8 <= n) {
            const uint4 v = *(const uint4*)(w + j);
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; k++)
                cnt += (cmap[(d[k] >> 7) & 511u] == 15) + (cmap[d[k] >> 23] == 15);
        } else {
            for (uint32_t e = 0; e < 8; e++)
                if (j + e < n) cnt += cmap[w[j + e] >> 7] == 15;
        }
    }
    for (int off = 32; off; off >>= 1) cnt += __shfl_xor(cnt, off);
    if (lane == 0) esc[blk] = cnt;
}

// one wave per block: lane l packs weights 32 l .. 32 l + 31 of the block
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* w, uint64_t n, const uint8_t* code_of,
                                                   uint64_t n_blocks, const uint32_t* first, uint8_t* blob,
                                                   uint64_t esc_off) {
    __shared__ uint8_t cmap[512];
    for (uint32_t i = threadIdx.x; i < 512; i += 256) cmap[i] = code_of[i];
    __syncthreads();
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t blk = blockIdx.x * 4ull + (threadIdx.x >> 6);
    if (blk >= n_blocks) return;
    const uint64_t j0 = blk * kFixBlockW + 32ull * lane;
    uint32_t cw[4] = {0, 0, 0, 0}, fr[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t esc_mask = 0;
    uint32_t v[32];
    if (j0 + 32 <= n) {
        const uint4* p = (const uint4*)(w + j0);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint4 q = p[k];
            v[8 * k + 0] = q.x & 0xFFFFu; v[8 * k + 1] = q.x >> 16;
            v[8 * k + 2] = q.y & 0xFFFFu; v[8 * k + 3] = q.y >> 16;
            v[8 * k + 4] = q.z & 0xFFFFu; v[8 * k + 5] = q.z >> 16;
            v[8 * k + 6] = q.w & 0xFFFFu; v[8 * k + 7] = q.w >> 16;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; i++) v[i] = j0 + i < n ? w[j0 + i] : 0xFFFFFFFFu;   // past n: code 0, fraction 0
    }
#pragma unroll
    for (int i = 0; i < 32; i++) {
        const bool live = v[i] != 0xFFFFFFFFu;
        const uint32_t s = live ? v[i] >> 7 : 0, f = live ? v[i] & 127u : 0;
        const uint32_t code = live ? cmap[s] : 0u;
        cw[i / 8] |= code << (4 * (i % 8));
        const int bit = 7 * i;
        fr[bit / 32] |= f << (bit % 32);
        if (bit % 32 > 25) fr[bit / 32 + 1] |= f >> (32 - bit % 32);
        if (code == 15) esc_mask |= 1u << i;
    }
    uint32_t* plane = (uint32_t*)(blob + kFixHeader + (uint64_t)kFixBlockBytes * blk) + lane;
#pragma unroll
    for (int k = 0; k < 4; k++) plane[64 * k] = cw[k];
#pragma unroll
    for (int k = 0; k < 7; k++) plane[256 + 64 * k] = fr[k];
    // the lane's escapes, in weight order, after the escapes of the lanes below it
    const uint32_t cnt = (uint32_t)__builtin_popcount(esc_mask);
    uint32_t incl = cnt;
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(incl, d);
        if (lane >= (uint32_t)d) incl += o;
    }
    uint16_t* e = (uint16_t*)(blob + esc_off) + first[blk] + (incl - cnt);
    for (uint32_t m = esc_mask; m; m &= m - 1) *e++ = (uint16_t)(w[j0 + __builtin_ctz(m)] >> 7);   // re-read: rare
}

}  // namespace

extern "C" {

int bsk_fixed_sym_count(const uint16_t* w, uint64_t n, unsigned long long* counts, void* stream) {
    if (n == 0) return 0;
    const uint32_t g = (uint32_t)std::min<uint64_t>((n + (1u << 16) - 1) >> 16, 2048);
    hipLaunchKernelGGL(sym_count_kernel, dim3(g), dim3(256), 0, (hipStream_t)stream, w, n, counts);
    return (int)hipGetLastError();
}

int bsk_fixed_block_esc(const uint16_t* w, uint64_t n, const uint8_t* code_of, uint64_t n_blocks, uint32_t* esc,
                        void* stream) {
    if (n_blocks == 0) return 0;
    hipLaunchKernelGGL(block_esc_kernel, dim3((uint32_t)((n_blocks + 3) / 4)), dim3(256), 0, (hipStream_t)stream, w, n,
                       code_of, n_blocks, esc);
    return (int)hipGetLastError();
}

int bsk_fixed_pack(const uint16_t* w, uint64_t n, const uint8_t* code_of, uint64_t n_blocks, const uint32_t* first,
                   uint8_t* blob, uint64_t esc_off, void* stream) {
    if (n_blocks == 0) return 0;
    hipLaunchKernelGGL(pack_kernel, dim3((uint32_t)((n_blocks + 3) / 4)), dim3(256), 0, (hipStream_t)stream, w, n,
                       code_of, n_blocks, first, blob, esc_off);
    return (int)hipGetLastError();
}

}  // extern "C"
