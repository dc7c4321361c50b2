// bs_fixed.hip -- kernels of the fixed-width lane-stream form (gfx950):
// decode, and decode fused with a matrix-vector product.
//
// The form keeps every weight as an 11-bit code word (a 4-bit symbol code,
// 15 = escape, and the exact 7-bit fraction) in 2048-weight blocks of 64
// lanes [NVLC card, runtime paragraphs: the GPU runtime decodes fixed-width,
// lane-oriented streams derived once from the canonical model, and its
// compressed-only runtime multiplies with weights decoded where they are
// used; the layout is the library's own and is given in bs.h].  Nothing in a
// block depends on another block, so both kernels are plain data-parallel
// passes:
//   - one wavefront takes a block: each lane loads its 4 code dwords and 7
//     fraction dwords, every load instruction covering 256 contiguous bytes;
//   - a 256-entry LDS table maps a code byte (two weights) to both symbols
//     already in place (s << 7 in each 16-bit half; code 15 gives 0), and the
//     two fractions are inserted with a shift and masks;
//   - the lane's 16 output dwords go to a per-wave LDS block (its four 16-B
//     pieces rotated by lane pair, so the writes of a wave spread over all
//     banks) and escaped symbols are OR-ed in there;
//   - escapes: the block's range of the escape list (from the per-block
//     offsets) is staged in LDS while the planes load; a lane's escapes
//     start at the wave's exclusive prefix of its escape count, and an
//     escape's rank among the lane's follows from the codes below it;
//   - decode: the block leaves LDS as 16-B non-temporal stores, 1 KiB of
//     contiguous output per instruction (the output is not read again by
//     this kernel, so it bypasses the caches' normal allocation);
//   - product: a workgroup owns whole rows (groups of rows that end on a
//     block boundary) and deals their blocks to its waves; each lane reads
//     its own 32 patched weights back and multiplies them with x (packed BF16
//     pairs, v_dot2 with fp32 accumulation), the waves sum per row (DPP
//     steps, then LDS), and the workgroup stores its rows' totals.  Nothing
//     is written but y, and no atomics are used.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "bs_device.h"
#include "bs_fixed_device.h"
#include "bs_wave.h"

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

// A block's loaded data: the lane's code and fraction dwords, its share of
// the block's first escapes (two dwords, up to 254 escapes for the wave) and
// the block's escape range.
struct BlockIn {
    uint32_t c[4], f[7];
    uint32_t ev0, ev1;
    uint64_t eb0;           // the block's first escape (0 when its range is bad)
    uint32_t cnt;           // escapes in its range
    uint32_t bad;
};

// Issue the loads of block blk (nothing waits for them here).
__device__ __forceinline__ BlockIn load_block(const FixedArgs& a, uint64_t blk, uint32_t lane) {
    BlockIn b;
    const uint32_t* plane = (const uint32_t*)(a.blob + kFixHeader + (uint64_t)kFixBlockBytes * blk) + lane;
#pragma unroll
    for (int k = 0; k < 4; k++) b.c[k] = plane[64 * k];
#pragma unroll
    for (int k = 0; k < 7; k++) b.f[k] = plane[256 + 64 * k];
    const uint32_t* offs = (const uint32_t*)(a.blob + kFixHeader + (uint64_t)kFixBlockBytes * a.n_blocks);
    const uint64_t e0 = offs[blk];
    const uint64_t e1 = blk + 1 < a.n_blocks ? (uint64_t)offs[blk + 1] : a.n_esc;
    b.bad = 0;
    b.cnt = 0;
    if (e0 <= e1 && e1 <= a.n_esc) b.cnt = (uint32_t)std::min<uint64_t>(e1 - e0, kFixBlockW + 1);
    else b.bad = 2u;
    b.eb0 = b.bad ? 0 : e0;
    // dwords from the one holding escape eb0 (the escape list is 4-B aligned
    // and padded, so the dword holding the last escape is inside the blob)
    const uint32_t* ew = (const uint32_t*)(a.blob + a.esc_off) + (b.eb0 >> 1);
    const uint32_t ndw = (std::min<uint32_t>(b.cnt, kFixEscLds - 2) + (uint32_t)(b.eb0 & 1) + 1) >> 1;
    b.ev0 = b.ev1 = 0;
    if (ndw) {
        b.ev0 = ew[std::min(lane, ndw - 1)];
        b.ev1 = ew[std::min(lane + 64, ndw - 1)];
    }
    return b;
}

// Decode a loaded block into the wave's LDS block st (lane l's 32 weights at
// dwords 16 l .. 16 l + 15, 16-B piece k at slot (k + l / 2) mod 4); returns
// the block's status bits (this lane's view).  el: the wave's escape staging.
__device__ __forceinline__ uint32_t finish_block(const FixedArgs& a, const BlockIn& b, uint32_t lane,
                                                 const uint32_t* lut, uint32_t* st, uint16_t* el) {
    uint32_t bad = b.bad;
    const uint32_t cnt = b.cnt;
    // escape eb0 + r is LDS half-word sh + r for r < lim, else read from HBM
    const uint16_t* eb = (const uint16_t*)(a.blob + a.esc_off) + b.eb0;
    const uint32_t* ew = (const uint32_t*)(a.blob + a.esc_off) + (b.eb0 >> 1);
    const uint32_t sh = (uint32_t)(b.eb0 & 1);
    const uint32_t lim = std::min<uint32_t>(cnt, kFixEscLds - 2);
    const uint32_t ndw = (lim + sh + 1) >> 1;

    // escapes in the lane's codes: bit 4 i + k of m <-> weight 8 k + i of the lane
    const uint32_t m =
        nibbles_15(b.c[0]) | nibbles_15(b.c[1]) << 1 | nibbles_15(b.c[2]) << 2 | nibbles_15(b.c[3]) << 3;
    uint32_t total;
    const uint32_t pre = wave_prefix((uint32_t)__builtin_popcount(m), total);
    if (total != cnt) bad |= 1u;

    // symbols and fractions, two weights per dword
    uint32_t o[16];
#pragma unroll
    for (int p = 0; p < 16; p++) {
        const uint32_t sy = lut[(b.c[p >> 2] >> (8 * (p & 3))) & 0xFFu];
        const int q = (14 * p) >> 5, r = (14 * p) & 31;
        const uint32_t w = r <= 18 ? b.f[q] >> r : __builtin_amdgcn_alignbit(b.f[q + 1], b.f[q], r);
        o[p] = sy | (w & 0x7Fu) | ((w << 9) & 0x7F0000u);
    }
    uint32_t* el32 = (uint32_t*)el;
    if (lane < ndw) el32[lane] = b.ev0;
    if (lane + 64 < ndw) el32[lane + 64] = b.ev1;
    for (uint32_t u = 2; 64 * u < ndw; u++)          // blocks with more escapes (rare)
        if (lane + 64 * u < ndw) el32[lane + 64 * u] = ew[lane + 64 * u];
    const uint32_t rot = lane >> 1;
#pragma unroll
    for (uint32_t k = 0; k < 4; k++)
        *(v4u*)(st + 16 * lane + 4 * ((k + rot) & 3u)) = v4u{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
    wave_lds_fence();

    // escaped symbols: the rank of an escape among the lane's is the count
    // of the lane's escapes at lower weights
    for (uint32_t left = m; left;) {
        const uint32_t bit = __builtin_ctz(left);
        left &= left - 1;
        const uint32_t k = bit & 3u, i = bit >> 2;
        const uint32_t km = 0x11111111u << k;
        const uint32_t below = (km - 0x11111111u) | (km & ((1u << (4 * i)) - 1u));
        const uint32_t r = pre + (uint32_t)__builtin_popcount(m & below);
        uint32_t s = 0;
        if (r < lim) s = el[sh + r];
        else if (r < cnt) s = eb[r];
        if (r >= cnt) bad |= 1u;
        if (s > 511u) { bad |= 4u; s = 0; }
        atomicOr(st + 16 * lane + 4 * ((k + rot) & 3u) + (i >> 1), s << (7 + 16 * (i & 1u)));
    }
    wave_lds_fence();
    return bad;
}

__device__ __forceinline__ void write_status(const FixedArgs& a, uint64_t blk, uint32_t bad, uint32_t lane) {
    if (!a.status) return;
    uint32_t any = 0;
#pragma unroll
    for (uint32_t bit = 0; bit < 3; bit++)
        if (__builtin_amdgcn_ballot_w64((bad >> bit) & 1u)) any |= 1u << bit;
    if (lane == 0) a.status[blk] = any;
}

// the 256-entry pair table: entry b = both symbols of code byte b in place
__device__ __forceinline__ void build_lut(const FixedArgs& a, uint32_t t, uint32_t* lut) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (uint32_t k = 0; k < 15; k++) {
        const uint32_t sym = (a.tab[k >> 1] >> (16 * (k & 1))) & 511u;
        lo = (t & 15u) == k ? sym : lo;
        hi = (t >> 4) == k ? sym : hi;
    }
    lut[t] = (lo << 7) | (hi << 23);
}

// decode: one wave per block at a time, out written with 16-B stores
// Blocks g*4 + wave, then every (ng*4)-th after, of one tensor: decoded,
// staged in LDS and stored (the LUT of that tensor already in LDS).
__device__ __forceinline__ void decode_blocks(const FixedArgs& a, uint32_t g, uint32_t ng, uint32_t wave,
                                              uint32_t lane, const uint32_t* lut, uint32_t* st, uint16_t* el) {
    for (uint64_t blk = (uint64_t)g * kFixWaves + wave; blk < a.n_blocks; blk += (uint64_t)ng * kFixWaves) {
        const uint32_t bad = finish_block(a, load_block(a, blk, lane), lane, lut, st, el);
        // out: 16-B pieces in order, 1 KiB per store instruction; the last,
        // partial block word by word
        uint16_t* ob = a.out + blk * kFixBlockW;
        const uint64_t left_w = a.n - blk * kFixBlockW;
        if (left_w >= kFixBlockW) {
#pragma unroll
            for (uint32_t u = 0; u < 4; u++) {
                const uint32_t cc = 64 * u + lane, L = cc >> 2, pc = cc & 3u;
                const v4u v = *(const v4u*)(st + 16 * L + 4 * ((pc + (L >> 1)) & 3u));
                __builtin_nontemporal_store(v, (v4u*)(ob + 8 * cc));
            }
        } else {
            const uint16_t* st16 = (const uint16_t*)st;
            for (uint32_t e = lane; e < (uint32_t)left_w; e += 64) {
                const uint32_t L = e >> 5, wi = e & 31u;
                ob[e] = st16[32 * L + 8 * (((wi >> 3) + (L >> 1)) & 3u) + (wi & 7u)];
            }
        }
        write_status(a, blk, bad, lane);
    }
}

__global__ __launch_bounds__(64 * kFixWaves, 8) void fixed_decode_kernel(FixedArgs a) {
    __shared__ uint32_t lut[256];
    __shared__ __attribute__((aligned(16))) uint32_t stage[kFixWaves][kFixBlockW / 2];
    __shared__ __attribute__((aligned(4))) uint16_t escl[kFixWaves][kFixEscLds];

    const uint32_t t = threadIdx.x, lane = t & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);
    build_lut(a, t, lut);
    __syncthreads();
    decode_blocks(a, blockIdx.x, gridDim.x, wave, lane, lut, stage[wave], escl[wave]);
}

// Several tensors in one launch: tensor i owns workgroups wg_start[i] ..
// wg_start[i + 1] - 1 (a share of the grid in proportion to its blocks), so
// each workgroup builds one LUT and the tails of the tensors overlap instead
// of each ending its own launch.
__global__ __launch_bounds__(64 * kFixWaves, 8) void fixed_decode_many_kernel(const FixedMany m) {
    __shared__ uint32_t lut[256];
    __shared__ __attribute__((aligned(16))) uint32_t stage[kFixWaves][kFixBlockW / 2];
    __shared__ __attribute__((aligned(4))) uint16_t escl[kFixWaves][kFixEscLds];

    uint32_t i = 0;
    for (uint32_t k = 1; k < m.count; k++)
        if (m.wg_start[k] <= blockIdx.x) i = k;
    const FixedArgs& a = m.a[i];
    const uint32_t t = threadIdx.x, lane = t & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);
    build_lut(a, t, lut);
    __syncthreads();
    decode_blocks(a, blockIdx.x - m.wg_start[i], m.wg_start[i + 1] - m.wg_start[i], wave, lane, lut, stage[wave],
                  escl[wave]);
}

// The fused product: workgroup g takes row groups g, g + groups, ...: a
// group is group_units units of whole rows (so it starts and ends on a block
// boundary), its blocks dealt to the four waves in turn.  For each block,
// each lane multiplies its 32 weights with x, the wave sums the lanes of each
// row present (DPP steps) and lane 0 adds the sums to its wave's row totals
// in LDS; at the end of the group the workgroup adds the four waves' totals
// in wave order and stores them to y.  Every y[r] is summed in one fixed
// order, so the result is the same on every run.
__global__ __launch_bounds__(64 * kFixWaves) void fixed_gemv_kernel(FixedArgs a) {
    __shared__ uint32_t lut[256];
    __shared__ __attribute__((aligned(16))) uint32_t stage[kFixWaves][kFixBlockW / 2];
    __shared__ __attribute__((aligned(4))) uint16_t escl[kFixWaves][kFixEscLds];
    __shared__ float rowsum[kFixWaves][64];

    const uint32_t t = threadIdx.x, lane = t & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);
    build_lut(a, t, lut);

    uint32_t* st = stage[wave];
    uint16_t* el = escl[wave];
    float* rs = rowsum[wave];
    const uint32_t rot = lane >> 1;
    const uint32_t grows = a.unit_rows * a.group_units;
    const uint64_t gblocks = (uint64_t)a.unit_blocks * a.group_units;
    // the lane's row in the group and column in the wave's first block (the
    // group starts on a block), then advanced by kFixWaves blocks at a time
    const uint32_t jr0 = wave * kFixBlockW + 32 * lane;
    const uint32_t rr0 = jr0 / a.cols, cc0 = jr0 - rr0 * a.cols;
    for (uint64_t g = blockIdx.x; g < a.n_groups; g += gridDim.x) {
        const uint64_t ra = g * grows;
        const uint32_t nrows = (uint32_t)std::min<uint64_t>(grows, a.rows - ra);
        const uint64_t b0 = g * gblocks;
        const uint32_t nblk = (uint32_t)((nrows * (uint64_t)a.cols + kFixBlockW - 1) / kFixBlockW);
        __syncthreads();              // the previous group's totals have been read (and the table built)
        rs[lane] = 0.f;
        __syncthreads();
        uint32_t rr = rr0, col = cc0;
        for (uint32_t k = wave; k < nblk; k += kFixWaves) {
            const uint64_t blk = b0 + k;
            const bool live = rr < nrows;   // cols % 32 == 0 keeps a lane's 32 weights in one row
            v4u xv[4] = {};
            if (live) {
                const v4u* xp = (const v4u*)(a.gx + col);
#pragma unroll
                for (int q = 0; q < 4; q++) xv[q] = xp[q];
            }
            const uint32_t bad = finish_block(a, load_block(a, blk, lane), lane, lut, st, el);
            float sum = 0.f;
#pragma unroll
            for (uint32_t q = 0; q < 4; q++) {
                const v4u wv = *(const v4u*)(st + 16 * lane + 4 * ((q + rot) & 3u));
                const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
                const uint32_t xd[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
#pragma unroll
                for (int h = 0; h < 4; h++)
                    sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[h]),
                                                          __builtin_bit_cast(bf16x2, xd[h]), sum, false);
            }
            if (!live) sum = 0.f;
            // the block's rows, from lane 0's to the last live lane's
            const uint32_t r_first = __builtin_amdgcn_readfirstlane(rr);
            const uint32_t r_last = std::min<uint32_t>(__builtin_amdgcn_readlane(rr, 63), nrows - 1);
            for (uint32_t q = r_first; q <= r_last; q++) {
                const float s = wave_sum_dpp(rr == q ? sum : 0.f);
                if (lane == 0) rs[q] += s;
            }
            write_status(a, blk, bad, lane);
            wave_lds_fence();
            col += a.r_step;
            rr += a.q_step;
            if (col >= a.cols) { col -= a.cols; rr++; }
        }
        __syncthreads();
        if (t < nrows) a.gy[ra + t] = ((rowsum[0][t] + rowsum[1][t]) + rowsum[2][t]) + rowsum[3][t];
    }
}

// The fused product with a batch of vectors, Y[n][r] = sum over c of W[r][c] X[n][c],
// on the matrix cores.  A work item is a group of 16 MF rows and a share of
// their panels of 2048 columns (rows start on a block, cols % 2048 == 0, so a
// panel of a row is one whole block).  For each panel the kGemmWaves waves
// decode the group's 16 MF blocks into LDS, 16 MF / kGemmWaves each, then
// multiply the panel with X with v_mfma_f32_16x16x32_bf16 (A: 16 rows x 32
// columns of the panel, a 16-B piece per lane read back through the decode's
// piece rotation; B: 32 columns x 16 batch rows of X, 16 B per lane from X in
// HBM or L2, one load serving MF row tiles); the next panel's blocks are
// loaded while one is multiplied.  The waves split the batch into NT tiles of
// 16 and each tile's columns among kGemmWaves / NT waves; the K slices are
// added in wave order.
//
// MF 1: a workgroup takes all panels of its 16 rows and stores its part of Y.
// MF 2 halves the X traffic per row (each X element feeds 32 rows); so that
// as many workgroups stay busy, ksplit 2 gives the first half of a group's
// panels to one work item and the second half to another.  The first stores its partial sums
// in Y, the second in the workspace, and combine_kernel, launched next on the
// same stream, adds the second into the first: every Y entry is P0 + P1, one
// value on every run.  (Combining in this kernel, by whichever work item
// arrives second, needs an agent-scope acquire, which invalidates the XCD's
// L2 and with it the X lines the other workgroups are reading; it measured
// slower than the second launch.)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Y += P: the split product's second half added into the first, n floats
// (16 B per thread and step where both are 16-B aligned, then the tail)
__global__ __launch_bounds__(256) void combine_kernel(float* __restrict__ y, const float* __restrict__ part, uint64_t n) {
    const uint64_t t = (uint64_t)blockIdx.x * 256 + threadIdx.x, stride = (uint64_t)gridDim.x * 256;
    uint64_t n4 = 0;
    if ((((uintptr_t)y | (uintptr_t)part) & 15) == 0) {
        n4 = n / 4;
        for (uint64_t i = t; i < n4; i += stride) {
            float4 a = ((float4*)y)[i];
            const float4 b = ((const float4*)part)[i];
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
            ((float4*)y)[i] = a;
        }
    }
    for (uint64_t i = 4 * n4 + t; i < n; i += stride) y[i] += part[i];
}

template <int NT, int MF>
__global__ __launch_bounds__(64 * kGemmWaves) void fixed_gemm_kernel(FixedArgs a) {
    constexpr uint32_t kRows = 16 * MF;               // rows of a work item
    __shared__ uint32_t lut[256];
    __shared__ __attribute__((aligned(16))) uint8_t wbuf[kRows][kGemmRowBytes];
    __shared__ __attribute__((aligned(4))) uint16_t escl[kGemmWaves][kFixEscLds];
    // the waves' K slices: a table of their own at MF 1; at MF 2 they go over
    // the decoded rows once the last panel is multiplied
    __shared__ f32x4 red1[MF == 1 ? kGemmWaves : 1][64];
    static_assert(MF == 1 || sizeof(wbuf) >= sizeof(f32x4) * kGemmWaves * MF * 64, "K-slice table over wbuf");
    f32x4* red = MF == 1 ? &red1[0][0] : (f32x4*)&wbuf[0][0];

    const uint32_t t = threadIdx.x, lane = t & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);
    if (t < 256) build_lut(a, t, lut);
    uint16_t* el = escl[wave];
    constexpr uint32_t kWpt = kGemmWaves / NT;     // waves per batch tile
    constexpr uint32_t kSlice = kFixBlockW / kWpt; // panel columns per wave
    const uint32_t nt = wave / kWpt, ks = wave % kWpt;
    const uint32_t bpr = a.cols / kFixBlockW;
    const uint32_t split = MF == 2 && a.ksplit == 2 && bpr >= 2 ? 2u : 1u;   // every share holds a panel
    const uint32_t p_mid = (bpr + 1) / 2;          // the first share's panels: 0 .. p_mid - 1
    const uint64_t groups = (a.rows + kRows - 1) / kRows;
    const uint64_t items = groups * split;
    for (uint64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const uint64_t g = item / split;
        const uint32_t kh = (uint32_t)(item % split);
        const uint32_t p0 = split == 1 ? 0u : (kh == 0 ? 0u : p_mid);
        const uint32_t p1 = split == 1 ? bpr : (kh == 0 ? p_mid : bpr);
        const uint64_t r0 = kRows * g;
        f32x4 acc[MF];
#pragma unroll
        for (int m = 0; m < MF; m++) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        constexpr uint32_t kRpw = kRows / kGemmWaves;   // rows (blocks of a panel) per wave
        uint32_t mr[kRpw];
        bool has[kRpw];
        BlockIn in[kRpw];
        // this wave's blocks of the first panel; each later panel's are
        // loaded while the current one is multiplied
#pragma unroll
        for (uint32_t h = 0; h < kRpw; h++) {
            mr[h] = kRpw * wave + h;
            has[h] = r0 + mr[h] < a.rows;
            if (has[h]) in[h] = load_block(a, (r0 + mr[h]) * bpr + p0, lane);
        }
        // B operands: 16 B of X per lane and k step.  Rows past the batch read
        // row 0; they only feed D columns that are never stored.  The loads go
        // out kU at a time, each group while the one before it is multiplied,
        // and a panel's first group is issued before its blocks are decoded.
        // offsets in 32 bits (batch <= 64 and cols < 2^26; batch x rows < 2^32)
        const uint32_t n = nt * 16 + (lane & 15);
        const uint16_t* xrow = a.gx + ((n < a.batch ? n : 0u) * a.cols + ks * kSlice + 8 * (lane >> 4));
        constexpr uint32_t kNs = kSlice / 32;               // k steps per wave and panel
        // X loads in flight per group: 8, or 2 where each feeds two row tiles
        // (4 made the compiler spill 6 registers at NT 4 and ran 13% slower
        // at batch 64)
        constexpr uint32_t kUmax = MF == 2 ? 2 : 8;
        constexpr uint32_t kU = kNs < kUmax ? kNs : kUmax;
        bf16x8 bv[kU];
        for (uint32_t p = p0; p < p1; p++) {
#pragma unroll
            for (uint32_t u = 0; u < kU; u++) bv[u] = *(const bf16x8*)(xrow + (uint64_t)p * kFixBlockW + 32 * u);
            __syncthreads();          // the previous panel (or K-slice table) is consumed, the table built
#pragma unroll
            for (uint32_t h = 0; h < kRpw; h++) {
                uint32_t* st = (uint32_t*)wbuf[mr[h]];
                if (has[h]) {
                    const uint64_t blk = (r0 + mr[h]) * bpr + p;
                    const uint32_t bad = finish_block(a, in[h], lane, lut, st, el);
                    write_status(a, blk, bad, lane);
                } else {
#pragma unroll
                    for (uint32_t k = 0; k < 4; k++) *(v4u*)(st + 16 * lane + 4 * k) = v4u{0u, 0u, 0u, 0u};
                }
            }
            __syncthreads();
            // the next panel's blocks load while this one is multiplied
            if (p + 1 < p1) {
#pragma unroll
                for (uint32_t h = 0; h < kRpw; h++)
                    if (has[h]) in[h] = load_block(a, (r0 + mr[h]) * bpr + p + 1, lane);
            }
            const uint16_t* xr = xrow + (uint64_t)p * kFixBlockW;
#pragma unroll
            for (uint32_t s0 = 0; s0 < kNs; s0 += kU) {
                bf16x8 cur[kU];
#pragma unroll
                for (uint32_t u = 0; u < kU; u++) cur[u] = bv[u];
                if (s0 + kU < kNs) {
#pragma unroll
                    for (uint32_t u = 0; u < kU; u++) bv[u] = *(const bf16x8*)(xr + 32 * (s0 + kU + u));
                }
#pragma unroll
                for (uint32_t u = 0; u < kU; u++) {
                    const uint32_t e0 = ks * kSlice + 32 * (s0 + u) + 8 * (lane >> 4);
                    const uint32_t L = e0 >> 5, kp = (e0 >> 3) & 3u;
                    const uint32_t off = 64 * L + 16 * ((kp + (L >> 1)) & 3u);
#pragma unroll
                    for (int m = 0; m < MF; m++) {
                        const bf16x8 av = *(const bf16x8*)(wbuf[16 * m + (lane & 15)] + off);
                        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, cur[u], acc[m], 0, 0, 0);
                    }
                }
            }
        }
        if (MF == 2) __syncthreads();     // every wave is done with the decoded rows
#pragma unroll
        for (int m = 0; m < MF; m++) red[(wave * MF + m) * 64 + lane] = acc[m];
        __syncthreads();
        f32x4 sum[MF];
#pragma unroll
        for (int m = 0; m < MF; m++) sum[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (ks == 0) {
#pragma unroll
            for (int m = 0; m < MF; m++) {
                sum[m] = red[(wave * MF + m) * 64 + lane];
#pragma unroll
                for (uint32_t w2 = 1; w2 < kWpt; w2++) sum[m] += red[((wave + w2) * MF + m) * 64 + lane];
            }
        }
        // D row 4 (lane / 16) + i of row tile m, column lane % 16
        float* dst = split == 2 && kh == 1 ? a.gpart : a.gy;
        if (ks == 0) {
            const uint32_t rows = (uint32_t)a.rows, rg = (uint32_t)r0 + 4 * (lane >> 4);
#pragma unroll
            for (int m = 0; m < MF; m++)
#pragma unroll
                for (uint32_t i = 0; i < 4; i++) {
                    const uint32_t r = rg + 16 * m + i;
                    if (n < a.batch && r < rows) dst[n * rows + r] = sum[m][i];
                }
        }
    }
}

}  // namespace

extern "C" int bsk_fixed_decode_many(const FixedMany* m, void* stream) {
    if (m->count == 0 || m->wg_start[m->count] == 0) return 0;
    hipLaunchKernelGGL(fixed_decode_many_kernel, dim3(m->wg_start[m->count]), dim3(64 * kFixWaves), 0,
                       (hipStream_t)stream, *m);
    return (int)hipGetLastError();
}

extern "C" int bsk_fixed_gemm(const FixedArgs* args, uint32_t n_groups, int rows32, void* stream) {
    if (n_groups == 0 || args->rows == 0) return 0;
    const dim3 grid(n_groups), block(64 * kGemmWaves);
    hipStream_t st = (hipStream_t)stream;
    const uint32_t nt = (args->batch + 15) / 16;
    if (rows32) {
        if (args->ksplit != 1 && args->ksplit != 2) return (int)hipErrorInvalidValue;
        if (args->ksplit == 2 && (!args->gpart || args->cols < 2 * kFixBlockW)) return (int)hipErrorInvalidValue;
        switch (nt) {
            case 1: hipLaunchKernelGGL((fixed_gemm_kernel<1, 2>), grid, block, 0, st, *args); break;
            case 2: hipLaunchKernelGGL((fixed_gemm_kernel<2, 2>), grid, block, 0, st, *args); break;
            case 3:
            case 4: hipLaunchKernelGGL((fixed_gemm_kernel<4, 2>), grid, block, 0, st, *args); break;
            default: return (int)hipErrorInvalidValue;
        }
        if (args->ksplit == 2) {
            const uint64_t n = (uint64_t)args->batch * args->rows;
            const uint32_t cgrid = (uint32_t)std::min<uint64_t>((n / 4 + 255) / 256 + 1, 2048);
            hipLaunchKernelGGL(combine_kernel, dim3(cgrid), dim3(256), 0, st, args->gy, args->gpart, n);
        }
        return (int)hipGetLastError();
    }
    switch (nt) {
        case 1: hipLaunchKernelGGL((fixed_gemm_kernel<1, 1>), grid, block, 0, st, *args); break;
        case 2: hipLaunchKernelGGL((fixed_gemm_kernel<2, 1>), grid, block, 0, st, *args); break;
        case 3:
        case 4: hipLaunchKernelGGL((fixed_gemm_kernel<4, 1>), grid, block, 0, st, *args); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

extern "C" int bsk_fixed_decode(const FixedArgs* args, uint32_t n_groups, void* stream) {
    if (n_groups == 0 || args->n_blocks == 0) return 0;
    hipLaunchKernelGGL(fixed_decode_kernel, dim3(n_groups), dim3(64 * kFixWaves), 0, (hipStream_t)stream, *args);
    return (int)hipGetLastError();
}

extern "C" int bsk_fixed_gemv(const FixedArgs* args, uint32_t n_groups, void* stream) {
    if (n_groups == 0 || args->n_groups == 0) return 0;
    hipLaunchKernelGGL(fixed_gemv_kernel, dim3(n_groups), dim3(64 * kFixWaves), 0, (hipStream_t)stream, *args);
    return (int)hipGetLastError();
}
