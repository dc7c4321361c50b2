// bs_kernels.hip -- HIP kernels (gfx950) of the lossless BF16 weight codec.
//
// What is decoded [Qwen3.8-27B-BF16-NVLC-Lossless model card, codec
// paragraph]: each BF16 word w = s << 7 | f, where the joint (sign, exponent)
// symbol s is rANS-coded with a per-tensor model and the fraction f with the
// distribution selected by s; non-BF16 spans are copied verbatim.
//
// Kernels here (the decode kernel is in bs_decode.hip):
//   hist_kernel                    -- model building: one pass of field
//                                     histograms with LDS-privatised counters
//   lut_kernel                     -- per-record decode lookup tables
//   raw_copy_kernel                -- verbatim residual spans
//   compare_kernel                 -- byte compare for verification
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "bs_device.h"

using namespace bsd;

namespace {

// ------------------------------------------------------------------ histograms

constexpr int kHistThreads = 1024;

// One pass over the words of a tensor.  cf[e * 128 + f] counts exponent e and
// fraction f over both signs (the sign-merged fraction counts that the choice
// of coded contexts needs), and cneg[8 e + h] counts the negative words of
// exponent e whose fraction has high three bits h, from which the sign split
// follows: the (sign, exponent) counts cs[256 + e] = sum_h cneg[8 e + h],
// cs[e] = sum_f cf[e][f] - cs[256 + e], and the joint (sign, exponent, h)
// counts of layout 3.  The counters are privatised in LDS per workgroup
// (128 KiB + 8 KiB); keyed by h, the negative counts of one exponent also
// fall in 8 bins, because a tensor's exponents concentrate on a few values
// and same-address LDS atomics serialise.
__global__ __launch_bounds__(kHistThreads) void hist_kernel(const uint16_t* __restrict__ w, uint64_t n,
                                                             unsigned long long* __restrict__ cf,
                                                             unsigned long long* __restrict__ cneg) {
    __shared__ uint32_t hb[256 * 128];
    __shared__ uint32_t hn[256 * 8];
    for (uint32_t i = threadIdx.x; i < 256 * 128; i += blockDim.x) hb[i] = 0;
    for (uint32_t i = threadIdx.x; i < 256 * 8; i += blockDim.x) hn[i] = 0;
    __syncthreads();
    // aligned body in 16-B pieces, head and tail word by word
    const uint64_t addr = (uint64_t)(uintptr_t)w;
    uint64_t head = ((16 - (addr & 15)) & 15) / 2;
    if (head > n) head = n;
    const uint64_t body = (n - head) / 8;
    const uint4* p = (const uint4*)(w + head);
    const uint64_t gtid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t gsz = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = gtid; i < body; i += gsz) {
        const uint4 v = p[i];
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const uint32_t x = (d[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
            atomicAdd(&hb[x & 0x7FFFu], 1u);
            if (x & 0x8000u) atomicAdd(&hn[(x >> 4) & 0x7FFu], 1u);
        }
    }
    const uint64_t rest0 = head + body * 8;
    for (uint64_t i = gtid; i < head + (n - rest0); i += gsz) {
        const uint64_t j = i < head ? i : rest0 + (i - head);
        const uint32_t x = w[j];
        atomicAdd(&hb[x & 0x7FFFu], 1u);
        if (x & 0x8000u) atomicAdd(&hn[(x >> 4) & 0x7FFu], 1u);
    }
    __syncthreads();
    for (uint32_t b = threadIdx.x; b < 256 * 128; b += blockDim.x)
        if (hb[b]) atomicAdd(&cf[b], (unsigned long long)hb[b]);
    for (uint32_t b = threadIdx.x; b < 256 * 8; b += blockDim.x)
        if (hn[b]) atomicAdd(&cneg[b], (unsigned long long)hn[b]);
}

// ------------------------------------------------------------------ lookup tables

__device__ __forceinline__ uint32_t ld16(const uint8_t* p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }

// last index i in [0, A) with cum[i] <= v (cum non-decreasing, cum[0] = 0)
__device__ __forceinline__ uint32_t last_le(const uint32_t* cum, uint32_t A, uint32_t v) {
    uint32_t lo = 0, hi = A;  // answer in [lo, hi)
    while (hi - lo > 1) {
        uint32_t mid = (lo + hi) >> 1;
        if (cum[mid] <= v) lo = mid; else hi = mid;
    }
    return lo;
}

// One workgroup per BF16 record: expand the container's compact tables into
// the record's lookup-table image (layout in bs_device.h).
__global__ __launch_bounds__(256) void lut_kernel(const uint8_t* __restrict__ c, const RecDev* __restrict__ recs,
                                                  uint8_t* __restrict__ luts) {
    __shared__ uint32_t qs[512], cums[512], route[512];
    __shared__ uint32_t qf[kMaxTables + 1][128], cumf[kMaxTables + 1][128];
    const RecDev r = recs[blockIdx.x];
    const uint8_t* body = c + r.body;
    for (uint32_t i = threadIdx.x; i < 512; i += blockDim.x) { qs[i] = 0; route[i] = 0; }
    __syncthreads();
    for (uint32_t k = threadIdx.x; k < r.n_sym; k += blockDim.x) {
        uint32_t s = ld16(body + r.stab_off + 4 * k);
        qs[s] = ld16(body + r.stab_off + 4 * k + 2);
        route[s] = body[r.route_off + k];
    }
    const uint32_t nt = r.n_tables + 1;
    if (r.layout == 3) {
        // layout 3 (image layout with kJointBytes): the joint (s, h) entries,
        // then the s entries of the lanes' last groups
        __shared__ uint32_t cumt[512 * 8];
        __shared__ uint32_t qtl[512 * 8];
        for (uint32_t i = threadIdx.x; i < 512 * 8; i += blockDim.x) qtl[i] = 0;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < 8 * r.n_sym; i += blockDim.x) {
            const uint32_t k = i / 8, h = i % 8;
            qtl[8 * ld16(body + r.stab_off + 4 * k) + h] = ld16(body + r.ftab_off + 2 * i);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t a = 0;
            for (int s = 0; s < 512; s++) { cums[s] = a; a += qs[s]; }
            a = 0;
            for (int t = 0; t < 512 * 8; t++) { cumt[t] = a; a += qtl[t]; }
        }
        __syncthreads();
        uint2* jo = (uint2*)(luts + r.lut_off);
        for (uint32_t i = threadIdx.x; i < (1u << kJointBits); i += blockDim.x) {
            const uint32_t t = last_le(cumt, 512 * 8, i);
            jo[i] = make_uint2(qtl[t], ((t >> 3) << 7 | (t & 7u) << 4) | (i - cumt[t]) << 16);
        }
        uint2* so = (uint2*)(luts + r.lut_off + kJointBytes);
        for (uint32_t slot = threadIdx.x; slot < (1u << r.m_s); slot += blockDim.x) {
            const uint32_t s = last_le(cums, 512, slot);
            so[slot] = make_uint2(qs[s], s | (slot - cums[s]) << 16);
        }
        return;
    }
    if (r.layout == 2) {
        // layout 2 (the image layout is described with kHPageBytes): 8-byte s
        // entries, then 2 KiB h pages indexed by 8 state bits; page 0 is
        // flat (q_h = 2^(M_h - 3))
        __shared__ uint32_t qh[kMaxHTablesDev + 1][8], cumh[kMaxHTablesDev + 1][8];
        for (uint32_t i = threadIdx.x; i < nt * 8; i += blockDim.x) {
            const uint32_t t = i / 8, h = i % 8;
            qh[t][h] = t == 0 ? (1u << (r.m_f - 3)) : body[r.ftab_off + 8 * (t - 1) + h];
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t a = 0;
            for (int s = 0; s < 512; s++) { cums[s] = a; a += qs[s]; }
        }
        if (threadIdx.x >= 64 && threadIdx.x < 64 + nt) {
            const uint32_t t = threadIdx.x - 64;
            uint32_t a = 0;
            for (int h = 0; h < 8; h++) { cumh[t][h] = a; a += qh[t][h]; }
        }
        __syncthreads();
        uint2* so = (uint2*)(luts + r.lut_off);
        const uint32_t ns = 1u << r.m_s;
        for (uint32_t slot = threadIdx.x; slot < ns; slot += blockDim.x) {
            const uint32_t s = last_le(cums, 512, slot);
            const uint32_t page = (8u * ns + route[s] * kHPageBytes) / 2048;
            so[slot] = make_uint2(qs[s] | page << 24, s | (slot - cums[s]) << 16);
        }
        uint2* ho = (uint2*)(luts + r.lut_off + 8ull * ns);
        const uint32_t hmask = (1u << r.m_f) - 1;
        for (uint32_t i = threadIdx.x; i < nt * 256; i += blockDim.x) {
            const uint32_t t = i / 256, b = i % 256, slot = b & hmask;
            const uint32_t h = last_le(cumh[t], 8, slot);
            ho[i] = make_uint2((qh[t][h] << (8 - r.m_f)) | (h << 29), qh[t][h] * (b >> r.m_f) + slot - cumh[t][h]);
        }
        return;
    }
    for (uint32_t i = threadIdx.x; i < nt * 128; i += blockDim.x) {
        uint32_t t = i / 128, f = i % 128;
        qf[t][f] = t == 0 ? (1u << (r.m_f - 7)) : ld16(body + r.ftab_off + 256 * (t - 1) + 2 * f);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t a = 0;
        for (int s = 0; s < 512; s++) { cums[s] = a; a += qs[s]; }
    }
    if (threadIdx.x >= 64 && threadIdx.x < 64 + nt) {
        uint32_t t = threadIdx.x - 64, a = 0;
        for (int f = 0; f < 128; f++) { cumf[t][f] = a; a += qf[t][f]; }
    }
    __syncthreads();
    uint2* out = (uint2*)(luts + r.lut_off);
    const uint32_t ns = 1u << r.m_s;
    for (uint32_t slot = threadIdx.x; slot < ns; slot += blockDim.x) {
        uint32_t s = last_le(cums, 512, slot);
        uint32_t page = (slut_bytes(r.compact) + route[s] * fpage_bytes(r.compact)) >> 11;
        out[slot] = make_uint2(qs[s] | (page << 24), s | ((slot - cums[s]) << 20));
    }
    uint2* fo = (uint2*)(luts + r.lut_off + 8ull * ns);
    const uint32_t nf = 1u << r.m_f;
    for (uint32_t i = threadIdx.x; i < nt * nf; i += blockDim.x) {
        uint32_t t = i / nf, slot = i % nf;
        uint32_t f = last_le(cumf[t], 128, slot);
        fo[t * (fpage_bytes(r.compact) / 8) + slot] = make_uint2(qf[t][f] | (f << 25), slot - cumf[t][f]);
    }
}

// ------------------------------------------------------------------ residual and compare

__global__ __launch_bounds__(256) void raw_copy_kernel(const uint8_t* __restrict__ c, const RawDev* __restrict__ raw,
                                                       uint8_t* __restrict__ out, uint64_t out_base) {
    const RawDev rd = raw[blockIdx.y];
    const uint8_t* s = c + rd.src;
    uint8_t* d = out + (rd.dst - out_base);
    const uint64_t gtid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t gsz = (uint64_t)gridDim.x * blockDim.x;
    if ((((uintptr_t)s | (uintptr_t)d) & 15) == 0) {
        const uint64_t n16 = rd.n / 16;
        for (uint64_t i = gtid; i < n16; i += gsz) ((uint4*)d)[i] = ((const uint4*)s)[i];
        for (uint64_t i = n16 * 16 + gtid; i < rd.n; i += gsz) d[i] = s[i];
    } else {
        for (uint64_t i = gtid; i < rd.n; i += gsz) d[i] = s[i];
    }
}

__global__ __launch_bounds__(256) void compare_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                      uint64_t n, unsigned long long* __restrict__ res) {
    const uint64_t gtid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t gsz = (uint64_t)gridDim.x * blockDim.x;
    unsigned long long bad = 0, first = ~0ull;
    if ((((uintptr_t)a | (uintptr_t)b) & 15) == 0) {
        const uint64_t n16 = n / 16;
        for (uint64_t i = gtid; i < n16; i += gsz) {
            uint4 u = ((const uint4*)a)[i], v = ((const uint4*)b)[i];
            uint32_t du[4] = {u.x ^ v.x, u.y ^ v.y, u.z ^ v.z, u.w ^ v.w};
#pragma unroll
            for (int k = 0; k < 4; k++) {
                for (int j = 0; j < 4; j++) {
                    if ((du[k] >> (8 * j)) & 0xFF) {
                        bad++;
                        unsigned long long idx = 16 * i + 4 * k + j;
                        if (idx < first) first = idx;
                    }
                }
            }
        }
        for (uint64_t i = n16 * 16 + gtid; i < n; i += gsz)
            if (a[i] != b[i]) { bad++; if (i < first) first = i; }
    } else {
        for (uint64_t i = gtid; i < n; i += gsz)
            if (a[i] != b[i]) { bad++; if (i < first) first = i; }
    }
    if (bad) {
        atomicAdd(&res[0], bad);
        atomicMin(&res[1], first);
    }
}

inline int grid_for(uint64_t work, uint64_t per_block, int cap) {
    uint64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > (uint64_t)cap) g = cap;
    return (int)g;
}

}  // namespace

extern "C" {

int bsk_device_cus(int* cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    return (int)hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
}

int bsk_hist(const uint16_t* d_w, uint64_t n, unsigned long long* d_cf, unsigned long long* d_cneg, void* stream) {
    // about a million words per workgroup: each workgroup zeroes and flushes
    // 136 KiB of counters, so small tensors get few workgroups
    int cus = 0;
    if (bsk_device_cus(&cus) != 0 || cus <= 0) cus = 256;
    const uint64_t want = (n + (1u << 20) - 1) >> 20;
    const int g = (int)std::max<uint64_t>(1, std::min<uint64_t>(want, (uint64_t)cus));
    hipLaunchKernelGGL(hist_kernel, dim3(g), dim3(kHistThreads), 0, (hipStream_t)stream, d_w, n, d_cf, d_cneg);
    return (int)hipGetLastError();
}

int bsk_build_luts(const uint8_t* d_container, const RecDev* d_recs, uint32_t n_recs, uint8_t* d_luts, void* stream) {
    if (n_recs == 0) return 0;
    hipLaunchKernelGGL(lut_kernel, dim3(n_recs), dim3(256), 0, (hipStream_t)stream, d_container, d_recs, d_luts);
    return (int)hipGetLastError();
}

int bsk_raw_copy(const uint8_t* d_container, const RawDev* d_raw, uint32_t n_raw, uint8_t* d_out, uint64_t out_base,
                 void* stream) {
    if (n_raw == 0) return 0;
    hipLaunchKernelGGL(raw_copy_kernel, dim3(64, n_raw), dim3(256), 0, (hipStream_t)stream, d_container, d_raw, d_out,
                       out_base);
    return (int)hipGetLastError();
}

int bsk_compare(const uint8_t* a, const uint8_t* b, uint64_t n, unsigned long long* d_result, void* stream) {
    int g = grid_for(n, 256ull * 64, 4096);
    hipLaunchKernelGGL(compare_kernel, dim3(g), dim3(256), 0, (hipStream_t)stream, a, b, n, d_result);
    return (int)hipGetLastError();
}

}  // extern "C"
