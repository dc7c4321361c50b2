// bs_fixed.cpp -- the fixed-width lane-stream form: host transcoder, header
// validation, and the decode and fused matrix-vector product entry points.
//
// The form is derived once from a BF16 tensor (the canonical container's
// decode) and read by a kernel without any sequential chain [NVLC card,
// runtime paragraphs: the measured GPU runtime derives fixed-width,
// lane-oriented streams at initialisation].  Layout: see bs.h.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <array>
#include <new>
#include <vector>

#include "bs_device.h"
#include "bs_fixed_device.h"
#include "bs_encode_device.h"
#include "bs_internal.h"

using namespace bs;

namespace {

constexpr char kFixMagic[8] = {'B', 'F', '1', '6', 'F', 'I', 'X', '1'};
constexpr uint32_t kFixVersion = 1;
constexpr uint64_t kEscapeCode = 15;

uint64_t fixed_blocks(uint64_t n) { return (n + bsd::kFixBlockW - 1) / bsd::kFixBlockW; }
uint64_t fixed_esc_off(uint64_t nb) { return bsd::kFixHeader + (uint64_t)(bsd::kFixBlockBytes + 4) * nb; }

// codes 0..14: the up to 15 most frequent symbols, count descending, ties to
// the lower symbol
uint32_t fixed_table(const uint64_t* cs, uint16_t* table) {
    std::array<uint32_t, 512> order;
    for (uint32_t s = 0; s < 512; s++) order[s] = s;
    std::stable_sort(order.begin(), order.end(), [&](uint32_t x, uint32_t y) { return cs[x] > cs[y]; });
    uint32_t m = 0;
    for (uint32_t k = 0; k < 15 && cs[order[k]]; k++) table[m++] = (uint16_t)order[k];
    for (uint32_t k = m; k < 16; k++) table[k] = 0;
    return m;
}

// one block: code and fraction planes, and its escapes from esc (in weight order)
void pack_block(const uint16_t* w, uint64_t n, uint64_t blk, const uint8_t* code_of, uint8_t* base, uint8_t* esc) {
    for (uint32_t l = 0; l < 64; l++) {
        const uint64_t j0 = blk * bsd::kFixBlockW + 32ull * l;
        uint32_t cw[4] = {0, 0, 0, 0}, fr[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (uint32_t i = 0; i < 32 && j0 + i < n; i++) {
            const uint32_t x = w[j0 + i], s = x >> 7, f = x & 0x7Fu, code = code_of[s];
            cw[i / 8] |= code << (4 * (i % 8));
            const uint32_t bit = 7 * i;
            fr[bit / 32] |= f << (bit % 32);
            if (bit % 32 > 25) fr[bit / 32 + 1] |= f >> (32 - bit % 32);
            if (code == kEscapeCode) { wr16(esc, s); esc += 2; }
        }
        for (uint32_t k = 0; k < 4; k++) wr32(base + 4 * (64 * k + l), cw[k]);
        for (uint32_t k = 0; k < 7; k++) wr32(base + 1024 + 4 * (64 * k + l), fr[k]);
    }
}

bool info_consistent(const bs_fixed_info* info) {
    if (info->n_blocks != fixed_blocks(info->n) || info->esc_off != fixed_esc_off(info->n_blocks) ||
        info->n_esc > 0xFFFFFFFFull || info->bytes < info->esc_off + 2 * info->n_esc) {
        set_error("bs_fixed_info not from bs_fixed_info_get");
        return false;
    }
    for (uint32_t k = 0; k < 16; k++)
        if (info->table[k] > 511 || (k == 15 && info->table[k])) { set_error("bad symbol table"); return false; }
    return true;
}

// kernel arguments common to the decode and the product
bs_status fixed_args(const bs_fixed_info* info, const void* d_blob, bsd::FixedArgs& a) {
    if (!info || !d_blob) { set_error("NULL argument"); return BS_E_INVAL; }
    if ((uintptr_t)d_blob & 15) { set_error("blob must be 16-B aligned"); return BS_E_INVAL; }
    if (!info_consistent(info)) return BS_E_INVAL;
    memset(&a, 0, sizeof a);
    a.blob = (const uint8_t*)d_blob;
    a.n = info->n;
    a.n_blocks = info->n_blocks;
    a.n_esc = info->n_esc;
    a.esc_off = info->esc_off;
    for (uint32_t k = 0; k < 15; k++) a.tab[k / 2] |= (uint32_t)info->table[k] << (16 * (k % 2));
    return BS_OK;
}

// one wave per work item (a block, or a unit of rows) up to 16 workgroups per
// CU; beyond, waves stride
uint32_t fixed_groups(uint64_t items) {
    int cus = 0;
    if (bsk_device_cus(&cus) != 0 || cus <= 0) cus = 256;
    const uint64_t want = (items + bsd::kFixWaves - 1) / bsd::kFixWaves;
    return (uint32_t)std::min<uint64_t>(want, 16ull * (uint64_t)cus);
}

}  // namespace

extern "C" {

bs_status bs_fixed_encode_host(const uint16_t* w, uint64_t n, uint32_t threads, bs_blob** out) {
    if (!out || (n && !w)) { set_error("NULL argument"); return BS_E_INVAL; }
    *out = nullptr;
    try {
        const uint32_t nt = pick_threads(threads);
        const uint64_t nb = fixed_blocks(n);
        // symbol counts
        const uint64_t slice = 1ull << 20, n_slices = (n + slice - 1) / slice;
        std::vector<std::array<uint64_t, 512>> part(n_slices);
        parallel_for(n_slices, nt, [&](uint64_t i) {
            auto& h = part[i];
            h.fill(0);
            for (uint64_t j = i * slice, e = std::min(n, j + slice); j < e; j++) h[w[j] >> 7]++;
        });
        uint64_t cs[512] = {0};
        for (auto& h : part)
            for (uint32_t s = 0; s < 512; s++) cs[s] += h[s];
        uint16_t table[16];
        const uint32_t m = fixed_table(cs, table);
        uint8_t code_of[512];
        memset(code_of, (int)kEscapeCode, sizeof code_of);
        for (uint32_t k = 0; k < m; k++) code_of[table[k]] = (uint8_t)k;
        // escapes per block, then each block's first
        std::vector<uint64_t> first(nb + 1, 0);
        parallel_for(nb, nt, [&](uint64_t b) {
            uint64_t e = 0;
            for (uint64_t j = b * bsd::kFixBlockW, end = std::min(n, j + bsd::kFixBlockW); j < end; j++)
                e += code_of[w[j] >> 7] == kEscapeCode;
            first[b + 1] = e;
        });
        for (uint64_t b = 0; b < nb; b++) first[b + 1] += first[b];
        const uint64_t n_esc = first[nb];
        if (n_esc > 0xFFFFFFFFull) { set_error("more than 2^32 - 1 escapes"); return BS_E_INVAL; }
        const uint64_t esc_off = fixed_esc_off(nb);
        auto* blob = new bs_blob;
        blob->bytes.assign(align_up(esc_off + 2 * n_esc, 16), 0);
        uint8_t* b = blob->bytes.data();
        memcpy(b, kFixMagic, 8);
        wr32(b + 8, kFixVersion);
        wr64(b + 16, n);
        wr64(b + 24, nb);
        wr64(b + 32, esc_off);
        wr64(b + 40, n_esc);
        for (uint32_t k = 0; k < 16; k++) wr16(b + 64 + 2 * k, table[k]);
        parallel_for(nb, nt, [&](uint64_t blk) {
            wr32(b + bsd::kFixHeader + (uint64_t)bsd::kFixBlockBytes * nb + 4 * blk, (uint32_t)first[blk]);
            pack_block(w, n, blk, code_of, b + bsd::kFixHeader + (uint64_t)bsd::kFixBlockBytes * blk,
                       b + esc_off + 2 * first[blk]);
        });
        *out = blob;
        return BS_OK;
    } catch (const std::bad_alloc&) {
        set_error("out of host memory");
        return BS_E_NOMEM;
    }
}

uint64_t bs_fixed_max_bytes(uint64_t n) {
    const uint64_t nb = fixed_blocks(n);
    return align_up(fixed_esc_off(nb) + 2 * n, 16);
}

bs_status bs_fixed_encode_device(const void* d_words, uint64_t n, void* d_out, uint64_t capacity, uint64_t* out_len,
                                 void* stream) {
    if (!out_len || (!d_words && n) || !d_out) { set_error("NULL argument"); return BS_E_INVAL; }
    if (((uintptr_t)d_words | (uintptr_t)d_out) & 15) { set_error("words and output must be 16-B aligned"); return BS_E_INVAL; }
    hipStream_t hs = (hipStream_t)stream;
    const uint64_t nb = fixed_blocks(n);
    const uint64_t esc_off = fixed_esc_off(nb);
    // scratch: 512 symbol counts, the code of each symbol, escapes and first escape of each block
    const uint64_t o_codes = 512 * 8, o_esc = align_up(o_codes + 512, 256), o_first = align_up(o_esc + 4 * nb, 256);
    uint8_t* d_s = nullptr;
    hipError_t e = hipMalloc(&d_s, o_first + 4 * nb + 16);
    if (e != hipSuccess) { set_error("transcoder scratch: %s", hipGetErrorString(e)); return BS_E_NOMEM; }
    auto done = [&](bs_status rc) { (void)hipStreamSynchronize(hs); (void)hipFree(d_s); return rc; };
    auto hip = [&](hipError_t he, const char* what) { set_error("%s: %s", what, hipGetErrorString(he)); return done(BS_E_HIP); };
    try {
        std::vector<uint64_t> cs(512, 0);
        int ke = bsk_zero(d_s, 512 * 8, stream);
        if (!ke) ke = bsk_fixed_sym_count((const uint16_t*)d_words, n, (unsigned long long*)d_s, stream);
        if (ke) return hip((hipError_t)ke, "symbol counts");
        e = hipMemcpyAsync(cs.data(), d_s, 512 * 8, hipMemcpyDeviceToHost, hs);
        if (e == hipSuccess) e = hipStreamSynchronize(hs);
        if (e != hipSuccess) return hip(e, "symbol counts");
        uint16_t table[16];
        const uint32_t m = fixed_table(cs.data(), table);
        uint8_t code_of[512];
        memset(code_of, (int)kEscapeCode, sizeof code_of);
        for (uint32_t k = 0; k < m; k++) code_of[table[k]] = (uint8_t)k;
        std::vector<uint32_t> esc(nb), first(nb + 1, 0);
        e = hipMemcpyAsync(d_s + o_codes, code_of, 512, hipMemcpyHostToDevice, hs);
        if (e != hipSuccess) return hip(e, "symbol codes");
        ke = bsk_fixed_block_esc((const uint16_t*)d_words, n, d_s + o_codes, nb, (uint32_t*)(d_s + o_esc), stream);
        if (ke) return hip((hipError_t)ke, "escape counts");
        if (nb) e = hipMemcpyAsync(esc.data(), d_s + o_esc, 4 * nb, hipMemcpyDeviceToHost, hs);
        if (e == hipSuccess) e = hipStreamSynchronize(hs);
        if (e != hipSuccess) return hip(e, "escape counts");
        uint64_t n_esc = 0;
        for (uint64_t b = 0; b < nb; b++) { first[b] = (uint32_t)n_esc; n_esc += esc[b]; }
        if (n_esc > 0xFFFFFFFFull) { set_error("more than 2^32 - 1 escapes"); return done(BS_E_INVAL); }
        const uint64_t len = align_up(esc_off + 2 * n_esc, 16);
        *out_len = len;
        if (capacity < len) {
            set_error("capacity %llu < %llu", (unsigned long long)capacity, (unsigned long long)len);
            return done(BS_E_NOSPACE);
        }
        std::vector<uint8_t> head(bsd::kFixHeader, 0), tail(len - esc_off - 2 * n_esc, 0);
        memcpy(head.data(), kFixMagic, 8);
        wr32(head.data() + 8, kFixVersion);
        wr64(head.data() + 16, n);
        wr64(head.data() + 24, nb);
        wr64(head.data() + 32, esc_off);
        wr64(head.data() + 40, n_esc);
        for (uint32_t k = 0; k < 16; k++) wr16(head.data() + 64 + 2 * k, table[k]);
        uint8_t* o = (uint8_t*)d_out;
        e = hipMemcpyAsync(o, head.data(), head.size(), hipMemcpyHostToDevice, hs);
        if (e == hipSuccess && nb)
            e = hipMemcpyAsync(o + bsd::kFixHeader + (uint64_t)bsd::kFixBlockBytes * nb, first.data(), 4 * nb,
                               hipMemcpyHostToDevice, hs);
        if (e == hipSuccess && nb) e = hipMemcpyAsync(d_s + o_first, first.data(), 4 * nb, hipMemcpyHostToDevice, hs);
        if (e == hipSuccess && !tail.empty())
            e = hipMemcpyAsync(o + esc_off + 2 * n_esc, tail.data(), tail.size(), hipMemcpyHostToDevice, hs);
        if (e != hipSuccess) return hip(e, "transcoder header");
        ke = bsk_fixed_pack((const uint16_t*)d_words, n, d_s + o_codes, nb, (const uint32_t*)(d_s + o_first), o, esc_off,
                            stream);
        if (ke) return hip((hipError_t)ke, "pack");
        e = hipStreamSynchronize(hs);                 // the host buffers above must outlive the copies
        if (e != hipSuccess) return hip(e, "transcode");
        return done(BS_OK);
    } catch (const std::bad_alloc&) {
        set_error("out of host memory");
        return done(BS_E_NOMEM);
    }
}

bs_status bs_fixed_info_get(const void* h_header, uint64_t header_len, uint64_t blob_len, bs_fixed_info* info) {
    if (!h_header || !info) { set_error("NULL argument"); return BS_E_INVAL; }
    const uint8_t* h = (const uint8_t*)h_header;
    if (header_len < bsd::kFixHeader || blob_len < bsd::kFixHeader || memcmp(h, kFixMagic, 8) != 0) {
        set_error("not a fixed-width blob");
        return BS_E_FORMAT;
    }
    if (rd32(h + 8) != kFixVersion) { set_error("fixed-width blob version %u", rd32(h + 8)); return BS_E_VERSION; }
    bs_fixed_info fi;
    memset(&fi, 0, sizeof fi);
    fi.n = rd64(h + 16);
    fi.n_blocks = rd64(h + 24);
    fi.esc_off = rd64(h + 32);
    fi.n_esc = rd64(h + 40);
    if (fi.n > (1ull << 50) || fi.n_blocks != fixed_blocks(fi.n) || fi.esc_off != fixed_esc_off(fi.n_blocks) ||
        fi.n_esc > fi.n || fi.n_esc > 0xFFFFFFFFull) {
        set_error("fixed-width header fields inconsistent");
        return BS_E_FORMAT;
    }
    fi.bytes = align_up(fi.esc_off + 2 * fi.n_esc, 16);
    if (fi.bytes > blob_len) { set_error("fixed-width blob truncated (%llu of %llu bytes)",
                                         (unsigned long long)blob_len, (unsigned long long)fi.bytes);
        return BS_E_FORMAT; }
    for (uint32_t k = 0; k < 16; k++) {
        fi.table[k] = (uint16_t)rd16(h + 64 + 2 * k);
        if (fi.table[k] > 511 || (k == 15 && fi.table[k] != 0)) { set_error("bad symbol table"); return BS_E_FORMAT; }
    }
    *info = fi;
    return BS_OK;
}

bs_status bs_fixed_decode_async(const bs_fixed_info* info, const void* d_blob, void* d_out, uint64_t out_capacity,
                                uint32_t* d_status, void* stream) {
    if (!info || !d_blob || (!d_out && info->n)) { set_error("NULL argument"); return BS_E_INVAL; }
    if ((uintptr_t)d_out & 15) { set_error("output must be 16-B aligned"); return BS_E_INVAL; }
    if (!info_consistent(info)) return BS_E_INVAL;
    if (out_capacity < 2 * info->n) { set_error("output capacity %llu < %llu", (unsigned long long)out_capacity,
                                                (unsigned long long)(2 * info->n));
        return BS_E_NOSPACE; }
    if (info->n == 0) return BS_OK;
    bsd::FixedArgs a;
    const bs_status rc = fixed_args(info, d_blob, a);
    if (rc != BS_OK) return rc;
    a.out = (uint16_t*)d_out;
    a.status = d_status;
    const int e = bsk_fixed_decode(&a, fixed_groups(info->n_blocks), stream);
    if (e != 0) { set_error("fixed decode launch: %s", hipGetErrorString((hipError_t)e)); return BS_E_HIP; }
    return BS_OK;
}

static_assert(bsd::kFixManyMax == BS_FIXED_MANY_MAX, "the header's limit is the kernel's");

bs_status bs_fixed_decode_many_async(const bs_fixed_info* infos, const void* const* d_blobs, void* const* d_outs,
                                     const uint64_t* out_capacities, uint32_t* const* d_status, uint32_t count,
                                     void* stream) {
    if (count > bsd::kFixManyMax) { set_error("%u blobs in one call (at most %u)", count, bsd::kFixManyMax); return BS_E_INVAL; }
    if (count && (!infos || !d_blobs || !d_outs || !out_capacities)) { set_error("NULL argument"); return BS_E_INVAL; }
    bsd::FixedMany m;
    memset(&m, 0, sizeof m);
    uint64_t blocks = 0;
    for (uint32_t i = 0; i < count; i++) {
        const bs_fixed_info* info = &infos[i];
        if (!d_outs[i] && info->n) { set_error("NULL output %u", i); return BS_E_INVAL; }
        if ((uintptr_t)d_outs[i] & 15) { set_error("output %u must be 16-B aligned", i); return BS_E_INVAL; }
        bsd::FixedArgs a;
        const bs_status rc = fixed_args(info, d_blobs[i], a);
        if (rc != BS_OK) return rc;
        if (out_capacities[i] < 2 * info->n) {
            set_error("output %u capacity %llu < %llu", i, (unsigned long long)out_capacities[i],
                      (unsigned long long)(2 * info->n));
            return BS_E_NOSPACE;
        }
        if (info->n == 0) continue;
        a.out = (uint16_t*)d_outs[i];
        a.status = d_status ? d_status[i] : nullptr;
        m.a[m.count++] = a;
        blocks += info->n_blocks;
    }
    if (m.count == 0) return BS_OK;
    // workgroups in proportion to blocks: at least one per tensor, never more
    // than its blocks need
    const uint64_t total = fixed_groups(blocks);
    uint32_t g = 0;
    for (uint32_t k = 0; k < m.count; k++) {
        const uint64_t nb = m.a[k].n_blocks;
        const uint64_t need = (nb + bsd::kFixWaves - 1) / bsd::kFixWaves;
        const uint64_t share = std::max<uint64_t>(1, (uint64_t)((unsigned __int128)total * nb / blocks));
        m.wg_start[k] = g;
        g += (uint32_t)std::min(need, share);
    }
    m.wg_start[m.count] = g;
    const int e = bsk_fixed_decode_many(&m, stream);
    if (e != 0) { set_error("fixed decode launch: %s", hipGetErrorString((hipError_t)e)); return BS_E_HIP; }
    return BS_OK;
}

bs_status bs_fixed_gemv_async(const bs_fixed_info* info, const void* d_blob, uint64_t rows, uint64_t cols,
                              const void* d_x, float* d_y, uint32_t* d_status, void* stream) {
    bsd::FixedArgs a;
    const bs_status rc = fixed_args(info, d_blob, a);
    if (rc != BS_OK) return rc;
    if (!d_x || !d_y) { set_error("NULL argument"); return BS_E_INVAL; }
    if (cols == 0 || cols % 32 || cols >= (1ull << 26) || info->n % cols || rows != info->n / cols) {
        set_error("a %llu x %llu matrix does not fit %llu weights with columns a multiple of 32 below 2^26",
                  (unsigned long long)rows, (unsigned long long)cols, (unsigned long long)info->n);
        return BS_E_INVAL;
    }
    if ((uintptr_t)d_x & 15) { set_error("x must be 16-B aligned"); return BS_E_INVAL; }
    a.status = d_status;
    a.gx = (const uint16_t*)d_x;
    a.gy = d_y;
    a.rows = rows;
    a.cols = (uint32_t)cols;
    // units of rows that end on a block boundary (lcm(cols, 2048) weights),
    // grouped so that a workgroup gets about one block per wave and at most
    // 64 rows
    uint64_t g = bsd::kFixBlockW, c = cols;
    while (c) { const uint64_t r = g % c; g = c; c = r; }
    a.unit_rows = (uint32_t)(bsd::kFixBlockW / g);
    a.unit_blocks = (uint32_t)(cols / g);
    a.group_units = std::max<uint32_t>(1, std::min<uint32_t>(bsd::kFixWaves / a.unit_blocks, 64 / a.unit_rows));
    const uint64_t grows = (uint64_t)a.unit_rows * a.group_units;
    a.n_groups = (rows + grows - 1) / grows;
    a.q_step = (uint32_t)(bsd::kFixWaves * bsd::kFixBlockW / cols);
    a.r_step = (uint32_t)(bsd::kFixWaves * bsd::kFixBlockW % cols);
    int cus = 0;
    if (bsk_device_cus(&cus) != 0 || cus <= 0) cus = 256;
    const uint32_t groups = (uint32_t)std::min<uint64_t>(a.n_groups, 16ull * (uint64_t)cus);
    const int e = bsk_fixed_gemv(&a, groups, stream);
    if (e != 0) { set_error("fixed product launch: %s", hipGetErrorString((hipError_t)e)); return BS_E_HIP; }
    return BS_OK;
}

uint64_t bs_fixed_gemm_work_bytes(uint64_t rows, uint64_t cols, uint32_t batch) {
    // the split product pays off once X's traffic counts: from batch 8
    // (4096 x 4096: 2-3% at batches 8-16, 11% at 20-24, level or slower
    // below 8), with at least two panels to share out
    if (rows == 0 || cols < 2 * bsd::kFixBlockW || cols % bsd::kFixBlockW || batch < 8 || batch > 64) return 0;
    return 4ull * batch * rows;
}

bs_status bs_fixed_gemm_async(const bs_fixed_info* info, const void* d_blob, uint64_t rows, uint64_t cols,
                              uint32_t batch, const void* d_x, float* d_y, uint32_t* d_status, void* d_work,
                              uint64_t work_bytes, void* stream) {
    bsd::FixedArgs a;
    const bs_status rc = fixed_args(info, d_blob, a);
    if (rc != BS_OK) return rc;
    if (!d_x || !d_y) { set_error("NULL argument"); return BS_E_INVAL; }
    if (cols == 0 || cols % bsd::kFixBlockW || cols >= (1ull << 26) || info->n % cols || rows != info->n / cols) {
        set_error("a %llu x %llu matrix does not fit %llu weights with columns a multiple of 2048 below 2^26",
                  (unsigned long long)rows, (unsigned long long)cols, (unsigned long long)info->n);
        return BS_E_INVAL;
    }
    if (batch == 0 || batch > 64) { set_error("batch %u outside 1..64", batch); return BS_E_INVAL; }
    if (rows >= (1ull << 26)) { set_error("%llu rows, at most 2^26 - 1", (unsigned long long)rows); return BS_E_INVAL; }
    if ((uintptr_t)d_x & 15) { set_error("X must be 16-B aligned"); return BS_E_INVAL; }
    a.status = d_status;
    a.gx = (const uint16_t*)d_x;
    a.gy = d_y;
    a.rows = rows;
    a.cols = (uint32_t)cols;
    a.batch = batch;
    a.ksplit = 1;
    a.gpart = nullptr;
    // the split product: 32 rows per work item, two items per group of rows
    // (cols >= 4096), given a workspace for the second half's sums
    const uint64_t groups32 = (rows + 31) / 32;
    const bool split = d_work != nullptr && cols >= 2 * bsd::kFixBlockW;
    if (split) {
        if ((uintptr_t)d_work & 255) { set_error("the workspace must be 256-B aligned"); return BS_E_INVAL; }
        if (work_bytes < 4ull * batch * rows) {
            set_error("workspace of %llu B, %llu B needed", (unsigned long long)work_bytes,
                      (unsigned long long)(4ull * batch * rows));
            return BS_E_INVAL;
        }
        const uintptr_t w0 = (uintptr_t)d_work, y0 = (uintptr_t)d_y, sz = (uintptr_t)(4ull * batch * rows);
        if (w0 < y0 + sz && y0 < w0 + sz) { set_error("the workspace overlaps Y"); return BS_E_INVAL; }
        a.ksplit = 2;
        a.gpart = (float*)d_work;
    }
    int cus = 0;
    if (bsk_device_cus(&cus) != 0 || cus <= 0) cus = 256;
    const uint64_t items = split ? 2 * groups32 : (rows + 15) / 16;
    const uint32_t groups = (uint32_t)std::min<uint64_t>(items, 8ull * (uint64_t)cus);
    const int e = bsk_fixed_gemm(&a, groups, split ? 1 : 0, stream);
    if (e != 0) { set_error("fixed batched product launch: %s", hipGetErrorString((hipError_t)e)); return BS_E_HIP; }
    return BS_OK;
}

}  // extern "C"
