// bs_plan.cpp -- decode plans, the decode entry point and verification.
//
// A plan holds, in device memory, the validated record descriptors of a
// container, grouped by lanes-per-thread class with each class's running chunk
// count, and each record's decode lookup tables, built once by a HIP kernel.
// Decoding a record range is then one kernel launch per class present (each
// workgroup takes a run of chunks inside one record) plus
// one for the verbatim residual spans [Qwen3.8-27B-BF16-NVLC-Lossless card,
// codec paragraph: the residual keeps non-BF16 spans].  A decode call uploads
// nothing.
// Verification re-reads the per-chunk status, compares bytes on the device and
// checks each record's sha256 [Gemma 2 9B Instruct -- Lossless Compressed
// card, "What lossless means": every tensor is hash-checked at decompression].
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "bs_device.h"
#include "bs_internal.h"
#include "bs_model.h"

using namespace bs;

struct bs_plan {
    int device = 0;
    const uint8_t* d_container = nullptr;
    uint64_t len = 0;
    Container c;
    // one record list per launch class: records with 1, 2 or 4 lanes per
    // thread share one kernel (16-wave workgroups), in the full or the compact
    // LDS layout; eight lanes per thread have their own (8-wave workgroups)
    // layout; records of layout 2 (one renormalisation per weight) form the
    // fourth class, with their own kernel, and records of layout 3 (the same
    // with one joint symbol per weight) the fifth, with that kernel's
    // joint-symbol instances
    static constexpr int kClasses = 5;
    static constexpr uint32_t kMaxR[kClasses] = {4, 4, 8, 4, 4};
    static constexpr bool kCompact[kClasses] = {false, true, false, false, false};
    static constexpr int kLayout2 = 3;
    static constexpr int kLayout3 = 4;
    int cus = 256;
    std::vector<uint32_t> dev_index;   // record -> index in d_recs (BF16) or d_raws (RAW)
    std::vector<uint32_t> rclass;      // record -> class (BF16)
    std::vector<uint32_t> cls_pos;     // record -> entry in its class list (BF16)
    std::vector<uint32_t> cls_recs[kClasses], cls_start[kClasses];
    std::vector<uint32_t> cls_R[kClasses];   // lanes per thread of each class entry
    std::vector<bsd::RawDev> raws;
    std::vector<bsd::RecDev> h_recs;   // host copy of d_recs (a launch of one record passes it by value)
    bsd::RecDev* d_recs = nullptr;
    uint32_t* d_cls_recs[kClasses] = {};
    uint32_t* d_cls_start[kClasses] = {};
    bsd::RawDev* d_raws = nullptr;
    uint8_t* d_luts = nullptr;
    unsigned long long* d_cmp = nullptr;   // compare results (2 words)
    uint64_t device_bytes = 0;             // everything allocated above
};

namespace {

// a packed small record's start (table staging, unit opening) in lane steps
constexpr uint32_t kPackStartSteps = 64;

void plan_free(bs_plan* p) {
    if (!p) return;
    if (p->d_recs) (void)hipFree(p->d_recs);
    for (int k = 0; k < bs_plan::kClasses; k++) {
        if (p->d_cls_recs[k]) (void)hipFree(p->d_cls_recs[k]);
        if (p->d_cls_start[k]) (void)hipFree(p->d_cls_start[k]);
    }
    if (p->d_raws) (void)hipFree(p->d_raws);
    if (p->d_luts) (void)hipFree(p->d_luts);
    if (p->d_cmp) (void)hipFree(p->d_cmp);
    delete p;
}

bs_status hip_err(hipError_t e, const char* what) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return BS_E_HIP;
}

// records [first, first+count) -> the run of class entries [e0, e1) of each
// class (class lists keep container order) and the residual range [r0, r1)
void ranges(const bs_plan* p, uint32_t first, uint32_t count, uint32_t* e0, uint32_t* e1, uint32_t& r0,
            uint32_t& r1) {
    r0 = r1 = 0;
    bool have_e[bs_plan::kClasses] = {}, have_r = false;
    for (int k = 0; k < bs_plan::kClasses; k++) e0[k] = e1[k] = 0;
    for (uint32_t i = first; i < first + count; i++) {
        const Record& r = p->c.recs[i];
        if (r.kind == BS_KIND_BF16) {
            const uint32_t k = p->rclass[i];
            if (!have_e[k]) { e0[k] = p->cls_pos[i]; have_e[k] = true; }
            e1[k] = p->cls_pos[i] + 1;
        } else {
            if (!have_r) { r0 = p->dev_index[i]; have_r = true; }
            r1 = p->dev_index[i] + 1;
        }
    }
}

// Launch shape for the class entries [e0, e1) of class k: every record is cut
// into runs of `run` units (chunk streams), one workgroup per run (a workgroup's tables and
// rings fill a CU's LDS, or half of it in the compact layout).  `run` is the
// smallest length whose run count fits the workgroups that run at once; when
// the records alone outnumber those, runs are sized to the average share.
//
// Small records next to large ones (a layer's norm vectors beside its
// matrices, layouts 2 and 3): a record of at most `waves` units decodes in
// one round of a workgroup, far sooner than a run of a large record, and would
// leave its CU idle for the rest of the launch.  Such records are packed
// `pack` to a workgroup, which decodes them one after another (each with its
// own table image), and the large records' runs spread over the other CUs.
// A pack is sized so that its records, timed as lane steps of a lone wave,
// take at most half as long as a large run's lane steps (a wave on a loaded
// CU steps about three times slower than a lone one).  small = 0: no packing.
void launch_shape(const bs_plan* p, int k, uint32_t e0, uint32_t e1, uint32_t& waves, uint32_t& run,
                  uint32_t& groups, uint32_t& small, uint32_t& pack) {
    const std::vector<uint32_t>& st = p->cls_start[k];
    auto units = [&](uint32_t e) { return st[e + 1] - st[e]; };
    // workgroups that run at once: one per CU, or two in the compact layout
    // when their registers allow it (up to 2 lanes per thread)
    uint32_t rmax = 0;
    for (uint32_t e = e0; e < e1; e++) rmax = std::max(rmax, p->cls_R[k][e]);
    const uint32_t cus = (uint32_t)p->cus * (bs_plan::kCompact[k] && rmax <= 2 ? 2 : 1);
    // the shortest run whose workgroup count over the records with big(e)
    // fits `slots`, and that count
    auto fit = [&](uint32_t slots, auto big, uint32_t& len, uint32_t& count) {
        uint64_t total = 0;
        uint32_t biggest = 0;
        for (uint32_t e = e0; e < e1; e++)
            if (big(e)) { total += units(e); biggest = std::max(biggest, units(e)); }
        auto cnt = [&](uint32_t l) {
            uint64_t g = 0;
            for (uint32_t e = e0; e < e1; e++)
                if (big(e)) g += (units(e) + l - 1) / l;
            return g;
        };
        uint32_t lo = (uint32_t)std::max<uint64_t>(1, (total + slots - 1) / slots), hi = std::max(lo, biggest);
        if (cnt(hi) > slots) {
            len = lo;
        } else {
            while (lo < hi) {
                const uint32_t mid = lo + (hi - lo) / 2;
                if (cnt(mid) <= slots) hi = mid; else lo = mid + 1;
            }
            len = lo;
        }
        count = (uint32_t)cnt(len);
    };
    // waves per workgroup: a layout-2 or -3 workgroup's rings follow its
    // records' table image, whose size varies: as many as fit after the largest
    uint32_t wlim = bsd::max_waves(bs_plan::kMaxR[k]);
    const bool l23 = k == bs_plan::kLayout2 || k == bs_plan::kLayout3;
    if (l23) {
        uint32_t rb = 0;
        for (uint32_t e = e0; e < e1; e++) {
            const bsd::RecDev& d = p->h_recs[p->cls_recs[k][e]];
            rb = std::max(rb, k == bs_plan::kLayout3 ? bsd::l3_ring_base(d.m_s) : bsd::l2_ring_base(d.m_s, d.n_tables));
        }
        wlim = std::min(wlim, bsd::l2_max_waves(rb));
    }
    fit(cus, [](uint32_t) { return true; }, run, groups);
    waves = std::min(wlim, run);
    small = pack = 0;
    if (!l23 || e1 - e0 < 2) return;

    // lane steps of a record's unit: the weights of a chunk's lane
    auto steps = [&](uint32_t e) {
        const bsd::RecDev& d = p->h_recs[p->cls_recs[k][e]];
        return (uint32_t)((std::min<uint64_t>(d.n, d.W) + d.K - 1) / d.K);
    };
    auto is_small = [&](uint32_t e) { return units(e) != 0 && units(e) <= wlim; };
    uint32_t n_small = 0, c_small = 0, s_big = 0;
    for (uint32_t e = e0; e < e1; e++) {
        if (is_small(e)) { n_small++; c_small = std::max(c_small, steps(e) + kPackStartSteps); }
        else if (units(e)) s_big = std::max(s_big, steps(e));
    }
    if (n_small == 0 || s_big == 0) return;
    auto big = [&](uint32_t e) { return units(e) > wlim; };
    for (uint32_t np = 1; np < cus && np <= n_small;) {
        uint32_t len, count;
        fit(cus - np, big, len, count);
        if (len < wlim) return;                                   // large runs of a single round: nothing to gain
        const uint64_t budget = 3ull * ((len + wlim - 1) / wlim) * s_big / 2;
        const uint32_t per = (uint32_t)std::min<uint64_t>(budget / c_small, n_small);
        if (per < 2) return;
        const uint32_t need = (n_small + per - 1) / per;
        if (need <= np) {
            run = len;
            waves = wlim;
            groups = count + need;
            small = wlim;
            pack = per;
            return;
        }
        np = need;
    }
}

uint64_t out_extent(const bs_plan* p, uint32_t first, uint32_t count) {
    if (!count) return 0;
    const uint64_t base = p->c.recs[first].out_offset;
    uint64_t e = 0;
    for (uint32_t i = first; i < first + count; i++) {
        const Record& r = p->c.recs[i];
        if (r.out_offset < base) return UINT64_MAX;   // records must ascend in output offset
        e = std::max(e, r.out_offset + r.out_bytes() - base);
    }
    return e;
}

}  // namespace

extern "C" {

bs_status bs_plan_create(const void* h_container, uint64_t len, const void* d_container, void* stream,
                         bs_plan** out) {
    if (!out || !h_container || !d_container) { set_error("NULL argument"); return BS_E_INVAL; }
    if ((uintptr_t)d_container & 15) { set_error("device container must be 16-byte aligned"); return BS_E_INVAL; }
    bs_plan* p = new (std::nothrow) bs_plan();
    if (!p) return BS_E_NOMEM;
    bs_status rc = parse_container((const uint8_t*)h_container, len, p->c);
    if (rc) { delete p; return rc; }
    p->d_container = (const uint8_t*)d_container;
    p->len = len;
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) { plan_free(p); return hip_err(e, "hipGetDevice"); }
    int cus = 0;
    if (bsk_device_cus(&cus) != 0 || cus <= 0) cus = 256;
    p->cus = cus;
    const uint32_t n = p->c.n_records;
    if (p->c.n_streams > 0xFFFFFFFFull) { plan_free(p); set_error("too many chunk streams"); return BS_E_FORMAT; }
    std::vector<bsd::RecDev> recs;
    uint64_t lut_bytes = 0;
    p->dev_index.assign(n, 0);
    p->rclass.assign(n, 0);
    p->cls_pos.assign(n, 0);
    for (int k = 0; k < bs_plan::kClasses; k++) p->cls_start[k].push_back(0);
    for (uint32_t i = 0; i < n; i++) {
        const Record& r = p->c.recs[i];
        if (r.kind == BS_KIND_RAW) {
            p->dev_index[i] = (uint32_t)p->raws.size();
            p->raws.push_back({r.rec_offset, r.out_offset, r.n});
            continue;
        }
        p->dev_index[i] = (uint32_t)recs.size();
        bsd::RecDev d{};
        d.body = r.rec_offset;
        d.index_off = r.index_off;
        d.out_off = r.out_offset;
        d.n = r.n;
        d.lut_off = lut_bytes;
        d.W = r.W;
        d.K = r.K;
        d.n_chunks = r.n_chunks;
        d.status_base = (uint32_t)r.stream_base;
        d.m_s = r.m_s;
        d.m_f = r.m_f;
        d.n_tables = r.n_tables;
        d.streams_log2 = 0;
        while ((1u << d.streams_log2) < r.S) d.streams_log2++;
        d.P = r.K / r.S;
        d.lanes_per_thread = d.P <= 64 ? 1 : d.P / 64;
        d.n_sym = r.n_sym;
        d.stab_off = r.stab_off;
        d.route_off = r.route_off;
        d.ftab_off = r.ftab_off;
        const uint32_t R = d.lanes_per_thread;
        d.layout = r.layout;
        uint32_t k;
        if (r.layout >= 2) {
            if (R > 4) {
                plan_free(p);
                set_error("record %u: layout %u decodes with at most 256 lanes per word stream (it has %u)", i, r.layout,
                          d.P);
                return BS_E_INVAL;
            }
            d.compact = 0;
            lut_bytes += r.layout == 3 ? bsd::l3_ring_base(r.m_s) : bsd::l2_ring_base(r.m_s, r.n_tables);
            k = r.layout == 3 ? bs_plan::kLayout3 : bs_plan::kLayout2;
        } else {
            d.compact = R <= 4 && r.m_s <= 11 && r.m_f <= 9;
            lut_bytes += (8ull << r.m_s) + (r.n_tables + 1ull) * bsd::fpage_bytes(d.compact);
            k = R == 8 ? 2 : d.compact ? 1 : 0;
        }
        p->rclass[i] = k;
        p->cls_pos[i] = (uint32_t)p->cls_recs[k].size();
        p->cls_recs[k].push_back((uint32_t)recs.size());
        p->cls_R[k].push_back(R);
        p->cls_start[k].push_back(p->cls_start[k].back() + r.n_chunks * r.S);
        recs.push_back(d);
    }
    hipStream_t s = (hipStream_t)stream;
    auto up = [&](void** dst, const void* src, size_t bytes) -> hipError_t {
        hipError_t ee = hipMalloc(dst, std::max<size_t>(bytes, 16));
        p->device_bytes += std::max<size_t>(bytes, 16);
        if (ee != hipSuccess || !bytes) return ee;
        return hipMemcpyAsync(*dst, src, bytes, hipMemcpyHostToDevice, s);
    };
    p->h_recs = recs;
    e = up((void**)&p->d_recs, recs.data(), recs.size() * sizeof(bsd::RecDev));
    for (int k = 0; k < bs_plan::kClasses && e == hipSuccess; k++) {
        e = up((void**)&p->d_cls_recs[k], p->cls_recs[k].data(), p->cls_recs[k].size() * 4);
        if (e == hipSuccess) e = up((void**)&p->d_cls_start[k], p->cls_start[k].data(), p->cls_start[k].size() * 4);
    }
    if (e == hipSuccess) e = up((void**)&p->d_raws, p->raws.data(), p->raws.size() * sizeof(bsd::RawDev));
    if (e == hipSuccess) e = hipMalloc(&p->d_luts, std::max<uint64_t>(lut_bytes, 16));
    if (e == hipSuccess) e = hipMalloc(&p->d_cmp, 2 * sizeof(unsigned long long));
    p->device_bytes += std::max<uint64_t>(lut_bytes, 16) + 2 * sizeof(unsigned long long);
    if (e == hipSuccess) e = (hipError_t)bsk_build_luts(p->d_container, p->d_recs, (uint32_t)recs.size(), p->d_luts, stream);
    // the host vectors passed to the copies above must outlive them
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        rc = hip_err(e, "plan upload");
        plan_free(p);
        return rc;
    }
    *out = p;
    return BS_OK;
}

void bs_plan_destroy(bs_plan* plan) { plan_free(plan); }

bs_status bs_plan_rebind(bs_plan* plan, const void* d_container) {
    if (!plan || !d_container) { set_error("NULL argument"); return BS_E_INVAL; }
    if ((uintptr_t)d_container & 15) { set_error("device container must be 16-byte aligned"); return BS_E_INVAL; }
    plan->d_container = (const uint8_t*)d_container;
    return BS_OK;
}

uint64_t bs_plan_container_bytes(const bs_plan* plan) { return plan ? plan->len : 0; }

}  // extern "C"

namespace bs {
uint64_t plan_device_bytes(const bs_plan* plan) { return plan ? plan->device_bytes : 0; }
uint64_t plan_status_words(const bs_plan* plan) { return plan ? plan->c.n_streams : 0; }
uint32_t plan_records(const bs_plan* plan) { return plan ? plan->c.n_records : 0; }
}  // namespace bs

extern "C" {

uint32_t bs_plan_waves_per_block(const bs_plan* plan) {
    if (!plan) return 0;
    uint32_t w = 0;
    for (int k = 0; k < bs_plan::kClasses; k++) {
        if (!plan->cls_start[k].back()) continue;
        uint32_t waves, run, groups, small, pack;
        launch_shape(plan, k, 0, (uint32_t)plan->cls_recs[k].size(), waves, run, groups, small, pack);
        w = std::max(w, waves);
    }
    return w;
}

uint32_t bs_plan_packs(const bs_plan* plan, uint32_t first, uint32_t count) {
    if (!plan || first > plan->c.n_records || count > plan->c.n_records - first || !count) return 0;
    uint32_t e0[bs_plan::kClasses], e1[bs_plan::kClasses], r0, r1;
    ranges(plan, first, count, e0, e1, r0, r1);
    uint32_t n = 0;
    for (int k = 0; k < bs_plan::kClasses; k++) {
        if (e1[k] <= e0[k] || plan->cls_start[k][e1[k]] <= plan->cls_start[k][e0[k]]) continue;
        uint32_t waves, run, groups, small, pack;
        launch_shape(plan, k, e0[k], e1[k], waves, run, groups, small, pack);
        if (!pack) continue;
        uint32_t n_small = 0;
        for (uint32_t e = e0[k]; e < e1[k]; e++) {
            const uint32_t u = plan->cls_start[k][e + 1] - plan->cls_start[k][e];
            n_small += u != 0 && u <= small;
        }
        n += (n_small + pack - 1) / pack;
    }
    return n;
}

uint64_t bs_plan_out_bytes(const bs_plan* plan, uint32_t first, uint32_t count) {
    if (!plan || first > plan->c.n_records || count > plan->c.n_records - first) return 0;
    return out_extent(plan, first, count);
}

bs_status bs_decode_async(const bs_plan* p, uint32_t first, uint32_t count, void* d_out, uint64_t out_capacity,
                          uint32_t* d_status, void* stream) {
    if (!p || (!d_out && count) || (!d_status && p->c.n_streams)) { set_error("NULL argument"); return BS_E_INVAL; }
    if (first > p->c.n_records || count > p->c.n_records - first) { set_error("record range out of bounds"); return BS_E_INVAL; }
    if ((uintptr_t)d_out & 15) { set_error("output must be 16-byte aligned"); return BS_E_INVAL; }
    if (!count) return BS_OK;
    const uint64_t need = out_extent(p, first, count);
    if (need == UINT64_MAX) { set_error("records of the range do not ascend in output offset"); return BS_E_INVAL; }
    if (need > out_capacity) {
        set_error("output needs %llu bytes, capacity is %llu", (unsigned long long)need, (unsigned long long)out_capacity);
        return BS_E_NOSPACE;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != p->device) { set_error("plan belongs to device %d", p->device); return BS_E_INVAL; }
    uint32_t e0[bs_plan::kClasses], e1[bs_plan::kClasses], r0, r1;
    ranges(p, first, count, e0, e1, r0, r1);
    const uint64_t out_base = p->c.recs[first].out_offset;
    for (int k = 0; k < bs_plan::kClasses; k++) {
        if (e1[k] <= e0[k]) continue;
        if (p->cls_start[k][e1[k]] <= p->cls_start[k][e0[k]]) continue;
        bsd::DecodeArgs a{};
        a.container = p->d_container;
        a.recs = p->d_recs;
        a.cls.recs = p->d_cls_recs[k];
        a.cls.start = p->d_cls_start[k];
        a.luts = p->d_luts;
        a.out = (uint8_t*)d_out;
        a.status = d_status;
        a.out_base = out_base;
        a.i0 = e0[k];
        a.i1 = e1[k];
        if (e1[k] - e0[k] == 1) a.one = p->h_recs[p->cls_recs[k][e0[k]]];
        uint32_t groups;
        launch_shape(p, k, e0[k], e1[k], a.waves, a.run, groups, a.small_units, a.pack);
        // the specialised kernel when every record of the launch has the same
        // lanes per thread, else the mixed one
        uint32_t rmin = 8, rmax = 0;
        for (uint32_t i = e0[k]; i < e1[k]; i++) {
            const uint32_t R = p->cls_R[k][i];
            rmin = std::min(rmin, R);
            rmax = std::max(rmax, R);
        }
        const uint32_t variant = rmin == rmax ? rmax : rmax <= 2 ? 0 : 3;
        int e = k == bs_plan::kLayout2   ? bsk_decode2(&a, groups, variant, stream)
                : k == bs_plan::kLayout3 ? bsk_decode3(&a, groups, variant, stream)
                                         : bsk_decode(&a, groups, variant, bs_plan::kCompact[k], stream);
        if (e) return hip_err((hipError_t)e, "decode launch");
    }
    if (r1 > r0) {
        int e = bsk_raw_copy(p->d_container, p->d_raws + r0, r1 - r0, (uint8_t*)d_out, out_base, stream);
        if (e) return hip_err((hipError_t)e, "residual copy launch");
    }
    return BS_OK;
}

bs_status bs_gemv_async(const bs_plan* p, uint32_t record, uint64_t rows, uint64_t cols, const void* d_x, float* d_y,
                        uint32_t* d_status, void* stream) {
    if (!p || !d_x || !d_y || (!d_status && p->c.n_streams)) { set_error("NULL argument"); return BS_E_INVAL; }
    if (record >= p->c.n_records) { set_error("record %u out of range", record); return BS_E_INVAL; }
    const Record& rec = p->c.recs[record];
    if (rec.kind != BS_KIND_BF16) { set_error("record %u is not a BF16 record", record); return BS_E_INVAL; }
    if (cols < 512 || cols % 8 || rows == 0 || rows * cols != rec.n || rec.n / cols != rows) {
        set_error("record %u holds %llu weights: not a %llu x %llu matrix with a multiple of 8 (at least 512) columns",
                  record, (unsigned long long)rec.n, (unsigned long long)rows, (unsigned long long)cols);
        return BS_E_INVAL;
    }
    if (((uintptr_t)d_x & 15) || ((uintptr_t)d_y & 3)) { set_error("x must be 16-byte aligned, y 4-byte aligned"); return BS_E_INVAL; }
    const int k = (int)p->rclass[record];
    if (bs_plan::kCompact[k] || bs_plan::kMaxR[k] > 4) {
        set_error("the fused product runs on records in the full table layout with at most 4 lanes per thread");
        return BS_E_INVAL;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != p->device) { set_error("plan belongs to device %d", p->device); return BS_E_INVAL; }
    const uint32_t e = p->cls_pos[record];
    bsd::DecodeArgs a{};
    a.container = p->d_container;
    a.recs = p->d_recs;
    a.cls.recs = p->d_cls_recs[k];
    a.cls.start = p->d_cls_start[k];
    a.luts = p->d_luts;
    a.out = nullptr;
    a.status = d_status;
    a.out_base = rec.out_offset;
    a.i0 = e;
    a.i1 = e + 1;
    a.one = p->h_recs[p->cls_recs[k][e]];
    a.gx = (const uint16_t*)d_x;
    a.gy = d_y;
    a.gcols = cols;
    uint32_t groups, small, pack;
    launch_shape(p, k, e, e + 1, a.waves, a.run, groups, small, pack);
    if (p->cls_start[k][e + 1] == p->cls_start[k][e]) groups = 0;
    const int err = k == bs_plan::kLayout2   ? bsk_gemv2(&a, groups, p->cls_R[k][e], rows, stream)
                    : k == bs_plan::kLayout3 ? bsk_gemv3(&a, groups, p->cls_R[k][e], rows, stream)
                                             : bsk_gemv(&a, groups, p->cls_R[k][e], rows, stream);
    if (err) return hip_err((hipError_t)err, "fused product launch");
    return BS_OK;
}

bs_status bs_verify(const bs_plan* p, uint32_t first, uint32_t count, const void* d_out, const void* d_ref,
                    const uint32_t* d_status, uint32_t flags, void* stream, bs_report* rep) {
    if (!p || !rep) { set_error("NULL argument"); return BS_E_INVAL; }
    if (first > p->c.n_records || count > p->c.n_records - first) { set_error("record range out of bounds"); return BS_E_INVAL; }
    memset(rep, 0, sizeof(*rep));
    rep->first_bad_chunk = UINT64_MAX;
    rep->first_mismatch = UINT64_MAX;
    rep->first_hash_bad = UINT32_MAX;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_err(e, "stream");
    const uint64_t base = count ? p->c.recs[first].out_offset : 0;
    bool corrupt = false, mismatch = false;
    if ((flags & BS_VERIFY_STATUS) && count) {
        if (!d_status && p->c.n_streams) { set_error("NULL status"); return BS_E_INVAL; }
        for (uint32_t i = first; i < first + count; i++) {
            const Record& r = p->c.recs[i];
            if (r.kind != BS_KIND_BF16 || !r.n_chunks) continue;
            std::vector<uint32_t> st((size_t)r.n_chunks * r.S);
            e = hipMemcpy(st.data(), d_status + r.stream_base, 4ull * st.size(), hipMemcpyDeviceToHost);
            if (e != hipSuccess) return hip_err(e, "status read-back");
            for (uint32_t k = 0; k < r.n_chunks; k++) {
                rep->chunks_checked++;
                bool bad = false;
                for (uint32_t s2 = 0; s2 < r.S; s2++) bad |= st[(size_t)k * r.S + s2] != 0;
                if (bad) {
                    rep->chunks_bad++;
                    rep->first_bad_chunk = std::min<uint64_t>(rep->first_bad_chunk, r.chunk_base + k);
                    corrupt = true;
                }
            }
        }
    }
    if ((flags & BS_VERIFY_COMPARE) && count) {
        if (!d_out || !d_ref) { set_error("compare needs d_out and d_ref"); return BS_E_INVAL; }
        for (uint32_t i = first; i < first + count; i++) {
            const Record& r = p->c.recs[i];
            const uint64_t off = r.out_offset - base, nb = r.out_bytes();
            if (!nb) continue;
            unsigned long long res[2] = {0, ~0ull};
            e = hipMemcpyAsync(p->d_cmp, res, sizeof(res), hipMemcpyHostToDevice, s);
            if (e == hipSuccess)
                e = (hipError_t)bsk_compare((const uint8_t*)d_out + off, (const uint8_t*)d_ref + off, nb, p->d_cmp, stream);
            if (e == hipSuccess) e = hipMemcpyAsync(res, p->d_cmp, sizeof(res), hipMemcpyDeviceToHost, s);
            if (e == hipSuccess) e = hipStreamSynchronize(s);
            if (e != hipSuccess) return hip_err(e, "compare");
            rep->bytes_compared += nb;
            if (res[0]) {
                mismatch = true;
                rep->bytes_mismatched += res[0];
                rep->first_mismatch = std::min<uint64_t>(rep->first_mismatch, off + res[1]);
            }
        }
    }
    if ((flags & BS_VERIFY_SHA256) && count) {
        if (!d_out) { set_error("sha256 check needs d_out"); return BS_E_INVAL; }
        std::vector<uint8_t> host;
        for (uint32_t i = first; i < first + count; i++) {
            const Record& r = p->c.recs[i];
            const uint64_t nb = r.out_bytes();
            try { host.resize(nb); } catch (const std::bad_alloc&) { set_error("out of host memory"); return BS_E_NOMEM; }
            if (nb) {
                e = hipMemcpy(host.data(), (const uint8_t*)d_out + (r.out_offset - base), nb, hipMemcpyDeviceToHost);
                if (e != hipSuccess) return hip_err(e, "read-back");
            }
            uint8_t dg[32];
            sha256(host.data(), nb, dg);
            rep->records_hashed++;
            if (memcmp(dg, r.sha, 32) != 0) {
                rep->records_hash_bad++;
                rep->first_hash_bad = std::min(rep->first_hash_bad, i);
                mismatch = true;
            }
        }
    }
    if (corrupt) return BS_E_CORRUPT;
    if (mismatch) return BS_E_MISMATCH;
    return BS_OK;
}

}  // extern "C"
