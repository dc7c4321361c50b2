// bs_stream.cpp -- layers streamed on demand under a device-memory budget.
//
// [Gemma 2 9B Instruct -- Lossless Compressed card, "Low-VRAM streaming":
// layers are streamed on demand with an LRU bound on the device memory they
// use.]  The containers stay in pinned host memory.  A layer that is not
// resident is copied into one of two device staging buffers on the
// streamer's copy stream and decoded on the caller's stream into a fixed-size
// slot; the least recently used slot that is not acquired is reused.  HIP
// events order everything:
//   - a copy into a staging buffer waits for the decode that last read it;
//   - a decode waits for its copy and for the last release of the slot's
//     previous layer;
//   - a hit from another stream waits for the slot's decode, and so does a
//     decode into a slot whose last decode ran on another stream (a layer
//     prefetched there and never acquired has no release to wait for).
// Every buffer is allocated at creation; nothing on the acquire path
// allocates or synchronises the host.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "bs_internal.h"

using namespace bs;

struct bs_streamer {
    uint32_t n_layers = 0;
    uint8_t* h_arena = nullptr;               // pinned copies of the containers
    std::vector<uint8_t*> h_ptr;
    std::vector<uint64_t> len;
    std::vector<bs_plan*> plans;
    std::vector<uint32_t> n_records;
    uint32_t* d_status = nullptr;             // every layer's stream status words
    std::vector<uint64_t> status_off;
    uint64_t slot_bytes = 0, staging_bytes = 0;
    uint32_t n_slots = 0;
    uint8_t* d_slots = nullptr;
    uint8_t* d_staging[2] = {nullptr, nullptr};
    hipStream_t copy_stream = nullptr;
    hipEvent_t ev_copied[2] = {nullptr, nullptr}, ev_staging_free[2] = {nullptr, nullptr};
    bool staging_used[2] = {false, false};
    uint32_t next_staging = 0;
    std::vector<hipEvent_t> ev_ready, ev_free;  // per slot
    std::vector<uint8_t> free_recorded;         // ev_free recorded during the slot's current layer
    std::vector<uint8_t> free_ever;             // ev_free recorded at all
    std::vector<int64_t> slot_layer;            // layer held, -1 if none
    std::vector<uint32_t> pins;
    std::vector<uint64_t> stamp;                // last use, for LRU
    std::vector<hipStream_t> decoded_on;
    std::vector<uint8_t> decoded_ever;          // ev_ready recorded at all
    std::vector<int64_t> layer_slot;            // slot of a layer, -1 if not resident
    uint64_t clock = 0;
    bs_streamer_stats st{};
};

namespace {

bs_status hip_fail(hipError_t e, const char* what) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return BS_E_HIP;
}

void streamer_free(bs_streamer* s) {
    if (!s) return;
    (void)hipDeviceSynchronize();
    for (bs_plan* p : s->plans) bs_plan_destroy(p);
    for (int j = 0; j < 2; j++) {
        if (s->ev_copied[j]) (void)hipEventDestroy(s->ev_copied[j]);
        if (s->ev_staging_free[j]) (void)hipEventDestroy(s->ev_staging_free[j]);
        if (s->d_staging[j]) (void)hipFree(s->d_staging[j]);
    }
    for (hipEvent_t e : s->ev_ready)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : s->ev_free)
        if (e) (void)hipEventDestroy(e);
    if (s->copy_stream) (void)hipStreamDestroy(s->copy_stream);
    if (s->d_slots) (void)hipFree(s->d_slots);
    if (s->d_status) (void)hipFree(s->d_status);
    if (s->h_arena) (void)hipHostFree(s->h_arena);
    delete s;
}

// the unacquired slot used longest ago (empty slots first), or -1
int64_t victim(const bs_streamer* s) {
    int64_t best = -1;
    for (uint32_t k = 0; k < s->n_slots; k++) {
        if (s->pins[k]) continue;
        if (best < 0 || s->stamp[k] < s->stamp[best]) best = k;
    }
    return best;
}

// copy layer's container to a staging buffer and decode it into slot k on `stream`
bs_status load(bs_streamer* s, uint32_t layer, uint32_t k, hipStream_t stream) {
    const uint32_t j = s->next_staging;
    s->next_staging ^= 1u;
    hipError_t e = hipSuccess;
    if (s->staging_used[j]) e = hipStreamWaitEvent(s->copy_stream, s->ev_staging_free[j], 0);
    if (e == hipSuccess)
        e = hipMemcpyAsync(s->d_staging[j], s->h_ptr[layer], s->len[layer], hipMemcpyHostToDevice, s->copy_stream);
    if (e == hipSuccess) e = hipEventRecord(s->ev_copied[j], s->copy_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, s->ev_copied[j], 0);
    if (e == hipSuccess && s->free_ever[k]) e = hipStreamWaitEvent(stream, s->ev_free[k], 0);
    if (e == hipSuccess && s->decoded_ever[k] && s->decoded_on[k] != stream)
        e = hipStreamWaitEvent(stream, s->ev_ready[k], 0);
    if (e != hipSuccess) return hip_fail(e, "streamer copy");
    if (s->slot_layer[k] >= 0) {
        s->layer_slot[s->slot_layer[k]] = -1;
        s->st.evictions++;
    }
    s->slot_layer[k] = -1;
    bs_status rc = bs_plan_rebind(s->plans[layer], s->d_staging[j]);
    if (rc == BS_OK)
        rc = bs_decode_async(s->plans[layer], 0, s->n_records[layer], s->d_slots + (uint64_t)k * s->slot_bytes,
                             s->slot_bytes, s->d_status + s->status_off[layer], stream);
    if (rc != BS_OK) return rc;
    e = hipEventRecord(s->ev_staging_free[j], stream);
    if (e == hipSuccess) e = hipEventRecord(s->ev_ready[k], stream);
    if (e != hipSuccess) return hip_fail(e, "streamer event");
    s->staging_used[j] = true;
    s->slot_layer[k] = layer;
    s->layer_slot[layer] = k;
    s->decoded_on[k] = stream;
    s->decoded_ever[k] = 1;
    s->free_recorded[k] = 0;
    s->st.h2d_bytes += s->len[layer];
    return BS_OK;
}

// resident slot of `layer` (loading it on a miss), or an error
bs_status resident(bs_streamer* s, uint32_t layer, hipStream_t stream, uint32_t* slot) {
    if (!s || layer >= s->n_layers) { set_error("layer out of range"); return BS_E_INVAL; }
    int64_t k = s->layer_slot[layer];
    if (k >= 0) {
        s->st.hits++;
        if (s->decoded_on[k] != stream) {
            const hipError_t e = hipStreamWaitEvent(stream, s->ev_ready[k], 0);
            if (e != hipSuccess) return hip_fail(e, "streamer wait");
        }
    } else {
        s->st.misses++;
        k = victim(s);
        if (k < 0) { set_error("every slot holds an acquired layer"); return BS_E_NOSPACE; }
        const bs_status rc = load(s, layer, (uint32_t)k, stream);
        if (rc != BS_OK) return rc;
    }
    s->stamp[k] = ++s->clock;
    *slot = (uint32_t)k;
    return BS_OK;
}

}  // namespace

extern "C" {

bs_status bs_streamer_create(const void* const* h_containers, const uint64_t* lens, uint32_t n_layers,
                             uint64_t vram_budget, void* stream, bs_streamer** out) {
    if (!out || !h_containers || !lens || n_layers == 0) { set_error("NULL argument or no layers"); return BS_E_INVAL; }
    *out = nullptr;
    bs_streamer* s = new (std::nothrow) bs_streamer();
    if (!s) return BS_E_NOMEM;
    s->n_layers = n_layers;
    // validate every container and size the slots and staging buffers
    uint64_t arena = 0, max_len = 16, max_out = 16, status_words = 0;
    std::vector<uint64_t> out_bytes(n_layers);
    for (uint32_t i = 0; i < n_layers; i++) {
        bs_container_info ci;
        if (!h_containers[i]) { streamer_free(s); set_error("NULL container %u", i); return BS_E_INVAL; }
        const bs_status rc = bs_container_info_get(h_containers[i], lens[i], &ci);
        if (rc != BS_OK) { streamer_free(s); return rc; }
        s->len.push_back(lens[i]);
        s->status_off.push_back(status_words);
        status_words += std::max<uint64_t>(ci.n_streams, 1);
        out_bytes[i] = ci.out_len;
        arena += align_up(lens[i], 256);
        max_len = std::max(max_len, lens[i]);
        max_out = std::max(max_out, ci.out_len);
    }
    s->staging_bytes = align_up(max_len, 256);
    s->slot_bytes = align_up(max_out, 256);
    const uint64_t fixed = 2 * s->staging_bytes;
    if (vram_budget < fixed + 2 * s->slot_bytes) {
        set_error("budget %llu B holds fewer than two slots (needs %llu B: two staging buffers of %llu B and slots of %llu B)",
                  (unsigned long long)vram_budget, (unsigned long long)(fixed + 2 * s->slot_bytes),
                  (unsigned long long)s->staging_bytes, (unsigned long long)s->slot_bytes);
        streamer_free(s);
        return BS_E_INVAL;
    }
    s->n_slots = (uint32_t)std::min<uint64_t>((vram_budget - fixed) / s->slot_bytes, n_layers);
    hipError_t e = hipHostMalloc((void**)&s->h_arena, arena, hipHostMallocDefault);
    if (e != hipSuccess) { streamer_free(s); set_error("pinned host memory (%llu B)", (unsigned long long)arena); return BS_E_NOMEM; }
    uint64_t off = 0;
    for (uint32_t i = 0; i < n_layers; i++) {
        s->h_ptr.push_back(s->h_arena + off);
        memcpy(s->h_arena + off, h_containers[i], lens[i]);
        off += align_up(lens[i], 256);
    }
    for (int j = 0; j < 2 && e == hipSuccess; j++) e = hipMalloc(&s->d_staging[j], s->staging_bytes);
    if (e == hipSuccess) e = hipMalloc(&s->d_slots, (uint64_t)s->n_slots * s->slot_bytes);
    if (e == hipSuccess) e = hipMalloc(&s->d_status, 4 * status_words);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&s->copy_stream, hipStreamNonBlocking);
    for (int j = 0; j < 2 && e == hipSuccess; j++) {
        e = hipEventCreateWithFlags(&s->ev_copied[j], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&s->ev_staging_free[j], hipEventDisableTiming);
    }
    s->ev_ready.assign(s->n_slots, nullptr);
    s->ev_free.assign(s->n_slots, nullptr);
    for (uint32_t k = 0; k < s->n_slots && e == hipSuccess; k++) {
        e = hipEventCreateWithFlags(&s->ev_ready[k], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&s->ev_free[k], hipEventDisableTiming);
    }
    if (e != hipSuccess) {
        const bs_status rc = e == hipErrorOutOfMemory ? BS_E_NOMEM : hip_fail(e, "streamer setup");
        if (rc == BS_E_NOMEM) set_error("device memory for the streamer");
        streamer_free(s);
        return rc;
    }
    // one plan per layer: its tables are built from a device copy once
    hipStream_t hs = (hipStream_t)stream;
    for (uint32_t i = 0; i < n_layers; i++) {
        e = hipMemcpyAsync(s->d_staging[0], s->h_ptr[i], lens[i], hipMemcpyHostToDevice, hs);
        if (e != hipSuccess) { streamer_free(s); return hip_fail(e, "streamer plan upload"); }
        bs_plan* p = nullptr;
        const bs_status rc = bs_plan_create(s->h_ptr[i], lens[i], s->d_staging[0], stream, &p);   // synchronises
        if (rc != BS_OK) { streamer_free(s); return rc; }
        s->plans.push_back(p);
        s->n_records.push_back(plan_records(p));
        s->st.plan_bytes += plan_device_bytes(p);
    }
    s->free_recorded.assign(s->n_slots, 0);
    s->free_ever.assign(s->n_slots, 0);
    s->slot_layer.assign(s->n_slots, -1);
    s->pins.assign(s->n_slots, 0);
    s->stamp.assign(s->n_slots, 0);
    s->decoded_on.assign(s->n_slots, nullptr);
    s->decoded_ever.assign(s->n_slots, 0);
    s->layer_slot.assign(n_layers, -1);
    s->st.n_layers = n_layers;
    s->st.n_slots = s->n_slots;
    s->st.slot_bytes = s->slot_bytes;
    s->st.staging_bytes = s->staging_bytes;
    *out = s;
    return BS_OK;
}

void bs_streamer_destroy(bs_streamer* s) { streamer_free(s); }

bs_status bs_streamer_acquire(bs_streamer* s, uint32_t layer, void* stream, void** d_layer) {
    if (!d_layer) { set_error("NULL argument"); return BS_E_INVAL; }
    uint32_t k = 0;
    const bs_status rc = resident(s, layer, (hipStream_t)stream, &k);
    if (rc != BS_OK) return rc;
    s->pins[k]++;
    *d_layer = s->d_slots + (uint64_t)k * s->slot_bytes;
    return BS_OK;
}

bs_status bs_streamer_release(bs_streamer* s, uint32_t layer, void* stream) {
    if (!s || layer >= s->n_layers || s->layer_slot[layer] < 0 || !s->pins[s->layer_slot[layer]]) {
        set_error("layer is not acquired");
        return BS_E_INVAL;
    }
    const uint32_t k = (uint32_t)s->layer_slot[layer];
    hipStream_t hs = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    // keep earlier releases of the same residency ordered before this one
    if (s->free_recorded[k]) e = hipStreamWaitEvent(hs, s->ev_free[k], 0);
    if (e == hipSuccess) e = hipEventRecord(s->ev_free[k], hs);
    if (e != hipSuccess) return hip_fail(e, "streamer release");
    s->free_recorded[k] = 1;
    s->free_ever[k] = 1;
    s->pins[k]--;
    return BS_OK;
}

bs_status bs_streamer_prefetch(bs_streamer* s, uint32_t layer, void* stream) {
    uint32_t k = 0;
    return resident(s, layer, (hipStream_t)stream, &k);
}

bs_status bs_streamer_get_stats(const bs_streamer* s, bs_streamer_stats* stats) {
    if (!s || !stats) { set_error("NULL argument"); return BS_E_INVAL; }
    *stats = s->st;
    return BS_OK;
}

}  // extern "C"
