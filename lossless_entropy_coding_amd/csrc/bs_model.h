// bs_model.h -- per-tensor model (internal).
#pragma once
#include <stdint.h>

#include <array>
#include <vector>

#include "bs.h"
#include "bs_internal.h"

namespace bs {

struct Model {
    uint64_t n = 0;                              // weights the model was built from
    uint32_t m_s = 12, m_f = 10;
    uint32_t n_sym = 0;                          // occupied (sign, exponent) symbols
    uint32_t n_tables = 0;                       // coded fraction tables (ids 1..n_tables)
    std::array<uint64_t, 512> counts_s{};        // cs[s]
    std::array<uint32_t, 512> q_s{};             // sums to 2^m_s
    std::array<uint32_t, 512> route{};           // fraction table id of each occupied s (0 = flat)
    std::array<std::array<uint32_t, 128>, kMaxTables> q_f{};  // layout 1: table t at index t-1, sums to 2^m_f
    uint32_t layout = 1;                         // 2: m_f is M_h = 16 - m_s; 3: m_f is M_t = 13
    std::array<std::array<uint32_t, 8>, kMaxHTables> q_h{};   // layout 2: table t at index t-1, sums to 2^m_f
    std::array<uint32_t, 512 * 8> q_t{};         // layout 3: q of the joint symbol 8 s + h, sums to 2^13
};

bool params_ok(const bs_params* p);
// counters of the device histogram (hist kernel): 256 x 128 sign-merged
// (exponent, fraction) counts, then 256 x 8 negative counts per (exponent,
// high three fraction bits)
constexpr size_t kHistCounters = 256 * 128 + 256 * 8;
bs_status model_from_counts(Model& md, const bs_params* p, uint64_t n, const unsigned long long* cnt,
                            std::array<uint64_t, 128>* merged, uint64_t* ct);
bool quantise(const uint64_t* counts, uint32_t A, uint32_t M, uint32_t* q);
const char* last_error();

}  // namespace bs

// the public opaque type of bs.h
struct bs_tables : bs::Model {};
