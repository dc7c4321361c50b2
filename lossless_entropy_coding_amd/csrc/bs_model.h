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
    std::array<std::array<uint32_t, 128>, kMaxTables> q_f{};  // table t at index t-1, sums to 2^m_f
};

bool params_ok(const bs_params* p);
bool quantise(const uint64_t* counts, uint32_t A, uint32_t M, uint32_t* q);
const char* last_error();

}  // namespace bs
