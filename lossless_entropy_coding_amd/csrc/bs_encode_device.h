// bs_encode_device.h -- structures shared by the host side of the library and
// the GPU encoder's kernels (gfx950).  Not part of the public C ABI.
#pragma once
#include <stdint.h>

#include "bs_device.h"

namespace bsd {

// GPU encoder.  Per BF16 record, the encode tables (in device memory): for
// each s, q | cum << 16 (q <= 2^12, cum < 2^12); for each fraction table t
// (0 = flat) and f, the same; the fraction table of each s.
struct EncTabDev {
    uint32_t s_qc[512];
    uint32_t f_qc[(kMaxTables + 1) * 128];
    uint8_t route[512];
    uint32_t h_qc[(kMaxHTablesDev + 1) * 8];   // layout 2: q | cum << 16 of each h table (0 = flat) and h
    uint32_t t_qc[512 * 8];                    // layout 3: q | cum << 16 of the joint symbol 8 s + h
};

// One BF16 record to encode: its chunks' streams (chunk c, stream st = unit
// c * S + st) are coded by one wavefront each into scratch.
struct EncArgs {
    const uint16_t* w;          // n weights, 16-B aligned
    uint64_t n;
    uint32_t W, K, S, P;        // P = K / S lanes per stream
    uint32_t n_chunks, m_s, m_f;   // layout 2: m_f is M_h
    uint32_t layout;
    const EncTabDev* tab;
    uint16_t* words;            // unit u's words (in emission order) at words + u * 2 * (W / S)
    uint32_t* states;           // chunk c lane l at states + c * K + l
    uint32_t* counts;           // unit u: counts[2u] words, counts[2u + 1] sum of its lanes' length codes
    // assembly
    uint8_t* out;               // the record's first byte in the container
    const uint64_t* chunk_off;  // payload offset of each chunk from the record start
    const uint32_t* unit_start; // 16-bit unit where each stream starts in its chunk's stream area
    const uint32_t* unit_mu;    // 16-bit units of each stream's state bits
};

}  // namespace bsd

// Launchers (bs_encode.hip).  All return a hipError_t as int.
extern "C" {
// GPU encoder: code every stream of a record into scratch (lanes per thread R
// = 1, 2, 4 or 8), then write the record's chunk payloads into the container
int bsk_encode(const bsd::EncArgs* args, uint32_t R, void* stream);
int bsk_assemble(const bsd::EncArgs* args, void* stream);
// fill n bytes at d with zero (a kernel, so that the work stays capturable)
int bsk_zero(void* d, uint64_t n, void* stream);
}
