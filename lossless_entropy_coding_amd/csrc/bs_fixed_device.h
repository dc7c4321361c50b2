// bs_fixed_device.h -- structures shared by the host side of the library and
// the kernels of the fixed-width lane-stream form (gfx950).  Not part of the
// public C ABI.
#pragma once
#include <stdint.h>

namespace bsd {

// fixed-width lane-stream form (layout in bs.h): one wavefront decodes a
// block of 2048 weights (64 lanes x 32) at a time
constexpr uint32_t kFixHeader = 96;
constexpr uint32_t kFixBlockW = 2048;
constexpr uint32_t kFixBlockBytes = 2816;
constexpr uint32_t kFixWaves = 4;           // waves per workgroup
constexpr uint32_t kFixEscLds = 256;        // escape staging per wave in LDS (up to 254 escapes; more are read from HBM)

struct FixedArgs {
    const uint8_t* blob;    // the whole blob (header at 0)
    uint16_t* out;          // n BF16 words (decode)
    uint32_t* status;       // n_blocks words or null
    uint64_t n, n_blocks, n_esc, esc_off;
    uint32_t tab[8];        // symbols of codes 0..15, two per word (code 2k low); code 15 = 0
    // fused product with a vector: the weights are a row-major rows x cols
    // matrix (cols a multiple of 32), y[r] = sum over c of W[r, c] x[c] in
    // fp32.  A unit of unit_rows = 2048 / gcd(cols, 2048) rows spans exactly
    // unit_blocks = cols / gcd(cols, 2048) whole blocks; a workgroup owns a
    // group of group_units units (at most 64 rows) and stores its rows.
    const uint16_t* gx;     // x: cols BF16 words, 16-B aligned
    float* gy;              // y: rows floats
    uint64_t rows;
    uint64_t n_groups;      // ceil(rows / (unit_rows * group_units))
    uint32_t cols;          // below 2^26
    uint32_t unit_rows;
    uint32_t unit_blocks;
    uint32_t group_units;
    uint32_t q_step, r_step;  // kFixWaves * 2048 = q_step * cols + r_step
    // fused product with a batch of vectors (MFMA): X batch x cols in gx
    // (row-major BF16), Y batch x rows in gy (row-major fp32), cols a
    // multiple of 2048 so that every row starts on a block
    uint32_t batch;
    uint32_t ksplit;        // 1, or 2: two workgroups share a group of rows, one half of its panels each
    // the split product's workspace: the second half's partial sums
    // (batch x rows fp32, laid out as Y)
    float* gpart;
};

// several tensors decoded in one launch: tensor i takes workgroups
// wg_start[i] .. wg_start[i + 1] - 1 (every tensor at least one)
constexpr uint32_t kFixManyMax = 16;
struct FixedMany {
    FixedArgs a[kFixManyMax];
    uint32_t wg_start[kFixManyMax + 1];
    uint32_t count;
};

#ifndef BS_GEMM_WAVES
#define BS_GEMM_WAVES 16
#endif
constexpr uint32_t kGemmWaves = BS_GEMM_WAVES;   // waves per workgroup of the batched product (8 or 16; one block of a panel each at 16)
constexpr uint32_t kGemmRowBytes = 4112;    // LDS per decoded row block: 4096 B + 16 B, so the 16 rows start on different banks

}  // namespace bsd

// Launchers (bs_fixed.hip).  All return a hipError_t as int.
extern "C" {
// decode a fixed-width blob: n_groups workgroups of kFixWaves waves, each wave
// striding over the blocks
int bsk_fixed_decode(const bsd::FixedArgs* args, uint32_t n_groups, void* stream);
// decode up to kFixManyMax blobs in one launch of wg_start[count] workgroups
int bsk_fixed_decode_many(const bsd::FixedMany* m, void* stream);
// the fused product of a fixed-width blob with a batch of vectors: one
// workgroup of kGemmWaves waves per 16 rows (rows32 0), or per 32 rows and
// args->ksplit shares of the panels (rows32 1; with 2 shares a second launch
// adds the workspace's sums into Y); n_groups workgroups, striding
int bsk_fixed_gemm(const bsd::FixedArgs* args, uint32_t n_groups, int rows32, void* stream);
// the fused product of a fixed-width blob with a vector: n_groups workgroups
// of kFixWaves waves, each workgroup striding over the row groups
int bsk_fixed_gemv(const bsd::FixedArgs* args, uint32_t n_groups, void* stream);
}

// Launchers (bs_fixed_encode.hip): the fixed-width form built on the GPU.
extern "C" {
// 512 (sign, exponent) symbol counts added into counts (zeroed by the caller)
int bsk_fixed_sym_count(const uint16_t* w, uint64_t n, unsigned long long* counts, void* stream);
// escapes of each block, given the code of every symbol (15 = escape)
int bsk_fixed_block_esc(const uint16_t* w, uint64_t n, const uint8_t* code_of, uint64_t n_blocks, uint32_t* esc,
                        void* stream);
// the code and fraction planes of every block, and the escapes from each block's first
int bsk_fixed_pack(const uint16_t* w, uint64_t n, const uint8_t* code_of, uint64_t n_blocks, const uint32_t* first,
                   uint8_t* blob, uint64_t esc_off, void* stream);
}
