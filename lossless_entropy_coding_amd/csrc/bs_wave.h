// bs_wave.h -- wavefront helpers shared by the library's HIP kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>

namespace bsd {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum of v over the wave (64 lanes), returned to every lane: quad, row and
// row-broadcast DPP steps leave the total in lane 63
__device__ __forceinline__ float wave_sum_dpp(float v) {
#define BS_DPP_ADD(ctrl, rows) \
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, rows, 0xF, false))
    BS_DPP_ADD(0xB1, 0xF);    // quad_perm [1,0,3,2]
    BS_DPP_ADD(0x4E, 0xF);    // quad_perm [2,3,0,1]
    BS_DPP_ADD(0x124, 0xF);   // row_ror:4
    BS_DPP_ADD(0x128, 0xF);   // row_ror:8: every lane holds its row's sum
    BS_DPP_ADD(0x142, 0xA);   // row_bcast:15 into rows 1 and 3
    BS_DPP_ADD(0x143, 0xC);   // row_bcast:31 into rows 2 and 3
#undef BS_DPP_ADD
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

}  // namespace bsd
