// Matrix-core helpers shared by the kernels that run bf16 MFMAs on fp32 data (gfx950, wave64):
// exact three-term bf16 splits of fp32 operands, operand fetches from LDS rows, wave-wide
// reductions and in-wave LDS ordering.
#pragma once

#include "gdn_device.h"

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Exact split of 8 fp32 values into three bf16 vectors (hi + mid + lo == x for normal x): each
// term takes the next 8 significant bits by truncation, so every remainder is exact.  Terms
// shrink by 2^-7 and 2^-15 relative to x.
__device__ __forceinline__ void split3(const float *x, bf16x8 &hi, bf16x8 &mid, bf16x8 &lo) {
    u32x4 h, m, l;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t b0 = __float_as_uint(x[2 * p]), b1 = __float_as_uint(x[2 * p + 1]);
        const float r0 = x[2 * p] - __uint_as_float(b0 & 0xFFFF0000u);
        const float r1 = x[2 * p + 1] - __uint_as_float(b1 & 0xFFFF0000u);
        const uint32_t c0 = __float_as_uint(r0), c1 = __float_as_uint(r1);
        const float t0 = r0 - __uint_as_float(c0 & 0xFFFF0000u);
        const float t1 = r1 - __uint_as_float(c1 & 0xFFFF0000u);
        h[p] = (b0 >> 16) | (b1 & 0xFFFF0000u);
        m[p] = (c0 >> 16) | (c1 & 0xFFFF0000u);
        l[p] = (__float_as_uint(t0) >> 16) | (__float_as_uint(t1) & 0xFFFF0000u);
    }
    hi = __builtin_bit_cast(bf16x8, h);
    mid = __builtin_bit_cast(bf16x8, m);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Operand of one 32-wide k-step from a bf16 row in LDS: elements c0 .. c0+3 and c0+16 .. c0+19.
__device__ __forceinline__ bf16x8 row_operand(const char *row, int c0) {
    const uint2 a = *reinterpret_cast<const uint2 *>(row + c0 * 2);
    const uint2 b = *reinterpret_cast<const uint2 *>(row + (c0 + 16) * 2);
    const u32x4 v = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float bf16_at(const char *row, int i) {
    return __uint_as_float(uint32_t(*reinterpret_cast<const uint16_t *>(row + i * 2)) << 16);
}

// Sum over the 64 lanes with DPP only: octets, the row of 16, then row broadcasts 15 and 31
// (rows 1 and 3 add the row below, rows 2 and 3 add lanes 0-31); lane 63 holds the total, which
// every lane receives.
__device__ __forceinline__ float wave_total(float x) {
    x = octet_sum(x);
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xA, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xC, 0xF, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// LDS accesses of one wave stay in program order across its lanes.
__device__ __forceinline__ void wave_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace gdn
