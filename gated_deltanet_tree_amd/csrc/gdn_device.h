// Device-side helpers shared by the HIP translation units (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"

namespace gdn {

typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) {
    return __uint_as_float(uint32_t(x) << 16);
}
// Inverse of to_f32 for a value that came from T (exact: a widened bf16 has zero low bits).
template <typename T> __device__ __forceinline__ T from_exact_f32(float x);
template <> __device__ __forceinline__ float from_exact_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_exact_f32<bf16_t>(float x) {
    return bf16_t(__float_as_uint(x) >> 16);
}

// Sum over the 8 consecutive lanes of an aligned lane octet; every lane of the octet gets
// the total. Two quad permutations (xor 1, xor 2) then the half-row mirror (lane i <-> 7-i),
// which pairs each quad with the other quad of the octet. All three are DPP moves.
__device__ __forceinline__ float octet_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
    return x;
}

// Workgroups are dealt round-robin to the 8 XCDs. Give XCD x a contiguous range of logical
// work items so neighbours in logical order (sibling chains reading one boundary state,
// consecutive channels) share an L2.  Bijective on [0, n).
__device__ __forceinline__ uint32_t xcd_logical(uint32_t b, uint32_t n) {
    const uint32_t q = n >> 3, r = n & 7, x = b & 7, k = b >> 3;
    return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

}  // namespace gdn

#define GDN_LAUNCH_CHECK(what)                                                              \
    do {                                                                                    \
        hipError_t e_ = hipGetLastError();                                                  \
        if (e_ != hipSuccess)                                                               \
            return ::gdn::fail(GDN_EDEVICE, "%s: %s", what, hipGetErrorString(e_));         \
    } while (0)
