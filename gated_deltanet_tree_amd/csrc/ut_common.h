// Helpers shared by the tree-masked UT verify kernels (gfx950).
#pragma once

#include "verify_common.h"

namespace gdn {

constexpr size_t kUtMaxLdsBytes = 160 * 1024;  // one workgroup may take the whole CU's LDS

typedef __attribute__((address_space(3))) void lds_void;

__host__ __device__ constexpr size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

// One 64-lane direct load from per-lane source addresses into LDS at lds_base, which must be
// the same for the whole wave.  16-byte loads land at lds_base + 16 l; 4-byte and 2-byte loads
// land at lds_base + 4 l, a 2-byte value zero-extended to a dword.
template <int BYTES> __device__ __forceinline__ void to_lds(const void *src, void *lds_base);
template <> __device__ __forceinline__ void to_lds<16>(const void *src, void *lds_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_void *)lds_base, 16, 0, 0);
}
template <> __device__ __forceinline__ void to_lds<4>(const void *src, void *lds_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_void *)lds_base, 4, 0, 0);
}
template <> __device__ __forceinline__ void to_lds<2>(const void *src, void *lds_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_void *)lds_base, 2, 0, 0);
}

// beta or gate as fp32 from its dword slot (bf16 arrives zero-extended in the low half)
template <typename TIn> __device__ __forceinline__ float slot_f32(uint32_t x) {
    return sizeof(TIn) == 2 ? __uint_as_float(x << 16) : __uint_as_float(x);
}

struct UtUnit {  // (layer, sequence, head) of a workgroup, from its XCD-aware logical id
    int layer_rel, seq, h;
};
__device__ __forceinline__ UtUnit ut_unit(const VerifyParams &P) {
    // Grids are capped at kMaxBlocks workgroups, so block arithmetic stays in 32 bits.
    const uint32_t logical = xcd_logical(blockIdx.x, uint32_t(P.n_blocks));
    const uint32_t per = uint32_t(P.S) * uint32_t(P.H);
    UtUnit u;
    u.layer_rel = int(logical / per);
    u.seq = int((logical % per) / uint32_t(P.H));
    u.h = int(logical % uint32_t(P.H));
    return u;
}

// The matrix-core UT kernel (bf16 inputs, d = 128).
gdn_status launch_ut_mfma(const VerifyParams &P, int n_max, int nrec_max, int nlv_max,
                          int nf_max, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

}  // namespace gdn
