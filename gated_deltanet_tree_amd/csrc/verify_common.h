// Device pieces shared by the verify kernels (chain-resident and tree-masked UT): kernel
// parameters, the lane layout of a d x d fp32 tile over the workgroup, and the LDS staging of
// pending fold rows and node inputs.
#pragma once

#include "gdn_device.h"

namespace gdn {

struct VerifyParams {
    const void *q, *k, *v, *beta, *gate;
    float *state;
    float *bank_k[2], *bank_u[2], *bank_lg[2];
    const int32_t *role, *pending;
    const int32_t *rows;  // [S][max_nodes]: bank row of each pending factor, in path order
    float *boundary;
    float *out;
    const int32_t *img;
    int64_t off_seq, off_chain, off_cnodes, off_cseq, off_csrc, off_store, off_parent, off_depth;
    // tree-masked verify plan in the image (see gdn_tree.h)
    int64_t off_ut_rec_base, off_ut_node_rec, off_ut_lv_base, off_ut_lvn, off_ut_lvnode,
        off_ut_rec_anc;
    int32_t S, H, T, max_nodes, n_boundaries, layer_begin;
    int32_t chain_begin, n_chains;  // chains of this wave
    int64_t n_blocks;
    int32_t fold_only;  // flush: one workgroup per (layer, seq, head), fold + store only
};

// Host: validates the verify arguments against the schedule image and fills the kernel
// parameters shared by every verify entry point (q, k, v may be absent when !need_qkv).
gdn_status verify_setup(const gdn_verify_args *a, const int32_t *host_image,
                        const int32_t *dev_image, VerifyParams &P, ImageView &v,
                        bool need_boundary, bool need_qkv = true);

template <int D> struct Tile {
    static constexpr int RW = D >= 32 ? 32 : D;       // rows per wave
    static constexpr int NW = D / RW;                 // waves per workgroup
    static constexpr int THREADS = 64 * NW;
    static constexpr int M = RW / 8;                  // rows per lane
    static constexpr int COLS = D / 8;                // columns per lane
    static constexpr int VEC = COLS >= 4 ? 4 : COLS;  // contiguous columns per access
    static constexpr int NP = COLS / VEC;             // column groups per lane
    static_assert(D % 16 == 0 && RW % 8 == 0, "unsupported head dim");
};

template <int VEC> struct VecT;
template <> struct VecT<4> {
    typedef float4 type;
    static __device__ __forceinline__ void get(const float *p, float *o) {
        float4 t = *reinterpret_cast<const float4 *>(p);
        o[0] = t.x; o[1] = t.y; o[2] = t.z; o[3] = t.w;
    }
    static __device__ __forceinline__ void put(float *p, const float *o) {
        *reinterpret_cast<float4 *>(p) = make_float4(o[0], o[1], o[2], o[3]);
    }
};
template <> struct VecT<2> {
    typedef float2 type;
    static __device__ __forceinline__ void get(const float *p, float *o) {
        float2 t = *reinterpret_cast<const float2 *>(p);
        o[0] = t.x; o[1] = t.y;
    }
    static __device__ __forceinline__ void put(float *p, const float *o) {
        *reinterpret_cast<float2 *>(p) = make_float2(o[0], o[1]);
    }
};

#ifndef GDN_VERIFY_MIN_WAVES
#define GDN_VERIFY_MIN_WAVES 3  // waves per SIMD the register budget must allow
#endif
#ifndef GDN_REVERSE_LIGHT_WAVES
#define GDN_REVERSE_LIGHT_WAVES 1
#endif
#ifndef GDN_STAGE_ITEMS
#define GDN_STAGE_ITEMS 8  // items (fold rows or nodes) staged per LDS block
#endif

// Staging of a block of items into LDS.  An item is a pending fold row (fp32 k, u, lg) or a
// node (k, q, v, beta, g in the input dtype).  Its LDS slot holds fp32 [k | q | v-or-u |
// scalar0 | scalar1 | pad]: scalar0 = beta or lg, scalar1 = g.
//   - The block's node ids (for a fold row: its bank row, from the pending row map) are
//     uniform: they are read with scalar loads and stay in SGPRs.
//   - Every thread owns NCH 16-byte vector chunks of the block's vectors; the first 2 PB
//     threads also fetch one per-item scalar each.
// Loads keep their raw bits until stage_commit, so issuing them never waits on memory; the
// loads for block b+1 are issued right after block b is published, so their latency hides
// behind a whole block of work.
template <int D, typename TIn, int PB_ = GDN_STAGE_ITEMS> struct Stager {
    static constexpr int THREADS = Tile<D>::THREADS;
    static constexpr int PB = PB_;
    static constexpr int NODE_CV = D * int(sizeof(TIn)) / 16;  // 16-byte chunks per node vector
    static constexpr int FOLD_CV = D * 4 / 16;                 // 16-byte chunks per fold vector
    static constexpr int VCH = (3 * NODE_CV > 2 * FOLD_CV) ? 3 * NODE_CV : 2 * FOLD_CV;
    static constexpr int NCH = (PB * VCH + THREADS - 1) / THREADS;
    static constexpr int SLOT = 3 * D + 4;
    uint4 v[NCH];     // per thread: raw vector chunks
    uint32_t sc;      // per thread: raw bits of one per-item scalar (thread < 2 PB)
    int node[PB];     // uniform: global node id of each node item, bank row of each fold row
};

// Per-workgroup context of the staging helpers.  Passed by value and unpacked into scalars
// before any pointer is selected, so that no private (scratch) copy is ever needed.
struct ChainCtx {
    int L, n_items, nbeg, h, layer, T, H, max_nodes;
    int64_t bank_row0, off_cnodes;
    const int32_t *prow;  // the sequence's pending row map
    const float *pk, *pu, *plg;
    const void *k, *q, *v, *beta, *gate;
    const int32_t *img;
};

__device__ __forceinline__ const void *pick3(int i, const void *a, const void *b, const void *c) {
    const uintptr_t ua = reinterpret_cast<uintptr_t>(a), ub = reinterpret_cast<uintptr_t>(b),
                    uc = reinterpret_cast<uintptr_t>(c);
    return reinterpret_cast<const void *>(i == 0 ? ua : (i == 1 ? ub : uc));
}

template <int D, typename TIn, int PB>
__device__ __forceinline__ void stage_issue(Stager<D, TIn, PB> &st, const ChainCtx c, int it0,
                                            int tid) {
    using SG = Stager<D, TIn, PB>;
    const int it1 = min(c.n_items, it0 + SG::PB);
#pragma unroll
    for (int jj = 0; jj < SG::PB; ++jj) {  // uniform: node ids / bank rows of the block
        const int item = it0 + jj;
        int id = 0;
        if (item < c.L)  // the map comes from the commit call; the clamp keeps a bad entry in the bank
            id = min(max(c.prow[item], 0), c.max_nodes - 1);
        else if (item < it1)
            id = c.img[c.off_cnodes + c.nbeg + (item - c.L)];
        st.node[jj] = id;
    }
    // Thread t < 2 PB fetches scalar t / PB (0: beta or lg, 1: g) of item it0 + t % PB; the
    // raw bits are converted only in stage_commit, so nothing here waits for memory.
    st.sc = 0;
    if (tid < 2 * SG::PB) {
        const int rel = tid % SG::PB, which = tid / SG::PB, item = it0 + rel;
        if (item < it1) {
            int node = st.node[0];
#pragma unroll
            for (int jj = 1; jj < SG::PB; ++jj)
                if (rel == jj) node = st.node[jj];
            if (item < c.L) {
                if (which == 0) st.sc = __float_as_uint(c.plg[c.bank_row0 + node]);
            } else {
                const int64_t row = (int64_t(c.layer) * c.T + node) * c.H + c.h;
                const TIn *src = static_cast<const TIn *>(which == 0 ? c.beta : c.gate) + row;
                if (sizeof(TIn) == 2)
                    st.sc = *reinterpret_cast<const uint16_t *>(src);
                else
                    st.sc = *reinterpret_cast<const uint32_t *>(src);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < SG::NCH; ++i) {
        const int j = tid + i * SG::THREADS;
        const int rel = j / SG::VCH, item = it0 + rel, ch = j % SG::VCH;
        st.v[i] = make_uint4(0, 0, 0, 0);
        if (j >= SG::PB * SG::VCH || item >= it1) continue;
        int node = st.node[0];
#pragma unroll
        for (int jj = 1; jj < SG::PB; ++jj)
            if (rel == jj) node = st.node[jj];
        if (item < c.L) {
            if (ch < 2 * SG::FOLD_CV) {
                const float *src = static_cast<const float *>(pick3(ch < SG::FOLD_CV ? 0 : 1, c.pk, c.pu, c.pu)) +
                                   (c.bank_row0 + node) * D;
                st.v[i] = reinterpret_cast<const uint4 *>(src)[ch % SG::FOLD_CV];
            }
        } else if (ch < 3 * SG::NODE_CV) {
            const int vec = ch / SG::NODE_CV;
            const void *base = pick3(vec, c.k, c.q, c.v);
            const int64_t row = (int64_t(c.layer) * c.T + node) * c.H + c.h;
            st.v[i] = reinterpret_cast<const uint4 *>(static_cast<const TIn *>(base) + row * D)
                [ch % SG::NODE_CV];
        }
    }
}

template <int D, typename TIn, int PB>
__device__ __forceinline__ void stage_commit(const Stager<D, TIn, PB> &st, float *buf,
                                             const ChainCtx c, int it0, int tid) {
    using SG = Stager<D, TIn, PB>;
    const int it1 = min(c.n_items, it0 + SG::PB);
#pragma unroll
    for (int i = 0; i < SG::NCH; ++i) {
        const int j = tid + i * SG::THREADS;
        const int item = it0 + j / SG::VCH, ch = j % SG::VCH;
        if (j >= SG::PB * SG::VCH || item >= it1) continue;
        float *slot = buf + (item - it0) * SG::SLOT;
        const uint4 x = st.v[i];
        if (item < c.L) {
            if (ch < 2 * SG::FOLD_CV) {
                float *dst = slot + (ch < SG::FOLD_CV ? 0 : 2 * D) + (ch % SG::FOLD_CV) * 4;
                *reinterpret_cast<float4 *>(dst) = make_float4(
                    __uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                    __uint_as_float(x.w));
            }
        } else if (ch < 3 * SG::NODE_CV) {
            const int vec = ch / SG::NODE_CV, idx = ch % SG::NODE_CV;
            if (sizeof(TIn) == 2) {
                float *dst = slot + vec * D + idx * 8;
                *reinterpret_cast<float4 *>(dst) =
                    make_float4(bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y));
                *reinterpret_cast<float4 *>(dst + 4) =
                    make_float4(bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w));
            } else {
                *reinterpret_cast<float4 *>(slot + vec * D + idx * 4) = make_float4(
                    __uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                    __uint_as_float(x.w));
            }
        }
    }
    if (tid < 2 * SG::PB) {
        const int rel = tid % SG::PB, which = tid / SG::PB, item = it0 + rel;
        if (item < it1) {
            const bool raw16 = sizeof(TIn) == 2 && item >= c.L;
            buf[rel * SG::SLOT + 3 * D + which] = __uint_as_float(raw16 ? st.sc << 16 : st.sc);
        }
    }
}

}  // namespace gdn
