// Helpers shared by the tree-masked UT verify kernels (gfx950).
#pragma once

#include "mfma_common.h"
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

// (layer, sequence, head) of a workgroup, in dispatch order (sequence-major, heads fastest):
// consecutive workgroups go to the 8 XCDs in turn, so each XCD takes every eighth head of every
// sequence.  These workgroups share no input but the small per-sequence plan, and this order
// measured faster than giving each XCD a contiguous range of (sequence, head) items: 89.5
// against 91.6 us per fused launch on 32 sequences x 48 heads, 94.9 against 95.7 us on the
// 64-node trees, about 0.5% on the UT verify.
struct UtUnit {
    int layer_rel, seq, h;
};
__device__ __forceinline__ UtUnit ut_unit(const VerifyParams &P) {
    // Grids are capped at kMaxBlocks workgroups, so block arithmetic stays in 32 bits.
    const uint32_t logical = blockIdx.x;
    const uint32_t per = uint32_t(P.S) * uint32_t(P.H);
    UtUnit u;
    u.layer_rel = int(logical / per);
    u.seq = int((logical % per) / uint32_t(P.H));
    u.h = int(logical % uint32_t(P.H));
    return u;
}

// Row m of the dense Y and Z (ys floats each, 16-byte aligned): zeros, then 1 and q_m.k_m on the
// diagonal; the ancestor entries are written after.
__device__ __forceinline__ void dense_row_init(float *yr, float *zr, int ys, int m, float kq) {
    for (int k = 0; k < ys; k += 4) {
        *reinterpret_cast<float4 *>(yr + k) = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4 *>(zr + k) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    yr[m] = 1.f;
    zr[m] = kq;
}

// Rows n of Y = T^-1 and Z = C' T^-1 from n's own root path: Y T = I and Z T = C' restricted to
// the ancestor relation give, for the ancestor a_t at distance t + 1 (record q1 + t),
//   y_t = -(T[n][a_t] + sum_{s<t} y_s T[a_s][a_t])
//   z_t = C'[n][a_t] - ((q_n.k_n) T[n][a_t] + sum_{s<t} z_s T[a_s][a_t])
// where T[a_s][a_t] is record rp_s + t - s of a_s's block (rp_s = its start).  Every read is
// independent of the results, so a lane needs two rounds of loads and then only FMAs; y_t and z_t
// go to column a_t of the node's dense rows yr, zr.  YD bounds the tree's depth; terms past the
// node's depth d are computed and dropped.  Their inner reads (records bs_s + t with
// bs_s = rp_s - s, a compile-time offset from one base per s) may run up to YD - 2 records past
// the node's block: into the next node's records or the table after recC, never past the tables,
// and only into dropped terms.
template <int YD>
__device__ __forceinline__ void yz_rows(int q1, int d, float kq, const float *recC,
                                        const float *recQ, const int *recP, const int *recM,
                                        float *yr, float *zr) {
    int tb[YD];  // rp_s - s, a record index: 32 bits per term rather than a pointer
#pragma unroll
    for (int s = 0; s < YD; ++s) tb[s] = recP[q1 + min(s, d - 1)] - s;
    float y[YD], z[YD];
#pragma unroll
    for (int t = 0; t < YD; ++t) {
        const int tc = min(t, d - 1);
        const float tn = recC[q1 + tc];
        float ya = tn, za = kq * tn;
#pragma unroll
        for (int s = 0; s < t; ++s) {
            const float ts = recC[tb[s] + t];
            ya = fmaf(y[s], ts, ya);
            za = fmaf(z[s], ts, za);
        }
        y[t] = -ya;
        z[t] = recQ[q1 + tc] - za;
        if (t < d) {
            const int am = recM[q1 + t];  // a_t, the dense column
            yr[am] = y[t];
            zr[am] = z[t];
        }
    }
}

// Y = T^-1 and Z = C' Y of the tree (record (n, t) = ancestor a_t of n at distance t + 1, at
// q1 + t with q1 = poff[n] + 1; recP = block start of the record's node, recT = t, -1 on a node's
// own record), all on wave 0, as dense rows for the matrix-core u/o pass: Yd[m][k] = Y[m][k] on
// m's ancestors, 1 on the diagonal and 0 elsewhere; Zd likewise with q_m.k_m on the diagonal.
// Rows are ys = round4(n) floats; rows past n are left as they are (their products are never
// stored).  Trees up to depth MAXD: one lane per node (yz_rows).  Deeper trees: level by level on
// the records (recY, recZ) with
//   Y[n][a_t] = -T[n][a_t] - sum_{s<t} T[n][a_s] Y[a_s][a_t]
//   Z[n][a_t] = (q_n.k_n) Y[n][a_t] + C'[n][a_t] + sum_{s<t} C'[n][a_s] Y[a_s][a_t]
// (level lv's blocks of lv + 1 records are contiguous from record r_lv; every term read belongs
// to a shallower level), then spread into the dense rows.  Needs a barrier before the results are
// read by other waves.
template <int MAXD = 16>
__device__ __forceinline__ void tree_inverse(int n, int dmax, int lane, int w, const int *poff,
                                             const int *dep, const int *lvn, const int *recM,
                                             const int *recP, const int *recT,
                                             const float *recC, const float *recQ,
                                             const float *kqd, float *recY, float *recZ,
                                             float *Yd, float *Zd, int ys) {
    static_assert(MAXD == 12 || MAXD == 16, "register form up to depth 12 or 16");
    if (w != 0) return;
    if (dmax <= MAXD) {
        for (int nd = lane; nd < n; nd += 64) {
            const int q1 = poff[nd] + 1, d = dep[nd];
            const float kq = kqd[nd];
            float *yr = Yd + nd * ys, *zr = Zd + nd * ys;
            dense_row_init(yr, zr, ys, nd, kq);
            if (d == 0) continue;
            if (dmax <= 4)
                yz_rows<4>(q1, d, kq, recC, recQ, recP, recM, yr, zr);
            else if (dmax <= 8)
                yz_rows<8>(q1, d, kq, recC, recQ, recP, recM, yr, zr);
            else if (MAXD == 12 || dmax <= 12)
                yz_rows<12>(q1, d, kq, recC, recQ, recP, recM, yr, zr);
            else
                yz_rows<MAXD>(q1, d, kq, recC, recQ, recP, recM, yr, zr);
        }
        return;
    }
    int r_lv = lvn[1] - lvn[0];  // level 0: one record per root
    for (int lv = 1; lv <= dmax; ++lv) {
        const int nrec_lv = (lvn[lv + 1] - lvn[lv]) * (lv + 1);
        for (int it = lane; it < nrec_lv; it += 64) {
            const int q = r_lv + it, t = recT[q];
            if (t < 0) continue;
            const int q1 = q - t;
            float ya = recC[q], za = recQ[q];
            for (int s0 = 0; s0 < t; s0 += 4) {  // four terms with independent reads
                int sp[4];
                float cc[4], cq[4], yv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s2 = min(s0 + j, t - 1);
                    sp[j] = recP[q1 + s2] + (t - s2);
                    cc[j] = recC[q1 + s2];
                    cq[j] = recQ[q1 + s2];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) yv[j] = recY[sp[j]];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (s0 + j >= t) break;
                    ya = fmaf(cc[j], yv[j], ya);
                    za = fmaf(cq[j], yv[j], za);
                }
            }
            recY[q] = -ya;
            recZ[q] = fmaf(kqd[recM[q1 - 1]], -ya, za);
        }
        r_lv += nrec_lv;
        wave_order();
    }
    for (int m = lane; m < n; m += 64) {
        float *yr = Yd + m * ys, *zr = Zd + m * ys;
        dense_row_init(yr, zr, ys, m, kqd[m]);
        const int q1 = poff[m] + 1, d = dep[m];
        for (int t = 0; t < d; ++t) {
            yr[recM[q1 + t]] = recY[q1 + t];
            zr[recM[q1 + t]] = recZ[q1 + t];
        }
    }
}

// u and o of every (node, state row) on the fp32 matrix cores: U = Yd W and O = GR + Zd W over
// the wave's state rows 16 NT w .. 16 NT w + 16 NT - 1 (NT N tiles of 16 rows), which makes
//   u_n = w_n + sum_{t < d_n} Y[n][a_t] w_{a_t},  o_n = G_n r_n + (q_n.k_n) w_n + sum_t Z[n][a_t] w_{a_t}.
// M tiles of 16 nodes, N tiles of 16 state rows, K steps of 4 nodes; ancestors precede their
// descendants, so node tile mt needs the K steps below node 16mt + 16 only.  W row k (stride ws
// floats) past the tree is read clamped to row n - 1, where Yd and Zd hold 0.  u goes to bank row
// n (stride 128), o to out0 + n * out_stride.  Needs Yd, Zd, W and GR complete (a barrier after
// tree_inverse and the epilogue).
template <int NT>
__device__ __forceinline__ void tree_apply_rows(int n, int ys, int w, int lane, const float *Yd,
                                                const float *Zd, const float *Wm,
                                                const float *GR, int ws, float *bank_u0,
                                                float *out0, int64_t out_stride) {
    const int lr = lane & 15, lg = lane >> 4;
    const int MT = (n + 15) >> 4, KT = (n + 3) >> 2;
    const int row0 = 16 * NT * w;
    for (int mt = 0; mt < MT; ++mt) {
        const int ksn = min(4 * mt + 4, KT);
        const float *ya = Yd + (16 * mt + lr) * ys + lg, *za = Zd + (16 * mt + lr) * ys + lg;
        floatx4 au[NT], ao[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int i = row0 + 16 * nt + lr;
            au[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r) ao[nt][r] = GR[min(16 * mt + 4 * lg + r, n - 1) * ws + i];
        }
        for (int ks = 0; ks < ksn; ++ks) {
            const float yv = ya[4 * ks], zv = za[4 * ks];
            const float *wr = Wm + min(4 * ks + lg, n - 1) * ws + row0 + lr;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float b = wr[16 * nt];
                au[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(yv, b, au[nt], 0, 0, 0);
                ao[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(zv, b, ao[nt], 0, 0, 0);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int nd = 16 * mt + 4 * lg + r;
            if (nd >= n) break;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int i = row0 + 16 * nt + lr;
                bank_u0[int64_t(nd) * 128 + i] = au[nt][r];
                out0[int64_t(nd) * out_stride + i] = ao[nt][r];
            }
        }
    }
}

// Four waves of 32 state rows (wave w owns rows 32w .. 32w + 31).
__device__ __forceinline__ void tree_apply_mfma(int n, int ys, int w, int lane, const float *Yd,
                                                const float *Zd, const float *Wm,
                                                const float *GR, int ws, float *bank_u0,
                                                float *out0, int64_t out_stride) {
    tree_apply_rows<2>(n, ys, w, lane, Yd, Zd, Wm, GR, ws, bank_u0, out0, out_stride);
}

// The matrix-core UT kernel (bf16 inputs, d = 128).
gdn_status launch_ut_mfma(const VerifyParams &P, int n_max, int nrec_max, int nlv_max,
                          int nf_max, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

}  // namespace gdn
