// Tree-masked UT verify on the matrix cores, for bf16 inputs and d = 128 (gfx950).
//
// Same method as the vector UT kernel ("Lucebox SpecLA and Gated DeltaNet state-resident
// verification" guide, mechanism 1, topology-mask form): with S0 the committed state after
// the deferred fold (mechanism 4), p_n = S0 k_n, r_n = S0 q_n and
//   w_n = beta_n (v_n - G_n p_n),
//   T[n][a] = beta_n E(n,a) (k_n . k_a)   for a a strict ancestor of n, T[n][n] = 1,
// the residual vectors solve T U = W, and the outputs are o_n = G_n r_n + sum_{a in A(n)}
// C[n][a] u_a with C[n][n] = q_n . k_n and C[n][a] = E(n,a) (q_n . k_a).  Both Y = T^-1 and
// Z = C Y are supported on ancestor-or-self pairs only (a product of two matrices that are
// zero off the ancestor relation stays zero off it), so
//   u_n = sum_{m in A(n)} Y[n][m] w_m,   o_n = G_n r_n + sum_{m in A(n)} Z[n][m] w_m,
// one independent short sum per (node, row), with no recurrence over the rows.
//
// Two launches per call:
//   prep  one wave per (layer, sequence, head).  Everything that does not involve the state:
//         the tree tables, the pair coefficients T and C ([k; q] K^T on the matrix cores), Y
//         level by level and Z, written as one record {m, Y[n][m], Z[n][m]} per
//         ancestor-or-self pair plus one {records offset, depth, G_n, beta_n} per node; also
//         the banked keys and log-gates.  Its chains of dependent LDS accesses run at high
//         occupancy (small LDS, one wave), where other waves hide their latency.
//   main  one workgroup of 4 waves per (layer, sequence, head): the fold and write-back of
//         the committed state, [k; q] S0^T on the matrix cores, then u and o per (node, row).
//
// Matrix-core layout of the main kernel (v_mfma_f32_16x16x32_bf16, fp32 accumulate): wave w
// owns state rows [32w, 32w+32); lane l holds rows 32w + 16nt + (l % 16) and columns
// 16mt + 4(l / 16) + e (nt < 2, mt < 8, e < 4), which are exactly the B operands of a 32-wide
// k-step kb when that step takes columns {32kb + 4(l/16) + e} and {32kb + 16 + 4(l/16) + e};
// the A operands (rows of k and q, from LDS) use the same column order.  S0 is fp32 and enters
// as an exact sum of three bf16 terms (top, next and last 8 significant bits), k and q are
// bf16, so every product is exact and only the fp32 accumulation rounds.
#include <hip/hip_ext.h>

#include "ut_common.h"

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kUtD = 128;

// Workspace records per (layer, sequence, head): n_max node records then nrec_max pair records.
__host__ __device__ inline size_t ut_ws_records(int n_max, int nrec_max) {
    return size_t(n_max) + size_t(nrec_max);
}

// LDS of the prep kernel for trees of at most n nodes and nrec ancestor-or-self records.
struct UtPrepLayout {
    static constexpr int CPV = kUtD * 2 / 16;  // 16-byte chunks per bf16 vector
    // k | q plus one pad chunk: consecutive node rows start 4 banks apart, so the 16 rows an
    // MFMA operand read touches hit distinct banks.
    static constexpr int CPN = 2 * CPV + 1;
    static constexpr int NODE_BYTES = CPN * 16;
    size_t in, bg, pd, tabs, recs, total;
    __host__ __device__ UtPrepLayout(int n, int nrec) {
        const size_t n64 = round_up(size_t(n), 64);
        in = 0;
        bg = in + round_up(size_t(n) * CPN, 64) * 16;  // beta | gate  [n64] x u32
        pd = bg + 2 * n64 * 4;                         // parent | depth [n64] int
        tabs = pd + 2 * n64 * 4;
        // poff[n] | gam[n] | kq[n] | maxdep | lvoff[n+2] | recI | recM | recP | recE | recC |
        // recQ [nrec]
        recs = round_up(tabs + (size_t(4) * n + 3 + size_t(6) * nrec) * 4, 16);
        total = recs + size_t(nrec) * 16;  // rec4 {m, Y, Z, 0}
    }
};

// LDS of the main kernel for trees of at most n nodes, nrec records and nf pending rows.
struct UtMainLayout {
    static constexpr int D = kUtD;
    static constexpr int CPV = D * 2 / 16;
    static constexpr int CPN = 3 * CPV + 1;  // k | q | v + pad chunk (bank spread, as above)
    static constexpr int NODE_BYTES = CPN * 16;
    static constexpr int WS = D + 4;         // row stride of W and GR in floats (bank spread)
    static constexpr int CPR = D * 4 / 16;   // 16-byte chunks per fp32 fold row
    size_t in, ws, work, fold_k, fold_u, fold_lg, gr, total;
    __host__ __device__ UtMainLayout(int n, int nrec, int nf) {
        in = 0;
        ws = in + round_up(size_t(n) * CPN, 64) * 16;  // node records [n] | pair records [nrec]
        work = ws + round_up(size_t(n) + size_t(nrec), 64) * 16;
        const size_t fk = round_up(size_t(nf) * CPR, 64) * 16;  // W | GR alias the fold rows
        fold_k = work;
        fold_u = work + fk;
        fold_lg = work + 2 * fk;
        const size_t fold_bytes = 2 * fk + round_up(size_t(nf), 64) * 4;
        gr = work + size_t(n) * WS * 4;
        const size_t wg_bytes = size_t(2) * n * WS * 4;
        total = work + (wg_bytes > fold_bytes ? wg_bytes : fold_bytes);
    }
};

// Exact split of 8 fp32 values into three bf16 vectors (hi + mid + lo == x for normal x): each
// term takes the next 8 significant bits by truncation, so every remainder is exact.
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

// Orders LDS accesses of one wave across lanes: the compiler keeps them in program order and
// the hardware performs one wave's LDS instructions in issue order.
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

// First workspace record of a (layer, sequence, head).
__device__ __forceinline__ size_t ut_ws_base(const VerifyParams &P, const UtUnit &u,
                                             int n_max, int nrec_max) {
    return ((size_t(u.layer_rel) * P.S + u.seq) * P.H + u.h) * ut_ws_records(n_max, nrec_max);
}

// ------------------------------------------------------------------------------------------
// prep: one wave per (layer, sequence, head)
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64)
void verify_ut_prep_kernel(VerifyParams P, int n_max, int nrec_max) {
    constexpr int D = kUtD;
    using LY = UtPrepLayout;
    extern __shared__ __align__(16) float dyn[];
    char *lds = reinterpret_cast<char *>(dyn);
    const LY lay(n_max, nrec_max);
    const size_t n64 = round_up(size_t(n_max), 64);
    const char *IN = lds + lay.in;
    const uint32_t *Bl = reinterpret_cast<const uint32_t *>(lds + lay.bg);
    const uint32_t *Gt = Bl + n64;
    const int *par = reinterpret_cast<const int *>(lds + lay.pd);
    const int *dep = par + n64;
    int *poff = reinterpret_cast<int *>(lds + lay.tabs);
    float *gam = reinterpret_cast<float *>(poff + n_max);
    float *kq = gam + n_max;
    int *maxdep = reinterpret_cast<int *>(kq + n_max);
    int *lvoff = maxdep + 1;  // first record of each depth level
    // Record q of node n at distance s + 1 (s = -1: n itself): recI = depth(n) << 16 | (s + 1),
    // recM = the ancestor, recP = that ancestor's first record, recE = E(n, ancestor),
    // recC = T[n][ancestor], recQ = C[n][ancestor].
    int *recI = lvoff + n_max + 2, *recM = recI + nrec_max, *recP = recM + nrec_max;
    float *recE = reinterpret_cast<float *>(recP + nrec_max);
    float *recC = recE + nrec_max, *recQ = recC + nrec_max;
    float4 *rec4 = reinterpret_cast<float4 *>(lds + lay.recs);

    const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
    const UtUnit un = ut_unit(P);
    const int layer = P.layer_begin + un.layer_rel, seq = un.seq, h = un.h;
    const int seq_off = P.img[P.off_seq + seq];
    const int n = P.img[P.off_seq + seq + 1] - seq_off;
    const int role = P.role[seq];
    const int64_t sh = (int64_t(layer) * P.S + seq) * P.H + h;
    const int64_t row0_bank = sh * P.max_nodes;
    const int64_t node_row0 = (int64_t(layer) * P.T + seq_off) * P.H + h;  // node 0's row
    if (n == 0) return;

    // ---- direct loads: k, q, beta, g, parents, depths ------------------------------------
    {
        const char *kb = static_cast<const char *>(P.k), *qb = static_cast<const char *>(P.q);
        const int total = n * LY::CPN;
        for (int base = 0; base < total; base += 64) {
            const int c = min(base + lane, total - 1);  // padding lanes re-read the last chunk
            const int node = c / LY::CPN, r = c % LY::CPN;
            const bool real = r < 2 * LY::CPV;  // the pad chunk re-reads the key's first chunk
            const int vec = real ? r / LY::CPV : 0, idx = real ? r % LY::CPV : 0;
            const char *src = (vec == 0 ? kb : qb) + (node_row0 + int64_t(node) * P.H) * D * 2 +
                              idx * 16;
            to_lds<16>(src, lds + lay.in + size_t(base) * 16);
        }
        for (int base = 0; base < int(4 * n64); base += 64) {
            const int which = base / int(n64), t = min(base % int(n64) + lane, n - 1);
            if (which < 2) {  // beta, gate
                const bf16_t *src = static_cast<const bf16_t *>(which == 0 ? P.beta : P.gate) +
                                    node_row0 + int64_t(t) * P.H;
                to_lds<2>(src, lds + lay.bg + size_t(base) * 4);
            } else {  // parent, depth (global ids / edges)
                const int32_t *src =
                    P.img + (which == 2 ? P.off_parent : P.off_depth) + seq_off + t;
                to_lds<4>(src, lds + lay.pd + size_t(base - 2 * int(n64)) * 4);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // every direct load has landed in LDS
    wave_lds_order();

    // ---- tables --------------------------------------------------------------------------
    // Every node owns a block of depth + 1 records (itself, then its ancestors nearest first).
    // Blocks are laid out by depth level, and by index inside a level, so that the records of
    // one level are contiguous: lvoff[lv] .. lvoff[lv + 1].
    {
        int dmax = 0;
        for (int c = 0; c < n; c += 64) dmax = max(dmax, c + lane < n ? dep[c + lane] : 0);
#pragma unroll
        for (int d2 = 32; d2 >= 1; d2 >>= 1) dmax = max(dmax, __shfl_xor(dmax, d2));
        int base = 0;
        for (int lv = 0; lv <= dmax; ++lv) {
            if (lane == 0) lvoff[lv] = base;
            int run = 0;
            for (int c = 0; c < n; c += 64) {
                const int t = c + lane;
                const bool on = t < n && dep[t] == lv;
                const uint64_t m = __ballot(on);
                const int below = __builtin_amdgcn_mbcnt_hi(
                    uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0));
                if (on) poff[t] = base + (run + below) * (lv + 1);
                run += __popcll(m);
            }
            base += run * (lv + 1);
        }
        if (lane == 0) {
            lvoff[dmax + 1] = base;
            *maxdep = dmax;
        }
    }
    wave_lds_order();
    for (int t = lane; t < n; t += 64) {
        const int o = poff[t], dt = dep[t];
        recI[o] = dt << 16;
        recM[o] = t;
        recP[o] = o;
        recE[o] = 1.f;
        float E = slot_f32<bf16_t>(Gt[t]);
        int a = par[t] - seq_off;  // global -> local; only depth(t) steps: never the root's -1
        for (int s2 = 0; s2 < dt; ++s2) {
            recI[o + 1 + s2] = (dt << 16) | (s2 + 1);
            recM[o + 1 + s2] = a;
            recP[o + 1 + s2] = poff[a];
            recE[o + 1 + s2] = E;
            E *= slot_f32<bf16_t>(Gt[a]);
            a = par[a] - seq_off;
        }
        gam[t] = E;
    }
    wave_lds_order();

    // ---- pair coefficients: [k; q] K^T on the matrix cores -----------------------------
    // M tile jt stacks k (rows 0-7) and q (rows 8-15) of nodes 8jt .. 8jt+7; N tile at holds
    // the keys of nodes 16at .. 16at+15.  Lane (lr, lg) receives rows 4lg + r: k . k_a for
    // lg < 2 and q . k_a for lg >= 2, of node 8jt + 4(lg & 1) + r, with a = 16at + lr.
    const int JT = (n + 7) >> 3, AT = (n + 15) >> 4;
    for (int ti = 0; ti < JT * AT; ++ti) {
        const int jt = ti / AT, at = ti % AT;
        const int xn = 8 * jt + (lr & 7), kn = 16 * at + lr;
        const char *xrow = IN + size_t(xn) * LY::NODE_BYTES + (lr >> 3) * D * 2;
        const char *krow = IN + size_t(kn) * LY::NODE_BYTES;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 z = {};
            const bf16x8 a = xn < n ? row_operand(xrow, 32 * kb + 4 * lg) : z;
            const bf16x8 b = kn < n ? row_operand(krow, 32 * kb + 4 * lg) : z;
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
        }
        const int an = 16 * at + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int nd = 8 * jt + 4 * (lg & 1) + r;
            const bool is_q = lg >= 2;
            if (nd >= n || an >= n) continue;
            if (an == nd) {
                if (is_q) kq[nd] = acc[r];
                continue;
            }
            const int dn = dep[nd], da = dep[an];
            if (da >= dn) continue;
            const int q = poff[nd] + dn - da;  // record of the ancestor at distance dn - da
            if (recM[q] != an) continue;
            if (is_q)
                recQ[q] = recE[q] * acc[r];
            else
                recC[q] = slot_f32<bf16_t>(Bl[nd]) * recE[q] * acc[r];
        }
    }
    wave_lds_order();

    // ---- Y = T^-1 and Z = C Y on ancestor-or-self records ------------------------------
    // Record poff[n] is n itself; poff[n] + 1 + s is n's ancestor at distance s + 1.  Y[n][m]
    // for m = anc_s(n) needs Y[a][m] of the nodes a strictly between, all on lower levels, so
    // the levels are walked in order.  The term of anc_t(n) reads Y[anc_t(n)][anc_s(n)], which
    // is record recP[q0 + 1 + t] + s - t.
    const int dmax = *maxdep, nrec = lvoff[dmax + 1];
    for (int t = lane; t < n; t += 64)
        rec4[poff[t]] = make_float4(__int_as_float(t), 1.f, kq[t], 0.f);
    wave_lds_order();
    for (int lv = 1; lv <= dmax; ++lv) {
        const int b0 = lvoff[lv], b1 = lvoff[lv + 1];
        for (int q = b0 + lane; q < b1; q += 64) {
            const int sd = (q - b0) % (lv + 1) - 1;
            if (sd < 0) continue;
            const int q1 = q - sd;  // first ancestor record of the node
            float y = -recC[q], y2 = 0.f;
            int t = 0;
            for (; t + 2 <= sd; t += 2) {
                const float c0 = recC[q1 + t], c1 = recC[q1 + t + 1];
                const int p0 = recP[q1 + t], p1 = recP[q1 + t + 1];
                y = fmaf(-c0, rec4[p0 + sd - t].y, y);
                y2 = fmaf(-c1, rec4[p1 + sd - t - 1].y, y2);
            }
            if (t < sd) y = fmaf(-recC[q1 + t], rec4[recP[q1 + t] + sd - t].y, y);
            rec4[q] = make_float4(__int_as_float(recM[q]), y + y2, 0.f, 0.f);
        }
        wave_lds_order();
    }
    for (int q = lane; q < nrec; q += 64) {
        const int sd = (recI[q] & 0xFFFF) - 1;
        if (sd < 0) continue;
        const int q1 = q - sd;
        float z = fmaf(rec4[q1 - 1].z, rec4[q].y, recQ[q]), z2 = 0.f;  // self record: kq
        int t = 0;
        for (; t + 2 <= sd; t += 2) {
            const float c0 = recQ[q1 + t], c1 = recQ[q1 + t + 1];
            const int p0 = recP[q1 + t], p1 = recP[q1 + t + 1];
            z = fmaf(c0, rec4[p0 + sd - t].y, z);
            z2 = fmaf(c1, rec4[p1 + sd - t - 1].y, z2);
        }
        if (t < sd) z = fmaf(recQ[q1 + t], rec4[recP[q1 + t] + sd - t].y, z);
        rec4[q].z = z + z2;
    }
    wave_lds_order();

    // ---- records to the workspace; banked keys and log-gates ---------------------------
    float4 *ws = reinterpret_cast<float4 *>(P.boundary) + ut_ws_base(P, un, n_max, nrec_max);
    for (int t = lane; t < n; t += 64)
        ws[t] = make_float4(__int_as_float(poff[t]), __int_as_float(dep[t]), gam[t],
                            slot_f32<bf16_t>(Bl[t]));
    for (int q = lane; q < nrec; q += 64) ws[n_max + q] = rec4[q];
    float *wk = P.bank_k[role ^ 1], *wlg = P.bank_lg[role ^ 1];
    for (int e = lane; e < n * (D / 4); e += 64) {
        const int nd = e / (D / 4), c = (e % (D / 4)) * 4;
        const uint2 x = *reinterpret_cast<const uint2 *>(IN + size_t(nd) * LY::NODE_BYTES + c * 2);
        *reinterpret_cast<float4 *>(wk + (row0_bank + nd) * D + c) =
            make_float4(bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y));
    }
    for (int t = lane; t < n; t += 64) wlg[row0_bank + t] = logf(slot_f32<bf16_t>(Gt[t]));
}

// ------------------------------------------------------------------------------------------
// main: one workgroup of 4 waves per (layer, sequence, head)
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256, GDN_VERIFY_MIN_WAVES)
void verify_ut_main_kernel(VerifyParams P, int n_max, int nrec_max, int nf_max) {
    constexpr int D = kUtD, THREADS = 256, NW = 4, JC = 4;
    using LY = UtMainLayout;
    extern __shared__ __align__(16) float dyn[];
    char *lds = reinterpret_cast<char *>(dyn);
    const LY lay(n_max, nrec_max, nf_max);
    const char *IN = lds + lay.in;
    const float4 *NI = reinterpret_cast<const float4 *>(lds + lay.ws);  // node records
    const float4 *REC = NI + n_max;                                     // pair records
    float *Wm = reinterpret_cast<float *>(lds + lay.work);
    float *GR = reinterpret_cast<float *>(lds + lay.gr);
    const float *FK = reinterpret_cast<const float *>(lds + lay.fold_k);
    const float *FU = reinterpret_cast<const float *>(lds + lay.fold_u);
    const float *FL = reinterpret_cast<const float *>(lds + lay.fold_lg);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const UtUnit un = ut_unit(P);
    const int layer = P.layer_begin + un.layer_rel, seq = un.seq, h = un.h;
    const int seq_off = P.img[P.off_seq + seq];
    const int n = P.img[P.off_seq + seq + 1] - seq_off;
    // pending counts come from the commit call, which bounds them by the bank rows; the clamp
    // keeps a corrupted count from reading past the bank.
    const int role = P.role[seq], L = min(max(P.pending[seq], 0), P.max_nodes);
    const int64_t sh = (int64_t(layer) * P.S + seq) * P.H + h;
    float *committed = P.state + sh * D * D;
    const int64_t row0_bank = sh * P.max_nodes;
    const int64_t node_row0 = (int64_t(layer) * P.T + seq_off) * P.H + h;  // node 0's row

    // ---- direct loads: k, q, v, the prep records, the pending fold rows -----------------
    {
        const char *kb = static_cast<const char *>(P.k), *qb = static_cast<const char *>(P.q),
                   *vb = static_cast<const char *>(P.v);
        const int total = n * LY::CPN;
        for (int base = w * 64; base < total; base += NW * 64) {
            const int c = min(base + lane, total - 1);  // padding lanes re-read the last chunk
            const int node = c / LY::CPN, r = c % LY::CPN;
            const bool real = r < 3 * LY::CPV;  // the pad chunk re-reads the key's first chunk
            const int vec = real ? r / LY::CPV : 0, idx = real ? r % LY::CPV : 0;
            const char *src = (vec == 0 ? kb : (vec == 1 ? qb : vb)) +
                              (node_row0 + int64_t(node) * P.H) * D * 2 + idx * 16;
            to_lds<16>(src, lds + lay.in + size_t(base) * 16);
        }
        if (n > 0) {  // node records [0, n_max) then pair records: the whole unit is copied
            const float4 *ws = reinterpret_cast<const float4 *>(P.boundary) +
                               ut_ws_base(P, un, n_max, nrec_max);
            const int chunks = int(ut_ws_records(n_max, nrec_max));
            for (int base = w * 64; base < chunks; base += NW * 64)
                to_lds<16>(ws + min(base + lane, chunks - 1), lds + lay.ws + size_t(base) * 16);
        }
        if (L > 0) {
            const float *pk = P.bank_k[role] + row0_bank * D, *pu = P.bank_u[role] + row0_bank * D;
            const int rows_chunks = L * LY::CPR;
            const int fk_chunks = int(round_up(size_t(nf_max) * LY::CPR, 64));
            for (int base = w * 64; base < 2 * fk_chunks; base += NW * 64) {
                const int which = base / fk_chunks, b2 = base % fk_chunks;
                if (b2 >= rows_chunks) continue;
                const int c = min(b2 + lane, rows_chunks - 1);
                const float *src = (which == 0 ? pk : pu) + c * 4;
                to_lds<16>(src, lds + lay.fold_k + size_t(base) * 16);
            }
            const float *plg = P.bank_lg[role] + row0_bank;
            for (int base = w * 64; base < L; base += NW * 64)
                to_lds<4>(plg + min(base + lane, L - 1), lds + lay.fold_lg + size_t(base) * 4);
        }
    }
    __syncthreads();  // waits for every direct load (the barrier's fence covers them)

    float s[2][8][4];  // rows 32w + 16nt + lr, columns 16mt + 4lg + e
    {
        const float *tile = committed + (32 * w + lr) * D + 4 * lg;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                const float4 x = *reinterpret_cast<const float4 *>(tile + 16 * nt * D + 16 * mt);
                s[nt][mt][0] = x.x;
                s[nt][mt][1] = x.y;
                s[nt][mt][2] = x.z;
                s[nt][mt][3] = x.w;
            }
    }

    // ---- F. deferred commit: fold the pending rows, write the committed state once --------
    for (int f = 0; f < L; ++f) {
        const float gf = expf(FL[f]);
        const float u0 = FU[f * D + 32 * w + lr], u1 = FU[f * D + 32 * w + 16 + lr];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const float4 k4 = *reinterpret_cast<const float4 *>(FK + f * D + 16 * mt + 4 * lg);
            const float kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[0][mt][e] = fmaf(u0, kk[e], gf * s[0][mt][e]);
                s[1][mt][e] = fmaf(u1, kk[e], gf * s[1][mt][e]);
            }
        }
    }
    if (L > 0) {
        float *tile = committed + (32 * w + lr) * D + 4 * lg;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                *reinterpret_cast<float4 *>(tile + 16 * nt * D + 16 * mt) =
                    make_float4(s[nt][mt][0], s[nt][mt][1], s[nt][mt][2], s[nt][mt][3]);
    }
    __syncthreads();  // fold rows are dead: their LDS becomes W and GR

    // ---- A. p_n = S0 k_n, r_n = S0 q_n on the matrix cores; w_n and G_n r_n to LDS -------
    const int JT = (n + 7) >> 3;
    for (int jt0 = 0; jt0 < JT; jt0 += JC) {
        floatx4 acc[JC][2];
#pragma unroll
        for (int jc = 0; jc < JC; ++jc)
            acc[jc][0] = acc[jc][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            bf16x8 bh[2], bm[2], bl[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const float x[8] = {s[nt][2 * kb][0],     s[nt][2 * kb][1],
                                    s[nt][2 * kb][2],     s[nt][2 * kb][3],
                                    s[nt][2 * kb + 1][0], s[nt][2 * kb + 1][1],
                                    s[nt][2 * kb + 1][2], s[nt][2 * kb + 1][3]};
                split3(x, bh[nt], bm[nt], bl[nt]);
            }
#pragma unroll
            for (int jc = 0; jc < JC; ++jc) {
                const int jt = jt0 + jc;
                if (jt >= JT) break;
                const int xn = 8 * jt + (lr & 7);
                const bf16x8 z = {};
                const bf16x8 a = xn < n
                    ? row_operand(IN + size_t(xn) * LY::NODE_BYTES + (lr >> 3) * D * 2,
                                  32 * kb + 4 * lg)
                    : z;
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    acc[jc][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl[nt], acc[jc][nt], 0, 0, 0);
                    acc[jc][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bm[nt], acc[jc][nt], 0, 0, 0);
                    acc[jc][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh[nt], acc[jc][nt], 0, 0, 0);
                }
            }
        }
        // Lane (lr, lg) holds rows 4lg + r of each M tile: p of node 8jt + 4lg + r for lg < 2,
        // r of node 8jt + 4(lg - 2) + r for lg >= 2, at state row 32w + 16nt + lr.
#pragma unroll
        for (int jc = 0; jc < JC; ++jc) {
            const int jt = jt0 + jc;
            if (jt >= JT) break;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int nd = 8 * jt + 4 * (lg & 1) + r;
                if (nd >= n) continue;
                const float4 ni = NI[nd];  // {records offset, depth, G, beta}
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int i = 32 * w + 16 * nt + lr;
                    if (lg < 2) {
                        const float v = bf16_at(IN + size_t(nd) * LY::NODE_BYTES + 2 * D * 2, i);
                        Wm[nd * LY::WS + i] = ni.w * fmaf(-ni.z, acc[jc][nt][r], v);
                    } else {
                        GR[nd * LY::WS + i] = ni.z * acc[jc][nt][r];
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- O. u_n, o_n per (node, row); banked u ------------------------------------------
    {
        float *wu = P.bank_u[role ^ 1];
        float *out0 = P.out + node_row0 * D;
        const int i = tid & (D - 1);
        for (int nd = tid >> 7; nd < n; nd += THREADS / D) {
            const float4 ni = NI[nd];
            float u = 0.f, u2 = 0.f, o = GR[nd * LY::WS + i], o2 = 0.f;
            int q = __float_as_int(ni.x);
            const int qe = q + __float_as_int(ni.y) + 1;
            for (; q + 2 <= qe; q += 2) {
                const float4 r0 = REC[q], r1 = REC[q + 1];
                const float w0 = Wm[__float_as_int(r0.x) * LY::WS + i];
                const float w1 = Wm[__float_as_int(r1.x) * LY::WS + i];
                u = fmaf(r0.y, w0, u);
                o = fmaf(r0.z, w0, o);
                u2 = fmaf(r1.y, w1, u2);
                o2 = fmaf(r1.z, w1, o2);
            }
            if (q < qe) {
                const float4 r0 = REC[q];
                const float w0 = Wm[__float_as_int(r0.x) * LY::WS + i];
                u = fmaf(r0.y, w0, u);
                o = fmaf(r0.z, w0, o);
            }
            wu[(row0_bank + nd) * D + i] = u + u2;
            out0[int64_t(nd) * P.H * D + i] = o + o2;
        }
    }
}

size_t ut_mfma_workspace_bytes(int n_layers, int S, int H, int n_max, int np_max) {
    return size_t(n_layers) * S * H * ut_ws_records(n_max, np_max + n_max) * 16;
}

gdn_status launch_ut_mfma(const VerifyParams &P, int n_max, int np_max, int nf_max,
                          hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const int nrec_max = np_max + n_max;
    const size_t lds_prep = UtPrepLayout(n_max, nrec_max).total;
    const size_t lds_main = UtMainLayout(n_max, nrec_max, nf_max).total;
    const size_t lds = lds_prep > lds_main ? lds_prep : lds_main;
    if (lds > kUtMaxLdsBytes)
        return fail(GDN_EINVAL, "gdn_tree_verify_ut: trees of %d nodes with %d ancestor pairs "
                    "and %d bank rows need %zu bytes of LDS (limit %zu); use gdn_tree_verify",
                    n_max, np_max, nf_max, lds, kUtMaxLdsBytes);
    if (P.n_blocks <= 0) return GDN_OK;
    if (P.boundary == nullptr)
        return fail(GDN_EINVAL, "gdn_tree_verify_ut: bf16 inputs at d = 128 need a workspace "
                    "of gdn_verify_ut_workspace_bytes() bytes");
    const dim3 grid(uint32_t(P.n_blocks));
    if (start == nullptr && stop == nullptr) {
        hipLaunchKernelGGL(verify_ut_prep_kernel, grid, dim3(64), lds_prep, stream, P, n_max,
                           nrec_max);
        GDN_LAUNCH_CHECK("verify_ut_prep_kernel");
        hipLaunchKernelGGL(verify_ut_main_kernel, grid, dim3(256), lds_main, stream, P, n_max,
                           nrec_max, nf_max);
    } else {  // start stamped by the prep dispatch, stop by the main dispatch
        hipExtLaunchKernelGGL(verify_ut_prep_kernel, grid, dim3(64), uint32_t(lds_prep), stream,
                              start, nullptr, 0, P, n_max, nrec_max);
        GDN_LAUNCH_CHECK("verify_ut_prep_kernel");
        hipExtLaunchKernelGGL(verify_ut_main_kernel, grid, dim3(256), uint32_t(lds_main), stream,
                              nullptr, stop, 0, P, n_max, nrec_max, nf_max);
    }
    GDN_LAUNCH_CHECK("verify_ut_main_kernel");
    return GDN_OK;
}

}  // namespace gdn
