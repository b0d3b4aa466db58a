// Tree-masked UT verify: every node of a tree from the committed state and the factors of its
// ancestors, with no per-node state, no boundary tiles and no dependency waves, for gfx950.
//
// "Lucebox SpecLA and Gated DeltaNet state-resident verification" guide, mechanism 1, names a
// topology-mask (UT decomposition) form of the tree verify beside the chain kernels.  It
// follows from unrolling S_n = g_n S_parent + u_n k_n^T down n's root path A(n):
//   S_n = G_n S0 + sum_{j in A(n)} E(n,j) u_j k_j^T,   G_n = prod_{m in A(n)} g_m,
//   E(n,j) = product of the gates on the path strictly below j down to n (E(n,n) = 1),
// so, with p_n = S0 k_n and r_n = S0 q_n,
//   u_n = beta_n (v_n - G_n p_n - sum_{j in A(n), j != n} E(n,j) (k_n . k_j) u_j)
//   o_n = G_n r_n + sum_{j in A(n)} E(n,j) (q_n . k_j) u_j.
// Parents have lower indices than their children, so walking the tree in index order finds
// every ancestor's u_j already computed.  S0 is the committed state after the deferred fold
// of mechanism 4 (written back once); it stays in VGPRs and p_n, r_n are its only products.
// E is formed by multiplying gates along the path, never by dividing two root-path products,
// so deep paths with small gates cannot underflow a quotient.
//
// One workgroup per (layer, sequence, head), with the chain kernel's tile layout (every row's
// columns in one lane octet).  The whole tree is handled in LDS:
//   0. direct global->LDS loads (global_load_lds) bring in every node's k, q, v, beta, g, the
//      parents and depths, and the pending fold rows, while the state tile loads into VGPRs;
//      one wait, one barrier;
//   1. tree tables: pair offsets (prefix sum of depths), every node's ancestor list (nearest
//      first) with the gate products E along it, and G_n;
//   2. the fold: S <- exp(lg) S + u k^T per pending row, then S is written back once;
//   A. p_n = S0 k_n and r_n = S0 q_n for all nodes (octet reductions), keys banked;
//   K. one lane octet per (node, strict ancestor) pair: E (k_n . k_a) and E (q_n . k_a);
//   B. one thread per row runs u_n[r] over the nodes in index order (u overwrites p in LDS);
//   C. all threads form o_n[r], parallel over (node, row).
// No global load happens after step 0, so no wait on memory sits inside the node work; all
// global stores are fire-and-forget.
#include <hip/hip_ext.h>

#include <algorithm>

#include "ut_common.h"

namespace gdn {

// Byte offsets of the dynamic LDS regions for trees of at most n nodes, np (node, strict
// ancestor) pairs and at most nf pending fold rows.  Regions filled by direct loads are
// padded to whole 64-lane instructions.
template <int D, typename TIn> struct UtLayout {
    static constexpr int CPV = D * int(sizeof(TIn)) / 16;  // 16-byte chunks per input vector
    static constexpr int CPN = 3 * CPV;                      // per node: k | q | v
    static constexpr int CPR = D * 4 / 16;                   // per fp32 fold row
    size_t in, bg, pd, work, fold_k, fold_u, fold_lg, pairs, tabs, total;
    __host__ __device__ UtLayout(int n, int np, int nf) {
        const size_t n64 = round_up(size_t(n), 64);
        in = 0;
        bg = in + round_up(size_t(n) * CPN, 64) * 16;           // beta | gate  [n64] x u32
        pd = bg + 2 * n64 * 4;                                  // parent | depth [n64] int
        work = pd + 2 * n64 * 4;                                // P/U [n][D] | R [n][D]
        const size_t fk = round_up(size_t(nf) * CPR, 64) * 16;  // fold rows, aliasing work
        const size_t fold_bytes = 2 * fk + round_up(size_t(nf), 64) * 4;
        fold_k = work;
        fold_u = work + fk;
        fold_lg = work + 2 * fk;
        const size_t pr = size_t(2) * n * D * 4;
        pairs = work + (pr > fold_bytes ? pr : fold_bytes);     // anc|pnode|E|cK|cQ [np]
        tabs = pairs + size_t(np) * 5 * 4;                      // aoff[n+1] | G[n] | kq[n]
        total = tabs + (size_t(3) * n + 1) * 4;
    }
};

// VEC (4 or 2) consecutive elements of input vector `vec` (0 k, 1 q, 2 v) of a node, fp32.
template <int D, typename TIn, int VEC>
__device__ __forceinline__ void in_vec(const char *lds, int node, int vec, int col, float *o) {
    const char *p = lds + (size_t(node) * 3 + vec) * D * sizeof(TIn) + size_t(col) * sizeof(TIn);
    if (sizeof(TIn) == 2 && VEC == 4) {
        const uint2 x = *reinterpret_cast<const uint2 *>(p);
        o[0] = bf16_lo(x.x);
        o[1] = bf16_hi(x.x);
        o[2] = bf16_lo(x.y);
        o[3] = bf16_hi(x.y);
    } else if (sizeof(TIn) == 2) {
        const uint32_t x = *reinterpret_cast<const uint32_t *>(p);
        o[0] = bf16_lo(x);
        o[1] = bf16_hi(x);
    } else if (VEC == 4) {
        const float4 x = *reinterpret_cast<const float4 *>(p);
        o[0] = x.x;
        o[1] = x.y;
        o[2] = x.z;
        o[3] = x.w;
    } else {
        const float2 x = *reinterpret_cast<const float2 *>(p);
        o[0] = x.x;
        o[1] = x.y;
    }
}

template <int D, typename TIn>
__device__ __forceinline__ float in_elem(const char *lds, int node, int vec, int i) {
    const char *p = lds + (size_t(node) * 3 + vec) * D * sizeof(TIn) + size_t(i) * sizeof(TIn);
    if (sizeof(TIn) == 2) return bf16_lo(*reinterpret_cast<const uint16_t *>(p));
    return *reinterpret_cast<const float *>(p);
}

template <int D, typename TIn>
__global__ __launch_bounds__(Tile<D>::THREADS, sizeof(TIn) == 2 ? GDN_VERIFY_MIN_WAVES : 2)
void verify_ut_kernel(VerifyParams P, int n_max, int np_max, int nf_max) {
    using TL = Tile<D>;
    using LY = UtLayout<D, TIn>;
    constexpr int M = TL::M, NP = TL::NP, VEC = TL::VEC, THREADS = TL::THREADS, NW = TL::NW;
    constexpr int NOCT = THREADS / 8;  // lane octets per workgroup
    typedef VecT<VEC> V;
    extern __shared__ __align__(16) float dyn[];
    char *lds = reinterpret_cast<char *>(dyn);
    const LY lay(n_max, np_max, nf_max);
    const size_t n64 = round_up(size_t(n_max), 64);
    const char *IN = lds + lay.in;
    const uint32_t *Bl = reinterpret_cast<const uint32_t *>(lds + lay.bg);  // one dword per node
    const uint32_t *Gt = Bl + n64;
    const int *par = reinterpret_cast<const int *>(lds + lay.pd);
    const int *dep = par + n64;
    float *PU = reinterpret_cast<float *>(lds + lay.work);  // p, then u in place
    float *Rr = PU + size_t(n_max) * D;
    const float *FK = reinterpret_cast<const float *>(lds + lay.fold_k);
    const float *FU = reinterpret_cast<const float *>(lds + lay.fold_u);
    const float *FL = reinterpret_cast<const float *>(lds + lay.fold_lg);
    int *anc = reinterpret_cast<int *>(lds + lay.pairs);
    int *pnode = anc + np_max;
    float *Ep = reinterpret_cast<float *>(pnode + np_max);
    float *cK = Ep + np_max, *cQ = cK + np_max;
    int *aoff = reinterpret_cast<int *>(lds + lay.tabs);
    float *gam = reinterpret_cast<float *>(aoff + n_max + 1);
    float *kqn = gam + n_max;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
    const int rg = lane >> 3, cl = lane & 7, oc = tid >> 3;
    // Grids are capped at kMaxBlocks workgroups, so block arithmetic stays in 32 bits.
    const uint32_t logical = xcd_logical(blockIdx.x, uint32_t(P.n_blocks));
    const uint32_t per = uint32_t(P.S) * uint32_t(P.H);
    const int layer_rel = int(logical / per);
    const int seq = int((logical % per) / uint32_t(P.H)), h = int(logical % uint32_t(P.H));
    const int layer = P.layer_begin + layer_rel;
    const int seq_off = P.img[P.off_seq + seq];
    const int n = P.img[P.off_seq + seq + 1] - seq_off;
    const int role = P.role[seq], L = min(max(P.pending[seq], 0), P.max_nodes);
    const int64_t sh = (int64_t(layer) * P.S + seq) * P.H + h;
    float *committed = P.state + sh * D * D;
    const int64_t row0_bank = sh * P.max_nodes;
    float *wk = P.bank_k[role ^ 1], *wu = P.bank_u[role ^ 1], *wlg = P.bank_lg[role ^ 1];

    // The committed tile is requested first: its address needs only the workgroup's ids.
    const int row0 = w * TL::RW + rg;
    const int col0 = cl * VEC;
    const int toff = row0 * D + col0;
#define GDN_T(m, p) (toff + (m) * 8 * D + (p) * 8 * VEC)
#define GDN_ROW(m) (row0 + 8 * (m))
#define GDN_COL(p) (col0 + (p) * 8 * VEC)
    float s[M][NP][VEC];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int p = 0; p < NP; ++p) V::get(committed + GDN_T(m, p), s[m][p]);

    // ---- 0. direct loads of the tree's inputs, tables and pending rows into LDS ----------
    const int64_t node_row0 = (int64_t(layer) * P.T + seq_off) * P.H + h;  // node 0's row
    {
        const char *kb = static_cast<const char *>(P.k), *qb = static_cast<const char *>(P.q),
                   *vb = static_cast<const char *>(P.v);
        const int total = n * LY::CPN;
        for (int base = w * 64; base < total; base += NW * 64) {
            const int c = min(base + lane, total - 1);  // padding lanes re-read the last chunk
            const int node = c / LY::CPN, r = c % LY::CPN, vec = r / LY::CPV, idx = r % LY::CPV;
            const char *src = (vec == 0 ? kb : (vec == 1 ? qb : vb)) +
                              (node_row0 + int64_t(node) * P.H) * D * int64_t(sizeof(TIn)) + idx * 16;
            to_lds<16>(src, lds + lay.in + size_t(base) * 16);
        }
        for (int base = w * 64; base < int(4 * n64); base += NW * 64) {
            const int which = base / int(n64), t = min(base % int(n64) + lane, n - 1);
            if (which < 2) {  // beta, gate
                const TIn *src = static_cast<const TIn *>(which == 0 ? P.beta : P.gate) +
                                 node_row0 + int64_t(t) * P.H;
                to_lds<int(sizeof(TIn))>(src, lds + lay.bg + size_t(base) * 4);
            } else {  // parent, depth (global ids / edges)
                const int32_t *src =
                    P.img + (which == 2 ? P.off_parent : P.off_depth) + seq_off + t;
                to_lds<4>(src, lds + lay.pd + size_t(base - 2 * int(n64)) * 4);
            }
        }
        if (L > 0) {
            // pending factor f sits in bank row rm[f] (the commit's row map, clamped to the bank)
            const int32_t *rm = P.rows + int64_t(seq) * P.max_nodes;
            const int mrow = P.max_nodes - 1;
            const float *pk = P.bank_k[role] + row0_bank * D, *pu = P.bank_u[role] + row0_bank * D;
            const int rows_chunks = L * LY::CPR;
            const int fk_chunks = int(round_up(size_t(nf_max) * LY::CPR, 64));
            for (int base = w * 64; base < 2 * fk_chunks; base += NW * 64) {
                const int which = base / fk_chunks, b2 = base % fk_chunks;
                if (b2 >= rows_chunks) continue;
                const int c = min(b2 + lane, rows_chunks - 1);
                const int br = min(max(rm[c / LY::CPR], 0), mrow);
                const float *src = (which == 0 ? pk : pu) + int64_t(br) * D + (c % LY::CPR) * 4;
                to_lds<16>(src, lds + lay.fold_k + size_t(base) * 16);
            }
            const float *plg = P.bank_lg[role] + row0_bank;
            for (int base = w * 64; base < L; base += NW * 64)
                to_lds<4>(plg + min(max(rm[min(base + lane, L - 1)], 0), mrow),
                          lds + lay.fold_lg + size_t(base) * 4);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- 1. tree tables --------------------------------------------------------------
    if (w == 0) {
        int carry = 0;
        if (lane == 0) aoff[0] = 0;
        for (int base = 0; base < n; base += 64) {
            const int t = base + lane;
            int x = t < n ? dep[t] : 0;
#pragma unroll
            for (int d2 = 1; d2 < 64; d2 <<= 1) {
                const int y = __shfl_up(x, d2);
                if (lane >= d2) x += y;
            }
            if (t < n) aoff[t + 1] = carry + x;
            carry += __shfl(x, 63);
        }
    }
    __syncthreads();
    for (int t = tid; t < n; t += THREADS) {
        const int o = aoff[t];
        float E = slot_f32<TIn>(Gt[t]);
        int a = par[t] - seq_off;  // global -> local; only depth(t) steps: never the root's -1
        for (int s2 = 0; s2 < dep[t]; ++s2) {
            anc[o + s2] = a;
            pnode[o + s2] = t;
            Ep[o + s2] = E;
            E *= slot_f32<TIn>(Gt[a]);
            a = par[a] - seq_off;
        }
        gam[t] = E;
    }

    // ---- 2. deferred commit ----------------------------------------------------------
    for (int i = 0; i < L; ++i) {
        const float gf = expf(FL[i]);
        float uf[M];
#pragma unroll
        for (int m = 0; m < M; ++m) uf[m] = FU[i * D + GDN_ROW(m)];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float kc[VEC];
            V::get(FK + i * D + GDN_COL(p), kc);
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int e = 0; e < VEC; ++e) s[m][p][e] = fmaf(uf[m], kc[e], gf * s[m][p][e]);
        }
    }
    if (L > 0) {  // the committed state is written back exactly once
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int p = 0; p < NP; ++p) V::put(committed + GDN_T(m, p), s[m][p]);
    }
    __syncthreads();  // fold rows are dead; their LDS becomes P/U and R

    // ---- A. p = S0 k, r = S0 q for every node; keys and log-gates banked ---------------
    for (int i = 0; i < n; ++i) {
        float a[M], b[M], kq = 0.f;
#pragma unroll
        for (int m = 0; m < M; ++m) a[m] = b[m] = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float kc[VEC], qc[VEC];
            in_vec<D, TIn, VEC>(IN, i, 0, GDN_COL(p), kc);
            in_vec<D, TIn, VEC>(IN, i, 1, GDN_COL(p), qc);
#pragma unroll
            for (int e = 0; e < VEC; ++e) kq = fmaf(kc[e], qc[e], kq);
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    a[m] = fmaf(s[m][p][e], kc[e], a[m]);
                    b[m] = fmaf(s[m][p][e], qc[e], b[m]);
                }
        }
        kq = octet_sum(kq);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            a[m] = octet_sum(a[m]);
            b[m] = octet_sum(b[m]);
        }
#pragma unroll
        for (int m = 0; m < M; ++m)
            if (cl == m) {
                PU[i * D + GDN_ROW(m)] = a[m];
                Rr[i * D + GDN_ROW(m)] = b[m];
            }
        if (tid == 0) {
            kqn[i] = kq;
            wlg[row0_bank + i] = logf(slot_f32<TIn>(Gt[i]));
        }
        if (w == 0 && rg == 0) {
            float *krow = wk + (row0_bank + i) * D;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                float kc[VEC];
                in_vec<D, TIn, VEC>(IN, i, 0, GDN_COL(p), kc);
                V::put(krow + GDN_COL(p), kc);
            }
        }
    }

    // ---- K. coefficients of every (node, strict ancestor) pair -------------------------
    const int npairs = aoff[n];
    for (int q = oc; q < npairs; q += NOCT) {
        const int i = pnode[q], a = anc[q];
        float dk = 0.f, dq = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float kn[VEC], qn[VEC], ka[VEC];
            in_vec<D, TIn, VEC>(IN, i, 0, GDN_COL(p), kn);
            in_vec<D, TIn, VEC>(IN, i, 1, GDN_COL(p), qn);
            in_vec<D, TIn, VEC>(IN, a, 0, GDN_COL(p), ka);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                dk = fmaf(kn[e], ka[e], dk);
                dq = fmaf(qn[e], ka[e], dq);
            }
        }
        dk = octet_sum(dk);
        dq = octet_sum(dq);
        if (cl == 0) {
            cK[q] = Ep[q] * dk;
            cQ[q] = Ep[q] * dq;
        }
    }
    __syncthreads();

    // ---- B. u_n[r] = beta_n (v_n[r] - G_n p_n[r] - sum_a E (k_n . k_a) u_a[r]) ---------
    // The ancestor terms are independent of each other: four are read per round so their
    // LDS latencies overlap.
    for (int r = tid; r < D; r += THREADS) {
        for (int i = 0; i < n; ++i) {
            float acc = in_elem<D, TIn>(IN, i, 2, r) - gam[i] * PU[i * D + r];
            int q = aoff[i];
            const int qe = aoff[i + 1];
            float acc2 = 0.f;
            for (; q + 4 <= qe; q += 4) {
                const int a0 = anc[q], a1 = anc[q + 1], a2 = anc[q + 2], a3 = anc[q + 3];
                const float c0 = cK[q], c1 = cK[q + 1], c2 = cK[q + 2], c3 = cK[q + 3];
                const float u0 = PU[a0 * D + r], u1 = PU[a1 * D + r];
                const float u2 = PU[a2 * D + r], u3 = PU[a3 * D + r];
                acc = fmaf(-c0, u0, acc);
                acc2 = fmaf(-c1, u1, acc2);
                acc = fmaf(-c2, u2, acc);
                acc2 = fmaf(-c3, u3, acc2);
            }
            for (; q < qe; ++q) acc = fmaf(-cK[q], PU[anc[q] * D + r], acc);
            const float u = slot_f32<TIn>(Bl[i]) * (acc + acc2);
            PU[i * D + r] = u;
            wu[(row0_bank + i) * D + r] = u;
        }
    }
    __syncthreads();

    // ---- C. o_n[r] = G_n r_n[r] + (q_n . k_n) u_n[r] + sum_a E (q_n . k_a) u_a[r] ------
    float *out0 = P.out + node_row0 * D;
    for (int e = tid; e < n * D; e += THREADS) {
        const int i = e / D, r = e % D;
        float o = fmaf(kqn[i], PU[i * D + r], gam[i] * Rr[i * D + r]);
        float o2 = 0.f;
        int q = aoff[i];
        const int qe = aoff[i + 1];
        for (; q + 4 <= qe; q += 4) {
            const int a0 = anc[q], a1 = anc[q + 1], a2 = anc[q + 2], a3 = anc[q + 3];
            const float c0 = cQ[q], c1 = cQ[q + 1], c2 = cQ[q + 2], c3 = cQ[q + 3];
            const float u0 = PU[a0 * D + r], u1 = PU[a1 * D + r];
            const float u2 = PU[a2 * D + r], u3 = PU[a3 * D + r];
            o = fmaf(c0, u0, o);
            o2 = fmaf(c1, u1, o2);
            o = fmaf(c2, u2, o);
            o2 = fmaf(c3, u3, o2);
        }
        for (; q < qe; ++q) o = fmaf(cQ[q], PU[anc[q] * D + r], o);
        out0[int64_t(i) * P.H * D + r] = o + o2;
    }
#undef GDN_T
#undef GDN_ROW
#undef GDN_COL
}

template <int D, typename TIn>
static gdn_status launch_ut(const VerifyParams &P, int n_max, int np_max, int nf_max,
                            hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const size_t lds = UtLayout<D, TIn>(n_max, np_max, nf_max).total;
    if (lds > kUtMaxLdsBytes)
        return fail(GDN_EINVAL, "gdn_tree_verify_ut: trees of %d nodes with %d ancestor pairs "
                    "and %d bank rows need %zu bytes of LDS (limit %zu); use gdn_tree_verify",
                    n_max, np_max, nf_max, lds, kUtMaxLdsBytes);
    if (P.n_blocks <= 0) return GDN_OK;
    if (start == nullptr && stop == nullptr)
        hipLaunchKernelGGL((verify_ut_kernel<D, TIn>), dim3(uint32_t(P.n_blocks)),
                           dim3(Tile<D>::THREADS), lds, stream, P, n_max, np_max, nf_max);
    else
        hipExtLaunchKernelGGL((verify_ut_kernel<D, TIn>), dim3(uint32_t(P.n_blocks)),
                              dim3(Tile<D>::THREADS), uint32_t(lds), stream, start, stop, 0, P,
                              n_max, np_max, nf_max);
    GDN_LAUNCH_CHECK("verify_ut_kernel");
    return GDN_OK;
}

// Largest tree and largest number of (node, strict ancestor) pairs of any tree of a schedule.
static void ut_tree_bounds(const int32_t *host_image, const ImageView &v, int &n_max,
                           int &np_max) {
    n_max = v.max_tree;
    np_max = 0;
    for (int b = 0; b < v.n_seqs; ++b) {
        int pairs = 0;
        for (int g = host_image[v.off_seq + b]; g < host_image[v.off_seq + b + 1]; ++g)
            pairs += host_image[v.off_depth + g];
        np_max = std::max(np_max, pairs);
    }
}

static gdn_status run_ut(const gdn_verify_args *a, const int32_t *host_image,
                         const int32_t *dev_image, void *stream, hipEvent_t start,
                         hipEvent_t stop) {
    VerifyParams P;
    ImageView v;
    gdn_status st = verify_setup(a, host_image, dev_image, P, v, false);
    if (st != GDN_OK || a->n_seqs == 0) return st;
    P.off_parent = v.off_parent;
    P.off_depth = v.off_depth;
    P.n_blocks = int64_t(a->n_layers) * a->n_seqs * a->n_heads;
    if (P.n_blocks > kMaxBlocks)
        return fail(GDN_EINVAL, "gdn_tree_verify_ut: too many workgroups for one launch");
    int n_max = 0, np_max = 0;
    ut_tree_bounds(host_image, v, n_max, np_max);
    const int nf_max = a->max_nodes;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a->head_dim == 128 && a->in_dtype == GDN_BF16) {
        if (v.ut_records < 0)
            return fail(GDN_EINVAL, "gdn_tree_verify_ut: the schedule has no tree-masked plan "
                        "(its trees need more than %d records per node); use gdn_tree_verify",
                        kUtRecordsPerNode);
        P.off_ut_rec_base = v.off_ut_rec_base;
        P.off_ut_node_rec = v.off_ut_node_rec;
        P.off_ut_lv_base = v.off_ut_lv_base;
        P.off_ut_lvn = v.off_ut_lvn;
        P.off_ut_lvnode = v.off_ut_lvnode;
        P.off_ut_rec_anc = v.off_ut_rec_anc;
        return launch_ut_mfma(P, n_max, v.ut_max_records, v.ut_max_levels, nf_max, s, start,
                              stop);
    }
    if (a->head_dim == 128)
        return launch_ut<128, float>(P, n_max, np_max, nf_max, s, start, stop);
    return a->in_dtype == GDN_BF16
        ? launch_ut<16, bf16_t>(P, n_max, np_max, nf_max, s, start, stop)
        : launch_ut<16, float>(P, n_max, np_max, nf_max, s, start, stop);
}

}  // namespace gdn

using namespace gdn;

extern "C" gdn_status gdn_tree_verify_ut(const gdn_verify_args *a, const int32_t *host_image,
                                         const int32_t *dev_image, void *stream) {
    clear_error();
    return run_ut(a, host_image, dev_image, stream, nullptr, nullptr);
}

extern "C" gdn_status gdn_tree_verify_ut_timed(const gdn_verify_args *a,
                                               const int32_t *host_image,
                                               const int32_t *dev_image, void *start_event,
                                               void *stop_event, void *stream) {
    clear_error();
    if (start_event == nullptr || stop_event == nullptr)
        return fail(GDN_EINVAL, "gdn_tree_verify_ut_timed: null event");
    return run_ut(a, host_image, dev_image, stream, static_cast<hipEvent_t>(start_event),
                  static_cast<hipEvent_t>(stop_event));
}
