// Tree-masked UT verify on the matrix cores, for bf16 inputs and d = 128 (gfx950).
//
// Same method as the vector UT kernel ("Lucebox SpecLA and Gated DeltaNet state-resident
// verification" guide, mechanism 1, topology-mask form): with S0 the committed state after
// the deferred fold (mechanism 4), p_n = S0 k_n, r_n = S0 q_n and
//   w_n = beta_n (v_n - G_n p_n),
//   T[n][a] = beta_n E(n,a) (k_n . k_a)   for a a strict ancestor of n, T[n][n] = 1,
// the residual vectors solve T U = W (T is unit lower triangular in any topological order and
// zero off the ancestor relation), and the outputs are
//   o_n = G_n r_n + (q_n . k_n) u_n + sum_{a strict ancestor} E(n,a) (q_n . k_a) u_a.
//
// One workgroup of 4 waves per (layer, sequence, head):
//   0. direct global->LDS loads of k, q, v, beta, g, parents, depths and the pending fold
//      rows; one barrier;
//   1. the tree's plan (from the schedule image: nodes grouped by depth level, one block of
//      records per node, itself then its ancestors nearest first) gets the gate products E
//      and G_n; keys and log-gates are banked; then the state tile loads into VGPRs are
//      issued, to land while
//   2. the pair products [k; q] K^T run on the matrix cores and give T and C on the records;
//   3. the pending rows are folded in closed form, S = G S0 + sum_f c_f u_f k_f^T (G the product
//      of the pending gates, c_f that of the gates after row f), and S is written back once;
//   4. [k; q] S0^T runs on the matrix cores; its epilogue writes w_n and G_n r_n to LDS;
//   5. wave 0 forms Y = T^-1 and Z = C' Y as dense rows over the consumed node rows, and
//      U = Y W, O = G r + Z W run on the matrix cores; u is banked, o stored.
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16, fp32 accumulate): wave w owns state rows
// [32w, 32w+32); lane l holds rows 32w + 16nt + (l % 16) and columns 16mt + 4(l / 16) + e
// (nt < 2, mt < 8, e < 4), which are exactly the B operands of a 32-wide k-step kb when that
// step takes columns {32kb + 4(l/16) + e} and {32kb + 16 + 4(l/16) + e}; the A operands (rows of
// k and q, from LDS) use the same column order.  S0 is fp32 and enters as an exact sum of three
// bf16 terms (top, next and last 8 significant bits), k and q are bf16, so every product is
// exact and only the fp32 accumulation rounds.
#include <hip/hip_ext.h>

#include "mfma_common.h"
#include "ut_common.h"

namespace gdn {

constexpr int kUtD = 128;

// LDS regions for trees of at most n nodes, nrec records and nlv level entries, and at most nf
// pending rows.  Regions filled by direct loads are padded to whole 64-lane instructions.
struct UtLayout5 {
    static constexpr int D = kUtD;
    static constexpr int CPV = D * 2 / 16;  // 16-byte chunks per bf16 vector
    // A node's k | q | v take 3 CPV chunks plus one pad chunk: rows of consecutive nodes then
    // start 4 banks apart, so the 16 rows an MFMA operand read touches hit distinct banks.
    static constexpr int CPN = 3 * CPV + 1;
    static constexpr int NODE_BYTES = CPN * 16;
    static constexpr int WS = D + 4;        // row stride of W and GR in floats (same reason)
    static constexpr int CPR = D * 4 / 16;  // 16-byte chunks per fp32 fold row
    size_t in, bg, pd, work, fold_k, fold_u, gr, plan, tabs, total;
    size_t n64, lv64, rec64;
    __host__ __device__ UtLayout5(int n, int nrec, int nlv, int nf) {
        n64 = round_up(size_t(n), 64);
        lv64 = round_up(size_t(nlv), 64);
        rec64 = round_up(size_t(nrec), 64);
        in = 0;
        // node rows; after the S0 epilogue, the dense Y and Z rows of the u/o pass (round16(n)
        // rows of round4(n) floats each)
        const size_t rows = round_up(size_t(n) * CPN, 64) * 16;
        const size_t dense = 2 * round_up(size_t(n), 16) * round_up(size_t(n), 4) * 4;
        bg = in + (rows > dense ? rows : dense);  // beta | gate  [n64] x u32
        pd = bg + 2 * n64 * 4;                         // parent | depth [n64] int
        work = pd + 2 * n64 * 4;                       // W [n][WS] | GR [n][WS], after the fold
        const size_t fk = round_up(size_t(nf) * CPR, 64) * 16;
        fold_k = work;
        fold_u = work + fk;
        const size_t fold_bytes = 2 * fk;
        gr = work + size_t(n) * WS * 4;
        const size_t wg_bytes = size_t(2) * n * WS * 4;
        // plan (direct loads): poff [n64] | lvn [lv64] | recM [rec64]
        plan = work + (wg_bytes > fold_bytes ? wg_bytes : fold_bytes);
        tabs = plan + (n64 + lv64 + rec64) * 4;
        // gam[n] | kq[n] | recE=recY | recC | recQ | recZ [nrec] (f32) | recP | recT [nrec] (int)
        total = tabs + (size_t(2) * n + size_t(6) * nrec) * 4;
    }
};

// ------------------------------------------------------------------------------------------
// one workgroup of 4 waves per (layer, sequence, head)
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256, GDN_VERIFY_MIN_WAVES)
void verify_ut_mfma_kernel(VerifyParams P, const int32_t *__restrict__ plan,
                           const int32_t *__restrict__ rows, int n_max, int nrec_max, int nlv_max,
                           int nf_max) {
    constexpr int D = kUtD, THREADS = 256, NW = 4, JC = 4;
    using LY = UtLayout5;
    extern __shared__ __align__(16) float dyn[];
    char *lds = reinterpret_cast<char *>(dyn);
    const LY lay(n_max, nrec_max, nlv_max, nf_max);
    const size_t n64 = round_up(size_t(n_max), 64);
    const char *IN = lds + lay.in;
    const uint32_t *Bl = reinterpret_cast<const uint32_t *>(lds + lay.bg);
    const uint32_t *Gt = Bl + n64;
    const int *par = reinterpret_cast<const int *>(lds + lay.pd);
    const int *dep = par + n64;
    float *Wm = reinterpret_cast<float *>(lds + lay.work);  // w_n, overwritten by u_n
    float *GR = reinterpret_cast<float *>(lds + lay.gr);
    const float *FK = reinterpret_cast<const float *>(lds + lay.fold_k);
    const float *FU = reinterpret_cast<const float *>(lds + lay.fold_u);
    // Plan of this tree (from the schedule image): record q of node n is q = poff[n] for n
    // itself and poff[n] + 1 + t for its ancestor at distance t + 1; recM = that node.
    int *poff = reinterpret_cast<int *>(lds + lay.plan);
    int *lvn = poff + lay.n64;      // first node of each depth level, in (depth, id) order
    int *recM = lvn + lay.lv64;
    float *gam = reinterpret_cast<float *>(lds + lay.tabs);
    float *kq = gam + n_max;
    // recE = E(n, that node), later Y[n][that node]; recC = T[n][it], recQ = C[n][it], recZ = Z;
    // recP = block start of the record's node, recT = its distance - 1 (-1: the node itself)
    float *recE = kq + n_max, *recC = recE + nrec_max, *recQ = recC + nrec_max;
    float *recZ = recQ + nrec_max, *recY = recE;
    int *recP = reinterpret_cast<int *>(recZ + nrec_max), *recT = recP + nrec_max;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const UtUnit un = ut_unit(P);
    const int layer = P.layer_begin + un.layer_rel, seq = un.seq, h = un.h;
    // Image words are read through `plan` (a no-alias argument) and before any direct load, so
    // that they are scalar loads: a vector load here would make the wave wait for every direct
    // load issued before it.
    const int seq_off = plan[P.off_seq + seq];
    const int n = plan[P.off_seq + seq + 1] - seq_off;
    const int r0 = plan[P.off_ut_rec_base + seq], nrec = plan[P.off_ut_rec_base + seq + 1] - r0;
    const int l0 = plan[P.off_ut_lv_base + seq], nlv = plan[P.off_ut_lv_base + seq + 1] - l0;
    // dense Y and Z rows of the u/o pass, over the node rows once the epilogue is done
    const int ys = (n + 3) & ~3;
    float *Yd = reinterpret_cast<float *>(lds + lay.in);
    float *Zd = Yd + ((n + 15) & ~15) * ys;
    // pending counts come from the commit call, which bounds them by the bank rows; the clamp
    // keeps a corrupted count from reading past the bank.
    const int role = P.role[seq], L = min(max(P.pending[seq], 0), P.max_nodes);
    const int64_t sh = (int64_t(layer) * P.S + seq) * P.H + h;
    float *committed = P.state + sh * D * D;
    const int64_t row0_bank = sh * P.max_nodes;
    const int64_t node_row0 = (int64_t(layer) * P.T + seq_off) * P.H + h;  // node 0's row
    // Pending factor f sits in bank row rm[f] (the commit's row map; clamped to the bank).
    // Lane f < 64 requests its factor's row now and uses it after the first barrier (touching
    // it earlier would wait for the load); the index stays in the sequence's map for any L.
    const int32_t *rm = rows + int64_t(seq) * P.max_nodes;
    const int mrow = P.max_nodes - 1;
    const int rml_raw = rm[min(lane, max(L - 1, 0))];

    // ---- 0. direct loads: k, q, v, beta, g, parents, depths, pending fold rows ----------
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
        for (int base = w * 64; base < int(4 * n64); base += NW * 64) {
            if (n == 0) break;
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
        if (n > 0) {  // the tree's plan: node blocks, level lists, ancestor records
            const int32_t *srcs[3] = {P.img + P.off_ut_node_rec + seq_off,
                                      P.img + P.off_ut_lvn + l0, P.img + P.off_ut_rec_anc + r0};
            const int counts[3] = {n, nlv, nrec};
            int *dsts[3] = {poff, lvn, recM};
#pragma unroll
            for (int a = 0; a < 3; ++a)
                for (int base = w * 64; base < counts[a]; base += NW * 64)
                    to_lds<4>(srcs[a] + min(base + lane, counts[a] - 1), dsts[a] + base);
        }
        if (L > 0) {
            const float *pk = P.bank_k[role] + row0_bank * D, *pu = P.bank_u[role] + row0_bank * D;
            const int rows_chunks = L * LY::CPR;
            const int fk_chunks = int(round_up(size_t(nf_max) * LY::CPR, 64));
            static_assert(64 == 2 * LY::CPR, "one load instruction covers two fold rows");
            for (int base = w * 64; base < 2 * fk_chunks; base += NW * 64) {
                const int which = base / fk_chunks, b2 = base % fk_chunks;
                if (b2 >= rows_chunks) continue;
                const int c = min(b2 + lane, rows_chunks - 1);
                // the instruction's two factors and their bank rows (uniform: scalar loads)
                const int fa = b2 / LY::CPR, fb = min(fa + 1, L - 1);
                const int ra = min(max(rm[fa], 0), mrow), rb = min(max(rm[fb], 0), mrow);
                const float *src = (which == 0 ? pk : pu) +
                                   int64_t(c / LY::CPR == fa ? ra : rb) * D + (c % LY::CPR) * 4;
                to_lds<16>(src, lds + lay.fold_k + size_t(base) * 16);
            }
        }
    }
    __syncthreads();  // waits for every direct load (the barrier's fence covers them)

    // ln g of pending factor `lane` (lanes < L), for the fold; requested before the tile so
    // that waiting for the tile covers it
    const float *plg = P.bank_lg[role] + row0_bank;
    float lgr = 0.f;
    if (lane < L) lgr = plg[min(max(rml_raw, 0), mrow)];

    // ---- 1. gate products along every record block ------------------------------------
    //   E(n, anc_0) = g_n, E(n, anc_{t+1}) = E(n, anc_t) g_{anc_t}, G_n = E(n, root) g_root,
    // in groups of four records whose reads are independent; recP and recT on the way.
    for (int t = tid; t < n; t += THREADS) {
        const int o = poff[t], dt = dep[t];
        float E = slot_f32<bf16_t>(Gt[t]);
        recT[o] = -1;
        for (int s0 = 0; s0 < dt; s0 += 4) {
            int a[4], pa[4];
            float ga[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) a[j] = s0 + j < dt ? recM[o + 1 + s0 + j] : t;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pa[j] = poff[a[j]];
                ga[j] = slot_f32<bf16_t>(Gt[a[j]]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (s0 + j >= dt) break;
                const int q = o + 1 + s0 + j;
                recE[q] = E;
                recP[q] = pa[j];
                recT[q] = s0 + j;
                E *= ga[j];
            }
        }
        gam[t] = E;
    }
    __syncthreads();
    {  // banked keys (exact fp32 widening) and log-gates: stores only, issued early
        float *wk = P.bank_k[role ^ 1], *wlg = P.bank_lg[role ^ 1];
        for (int e = tid; e < n * (D / 4); e += THREADS) {
            const int nd = e / (D / 4), c = (e % (D / 4)) * 4;
            const uint2 x =
                *reinterpret_cast<const uint2 *>(IN + size_t(nd) * LY::NODE_BYTES + c * 2);
            *reinterpret_cast<float4 *>(wk + (row0_bank + nd) * D + c) =
                make_float4(bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y));
        }
        for (int t = tid; t < n; t += THREADS)
            wlg[row0_bank + t] = logf(slot_f32<bf16_t>(Gt[t]));
    }

    // The state tile is requested now, behind the bank stores; its latency hides behind the
    // pair phase, which needs only LDS.  Requested before the gate products, the first round's
    // tile loads went out ahead of the bank stores and lengthened the launch by ~1.7 us.
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

    // ---- 2. pair coefficients: [k; q] K^T on the matrix cores ---------------------------
    // M tile jt interleaves k and q of nodes 8jt .. 8jt+7 (row 2j + 0/1 = k/q of node 8jt + j);
    // N tile at holds the keys of nodes 16at .. 16at+15.  Lane (lr, lg) receives rows 4lg + r:
    // of node 8jt + 2lg + r/2, k . k_a for even r and q . k_a for odd r, with a = 16at + lr.
    // Nodes past the tree are clamped to its last; their products are never used.
    // A key a pairs with node n only if a <= n (an ancestor, or n itself), so M tile jt (nodes
    // up to 8jt + 7) needs the key tiles at <= jt / 2 only: (jt / 2) + 1 tiles per M tile.
    const int JT = (n + 7) >> 3;
    int n_tiles = 0;
    for (int j = 0; j < JT; ++j) n_tiles += (j >> 1) + 1;
    for (int ti = w; ti < n_tiles; ti += NW) {
        int jt = 0, at = ti;
        while (at > (jt >> 1)) at -= (jt++ >> 1) + 1;
        const int xn = min(8 * jt + (lr >> 1), n - 1), kn = min(16 * at + lr, n - 1);
        const char *xrow = IN + size_t(xn) * LY::NODE_BYTES + (lr & 1) * D * 2;
        const char *krow = IN + size_t(kn) * LY::NODE_BYTES;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row_operand(xrow, 32 * kb + 4 * lg),
                                                         row_operand(krow, 32 * kb + 4 * lg), acc,
                                                         0, 0, 0);
        const int an = 16 * at + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int nd = 8 * jt + 2 * lg + (r >> 1);
            const bool is_q = r & 1;
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

    // ---- 3. deferred commit: fold the pending rows, write the committed state once --------
    // S_L = G S0 + sum_f c_f u_f k_f^T with G the product of the L pending gates (exp of the sum
    // of their logs) and c_f that of the gates after row f: the tile is scaled once, then each
    // row costs one FMA per element.
    // Rows run last to first so that c builds up backward (c_{L-1} = 1, c_{f-1} = c_f g_f).
    if (L > 0) {
        float lg_part = lgr;  // this lane's share of the pending log gates
        for (int f = 64 + lane; f < L; f += 64) lg_part += plg[min(max(rm[f], 0), mrow)];
        const float G = expf(wave_total(lg_part));
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[0][mt][e] *= G;
                s[1][mt][e] *= G;
            }
        float c = 1.f;
        for (int f = L - 1; f >= 0; --f) {
            const float u0 = c * FU[f * D + 32 * w + lr], u1 = c * FU[f * D + 32 * w + 16 + lr];
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                const float4 k4 = *reinterpret_cast<const float4 *>(FK + f * D + 16 * mt + 4 * lg);
                const float kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    s[0][mt][e] = fmaf(u0, kk[e], s[0][mt][e]);
                    s[1][mt][e] = fmaf(u1, kk[e], s[1][mt][e]);
                }
            }
            c *= expf(f < 64 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lgr), f))
                             : plg[min(max(rm[f], 0), mrow)]);
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
    __syncthreads();  // fold rows are dead: their LDS becomes W and GR; pair terms are done


    // ---- 4. p_n = S0 k_n, r_n = S0 q_n on the matrix cores; w_n and G_n r_n to LDS -------
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
                // k (even lr) or q (odd lr) of node 8jt + lr/2, clamped to the tree's last node
                const int xn = min(8 * jt + (lr >> 1), n - 1);
                const bf16x8 a =
                    row_operand(IN + size_t(xn) * LY::NODE_BYTES + (lr & 1) * D * 2, 32 * kb + 4 * lg);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    acc[jc][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl[nt], acc[jc][nt], 0, 0, 0);
                    acc[jc][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bm[nt], acc[jc][nt], 0, 0, 0);
                    acc[jc][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh[nt], acc[jc][nt], 0, 0, 0);
                }
            }
        }
        // Lane (lr, lg) holds rows 4lg + r of each M tile: p (even r) and r (odd r) of node
        // 8jt + 2lg + r/2 at state row 32w + 16nt + lr.
#pragma unroll
        for (int jc = 0; jc < JC; ++jc) {
            const int jt = jt0 + jc;
            if (jt >= JT) break;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int nd = 8 * jt + 2 * lg + j;
                if (nd >= n) continue;
                const float G = gam[nd], beta = slot_f32<bf16_t>(Bl[nd]);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int i = 32 * w + 16 * nt + lr;
                    const float v = bf16_at(IN + size_t(nd) * LY::NODE_BYTES + 2 * D * 2, i);
                    Wm[nd * LY::WS + i] = beta * fmaf(-G, acc[jc][nt][2 * j], v);
                    GR[nd * LY::WS + i] = G * acc[jc][nt][2 * j + 1];
                }
            }
        }
    }
    __syncthreads();

    // ---- 5. u_n = sum_a Y[n][a] w_a, o_n = G_n r_n + sum_a Z[n][a] w_a, every (node, row) ---
    // Y = T^-1 and Z = C' Y as dense rows over the consumed node rows (wave 0; one lane per node
    // up to depth 16)
    tree_inverse(n, n > 0 ? plan[P.off_ut_lv_base + seq + 1] - plan[P.off_ut_lv_base + seq] - 2 : 0,
                 lane, w, poff, dep, lvn, recM, recP, recT, recC, recQ, kq, recY, recZ, Yd, Zd, ys);
    __syncthreads();
    tree_apply_mfma(n, ys, w, lane, Yd, Zd, Wm, GR, LY::WS, P.bank_u[role ^ 1] + row0_bank * D,
                    P.out + node_row0 * D, int64_t(P.H) * D);
}

gdn_status launch_ut_mfma(const VerifyParams &P, int n_max, int nrec_max, int nlv_max,
                          int nf_max, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const size_t lds = UtLayout5(n_max, nrec_max, nlv_max, nf_max).total;
    if (lds > kUtMaxLdsBytes)
        return fail(GDN_EINVAL, "gdn_tree_verify_ut: trees of %d nodes with %d records "
                    "and %d bank rows need %zu bytes of LDS (limit %zu); use gdn_tree_verify",
                    n_max, nrec_max, nf_max, lds, kUtMaxLdsBytes);
    if (P.n_blocks <= 0) return GDN_OK;
    const dim3 grid(uint32_t(P.n_blocks));
    if (start == nullptr && stop == nullptr)
        hipLaunchKernelGGL(verify_ut_mfma_kernel, grid, dim3(256), lds, stream, P, P.img, P.rows,
                           n_max, nrec_max, nlv_max, nf_max);
    else
        hipExtLaunchKernelGGL(verify_ut_mfma_kernel, grid, dim3(256), uint32_t(lds), stream,
                              start, stop, 0, P, P.img, P.rows, n_max, nrec_max, nlv_max, nf_max);
    GDN_LAUNCH_CHECK("verify_ut_mfma_kernel");
    return GDN_OK;
}

}  // namespace gdn
