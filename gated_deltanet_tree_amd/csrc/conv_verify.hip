// Fused tree conv -> SiLU -> unit length prologue feeding the tree-masked verify, on the matrix
// cores (gfx950, bf16 inputs, d = 128).
//
// Pages: "Luce DFlash server README", section "How it works": in tree verify each node's conv
// window is gathered along its parent chain, and the conv feeds the recurrent layer.  "Lucebox
// SpecLA and Gated DeltaNet state-resident verification" guide: mechanism 1 (the conv window
// gets the state-resident treatment; the topology-mask form of the verify), mechanism 3 (the
// conv raw input is banked beside the key, the residual vector and the log gate), mechanism 4
// (pending factors and pending conv inputs are folded into the committed state and window
// before the verify).  The pages do not write out how the conv output becomes q, k and v; this
// kernel takes the plain reading of a hybrid GDN layer: the conv runs over 3 H d channels laid
// out [q heads | k heads | v heads], every conv output goes through SiLU (y / (1 + e^-y)), q and
// k are divided by their Euclidean length (floored at 1e-6) and v is used as it comes.
//
// With S0 the committed state after the fold, G_n the product of the gates on n's root path and
// E(n,a) the product of the gates strictly below a down to n, the verify is the tree-masked form
//   T[n][a] = beta_n E(n,a) (k_n . k_a)  (a a strict ancestor; T[n][n] = 1),
//   w_n = beta_n (v_n - G_n S0 k_n),   T u = w,
//   o_n = G_n S0 q_n + sum_{a in A(n)} C'[n][a] u_a,  C'[n][a] = E(n,a) (q_n . k_a), C'[n][n] = q_n . k_n.
// The system is not solved level by level here: one wave forms Y = T^-1 and Z = C' Y as dense
// rows, after which every (node, state row) is independent and all of them are two small
// matrix products:
//   u_n = sum_{a in A(n)} Y[n][a] w_a,   o_n = G_n S0 q_n + sum_{a in A(n)} Z[n][a] w_a.
//
// One workgroup of 8 waves per (layer, sequence, head):
//   0. direct loads of beta, g, parents, depths and the tree's plan; the committed conv
//      windows and the q/k conv weights to registers;
//   1. direct loads of the head's q, k and v conv-input rows of every node, landing while each
//      of the head's 3 x 128 channels folds its conv window, keeps it in LDS and writes it
//      back, and per record the ancestor offsets, distances and gate products are formed;
//   2. the first chunk of pending fold rows is requested into registers; raw conv inputs
//      banked; prologue: per node, conv of the q and k channels along the parent chain, SiLU,
//      unit length; fp32 rows to LDS, keys to the write bank;
//   3. the state tile loads are issued (they land during this phase); pair products [k; q] K^T
//      on the matrix cores; the fold rows go to LDS over the consumed q and k conv-input
//      planes;
//   4. the pending rows are folded into the tile on the matrix cores and the committed state is
//      written back once; [k; q] S0^T on the matrix cores; the epilogue evaluates the v channels
//      (conv and SiLU) and writes w_n and G_n S0 q_n; wave 0 forms Y and Z as dense rows;
//   5. U = Y W and O = G r + Z W on the matrix cores; u banked, o stored.
// Matrix-core layout: wave w owns state rows [16w, 16w+16), lane l holds row 16w + (l % 16) and
// columns 16mt + 4(l/16) + e.  q and k are fp32 here, so the products run on the fp32 matrix
// cores (v_mfma_f32_16x16x4f32): for the 4-column step {16mt + 4(l/16) + e}, lane l already holds
// the state element it contributes as B, and one float4 LDS read per mt gives its A elements for
// the four steps e = 0..3.  Accumulation is fp32, as in a vector dot product.
#include <hip/hip_ext.h>

#include "mfma_common.h"
#include "ut_common.h"

namespace gdn {

namespace {

constexpr int kCvD = 128;
constexpr int kCvThreads = 512;  // 8 waves; wave w owns state rows [16w, 16w + 16)
constexpr int kCvWaves = kCvThreads / 64;
constexpr float kNormFloor = 1e-6f;
constexpr int kFoldRows = 2 * kCvThreads / 64;  // pending rows per stage: 2 chunks per thread, 64 per row

struct ConvVerifyParams {
    VerifyParams V;
    const bf16_t *x;     // [Ly][T][C] conv inputs
    const bf16_t *w;     // [Ly][C][4] conv weights, tap 3 multiplies the node's own input
    float *cstate;       // [Ly][S][C][3] committed conv window, oldest first
    bf16_t *bank_x[2];   // [Ly][S][max_nodes][C] conv-input banks (the raw bf16 inputs)
    int32_t C;           // 3 H d
};

// LDS regions for trees of at most n nodes, nrec records and nlv level entries, with nfc pending
// rows folded per chunk.
//   X:  the bf16 conv-input planes [v | q | k] (n rows of 256 bytes each); once the q and k rows
//       are consumed, the pending fold rows (k | u | c) take their place, and after the fold the
//       dense Y and Z rows; the v plane lives until the S0 epilogue.
//   KQ: the fp32 k and q rows (k_n at row 2n, q_n at 2n + 1, stride KS); each pass of S0
//       products consumes the rows of its nodes, after which w_n takes row 2n and G_n S0 q_n
//       row 2n + 1.
struct CvLayout {
    static constexpr int D = kCvD;
    static constexpr int XROW = D * 2;      // bytes of one bf16 conv-input row of one block
    static constexpr int KS = D + 4;        // fp32 row stride (floats): 16 rows hit distinct banks
    static constexpr int CPR = D * 4 / 16;  // 16-byte chunks per fp32 fold row
    size_t xv, xq, kq, fold_k, fold_u, fold_c, bg, pd, plan, tabs, x0s, wv, total;
    size_t n64, lv64, rec64;

    __host__ __device__ static size_t fold_chunks(int r) { return round_up(size_t(r) * CPR, 64); }
    __host__ __device__ static size_t fold_bytes(int r) {
        return 2 * fold_chunks(r) * 16 + round_up(size_t(r), 64) * 4;
    }
    // direct-load footprint of the three conv-input planes
    __host__ __device__ static size_t xin_bytes(int n) { return round_up(size_t(48) * n, 64) * 16; }
    __host__ __device__ static size_t rows_bytes(int rows) { return size_t(rows) * KS * 4; }
    // dense Y and Z rows of the u/o pass: round16(n) rows of round4(n) floats each
    __host__ __device__ static size_t dense_bytes(int n) {
        return 2 * round_up(size_t(n), 16) * round_up(size_t(n), 4) * 4;
    }
    // room after the v plane: the q and k planes (with the direct-load padding), at least
    // min(nf, 4) fold rows and the dense Y and Z rows
    __host__ __device__ static size_t fold_room(int n, int nf) {
        const size_t a = xin_bytes(n) - size_t(n) * XROW, b = fold_bytes(nf < 4 ? nf : 4);
        const size_t c = dense_bytes(n), ab = a > b ? a : b;
        return ab > c ? ab : c;
    }
    // Pending rows per fold chunk: as many as the room holds.
    static int fold_rows(int n, int nf) {
        const size_t room = fold_room(n, nf);
        int r = 1;
        while (r < nf && fold_bytes(r + 1) <= room) ++r;
        return r;
    }

    __host__ __device__ CvLayout(int n, int nrec, int nlv, int nf, int nfc) {
        n64 = round_up(size_t(n), 64);
        lv64 = round_up(size_t(nlv), 64);
        rec64 = round_up(size_t(nrec), 64);
        xv = 0;
        xq = size_t(n) * XROW;
        fold_k = xq;
        fold_u = xq + fold_chunks(nfc) * 16;
        fold_c = fold_u + fold_chunks(nfc) * 16;
        kq = round_up(xq + fold_room(n, nf), 16);
        size_t p = kq + rows_bytes(2 * n);
        bg = p;                   // beta | gate [n64] u32 slots
        p += 2 * n64 * 4;
        pd = p;                   // parent | depth [n64] int (global parent ids)
        p += 2 * n64 * 4;
        plan = p;                 // poff [n64] | lvn [lv64] | recM [rec64]
        p += (n64 + lv64 + rec64) * 4;
        tabs = p;                 // gam | kqd [n] | recE=recY | recC | recQ | recZ [nrec] (f32),
                                  // recP | recT [nrec], anc [n][4] (int)
        p += (size_t(2) * n + size_t(6) * nrec + size_t(4) * n) * 4;
        x0s = round_up(p, 16);    // folded conv window [3 taps][3 D channels]
        wv = x0s + size_t(3) * 3 * D * 4;  // v-block conv weights [D channels][4 taps], bf16
        total = wv + size_t(D) * 4 * 2;
    }
};

// Inclusive suffix sum over lanes 0-15 (lane l gets the sum of lanes l .. 15); other lanes get
// partial sums that are not used.
__device__ __forceinline__ float chunk_suffix_sum(float x) {
    const int lane = int(__lane_id());
#pragma unroll
    for (int d = 1; d < 16; d *= 2) {
        const float y = __shfl_down(x, d);
        x += lane + d < 16 ? y : 0.f;
    }
    return x;
}

// Pending rows f0 .. f0 + cnt - 1 (cnt <= kFoldRows) go through registers into LDS: 16-byte chunk
// c of thread t is c = t + 512 j (j < 2), row c / 64, key half (c % 64 < 32) or residual half;
// the row is uniform over a wave (w + 8 j), its bank row comes from the pending row map.
// With the rows, wave 0 stages each row's fold coefficient c_f = exp(sum of the log gates of the
// pending rows after f): an exclusive suffix scan over the chunk (lane f sums the log gates of
// lanes f + 1 .. 15, never its own, so a zero gate's -inf is only ever added, and c_f = 0 for
// every row before it) plus fold_carry, the sum over the chunks already staged (they hold later
// rows).  Register loads rather than direct-to-LDS loads: an LDS read after a direct load waits
// for every older memory operation of the wave.  Two named registers (no array), so nothing of
// it goes to scratch.
__device__ __forceinline__ uint4 fold_chunk_load(const float *pk, const float *pu, int row,
                                                 int lane) {
    const int half = (lane >> 5) & 1, idx = lane & 31;
    return *reinterpret_cast<const uint4 *>((half ? pu : pk) + row * kCvD + idx * 4);
}
__device__ __forceinline__ void fold_chunk_store(float *fk, float *fu, int cnt, int c, uint4 v) {
    if (c < 64 * cnt) {
        const int r = c >> 6, half = (c >> 5) & 1, idx = c & 31;
        *reinterpret_cast<uint4 *>((half ? fu : fk) + r * kCvD + idx * 4) = v;
    }
}
#define GDN_FOLD_LOAD(f0, cnt)                                                          \
    do {                                                                                \
        const int lc_ = (cnt) - 1;                                                      \
        fv0 = fold_chunk_load(pend_k, pend_u, pend_row((f0) + min(w, lc_)), lane);      \
        fv1 = fold_chunk_load(pend_k, pend_u, pend_row((f0) + min(w + 8, lc_)), lane);  \
        const int fl_ = (f0) + min(lane, lc_), rl_ = __shfl(rml, min(fl_, 63));         \
        flv = pend_lg[fl_ < 64 ? rl_ : min(max(rm[fl_], 0), mrow)];                     \
    } while (0)
#define GDN_FOLD_STORE(cnt)                                                             \
    do {                                                                                \
        fold_chunk_store(fold_k, fold_u, (cnt), tid, fv0);                              \
        fold_chunk_store(fold_k, fold_u, (cnt), tid + 512, fv1);                        \
        if (w == 0) {                                                                   \
            const float v_ = lane < (cnt) ? flv : 0.f;                                  \
            const float n_ = __shfl_down(v_, 1);                                        \
            const float x_ = chunk_suffix_sum(lane + 1 < 16 ? n_ : 0.f);                \
            if (lane < (cnt)) fold_c[lane] = expf(fold_carry + x_);                     \
            fold_carry += __shfl(x_ + v_, 0);                                           \
        }                                                                               \
    } while (0)

// SiLU, y / (1 + e^-y), with the hardware exp and reciprocal (each within about an ulp).
__device__ __forceinline__ float silu(float y) {
    return y * __builtin_amdgcn_rcpf(1.f + __expf(-y));
}

// conv of one channel at a node: taps up the parent chain, committed-window entries above the
// root (c0 oldest); weight tap 3 multiplies the node's own input.
__device__ __forceinline__ float conv4(const float wt[4], float x0, float x1, float x2, float x3,
                                       int dt, float c0, float c1, float c2) {
    const float a1 = dt >= 1 ? x1 : c2;
    const float a2 = dt >= 2 ? x2 : (dt == 1 ? c2 : c1);
    const float a3 = dt >= 3 ? x3 : (dt == 2 ? c2 : (dt == 1 ? c1 : c0));
    return fmaf(wt[3], x0, fmaf(wt[2], a1, fmaf(wt[1], a2, wt[0] * a3)));
}

}  // namespace

// DEEP = false, trees of depth <= 12: 6 waves per SIMD, three workgroups of 8 waves per CU (the
// LDS allows three for trees like the batched workload's), which needs at most 80 VGPRs per
// lane; the per-lane inverse runs up to depth 12.  DEEP = true, a tree deeper than 12 in the
// batch: 4 waves per SIMD (128 VGPRs), room for the per-lane inverse up to depth 16.  Trees that
// deep mostly need more LDS than three workgroups per CU leave, so occupancy is not what they
// give up; past depth 16 both forms solve level by level.
template <bool DEEP>
__global__ __launch_bounds__(kCvThreads, DEEP ? 4 : 6)
void conv_verify_kernel(ConvVerifyParams CP, const int32_t *__restrict__ plan,
                        const int32_t *__restrict__ rows, int n_max, int nrec_max, int nlv_max,
                        int nf, int nfc) {
    constexpr int D = kCvD, THREADS = kCvThreads, NW = kCvWaves, JC = 3;
    using LY = CvLayout;
    const VerifyParams &P = CP.V;
    extern __shared__ __align__(16) float dyn[];
    char *lds = reinterpret_cast<char *>(dyn);
    const LY lay(n_max, nrec_max, nlv_max, nf, nfc);
    const size_t n64 = lay.n64;
    const uint32_t *Bl = reinterpret_cast<const uint32_t *>(lds + lay.bg);
    const uint32_t *Gt = Bl + n64;
    const int *par = reinterpret_cast<const int *>(lds + lay.pd);
    const int *dep = par + n64;
    float *KQ = reinterpret_cast<float *>(lds + lay.kq);
    float *Wm = KQ, *GR = KQ + LY::KS;  // row n at 2 n KS: over k_n and q_n once consumed
    constexpr int WS = 2 * LY::KS;      // row stride of W and GR
    const float *FK = reinterpret_cast<const float *>(lds + lay.fold_k);
    const float *FU = reinterpret_cast<const float *>(lds + lay.fold_u);
    const float *FC = reinterpret_cast<const float *>(lds + lay.fold_c);
    // Plan of this tree (from the schedule image): record poff[n] is n itself, poff[n] + d its
    // ancestor at distance d; recM = that node.
    int *poff = reinterpret_cast<int *>(lds + lay.plan);
    int *lvn = poff + n64;      // first node of each depth level, in (depth, id) order
    int *recM = lvn + lay.lv64;
    float *gam = reinterpret_cast<float *>(lds + lay.tabs);
    float *kqd = gam + n_max;
    // recE = E(n, that node), later Y[n][that node]; recC = T, recQ = C', recZ = Z on the
    // ancestor records; recP = poff of the record's node, recT = its distance - 1 (-1: itself)
    float *recE = kqd + n_max, *recC = recE + nrec_max, *recQ = recC + nrec_max;
    float *recZ = recQ + nrec_max;
    int *recP = reinterpret_cast<int *>(recZ + nrec_max);
    int *recT = recP + nrec_max;
    int4 *anc = reinterpret_cast<int4 *>(recT + nrec_max);  // 3 nearest ancestors (local ids)
    float *recY = recE;
    float *X0s = reinterpret_cast<float *>(lds + lay.x0s);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int row0 = 16 * w;  // this wave's first state row
    const UtUnit un = ut_unit(P);
    const int layer = P.layer_begin + un.layer_rel, seq = un.seq, h = un.h;
    // Image words are read through `plan` (a no-alias argument) and before any direct load, so
    // that they are scalar loads: a vector load here would make the wave wait for every direct
    // load issued before it.
    const int seq_off = plan[P.off_seq + seq];
    const int n = plan[P.off_seq + seq + 1] - seq_off;
    const int r0 = plan[P.off_ut_rec_base + seq], nrec = plan[P.off_ut_rec_base + seq + 1] - r0;
    const int l0 = plan[P.off_ut_lv_base + seq], nlv = plan[P.off_ut_lv_base + seq + 1] - l0;
    // dense Y and Z rows of the u/o pass, over the fold rows once the fold is done
    const int ys = (n + 3) & ~3;
    float *Yd = reinterpret_cast<float *>(lds + lay.xq);
    float *Zd = Yd + ((n + 15) & ~15) * ys;
    // pending counts come from the commit call, which bounds them by the bank rows; the clamp
    // keeps a corrupted count from reading past the banks.
    const int role = P.role[seq], L = min(max(P.pending[seq], 0), P.max_nodes);
    const int64_t sh = (int64_t(layer) * P.S + seq) * P.H + h;
    const int64_t ls = int64_t(layer) * P.S + seq;
    float *committed = P.state + sh * D * D;
    const int64_t row0_bank = sh * P.max_nodes;
    const int64_t node_row0 = (int64_t(layer) * P.T + seq_off) * P.H + h;  // node 0's (beta, g, o) row
    const int C = CP.C, HD = P.H * D;
    // node 0's conv inputs, q block of head h; block b adds b H d
    const bf16_t *xrow0 = CP.x + (int64_t(layer) * P.T + seq_off) * C + h * D;

    const float *pend_k = P.bank_k[role] + row0_bank * D, *pend_u = P.bank_u[role] + row0_bank * D;
    const float *pend_lg = P.bank_lg[role] + row0_bank;
    // Pending factor f sits in bank row rm[f] (the commit's row map; clamped to the bank).  Lane
    // f < 64 requests the row of factor f now and uses it after the first barrier (touching it
    // earlier would wait for the load); the three rows of the conv window's inputs are uniform,
    // scalar loads.  Indices stay in the sequence's map for any L.
    const int32_t *rm = rows + int64_t(seq) * P.max_nodes;
    const int mrow = P.max_nodes - 1;
    const int rml_raw = rm[min(lane, max(L - 1, 0))];
    int wrow[3];
#pragma unroll
    for (int e = 0; e < 3; ++e) wrow[e] = rm[max(L - 3 + e, 0)];
    int rml = 0;  // set after the first barrier
    // bank row of pending factor f, f uniform
    auto pend_row = [&](int f) {
        return f < 64 ? __builtin_amdgcn_readlane(rml, f) : min(max(rm[f], 0), mrow);
    };
    float *fold_k = reinterpret_cast<float *>(lds + lay.fold_k);
    float *fold_u = reinterpret_cast<float *>(lds + lay.fold_u);
    float *fold_c = reinterpret_cast<float *>(lds + lay.fold_c);
    uint4 fv0, fv1;
    float flv, fold_carry = 0.f;

    // ---- 0. loads ------------------------------------------------------------------------
    {
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
        if (w == NW - 1)  // the v block's conv weights: 128 channels x 4 taps, one load per lane
            to_lds<16>(CP.w + (int64_t(layer) * C + 2 * HD + h * D + 2 * lane) * 4,
                       lds + lay.wv);
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
    }
    // committed conv window (thread 128 + cc owns channel cc of the head's 3 x 128) with its
    // last pending inputs; the conv weights of the block this wave's prologue evaluates (waves
    // of even index the q block, odd the k block), two channels per lane
    const int chan = tid - (THREADS - 3 * D);  // waves 2-7 own the channels, waves 0-1 the tables
    const bool has_ch = chan >= 0;
    float win[3], pend[3];
    {
        const int ccl = has_ch ? chan : 0;  // threads without a channel re-read channel 0
        const int64_t ch = int64_t(ccl >> 7) * HD + h * D + (ccl & (D - 1));
        const float *cs = CP.cstate + (ls * C + ch) * 3;
        const bf16_t *pb = CP.bank_x[role] + ls * P.max_nodes * C + ch;
#pragma unroll
        for (int e = 0; e < 3; ++e) {
            win[e] = cs[e];
            // pending input L - 3 + e, when it exists
            pend[e] = L >= 3 - e ? to_f32(pb[int64_t(min(max(wrow[e], 0), mrow)) * C]) : 0.f;
        }
    }
    const int qk_blk = w & 1;  // 0: q, 1: k
    const uint4 wraw = *reinterpret_cast<const uint4 *>(
        CP.w + (int64_t(layer) * C + qk_blk * HD + h * D + 2 * lane) * 4);
    __syncthreads();  // waits for every direct load (the barrier's fence covers them)

    // this lane's share of the pending log gates (factor `lane`, then every 64th): their sum
    // gives the fold's gate product; requested ahead of the tile, so waiting for the tile
    // covers them
    rml = min(max(rml_raw, 0), mrow);
    float lg_part = lane < L ? pend_lg[rml] : 0.f;
    for (int f = 64 + lane; f < L; f += 64) lg_part += pend_lg[min(max(rm[f], 0), mrow)];

    // ---- 1. conv-input planes requested; conv-window fold; record tables -----------------
    // The planes are requested here rather than with the tables: they land while the windows
    // and records are formed (the barrier at the end of the phase waits for them).
    {
        // Waves 1-7 only: wave 0 walks the records next, and the compiler makes a wave wait
        // for its own outstanding direct loads before the walk's 16-byte ancestor writes.
        const int total = 48 * n;  // planes v | q | k, 16 chunks per node row
        for (int base = (w - 1) * 64; w > 0 && base < total; base += (NW - 1) * 64) {
            const int c = min(base + lane, total - 1);  // padding lanes re-read the last chunk
            const int p = c / (16 * n), r = c - p * 16 * n, node = r >> 4, idx = r & 15;
            const int blk = p == 0 ? 2 : p - 1;
            const char *src = reinterpret_cast<const char *>(xrow0 + int64_t(node) * C +
                                                             blk * HD) + idx * 16;
            to_lds<16>(src, lds + lay.xv + size_t(base) * 16);
        }
    }
    // conv window: only the last three pending inputs survive
    if (has_ch) {
        const int cc = chan;
        float w0 = win[0], w1 = win[1], w2 = win[2];
        if (L >= 3) {
            w0 = pend[0]; w1 = pend[1]; w2 = pend[2];
        } else if (L == 2) {
            w0 = w2; w1 = pend[1]; w2 = pend[2];
        } else if (L == 1) {
            w0 = w1; w1 = w2; w2 = pend[2];
        }
        X0s[cc] = w0;
        X0s[3 * D + cc] = w1;
        X0s[6 * D + cc] = w2;
        if (L > 0) {
            float *cs = CP.cstate + (ls * C + int64_t(cc >> 7) * HD + h * D + (cc & (D - 1))) * 3;
            cs[0] = w0;
            cs[1] = w1;
            cs[2] = w2;
        }
    }
    // Per node t: along its record block, in groups of four records whose reads are independent,
    //   E(t, anc_0) = g_t, E(t, anc_{s+1}) = E(t, anc_s) g_{anc_s}, G_t = E(t, root) g_root;
    // recP = the block start of each ancestor, recT its distance - 1; anc = 3 nearest ancestors.
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
            if (s0 == 0) anc[t] = make_int4(a[0], a[1], a[2], 0);
        }
        if (dt == 0) anc[t] = make_int4(t, t, t, 0);
        gam[t] = E;
        P.bank_lg[role ^ 1][row0_bank + t] = logf(slot_f32<bf16_t>(Gt[t]));
    }
    __syncthreads();  // planes, windows, records and ancestors in LDS
    // the first fold chunk's rows: waited for after the pair products
    if (L > 0) GDN_FOLD_LOAD(L - min(L, nfc), min(L, nfc));
    // raw conv inputs to the write bank, from the planes (stores only, ahead of the prologue)
    {
        bf16_t *bx = CP.bank_x[role ^ 1] + ls * P.max_nodes * C + h * D;
        for (int e = tid; e < n * 3 * (D / 8); e += THREADS) {  // (node, block, 8 channels)
            const int nd = e / (3 * (D / 8)), r = e % (3 * (D / 8));
            const int p = r / (D / 8), c = (r % (D / 8)) * 8;  // plane v | q | k
            const int blk = p == 0 ? 2 : p - 1;
            *reinterpret_cast<uint4 *>(bx + int64_t(nd) * C + blk * HD + c) =
                *reinterpret_cast<const uint4 *>(lds + lay.xv + (size_t(p) * n + nd) * LY::XROW +
                                                 c * 2);
        }
    }

    // ---- 2. prologue: q and k from the conv ----------------------------------------------
    // Wave w evaluates block qk_blk (q or k) of nodes w/2, w/2 + NW/2, ...; a lane owns two
    // adjacent channels: conv along the parent chain, SiLU, a wave sum of squares, unit length.
    {
        const char *XB = lds + lay.xv + size_t(1 + qk_blk) * n * LY::XROW;  // plane q or k
        float wt[2][4], cw[2][3];
        const uint32_t r4[4] = {wraw.x, wraw.y, wraw.z, wraw.w};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            wt[e][0] = bf16_lo(r4[2 * e]);
            wt[e][1] = bf16_hi(r4[2 * e]);
            wt[e][2] = bf16_lo(r4[2 * e + 1]);
            wt[e][3] = bf16_hi(r4[2 * e + 1]);
#pragma unroll
            for (int j = 0; j < 3; ++j) cw[e][j] = X0s[j * 3 * D + qk_blk * D + 2 * lane + e];
        }
        // k_n at KQ row 2n, q_n at 2n + 1
        float *dst0 = KQ + size_t(1 - qk_blk) * LY::KS + 2 * lane;
        for (int nd = w >> 1; nd < n; nd += NW / 2) {
            const int dt = dep[nd];
            const int4 an = anc[nd];
            const int rws[4] = {nd, an.x, an.y, an.z};
            uint32_t xw[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                xw[t] = *reinterpret_cast<const uint32_t *>(XB + size_t(rws[t]) * LY::XROW + 4 * lane);
            float y[2], ss = 0.f;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float x0 = e ? bf16_hi(xw[0]) : bf16_lo(xw[0]);
                const float x1 = e ? bf16_hi(xw[1]) : bf16_lo(xw[1]);
                const float x2 = e ? bf16_hi(xw[2]) : bf16_lo(xw[2]);
                const float x3 = e ? bf16_hi(xw[3]) : bf16_lo(xw[3]);
                y[e] = silu(conv4(wt[e], x0, x1, x2, x3, dt, cw[e][0], cw[e][1], cw[e][2]));
                ss = fmaf(y[e], y[e], ss);
            }
            // 1 / max(|y|, floor) as rsqrt(max(|y|^2, floor^2))
            const float iv = __builtin_amdgcn_rsqf(fmaxf(wave_total(ss), kNormFloor * kNormFloor));
            *reinterpret_cast<float2 *>(dst0 + size_t(2 * nd) * LY::KS) =
                make_float2(y[0] * iv, y[1] * iv);
            if (qk_blk)  // keys to the write bank too, from the registers (no LDS round trip)
                *reinterpret_cast<float2 *>(P.bank_k[role ^ 1] + (row0_bank + nd) * D +
                                            2 * lane) = make_float2(y[0] * iv, y[1] * iv);
        }
    }
    __syncthreads();  // k and q rows complete; the q and k conv-input planes are consumed
    // The state tile, requested only now: issued in phase 1 with the other inputs, the first
    // round's 768 x 64 KB of tile loads queued ahead of the prologue's work and lengthened the
    // launch by ~2.5 us; here they land during the pair products.
    float s[8][4];  // row 16w + lr, columns 16mt + 4lg + e
    {
        const float *tile = committed + (row0 + lr) * D + 4 * lg;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const float4 x = *reinterpret_cast<const float4 *>(tile + 16 * mt);
            s[mt][0] = x.x;
            s[mt][1] = x.y;
            s[mt][2] = x.z;
            s[mt][3] = x.w;
        }
    }

    // ---- 3. pair coefficients on the matrix cores; the first fold chunk goes to LDS --------
    // M tile jt is KQ rows 16jt .. 16jt+15, i.e. k and q of nodes 8jt .. 8jt+7 interleaved; N
    // tile at holds the keys of nodes 16at .. 16at+15.  Lane (lr, lg) receives rows 4lg + r: of
    // node 8jt + 2lg + r/2, k . k_a for even r and q . k_a for odd r, with a = 16at + lr.  Rows
    // and keys past the tree are clamped to its last node; their products are never used.
    // A key a pairs with node n only if a <= n (an ancestor, or n itself), so M tile jt (nodes
    // up to 8jt + 7) needs the key tiles at <= jt / 2 only: (jt / 2) + 1 tiles per M tile.
    const int JT = (n + 7) >> 3;
    int n_tiles = 0;
    for (int j = 0; j < JT; ++j) n_tiles += (j >> 1) + 1;
    for (int ti = w; ti < n_tiles; ti += NW) {
        int jt = 0, at = ti;
        while (at > (jt >> 1)) at -= (jt++ >> 1) + 1;
        const int kn = 16 * at + lr;
        // fp32 operands straight from LDS: the 4-column step {16mt + 4lg + e} takes A[lr][lg]
        // and B[lg][lr] from one float4 read per lane and mt; two accumulators halve the chain.
        const float *xrow = KQ + size_t(min(16 * jt + lr, 2 * n - 1)) * LY::KS + 4 * lg;
        const float *krow = KQ + size_t(2 * min(kn, n - 1)) * LY::KS + 4 * lg;
        floatx4 acc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const float4 a4 = *reinterpret_cast<const float4 *>(xrow + 16 * mt);
            const float4 b4 = *reinterpret_cast<const float4 *>(krow + 16 * mt);
            const float av[4] = {a4.x, a4.y, a4.z, a4.w};
            const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc2[mt & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], acc2[mt & 1], 0, 0, 0);
        }
        const floatx4 acc = acc2[0] + acc2[1];
        const int an = 16 * at + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int nd = 8 * jt + 2 * lg + (r >> 1);
            const bool is_q = r & 1;
            if (nd >= n || an >= n) continue;
            if (an == nd) {
                if (is_q) kqd[nd] = acc[r];
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
    if (L > 0) GDN_FOLD_STORE(min(L, nfc));
    __syncthreads();  // T, C' and q.k on the records; the first fold chunk is in LDS

    // ---- 4. deferred commit: fold the pending rows, write the committed state once --------
    // S_L = G S0 + sum_i c_i u_i k_i^T with G the product of the L pending gates (exp of the sum
    // of their logs, loaded in phase 0) and c_i that of the gates after row i (staged with the
    // rows): the tile is scaled once, then the rank-L update runs on the matrix cores.  Chunks
    // of nfc rows come last chunk first (the staged one holds rows L - min(L, nfc) .. L - 1).
    if (L > 0) {
        const float G = expf(wave_total(lg_part));
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[mt][e] *= G;
        for (int hi = L; hi > 0; hi -= nfc) {
            const int lo = max(hi - nfc, 0), cnt = hi - lo;
            if (hi < L) {  // earlier chunks (more pending rows than one chunk holds)
                __syncthreads();
                GDN_FOLD_LOAD(lo, cnt);
                GDN_FOLD_STORE(cnt);
                __syncthreads();
            }
            // S^T += K^T (c u)^T on the fp32 matrix cores: s[mt] is the D tile of columns
            // 16mt.. and rows 16w..; the 4-row step from row k0 takes A[lr][lg] =
            // k_{k0+lg}[16mt + lr] and B[lg][lr] = c_{k0+lg} u_{k0+lg}[16w + lr].  Rows past the
            // chunk read its last row with c = 0.
            for (int k0 = 0; k0 < cnt; k0 += 4) {
                const int f = k0 + lg, fr = min(f, cnt - 1);
                const float cf = f < cnt ? FC[f] : 0.f;
                const float b0 = cf * FU[fr * D + row0 + lr];
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    const float a = FK[fr * D + 16 * mt + lr];
                    floatx4 t0 = {s[mt][0], s[mt][1], s[mt][2], s[mt][3]};
                    t0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b0, t0, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[mt][e] = t0[e];
                }
            }
        }
        float *tile = committed + (row0 + lr) * D + 4 * lg;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
            *reinterpret_cast<float4 *>(tile + 16 * mt) =
                make_float4(s[mt][0], s[mt][1], s[mt][2], s[mt][3]);
    }

    // p_n = S0 k_n, r_n = S0 q_n on the matrix cores; then w_n and G_n r_n to LDS.
    {
        const char *XV = lds + lay.xv;
        const int i = row0 + lr;  // this lane's state row in the epilogue
        for (int jt0 = 0; jt0 < JT; jt0 += JC) {
            // fp32 MFMA 16x16x4 per 4-column step {16mt + 4lg + e}: lane (lr, lg) gives A[lr][lg]
            // = KQ row 16jt + lr (k and q of node 8jt + lr/2; one float4 read per mt covers
            // e = 0..3, rows past the tree clamped to its last) and B[lg][lr] = its own tile
            // element s[mt][e].
            const float *arow[JC];
#pragma unroll
            for (int jc = 0; jc < JC; ++jc)
                arow[jc] = KQ + size_t(min(16 * (jt0 + jc) + lr, 2 * n - 1)) * LY::KS + 4 * lg;
            floatx4 acc[JC];
#pragma unroll
            for (int jc = 0; jc < JC; ++jc) acc[jc] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
                for (int jc = 0; jc < JC; ++jc) {
                    if (jt0 + jc >= JT) break;
                    const float4 a4 = *reinterpret_cast<const float4 *>(arow[jc] + 16 * mt);
                    const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[jc] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], s[mt][e], acc[jc],
                                                                       0, 0, 0);
                }
            }
            // W and GR of this pass's nodes take their k and q rows: every wave must be done
            // reading them.  The fold rows are dead past the first pass too.
            __syncthreads();
            // Lane (lr, lg) holds rows 4lg + r of each M tile: p (even r) and r (odd r) of node
            // 8jt + 2lg + r/2 at state row 16w + lr.  The v channel i: its taps and window.
            const uint2 wvr = *reinterpret_cast<const uint2 *>(lds + lay.wv + size_t(i) * 8);
            const float wv[4] = {bf16_lo(wvr.x), bf16_hi(wvr.x), bf16_lo(wvr.y), bf16_hi(wvr.y)};
            const float *cv = X0s + 2 * D + i;  // v channel i, taps 0..2
            const float cv0 = cv[0], cv1 = cv[3 * D], cv2 = cv[6 * D];
#pragma unroll
            for (int jc = 0; jc < JC; ++jc) {
                const int jt = jt0 + jc;
                if (jt >= JT) break;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int nd = 8 * jt + 2 * lg + j;
                    if (nd >= n) continue;
                    const float G = gam[nd];
                    const int dt = dep[nd];
                    const int4 an = anc[nd];
                    const float beta = slot_f32<bf16_t>(Bl[nd]);
                    const float v = silu(conv4(
                        wv, bf16_at(XV + size_t(nd) * LY::XROW, i),
                        bf16_at(XV + size_t(an.x) * LY::XROW, i),
                        bf16_at(XV + size_t(an.y) * LY::XROW, i),
                        bf16_at(XV + size_t(an.z) * LY::XROW, i), dt, cv0, cv1, cv2));
                    Wm[nd * WS + i] = beta * fmaf(-G, acc[jc][2 * j], v);
                    GR[nd * WS + i] = G * acc[jc][2 * j + 1];
                }
            }
        }
    }
    // Y = T^-1 and Z = C' Y on the records and their dense rows (over the dead fold rows), on
    // wave 0 while the other waves finish their epilogue.
    tree_inverse<DEEP ? 16 : 12>(
        n, n > 0 ? plan[P.off_ut_lv_base + seq + 1] - plan[P.off_ut_lv_base + seq] - 2 : 0, lane,
        w, poff, dep, lvn, recM, recP, recT, recC, recQ, kqd, recY, recZ, Yd, Zd, ys);
    __syncthreads();

    // ---- 5. u_n = sum_a Y[n][a] w_a, o_n = G_n r_n + sum_a Z[n][a] w_a, every (node, row) ---
    tree_apply_rows<1>(n, ys, w, lane, Yd, Zd, Wm, GR, WS, P.bank_u[role ^ 1] + row0_bank * D,
                       P.out + node_row0 * D, int64_t(P.H) * D);
}


namespace {

gdn_status run_conv_verify(const gdn_verify_args *va, const gdn_conv_args *ca,
                           const int32_t *host_image, const int32_t *dev_image, void *stream,
                           hipEvent_t start, hipEvent_t stop) {
    VerifyParams P;
    ImageView v;
    gdn_status st = verify_setup(va, host_image, dev_image, P, v, false, false);
    if (st != GDN_OK) return st;
    if (va->head_dim != kCvD || va->in_dtype != GDN_BF16)
        return fail(GDN_EINVAL, "gdn_tree_conv_verify: needs head_dim 128 and bf16 beta/gate "
                    "(got %d, dtype %d)", va->head_dim, va->in_dtype);
    if (ca == nullptr) return fail(GDN_EINVAL, "gdn_tree_conv_verify: null conv args");
    if (ca->in_dtype != GDN_BF16 || ca->width != 4)
        return fail(GDN_EINVAL, "gdn_tree_conv_verify: needs bf16 x/weight and conv width 4");
    if (int64_t(ca->channels) != 3ll * va->n_heads * kCvD)
        return fail(GDN_EINVAL, "gdn_tree_conv_verify: channels %d != 3 * n_heads * 128",
                    ca->channels);
    if (ca->n_seqs != va->n_seqs || ca->n_nodes != va->n_nodes ||
        ca->max_nodes != va->max_nodes || ca->layer_begin != va->layer_begin ||
        ca->n_layers != va->n_layers)
        return fail(GDN_EINVAL, "gdn_tree_conv_verify: conv and verify args disagree on "
                    "n_seqs/n_nodes/max_nodes/layer_begin/n_layers");
    if (va->n_seqs == 0) return GDN_OK;  // empty batch: nothing is read or written
    if (ca->role != va->role || ca->pending_len != va->pending_len ||
        ca->pending_rows != va->pending_rows)
        return fail(GDN_EINVAL, "gdn_tree_conv_verify: conv and verify args must share the "
                    "role, pending_len and pending_rows arrays");
    if (!ca->x || !ca->weight || !ca->conv_state || !ca->bank_x[0] || !ca->bank_x[1])
        return fail(GDN_EINVAL, "gdn_tree_conv_verify: null x/weight/conv_state/bank_x");
    if (reinterpret_cast<uintptr_t>(ca->x) % 16 || reinterpret_cast<uintptr_t>(ca->weight) % 16 ||
        reinterpret_cast<uintptr_t>(ca->bank_x[0]) % 16 ||
        reinterpret_cast<uintptr_t>(ca->bank_x[1]) % 16)
        return fail(GDN_EINVAL, "gdn_tree_conv_verify: x, weight and bank_x must be 16-byte "
                    "aligned");
    if (v.ut_records < 0)
        return fail(GDN_EINVAL, "gdn_tree_conv_verify: the schedule has no tree-masked plan "
                    "(its trees need more than %d records per node)", kUtRecordsPerNode);
    P.off_parent = v.off_parent;
    P.off_depth = v.off_depth;
    P.off_ut_rec_base = v.off_ut_rec_base;
    P.off_ut_node_rec = v.off_ut_node_rec;
    P.off_ut_lv_base = v.off_ut_lv_base;
    P.off_ut_lvn = v.off_ut_lvn;
    P.off_ut_lvnode = v.off_ut_lvnode;
    P.off_ut_rec_anc = v.off_ut_rec_anc;
    P.n_blocks = int64_t(va->n_layers) * va->n_seqs * va->n_heads;
    if (P.n_blocks > kMaxBlocks)
        return fail(GDN_EINVAL, "gdn_tree_conv_verify: too many workgroups for one launch");
    const int n_max = v.max_tree, nrec_max = v.ut_max_records, nlv_max = v.ut_max_levels;
    const int nf = va->max_nodes;
    const int nfc = std::min(CvLayout::fold_rows(n_max, nf), kFoldRows);
    const size_t lds = CvLayout(n_max, nrec_max, nlv_max, nf, nfc).total;
    if (lds > kUtMaxLdsBytes)
        return fail(GDN_EINVAL, "gdn_tree_conv_verify: trees of %d nodes with %d records need "
                    "%zu bytes of LDS (limit %zu)", n_max, nrec_max, lds, kUtMaxLdsBytes);
    ConvVerifyParams CP;
    CP.V = P;
    CP.x = static_cast<const bf16_t *>(ca->x);
    CP.w = static_cast<const bf16_t *>(ca->weight);
    CP.cstate = ca->conv_state;
    CP.bank_x[0] = static_cast<bf16_t *>(ca->bank_x[0]);
    CP.bank_x[1] = static_cast<bf16_t *>(ca->bank_x[1]);
    CP.C = ca->channels;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(uint32_t(P.n_blocks));
    // the deepest tree of the batch: its depth levels are nlv_max - 2
    if (nlv_max - 2 > 12) {
        if (start == nullptr && stop == nullptr)
            hipLaunchKernelGGL(conv_verify_kernel<true>, grid, dim3(kCvThreads), lds, s, CP, P.img,
                               P.rows, n_max, nrec_max, nlv_max, nf, nfc);
        else
            hipExtLaunchKernelGGL(conv_verify_kernel<true>, grid, dim3(kCvThreads), uint32_t(lds),
                                  s, start, stop, 0, CP, P.img, P.rows, n_max, nrec_max, nlv_max,
                                  nf, nfc);
    } else {
        if (start == nullptr && stop == nullptr)
            hipLaunchKernelGGL(conv_verify_kernel<false>, grid, dim3(kCvThreads), lds, s, CP,
                               P.img, P.rows, n_max, nrec_max, nlv_max, nf, nfc);
        else
            hipExtLaunchKernelGGL(conv_verify_kernel<false>, grid, dim3(kCvThreads),
                                  uint32_t(lds), s, start, stop, 0, CP, P.img, P.rows, n_max,
                                  nrec_max, nlv_max, nf, nfc);
    }
    GDN_LAUNCH_CHECK("conv_verify_kernel");
    return GDN_OK;
}

}  // namespace

}  // namespace gdn

using namespace gdn;

extern "C" gdn_status gdn_tree_conv_verify(const gdn_verify_args *va, const gdn_conv_args *ca,
                                           const int32_t *host_image, const int32_t *dev_image,
                                           void *stream) {
    clear_error();
    return run_conv_verify(va, ca, host_image, dev_image, stream, nullptr, nullptr);
}

extern "C" gdn_status gdn_tree_conv_verify_timed(const gdn_verify_args *va,
                                                 const gdn_conv_args *ca,
                                                 const int32_t *host_image,
                                                 const int32_t *dev_image, void *start_event,
                                                 void *stop_event, void *stream) {
    clear_error();
    if (start_event == nullptr || stop_event == nullptr)
        return fail(GDN_EINVAL, "gdn_tree_conv_verify_timed: null event");
    return run_conv_verify(va, ca, host_image, dev_image, stream,
                           static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
}
