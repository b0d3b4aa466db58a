// Chunked prefill of token sequences through the gated delta rule, on the matrix cores
// (gfx950, bf16 inputs, d = 128).
//
// After a flush ("Lucebox SpecLA and Gated DeltaNet state-resident verification" guide, the
// flush section) the runtime runs the GDN layer over plain token sequences.  A sequence is a
// tree without branching, so each chunk of C = 16 tokens is the tree-masked (UT) form of
// mechanism 1 on a chain, and the state carried from chunk to chunk is the deferred commit of
// mechanism 4 applied to the whole chunk.  With S the state at the chunk start (rows = d_v),
// G_t the product of the chunk's gates up to and including t, E(t,s) the product of the gates
// of tokens s+1 .. t, T[t][s] = beta_t E(t,s) (k_t . k_s) (s < t) and C'[t][s] = E(t,s)
// (q_t . k_s) (s <= t):
//   w_t = beta_t (v_t - G_t S k_t),   (I + T) U = W,   O = diag(G) Q S^T + C' U
//   S  <- G_{C-1} S + sum_t E(C-1,t) u_t k_t^T.
// Y = (I + T)^-1 depends on the chunk's inputs only: U = Y W.
//
// Work split: one workgroup of four waves per (layer, sequence, head, half of the state rows);
// wave r of half h holds rows 64h + 16r .. 64h + 16r + 15 in registers and walks the chunks.
// Per chunk, on the matrix cores and without leaving registers between steps:
//   [k; q] S^T with S as an exact bf16 x3 split,  w and G r,  U = Y W,  O = G r + C' U,
//   S^T <- G S^T + K^T (gamma U) with gamma U as an exact bf16 x3 split (two 32-deep products
//   per tile: hi and mid of the 16 tokens, then lo).
// Every product leaves its result where the next one takes its operand: the accumulator of
// lane (l % 16, l / 16) holds rows 4(l/16) .. 4(l/16)+3 of column l % 16, which is that lane's
// share of the next product's right operand when the summation index runs over 4(l/16) + step.
//
// The chunk tables are built off the state chain, in a three-stage pipeline with one barrier
// per step: in step i, one wave forms chunk i+1's gate products, K K^T and K Q^T, hence T, T^T
// and C'^T (stage A); another turns chunk i's T into Y by the Neumann product of the nilpotent T,
//   (I + T)^-1 = (I - T)(I + T^2)(I + T^4)(I + T^8),
// keeping each factor both as itself and as its transpose (the left operand of a product is its
// transpose in that layout) (stage B); and all four waves advance the state over chunk i-1.  The
// two table roles move to the next wave every step.  k and q rows are staged through registers two
// steps ahead into a four-deep LDS ring; each lane loads its own v values one step ahead.
// State layout: lane l of a wave holds rows 16r + (l % 16) and columns 16m + 4(l / 16) + e.
#include <hip/hip_ext.h>

#include "mfma_common.h"

namespace gdn {

namespace {

constexpr int kD = 128;
constexpr int kC = 16;                    // tokens per chunk
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHalfRows = kD / 2;         // state rows per workgroup
constexpr int kRowBytes = 2 * kD * 2 + 16;  // k | q | pad
constexpr int kRing = 4;                  // k/q chunks in LDS

struct PrefillParams {
    const void *q, *k, *v, *beta, *gate;
    float *state, *out;
    const int32_t *seq_off;
    int32_t S, H, T, layer_begin;
    int64_t n_blocks;
};

// One chunk's tables for the state waves: Y^T and C'^T in the accumulator layout (lane-major,
// four floats per lane: lane (c, g) holds Y[c][4g + e] and C'[c][4g + e]), and per token G_t,
// gamma_t = E(nc-1, t) (0 past the chunk) and beta_t.
struct ChunkTab {
    floatx4 yt[64], ct[64];
    float G[kC], gam[kC], beta[kC];
};

// Stage A's hand-over to stage B: T and T^T in the accumulator layout.  Before that, stage A
// uses the same bytes for its gate-product tables: ecol[s][t] = E(t, s) (t >= s) and
// erev[t][15 - s] = E(t, s) (s <= t).
union Handover {
    struct {
        floatx4 t[64], tt[64];
    } tt;
    struct {
        float ecol[kC][kC], erev[kC][kC];
    } e;
};

struct PrefillLds {
    char kq[kRing][kC * kRowBytes];  // k | q rows of a chunk, bf16
    uint32_t kt[2][kD * kC / 2];     // K^T of a chunk, bf16 [column][token], swizzled (kt_slot)
    ChunkTab tab[3];
    Handover ho[2];
    float bg[2][2 * kC];             // raw beta (0..C-1) and g (C..2C-1)
};

// Dword index in a K^T buffer of tokens 2p, 2p+1 (p < 8) of column j: the four 8-byte groups
// of a column's 16 tokens are permuted by XOR with (j / 4) mod 4, so that 16 lanes reading one
// group each of 16 consecutive columns hit distinct banks.
__device__ __forceinline__ int kt_slot(int j, int p) {
    return j * (kC / 2) + ((((p >> 1) ^ (j >> 2)) & 3) << 1) + (p & 1);
}

// K^T of a staged chunk from its k rows: thread i takes column i % 128 and tokens 8 (i / 128)
// .. +7, reads them as 2-byte loads (a wave reads 128 consecutive bytes of each row), packs the
// token pairs into dwords and writes two 8-byte groups.  (One thread per 16 bytes of a row with
// 16-bit stores sent the 16 lanes of a token to three or four banks: ~22% of the CU cycles were
// LDS bank conflicts.)
__device__ __forceinline__ void build_kt(const char *kq, uint32_t *kt, int tid) {
    const int j = tid & (kD - 1), h = tid >> 7;  // column, half of the chunk's tokens
    const uint16_t *col = reinterpret_cast<const uint16_t *>(kq + 8 * h * kRowBytes) + j;
    uint32_t v[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
        v[p] = uint32_t(col[(2 * p) * (kRowBytes / 2)]) |
               (uint32_t(col[(2 * p + 1) * (kRowBytes / 2)]) << 16);
    // tokens 8h + 2p, +1 sit in dword kt_slot(j, 4h + p); p = 0, 1 and p = 2, 3 are 8-byte groups
    *reinterpret_cast<uint2 *>(kt + kt_slot(j, 4 * h)) = make_uint2(v[0], v[1]);
    *reinterpret_cast<uint2 *>(kt + kt_slot(j, 4 * h + 2)) = make_uint2(v[2], v[3]);
}

// Register staging of a chunk's k and q: thread i holds 16 bytes of each (token i / 16, piece
// i % 16); threads 128 .. 159 one beta or g.  Tokens past the chunk repeat its last token.
struct Staged {
    u32x4 k, q;
    uint32_t bg;
};

__device__ __forceinline__ void stage_load(Staged &r, const PrefillParams &P, int64_t crow, int nc,
                                           int tid) {
    const int tk = min(tid >> 4, nc - 1);
    const int ok = tk * P.H * kD * 2 + (tid & 15) * 16;  // from the chunk's first row
    r.k = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(P.k) + crow * kD * 2 + ok);
    r.q = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(P.q) + crow * kD * 2 + ok);
    if (tid >= 128 && tid < 128 + 2 * kC) {
        const int i = tid - 128;
        const int t = min(i % kC, nc - 1);
        r.bg = *(static_cast<const bf16_t *>(i < kC ? P.beta : P.gate) + crow + int64_t(t) * P.H);
    }
}

__device__ __forceinline__ void stage_store(const Staged &r, PrefillLds &sm, int chunk, int tid) {
    char *row = sm.kq[chunk % kRing] + (tid >> 4) * kRowBytes + (tid & 15) * 16;
    *reinterpret_cast<u32x4 *>(row) = r.k;
    *reinterpret_cast<u32x4 *>(row + kD * 2) = r.q;
    if (tid >= 128 && tid < 128 + 2 * kC) sm.bg[chunk & 1][tid - 128] = __uint_as_float(r.bg << 16);
}

// P = A B for 16 x 16 fp32 matrices held in the accumulator layout (lane (c, g) holds rows
// 4g .. 4g+3 of column c): the left operand is passed as the layout of A^T, the right one as
// the layout of B, the summation index of step j in lane group g being 4g + j.
__device__ __forceinline__ floatx4 mm(floatx4 at, floatx4 b, floatx4 acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(at[j], b[j], acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ floatx4 plus_identity(floatx4 x, int lr, int lg, float sign) {
    floatx4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = (4 * lg + r == lr ? 1.f : 0.f) + sign * x[r];
    return y;
}

// Stage A for a chunk of nc tokens (k, q rows in `kq`, raw beta and g in `bg`), by one wave:
// gate products, K K^T and K Q^T, then T and T^T to the hand-over and C'^T, G, gamma and beta to
// the chunk's table.
__device__ __forceinline__ void stage_a(const char *kq, const float *bg, ChunkTab &tb, Handover &ho,
                                        int nc, int lane) {
    const int lr = lane & 15, lg = lane >> 4;
    {
        // Gate products: lanes 0-15 the column E(., s) for s = lane (upwards from s), lanes
        // 16-31 the row E(t, .) for t = lane - 16 (downwards from t, stored reversed so that
        // both halves write step i to position i); exact products in fp32.  Each lane reads its
        // own factor sequence through a per-lane pointer (a select between two register arrays
        // would become a dynamic index).
        const bool up = lane < kC;
        const float *fp = bg + (up ? kC : 2 * kC);
        const int step = up ? 1 : -1;
        float x = 1.f, ev[kC];
        ev[0] = 1.f;  // step 0 takes no factor in either direction
#pragma unroll
        for (int i = 1; i < kC; ++i) {
            const float f = fp[step * i];
            const bool take = up ? i > lr : (kC - 1 - i) < lr;
            x = take ? x * f : x;
            ev[i] = x;
        }
        if (lane < 2 * kC) {
            float *dst = up ? &ho.e.ecol[lr][0] : &ho.e.erev[lr][0];
#pragma unroll
            for (int i = 0; i < kC; i += 4)
                *reinterpret_cast<floatx4 *>(dst + i) = floatx4{ev[i], ev[i + 1], ev[i + 2], ev[i + 3]};
        }
    }
    // K K^T and K Q^T (bf16, exact products): lane (c, g) receives rows 4g + r against column c
    floatx4 kk = {0.f, 0.f, 0.f, 0.f}, kqp = {0.f, 0.f, 0.f, 0.f};
    {
        const char *row = kq + lr * kRowBytes;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const bf16x8 ka = row_operand(row, 32 * b + 4 * lg);
            kk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ka, kk, 0, 0, 0);
            kqp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, row_operand(row + kD * 2, 32 * b + 4 * lg),
                                                          kqp, 0, 0, 0);
        }
    }
    wave_order();  // the gate products are in LDS
    const floatx4 up4 = *reinterpret_cast<const floatx4 *>(&ho.e.ecol[lr][4 * lg]);  // E(4g+r, c)
    const floatx4 dnr = *reinterpret_cast<const floatx4 *>(&ho.e.erev[lr][12 - 4 * lg]);
    const floatx4 dn4 = {dnr[3], dnr[2], dnr[1], dnr[0]};  // E(c, 4g+r)
    const floatx4 b4 = *reinterpret_cast<const floatx4 *>(bg + 4 * lg);
    const float bc = bg[lr];
    float G = 0.f, gam = 0.f;
    if (lane < kC) {
        G = bg[kC] * ho.e.ecol[0][lane];                               // g_0 E(t, 0)
        gam = lane < nc ? ho.e.erev[nc - 1][kC - 1 - lane] : 0.f;      // E(nc-1, t)
    }
    floatx4 T, Tt, Ct;  // T, T^T and C'^T in the accumulator layout
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = 4 * lg + r;
        T[r] = lr < t ? b4[r] * up4[r] * kk[r] : 0.f;
        Tt[r] = t < lr ? bc * dn4[r] * kk[r] : 0.f;
        Ct[r] = t <= lr ? dn4[r] * kqp[r] : 0.f;
    }
    wave_order();  // every lane has read the gate products: the hand-over bytes may be reused
    ho.tt.t[lane] = T;
    ho.tt.tt[lane] = Tt;
    tb.ct[lane] = Ct;
    if (lane < kC) {
        tb.G[lane] = G;
        tb.gam[lane] = gam;
        tb.beta[lane] = bg[lane];
    }
}

// Stage B: Y^T from T and T^T, by one wave.
__device__ __forceinline__ void stage_b(const Handover &ho, ChunkTab &tb, int lane) {
    const int lr = lane & 15, lg = lane >> 4;
    const floatx4 T = ho.tt.t[lane], Tt = ho.tt.tt[lane];
    const floatx4 z = {0.f, 0.f, 0.f, 0.f};
    const floatx4 T2 = mm(Tt, T, z), T2t = mm(T, Tt, z);
    const floatx4 T4 = mm(T2t, T2, z), T4t = mm(T2, T2t, z);
    // M1^T = (I + T^2)^T (I - T)^T, M2^T = (I + T^4)^T M1^T, Y^T = (I + T^8)^T M2^T
    const floatx4 M1t = mm(plus_identity(T2, lr, lg, 1.f), plus_identity(Tt, lr, lg, -1.f), z);
    const floatx4 T8 = mm(T4t, T4, z);
    const floatx4 M2t = mm(plus_identity(T4, lr, lg, 1.f), M1t, z);
    tb.yt[lane] = mm(plus_identity(T8, lr, lg, 1.f), M2t, z);
}

// Exact bf16 x3 split of four values: b1 = {hi, mid}, b2 = {lo, 0}.
__device__ __forceinline__ void split3_pairs(const float *u, bf16x8 &b1, bf16x8 &b2) {
    float x[8] = {u[0], u[1], u[2], u[3], 0.f, 0.f, 0.f, 0.f};
    bf16x8 h, m, l;
    split3(x, h, m, l);
    const u32x4 hv = __builtin_bit_cast(u32x4, h), mv = __builtin_bit_cast(u32x4, m),
                lv = __builtin_bit_cast(u32x4, l);
    const u32x4 p1 = {hv[0], hv[1], mv[0], mv[1]}, p2 = {lv[0], lv[1], 0u, 0u};
    b1 = __builtin_bit_cast(bf16x8, p1);
    b2 = __builtin_bit_cast(bf16x8, p2);
}

// This lane's v values of a chunk (row R0 + (l % 16) of tokens 4(l / 16) + e, at element offset
// lofs[e] from the chunk's first row); tokens past the chunk read its first token instead.
__device__ __forceinline__ void load_v(uint16_t (&vr)[4], const PrefillParams &P, int64_t crow,
                                       int nc, const int (&lofs)[4], int lg) {
    const bf16_t *vb = static_cast<const bf16_t *>(P.v) + crow * kD;
#pragma unroll
    for (int e = 0; e < 4; ++e) vr[e] = vb[4 * lg + e < nc ? lofs[e] : lofs[e] - (4 * lg + e) * P.H * kD];
}

}  // namespace

// Three waves per SIMD (at most 168 VGPRs) and under 53,760 bytes of LDS: three workgroups per CU.
__global__ __launch_bounds__(kThreads, 3)
void prefill_kernel(PrefillParams P) {
    constexpr int D = kD;
    __shared__ __align__(16) PrefillLds sm;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t unit = xcd_logical(blockIdx.x, uint32_t(P.n_blocks));
    const int half = int(unit & 1u);
    const uint32_t pair = unit >> 1, per = uint32_t(P.S) * uint32_t(P.H);
    const int layer = P.layer_begin + int(pair / per);
    const int seq = int((pair % per) / uint32_t(P.H)), h = int(pair % uint32_t(P.H));
    const int t_begin = P.seq_off[seq], len = P.seq_off[seq + 1] - t_begin;
    const int n = (len + kC - 1) / kC;  // chunks
    if (n == 0) return;  // uniform over the workgroup: no barrier is skipped by part of it
    const int64_t row0 = (int64_t(layer) * P.T + t_begin) * P.H + h;  // token 0's (t, h) row
    // stage A runs on wave (i + rot) % 4 in step i and stage B two waves on: the table work
    // visits every SIMD in turn, whichever workgroups share a CU
    const int rot = int((blockIdx.x ^ (blockIdx.x >> 3) ^ (blockIdx.x >> 8)) & 3u);
    const int R0 = half * kHalfRows + 16 * w;  // first state row of this wave
    auto nc_of = [&](int x) { return min(kC, len - x * kC); };
    auto crow_of = [&](int x) { return row0 + int64_t(x) * kC * P.H; };

    float *state = P.state + ((int64_t(layer) * P.S + seq) * P.H + h) * D * D;
    floatx4 s[8];  // S^T tiles: row R0 + lr, columns 16m + 4lg + e
    {
        const float *tile = state + (R0 + lr) * D + 4 * lg;
#pragma unroll
        for (int m = 0; m < 8; ++m) s[m] = *reinterpret_cast<const floatx4 *>(tile + 16 * m);
    }
    // per-lane element offsets of this lane's output and v values (token 4lg + r, row R0 + lr)
    // from a chunk's first (t, h) row
    int lofs[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lofs[r] = (4 * lg + r) * P.H * D + R0 + lr;
    Staged st;
    stage_load(st, P, crow_of(0), nc_of(0), tid);
    stage_store(st, sm, 0, tid);
    uint16_t vr[4];
    __syncthreads();

    // Step i: stage chunk i+2, stage A of chunk i+1, stage B of chunk i, state over chunk i-1.
    for (int i = -1; i <= n; ++i) {
        const int wa = (i + 4 + rot) & 3, wb = (wa + 2) & 3;
        if (i + 2 < n) stage_load(st, P, crow_of(i + 2), nc_of(i + 2), tid);
        if (w == wa && i + 1 < n)
            stage_a(sm.kq[(i + 1) % kRing], sm.bg[(i + 1) & 1], sm.tab[(i + 1) % 3],
                    sm.ho[(i + 1) & 1], nc_of(i + 1), lane);
        if (w == wb && i >= 0 && i < n) stage_b(sm.ho[i & 1], sm.tab[i % 3], lane);
        if (i >= 1) {
            const int y = i - 1, nc = nc_of(y);
            const char *kq = sm.kq[y % kRing];
            const ChunkTab &tb = sm.tab[y % 3];
            // ---- [k; q] S^T: lane (lr, lg) receives token 4lg + r against row R0 + lr ------
            floatx4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                bf16x8 bh, bm, bl;
                {
                    const float x[8] = {s[2 * kb][0],     s[2 * kb][1],     s[2 * kb][2],
                                        s[2 * kb][3],     s[2 * kb + 1][0], s[2 * kb + 1][1],
                                        s[2 * kb + 1][2], s[2 * kb + 1][3]};  // columns 32kb + slots
                    split3(x, bh, bm, bl);
                }
                const bf16x8 a = row_operand(kq + lr * kRowBytes, 32 * kb + 4 * lg);
                const bf16x8 b = row_operand(kq + lr * kRowBytes + D * 2, 32 * kb + 4 * lg);
                ak = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, ak, 0, 0, 0);
                aq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, bl, aq, 0, 0, 0);
                ak = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bm, ak, 0, 0, 0);
                aq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, bm, aq, 0, 0, 0);
                ak = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, ak, 0, 0, 0);
                aq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, bh, aq, 0, 0, 0);
            }
            // ---- w_t = beta_t (v_t - G_t p_t) (0 past the chunk), o_t = G_t r_t ---------------
            const floatx4 G4 = *reinterpret_cast<const floatx4 *>(&tb.G[4 * lg]);
            const floatx4 B4 = *reinterpret_cast<const floatx4 *>(&tb.beta[4 * lg]);
            floatx4 wv, o;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * lg + r;
                const float v = __uint_as_float(uint32_t(vr[r]) << 16);
                wv[r] = t < nc ? B4[r] * fmaf(-G4[r], ak[r], v) : 0.f;
                o[r] = G4[r] * aq[r];
            }
            // ---- U = Y W, then O = G r + C' U -----------------------------------------------------
            const floatx4 u = mm(tb.yt[lane], wv, floatx4{0.f, 0.f, 0.f, 0.f});
            o = mm(tb.ct[lane], u, o);
            const floatx4 gm4 = *reinterpret_cast<const floatx4 *>(&tb.gam[4 * lg]);
            float ug[4];
            float *ob = P.out + crow_of(y) * D;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * lg + r;
                if (t < nc) ob[lofs[r]] = o[r];
                ug[r] = t < nc ? gm4[r] * u[r] : 0.f;
            }
            // ---- S^T <- G S^T + K^T (gamma U): two 32-deep bf16 products per tile -------------
            bf16x8 b1, b2;
            split3_pairs(ug, b1, b2);
            const float Ge = tb.G[nc - 1];
            const uint32_t *kt = sm.kt[y & 1];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                // k_t[16m + lr] for the lane's tokens 4lg .. 4lg+3, twice
                const uint2 kv = *reinterpret_cast<const uint2 *>(kt + kt_slot(16 * m + lr, 2 * lg));
                const u32x4 av = {kv.x, kv.y, kv.x, kv.y};
                const bf16x8 a = __builtin_bit_cast(bf16x8, av);
                s[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b2, s[m] * Ge, 0, 0, 0);
                s[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, s[m], 0, 0, 0);
            }
        }
        if (i >= 0 && i < n) {  // chunk i's v values and K^T, for step i + 1
            load_v(vr, P, crow_of(i), nc_of(i), lofs, lg);
            build_kt(sm.kq[i % kRing], sm.kt[i & 1], tid);
        }
        if (i + 2 < n) stage_store(st, sm, i + 2, tid);
        __syncthreads();
    }

    float *tile = state + (R0 + lr) * D + 4 * lg;
#pragma unroll
    for (int m = 0; m < 8; ++m) *reinterpret_cast<floatx4 *>(tile + 16 * m) = s[m];
}

}  // namespace gdn

using namespace gdn;

static gdn_status run_prefill(const gdn_prefill_args *a, const int32_t *host_seq_offsets,
                              void *stream, hipEvent_t start, hipEvent_t stop) {
    if (a == nullptr || host_seq_offsets == nullptr)
        return fail(GDN_EINVAL, "gdn_prefill: null arguments");
    if (a->n_seqs < 0 || a->n_heads < 1 || a->n_layers < 1 || a->layer_begin < 0 ||
        a->n_tokens < 0)
        return fail(GDN_EINVAL, "gdn_prefill: bad n_seqs/n_heads/n_layers/layer_begin/n_tokens");
    if (a->head_dim != 128 || a->in_dtype != GDN_BF16)
        return fail(GDN_EINVAL, "gdn_prefill: supports head_dim 128 with bf16 inputs (got %d, "
                    "dtype %d)", a->head_dim, a->in_dtype);
    if (host_seq_offsets[0] != 0 || host_seq_offsets[a->n_seqs] != a->n_tokens)
        return fail(GDN_EINVAL, "gdn_prefill: seq_offsets must run from 0 to n_tokens");
    for (int b = 0; b < a->n_seqs; ++b)
        if (host_seq_offsets[b + 1] < host_seq_offsets[b])
            return fail(GDN_EINVAL, "gdn_prefill: seq_offsets must not decrease (sequence %d)", b);
    if (a->n_seqs == 0) return GDN_OK;
    const void *ptrs[] = {a->q, a->k, a->v, a->beta, a->gate, a->state, a->out, a->seq_offsets};
    for (const void *p : ptrs)
        if (p == nullptr) return fail(GDN_EINVAL, "gdn_prefill: null device pointer");
    const void *al16[] = {a->q, a->k, a->v, a->state, a->out};
    for (const void *p : al16)
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
            return fail(GDN_EINVAL, "gdn_prefill: q/k/v/state/out must be 16-byte aligned");
    PrefillParams P;
    P.q = a->q;
    P.k = a->k;
    P.v = a->v;
    P.beta = a->beta;
    P.gate = a->gate;
    P.state = a->state;
    P.out = a->out;
    P.seq_off = a->seq_offsets;
    P.S = a->n_seqs;
    P.H = a->n_heads;
    P.T = a->n_tokens;
    P.layer_begin = a->layer_begin;
    P.n_blocks = int64_t(a->n_layers) * a->n_seqs * a->n_heads * 2;  // two halves of the rows
    if (P.n_blocks > kMaxBlocks) return fail(GDN_EINVAL, "gdn_prefill: too many workgroups");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (start == nullptr && stop == nullptr)
        hipLaunchKernelGGL(prefill_kernel, dim3(uint32_t(P.n_blocks)), dim3(kThreads), 0, s, P);
    else
        hipExtLaunchKernelGGL(prefill_kernel, dim3(uint32_t(P.n_blocks)), dim3(kThreads), 0, s,
                              start, stop, 0, P);
    GDN_LAUNCH_CHECK("prefill_kernel");
    return GDN_OK;
}

extern "C" gdn_status gdn_prefill(const gdn_prefill_args *a, const int32_t *host_seq_offsets,
                                  void *stream) {
    clear_error();
    return run_prefill(a, host_seq_offsets, stream, nullptr, nullptr);
}

extern "C" gdn_status gdn_prefill_timed(const gdn_prefill_args *a,
                                        const int32_t *host_seq_offsets, void *start_event,
                                        void *stop_event, void *stream) {
    clear_error();
    if (start_event == nullptr || stop_event == nullptr)
        return fail(GDN_EINVAL, "gdn_prefill_timed: null event");
    return run_prefill(a, host_seq_offsets, stream, static_cast<hipEvent_t>(start_event),
                       static_cast<hipEvent_t>(stop_event));
}
