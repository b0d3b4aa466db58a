// Chunked prefill of token sequences through the gated delta rule, on the matrix cores
// (gfx950, bf16 inputs, d = 128).
//
// After a flush ("Lucebox SpecLA and Gated DeltaNet state-resident verification" guide, the
// flush section) the runtime runs the GDN layer over plain token sequences.  A sequence is a
// tree without branching, so each chunk of C = 16 tokens is the tree-masked (UT) form of
// mechanism 1 on a chain, and the state carried from chunk to chunk is the deferred commit of
// mechanism 4 applied to the whole chunk.  With S the state at the chunk start (rows = d_v),
// G_t the product of the chunk's gates up to and including t and E(t,s) the product of the
// gates of tokens s+1 .. t:
//   u_t = beta_t (v_t - G_t S k_t - sum_{s<t} E(t,s) (k_t . k_s) u_s)
//   o_t = G_t S q_t + sum_{s<=t} E(t,s) (q_t . k_s) u_s
//   S  <- G_{C-1} S + sum_t E(C-1,t) u_t k_t^T.
//
// One wave per (layer, sequence, head, block of 32 state rows): the rows of S are independent,
// so four waves share a head without talking to each other.  Per chunk:
//   1. k, q, v, beta, g of the chunk land in LDS (direct loads); gate products G and E;
//   2. [k; q] K^T on the matrix cores (bf16, exact products) gives T[t][s] = beta_t E (k_t.k_s)
//      and C[t][s] = E (q_t.k_s);
//   3. [k; q] S^T on the matrix cores, S as an exact bf16 x3 split: w_t = beta_t (v_t - G_t p_t)
//      and G_t r_t per row;
//   4. each lane owns one state row and solves u over the chunk in registers, then forms o;
//   5. S^T <- G S^T + K^T (gamma u) by fp32 16x16x4 MFMAs that accumulate straight into the
//      state registers, which hold S^T in the accumulator layout.
// State layout (the same as the tree-masked verify): lane l holds rows 32rb + 16nt + (l % 16)
// and columns 16mt + 4(l / 16) + e.
#include <hip/hip_ext.h>

#include "mfma_common.h"
#include "ut_common.h"

namespace gdn {

namespace {

constexpr int kD = 128;
constexpr int kC = 16;                    // tokens per chunk
constexpr int kCpv = kD * 2 / 16;         // 16-byte chunks per bf16 vector
constexpr int kCpn = 3 * kCpv + 1;        // k | q | v + one pad chunk (bank spread)
constexpr int kNodeBytes = kCpn * 16;
// Direct loads move 64 chunks per instruction: the input rows are padded to whole instructions.
constexpr int kInChunks = (kC * kCpn + 63) / 64 * 64;
constexpr int kRowPad = 36;               // row stride (floats) of the per-row tables

struct PrefillParams {
    const void *q, *k, *v, *beta, *gate;
    float *state, *out;
    const int32_t *seq_off;
    int32_t S, H, T, layer_begin;
    int64_t n_blocks;
};

// LDS of one wave.
struct PrefillLds {
    char in[kInChunks * 16];         // k | q | v rows of the chunk, bf16
    uint32_t bg[2][kC];              // beta | gate slots (bf16 zero-extended)
    float G[kC], gam[kC];            // G_t and E(C-1, t)
    float E[kC][kC];                 // E[t][s]: product of the gates of tokens s+1 .. t
    float Tm[kC][kC], Cm[kC][kC];    // read as whole rows by every lane (broadcast)
    float W[kC][kRowPad], GR[kC][kRowPad], Ug[kC][kRowPad];
};

}  // namespace

// Two waves per SIMD (at most 256 VGPRs): the state (64 floats per lane) stays live through the
// split S0 products and the per-row solve.
__global__ __launch_bounds__(64, 2)
void prefill_kernel(PrefillParams P) {
    constexpr int D = kD;
    __shared__ __align__(16) PrefillLds sm;
    const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
    // (layer, sequence, head, row block), the row block fastest: the four waves of a head
    // read the same chunk inputs, next to each other on one XCD.
    const uint32_t logical = xcd_logical(blockIdx.x, uint32_t(P.n_blocks));
    const int rb = int(logical & 3);
    const uint32_t unit = logical >> 2;
    const uint32_t per = uint32_t(P.S) * uint32_t(P.H);
    const int layer = P.layer_begin + int(unit / per);
    const int seq = int((unit % per) / uint32_t(P.H)), h = int(unit % uint32_t(P.H));
    const int t_begin = P.seq_off[seq], len = P.seq_off[seq + 1] - t_begin;
    float *state = P.state + ((int64_t(layer) * P.S + seq) * P.H + h) * D * D;
    const int64_t row0 = (int64_t(layer) * P.T + t_begin) * P.H + h;  // token 0's (t, h) row

    float s[2][8][4];  // S^T tiles: rows 32rb + 16nt + lr, columns 16mt + 4lg + e
    {
        const float *tile = state + (32 * rb + lr) * D + 4 * lg;
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

    const char *kb = static_cast<const char *>(P.k), *qb = static_cast<const char *>(P.q),
               *vb = static_cast<const char *>(P.v);
    for (int c0 = 0; c0 < len; c0 += kC) {
        const int nc = min(kC, len - c0);
        // ---- 1. chunk inputs into LDS; gate products ------------------------------------
        const int64_t crow = row0 + int64_t(c0) * P.H;
#pragma unroll 1
        for (int base = 0; base < kInChunks; base += 64) {
            const int c = base + lane;
            const int t = min(c / kCpn, nc - 1), r = c % kCpn;  // rows past nc re-read the last
            const bool real = r < 3 * kCpv;
            const int vec = real ? r / kCpv : 0, idx = real ? r % kCpv : 0;
            const char *src = (vec == 0 ? kb : (vec == 1 ? qb : vb)) +
                              (crow + int64_t(t) * P.H) * D * 2 + idx * 16;
            to_lds<16>(src, sm.in + size_t(base) * 16);
        }
        if (lane < 2 * kC) {
            const int which = lane / kC, t = min(lane % kC, nc - 1);
            const bf16_t *src = static_cast<const bf16_t *>(which == 0 ? P.beta : P.gate) +
                                crow + int64_t(t) * P.H;
            to_lds<2>(src, &sm.bg[0][0]);
        }
        __builtin_amdgcn_s_waitcnt(0);  // the chunk is in LDS
        wave_order();
        if (lane < kC) {  // G_t over tokens 0..t; row s of E by a running product over t > s
            float gv[kC];
#pragma unroll
            for (int m = 0; m < kC; ++m) gv[m] = slot_f32<bf16_t>(sm.bg[1][m]);
            float gp = 1.f, e = 1.f;
#pragma unroll
            for (int m = 0; m < kC; ++m) {
                if (m <= lane) gp *= gv[m];
                if (m > lane) e *= gv[m];
                sm.E[m][lane] = m > lane ? e : (m == lane ? 1.f : 0.f);
            }
            sm.G[lane] = gp;
        }
        wave_order();
        if (lane < kC) sm.gam[lane] = lane < nc ? sm.E[nc - 1][lane] : 0.f;  // E(nc-1, t)

        // ---- 2. pair products [k; q] K^T: T and C -------------------------------------
        // M tile jt stacks k (rows 0-7) and q (rows 8-15) of tokens 8jt .. 8jt+7; N = the 16
        // keys of the chunk.  Lane (lr, lg) receives token 8jt + 4(lg & 1) + r against key lr.
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            const int xt = 8 * jt + (lr & 7);
            const char *xrow = sm.in + size_t(xt) * kNodeBytes + (lr >> 3) * D * 2;
            const char *krow = sm.in + size_t(lr) * kNodeBytes;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    row_operand(xrow, 32 * kk + 4 * lg), row_operand(krow, 32 * kk + 4 * lg),
                    acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 8 * jt + 4 * (lg & 1) + r, sk = lr;
                const float e = sm.E[t][sk];
                const bool in_t = t < nc && sk < nc;
                if (lg >= 2)
                    sm.Cm[t][sk] = (in_t && sk <= t) ? e * acc[r] : 0.f;
                else
                    sm.Tm[t][sk] =
                        (in_t && sk < t) ? slot_f32<bf16_t>(sm.bg[0][t]) * e * acc[r] : 0.f;
            }
        }
        wave_order();

        // ---- 3. [k; q] S^T: w_t and G_t r_t for this wave's 32 rows ---------------------
        {
            floatx4 acc[2][2];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) acc[jt][0] = acc[jt][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 bh[2], bm[2], bl[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const float x[8] = {s[nt][2 * kk][0],     s[nt][2 * kk][1],
                                        s[nt][2 * kk][2],     s[nt][2 * kk][3],
                                        s[nt][2 * kk + 1][0], s[nt][2 * kk + 1][1],
                                        s[nt][2 * kk + 1][2], s[nt][2 * kk + 1][3]};
                    split3(x, bh[nt], bm[nt], bl[nt]);
                }
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    const int xt = 8 * jt + (lr & 7);
                    const bf16x8 a = row_operand(sm.in + size_t(xt) * kNodeBytes + (lr >> 3) * D * 2,
                                                 32 * kk + 4 * lg);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        acc[jt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl[nt], acc[jt][nt], 0, 0, 0);
                        acc[jt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bm[nt], acc[jt][nt], 0, 0, 0);
                        acc[jt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh[nt], acc[jt][nt], 0, 0, 0);
                    }
                }
            }
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 8 * jt + 4 * (lg & 1) + r;
                    const float G = sm.G[t];
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const int il = 16 * nt + lr;  // row inside the wave's block
                        if (lg < 2) {
                            const float v = bf16_at(sm.in + size_t(t) * kNodeBytes + 2 * D * 2,
                                                    32 * rb + il);
                            sm.W[t][il] = slot_f32<bf16_t>(sm.bg[0][t]) * fmaf(-G, acc[jt][nt][r], v);
                        } else {
                            sm.GR[t][il] = G * acc[jt][nt][r];
                        }
                    }
                }
        }
        wave_order();

        // ---- 4. per row: u by forward substitution in registers, then o -----------------
        if (lane < 32) {
            const int il = lane;
            float u[kC];
            float *orow = P.out + (crow * D) + 32 * rb + il;
#pragma unroll
            for (int t = 0; t < kC; ++t) {
                float tr[kC], cr[kC];
#pragma unroll
                for (int q4 = 0; q4 < kC / 4; ++q4) {
                    const float4 a = *reinterpret_cast<const float4 *>(&sm.Tm[t][4 * q4]);
                    const float4 b = *reinterpret_cast<const float4 *>(&sm.Cm[t][4 * q4]);
                    tr[4 * q4] = a.x, tr[4 * q4 + 1] = a.y, tr[4 * q4 + 2] = a.z, tr[4 * q4 + 3] = a.w;
                    cr[4 * q4] = b.x, cr[4 * q4 + 1] = b.y, cr[4 * q4 + 2] = b.z, cr[4 * q4 + 3] = b.w;
                }
                float x = sm.W[t][il];
#pragma unroll
                for (int sk = 0; sk < t; ++sk) x = fmaf(-tr[sk], u[sk], x);
                u[t] = t < nc ? x : 0.f;
                float o = sm.GR[t][il];
#pragma unroll
                for (int sk = 0; sk <= t; ++sk) o = fmaf(cr[sk], u[sk], o);
                if (t < nc) orow[int64_t(t) * P.H * D] = o;
                sm.Ug[t][il] = sm.gam[t] * u[t];
                __builtin_amdgcn_sched_barrier(0);  // keep the rows' loads from piling up
            }
        }
        wave_order();

        // ---- 5. S^T <- G S^T + K^T (gamma u) ------------------------------------------------
        // 16 independent accumulator tiles per k-step, so the matrix-core ops pipeline.
        {
            const float Ge = sm.G[nc - 1];
            floatx4 a4[2][8];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
                    a4[nt][mt] = floatx4{Ge * s[nt][mt][0], Ge * s[nt][mt][1], Ge * s[nt][mt][2],
                                         Ge * s[nt][mt][3]};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int t = 4 * ks + lg;  // k index of this lane
                float kv[8], uv[2];
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
                    kv[mt] = bf16_at(sm.in + size_t(t) * kNodeBytes, 16 * mt + lr);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) uv[nt] = sm.Ug[t][16 * nt + lr];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int mt = 0; mt < 8; ++mt)
                        a4[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[mt], uv[nt],
                                                                          a4[nt][mt], 0, 0, 0);
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[nt][mt][e] = a4[nt][mt][e];
        }
        wave_order();  // the next chunk's loads overwrite the inputs read above
    }

    if (len > 0) {
        float *tile = state + (32 * rb + lr) * D + 4 * lg;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                *reinterpret_cast<float4 *>(tile + 16 * nt * D + 16 * mt) =
                    make_float4(s[nt][mt][0], s[nt][mt][1], s[nt][mt][2], s[nt][mt][3]);
    }
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
    P.n_blocks = int64_t(a->n_layers) * a->n_seqs * a->n_heads * 4;
    if (P.n_blocks > kMaxBlocks) return fail(GDN_EINVAL, "gdn_prefill: too many workgroups");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (start == nullptr && stop == nullptr)
        hipLaunchKernelGGL(prefill_kernel, dim3(uint32_t(P.n_blocks)), dim3(64), 0, s, P);
    else
        hipExtLaunchKernelGGL(prefill_kernel, dim3(uint32_t(P.n_blocks)), dim3(64), 0, s, start,
                              stop, 0, P);
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
