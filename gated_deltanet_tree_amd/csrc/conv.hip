// Tree-aware causal depthwise conv with the fused conv-window fold, for gfx950.
//
// "Luce DFlash server README", section "How it works": in tree verify each node's conv
// window is gathered along its parent chain, never in DFS order.  "Lucebox SpecLA and
// Gated DeltaNet state-resident verification" guide, mechanisms 1, 3 and 4: the conv window
// gets the same state-resident treatment as the recurrent state, the conv raw inputs are
// banked as accepted factors, and the next verify folds the pending ones into the
// committed window before using it.
//
// One thread per (layer, sequence, pair of adjacent channels); consecutive threads take
// consecutive pairs, so every access to x, the banks and the output is a coalesced row segment
// of 4 or 8 bytes per lane.  The thread keeps the committed window in registers, folds the
// pending bank rows (found through the pending row map) into it (only the last three can
// survive) and writes it back once.  The workgroup then tables, 64 nodes at a time, each node's
// global id and its three nearest ancestors' (one lane per node walks the parent links once),
// and every thread walks the table in blocks of nodes whose loads are all issued before any is
// used.  A node's window is read along its parent chain: the node's own input, up to three
// ancestors' inputs, then committed-window entries above the root.  Ancestor inputs were read
// moments earlier by the same thread, so they come from cache, not HBM.
#include "gdn_device.h"

namespace gdn {

struct ConvParams {
    const void *x, *w;
    float *cstate;
    void *bank[2];  // raw conv inputs, in the input dtype
    const int32_t *role, *pending;
    const int32_t *rows;  // [S][max_nodes] pending row map
    float *out;
    const int32_t *img;
    int64_t off_seq, off_parent, off_depth;
    int32_t S, C, T, max_nodes, layer_begin;
    int32_t fold_only;
};

// Three waves: a layer of 32 sequences x 18 432 channels (pairs per thread) is 1 536 workgroups,
// six per CU; four waves made 1 152, so half the CUs carried one workgroup more than the rest.
constexpr int kConvThreads = 192;
constexpr int kTapBlock = 64;  // nodes tabled per pass of the workgroup
constexpr int kConvSub = 8;    // nodes whose loads are issued together

// CPT adjacent channels of one element type, loaded and stored as one unit.
template <typename T, int CPT> struct ChanVec;
template <> struct ChanVec<bf16_t, 1> {
    typedef bf16_t raw;
    static __device__ float get(raw v, int) { return to_f32<bf16_t>(v); }
};
template <> struct ChanVec<float, 1> {
    typedef float raw;
    static __device__ float get(raw v, int) { return v; }
};
template <> struct ChanVec<bf16_t, 2> {
    typedef uint32_t raw;  // two bf16, channel c in the low half
    static __device__ float get(raw v, int e) { return __uint_as_float(e ? v & 0xFFFF0000u : v << 16); }
};
template <> struct ChanVec<float, 2> {
    typedef float2 raw;
    static __device__ float get(raw v, int e) { return e ? v.y : v.x; }
};

template <typename TIn, int CPT>
__global__ __launch_bounds__(kConvThreads) void tree_conv_kernel(ConvParams P,
                                                                 const int32_t *__restrict__ rows) {
    typedef ChanVec<TIn, CPT> CV;
    typedef typename CV::raw RawT;
    __shared__ int4 taps[kTapBlock];  // a node's global id and its ancestors' at distance 1..3
    __shared__ int deps[kTapBlock], pars[kTapBlock];
    const int c = (blockIdx.x * kConvThreads + threadIdx.x) * CPT;  // first channel
    const bool active = c < P.C;  // CPT divides C: all CPT channels exist
    const int seq = blockIdx.y;
    const int layer = P.layer_begin + blockIdx.z;
    const int role = P.role[seq], L = min(max(P.pending[seq], 0), P.max_nodes);  // bank rows
    const int64_t ls = int64_t(layer) * P.S + seq;  // (layer, seq)
    // The first table block's parent links and depths go out ahead of the window fold.  A
    // fold-only launch (flush) has no schedule image and touches none of it.
    int off = 0, n = 0, my_par = 0, my_dep = 0;
    const int32_t *par = nullptr, *dep = nullptr;
    if (!P.fold_only) {
        off = P.img[P.off_seq + seq];
        n = P.img[P.off_seq + seq + 1] - off;
        par = P.img + P.off_parent;
        dep = P.img + P.off_depth;
        if (int(threadIdx.x) < min(kTapBlock, n)) {
            my_par = par[off + threadIdx.x];
            my_dep = dep[off + threadIdx.x];
        }
    }
    float w0[CPT], w1[CPT], w2[CPT];  // committed window, oldest first
    if (active) {
        float *cs = P.cstate + (ls * P.C + c) * 3;
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            w0[e] = cs[3 * e];
            w1[e] = cs[3 * e + 1];
            w2[e] = cs[3 * e + 2];
        }
        if (L > 0) {
            // Only the last three pending inputs survive the fold; the row map (uniform, scalar
            // loads) says where they sit in the bank, clamped to its rows.
            const int32_t *rm = rows + int64_t(seq) * P.max_nodes;
            const int m = P.max_nodes - 1;
            const int i0 = L >= 3 ? min(max(rm[L - 3], 0), m) : 0;
            const int i1 = L >= 2 ? min(max(rm[L - 2], 0), m) : 0;
            const int i2 = min(max(rm[L - 1], 0), m);
            const TIn *pb = static_cast<const TIn *>(P.bank[role]) + ls * P.max_nodes * P.C + c;
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                const float r0 = L >= 3 ? to_f32(pb[int64_t(i0) * P.C + e]) : 0.f;
                const float r1 = L >= 2 ? to_f32(pb[int64_t(i1) * P.C + e]) : 0.f;
                const float r2 = to_f32(pb[int64_t(i2) * P.C + e]);
                if (L >= 3) {
                    w0[e] = r0; w1[e] = r1; w2[e] = r2;
                } else if (L == 2) {
                    w0[e] = w2[e]; w1[e] = r1; w2[e] = r2;
                } else {
                    w0[e] = w1[e]; w1[e] = w2[e]; w2[e] = r2;
                }
                cs[3 * e] = w0[e];
                cs[3 * e + 1] = w1[e];
                cs[3 * e + 2] = w2[e];
            }
        }
    }
    if (P.fold_only) return;  // a kernel argument: the whole grid returns here

    float k0[CPT], k1[CPT], k2[CPT], k3[CPT];
    const TIn *x = static_cast<const TIn *>(P.x) + int64_t(layer) * P.T * P.C + c;
    TIn *wb = static_cast<TIn *>(P.bank[role ^ 1]) + ls * P.max_nodes * P.C + c;
    float *y = P.out + int64_t(layer) * P.T * P.C + c;
    if (active) {
        const TIn *wt = static_cast<const TIn *>(P.w) + (int64_t(layer) * P.C + c) * 4;
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            k0[e] = to_f32(wt[4 * e]);
            k1[e] = to_f32(wt[4 * e + 1]);
            k2[e] = to_f32(wt[4 * e + 2]);
            k3[e] = to_f32(wt[4 * e + 3]);
        }
    }
    for (int b0 = 0; b0 < n; b0 += kTapBlock) {
        const int nb = min(kTapBlock, n - b0), base = off + b0;
        const int t = threadIdx.x;
        if (b0 > 0 && t < nb) {
            my_par = par[base + t];
            my_dep = dep[base + t];
        }
        __syncthreads();  // the previous block's table is consumed
        if (t < nb) {
            pars[t] = my_par;
            deps[t] = my_dep;
        }
        __syncthreads();
        if (t < nb) {  // ancestors inside the block from LDS, others from the image
            const int g = base + t, d = my_dep;
            auto parent = [&](int a) {
                return unsigned(a - base) < unsigned(nb) ? pars[a - base] : par[a];
            };
            const int a1 = d >= 1 ? my_par : g;
            const int a2 = d >= 2 ? parent(a1) : a1;
            const int a3 = d >= 3 ? parent(a2) : a2;
            taps[t] = make_int4(g, a1, a2, a3);
        }
        __syncthreads();
        if (!active) continue;
        for (int j0 = 0; j0 < nb; j0 += kConvSub) {
            RawT xv[kConvSub][4];
#pragma unroll
            for (int j = 0; j < kConvSub; ++j) {
                if (j0 + j >= nb) break;
                const int4 tp = taps[j0 + j];
                xv[j][0] = *reinterpret_cast<const RawT *>(x + int64_t(tp.x) * P.C);
                xv[j][1] = *reinterpret_cast<const RawT *>(x + int64_t(tp.y) * P.C);
                xv[j][2] = *reinterpret_cast<const RawT *>(x + int64_t(tp.z) * P.C);
                xv[j][3] = *reinterpret_cast<const RawT *>(x + int64_t(tp.w) * P.C);
            }
#pragma unroll
            for (int j = 0; j < kConvSub; ++j) {
                const int i = b0 + j0 + j;
                if (j0 + j >= nb) break;
                const int depth = deps[j0 + j];
                *reinterpret_cast<RawT *>(wb + int64_t(i) * P.C) = xv[j][0];  // raw, bit-exact
                float yv[CPT];
#pragma unroll
                for (int e = 0; e < CPT; ++e) {
                    // Taps one, two and three steps up the parent chain, else window entries.
                    const float x0 = CV::get(xv[j][0], e);
                    const float x1 = depth >= 1 ? CV::get(xv[j][1], e) : w2[e];
                    const float x2 = depth >= 2 ? CV::get(xv[j][2], e) : (depth == 1 ? w2[e] : w1[e]);
                    const float x3 = depth >= 3 ? CV::get(xv[j][3], e)
                                                : (depth == 2 ? w2[e] : (depth == 1 ? w1[e] : w0[e]));
                    yv[e] = fmaf(k3[e], x0, fmaf(k2[e], x1, fmaf(k1[e], x2, k0[e] * x3)));
                }
                float *yo = y + int64_t(off + i) * P.C;
                if constexpr (CPT == 2)
                    *reinterpret_cast<float2 *>(yo) = make_float2(yv[0], yv[1]);
                else
                    *yo = yv[0];
            }
        }
    }
}

static gdn_status check_conv_args(const gdn_conv_args *a, bool need_inputs) {
    if (a == nullptr) return fail(GDN_EINVAL, "conv args: null");
    if (a->width != 4) return fail(GDN_EINVAL, "conv args: width %d, only 4 supported", a->width);
    if (a->channels < 1 || a->n_layers < 1 || a->layer_begin < 0 || a->n_seqs < 0 ||
        a->max_nodes < 1)
        return fail(GDN_EINVAL, "conv args: bad channels/n_layers/layer_begin/n_seqs/max_nodes");
    if (a->in_dtype != GDN_F32 && a->in_dtype != GDN_BF16)
        return fail(GDN_EINVAL, "conv args: in_dtype %d", a->in_dtype);
    if (a->n_seqs == 0) return GDN_OK;  // empty batch: nothing is read or written
    if (!a->conv_state || !a->bank_x[0] || !a->bank_x[1] || !a->role || !a->pending_len ||
        !a->pending_rows)
        return fail(GDN_EINVAL, "conv args: null conv_state/bank/role/pending_len/pending_rows");
    if (need_inputs && (!a->x || !a->weight || !a->out))
        return fail(GDN_EINVAL, "conv args: null x/weight/out");
    if (a->n_seqs > 65535 || a->n_layers > 65535)
        return fail(GDN_EINVAL, "conv args: n_seqs and n_layers must be <= 65535");
    return GDN_OK;
}

// Two channels per thread when the channel count is even and every row the kernel touches
// (x, the banks, the output, the weights, the window) starts on a pair boundary; one otherwise.
static bool pairs_aligned(const ConvParams &P, int dtype) {
    if (P.C % 2 != 0) return false;
    const uintptr_t a = dtype == GDN_BF16 ? 4 : 8;
    const void *ptrs[] = {P.x, P.w, P.bank[0], P.bank[1], P.out};
    for (const void *p : ptrs)
        if (p != nullptr && reinterpret_cast<uintptr_t>(p) % a != 0) return false;
    return reinterpret_cast<uintptr_t>(P.out) % 8 == 0;
}

template <typename TIn, int CPT>
static void launch_conv_t(const ConvParams &P, int n_layers, hipStream_t stream) {
    const int threads = (P.C + CPT - 1) / CPT;
    dim3 grid((threads + kConvThreads - 1) / kConvThreads, P.S, n_layers);
    hipLaunchKernelGGL((tree_conv_kernel<TIn, CPT>), grid, dim3(kConvThreads), 0, stream, P,
                       P.rows);
}

static gdn_status launch_conv(const ConvParams &P, int n_layers, int dtype, hipStream_t stream) {
    if (P.S == 0) return GDN_OK;
    const bool two = pairs_aligned(P, dtype);
    if (dtype == GDN_BF16)
        two ? launch_conv_t<bf16_t, 2>(P, n_layers, stream) : launch_conv_t<bf16_t, 1>(P, n_layers, stream);
    else
        two ? launch_conv_t<float, 2>(P, n_layers, stream) : launch_conv_t<float, 1>(P, n_layers, stream);
    GDN_LAUNCH_CHECK("tree_conv_kernel");
    return GDN_OK;
}

static ConvParams conv_params(const gdn_conv_args *a) {
    ConvParams P{};
    P.x = a->x;
    P.w = a->weight;
    P.cstate = a->conv_state;
    P.bank[0] = a->bank_x[0];
    P.bank[1] = a->bank_x[1];
    P.role = a->role;
    P.pending = a->pending_len;
    P.rows = a->pending_rows;
    P.out = a->out;
    P.S = a->n_seqs;
    P.C = a->channels;
    P.T = a->n_nodes;
    P.max_nodes = a->max_nodes;
    P.layer_begin = a->layer_begin;
    return P;
}

gdn_status flush_conv(const gdn_conv_args *a, hipStream_t stream) {
    gdn_status st = check_conv_args(a, false);
    if (st != GDN_OK) return st;
    ConvParams P = conv_params(a);
    P.fold_only = 1;
    return launch_conv(P, a->n_layers, a->in_dtype, stream);
}

gdn_status check_flush_conv_args(const gdn_conv_args *a) { return check_conv_args(a, false); }

}  // namespace gdn

using namespace gdn;

extern "C" gdn_status gdn_tree_conv(const gdn_conv_args *a, const int32_t *host_image,
                                    const int32_t *dev_image, void *stream) {
    clear_error();
    gdn_status st = check_conv_args(a, true);
    if (st != GDN_OK) return st;
    if (!image_ok(host_image) || dev_image == nullptr)
        return fail(GDN_EINVAL, "gdn_tree_conv: missing or malformed schedule image");
    const ImageView v = view_image(host_image);
    if (v.n_seqs != a->n_seqs || v.n_nodes != a->n_nodes)
        return fail(GDN_EINVAL, "gdn_tree_conv: n_seqs/n_nodes differ from the schedule's");
    if (v.max_tree > a->max_nodes)
        return fail(GDN_ECAPACITY, "gdn_tree_conv: max_nodes %d < largest tree %d", a->max_nodes,
                    v.max_tree);
    ConvParams P = conv_params(a);
    P.img = dev_image;
    P.off_seq = v.off_seq;
    P.off_parent = v.off_parent;
    P.off_depth = v.off_depth;
    return launch_conv(P, a->n_layers, a->in_dtype, static_cast<hipStream_t>(stream));
}
