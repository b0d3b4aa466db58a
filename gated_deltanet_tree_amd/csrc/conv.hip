// Tree-aware causal depthwise conv with the fused conv-window fold, for gfx950.
//
// "Luce DFlash server README", section "How it works": in tree verify each node's conv
// window is gathered along its parent chain, never in DFS order.  "Lucebox SpecLA and
// Gated DeltaNet state-resident verification" guide, mechanisms 1, 3 and 4: the conv window
// gets the same state-resident treatment as the recurrent state, the conv raw inputs are
// banked as accepted factors, and the next verify folds the pending ones into the
// committed window before using it.
//
// One thread per (layer, sequence, channel); consecutive threads take consecutive channels,
// so every access to x, the banks and the output is a coalesced row segment.  The thread
// keeps the committed window in registers, folds the pending bank rows (found through the
// pending row map) into it (only the last three can survive), writes it back once, then walks its tree in index order in blocks
// of nodes whose loads are all issued before any is used.  A node's window is read along its
// parent chain: the node's own input, up to three ancestors' inputs, then committed-window
// entries above the root.  Ancestor inputs were read moments earlier by the same thread, so
// they come from cache, not HBM.
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

#ifndef GDN_CONV_BLOCK
#define GDN_CONV_BLOCK 16  // nodes whose loads are issued together
#endif

template <typename TIn>
__global__ __launch_bounds__(256) void tree_conv_kernel(ConvParams P,
                                                        const int32_t *__restrict__ rows) {
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    const int seq = blockIdx.y;
    const int layer = P.layer_begin + blockIdx.z;
    if (c >= P.C) return;
    const int role = P.role[seq], L = min(max(P.pending[seq], 0), P.max_nodes);  // bank rows
    const int64_t ls = int64_t(layer) * P.S + seq;  // (layer, seq)
    float *cs = P.cstate + (ls * P.C + c) * 3;
    float w0 = cs[0], w1 = cs[1], w2 = cs[2];  // committed window, oldest first
    if (L > 0) {
        // Only the last three pending inputs survive the fold; the row map (uniform, scalar
        // loads) says where they sit in the bank, clamped to its rows.
        const int32_t *rm = rows + int64_t(seq) * P.max_nodes;
        const int m = P.max_nodes - 1;
        const int i0 = L >= 3 ? min(max(rm[L - 3], 0), m) : 0;
        const int i1 = L >= 2 ? min(max(rm[L - 2], 0), m) : 0;
        const int i2 = min(max(rm[L - 1], 0), m);
        const TIn *pb = static_cast<const TIn *>(P.bank[role]) + ls * P.max_nodes * P.C + c;
        const float r0 = L >= 3 ? to_f32(pb[int64_t(i0) * P.C]) : 0.f;
        const float r1 = L >= 2 ? to_f32(pb[int64_t(i1) * P.C]) : 0.f;
        const float r2 = to_f32(pb[int64_t(i2) * P.C]);
        if (L >= 3) {
            w0 = r0; w1 = r1; w2 = r2;
        } else if (L == 2) {
            w0 = w2; w1 = r1; w2 = r2;
        } else {
            w0 = w1; w1 = w2; w2 = r2;
        }
        cs[0] = w0;
        cs[1] = w1;
        cs[2] = w2;
    }
    if (P.fold_only) return;

    const TIn *wt = static_cast<const TIn *>(P.w) + (int64_t(layer) * P.C + c) * 4;
    const float k0 = to_f32(wt[0]), k1 = to_f32(wt[1]), k2 = to_f32(wt[2]), k3 = to_f32(wt[3]);
    const int off = P.img[P.off_seq + seq], n = P.img[P.off_seq + seq + 1] - off;
    const TIn *x = static_cast<const TIn *>(P.x) + int64_t(layer) * P.T * P.C + c;
    TIn *wb = static_cast<TIn *>(P.bank[role ^ 1]) + ls * P.max_nodes * P.C + c;
    float *y = P.out + int64_t(layer) * P.T * P.C + c;
    const int32_t *par = P.img + P.off_parent, *dep = P.img + P.off_depth;
    for (int i0 = 0; i0 < n; i0 += GDN_CONV_BLOCK) {
        // Issue every load of the block first: the node inputs and the up-to-three ancestor
        // inputs of each node (ancestors were read before, so they come from cache).
        float xv[GDN_CONV_BLOCK][4];
#pragma unroll
        for (int j = 0; j < GDN_CONV_BLOCK; ++j) {
            const int i = i0 + j;
            if (i >= n) break;
            const int g = off + i, depth = dep[g];
            const int a1 = depth >= 1 ? par[g] : g;
            const int a2 = depth >= 2 ? par[a1] : a1;
            const int a3 = depth >= 3 ? par[a2] : a2;
            xv[j][0] = to_f32(x[int64_t(g) * P.C]);
            xv[j][1] = to_f32(x[int64_t(a1) * P.C]);
            xv[j][2] = to_f32(x[int64_t(a2) * P.C]);
            xv[j][3] = to_f32(x[int64_t(a3) * P.C]);
        }
#pragma unroll
        for (int j = 0; j < GDN_CONV_BLOCK; ++j) {
            const int i = i0 + j;
            if (i >= n) break;
            const int depth = dep[off + i];
            // Taps one, two and three steps up the parent chain, else committed-window entries.
            const float x1 = depth >= 1 ? xv[j][1] : w2;
            const float x2 = depth >= 2 ? xv[j][2] : (depth == 1 ? w2 : w1);
            const float x3 = depth >= 3 ? xv[j][3] : (depth == 2 ? w2 : (depth == 1 ? w1 : w0));
            wb[int64_t(i) * P.C] = from_exact_f32<TIn>(xv[j][0]);  // the raw input, bit-exact
            y[int64_t(off + i) * P.C] = fmaf(k3, xv[j][0], fmaf(k2, x1, fmaf(k1, x2, k0 * x3)));
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

static gdn_status launch_conv(const ConvParams &P, int n_layers, int dtype, hipStream_t stream) {
    if (P.S == 0) return GDN_OK;
    dim3 grid((P.C + 255) / 256, P.S, n_layers);
    if (dtype == GDN_BF16)
        hipLaunchKernelGGL(tree_conv_kernel<bf16_t>, grid, dim3(256), 0, stream, P, P.rows);
    else
        hipLaunchKernelGGL(tree_conv_kernel<float>, grid, dim3(256), 0, stream, P, P.rows);
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
