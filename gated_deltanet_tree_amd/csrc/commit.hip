// Accept -> commit bookkeeping, factor-bank compaction and the flush, for gfx950.
//
// "Lucebox SpecLA and Gated DeltaNet state-resident verification" guide, mechanism 3: the
// two FP32 banks alternate between "pending" and "being written"; an accepted path that is
// already in order just swaps their roles (no device copy), a branched one is compacted
// back into path order by a gather kernel.  Mechanism 4: the flush materialises the last
// pending path once, at the end of generation, on a switch to autoregressive decode or on
// cancel.
//
// Readings: "in order" = the path is [0, 1, ..., L-1]; compaction writes rows 0..L-1 of the
// bank that the last verify consumed (the pending one) and leaves the roles as they are.
// The kernels re-derive the per-sequence decision from the device copy of the paths, so no
// host-to-device copy happens inside the library.  The conv-input bank keeps the raw inputs in
// their own dtype (exact, like an FP32 copy), so its rows are copied as raw bits.
//
// Every fold reads pending factor i from bank row pending_rows[b][i].  The guide's mode
// (compaction) keeps that map the identity.  The row-map mode never copies: the written bank
// always becomes pending and the map holds the accepted path itself.  A factor row is 512
// contiguous bytes per head at d = 128, so a gathered row costs the fold what a compacted one
// does, and the gather kernel's read + write of every branched row (all layers) disappears.
#include <algorithm>
#include <vector>

#include "gdn_device.h"

namespace gdn {

gdn_status flush_state(const gdn_verify_args *a, hipStream_t stream);
gdn_status flush_conv(const gdn_conv_args *a, hipStream_t stream);
gdn_status check_flush_verify_args(const gdn_verify_args *a);
gdn_status check_flush_conv_args(const gdn_conv_args *a);

struct CompactParams {
    float *bk[2], *bu[2], *blg[2];
    char *bx[2];  // conv-input banks, elements of xbytes bytes (the conv's input dtype)
    int32_t xbytes;
    const int32_t *role, *paths, *path_off;
    int32_t S, H, D, C, max_nodes, layer_begin;
};

__device__ __forceinline__ bool path_in_order(const int32_t *path, int L) {
    for (int i = 0; i < L; ++i)
        if (path[i] != i) return false;
    return true;
}

// One workgroup per (layer, sequence, path position i): row path[i] of the written bank ->
// row i of the pending bank, for the key and residual rows of every head (float4 copies),
// the log gates and the conv input row.  Workgroups past the path's end, or of a sequence
// whose path is in order, exit at once.
__global__ __launch_bounds__(256) void compact_kernel(CompactParams P) {
    const int i = blockIdx.x, seq = blockIdx.y;
    const int layer = P.layer_begin + blockIdx.z;
    const int beg = P.path_off[seq], L = P.path_off[seq + 1] - beg;
    if (i >= L) return;
    const int32_t *path = P.paths + beg;
    if (path_in_order(path, L)) return;
    const int dst = P.role[seq], src = dst ^ 1, from = path[i];
    const int64_t ls = int64_t(layer) * P.S + seq;
    const int64_t hrows = int64_t(P.H) * P.max_nodes;  // rows of one (layer, seq)
    const int tid = threadIdx.x;
    const int dv = P.D / 4;  // float4 per row
    for (int e = tid; e < P.H * dv; e += blockDim.x) {
        const int h = e / dv, q = e % dv;
        const int64_t rd = (ls * hrows + int64_t(h) * P.max_nodes + i) * P.D;
        const int64_t rs = (ls * hrows + int64_t(h) * P.max_nodes + from) * P.D;
        reinterpret_cast<float4 *>(P.bk[dst] + rd)[q] = reinterpret_cast<const float4 *>(P.bk[src] + rs)[q];
        reinterpret_cast<float4 *>(P.bu[dst] + rd)[q] = reinterpret_cast<const float4 *>(P.bu[src] + rs)[q];
    }
    for (int h = tid; h < P.H; h += blockDim.x)
        P.blg[dst][ls * hrows + int64_t(h) * P.max_nodes + i] =
            P.blg[src][ls * hrows + int64_t(h) * P.max_nodes + from];
    if (P.bx[0] != nullptr) {  // raw bit copy of the row, in 2-byte units (C x xbytes is even)
        const int64_t rb = int64_t(P.C) * P.xbytes;
        const uint16_t *xs = reinterpret_cast<const uint16_t *>(P.bx[src] + (ls * P.max_nodes + from) * rb);
        uint16_t *xd = reinterpret_cast<uint16_t *>(P.bx[dst] + (ls * P.max_nodes + i) * rb);
        for (int64_t c = tid; c < rb / 2; c += blockDim.x) xd[c] = xs[c];
    }
}

// Runs after compact_kernel on the same stream, one workgroup per sequence: the row map, the
// role flip (row-map mode: every non-empty path; compaction: in-order paths) and the pending
// length.
__global__ __launch_bounds__(64) void commit_bookkeeping_kernel(
    int32_t *role, int32_t *pending, int32_t *rows, const int32_t *paths, const int32_t *path_off,
    int max_nodes, int mode) {
    const int seq = blockIdx.x;
    const int beg = path_off[seq], L = path_off[seq + 1] - beg;
    int32_t *rm = rows + int64_t(seq) * max_nodes;
    for (int i = threadIdx.x; i < L; i += blockDim.x)
        rm[i] = mode == GDN_COMMIT_ROW_MAP ? paths[beg + i] : i;
    if (threadIdx.x == 0) {
        if (L > 0 && (mode == GDN_COMMIT_ROW_MAP || path_in_order(paths + beg, L)))
            role[seq] ^= 1;
        pending[seq] = L;
    }
}

__global__ void clear_pending_kernel(int32_t *pending, int S) {
    const int seq = blockIdx.x * blockDim.x + threadIdx.x;
    if (seq < S) pending[seq] = 0;
}

__global__ __launch_bounds__(256) void row_gather_kernel(const float *src, float *dst,
                                                         int64_t row_elems,
                                                         const int32_t *src_rows,
                                                         const int32_t *dst_rows) {
    const int r = blockIdx.y;
    const int64_t s = int64_t(src_rows[r]) * row_elems, d = int64_t(dst_rows[r]) * row_elems;
    for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < row_elems;
         e += int64_t(gridDim.x) * blockDim.x)
        dst[d + e] = src[s + e];
}

}  // namespace gdn

using namespace gdn;

extern "C" gdn_status gdn_commit_path(const int32_t *host_image, const int32_t *paths,
                                      const int32_t *path_offsets, const int32_t *dev_paths,
                                      const int32_t *dev_path_offsets,
                                      const gdn_verify_args *va, const gdn_conv_args *ca,
                                      int32_t *role_host, int32_t *pending_host, int32_t mode,
                                      void *stream) {
    clear_error();
    if (!image_ok(host_image) || !dev_path_offsets || !pending_host)
        return fail(GDN_EINVAL, "gdn_commit_path: null argument or malformed schedule image");
    if (va == nullptr) return fail(GDN_EINVAL, "gdn_commit_path: null verify args");
    gdn_status st = check_flush_verify_args(va);
    if (st != GDN_OK) return st;
    if (ca != nullptr) {
        st = check_flush_conv_args(ca);
        if (st != GDN_OK) return st;
        if (ca->role != va->role || ca->pending_len != va->pending_len ||
            ca->pending_rows != va->pending_rows || ca->n_seqs != va->n_seqs ||
            ca->layer_begin != va->layer_begin || ca->n_layers != va->n_layers ||
            ca->max_nodes != va->max_nodes)
            return fail(GDN_EINVAL, "gdn_commit_path: conv args disagree with verify args on "
                        "role/pending_len/pending_rows/n_seqs/layers/max_nodes");
    }
    const ImageView v = view_image(host_image);
    if (v.n_seqs != va->n_seqs)
        return fail(GDN_EINVAL, "gdn_commit_path: n_seqs differs from the schedule's");
    if (v.max_tree > va->max_nodes)
        return fail(GDN_ECAPACITY, "gdn_commit_path: max_nodes smaller than the largest tree");
    CommitPlan plan;
    st = plan_commit(host_image, paths, path_offsets, role_host, mode, plan);
    if (st != GDN_OK) return st;
    const int32_t S = v.n_seqs;
    if (S == 0) return GDN_OK;
    const bool any_compaction = plan.any_compaction, any_path = plan.any_path;
    const int32_t max_len = plan.max_len;
    if (S > 65535 || va->n_layers > 65535)
        return fail(GDN_EINVAL, "gdn_commit_path: n_seqs and n_layers must be <= 65535");
    if (any_path && dev_paths == nullptr)
        return fail(GDN_EINVAL, "gdn_commit_path: null dev_paths");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (any_compaction) {
        CompactParams P{};
        for (int i = 0; i < 2; ++i) {
            P.bk[i] = va->bank_k[i];
            P.bu[i] = va->bank_u[i];
            P.blg[i] = va->bank_lg[i];
            P.bx[i] = ca ? static_cast<char *>(ca->bank_x[i]) : nullptr;
        }
        P.role = va->role;
        P.paths = dev_paths;
        P.path_off = dev_path_offsets;
        P.S = S;
        P.H = va->n_heads;
        P.D = va->head_dim;
        P.C = ca ? ca->channels : 0;
        P.xbytes = ca && ca->in_dtype == GDN_BF16 ? 2 : 4;
        P.max_nodes = va->max_nodes;
        P.layer_begin = va->layer_begin;
        hipLaunchKernelGGL(compact_kernel, dim3(max_len, S, va->n_layers), dim3(256), 0, s, P);
        GDN_LAUNCH_CHECK("compact_kernel");
    }
    hipLaunchKernelGGL(commit_bookkeeping_kernel, dim3(S), dim3(64), 0, s,
                       const_cast<int32_t *>(va->role), const_cast<int32_t *>(va->pending_len),
                       const_cast<int32_t *>(va->pending_rows), dev_paths, dev_path_offsets,
                       va->max_nodes, mode);
    GDN_LAUNCH_CHECK("commit_bookkeeping_kernel");
    for (int32_t b = 0; b < S; ++b) {
        role_host[b] = plan.role[size_t(b)];
        pending_host[b] = plan.pending[size_t(b)];
    }
    return GDN_OK;
}

extern "C" gdn_status gdn_compact_factors(const float *src, float *dst, int64_t row_elems,
                                          const int32_t *src_rows, const int32_t *dst_rows,
                                          int32_t n_rows, void *stream) {
    clear_error();
    if (n_rows < 0 || row_elems < 0) return fail(GDN_EINVAL, "gdn_compact_factors: negative size");
    if (n_rows == 0 || row_elems == 0) return GDN_OK;
    if (!src || !dst || !src_rows || !dst_rows)
        return fail(GDN_EINVAL, "gdn_compact_factors: null pointer");
    if (n_rows > 65535) return fail(GDN_EINVAL, "gdn_compact_factors: n_rows > 65535");
    if (src == dst) return fail(GDN_EINVAL, "gdn_compact_factors: src and dst must differ");
    const int64_t blocks = std::min<int64_t>((row_elems + 255) / 256, 1024);
    hipLaunchKernelGGL(row_gather_kernel, dim3(uint32_t(blocks), n_rows), dim3(256), 0,
                       static_cast<hipStream_t>(stream), src, dst, row_elems, src_rows, dst_rows);
    GDN_LAUNCH_CHECK("row_gather_kernel");
    return GDN_OK;
}

extern "C" gdn_status gdn_flush(const gdn_verify_args *va, const gdn_conv_args *ca,
                                int32_t *pending_host, void *stream) {
    clear_error();
    gdn_status st = check_flush_verify_args(va);
    if (st != GDN_OK) return st;
    if (ca != nullptr) {
        st = check_flush_conv_args(ca);
        if (st != GDN_OK) return st;
        if (ca->role != va->role || ca->pending_len != va->pending_len ||
            ca->pending_rows != va->pending_rows || ca->n_seqs != va->n_seqs ||
            ca->layer_begin != va->layer_begin || ca->n_layers != va->n_layers ||
            ca->max_nodes != va->max_nodes)
            return fail(GDN_EINVAL, "gdn_flush: conv args disagree with verify args");
    }
    if (pending_host == nullptr) return fail(GDN_EINVAL, "gdn_flush: null pending_host");
    const int32_t S = va->n_seqs;
    if (S == 0) return GDN_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = flush_state(va, s);
    if (st != GDN_OK) return st;
    if (ca != nullptr) {
        st = flush_conv(ca, s);
        if (st != GDN_OK) return st;
    }
    hipLaunchKernelGGL(clear_pending_kernel, dim3((S + 255) / 256), dim3(256), 0, s,
                       const_cast<int32_t *>(va->pending_len), S);
    GDN_LAUNCH_CHECK("clear_pending_kernel");
    for (int32_t b = 0; b < S; ++b) pending_host[b] = 0;
    return GDN_OK;
}
