// Chain-resident tree verify of the gated delta rule with the fused deferred commit, and the
// fold-only flush, for gfx950.
//
// "Lucebox SpecLA and Gated DeltaNet state-resident verification" guide:
//   mechanism 1 -- the nodes of one verify chain run back to back inside one workgroup with
//     the recurrent state tile held on chip; the tile is read once at the chain head;
//   mechanism 2 -- chains come from the heavy-light schedule; only boundary states are
//     written out, for the light chains of the next dependency wave;
//   mechanism 3 -- per node the key, the residual update vector u and ln g are banked;
//   mechanism 4 -- the root chain first folds the previous step's pending factors into the
//     committed state, writes it back once and verifies on the same live tile.
//
// Per node, with S the live tile (rows = d_v, columns = d_k):
//   a = S k, b = S q                      (one pass over the tile, octet reductions)
//   u = beta (v - g a)                    residual update vector
//   S <- g S + u k^T                      = g S (I - beta k k^T) + beta v k^T
//   o = g b + u (k . q)                   = S_new q, no second pass over the tile
// Fold of a pending row: S <- exp(lg) S + u k^T.
//
// Lane layout (d = 128: 4 waves, 256 threads).  Wave w owns rows [32w, 32w+32); lane l has
// row group rg = l/8 and column lane cl = l%8; it holds rows 32w + rg + 8m (m < 4) and the
// columns 32p + 4cl + e (p < 4, e < 4): 64 fp32 values.  A global float4 access of one
// (m, p) pair covers 8 rows x 128 contiguous bytes, so tile loads and stores are coalesced,
// and every row's 128 columns sit in one lane octet, so S k and S q need only an 8-lane DPP
// reduction -- no LDS round trip and no barrier for the matrix-vector products.
// d = 16: one wave, 2 rows x 2 columns per lane, same octet structure.
//
// Node inputs (k, q, v, beta, g) and fold rows (k, u, lg) are staged through a double-
// buffered LDS slot: the loads for item i+1 are issued before item i is computed and land
// in the other slot afterwards, so their latency hides behind a node of work.
#include "gdn_device.h"

namespace gdn {

struct VerifyParams {
    const void *q, *k, *v, *beta, *gate;
    float *state;
    float *bank_k[2], *bank_u[2], *bank_lg[2];
    const int32_t *role, *pending;
    float *boundary;
    float *out;
    const int32_t *img;
    int64_t off_seq, off_chain, off_cnodes, off_cseq, off_csrc, off_store;
    int32_t S, H, T, max_nodes, n_boundaries, layer_begin;
    int32_t chain_begin, n_chains;  // chains of this wave
    int64_t n_blocks;
    int32_t fold_only;  // flush: one workgroup per (layer, seq, head), fold + store only
};

template <int D> struct Tile {
    static constexpr int RW = D >= 32 ? 32 : D;       // rows per wave
    static constexpr int NW = D / RW;                 // waves per workgroup
    static constexpr int THREADS = 64 * NW;
    static constexpr int M = RW / 8;                  // rows per lane
    static constexpr int COLS = D / 8;                // columns per lane
    static constexpr int VEC = COLS >= 4 ? 4 : COLS;  // contiguous columns per access
    static constexpr int NP = COLS / VEC;             // column groups per lane
    static constexpr int SLOT = 3 * D + 2;            // LDS floats per staged item
    static_assert(D % 16 == 0 && RW % 8 == 0, "unsupported head dim");
};

template <int VEC> struct VecT;
template <> struct VecT<4> {
    typedef float4 type;
    static __device__ __forceinline__ void get(const float *p, float *o) {
        float4 t = *reinterpret_cast<const float4 *>(p);
        o[0] = t.x; o[1] = t.y; o[2] = t.z; o[3] = t.w;
    }
    static __device__ __forceinline__ void put(float *p, const float *o) {
        *reinterpret_cast<float4 *>(p) = make_float4(o[0], o[1], o[2], o[3]);
    }
};
template <> struct VecT<2> {
    typedef float2 type;
    static __device__ __forceinline__ void get(const float *p, float *o) {
        float2 t = *reinterpret_cast<const float2 *>(p);
        o[0] = t.x; o[1] = t.y;
    }
    static __device__ __forceinline__ void put(float *p, const float *o) {
        *reinterpret_cast<float2 *>(p) = make_float2(o[0], o[1]);
    }
};

// One thread's share of a staged item: an 8-byte chunk or a scalar, and where it goes.
struct Staged {
    uint2 raw;
    int dst;   // float index in the LDS slot, -1 = nothing
    int mode;  // 0: 2 x f32, 1: 4 x bf16, 2: f32 scalar, 3: bf16 scalar
};

template <int D, typename TIn>
__device__ __forceinline__ Staged stage_node(const VerifyParams &P, int64_t row, int tid) {
    // row = (layer * T + node) * H + head
    constexpr int PER = 8 / sizeof(TIn);  // elements per 8-byte chunk
    constexpr int CPV = D / PER;          // chunks per vector
    Staged s;
    s.dst = -1;
    s.mode = 0;
    s.raw = make_uint2(0, 0);
    if (tid < 3 * CPV) {
        const int vec = tid / CPV, idx = tid % CPV;
        const void *base = vec == 0 ? P.k : (vec == 1 ? P.q : P.v);
        const uint2 *src = reinterpret_cast<const uint2 *>(
            static_cast<const TIn *>(base) + row * D) + idx;
        s.raw = *src;
        s.dst = vec * D + idx * PER;
        s.mode = sizeof(TIn) == 2 ? 1 : 0;
    } else if (tid < 3 * CPV + 2) {
        const void *base = tid == 3 * CPV ? P.beta : P.gate;
        if (sizeof(TIn) == 2) {
            s.raw.x = static_cast<const bf16_t *>(base)[row];
            s.mode = 3;
        } else {
            s.raw.x = __float_as_uint(static_cast<const float *>(base)[row]);
            s.mode = 2;
        }
        s.dst = 3 * D + (tid - 3 * CPV);
    }
    return s;
}

template <int D>
__device__ __forceinline__ Staged stage_fold(const float *bk, const float *bu, const float *blg,
                                             int64_t rowv, int64_t rows, int tid) {
    // rowv = element offset of the bank row's vector, rows = index into the lg bank
    constexpr int CPV = D / 2;
    Staged s;
    s.dst = -1;
    s.mode = 0;
    s.raw = make_uint2(0, 0);
    if (tid < 2 * CPV) {
        const int which = tid / CPV, idx = tid % CPV;
        const float *base = (which == 0 ? bk : bu) + rowv;
        s.raw = reinterpret_cast<const uint2 *>(base)[idx];
        s.dst = (which == 0 ? 0 : 2 * D) + idx * 2;
    } else if (tid == 2 * CPV) {
        s.raw.x = __float_as_uint(blg[rows]);
        s.mode = 2;
        s.dst = 3 * D;
    }
    return s;
}

__device__ __forceinline__ void commit_stage(const Staged &s, float *slot) {
    if (s.dst < 0) return;
    switch (s.mode) {
    case 0:
        *reinterpret_cast<float2 *>(slot + s.dst) =
            make_float2(__uint_as_float(s.raw.x), __uint_as_float(s.raw.y));
        break;
    case 1:
        *reinterpret_cast<float4 *>(slot + s.dst) = make_float4(
            bf16_lo(s.raw.x), bf16_hi(s.raw.x), bf16_lo(s.raw.y), bf16_hi(s.raw.y));
        break;
    case 2: slot[s.dst] = __uint_as_float(s.raw.x); break;
    default: slot[s.dst] = bf16_lo(s.raw.x); break;
    }
}

template <int D, typename TIn>
__global__ __launch_bounds__(Tile<D>::THREADS) void verify_chain_kernel(VerifyParams P) {
    using TL = Tile<D>;
    constexpr int M = TL::M, NP = TL::NP, VEC = TL::VEC;
    typedef VecT<VEC> V;
    __shared__ __align__(16) float lds[2][TL::SLOT + 2];

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int rg = lane >> 3, cl = lane & 7;
    const int64_t logical = xcd_logical(blockIdx.x, P.n_blocks);

    int layer_rel, seq, h, chain = -1;
    if (P.fold_only) {
        const int64_t per = int64_t(P.S) * P.H;
        layer_rel = int(logical / per);
        const int64_t rem = logical % per;
        seq = int(rem / P.H);
        h = int(rem % P.H);
    } else {
        const int64_t per = int64_t(P.n_chains) * P.H;
        layer_rel = int(logical / per);
        const int64_t rem = logical % per;
        h = int(rem / P.n_chains);
        chain = P.chain_begin + int(rem % P.n_chains);
        seq = P.img[P.off_cseq + chain];
    }
    const int layer = P.layer_begin + layer_rel;
    const int src = P.fold_only ? -1 : P.img[P.off_csrc + chain];
    const int nbeg = P.fold_only ? 0 : P.img[P.off_chain + chain];
    const int nend = P.fold_only ? 0 : P.img[P.off_chain + chain + 1];
    const int seq_off = P.fold_only ? 0 : P.img[P.off_seq + seq];
    const int role = P.role[seq];
    const int L = src < 0 ? P.pending[seq] : 0;
    const int n_items = L + (nend - nbeg);
    if (n_items == 0) return;  // flush of a sequence with nothing pending

    const int64_t sh = (int64_t(layer) * P.S + seq) * P.H + h;  // (layer, seq, head)
    float *committed = P.state + sh * D * D;
    const float *start = src < 0 ? committed
        : P.boundary + ((int64_t(layer_rel) * P.n_boundaries + src) * P.H + h) * D * D;
    const float *pk = P.bank_k[role], *pu = P.bank_u[role], *plg = P.bank_lg[role];
    float *wk = P.bank_k[role ^ 1], *wu = P.bank_u[role ^ 1], *wlg = P.bank_lg[role ^ 1];
    const int64_t bank_row0 = sh * P.max_nodes;  // row index of (layer, seq, head, 0)

    int rows[M];
#pragma unroll
    for (int m = 0; m < M; ++m) rows[m] = w * TL::RW + rg + 8 * m;
    int cols[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) cols[p] = p * 8 * VEC + cl * VEC;

    // Stage item 0 and load the start tile.
    auto stage_item = [&](int it) -> Staged {
        if (it < L)
            return stage_fold<D>(pk, pu, plg, (bank_row0 + it) * D, bank_row0 + it, tid);
        const int node = P.img[P.off_cnodes + nbeg + (it - L)];
        return stage_node<D, TIn>(P, (int64_t(layer) * P.T + node) * P.H + h, tid);
    };
    Staged pending_stage = stage_item(0);

    float s[M][NP][VEC];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int p = 0; p < NP; ++p) V::get(start + rows[m] * D + cols[p], s[m][p]);

    commit_stage(pending_stage, lds[0]);
    __syncthreads();

    for (int it = 0; it < n_items; ++it) {
        const float *slot = lds[it & 1];
        const bool more = it + 1 < n_items;
        if (more) pending_stage = stage_item(it + 1);

        if (it < L) {
            // Deferred commit: S <- exp(lg) S + u k^T with a pending bank row.
            const float gl = expf(slot[3 * D]);
            float u[M];
#pragma unroll
            for (int m = 0; m < M; ++m) u[m] = slot[2 * D + rows[m]];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                float kc[VEC];
                V::get(slot + cols[p], kc);
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) s[m][p][e] = fmaf(u[m], kc[e], gl * s[m][p][e]);
            }
            if (it == L - 1) {  // the committed state is written back exactly once
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int p = 0; p < NP; ++p) V::put(committed + rows[m] * D + cols[p], s[m][p]);
            }
        } else {
            const int node = P.img[P.off_cnodes + nbeg + (it - L)];
            float a[M], b[M], kq = 0.f;
#pragma unroll
            for (int m = 0; m < M; ++m) a[m] = b[m] = 0.f;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                float kc[VEC], qc[VEC];
                V::get(slot + cols[p], kc);
                V::get(slot + D + cols[p], qc);
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
            const float beta = slot[3 * D], g = slot[3 * D + 1];
            float u[M], o[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                u[m] = beta * (slot[2 * D + rows[m]] - g * a[m]);
                o[m] = fmaf(u[m], kq, g * b[m]);
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                float kc[VEC];
                V::get(slot + cols[p], kc);
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) s[m][p][e] = fmaf(u[m], kc[e], g * s[m][p][e]);
            }

            // Outputs and factors: lane cl == m of each octet writes row m's o and u.
            const int local = node - seq_off;
            float *orow = P.out + ((int64_t(layer) * P.T + node) * P.H + h) * D;
            float *urow = wu + (bank_row0 + local) * D;
#pragma unroll
            for (int m = 0; m < M; ++m)
                if (cl == m) {
                    orow[rows[m]] = o[m];
                    urow[rows[m]] = u[m];
                }
            if (w == 0 && rg == 0) {
                float *krow = wk + (bank_row0 + local) * D;
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    float kc[VEC];
                    V::get(slot + cols[p], kc);
                    V::put(krow + cols[p], kc);
                }
            }
            if (tid == 0) wlg[bank_row0 + local] = logf(g);

            const int slot_id = P.img[P.off_store + node];
            if (slot_id >= 0) {  // boundary node: its state seeds later light chains
                float *dst = P.boundary +
                    ((int64_t(layer_rel) * P.n_boundaries + slot_id) * P.H + h) * D * D;
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int p = 0; p < NP; ++p) V::put(dst + rows[m] * D + cols[p], s[m][p]);
            }
        }

        if (more) commit_stage(pending_stage, lds[(it + 1) & 1]);
        __syncthreads();
    }
}

template <int D, typename TIn>
static gdn_status launch_verify(const VerifyParams &P, hipStream_t stream) {
    if (P.n_blocks <= 0) return GDN_OK;
    hipLaunchKernelGGL((verify_chain_kernel<D, TIn>), dim3(uint32_t(P.n_blocks)),
                       dim3(Tile<D>::THREADS), 0, stream, P);
    GDN_LAUNCH_CHECK("verify_chain_kernel");
    return GDN_OK;
}

static gdn_status dispatch_verify(const VerifyParams &P, int d, int dtype, hipStream_t stream) {
    if (d == 128)
        return dtype == GDN_BF16 ? launch_verify<128, bf16_t>(P, stream)
                                 : launch_verify<128, float>(P, stream);
    return dtype == GDN_BF16 ? launch_verify<16, bf16_t>(P, stream)
                             : launch_verify<16, float>(P, stream);
}

static gdn_status check_verify_args(const gdn_verify_args *a, bool need_schedule_inputs) {
    if (a == nullptr) return fail(GDN_EINVAL, "verify args: null");
    if (a->head_dim != 16 && a->head_dim != 128)
        return fail(GDN_EINVAL, "verify args: head_dim %d not in {16, 128}", a->head_dim);
    if (a->n_heads < 1 || a->n_layers < 1 || a->layer_begin < 0 || a->n_seqs < 0 ||
        a->max_nodes < 1)
        return fail(GDN_EINVAL, "verify args: bad n_heads/n_layers/layer_begin/n_seqs/max_nodes");
    if (a->in_dtype != GDN_F32 && a->in_dtype != GDN_BF16)
        return fail(GDN_EINVAL, "verify args: in_dtype %d", a->in_dtype);
    if (!a->state || !a->role || !a->pending_len)
        return fail(GDN_EINVAL, "verify args: null state/role/pending_len");
    for (int i = 0; i < 2; ++i)
        if (!a->bank_k[i] || !a->bank_u[i] || !a->bank_lg[i])
            return fail(GDN_EINVAL, "verify args: null bank pointer");
    if (need_schedule_inputs &&
        (!a->q || !a->k || !a->v || !a->beta || !a->gate || !a->out))
        return fail(GDN_EINVAL, "verify args: null q/k/v/beta/gate/out");
    return GDN_OK;
}

static gdn_status verify_setup(const gdn_verify_args *a, const int32_t *host_image,
                               const int32_t *dev_image, VerifyParams &P, ImageView &v) {
    gdn_status st = check_verify_args(a, true);
    if (st != GDN_OK) return st;
    if (!image_ok(host_image) || dev_image == nullptr)
        return fail(GDN_EINVAL, "gdn_tree_verify: missing or malformed schedule image");
    v = view_image(host_image);
    if (v.n_seqs != a->n_seqs || v.n_nodes != a->n_nodes)
        return fail(GDN_EINVAL, "gdn_tree_verify: n_seqs/n_nodes (%d/%d) differ from the "
                    "schedule's (%d/%d)", a->n_seqs, a->n_nodes, v.n_seqs, v.n_nodes);
    if (v.max_tree > a->max_nodes)
        return fail(GDN_ECAPACITY, "gdn_tree_verify: max_nodes %d < largest tree %d",
                    a->max_nodes, v.max_tree);
    if (v.n_boundaries > 0 && a->boundary == nullptr)
        return fail(GDN_EINVAL, "gdn_tree_verify: schedule has %d boundary nodes but no "
                    "boundary workspace", v.n_boundaries);
    P = VerifyParams{};
    P.q = a->q; P.k = a->k; P.v = a->v; P.beta = a->beta; P.gate = a->gate;
    P.state = a->state;
    for (int i = 0; i < 2; ++i) {
        P.bank_k[i] = a->bank_k[i];
        P.bank_u[i] = a->bank_u[i];
        P.bank_lg[i] = a->bank_lg[i];
    }
    P.role = a->role; P.pending = a->pending_len; P.boundary = a->boundary; P.out = a->out;
    P.img = dev_image;
    P.off_seq = v.off_seq; P.off_chain = v.off_chain; P.off_cnodes = v.off_cnodes;
    P.off_cseq = v.off_cseq; P.off_csrc = v.off_csrc; P.off_store = v.off_store;
    P.S = a->n_seqs; P.H = a->n_heads; P.T = a->n_nodes; P.max_nodes = a->max_nodes;
    P.n_boundaries = v.n_boundaries; P.layer_begin = a->layer_begin;
    return GDN_OK;
}

static gdn_status run_wave(VerifyParams P, const int32_t *host_image, const ImageView &v,
                           const gdn_verify_args *a, int wave, hipStream_t stream) {
    const int32_t c0 = host_image[v.off_wave + wave], c1 = host_image[v.off_wave + wave + 1];
    P.chain_begin = c0;
    P.n_chains = c1 - c0;
    P.n_blocks = int64_t(a->n_layers) * P.n_chains * a->n_heads;
    if (P.n_blocks > 0xFFFFFFFFll)
        return fail(GDN_EINVAL, "gdn_tree_verify: %lld workgroups exceed one launch",
                    (long long)P.n_blocks);
    return dispatch_verify(P, a->head_dim, a->in_dtype, stream);
}

}  // namespace gdn

using namespace gdn;

extern "C" size_t gdn_verify_workspace_bytes(const int32_t *host_image, int32_t n_heads,
                                             int32_t head_dim, int32_t n_layers) {
    if (!image_ok(host_image) || n_heads < 1 || head_dim < 1 || n_layers < 1) return 0;
    const ImageView v = view_image(host_image);
    return size_t(n_layers) * size_t(v.n_boundaries) * size_t(n_heads) * size_t(head_dim) *
           size_t(head_dim) * sizeof(float);
}

extern "C" gdn_status gdn_tree_verify(const gdn_verify_args *a, const int32_t *host_image,
                                      const int32_t *dev_image, void *stream) {
    clear_error();
    VerifyParams P;
    ImageView v;
    gdn_status st = verify_setup(a, host_image, dev_image, P, v);
    if (st != GDN_OK || a->n_seqs == 0) return st;
    for (int w = 0; w < v.n_waves; ++w) {
        st = run_wave(P, host_image, v, a, w, static_cast<hipStream_t>(stream));
        if (st != GDN_OK) return st;
    }
    return GDN_OK;
}

extern "C" gdn_status gdn_tree_verify_wave(const gdn_verify_args *a, const int32_t *host_image,
                                           const int32_t *dev_image, int32_t wave,
                                           void *stream) {
    clear_error();
    VerifyParams P;
    ImageView v;
    gdn_status st = verify_setup(a, host_image, dev_image, P, v);
    if (st != GDN_OK) return st;
    if (wave < 0 || wave >= v.n_waves)
        return fail(GDN_EINVAL, "gdn_tree_verify_wave: wave %d not in [0, %d)", wave, v.n_waves);
    return run_wave(P, host_image, v, a, wave, static_cast<hipStream_t>(stream));
}

// Flush helpers used by gdn_flush (commit.hip).
namespace gdn {
gdn_status flush_state(const gdn_verify_args *a, hipStream_t stream) {
    gdn_status st = check_verify_args(a, false);
    if (st != GDN_OK || a->n_seqs == 0) return st;
    VerifyParams P{};
    P.state = a->state;
    for (int i = 0; i < 2; ++i) {
        P.bank_k[i] = a->bank_k[i];
        P.bank_u[i] = a->bank_u[i];
        P.bank_lg[i] = a->bank_lg[i];
    }
    P.role = a->role;
    P.pending = a->pending_len;
    P.S = a->n_seqs;
    P.H = a->n_heads;
    P.max_nodes = a->max_nodes;
    P.layer_begin = a->layer_begin;
    P.fold_only = 1;
    P.n_blocks = int64_t(a->n_layers) * a->n_seqs * a->n_heads;
    if (P.n_blocks > 0xFFFFFFFFll) return fail(GDN_EINVAL, "gdn_flush: too many workgroups");
    return dispatch_verify(P, a->head_dim, a->in_dtype, stream);
}
gdn_status check_flush_verify_args(const gdn_verify_args *a) { return check_verify_args(a, false); }
}  // namespace gdn
