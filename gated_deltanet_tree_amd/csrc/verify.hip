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
#include <hip/hip_ext.h>

#include <mutex>

#include "verify_common.h"

namespace gdn {

// fp32 inputs need twice the staging registers; they get a 2-wave budget to avoid spills.
template <int D, typename TIn>
__global__ __launch_bounds__(Tile<D>::THREADS, sizeof(TIn) == 2 ? GDN_VERIFY_MIN_WAVES : 2)
void verify_chain_kernel(VerifyParams P, const int32_t *__restrict__ rows) {
    using TL = Tile<D>;
    using SG = Stager<D, TIn>;
    constexpr int M = TL::M, NP = TL::NP, VEC = TL::VEC;
    typedef VecT<VEC> V;
    __shared__ __align__(16) float lds[2][SG::PB * SG::SLOT];

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int rg = lane >> 3, cl = lane & 7;
    // Grids are capped at kMaxBlocks workgroups, so block arithmetic stays in 32 bits.
    uint32_t logical = xcd_logical(blockIdx.x, uint32_t(P.n_blocks));
#if GDN_REVERSE_LIGHT_WAVES
    if (P.chain_begin > 0) logical = uint32_t(P.n_blocks) - 1 - logical;
#endif

    int layer_rel, seq, h, chain = -1;
    if (P.fold_only) {
        const uint32_t per = uint32_t(P.S) * uint32_t(P.H);
        layer_rel = int(logical / per);
        const uint32_t rem = logical % per;
        seq = int(rem / uint32_t(P.H));
        h = int(rem % uint32_t(P.H));
    } else {
        const uint32_t per = uint32_t(P.n_chains) * uint32_t(P.H);
        layer_rel = int(logical / per);
        const uint32_t rem = logical % per;
        h = int(rem / uint32_t(P.n_chains));
        chain = P.chain_begin + int(rem % uint32_t(P.n_chains));
        seq = P.img[P.off_cseq + chain];
    }
    ChainCtx c;
    c.h = h;
    c.T = P.T;
    c.H = P.H;
    c.off_cnodes = P.off_cnodes;
    c.img = P.img;
    c.k = P.k;
    c.q = P.q;
    c.v = P.v;
    c.beta = P.beta;
    c.gate = P.gate;
    c.layer = P.layer_begin + layer_rel;
    const int src = P.fold_only ? -1 : P.img[P.off_csrc + chain];
    c.nbeg = P.fold_only ? 0 : P.img[P.off_chain + chain];
    const int nend = P.fold_only ? 0 : P.img[P.off_chain + chain + 1];
    const int seq_off = P.fold_only ? 0 : P.img[P.off_seq + seq];
    const int role = P.role[seq];
    c.L = src < 0 ? min(max(P.pending[seq], 0), P.max_nodes) : 0;  // clamp: bank rows
    c.n_items = c.L + (nend - c.nbeg);
    if (c.n_items == 0) return;  // flush of a sequence with nothing pending

    const int64_t sh = (int64_t(c.layer) * P.S + seq) * P.H + h;  // (layer, seq, head)
    float *committed = P.state + sh * D * D;
    const float *start = src < 0 ? committed
        : P.boundary + ((int64_t(layer_rel) * P.n_boundaries + src) * P.H + h) * D * D;
    c.pk = P.bank_k[role];
    c.pu = P.bank_u[role];
    c.plg = P.bank_lg[role];
    c.prow = rows + int64_t(seq) * P.max_nodes;  // a separate no-alias argument: scalar loads
    c.max_nodes = P.max_nodes;
    float *wk = P.bank_k[role ^ 1], *wu = P.bank_u[role ^ 1], *wlg = P.bank_lg[role ^ 1];
    c.bank_row0 = sh * P.max_nodes;  // row index of (layer, seq, head, 0)

    // Element offsets inside a d x d tile: thread part + compile-time part, so every tile
    // access is (uniform base, one 32-bit per-thread offset, immediate).
    const int row0 = w * TL::RW + rg;  // rows row0 + 8m
    const int col0 = cl * VEC;         // columns col0 + 8 VEC p
    const int toff = row0 * D + col0;
#define GDN_T(m, p) (toff + (m) * 8 * D + (p) * 8 * VEC)
#define GDN_ROW(m) (row0 + 8 * (m))
#define GDN_COL(p) (col0 + (p) * 8 * VEC)

    // The start tile is issued first: its address needs only the chain's own fields.
    float s[M][NP][VEC];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int p = 0; p < NP; ++p) V::get(start + GDN_T(m, p), s[m][p]);
    SG st;
    stage_issue(st, c, 0, tid);

    for (int it0 = 0, blk = 0; it0 < c.n_items; it0 += SG::PB, ++blk) {
        float *buf = lds[blk & 1];
        stage_commit(st, buf, c, it0, tid);
        __syncthreads();
        if (it0 + SG::PB < c.n_items) stage_issue(st, c, it0 + SG::PB, tid);
        const int it1 = min(c.n_items, it0 + SG::PB);
        for (int it = it0; it < it1; ++it) {
            const float *slot = buf + (it - it0) * SG::SLOT;
            // Both item kinds end in the same rank-1 update S <- g S + u k^T:
            //   pending fold row: g = exp(lg), u = banked residual;
            //   node:             g = gate,    u = beta (v - g S k).
            const bool fold = it < c.L;
            float g, u[M], o[M], kq = 0.f;
            int node = 0;
            if (fold) {
                g = expf(slot[3 * D]);
#pragma unroll
                for (int m = 0; m < M; ++m) u[m] = slot[2 * D + GDN_ROW(m)];
            } else {
                node = P.img[P.off_cnodes + c.nbeg + (it - c.L)];
                float a[M], b[M];
#pragma unroll
                for (int m = 0; m < M; ++m) a[m] = b[m] = 0.f;
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    float kc[VEC], qc[VEC];
                    V::get(slot + GDN_COL(p), kc);
                    V::get(slot + D + GDN_COL(p), qc);
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
                const float beta = slot[3 * D];
                g = slot[3 * D + 1];
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    u[m] = beta * (slot[2 * D + GDN_ROW(m)] - g * a[m]);
                    o[m] = fmaf(u[m], kq, g * b[m]);
                }
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                float kc[VEC];
                V::get(slot + GDN_COL(p), kc);
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) s[m][p][e] = fmaf(u[m], kc[e], g * s[m][p][e]);
            }

            if (fold) {
                if (it == c.L - 1) {  // the committed state is written back exactly once
#pragma unroll
                    for (int m = 0; m < M; ++m)
#pragma unroll
                        for (int p = 0; p < NP; ++p) V::put(committed + GDN_T(m, p), s[m][p]);
                }
                continue;
            }

            // Outputs and factors: lane cl == m of each octet writes row m's o and u.
            const int local = node - seq_off;
            float *orow = P.out + ((int64_t(c.layer) * P.T + node) * P.H + h) * D;
            float *urow = wu + (c.bank_row0 + local) * D;
#pragma unroll
            for (int m = 0; m < M; ++m)
                if (cl == m) {
                    orow[GDN_ROW(m)] = o[m];
                    urow[GDN_ROW(m)] = u[m];
                }
            if (w == 0 && rg == 0) {
                float *krow = wk + (c.bank_row0 + local) * D;
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    float kc[VEC];
                    V::get(slot + GDN_COL(p), kc);
                    V::put(krow + GDN_COL(p), kc);
                }
            }
            if (tid == 0) wlg[c.bank_row0 + local] = logf(g);

            const int slot_id = P.img[P.off_store + node];
            if (slot_id >= 0) {  // boundary node: its state seeds later light chains
                float *dst = P.boundary +
                    ((int64_t(layer_rel) * P.n_boundaries + slot_id) * P.H + h) * D * D;
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int p = 0; p < NP; ++p) V::put(dst + GDN_T(m, p), s[m][p]);
            }
        }
    }
#undef GDN_T
#undef GDN_ROW
#undef GDN_COL
}

template <int D, typename TIn>
static gdn_status launch_verify(const VerifyParams &P, hipStream_t stream, hipEvent_t start,
                                hipEvent_t stop) {
    if (P.n_blocks <= 0) return GDN_OK;
    if (start == nullptr && stop == nullptr) {
        hipLaunchKernelGGL((verify_chain_kernel<D, TIn>), dim3(uint32_t(P.n_blocks)),
                           dim3(Tile<D>::THREADS), 0, stream, P, P.rows);
    } else {  // timestamps taken by the dispatch itself: no extra packets on the stream
        hipExtLaunchKernelGGL((verify_chain_kernel<D, TIn>), dim3(uint32_t(P.n_blocks)),
                              dim3(Tile<D>::THREADS), 0, stream, start, stop, 0, P, P.rows);
    }
    GDN_LAUNCH_CHECK("verify_chain_kernel");
    return GDN_OK;
}

static gdn_status dispatch_verify(const VerifyParams &P, int d, int dtype, hipStream_t stream,
                                  hipEvent_t start = nullptr, hipEvent_t stop = nullptr) {
    if (d == 128)
        return dtype == GDN_BF16 ? launch_verify<128, bf16_t>(P, stream, start, stop)
                                 : launch_verify<128, float>(P, stream, start, stop);
    return dtype == GDN_BF16 ? launch_verify<16, bf16_t>(P, stream, start, stop)
                             : launch_verify<16, float>(P, stream, start, stop);
}

// need_schedule_inputs: beta, gate and out (and q, k, v when need_qkv) are read or written.
static gdn_status check_verify_args(const gdn_verify_args *a, bool need_schedule_inputs,
                                    bool need_qkv = true) {
    if (a == nullptr) return fail(GDN_EINVAL, "verify args: null");
    if (a->head_dim != 16 && a->head_dim != 128)
        return fail(GDN_EINVAL, "verify args: head_dim %d not in {16, 128}", a->head_dim);
    if (a->n_heads < 1 || a->n_layers < 1 || a->layer_begin < 0 || a->n_seqs < 0 ||
        a->max_nodes < 1)
        return fail(GDN_EINVAL, "verify args: bad n_heads/n_layers/layer_begin/n_seqs/max_nodes");
    if (a->in_dtype != GDN_F32 && a->in_dtype != GDN_BF16)
        return fail(GDN_EINVAL, "verify args: in_dtype %d", a->in_dtype);
    if (a->n_seqs == 0) return GDN_OK;  // empty batch: nothing is read or written
    if (!a->state || !a->role || !a->pending_len || !a->pending_rows)
        return fail(GDN_EINVAL, "verify args: null state/role/pending_len/pending_rows");
    for (int i = 0; i < 2; ++i)
        if (!a->bank_k[i] || !a->bank_u[i] || !a->bank_lg[i])
            return fail(GDN_EINVAL, "verify args: null bank pointer");
    if (need_schedule_inputs && (!a->beta || !a->gate || !a->out))
        return fail(GDN_EINVAL, "verify args: null beta/gate/out");
    if (need_schedule_inputs && need_qkv && (!a->q || !a->k || !a->v))
        return fail(GDN_EINVAL, "verify args: null q/k/v");
    // Tiles, rows and vectors are moved in 16-byte pieces.
    const void *aligned[] = {a->q, a->k, a->v, a->state, a->bank_k[0], a->bank_k[1],
                             a->bank_u[0], a->bank_u[1], a->workspace, a->out};
    for (const void *p : aligned)
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
            return fail(GDN_EINVAL, "verify args: q/k/v/state/bank/workspace/out pointers must "
                        "be 16-byte aligned");
    return GDN_OK;
}

gdn_status verify_setup(const gdn_verify_args *a, const int32_t *host_image,
                        const int32_t *dev_image, VerifyParams &P, ImageView &v,
                        bool need_boundary, bool need_qkv) {
    gdn_status st = check_verify_args(a, true, need_qkv);
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
    if (need_boundary && v.n_boundaries > 0 && a->workspace == nullptr)
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
    P.role = a->role; P.pending = a->pending_len; P.rows = a->pending_rows; P.boundary = a->workspace; P.out = a->out;
    P.img = dev_image;
    P.off_seq = v.off_seq; P.off_chain = v.off_chain; P.off_cnodes = v.off_cnodes;
    P.off_cseq = v.off_cseq; P.off_csrc = v.off_csrc; P.off_store = v.off_store;
    P.S = a->n_seqs; P.H = a->n_heads; P.T = a->n_nodes; P.max_nodes = a->max_nodes;
    P.n_boundaries = v.n_boundaries; P.layer_begin = a->layer_begin;
    return GDN_OK;
}

// ---- boundary-state scratch of gdn_tree_verify_noalloc ------------------------------------
// For callers that cannot allocate (HIP graph capture, tight serving loops): the boundary
// states live in a fixed array in device memory that the library holds on every GPU it runs
// on until the process ends.  In host code `scratch` names a host-side stand-in, not a device
// address: kernels receive the address that hipGetSymbolAddress returns for the current
// device, looked up once per device and kept.  Calls that overlap on one GPU share the array
// and race; nothing in it needs to start at zero (every boundary slot is written by its chain
// before a later wave reads it).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

}  // namespace gdn

static __device__ __align__(256) float scratch[gdn::kNoAllocScratchBytes / sizeof(float)];

namespace gdn {

static std::mutex g_scratch_mu;
static float *g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device

// Device address of `scratch` on the current device (looked up on the first call there).
static gdn_status scratch_address(float **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GDN_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(GDN_EINVAL, "device %d beyond the %d devices the scratch table holds", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(GDN_EDEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_dev[dev] = static_cast<float *>(p);
    }
    *out = g_scratch_dev[dev];
    return GDN_OK;
}

static gdn_status run_wave(VerifyParams P, const int32_t *host_image, const ImageView &v,
                           const gdn_verify_args *a, int wave, hipStream_t stream,
                           hipEvent_t start = nullptr, hipEvent_t stop = nullptr) {
    const int32_t c0 = host_image[v.off_wave + wave], c1 = host_image[v.off_wave + wave + 1];
    P.chain_begin = c0;
    P.n_chains = c1 - c0;
    P.n_blocks = int64_t(a->n_layers) * P.n_chains * a->n_heads;
    if (P.n_blocks > kMaxBlocks)
        return fail(GDN_EINVAL, "gdn_tree_verify: %lld workgroups exceed one launch",
                    (long long)P.n_blocks);
    return dispatch_verify(P, a->head_dim, a->in_dtype, stream, start, stop);
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
    gdn_status st = verify_setup(a, host_image, dev_image, P, v, true);
    if (st != GDN_OK || a->n_seqs == 0) return st;
    for (int w = 0; w < v.n_waves; ++w) {
        st = run_wave(P, host_image, v, a, w, static_cast<hipStream_t>(stream));
        if (st != GDN_OK) return st;
    }
    return GDN_OK;
}

extern "C" gdn_status gdn_tree_verify_noalloc(const gdn_verify_args *a,
                                              const int32_t *host_image,
                                              const int32_t *dev_image, void *stream) {
    clear_error();
    if (a == nullptr) return fail(GDN_EINVAL, "gdn_tree_verify_noalloc: null args");
    gdn_verify_args b = *a;
    b.workspace = nullptr;  // not used: the boundary states go to the library's scratch
    VerifyParams P;
    ImageView v;
    gdn_status st = verify_setup(&b, host_image, dev_image, P, v, false);
    if (st != GDN_OK || b.n_seqs == 0) return st;
    const size_t need = size_t(b.n_layers) * size_t(v.n_boundaries) * size_t(b.n_heads) *
                        size_t(b.head_dim) * size_t(b.head_dim) * sizeof(float);
    if (need > kNoAllocScratchBytes)
        return fail(GDN_ECAPACITY, "gdn_tree_verify_noalloc: %zu bytes of boundary states "
                    "(%d boundary nodes x %d heads x %d layers) exceed the fixed scratch of %zu "
                    "bytes; use gdn_tree_verify with a workspace", need, v.n_boundaries,
                    b.n_heads, b.n_layers, kNoAllocScratchBytes);
    if (need > 0) {
        float *scr = nullptr;
        st = scratch_address(&scr);
        if (st != GDN_OK) return st;
        P.boundary = scr;
    }
    for (int w = 0; w < v.n_waves; ++w) {
        st = run_wave(P, host_image, v, &b, w, static_cast<hipStream_t>(stream));
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
    gdn_status st = verify_setup(a, host_image, dev_image, P, v, true);
    if (st != GDN_OK) return st;
    if (wave < 0 || wave >= v.n_waves)
        return fail(GDN_EINVAL, "gdn_tree_verify_wave: wave %d not in [0, %d)", wave, v.n_waves);
    return run_wave(P, host_image, v, a, wave, static_cast<hipStream_t>(stream));
}

extern "C" gdn_status gdn_tree_verify_wave_timed(const gdn_verify_args *a,
                                                 const int32_t *host_image,
                                                 const int32_t *dev_image, int32_t wave,
                                                 void *start_event, void *stop_event,
                                                 void *stream) {
    clear_error();
    VerifyParams P;
    ImageView v;
    gdn_status st = verify_setup(a, host_image, dev_image, P, v, true);
    if (st != GDN_OK) return st;
    if (wave < 0 || wave >= v.n_waves)
        return fail(GDN_EINVAL, "gdn_tree_verify_wave_timed: wave %d not in [0, %d)", wave,
                    v.n_waves);
    if (start_event == nullptr || stop_event == nullptr)
        return fail(GDN_EINVAL, "gdn_tree_verify_wave_timed: null event");
    return run_wave(P, host_image, v, a, wave, static_cast<hipStream_t>(stream),
                    static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
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
    P.rows = a->pending_rows;
    P.S = a->n_seqs;
    P.H = a->n_heads;
    P.max_nodes = a->max_nodes;
    P.layer_begin = a->layer_begin;
    P.fold_only = 1;
    P.n_blocks = int64_t(a->n_layers) * a->n_seqs * a->n_heads;
    if (P.n_blocks > kMaxBlocks) return fail(GDN_EINVAL, "gdn_flush: too many workgroups");
    return dispatch_verify(P, a->head_dim, a->in_dtype, stream);
}
gdn_status check_flush_verify_args(const gdn_verify_args *a) { return check_verify_args(a, false); }
}  // namespace gdn
