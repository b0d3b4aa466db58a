/*
 * gdn_tree.h -- C ABI for verifying a speculative draft tree through Gated DeltaNet layers
 * on one AMD Instinct MI355X (gfx950).
 *
 * What the library computes (cited by page title and section):
 *   "Lucebox SpecLA and Gated DeltaNet state-resident verification" guide --
 *     section "Why speculative decoding is harder for linear-attention models": every GDN
 *       head carries a recurrent state S that each token advances with the gated delta rule,
 *       S <- g S (I - beta k k^T) + beta v k^T, read out as o = S q; in a candidate tree
 *       every node must see the state of its own root-to-node path, starting from the
 *       committed state, and rejected candidates must leave that state untouched;
 *     mechanism 1 (state-resident verification): consecutive nodes of one verify chain are
 *       processed inside one kernel with the state tile kept on chip, read once at the
 *       chain head and written once at its end; the depthwise conv window is handled the
 *       same way so siblings never pick up a DFS neighbour's conv history;
 *     mechanism 2 (HLD scheduling): heavy-light chains, only boundary states materialised,
 *       chains grouped into dependency waves, all chains of a wave launched together;
 *     mechanism 3 (accepted-factor cache): per node the key, the delta-rule residual
 *       update vector, the log decay gate and the conv raw input are kept in two FP32
 *       double-buffered banks; in-order acceptance swaps the banks, branched acceptance
 *       compacts rows back into path order (this library also offers a commit that copies
 *       nothing and records where the accepted rows sit: see gdn_commit_path);
 *     mechanism 4 (deferred fused commit): the next verify folds the pending factors into
 *       the committed state before verifying; a final flush materialises the last path.
 *   "Luce DFlash server README", section "How it works": DDTree verifies a parent-indexed
 *     tree of candidates in one target forward; the tree-aware conv gathers each node's
 *     window along its parent chain; after accept the state is that of the committed prefix.
 *
 * Conventions
 *   - Ownership: the caller allocates every buffer. Host arrays are plain memory; device
 *     arrays are device pointers (e.g. from torch on ROCm). The library allocates nothing,
 *     keeps no pointer after a call returns and has no global state except a per-thread
 *     error string (gdn_last_error) and the fixed device scratch of gdn_tree_verify_noalloc
 *     (with its per-device address, looked up once).
 *   - Streams: device calls take a hipStream_t as `void *stream` (NULL = default stream),
 *     only enqueue work and return. Host calls (schedule, sizes) are synchronous.
 *   - Errors: every call returns a gdn_status. All arguments are validated before anything
 *     is enqueued; on error nothing is launched and no output is touched. GDN_EDEVICE means
 *     the HIP runtime refused a launch; gdn_last_error() gives the text.
 *   - Tree ids: a sequence b has N_b >= 1 nodes with local ids 0..N_b-1, node 0 the root,
 *     parent[0] = -1 and 0 <= parent[i] < i. Global id = seq_offsets[b] + local id; T is the
 *     total node count of the batch.
 *   - Layers: every per-layer device array has a leading layer index; layer l's block starts
 *     at base + l * (size of one layer's block, in elements, as given per array below).
 *     Device calls process layers layer_begin .. layer_begin + n_layers - 1 (n_layers = 1
 *     is the per-layer pattern of a model forward).
 *   - Shapes: head_dim d = d_k = d_v in {16, 128}; conv width 4; N_b <= 1024.
 *   - Numerics: inputs bf16 or fp32; state, factors and outputs fp32; accumulation fp32.
 *   - Alignment: q, k, v, state, key/residual banks, workspace and out must be 16-byte
 *     aligned (tiles and rows move in 16-byte pieces); GDN_EINVAL otherwise.
 */
#ifndef GDN_TREE_H
#define GDN_TREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gdn_status;
#define GDN_OK         0
#define GDN_EINVAL    -1 /* null pointer, unsupported size or dtype, inconsistent counts */
#define GDN_ETREE     -2 /* a parent array is not a root-first tree with parent[i] < i   */
#define GDN_EPATH     -3 /* an accepted path is not a root path of its tree              */
#define GDN_ECAPACITY -4 /* a caller buffer is smaller than the call needs               */
#define GDN_EDEVICE   -5 /* the HIP runtime reported an error at enqueue                 */

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Text of the last error raised on the calling thread ("" if none). */
const char *gdn_last_error(void);

/* ------------------------------------------------------------------------------------
 * Heavy-light chain schedule (host, integer, deterministic).
 * SpecLA guide, mechanism 2. Rules (fixed where the page leaves them open):
 *   heavy child = child with the largest subtree, ties to the smallest index;
 *   a chain is the heavy path from the root or from a light child, root-to-leaf;
 *   wave(root chain) = 0, wave(c) = 1 + wave of the chain holding parent(head(c));
 *   boundary node = node with at least one light child; its state is stored once and
 *     every light chain hanging off it starts from it; slots by ascending global id;
 *   chains ordered by (wave, sequence, global head id); waves merged across the batch.
 *
 * The schedule is one int32 image, built on the host and copied verbatim to the device.
 * Layout for n_seqs = S and T total nodes (word offsets):
 *   [0]  magic 0x53444E47     [1] S   [2] T   [3] n_chains   [4] n_waves
 *   [5]  n_boundaries         [6] longest chain   [7] largest tree
 *   [8]  R = tree-masked verify records (sum over nodes of depth + 1), or -1 when R > 32 T
 *        and the plan below is absent (gdn_tree_verify_ut then refuses the batch)
 *   [9]  most records of one tree     [10] most depth levels + 1 of one tree   [11..15] zero
 *   seq_offsets   [S+1] at 16                       b's nodes: [seq_offsets[b], seq_offsets[b+1])
 *   wave_offsets  [T+1] at 17+S                     wave w: chains [wave_offsets[w], ..[w+1])
 *   chain_offsets [T+1] at 18+S+T                   chain c: chain_nodes[chain_offsets[c] ..)
 *   chain_nodes   [T]   at 19+S+2T                  global ids, root-to-leaf within a chain
 *   chain_seq     [T]   at 19+S+3T                  owning sequence of chain c
 *   chain_src     [T]   at 19+S+4T                  -1: committed state, else boundary slot
 *   node_store    [T]   at 19+S+5T                  slot written after node n, or -1
 *   node_parent   [T]   at 19+S+6T                  global parent id, -1 for roots
 *   node_depth    [T]   at 19+S+7T                  edges from the root
 * Tree-masked verify plan (per tree: nodes ordered by (depth, local id); each node owns a
 * block of depth + 1 records, blocks in that order: the node, then its ancestors nearest
 * first), with P = 19 + S + 8T:
 *   rec_base      [S+1] at P                         tree b's records: [rec_base[b], ..[b+1])
 *   node_rec      [T]   at P+S+1                     node's first record, relative to its tree
 *   lv_base       [S+1] at P+S+1+T                   tree b's level offsets start in lvn
 *   lvn           [T+S] at P+2S+2+T                  per tree: first position of depth level
 *                                                    d in lvnode, d = 0 .. dmax+1
 *   lvnode        [T]   at P+3S+2+2T                 per tree (at seq_offsets[b]): local ids
 *                                                    by (depth, id)
 *   rec_anc       [32T] at P+3S+2+3T                 local node id of each record
 *   total words = 21 + 4S + 43T. Arrays are sized for T; only the counted prefix is used.
 * ---------------------------------------------------------------------------------- */
size_t gdn_schedule_words(int32_t n_seqs, int32_t n_nodes_total);

/* parent_local: host [T], tree b's local parent array at parent_local[seq_offsets[b]..].
 * seq_offsets: host [n_seqs+1], seq_offsets[0] = 0, strictly increasing.
 * image: host [image_words], filled on success.
 * GDN_ETREE for a malformed tree, GDN_ECAPACITY if image_words is too small. */
gdn_status gdn_hld_schedule(const int32_t *parent_local, const int32_t *seq_offsets,
                            int32_t n_seqs, int32_t *image, size_t image_words);

/* ------------------------------------------------------------------------------------
 * Draft-tree builder (host): best-first tree over the draft's top-K candidates per position,
 * with a node budget, confidence pruning and a greedy-chain pre-seed.
 * Luce DFlash server README, "How it works" (best-first tree of up to 22 nodes spanning the
 * top-K branches of each position; chain pre-seed); SpecLA guide, the section on enabling it
 * with one flag (budget 22, tau 6, top-k 4; nodes scoring below q* - tau are pruned).
 *
 * For tree b, position i (0-based, the i-th token after the root) has top_k candidates with
 * log-probabilities logp[b][i][0..top_k-1], sorted descending (candidate 0 is the greedy
 * token), every value finite and <= 0.  A node at depth d takes candidate k of position d-1;
 * its children are the candidates of position d.
 *   score(root) = 0, score(node) = score(parent) + logp, fp32, summed along the path;
 *   q*(d) = the greedy chain's score at depth d = the best score at depth d;
 *   a node with score < q*(d) - tau (fp32) is pruned with its subtree; tau = INFINITY prunes
 *   nothing; tau < 0 or NaN is GDN_EINVAL;
 *   the budget counts the root;
 *   chain_seed != 0 places the greedy chain first (depths 1 .. min(n_positions, budget-1));
 *   every further node is the best remaining candidate: higher score first, then the
 *   shallower, then the smaller sequence of candidate ranks along the path.
 * Node ids are insertion order, so parent[i] < i: parent[b][0 .. n_nodes[b]) is directly a
 * valid `parent_local` tree for gdn_hld_schedule.
 *
 * logp:        host [n_trees][n_positions][top_k] fp32.
 * tokens:      host [n_trees][n_positions][top_k] token ids, or NULL when token is NULL.
 * root_tokens: host [n_trees], or NULL (the root's token is then -1).
 * parent, depth, rank, token, score: host [n_trees][budget], caller-owned outputs; rank is
 *   the candidate index of the node at its position (-1 for the root); slots at or beyond
 *   n_nodes[b] are set to -1 (score 0).  token may be NULL.
 * n_nodes:     host [n_trees], nodes of each tree (1 <= n_nodes[b] <= budget).
 * Limits: 0 <= n_positions <= 16, 1 <= top_k <= 16, budget >= 1; otherwise GDN_EINVAL and
 * nothing is written.  Deterministic; no device work. */
gdn_status gdn_ddtree_build(const float *logp, const int32_t *tokens,
                            const int32_t *root_tokens, int32_t n_trees, int32_t n_positions,
                            int32_t top_k, int32_t budget, float tau, int32_t chain_seed,
                            int32_t *parent, int32_t *depth, int32_t *rank, int32_t *token,
                            float *score, int32_t *n_nodes);

/* ------------------------------------------------------------------------------------
 * Tree verify with fused deferred commit (SpecLA guide, mechanisms 1, 2 and 4).
 *
 * For every node n of every tree, every head h, every layer l processed:
 *   S_n = g_n S_parent + u_n k_n^T,  u_n = beta_n (v_n - g_n S_parent k_n)
 *       (= g_n S_parent (I - beta_n k_n k_n^T) + beta_n v_n k_n^T)
 *   out[n] = S_n q_n
 * where S_parent of a root is the committed state AFTER the deferred fold:
 *   if pending_len[b] = L > 0:  S <- exp(lg_i) S + u_i k_i^T for pending factors i = 0..L-1,
 *   where factor i is row pending_rows[b][i] of the pending bank, and the folded state is
 *   written back to `state` (once, by the root chain).
 * Factors (k_n, u_n, lg_n = ln g_n) are written to row n (local id) of the write bank
 * 1 - role[b]. Rows of the pending bank role[b] are only read.
 *
 * Work: one launch per dependency wave, one workgroup per (layer, chain, head); the fp32
 * state tile stays in VGPRs for the whole chain; boundary nodes store their state once to
 * `workspace` for the light chains of later waves.
 * ---------------------------------------------------------------------------------- */
typedef struct {
    int32_t n_seqs;      /* S, must equal the schedule's                                   */
    int32_t n_heads;     /* H >= 1                                                         */
    int32_t head_dim;    /* d in {16, 128}                                                 */
    int32_t n_nodes;     /* T, must equal the schedule's                                   */
    int32_t max_nodes;   /* bank rows per (layer, seq, head); >= every N_b                 */
    int32_t layer_begin; /* first layer processed                                          */
    int32_t n_layers;    /* layers processed, >= 1                                         */
    int32_t in_dtype;    /* gdn_dtype of q, k, v, beta, gate                               */
    const void *q, *k;   /* [Ly][T][H][d]     (per-layer block T*H*d)                      */
    const void *v;       /* [Ly][T][H][d]                                                  */
    const void *beta;    /* [Ly][T][H]        (per-layer block T*H)                        */
    const void *gate;    /* [Ly][T][H]        g in [0, 1], linear (not log); g = 0 banks    */
                         /* ln g = -inf, whose fold coefficient is exactly 0 (the state    */
                         /* before that token is erased, as the recurrence says)           */
    float *state;        /* [Ly][S][H][d][d]  committed state, row = d_v index, in/out     */
    float *bank_k[2];    /* [Ly][S][H][max_nodes][d]  keys                                 */
    float *bank_u[2];    /* [Ly][S][H][max_nodes][d]  residual update vectors              */
    float *bank_lg[2];   /* [Ly][S][H][max_nodes]     log decay gates                      */
    const int32_t *role;        /* device [S]: index (0/1) of the pending bank             */
    const int32_t *pending_len; /* device [S]: pending rows to fold, 0 = none              */
    const int32_t *pending_rows; /* device [S][max_nodes]: bank row of pending factor i of   */
                                 /* sequence b, in path order; written by gdn_commit_path,   */
                                 /* entries i < pending_len[b] read by the fold; each within */
                                 /* [0, max_nodes) (out-of-range entries are clamped)        */
    float *workspace;    /* device scratch of gdn_tree_verify*: gdn_verify_workspace_bytes() */
                         /* bytes of boundary states; not used by gdn_tree_verify_ut*       */
    float *out;          /* [Ly][T][H][d] fp32 outputs                                     */
} gdn_verify_args;

/* Bytes of `workspace` that gdn_tree_verify needs for this schedule (the boundary states):
 * n_layers * n_boundaries * H * d * d * 4. */
size_t gdn_verify_workspace_bytes(const int32_t *host_image, int32_t n_heads, int32_t head_dim,
                                  int32_t n_layers);

/* host_image: the schedule on the host (read for launch sizes);
 * dev_image: the same words in device memory (read by the kernels). */
gdn_status gdn_tree_verify(const gdn_verify_args *args, const int32_t *host_image,
                           const int32_t *dev_image, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same work and results as gdn_tree_verify,
 * bit-identical, with the boundary states kept in a fixed 32 MiB array of device memory that
 * the library holds on every GPU it runs on until the process ends, instead of `workspace`
 * (ignored; may be NULL).  The call allocates nothing.  GDN_ECAPACITY (nothing launched) when
 * gdn_verify_workspace_bytes for the call exceeds 32 MiB = 33554432 bytes (512 boundary tiles
 * at d = 128: e.g. one 22-node tree's ~6 boundary nodes x 48 heads fits, a 32-tree batch does
 * not).  Every call on one GPU shares that GPU's array: calls that overlap on one GPU (two
 * streams, two threads) race and must be serialised by the caller. */
gdn_status gdn_tree_verify_noalloc(const gdn_verify_args *args, const int32_t *host_image,
                                   const int32_t *dev_image, void *stream);

/* Same work as gdn_tree_verify restricted to dependency wave `wave` (0 <= wave < n_waves):
 * calling it for waves 0, 1, ... in order on one stream equals gdn_tree_verify. */
gdn_status gdn_tree_verify_wave(const gdn_verify_args *args, const int32_t *host_image,
                                const int32_t *dev_image, int32_t wave, void *stream);

/* Same as gdn_tree_verify_wave, with the kernel's start and end timestamps recorded into
 * two caller-created HIP events (hipEvent_t, passed as void *) by the dispatch itself, so
 * timing adds no packet to the stream; hipEventElapsedTime(start, stop) then gives the
 * kernel's duration. GDN_EINVAL if either event is NULL. */
gdn_status gdn_tree_verify_wave_timed(const gdn_verify_args *args, const int32_t *host_image,
                                      const int32_t *dev_image, int32_t wave, void *start_event,
                                      void *stop_event, void *stream);

/* Tree-masked UT verify (SpecLA guide, mechanism 1: the topology-mask / UT decomposition
 * form of the same verify). Same arguments, results and bank/fold contract as
 * gdn_tree_verify, computed in one launch per call with no boundary tiles: unrolling the
 * recurrence down a node's root path gives
 *   u_n = beta_n (v_n - G_n S0 k_n - sum_{j strict ancestor} E(n,j) (k_n.k_j) u_j)
 *   out[n] = G_n S0 q_n + sum_{j ancestor or n} E(n,j) (q_n.k_j) u_j
 * with G_n the product of the gates on n's root path and E(n,j) the product of the gates
 * strictly below j down to n; S0 is the committed state after the deferred fold.
 * bf16 inputs at d = 128 run on the matrix cores (the S0 products and the pair products);
 * other dtypes and head dims run on the vector units.  One launch per call; `workspace` is not
 * used (may be NULL).  A tree must fit the LDS budget of one workgroup (160 KiB: about 64
 * nodes at d = 128 with bf16 inputs); larger trees give GDN_EINVAL and should use
 * gdn_tree_verify. */
gdn_status gdn_tree_verify_ut(const gdn_verify_args *args, const int32_t *host_image,
                              const int32_t *dev_image, void *stream);

/* gdn_tree_verify_ut with dispatch-recorded start/stop HIP events (see
 * gdn_tree_verify_wave_timed). */
gdn_status gdn_tree_verify_ut_timed(const gdn_verify_args *args, const int32_t *host_image,
                                    const int32_t *dev_image, void *start_event,
                                    void *stop_event, void *stream);

/* ------------------------------------------------------------------------------------
 * Chunked prefill (SpecLA guide, the flush section: after a flush, or without speculation,
 * the GDN layer runs over plain token sequences; the sequence path shares the commit
 * semantics of the tree path).  For every sequence b, head h and layer l processed:
 *   for t in the sequence, in order:  S <- g_t S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *                                     out[t] = S q_t,
 * starting from the committed state; the final S is written back to `state`.  Pending
 * factors are not read: call gdn_flush first when a tree verify left any.
 * Work: one 256-thread workgroup per (layer, sequence, head, half of the state rows) walks the
 * sequence in chunks of 16 tokens on the matrix cores (tree-masked form of a chain); the chunk
 * tables are built one and two chunks ahead of the state by waves taking turns.
 * ---------------------------------------------------------------------------------- */
typedef struct {
    int32_t n_seqs;      /* S                                                               */
    int32_t n_heads;     /* H >= 1                                                          */
    int32_t head_dim;    /* d, must be 128                                                  */
    int32_t n_tokens;    /* T: tokens of all sequences, packed                              */
    int32_t layer_begin; /* first layer processed                                           */
    int32_t n_layers;    /* layers processed, >= 1                                          */
    int32_t in_dtype;    /* must be GDN_BF16                                                */
    int32_t reserved;
    const void *q, *k, *v;      /* [Ly][T][H][d] bf16, 16-byte aligned                       */
    const void *beta, *gate;    /* [Ly][T][H] bf16, gate = g in [0, 1] (linear)              */
    const int32_t *seq_offsets; /* device [S+1]: sequence b holds tokens [off[b], off[b+1])  */
    float *state;        /* [Ly][S][H][d][d] fp32 committed states, in/out, 16-byte aligned */
    float *out;          /* [Ly][T][H][d] fp32 outputs, 16-byte aligned                     */
} gdn_prefill_args;

/* host_seq_offsets: the same offsets on the host (validated: 0 .. n_tokens, non-decreasing).
 * GDN_EINVAL for other head dims or dtypes, bad offsets, null or misaligned pointers; nothing
 * is launched then.  Empty sequences leave their states untouched. */
gdn_status gdn_prefill(const gdn_prefill_args *args, const int32_t *host_seq_offsets,
                       void *stream);

/* gdn_prefill with dispatch-recorded start/stop HIP events (see gdn_tree_verify_wave_timed). */
gdn_status gdn_prefill_timed(const gdn_prefill_args *args, const int32_t *host_seq_offsets,
                             void *start_event, void *stop_event, void *stream);

/* ------------------------------------------------------------------------------------
 * Tree-aware causal depthwise conv with fused conv-window fold (DFlash README, "How it
 * works", tree-aware conv gather; SpecLA guide, mechanisms 1, 3 and 4).
 *
 * Fold first: if pending_len[b] = L > 0, conv_state[b] <- last 3 of
 *   (conv_state[b] columns, bank_x[role[b]] rows pending_rows[b][0..L-1]), written back.
 * Then for node n, channel c:
 *   out[n][c] = sum_{j<4} weight[c][j] * win_n[j],  win_n = last 4 of
 *   (conv_state[b][c][0..2], x along n's root path ending with x[n][c]);
 * weight[c][3] multiplies the current token; no bias, no activation.
 * Raw inputs x[n] go to row n (local id) of bank_x[1 - role[b]], in in_dtype: the bank keeps
 * every raw input bit-exact, as the guide's FP32 bank does; for bf16 inputs the bf16 bits are
 * that exact value in half the bytes.
 * ---------------------------------------------------------------------------------- */
typedef struct {
    int32_t n_seqs;      /* S                                                              */
    int32_t channels;    /* Cch >= 1                                                       */
    int32_t width;       /* must be 4                                                      */
    int32_t n_nodes;     /* T                                                              */
    int32_t max_nodes;   /* bank rows per (layer, seq); >= every N_b                       */
    int32_t layer_begin;
    int32_t n_layers;
    int32_t in_dtype;    /* gdn_dtype of x, weight and bank_x (fold-only calls: of bank_x) */
    const void *x;       /* [Ly][T][Cch]                                                   */
    const void *weight;  /* [Ly][Cch][4]                                                   */
    float *conv_state;   /* [Ly][S][Cch][3] committed window, oldest first, in/out         */
    void *bank_x[2];     /* [Ly][S][max_nodes][Cch] raw inputs, in in_dtype                */
    const int32_t *role;         /* the same device arrays as the verify's                 */
    const int32_t *pending_len;
    const int32_t *pending_rows;
    float *out;          /* [Ly][T][Cch] fp32                                              */
} gdn_conv_args;

gdn_status gdn_tree_conv(const gdn_conv_args *args, const int32_t *host_image,
                         const int32_t *dev_image, void *stream);

/* ------------------------------------------------------------------------------------
 * Fused conv -> verify (DFlash README, "How it works": the tree-aware conv window is gathered
 * along the parent chain and feeds the recurrent layer; SpecLA guide, mechanism 1 for the
 * conv window and the topology-mask verify, mechanisms 3 and 4 for the banks and the fold).
 * One launch per call does the work of gdn_tree_conv followed by gdn_tree_verify_ut, with q, k
 * and v taken from the conv instead of from memory:
 *   y    = the tree conv of gdn_tree_conv (after the same conv-window fold), over channels laid
 *          out [q heads | k heads | v heads]: C = 3 H d, and head h's q, k and v channels are
 *          h d + i, H d + h d + i and 2 H d + h d + i (i < d);
 *   q, k, v = silu(y) of the three blocks, silu(y) = y / (1 + exp(-y));
 *   q and k of each (node, head) are divided by max(their Euclidean length, 1e-6); v as is;
 * then the verify, fold, factor banks and outputs of gdn_tree_verify_ut on those q, k, v.  The
 * banked key is the fp32 unit key; x[n] is banked in bank_x[1 - role] as gdn_tree_conv does,
 * and the folded conv window is written back to conv_state.  The pages do not spell out the
 * conv-to-q/k/v wiring; this is the plain reading of a hybrid GDN layer.
 * Ignored (may be NULL): va->q, va->k, va->v, va->workspace and ca->out (the conv output stays
 * on chip).  Requirements (GDN_EINVAL otherwise, nothing launched): head_dim 128; bf16 beta,
 * gate, x and weight (ca->in_dtype = GDN_BF16, so bank_x holds bf16); ca->channels = 3 H 128;
 * ca's n_seqs, n_nodes, max_nodes, layer_begin and n_layers equal va's; ca->role,
 * ca->pending_len and ca->pending_rows are va's arrays; x, weight and bank_x 16-byte aligned;
 * the schedule carries the tree-masked plan and the trees fit one workgroup's LDS (160 KiB: a
 * 64-node top-8 tree of depth 16 takes about 144 KiB).
 * Work: one workgroup per (layer, sequence, head), 8 waves of 16 state rows; the conv, SiLU and
 * normalisation run in its prologue, the rest as gdn_tree_verify_ut on the matrix cores.
 * ---------------------------------------------------------------------------------- */
gdn_status gdn_tree_conv_verify(const gdn_verify_args *va, const gdn_conv_args *ca,
                                const int32_t *host_image, const int32_t *dev_image,
                                void *stream);

/* gdn_tree_conv_verify with dispatch-recorded start/stop HIP events (see
 * gdn_tree_verify_wave_timed). */
gdn_status gdn_tree_conv_verify_timed(const gdn_verify_args *va, const gdn_conv_args *ca,
                                      const int32_t *host_image, const int32_t *dev_image,
                                      void *start_event, void *stop_event, void *stream);

/* ------------------------------------------------------------------------------------
 * Accept -> commit (SpecLA guide, mechanism 3). Enqueue after the last layer's verify and
 * conv of the step. For each sequence b with accepted root path P_b of length L_b:
 *   L_b = 0            : pending_len[b] = 0 (nothing to commit)
 *   mode GDN_COMMIT_COMPACT (the guide's accepted-factor cache):
 *     P_b = [0..L_b-1] : role[b] ^= 1 (the written bank becomes pending; no device copy)
 *     otherwise        : row P_b[i] of every write bank (k, u, lg for every head, x) is
 *                        copied to row i of the pending bank, for all n_layers layers;
 *     pending_rows[b][i] = i
 *   mode GDN_COMMIT_ROW_MAP (no copy in either case):
 *     role[b] ^= 1 and pending_rows[b][i] = P_b[i]: the next fold reads the accepted rows
 *     where the verify wrote them
 *   and pending_len[b] = L_b.  Both modes fold the same factors in the same order, so the
 *   committed states they lead to are bit-identical; only the bank rows differ.
 * paths: host, concatenated local ids; path_offsets: host [S+1].
 * dev_paths / dev_path_offsets: the same arrays in device memory, read by the enqueued
 * kernels (keep them until those have run).
 * role_host / pending_host: host mirrors [S], read and updated by the call.
 * va->role, va->pending_len and va->pending_rows (device) are updated on the stream; ca may
 * be NULL when no conv banks are kept, otherwise its role, pending_len and pending_rows
 * must be va's.  GDN_EPATH if some P_b is not a root path of tree b, GDN_EINVAL for an unknown
 * mode (nothing is enqueued then).
 * ---------------------------------------------------------------------------------- */
#define GDN_COMMIT_COMPACT 0
#define GDN_COMMIT_ROW_MAP 1
gdn_status gdn_commit_path(const int32_t *host_image, const int32_t *paths,
                           const int32_t *path_offsets, const int32_t *dev_paths,
                           const int32_t *dev_path_offsets, const gdn_verify_args *va,
                           const gdn_conv_args *ca, int32_t *role_host, int32_t *pending_host,
                           int32_t mode, void *stream);

/* Raw row gather used by gdn_commit_path, exported for direct use:
 * for r in [0, n_rows): dst[dst_rows[r] * row_elems ..] = src[src_rows[r] * row_elems ..]
 * (row_elems floats each). dst_rows/src_rows are device int32 arrays. Bit-exact copy. */
gdn_status gdn_compact_factors(const float *src, float *dst, int64_t row_elems,
                               const int32_t *src_rows, const int32_t *dst_rows,
                               int32_t n_rows, void *stream);

/* ------------------------------------------------------------------------------------
 * Flush (SpecLA guide, mechanism 4): at the end of generation, on a switch to
 * autoregressive decode or on cancel, fold the pending factors of every sequence into
 * `state` (and, if ca != NULL, the pending conv inputs into conv_state) for the n_layers
 * layers, then set pending_len to 0 (device, on the stream, and the host mirror now).
 * A sequence with nothing pending is left bit-identical.
 * ---------------------------------------------------------------------------------- */
gdn_status gdn_flush(const gdn_verify_args *va, const gdn_conv_args *ca, int32_t *pending_host,
                     void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_TREE_H */
