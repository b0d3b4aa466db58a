// Heavy-light chain schedule of a batch of candidate trees (host, integer, deterministic).
//
// "Lucebox SpecLA and Gated DeltaNet state-resident verification" guide, mechanism 2: the
// tree is cut into heavy-light chains -- the child with the largest subtree continues its
// parent's chain, every other child starts a chain of its own -- only boundary states are
// materialised, and chains are grouped into dependency waves that run in parallel.  The
// schedule is a pure function of the parent arrays; its compact image is copied as-is to
// the device.  Rules fixed where the page is silent (heavy ties, ordering, slot numbering)
// are stated in gdn_tree.h next to the image layout.
#include "gdn_internal.h"

#include <algorithm>
#include <cstring>
#include <vector>

namespace gdn {

size_t schedule_words(int32_t n_seqs, int32_t n_nodes) {
    const size_t S = size_t(n_seqs), T = size_t(n_nodes);
    return size_t(kImageHeader) + 3 + S + 8 * T                // chains, waves, nodes
           + 2 + 3 * S + 3 * T + size_t(kUtRecordsPerNode) * T;  // tree-masked verify plan
}

ImageView view_image(const int32_t *img) {
    ImageView v;
    v.n_seqs = img[1];
    v.n_nodes = img[2];
    v.n_chains = img[3];
    v.n_waves = img[4];
    v.n_boundaries = img[5];
    v.max_chain_len = img[6];
    v.max_tree = img[7];
    const int64_t S = v.n_seqs, T = v.n_nodes;
    v.off_seq = kImageHeader;
    v.off_wave = kImageHeader + 1 + S;
    v.off_chain = kImageHeader + 2 + S + T;
    v.off_cnodes = kImageHeader + 3 + S + 2 * T;
    v.off_cseq = v.off_cnodes + T;
    v.off_csrc = v.off_cnodes + 2 * T;
    v.off_store = v.off_cnodes + 3 * T;
    v.off_parent = v.off_cnodes + 4 * T;
    v.off_depth = v.off_cnodes + 5 * T;
    v.ut_records = img[8];
    v.ut_max_records = img[9];
    v.ut_max_levels = img[10];
    v.off_ut_rec_base = v.off_depth + T;
    v.off_ut_node_rec = v.off_ut_rec_base + S + 1;
    v.off_ut_lv_base = v.off_ut_node_rec + T;
    v.off_ut_lvn = v.off_ut_lv_base + S + 1;
    v.off_ut_lvnode = v.off_ut_lvn + T + S;
    v.off_ut_rec_anc = v.off_ut_lvnode + T;
    return v;
}

bool image_ok(const int32_t *img) {
    return img != nullptr && img[0] == kImageMagic && img[1] >= 0 && img[2] >= img[1] &&
           img[3] >= 0 && img[4] >= 0 && img[5] >= 0;
}

}  // namespace gdn

using namespace gdn;

extern "C" size_t gdn_schedule_words(int32_t n_seqs, int32_t n_nodes_total) {
    if (n_seqs < 0 || n_nodes_total < 0) return 0;
    return schedule_words(n_seqs, n_nodes_total);
}

extern "C" gdn_status gdn_hld_schedule(const int32_t *parent_local, const int32_t *seq_offsets,
                                       int32_t n_seqs, int32_t *image, size_t image_words) {
    clear_error();
    if (n_seqs < 0 || (n_seqs > 0 && (parent_local == nullptr || seq_offsets == nullptr)) ||
        image == nullptr)
        return fail(GDN_EINVAL, "gdn_hld_schedule: null pointer or negative n_seqs");
    if (n_seqs > 0 && seq_offsets[0] != 0)
        return fail(GDN_EINVAL, "gdn_hld_schedule: seq_offsets[0] must be 0");
    for (int32_t b = 0; b < n_seqs; ++b) {
        // in 64 bits: a caller's offset can be any int32, and the difference must not overflow
        const int64_t n = int64_t(seq_offsets[b + 1]) - int64_t(seq_offsets[b]);
        if (n < 1) return fail(GDN_ETREE, "gdn_hld_schedule: tree %d has no nodes", b);
        if (n > kMaxTreeNodes)
            return fail(GDN_EINVAL, "gdn_hld_schedule: tree %d has %lld nodes (max %d)", b,
                        (long long)n, kMaxTreeNodes);
    }
    const int32_t T = n_seqs > 0 ? seq_offsets[n_seqs] : 0;
    const size_t words = schedule_words(n_seqs, T);
    if (image_words < words)
        return fail(GDN_ECAPACITY, "gdn_hld_schedule: image needs %zu words, got %zu", words,
                    image_words);
    for (int32_t b = 0; b < n_seqs; ++b) {
        const int32_t off = seq_offsets[b], n = seq_offsets[b + 1] - off;
        if (parent_local[off] != -1)
            return fail(GDN_ETREE, "gdn_hld_schedule: tree %d: parent[0] = %d, expected -1", b,
                        parent_local[off]);
        for (int32_t i = 1; i < n; ++i) {
            const int32_t p = parent_local[off + i];
            if (p < 0 || p >= i)
                return fail(GDN_ETREE, "gdn_hld_schedule: tree %d: parent[%d] = %d is not in [0,%d)",
                            b, i, p, i);
        }
    }

    // Per-node subtree size, heavy child, owning chain head and chain wave.
    std::vector<int32_t> size(T, 1), heavy(T, -1), head_of(T, -1), wave_of_head(T, -1);
    struct Chain { int32_t wave, seq, head; };
    std::vector<Chain> chains;
    int32_t max_tree = 0;
    for (int32_t b = 0; b < n_seqs; ++b) {
        const int32_t off = seq_offsets[b], n = seq_offsets[b + 1] - off;
        max_tree = std::max(max_tree, n);
        for (int32_t i = n - 1; i >= 1; --i) size[off + parent_local[off + i]] += size[off + i];
        for (int32_t i = 1; i < n; ++i) {  // ascending index: only a strictly larger size wins
            const int32_t p = off + parent_local[off + i];
            if (heavy[p] < 0 || size[off + i] > size[heavy[p]]) heavy[p] = off + i;
        }
        for (int32_t i = 0; i < n; ++i) {  // heads in ascending id: a parent's chain is known
            const int32_t g = off + i;
            if (i > 0 && heavy[off + parent_local[g]] == g) continue;
            const int32_t w = (i == 0) ? 0 : wave_of_head[head_of[off + parent_local[g]]] + 1;
            wave_of_head[g] = w;
            for (int32_t m = g; m >= 0; m = heavy[m]) head_of[m] = g;
            chains.push_back({w, b, g});
        }
    }
    std::stable_sort(chains.begin(), chains.end(), [](const Chain &a, const Chain &c) {
        if (a.wave != c.wave) return a.wave < c.wave;
        if (a.seq != c.seq) return a.seq < c.seq;
        return a.head < c.head;
    });

    std::memset(image, 0, words * sizeof(int32_t));
    image[0] = kImageMagic;
    image[1] = n_seqs;
    image[2] = T;
    ImageView v = view_image(image);
    int32_t *seq_off = image + v.off_seq, *wave_off = image + v.off_wave,
            *chain_off = image + v.off_chain, *cnodes = image + v.off_cnodes,
            *cseq = image + v.off_cseq, *csrc = image + v.off_csrc, *store = image + v.off_store,
            *npar = image + v.off_parent, *ndep = image + v.off_depth;
    for (int32_t b = 0; b <= n_seqs; ++b) seq_off[b] = n_seqs > 0 ? seq_offsets[b] : 0;
    for (int32_t b = 0; b < n_seqs; ++b) {
        const int32_t off = seq_offsets[b], n = seq_offsets[b + 1] - off;
        npar[off] = -1;
        ndep[off] = 0;
        for (int32_t i = 1; i < n; ++i) {
            npar[off + i] = off + parent_local[off + i];
            ndep[off + i] = ndep[off + parent_local[off + i]] + 1;
        }
    }
    // Boundary nodes: parents of light heads, slots by ascending global id.
    std::vector<char> is_boundary(T, 0);
    for (const Chain &c : chains)
        if (npar[c.head] >= 0) is_boundary[npar[c.head]] = 1;
    int32_t n_boundaries = 0;
    for (int32_t g = 0; g < T; ++g) store[g] = is_boundary[g] ? n_boundaries++ : -1;

    int32_t n_waves = 0, pos = 0, longest = 0;
    for (size_t c = 0; c < chains.size(); ++c) {
        const Chain &ch = chains[c];
        n_waves = std::max(n_waves, ch.wave + 1);
        chain_off[c] = pos;
        cseq[c] = ch.seq;
        csrc[c] = npar[ch.head] < 0 ? -1 : store[npar[ch.head]];
        const int32_t start = pos;
        for (int32_t m = ch.head; m >= 0; m = heavy[m]) cnodes[pos++] = m;
        longest = std::max(longest, pos - start);
    }
    chain_off[chains.size()] = pos;
    for (int32_t w = 0; w <= n_waves; ++w) wave_off[w] = 0;
    for (const Chain &c : chains) wave_off[c.wave + 1] += 1;
    for (int32_t w = 0; w < n_waves; ++w) wave_off[w + 1] += wave_off[w];

    image[3] = int32_t(chains.size());
    image[4] = n_waves;
    image[5] = n_boundaries;
    image[6] = longest;
    image[7] = max_tree;

    // Tree-masked verify plan: per tree, nodes by (depth, id) with the first position of each
    // depth level, and one block of depth + 1 records per node in that order (the node, then
    // its ancestors nearest first, local ids).
    int64_t records = 0;
    for (int32_t g = 0; g < T; ++g) records += ndep[g] + 1;
    if (records > int64_t(kUtRecordsPerNode) * T) {
        image[8] = -1;  // too deep for the plan budget: no tree-masked verify for this batch
        return GDN_OK;
    }
    v = view_image(image);
    int32_t *rec_base = image + v.off_ut_rec_base, *node_rec = image + v.off_ut_node_rec,
            *lv_base = image + v.off_ut_lv_base, *lvn = image + v.off_ut_lvn,
            *lvnode = image + v.off_ut_lvnode, *rec_anc = image + v.off_ut_rec_anc;
    int32_t max_records = 0, max_levels = 0;
    rec_base[0] = 0;
    lv_base[0] = 0;
    std::vector<int32_t> order;
    for (int32_t b = 0; b < n_seqs; ++b) {
        const int32_t off = seq_offsets[b], n = seq_offsets[b + 1] - off;
        int32_t dmax = 0;
        for (int32_t i = 0; i < n; ++i) dmax = std::max(dmax, ndep[off + i]);
        int32_t *first = lvn + lv_base[b];
        for (int32_t d = 0; d <= dmax + 1; ++d) first[d] = 0;
        for (int32_t i = 0; i < n; ++i) ++first[ndep[off + i] + 1];
        for (int32_t d = 0; d <= dmax; ++d) first[d + 1] += first[d];
        order.assign(size_t(n), 0);  // counting sort by depth, ids ascending within a level
        std::vector<int32_t> fill(first, first + dmax + 1);
        for (int32_t i = 0; i < n; ++i) order[fill[ndep[off + i]]++] = i;
        int32_t pos = 0;
        int32_t *recs = rec_anc + rec_base[b];
        for (int32_t j = 0; j < n; ++j) {
            const int32_t t = order[j];
            lvnode[off + j] = t;
            node_rec[off + t] = pos;
            for (int32_t a = t; a >= 0; a = parent_local[off + a]) recs[pos++] = a;  // root: -1
        }
        rec_base[b + 1] = rec_base[b] + pos;
        lv_base[b + 1] = lv_base[b] + dmax + 2;
        max_records = std::max(max_records, pos);
        max_levels = std::max(max_levels, dmax + 2);
    }
    image[8] = int32_t(records);
    image[9] = max_records;
    image[10] = max_levels;
    return GDN_OK;
}
