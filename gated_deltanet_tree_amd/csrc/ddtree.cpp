// Best-first draft-tree builder (host): budget cap, confidence pruning, chain pre-seed.
//
// "Luce DFlash server README", How it works: the verified tree is a best-first tree of up to
// `budget` nodes over the top-K candidates of every draft position, optionally seeded with the
// greedy chain.  "Lucebox SpecLA and Gated DeltaNet state-resident verification" guide, the
// section on enabling it with one flag: tau is a confidence margin, and a node that scores
// below q* - tau is pruned.  Scores are fp32 sums of candidate log-probabilities along the
// path; q*(d) is the best score at depth d, which is the greedy chain's.
//
// The frontier is a binary heap of candidate children.  Its order is total: higher score,
// then smaller depth, then the lexicographically smaller sequence of candidate ranks along
// the path, packed 4 bits per position into one 64-bit key (position 1 in the top bits), so
// the tree is unique and equals "the best candidates in that order among those that survive
// pruning".  A popped candidate below its depth's threshold is dropped and never expanded,
// which prunes its subtree.
#include <cmath>
#include <cstdint>
#include <vector>

#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kMaxPositions = 16;
constexpr int kMaxTopK = 16;

struct Cand {
    float score;
    int32_t depth;
    uint64_t path;   // candidate ranks along the path, 4 bits each, position 1 highest
    int32_t parent;  // node id of the parent in the tree under construction
};

// True when a should be taken before b.
inline bool before(const Cand &a, const Cand &b) {
    if (a.score != b.score) return a.score > b.score;
    if (a.depth != b.depth) return a.depth < b.depth;
    return a.path < b.path;
}

class Frontier {
  public:
    void reset(size_t cap) {
        h_.clear();
        h_.reserve(cap);
    }
    bool empty() const { return h_.empty(); }
    void push(const Cand &c) {
        h_.push_back(c);
        size_t i = h_.size() - 1;
        while (i > 0) {
            const size_t p = (i - 1) / 2;
            if (!before(h_[i], h_[p])) break;
            std::swap(h_[i], h_[p]);
            i = p;
        }
    }
    Cand pop() {
        const Cand top = h_[0];
        h_[0] = h_.back();
        h_.pop_back();
        size_t i = 0;
        for (;;) {
            const size_t l = 2 * i + 1, r = l + 1;
            size_t best = i;
            if (l < h_.size() && before(h_[l], h_[best])) best = l;
            if (r < h_.size() && before(h_[r], h_[best])) best = r;
            if (best == i) break;
            std::swap(h_[i], h_[best]);
            i = best;
        }
        return top;
    }

  private:
    std::vector<Cand> h_;
};

inline uint64_t with_rank(uint64_t path, int depth, int k) {
    return path | (uint64_t(k) << (4 * (kMaxPositions - depth)));
}

}  // namespace

}  // namespace gdn

using namespace gdn;

extern "C" gdn_status gdn_ddtree_build(const float *logp, const int32_t *tokens,
                                       const int32_t *root_tokens, int32_t n_trees,
                                       int32_t n_positions, int32_t top_k, int32_t budget,
                                       float tau, int32_t chain_seed, int32_t *parent,
                                       int32_t *depth, int32_t *rank, int32_t *token,
                                       float *score, int32_t *n_nodes) {
    clear_error();
    const int L = n_positions, K = top_k;
    if (n_trees < 0 || L < 0 || L > kMaxPositions || K < 1 || K > kMaxTopK || budget < 1)
        return fail(GDN_EINVAL, "gdn_ddtree_build: need 0 <= n_positions <= %d, 1 <= top_k <= %d, "
                    "budget >= 1, n_trees >= 0", kMaxPositions, kMaxTopK);
    if (!(tau >= 0.f))
        return fail(GDN_EINVAL, "gdn_ddtree_build: tau must be >= 0 (INFINITY: no pruning)");
    if (n_trees == 0) return GDN_OK;
    if ((L > 0 && logp == nullptr) || parent == nullptr || depth == nullptr || rank == nullptr ||
        score == nullptr || n_nodes == nullptr || (token != nullptr && L > 0 && tokens == nullptr))
        return fail(GDN_EINVAL, "gdn_ddtree_build: null array");
    const int64_t per_tree = int64_t(L) * K;
    for (int64_t i = 0; i < int64_t(n_trees) * per_tree; ++i) {
        const float x = logp[i];
        if (!std::isfinite(x) || x > 0.f)
            return fail(GDN_EINVAL, "gdn_ddtree_build: log-probability %lld is not finite and <= 0",
                        (long long)i);
        if (i % K != 0 && x > logp[i - 1])
            return fail(GDN_EINVAL, "gdn_ddtree_build: candidates of a position must be sorted "
                        "by log-probability (entry %lld)", (long long)i);
    }

    Frontier frontier;
    std::vector<uint64_t> path(static_cast<size_t>(budget));
    float q[kMaxPositions + 1], thr[kMaxPositions + 1];
    for (int b = 0; b < n_trees; ++b) {
        const float *lp = logp + b * per_tree;
        int32_t *par = parent + int64_t(b) * budget, *dep = depth + int64_t(b) * budget;
        int32_t *rk = rank + int64_t(b) * budget;
        float *sc = score + int64_t(b) * budget;
        q[0] = 0.f;
        for (int d = 1; d <= L; ++d) q[d] = q[d - 1] + lp[(d - 1) * K];
        for (int d = 0; d <= L; ++d) thr[d] = std::isinf(tau) ? -INFINITY : q[d] - tau;

        int n = 0;
        auto add = [&](int32_t p, int32_t d, int32_t k, float s, uint64_t key) {
            par[n] = p;
            dep[n] = d;
            rk[n] = k;
            sc[n] = s;
            path[n] = key;
            ++n;
        };
        add(-1, 0, -1, 0.f, 0);
        const int chain = chain_seed ? (L < budget - 1 ? L : budget - 1) : 0;
        for (int d = 1; d <= chain; ++d) add(d - 1, d, 0, q[d], with_rank(path[d - 1], d, 0));

        frontier.reset(size_t(budget) * K + K);
        auto expand = [&](int node) {
            const int d = dep[node] + 1;
            if (d > L) return;
            for (int k = 0; k < K; ++k) {
                if (k == 0 && node < chain) continue;  // the next node of the seeded chain
                frontier.push(Cand{sc[node] + lp[(d - 1) * K + k], d,
                                   with_rank(path[node], d, k), node});
            }
        };
        for (int node = 0; node < n; ++node) expand(node);
        while (n < budget && !frontier.empty()) {
            const Cand c = frontier.pop();
            if (c.score < thr[c.depth]) continue;  // pruned with its whole subtree
            add(c.parent, c.depth, int32_t((c.path >> (4 * (kMaxPositions - c.depth))) & 15),
                c.score, c.path);
            expand(n - 1);
        }
        n_nodes[b] = n;
        if (token != nullptr) {
            int32_t *tk = token + int64_t(b) * budget;
            tk[0] = root_tokens != nullptr ? root_tokens[b] : -1;
            for (int i = 1; i < n; ++i) tk[i] = tokens[b * per_tree + (dep[i] - 1) * K + rk[i]];
            for (int i = n; i < budget; ++i) tk[i] = -1;
        }
        for (int i = n; i < budget; ++i) {
            par[i] = -1;
            dep[i] = -1;
            rk[i] = -1;
            sc[i] = 0.f;
        }
    }
    return GDN_OK;
}
