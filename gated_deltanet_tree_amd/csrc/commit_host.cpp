// Host side of accept -> commit (plain C++, no device work): the accepted paths are checked
// against their trees and the commit's bookkeeping (roles, pending lengths, whether a
// compaction is needed) is computed.  "Lucebox SpecLA and Gated DeltaNet state-resident
// verification" guide, mechanism 3: an accepted path is a root path of its tree; in-order
// acceptance swaps the bank roles, branched acceptance compacts the rows into path order.
#include "gdn_internal.h"

#include <algorithm>

namespace gdn {

gdn_status plan_commit(const int32_t *host_image, const int32_t *paths,
                       const int32_t *path_offsets, const int32_t *role_host, int32_t mode,
                       CommitPlan &plan) {
    if (!image_ok(host_image) || !path_offsets || !role_host)
        return fail(GDN_EINVAL, "gdn_commit_path: null argument or malformed schedule image");
    if (mode != GDN_COMMIT_COMPACT && mode != GDN_COMMIT_ROW_MAP)
        return fail(GDN_EINVAL, "gdn_commit_path: unknown mode %d", mode);
    const ImageView v = view_image(host_image);
    const int32_t S = v.n_seqs;
    plan = CommitPlan{};
    if (S == 0) return GDN_OK;
    if (path_offsets[0] != 0) return fail(GDN_EPATH, "gdn_commit_path: path_offsets[0] != 0");
    const int32_t *seq_off = host_image + v.off_seq, *npar = host_image + v.off_parent;
    plan.role.assign(role_host, role_host + S);
    plan.pending.assign(size_t(S), 0);
    for (int32_t b = 0; b < S; ++b) {
        // path b is paths[path_offsets[b] .. path_offsets[b + 1]); every earlier length was
        // checked non-negative, so beg >= 0 and the reads stay within paths[0 .. offsets[S])
        const int32_t beg = path_offsets[b];
        const int64_t L64 = int64_t(path_offsets[b + 1]) - beg;
        const int32_t n_b = seq_off[b + 1] - seq_off[b];
        if (L64 < 0 || L64 > n_b)
            return fail(GDN_EPATH, "gdn_commit_path: sequence %d: path length %lld not in "
                        "[0, %d]", b, (long long)L64, n_b);
        const int32_t L = int32_t(L64);
        if (L > 0 && paths == nullptr) return fail(GDN_EINVAL, "gdn_commit_path: null paths");
        if (role_host[b] != 0 && role_host[b] != 1)
            return fail(GDN_EINVAL, "gdn_commit_path: role[%d] = %d", b, role_host[b]);
        bool in_order = true;
        for (int32_t i = 0; i < L; ++i) {
            const int32_t node = paths[beg + i];
            if (node < 0 || node >= n_b)
                return fail(GDN_EPATH, "gdn_commit_path: sequence %d: node %d out of range", b,
                            node);
            const int32_t expect_parent = i == 0 ? -1 : seq_off[b] + paths[beg + i - 1];
            if (npar[seq_off[b] + node] != expect_parent)
                return fail(GDN_EPATH, "gdn_commit_path: sequence %d: path[%d] = %d does not "
                            "follow its parent", b, i, node);
            in_order = in_order && node == i;
        }
        plan.any_path = plan.any_path || L > 0;
        if (mode == GDN_COMMIT_ROW_MAP) {
            if (L > 0) plan.role[size_t(b)] ^= 1;
        } else {
            if (L > 0 && in_order) plan.role[size_t(b)] ^= 1;
            if (L > 0 && !in_order) plan.any_compaction = true;
            if (!in_order) plan.max_len = std::max(plan.max_len, L);
        }
        plan.pending[size_t(b)] = L;
    }
    return GDN_OK;
}

}  // namespace gdn
