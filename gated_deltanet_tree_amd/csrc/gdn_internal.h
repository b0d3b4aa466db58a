// Host-side internals shared by the library's translation units: error reporting, the
// schedule image view and launch limits.  Plain C++17, no HIP types.
#pragma once

#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/gdn_tree.h"

namespace gdn {

constexpr int32_t kImageMagic = 0x53444E47;
constexpr int32_t kImageHeader = 16;
constexpr int32_t kMaxTreeNodes = 1024;
// Largest grid of one verify or flush launch: the total work-item count of a dispatch
// (blocks x 256 threads at most) must fit in 32 bits, and the kernels' block arithmetic is
// 32-bit.
constexpr int64_t kMaxBlocks = 0xFFFFFFFFll / 256;
constexpr int32_t kMaxSeqs = 1 << 20;
// Record budget of the tree-masked verify plan in the schedule image, per node: a batch whose
// trees need more (sum of depth + 1 over its nodes > 32 T) gets no plan.
constexpr int32_t kUtRecordsPerNode = 32;

// Word offsets of the schedule image's arrays (see gdn_tree.h for the layout).
struct ImageView {
    int32_t n_seqs, n_nodes, n_chains, n_waves, n_boundaries, max_chain_len, max_tree;
    int64_t off_seq, off_wave, off_chain, off_cnodes, off_cseq, off_csrc, off_store,
        off_parent, off_depth;
    // tree-masked verify plan (ut_records < 0: absent)
    int32_t ut_records, ut_max_records, ut_max_levels;
    int64_t off_ut_rec_base, off_ut_node_rec, off_ut_lv_base, off_ut_lvn, off_ut_lvnode,
        off_ut_rec_anc;
};

size_t schedule_words(int32_t n_seqs, int32_t n_nodes);
ImageView view_image(const int32_t *img);
bool image_ok(const int32_t *img);

// Host bookkeeping of one commit (commit_host.cpp): new roles and pending lengths per
// sequence, whether any branched path needs the compacting gather, and its longest path.
struct CommitPlan {
    std::vector<int32_t> role, pending;
    bool any_compaction = false, any_path = false;
    int32_t max_len = 0;
};
// Checks the accepted paths (path_offsets [S+1], paths [path_offsets[S]]) against the trees of
// the schedule image and the roles, then fills `plan`.  GDN_EINVAL / GDN_EPATH on bad input.
gdn_status plan_commit(const int32_t *host_image, const int32_t *paths,
                       const int32_t *path_offsets, const int32_t *role_host, int32_t mode,
                       CommitPlan &plan);

// Per-thread last error; `fail` formats it and returns the status code.
void clear_error();
gdn_status fail(gdn_status code, const char *fmt, ...);

}  // namespace gdn
