// Driver of the commit's host-side path validation (plan_commit) for the sanitized host build:
// valid and malformed paths and offsets, every input in a heap block of exactly its size, so
// that any read past a caller's array or any signed overflow stops the run.  Prints "ok" and
// exits 0 when every case returns the expected status.
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <memory>
#include <vector>

#include "gdn_internal.h"

using gdn::CommitPlan;

static std::vector<int32_t> schedule_of(const std::vector<std::vector<int32_t>> &trees) {
    std::vector<int32_t> parents, offs{0};
    for (const auto &t : trees) {
        parents.insert(parents.end(), t.begin(), t.end());
        offs.push_back(offs.back() + int32_t(t.size()));
    }
    const int32_t S = int32_t(trees.size());
    std::vector<int32_t> image(gdn_schedule_words(S, offs.back()));
    if (gdn_hld_schedule(parents.data(), offs.data(), S, image.data(), image.size()) != GDN_OK) {
        std::printf("schedule failed: %s\n", gdn_last_error());
        std::exit(2);
    }
    return image;
}

// Runs plan_commit on exact-size heap copies of the arrays; returns the status.
static gdn_status run(const std::vector<int32_t> &image, const std::vector<int32_t> &paths,
                      const std::vector<int32_t> &offs, std::vector<int32_t> role, int32_t mode,
                      CommitPlan &plan) {
    std::unique_ptr<int32_t[]> p(paths.empty() ? nullptr : new int32_t[paths.size()]);
    for (size_t i = 0; i < paths.size(); ++i) p[i] = paths[i];
    std::unique_ptr<int32_t[]> o(new int32_t[offs.size()]);
    for (size_t i = 0; i < offs.size(); ++i) o[i] = offs[i];
    std::unique_ptr<int32_t[]> r(new int32_t[role.size()]);
    for (size_t i = 0; i < role.size(); ++i) r[i] = role[i];
    return gdn::plan_commit(image.data(), p.get(), o.get(), r.get(), mode, plan);
}

static int failures = 0;
static void expect(const char *what, gdn_status got, gdn_status want) {
    if (got != want) {
        std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, gdn_last_error());
        ++failures;
    }
}

int main() {
    const auto image = schedule_of({{-1, 0, 0, 1, 1, 2, 3}, {-1, 0, 1}});
    CommitPlan plan;
    const int32_t RM = GDN_COMMIT_ROW_MAP, CP = GDN_COMMIT_COMPACT;
    // valid: a branched path and an in-order path, in both modes
    expect("valid row map", run(image, {0, 1, 3, 6, 0, 1}, {0, 4, 6}, {0, 1}, RM, plan), GDN_OK);
    if (plan.role != std::vector<int32_t>{1, 0} || plan.pending != std::vector<int32_t>{4, 2})
        expect("row-map bookkeeping", GDN_EINVAL, GDN_OK);
    expect("valid compact", run(image, {0, 1, 3, 6, 0, 1}, {0, 4, 6}, {0, 1}, CP, plan), GDN_OK);
    if (!plan.any_compaction || plan.max_len != 4 || plan.role != std::vector<int32_t>{0, 0})
        expect("compact bookkeeping", GDN_EINVAL, GDN_OK);
    expect("empty paths", run(image, {}, {0, 0, 0}, {0, 0}, RM, plan), GDN_OK);
    // malformed
    expect("offsets[0] != 0", run(image, {0, 0}, {1, 1, 2}, {0, 0}, RM, plan), GDN_EPATH);
    expect("negative length", run(image, {0, 1}, {0, 2, 1}, {0, 0}, RM, plan), GDN_EPATH);
    expect("too long", run(image, {0, 1, 2, 0}, {0, 4, 4}, {0, 0}, RM, plan), GDN_EPATH);
    expect("overflowing length", run(image, {0}, {0, 1, INT_MIN}, {0, 0}, RM, plan), GDN_EPATH);
    expect("huge length", run(image, {0}, {0, INT_MAX, INT_MAX}, {0, 0}, RM, plan), GDN_EPATH);
    expect("not from the root", run(image, {1}, {0, 1, 1}, {0, 0}, RM, plan), GDN_EPATH);
    expect("broken link", run(image, {0, 2, 3}, {0, 3, 3}, {0, 0}, CP, plan), GDN_EPATH);
    expect("node out of range", run(image, {0, 7}, {0, 2, 2}, {0, 0}, RM, plan), GDN_EPATH);
    expect("negative node", run(image, {0, -1}, {0, 2, 2}, {0, 0}, RM, plan), GDN_EPATH);
    expect("repeated node", run(image, {0, 1, 1}, {0, 3, 3}, {0, 0}, RM, plan), GDN_EPATH);
    expect("bad role", run(image, {0}, {0, 1, 1}, {2, 0}, RM, plan), GDN_EINVAL);
    expect("unknown mode", run(image, {0}, {0, 1, 1}, {0, 0}, 7, plan), GDN_EINVAL);
    expect("null paths", gdn::plan_commit(image.data(), nullptr, std::vector<int32_t>{0, 1, 1}.data(),
                                          std::vector<int32_t>{0, 0}.data(), RM, plan),
           GDN_EINVAL);
    std::vector<int32_t> bad_image = image;
    bad_image[0] = 0;
    expect("bad image", run(bad_image, {0}, {0, 1, 1}, {0, 0}, RM, plan), GDN_EINVAL);
    if (failures == 0) std::printf("ok\n");
    return failures == 0 ? 0 : 1;
}
