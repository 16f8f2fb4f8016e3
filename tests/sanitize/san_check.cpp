// san_check.cpp -- libsa's host code under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_sanitize.py with g++ on
// the CPU; no GPU, no HIP runtime): the layout builder, the residue and
// compact views, the device image of every layout (listings, mask tables,
// lane-mask planes, block pairs and their step records, key-pair modes) and
// the work lists, over seeded random layouts and the full-size workloads.
// Each image is also checked for self-consistency: its sections lie inside
// the buffer, in order, and the step records point at valid masks.
// Exit status 0 when every check passes (a sanitizer report aborts).
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <vector>

#include "pack.h"
#include "sa_internal.h"

using namespace sa;

namespace {

uint64_t g_state = 0x5eed5eed2019ull;
uint64_t next()  // splitmix64
{
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
int64_t pick(int64_t lo, int64_t hi) { return lo + (int64_t)(next() % (uint64_t)(hi - lo + 1)); }

int g_fail = 0;
#define CHECK(cond, ...)                                 \
    do {                                                 \
        if (!(cond)) {                                   \
            std::fprintf(stderr, "check failed: " #cond " -- " __VA_ARGS__); \
            std::fprintf(stderr, "\n");                  \
            ++g_fail;                                    \
        }                                                \
    } while (0)

void check_image(sa_layout* L, const char* what)
{
    LayoutImage img;
    CHECK(pack_layout(L, &img) == SA_OK, "%s", what);
    const size_t total = img.host.size();
    const size_t offs[] = {img.off_masks, img.off_masks_t, img.off_planes, img.off_planes_t, img.off_row_ptr,
                           img.off_col_idx, img.off_mask_id, img.off_col_ptr, img.off_row_idx, img.off_col_mask,
                           img.off_gptr[0], img.off_gblk[0], img.off_gstep[0], img.off_gptr[1], img.off_gblk[1],
                           img.off_gstep[1], img.off_kmode};
    for (size_t a = 0; a < sizeof offs / sizeof offs[0]; ++a) {
        CHECK(offs[a] % 256 == 0 && offs[a] <= total, "%s: section %zu at %zu of %zu", what, a, offs[a], total);
        if (a) CHECK(offs[a] >= offs[a - 1], "%s: section %zu out of order", what, a);
    }
    CHECK(img.has_planes == (L->T == 64), "%s", what);
    const DevLayout v = place_layout(img, L, img.host.data());
    // Every step record names a mask that exists (or -1 full, -2 absent)
    // and a block inside the layout.
    for (int k = 0; k < 2; ++k) {
        const Groups& g = k == 0 ? L->qgroups : L->kgroups;
        const int32_t* ptr = k == 0 ? v.qgrp_ptr : v.kgrp_ptr;
        const int4* st = k == 0 ? v.qgrp_step : v.kgrp_step;
        const int64_t ng = (int64_t)g.ptr.size() - 1;
        for (int64_t gi = 0; gi < ng; ++gi)
            for (int32_t x = ptr[gi]; x < ptr[gi + 1]; ++x) {
                CHECK(st[x].x >= 0 && st[x].x < (k == 0 ? L->nkb : L->nqb), "%s: step block %d", what, st[x].x);
                CHECK(st[x].y >= -2 && st[x].y < L->n_masks, "%s: mask a %d", what, st[x].y);
                CHECK(st[x].z >= -2 && st[x].z < L->n_masks, "%s: mask b %d", what, st[x].z);
            }
    }
    for (ListKind kind : {kByQuery, kByQueryPair, kByKeyPair, kByQueryPairDq})
        for (int32_t B : {1, 3}) {
            sa_layout* hl[2] = {L, L};
            std::vector<Item> items;
            build_work_items(kind, B, 2, hl, 0, 0, 0, &items);
            const size_t per = kind == kByQuery ? L->row_ptr.size() - 1
                               : kind == kByKeyPair ? L->kgroups.ptr.size() - 1
                                                    : L->qgroups.ptr.size() - 1;
            CHECK(items.size() == (size_t)B * 2 * per * (size_t)L->view_l, "%s: %zu items", what, items.size());
            for (const Item& it : items)
                CHECK(it.bh >= 0 && it.bh < B * 2 && it.blk >= 0 && (size_t)it.blk < per && it.r >= 0 &&
                          it.r < L->view_l && it.slot == -1,
                      "%s: item", what);
        }
    // Chunked lists: every chunk inside its list, the chunks of a list
    // covering it exactly and in order, slots distinct and each named by
    // one item, the tables consistent.  Compact views' dK/dV lists in chunks
    // of compact_steps; other layouts' lists (not residue views) longer than
    // the threshold in near-equal chunks of at most plain_steps.
    for (ListKind kind : {kByQueryPair, kByKeyPair, kByQueryPairDq})
        for (int32_t steps : {1, 7, 64}) {
            sa_layout* hl[2] = {L, L};
            std::vector<Item> items;
            Split sp;
            const int32_t cst = kind == kByKeyPair ? steps : 0;
            const int32_t pmin = steps == 1 ? 3 : steps;
            build_work_items(kind, 2, 2, hl, cst, steps, pmin, &items, &sp);
            const std::vector<int32_t>& ptr = kind == kByKeyPair ? L->kgroups.ptr : L->qgroups.ptr;
            const size_t ng = ptr.size() - 1;
            const bool compact = kind == kByKeyPair && is_compact(L);
            CHECK((int64_t)sp.chunk_tab.size() == sp.slots, "%s: chunk table", what);
            if (compact) CHECK(sp.cheads.size() == 4 && sp.cgroups.size() == 4 * ng && sp.groups.empty(), "%s: compact tables", what);
            else CHECK(sp.cheads.empty() && sp.cgroups.empty(), "%s: no compact tables", what);
            if (L->view_l > 1) CHECK(sp.slots == 0, "%s: residue views are not chunked", what);
            std::vector<int> seen((size_t)sp.slots, 0);
            size_t plain_items = 0;
            for (const Item& it : items) {
                CHECK(it.blk >= 0 && (size_t)it.blk < ng, "%s: item block", what);
                if (it.slot < 0) {
                    ++plain_items;
                    const int32_t len = ptr[it.blk + 1] - ptr[it.blk];
                    CHECK(compact == false && (L->view_l > 1 || len <= std::max(pmin, steps)), "%s: unchunked long list", what);
                    continue;
                }
                CHECK(it.slot < sp.slots && it.r == 0, "%s: chunk item", what);
                if (it.slot >= sp.slots) continue;
                ++seen[(size_t)it.slot];
            }
            for (int x : seen) CHECK(x == 1, "%s: slot used %d times", what, x);
            // every list's chunks, through its table entry
            auto cover = [&](int32_t blk, int32_t first, int32_t chunks, int32_t cap, bool equal) {
                const int32_t len = ptr[blk + 1] - ptr[blk];
                int32_t at = 0, lo = INT32_MAX, hi = 0;
                for (int32_t c = 0; c < chunks; ++c) {
                    CHECK(first + c < sp.slots, "%s: chunk slot", what);
                    if (first + c >= sp.slots) return;
                    const int2 ct = sp.chunk_tab[(size_t)(first + c)];
                    CHECK(ct.x == at && ct.y >= 0 && ct.y <= cap, "%s: chunk %d of list %d: {%d, %d} at %d", what, c, blk, ct.x, ct.y, at);
                    at += ct.y;
                    lo = std::min(lo, ct.y);
                    hi = std::max(hi, ct.y);
                }
                CHECK(at == len, "%s: chunks cover %d of %d steps", what, at, len);
                if (equal) CHECK(chunks >= 2 && hi - lo <= 1, "%s: chunks not near-equal", what);
            };
            for (const int2& h : sp.cheads)
                for (size_t gi = 0; gi < ng; ++gi) {
                    const int2 gs = sp.cgroups[(size_t)h.y + gi];
                    const int32_t len = ptr[gi + 1] - ptr[gi];
                    CHECK(gs.y == std::max<int32_t>(1, (len + steps - 1) / steps), "%s: chunk count", what);
                    cover((int32_t)gi, gs.x, gs.y, steps, false);
                }
            for (const int4& g : sp.groups) {
                CHECK(g.x >= 0 && g.x < 4 && g.y >= 0 && (size_t)g.y < ng, "%s: group", what);
                if (g.y < 0 || (size_t)g.y >= ng) continue;
                const int32_t len = ptr[g.y + 1] - ptr[g.y];
                CHECK(len > std::max(pmin, steps) && g.w == (len + steps - 1) / steps, "%s: group chunks", what);
                cover(g.y, g.z, g.w, steps, true);
            }
            CHECK(plain_items + (size_t)sp.slots == items.size(), "%s: item count", what);
        }
}

void run_case(int pattern, int64_t n, int64_t l, int64_t c, int32_t T)
{
    char what[160];
    std::snprintf(what, sizeof what, "pattern %d n %lld l %lld c %lld T %d", pattern, (long long)n, (long long)l,
                  (long long)c, T);
    sa_layout* L = nullptr;
    const int st = build_layout(pattern, n, l, c, T, &L);
    CHECK(st == SA_OK, "%s: build %d (%s)", what, st, last_error());
    if (st != SA_OK) return;
    CHECK((int64_t)L->row_ptr.size() == L->nqb + 1 && L->row_ptr.back() == L->nnz, "%s", what);
    check_image(L, what);
    if (T == 64 && pattern == SA_STRIDED_B && n % l == 0) {
        sa_layout* rv = nullptr;
        CHECK(build_residue_view(n, l, &rv) == SA_OK, "%s: residue view", what);
        if (rv) {
            // l classes of a dense causal attention over n / l rows: the same pairs
            const int64_t m = n / l;
            CHECK(rv->allowed >= m * (m + 1) / 2, "%s: residue view pairs", what);
            check_image(rv, what);
            delete rv;
        }
    }
    if (T == 64 && pattern == SA_FIXED_B && n % l == 0 && (c & (c - 1)) == 0) {
        sa_layout* cv = nullptr;
        CHECK(build_compact_view(n, l, c, &cv) == SA_OK, "%s: compact view", what);
        if (cv) {
            CHECK(cv->allowed == L->allowed, "%s: compact view pairs %lld vs %lld", what, (long long)cv->allowed,
                  (long long)L->allowed);
            check_image(cv, what);
            delete cv;
        }
    }
    delete L;
}

}  // namespace

int main(int argc, char** argv)
{
    const int count = argc > 1 ? std::atoi(argv[1]) : 200;
    // Seeded random layouts: every pattern, block sizes of the kernels and of
    // the builder, strides and summary widths anywhere in range.
    const int32_t blocks[] = {8, 16, 32, 64, 64, 64, 128};
    for (int a = 0; a < count; ++a) {
        const int pattern = (int)pick(0, 4);
        const int32_t T = blocks[pick(0, 6)];
        const int64_t n = T * pick(1, T == 64 ? 48 : 24);
        const int64_t l = pick(0, 3) == 0 ? pick(1, 2 * n) : (int64_t)1 << pick(0, 8);
        int64_t c = pattern == SA_FIXED_B ? pick(1, l) : 1;
        if (pattern == SA_FIXED_B && pick(0, 1)) c = std::min<int64_t>(l, (int64_t)1 << pick(0, 7));
        run_case(pattern, n, l, c, T);
    }
    // The workloads' layouts at full size (block 64).
    run_case(SA_STRIDED_A, 3072, 128, 1, 64);
    run_case(SA_STRIDED_B, 3072, 128, 1, 64);
    run_case(SA_FIXED_A, 12288, 128, 32, 64);
    run_case(SA_FIXED_B, 12288, 128, 32, 64);
    run_case(SA_STRIDED_A, 12288, 128, 1, 64);
    run_case(SA_STRIDED_B, 12288, 128, 1, 64);
    run_case(SA_DENSE_CAUSAL, 12288, 1, 1, 64);
    run_case(SA_STRIDED_A, 65536, 256, 1, 64);
    run_case(SA_STRIDED_B, 65536, 256, 1, 64);
    // Rejected arguments return errors, and write nothing.
    sa_layout* L = nullptr;
    CHECK(build_layout(SA_FIXED_B, 256, 16, 17, 64, &L) == SA_ERR_INVALID_ARG && L == nullptr, "c > l");
    CHECK(build_layout(SA_STRIDED_A, 100, 16, 1, 64, &L) == SA_ERR_INVALID_ARG && L == nullptr, "n % block");
    CHECK(build_residue_view(1000, 7, &L) == SA_ERR_UNSUPPORTED && L == nullptr, "residue n % l");
    CHECK(build_compact_view(1024, 128, 24, &L) == SA_ERR_UNSUPPORTED && L == nullptr, "compact c not 2^k");
    std::printf("%d cases, %d failed checks\n", count + 9, g_fail);
    return g_fail ? 1 : 0;
}
