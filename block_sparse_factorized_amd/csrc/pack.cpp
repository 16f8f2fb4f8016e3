// pack.cpp -- host side of what libsa uploads (see pack.h): the device
// image of a layout -- the listings, the mask table and its transpose, the
// masks as per-register lane-mask planes of the 32x32 MFMA tiles, the block
// pairs with their per-step quadrant bits, the key-pair modes -- and the
// work lists of a call.  No HIP calls: capi.cpp uploads the results.
#include "pack.h"

#include <algorithm>
#include <cstring>
#include <numeric>

namespace sa {

int pack_layout(sa_layout* L, LayoutImage* img)
{
    const size_t nqb1 = (size_t)L->nqb + 1, nkb1 = (size_t)L->nkb + 1, nnz = (size_t)L->nnz;
    const size_t nwords = L->masks.size();
    // Sections, each 256-byte aligned: masks first (8-byte words).
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    size_t off_masks = 0;
    size_t off_masks_t = al(off_masks + nwords * 8);
    // Plane set 0 is all ones (a full block); mask m is set m + 1.
    const size_t nplanes = L->T == 64 ? (size_t)(L->n_masks + 1) * 64 : 0;
    size_t off_planes = al(off_masks_t + nwords * 8);
    size_t off_planes_t = al(off_planes + nplanes * 8);
    size_t off_row_ptr = al(off_planes_t + nplanes * 8);
    size_t off_col_idx = al(off_row_ptr + nqb1 * 4);
    size_t off_mask_id = al(off_col_idx + nnz * 4);
    size_t off_col_ptr = al(off_mask_id + nnz * 4);
    size_t off_row_idx = al(off_col_ptr + nkb1 * 4);
    size_t off_col_mask = al(off_row_idx + nnz * 4);
    const Groups* gs[2] = {&L->qgroups, &L->kgroups};
    size_t off_gptr[2], off_gblk[2], off_gstep[2];
    size_t cur = al(off_col_mask + nnz * 4);
    for (int k = 0; k < 2; ++k) {
        off_gptr[k] = cur;
        off_gblk[k] = al(off_gptr[k] + gs[k]->ptr.size() * 4);
        off_gstep[k] = al(off_gblk[k] + gs[k]->blk.size() * 4);
        cur = al(off_gstep[k] + gs[k]->step.size() * 4);
    }
    // Per key-block pair: which key halves each member's list ever touches.
    const size_t n_kgroups = L->kgroups.ptr.empty() ? 0 : L->kgroups.ptr.size() - 1;
    const size_t off_kmode = cur;
    cur = al(off_kmode + n_kgroups * 4);
    // Per key block: its pair and member.
    const size_t off_kblk = cur;
    cur = al(off_kblk + (size_t)L->nkb * 8);
    size_t total = cur;
    std::vector<unsigned char> host(total, 0);
    if (nwords) {
        memcpy(&host[off_masks], L->masks.data(), nwords * 8);
        // Transposed copies for kernels that walk a block by key column.
        const int64_t T = L->T, nw = T * T / 64;
        uint64_t* mt = (uint64_t*)&host[off_masks_t];
        for (int64_t m = 0; m < L->n_masks; ++m) {
            const uint64_t* src = &L->masks[m * nw];
            uint64_t* dst = mt + m * nw;
            for (int64_t r = 0; r < T; ++r)
                for (int64_t s2 = 0; s2 < T; ++s2) {
                    int64_t e = r * T + s2, f = s2 * T + r;
                    if ((src[e >> 6] >> (e & 63)) & 1ull) dst[f >> 6] |= 1ull << (f & 63);
                }
        }
    }
    if (nplanes) {
        uint64_t* pl = (uint64_t*)&host[off_planes];
        uint64_t* pt = (uint64_t*)&host[off_planes_t];
        std::fill(pl, pl + nplanes, ~0ull);
        std::fill(pt, pt + nplanes, ~0ull);
        auto bit = [&](int64_t m, int r, int s2) {
            int64_t e = (int64_t)r * 64 + s2;
            return (L->masks[m * 64 + (e >> 6)] >> (e & 63)) & 1ull;
        };
        for (int64_t m = 0; m < L->n_masks; ++m)
            for (int w = 0; w < 2; ++w)
                for (int reg = 0; reg < 32; ++reg) {
                    const int t = reg / 16, i = reg % 16;
                    uint64_t a = 0, b = 0;
                    for (int lane = 0; lane < 64; ++lane) {
                        const int inner = 32 * t + 8 * (i / 4) + 4 * (lane / 32) + i % 4;
                        const int outer = 32 * w + lane % 32;
                        a |= bit(m, outer, inner) << lane;
                        b |= bit(m, inner, outer) << lane;
                    }
                    pl[((m + 1) * 2 + w) * 32 + reg] = a;
                    pt[((m + 1) * 2 + w) * 32 + reg] = b;
                }
    }
    memcpy(&host[off_row_ptr], L->row_ptr.data(), nqb1 * 4);
    if (nnz) {
        memcpy(&host[off_col_idx], L->col_idx.data(), nnz * 4);
        memcpy(&host[off_mask_id], L->mask_id.data(), nnz * 4);
        memcpy(&host[off_row_idx], L->row_idx.data(), nnz * 4);
        std::vector<int32_t> col_mask(nnz);
        for (size_t a = 0; a < nnz; ++a) col_mask[a] = L->mask_id[L->csr_pos[a]];
        memcpy(&host[off_col_mask], col_mask.data(), nnz * 4);
    }
    memcpy(&host[off_col_ptr], L->col_ptr.data(), nkb1 * 4);
    // Quadrant occupancy of every mask (block size 64): bit 2*rh + ch of
    // quad: quadrant (query half rh, key half ch) has an allowed element; of
    // full: every element of it is allowed (its lane masks can be skipped).
    std::vector<uint8_t> quad((size_t)L->n_masks, 0), full((size_t)L->n_masks, 0), one1((size_t)L->n_masks, 0);
    if (L->T == 64)
        for (int64_t m = 0; m < L->n_masks; ++m) {
            uint32_t all = 0xFu;
            for (int r = 0; r < 64; ++r) {
                const uint64_t row = L->masks[m * 64 + r];  // query row r: bit s = key s
                const uint32_t lo = (uint32_t)row, hi = (uint32_t)(row >> 32);
                const int rh = r / 32;
                if (lo) quad[m] |= (uint8_t)(1u << (2 * rh));
                if (hi) quad[m] |= (uint8_t)(1u << (2 * rh + 1));
                if (lo != 0xffffffffu) all &= ~(1u << (2 * rh));
                if (hi != 0xffffffffu) all &= ~(1u << (2 * rh + 1));
            }
            full[m] = (uint8_t)all;
            // one[m]: the forward's lane (hh, query r) holds keys 32*ch + 8*g + 4*hh + e
            // (g, e < 4) of a quadrant; bit 2*rh + ch is set when every such
            // lane has at most one allowed key there.
            uint32_t one = 0xFu;
            for (int r = 0; r < 64; ++r) {
                const uint64_t row = L->masks[m * 64 + r];
                for (int ch = 0; ch < 2; ++ch)
                    for (int hh = 0; hh < 2; ++hh) {
                        int cnt = 0;
                        for (int g = 0; g < 4; ++g)
                            for (int e = 0; e < 4; ++e) cnt += (int)((row >> (32 * ch + 8 * g + 4 * hh + e)) & 1ull);
                        if (cnt > 1) one &= ~(1u << (2 * (r / 32) + ch));
                    }
            }
            one1[m] = (uint8_t)(one & ~all);
            if (one1[m] & quad[m]) L->one_quads = true;
        }
    auto quad_of = [&](int32_t m) -> uint32_t { return m == -1 ? 0xFu : m == -2 ? 0u : quad[m]; };
    auto full_of = [&](int32_t m) -> uint32_t { return m == -1 ? 0xFu : m == -2 ? 0u : full[m]; };
    auto one_of = [&](int32_t m) -> uint32_t { return m < 0 ? 0u : one1[m]; };
    int64_t pair_steps = 0, half_steps = 0;
    for (int k = 0; k < 2; ++k) {
        memcpy(&host[off_gptr[k]], gs[k]->ptr.data(), gs[k]->ptr.size() * 4);
        if (!gs[k]->blk.empty()) memcpy(&host[off_gblk[k]], gs[k]->blk.data(), gs[k]->blk.size() * 4);
        int32_t* st = (int32_t*)&host[off_gstep[k]];
        for (size_t x = 0; x < gs[k]->step.size(); x += 4) {
            st[x] = gs[k]->step[x];
            st[x + 1] = gs[k]->step[x + 1];
            st[x + 2] = gs[k]->step[x + 2];
            st[x + 3] = (int32_t)(quad_of(st[x + 1]) | quad_of(st[x + 2]) << 4 | full_of(st[x + 1]) << 8 |
                                  full_of(st[x + 2]) << 12 | one_of(st[x + 1]) << 16 | one_of(st[x + 2]) << 20);
            if (k == 0)
                for (int m = 0; m < 2; ++m)
                    for (int wr = 0; wr < 2; ++wr) {
                        const uint32_t lv = (quad_of(st[x + 1 + m]) >> (2 * wr)) & 3u;
                        const uint32_t o1 = (one_of(st[x + 1 + m]) >> (2 * wr)) & 3u;
                        if (lv == 3u && o1 != 3u)
                            ++pair_steps;
                        else if (lv != 0u)
                            ++half_steps;
                    }
        }
    }
    L->fwd_pair_steps = pair_steps;
    L->fwd_half_steps = half_steps;
    // Key-block pairs: a member whose list only ever has allowed elements in
    // one 32-key half gets mode 1 + that half (its two waves then share the
    // half and split the query halves), else mode 0.  Bits 0-1: member a,
    // bits 2-3: member b.
    {
        const int32_t* st = (const int32_t*)&host[off_gstep[1]];
        int32_t* km = (int32_t*)&host[off_kmode];
        for (size_t g = 0; g < n_kgroups; ++g) {
            uint32_t seen = 0;
            for (int32_t x = L->kgroups.ptr[g]; x < L->kgroups.ptr[g + 1]; ++x) seen |= (uint32_t)st[4 * x + 3];
            int32_t mode = 0;
            for (int m = 0; m < 2; ++m) {
                const uint32_t q = (seen >> (4 * m)) & 0xFu;
                const bool h0 = (q & 0x5u) != 0, h1 = (q & 0xAu) != 0;  // key half 0: bits 0, 2
                if (h0 != h1) mode |= (h0 ? 1 : 2) << (2 * m);
            }
            km[g] = mode;
        }
        int32_t* kg = (int32_t*)&host[off_kblk];
        for (int64_t b = 0; b < L->nkb; ++b) {
            kg[2 * b] = -1;
            kg[2 * b + 1] = 0;
        }
        for (size_t g = 0; g < n_kgroups; ++g)
            for (int m = 0; m < 2; ++m) {
                const int32_t b = L->kgroups.blk[2 * g + m];
                if (b >= 0 && b < L->nkb) {
                    kg[2 * b] = (int32_t)g;
                    kg[2 * b + 1] = m;
                }
            }
    }
    img->host = std::move(host);
    img->has_planes = nplanes != 0;
    img->off_masks = off_masks;
    img->off_masks_t = off_masks_t;
    img->off_planes = off_planes;
    img->off_planes_t = off_planes_t;
    img->off_row_ptr = off_row_ptr;
    img->off_col_idx = off_col_idx;
    img->off_mask_id = off_mask_id;
    img->off_col_ptr = off_col_ptr;
    img->off_row_idx = off_row_idx;
    img->off_col_mask = off_col_mask;
    img->off_kmode = off_kmode;
    img->off_kblk = off_kblk;
    for (int k = 0; k < 2; ++k) {
        img->off_gptr[k] = off_gptr[k];
        img->off_gblk[k] = off_gblk[k];
        img->off_gstep[k] = off_gstep[k];
    }
    return SA_OK;
}

DevLayout place_layout(const LayoutImage& img, const sa_layout* L, const unsigned char* b)
{
    DevLayout v;
    v.masks = (const uint64_t*)(b + img.off_masks);
    v.masks_t = (const uint64_t*)(b + img.off_masks_t);
    v.planes = img.has_planes ? (const uint64_t*)(b + img.off_planes) : nullptr;
    v.planes_t = img.has_planes ? (const uint64_t*)(b + img.off_planes_t) : nullptr;
    v.row_ptr = (const int32_t*)(b + img.off_row_ptr);
    v.col_idx = (const int32_t*)(b + img.off_col_idx);
    v.mask_id = (const int32_t*)(b + img.off_mask_id);
    v.col_ptr = (const int32_t*)(b + img.off_col_ptr);
    v.row_idx = (const int32_t*)(b + img.off_row_idx);
    v.col_mask = (const int32_t*)(b + img.off_col_mask);
    v.qgrp_ptr = (const int32_t*)(b + img.off_gptr[0]);
    v.qgrp_blk = (const int2*)(b + img.off_gblk[0]);
    v.qgrp_step = (const int4*)(b + img.off_gstep[0]);
    v.kgrp_ptr = (const int32_t*)(b + img.off_gptr[1]);
    v.kgrp_blk = (const int2*)(b + img.off_gblk[1]);
    v.kgrp_step = (const int4*)(b + img.off_gstep[1]);
    v.kgrp_mode = (const int32_t*)(b + img.off_kmode);
    v.kblk_grp = (const int2*)(b + img.off_kblk);
    v.vl = (int32_t)L->view_l;
    v.vm = (int32_t)L->view_m;
    v.kcl = L->key_cl;
    v.kgl = L->key_gl;
    v.koff = L->key_off;
    v.km = (int32_t)L->key_m;
    return v;
}

void build_work_items(ListKind kind, int32_t B, int32_t H, sa_layout* const* hl, int32_t compact_steps,
                      int32_t plain_steps, int32_t plain_min, std::vector<Item>* out, Split* split)
{
    auto listing = [&](const sa_layout* L) -> const std::vector<int32_t>& {
        switch (kind) {
        case kByQuery: return L->row_ptr;
        case kByQueryPair:
        case kByQueryPairDq: return L->qgroups.ptr;
        default: return L->kgroups.ptr;
        }
    };
    const bool pairs = kind != kByQuery;
    Split local;
    Split& sp = split ? *split : local;
    sp = Split();
    std::vector<Item> items;
    std::vector<int32_t> cost;
    // One chunk: an item, a slot and its table entry.
    auto add_chunk = [&](int32_t bh, int32_t blk, int32_t first, int32_t steps) {
        const int32_t slot = (int32_t)sp.slots++;
        sp.chunk_tab.push_back(make_int2(first, steps));
        items.push_back(Item{bh, blk, 0, slot});
        cost.push_back(steps);
    };
    for (int32_t bh = 0; bh < B * H; ++bh) {
        const sa_layout* L = hl[bh % H];
        const std::vector<int32_t>& ptr = listing(L);
        if (kind == kByKeyPair && compact_steps > 0 && is_compact(L)) {
            // every key-block pair of a compact view, in chunks of compact_steps
            sp.cheads.push_back(make_int2(bh, (int32_t)sp.cgroups.size()));
            for (int64_t blk = 0; blk + 1 < (int64_t)ptr.size(); ++blk) {
                const int32_t len = ptr[blk + 1] - ptr[blk];
                const int32_t chunks = std::max<int32_t>(1, (len + compact_steps - 1) / compact_steps);
                sp.cgroups.push_back(make_int2((int32_t)sp.slots, chunks));
                for (int32_t c = 0; c < chunks; ++c)
                    add_chunk(bh, (int32_t)blk, c * compact_steps, std::min(compact_steps, len - c * compact_steps));
            }
            continue;
        }
        // (a residue view walks its dense causal layout once per residue class)
        for (int64_t r = 0; r < L->view_l; ++r)
            for (int64_t blk = 0; blk + 1 < (int64_t)ptr.size(); ++blk) {
                const int32_t len = ptr[blk + 1] - ptr[blk];
                if (pairs && plain_steps > 0 && L->view_l == 1 && len > std::max(plain_min, plain_steps)) {
                    // near-equal chunks: chunk c walks steps [c*len/k, (c+1)*len/k)
                    const int32_t k = (len + plain_steps - 1) / plain_steps;
                    sp.groups.push_back(make_int4(bh, (int32_t)blk, (int32_t)sp.slots, k));
                    for (int32_t c = 0; c < k; ++c) {
                        const int32_t f0 = (int32_t)((int64_t)c * len / k), f1 = (int32_t)((int64_t)(c + 1) * len / k);
                        add_chunk(bh, (int32_t)blk, f0, f1 - f0);
                    }
                    continue;
                }
                items.push_back(Item{bh, (int32_t)blk, (int32_t)r, -1});
                cost.push_back(len);
            }
    }
    std::vector<size_t> order(items.size());
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](size_t u, size_t v) { return cost[u] > cost[v]; });
    std::vector<Item> sorted(items.size());
    for (size_t x = 0; x < items.size(); ++x) sorted[x] = items[order[x]];
    *out = std::move(sorted);
}

}  // namespace sa
