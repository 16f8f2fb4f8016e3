// capi.cpp -- the extern "C" entry points of libsa: argument checks, layout
// upload, work lists, kernel dispatch and error reporting.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "kernel_args.h"
#include "sa_internal.h"

namespace sa {

namespace {
thread_local std::string g_last_error;
}

int fail(int status, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

namespace {

int hip_fail(hipError_t e, const char* what)
{
    return fail(SA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// Upload a layout to the current device once; later calls return the view.
int device_layout(sa_layout* L, int dev, DevLayout* out)
{
    std::lock_guard<std::mutex> g(L->mu);
    auto it = L->dev.find(dev);
    if (it != L->dev.end()) {
        *out = it->second;
        return SA_OK;
    }
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
    }
    void* mem = nullptr;
    hipError_t e = hipMalloc(&mem, total);
    if (e != hipSuccess) return fail(SA_ERR_ALLOC, "layout upload: hipMalloc(%zu): %s", total, hipGetErrorString(e));
    e = hipMemcpy(mem, host.data(), total, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(mem);
        return hip_fail(e, "layout upload: hipMemcpy");
    }
    unsigned char* b = (unsigned char*)mem;
    DevLayout v;
    v.masks = (const uint64_t*)(b + off_masks);
    v.masks_t = (const uint64_t*)(b + off_masks_t);
    v.planes = nplanes ? (const uint64_t*)(b + off_planes) : nullptr;
    v.planes_t = nplanes ? (const uint64_t*)(b + off_planes_t) : nullptr;
    v.row_ptr = (const int32_t*)(b + off_row_ptr);
    v.col_idx = (const int32_t*)(b + off_col_idx);
    v.mask_id = (const int32_t*)(b + off_mask_id);
    v.col_ptr = (const int32_t*)(b + off_col_ptr);
    v.row_idx = (const int32_t*)(b + off_row_idx);
    v.col_mask = (const int32_t*)(b + off_col_mask);
    v.qgrp_ptr = (const int32_t*)(b + off_gptr[0]);
    v.qgrp_blk = (const int2*)(b + off_gblk[0]);
    v.qgrp_step = (const int4*)(b + off_gstep[0]);
    v.kgrp_ptr = (const int32_t*)(b + off_gptr[1]);
    v.kgrp_blk = (const int2*)(b + off_gblk[1]);
    v.kgrp_step = (const int4*)(b + off_gstep[1]);
    v.kgrp_mode = (const int32_t*)(b + off_kmode);
    v.vl = (int32_t)L->view_l;
    v.vm = (int32_t)L->view_m;
    v.kcl = L->key_cl;
    v.kgl = L->key_gl;
    v.koff = L->key_off;
    v.km = (int32_t)L->key_m;
    L->dev_mem[dev] = mem;
    L->dev[dev] = v;
    *out = v;
    return SA_OK;
}

// ---------------------------------------------------------------------------
// Work lists.  One item per (batch*head, block or block pair); ordered longest first so the
// heaviest blocks start early and the tail is made of short ones.  Cached per
// (kind, device, B, H, layouts).
enum ListKind { kByQuery = 0, kByQueryPair = 1, kByKeyPair = 2 };

struct Plan {
    Item* items;
    int count;
    int dev;
};

std::mutex g_plan_mu;
std::map<std::string, Plan> g_plans;
// layout serial -> keys of the cached work lists that name it; destroying the
// layout frees them (sa_layout_destroy), so a process that keeps building and
// destroying layouts does not accumulate work lists.
std::map<uint64_t, std::vector<std::string>> g_plan_keys;

int get_plan(ListKind kind, int dev, int32_t B, int32_t H, sa_layout* const* hl, Plan* out)
{
    std::string key = std::to_string(kind) + ":" + std::to_string(dev) + ":" + std::to_string(B) + ":" +
                      std::to_string(H);
    for (int32_t h = 0; h < H; ++h) key += ":" + std::to_string(hl[h]->serial);
    std::lock_guard<std::mutex> g(g_plan_mu);
    auto it = g_plans.find(key);
    if (it != g_plans.end()) {
        *out = it->second;
        return SA_OK;
    }
    auto listing = [&](const sa_layout* L) -> const std::vector<int32_t>& {
        switch (kind) {
        case kByQuery: return L->row_ptr;
        case kByQueryPair: return L->qgroups.ptr;
        default: return L->kgroups.ptr;
        }
    };
    // (a residue view walks its dense causal layout once per residue class)
    int64_t count = 0;
    for (int32_t bh = 0; bh < B * H; ++bh)
        count += ((int64_t)listing(hl[bh % H]).size() - 1) * hl[bh % H]->view_l;
    std::vector<Item> items((size_t)count);
    std::vector<int32_t> cost((size_t)count);
    size_t x = 0;
    for (int32_t bh = 0; bh < B * H; ++bh) {
        const sa_layout* L = hl[bh % H];
        const std::vector<int32_t>& ptr = listing(L);
        for (int64_t r = 0; r < L->view_l; ++r)
            for (int64_t blk = 0; blk + 1 < (int64_t)ptr.size(); ++blk, ++x) {
                items[x] = Item{bh, (int32_t)blk, (int32_t)r, 0};
                cost[x] = ptr[blk + 1] - ptr[blk];
            }
    }
    std::vector<size_t> order((size_t)count);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](size_t u, size_t v) { return cost[u] > cost[v]; });
    std::vector<Item> sorted((size_t)count);
    for (size_t a = 0; a < (size_t)count; ++a) sorted[a] = items[order[a]];
    void* mem = nullptr;
    hipError_t e = hipMalloc(&mem, sorted.size() * sizeof(Item));
    if (e != hipSuccess) return fail(SA_ERR_ALLOC, "work list: hipMalloc: %s", hipGetErrorString(e));
    e = hipMemcpy(mem, sorted.data(), sorted.size() * sizeof(Item), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(mem);
        return hip_fail(e, "work list: hipMemcpy");
    }
    Plan p{(Item*)mem, (int)count, dev};
    g_plans[key] = p;
    for (int32_t h = 0; h < H; ++h) {
        std::vector<std::string>& keys = g_plan_keys[hl[h]->serial];
        if (keys.empty() || keys.back() != key) keys.push_back(key);
    }
    *out = p;
    return SA_OK;
}

// Frees the cached work lists that name layout `serial`.
void release_plans(uint64_t serial)
{
    std::lock_guard<std::mutex> g(g_plan_mu);
    auto it = g_plan_keys.find(serial);
    if (it == g_plan_keys.end()) return;
    for (const std::string& key : it->second) {
        auto p = g_plans.find(key);
        if (p == g_plans.end()) continue;
        int cur = 0;
        if (hipGetDevice(&cur) == hipSuccess && hipSetDevice(p->second.dev) == hipSuccess) {
            (void)hipFree(p->second.items);
            (void)hipSetDevice(cur);
        }
        g_plans.erase(p);
    }
    g_plan_keys.erase(it);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Checks shared by sa_fwd and sa_bwd; fills the head table.
// compact: walk compact views (the forward and dQ kernels); the dK/dV
// kernel walks those layouts in their raster form, whose key blocks have
// more and shorter query lists (the compact view's first key blocks are
// listed by almost every query block, and a few long workgroups would set
// the launch time).
int common_checks(const char* fn, const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n,
                  int32_t d, int dtype, float scale, bool backward, bool compact, HeadTable* ht,
                  std::vector<sa_layout*>* hl, sa_layout** distinct_out, int* n_distinct)
{
    if (!head_layout) return fail(SA_ERR_INVALID_ARG, "%s: head_layout is NULL", fn);
    if (B < 1 || H < 1) return fail(SA_ERR_INVALID_ARG, "%s: B = %d, H = %d must be >= 1", fn, B, H);
    if (H > kMaxHeads) return fail(SA_ERR_INVALID_ARG, "%s: H = %d exceeds %d", fn, H, kMaxHeads);
    if (n < 1 || d < 1) return fail(SA_ERR_INVALID_ARG, "%s: n = %lld, d = %d must be >= 1", fn, (long long)n, d);
    if (dtype != SA_F32 && dtype != SA_BF16) return fail(SA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(SA_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
    const int32_t block = dtype == SA_F32 ? 16 : 64;
    bool ok;
    if (dtype == SA_F32)
        ok = !backward && d == 64;
    else
        ok = d == 64 || d == 128;
    if (!ok)
        return fail(SA_ERR_UNSUPPORTED, "%s: no kernel for dtype %s, d = %d%s", fn, dtype == SA_F32 ? "f32" : "bf16", d,
                    backward && dtype == SA_F32 ? " (backward is bf16 only)" : "");
    hl->assign(H, nullptr);
    int nl = 0;
    sa_layout* distinct[kMaxLayouts];
    for (int32_t h = 0; h < H; ++h) {
        sa_layout* L = const_cast<sa_layout*>(head_layout[h]);
        if (!L) return fail(SA_ERR_INVALID_ARG, "%s: head_layout[%d] is NULL", fn, h);
        if (L->n != n)
            return fail(SA_ERR_INVALID_ARG, "%s: head_layout[%d] was built for n = %lld, call has n = %lld", fn, h,
                        (long long)L->n, (long long)n);
        if (L->T != block)
            return fail(SA_ERR_UNSUPPORTED, "%s: head_layout[%d] has block %d; %s kernels need block %d", fn, h, L->T,
                        dtype == SA_F32 ? "f32" : "bf16", block);
        if (L->view && (compact || L->view_kind != 2)) L = L->view;  // the kernels walk the view
        int idx = -1;
        for (int a = 0; a < nl; ++a)
            if (distinct[a] == L) idx = a;
        if (idx < 0) {
            if (nl == kMaxLayouts)
                return fail(SA_ERR_INVALID_ARG, "%s: more than %d distinct layouts in one call", fn, kMaxLayouts);
            distinct[nl] = L;
            idx = nl++;
        }
        ht->head_lay[h] = (uint8_t)idx;
        (*hl)[h] = L;
    }
    int64_t max_items = 0;
    for (int32_t h = 0; h < H; ++h) max_items += (*hl)[h]->nqb * (*hl)[h]->view_l;
    if ((int64_t)B * max_items > (int64_t)1 << 30)
        return fail(SA_ERR_UNSUPPORTED, "%s: %lld work items is too many for one launch", fn,
                    (long long)((int64_t)B * max_items));
    *n_distinct = nl;
    for (int a = 0; a < nl; ++a) distinct_out[a] = distinct[a];
    return SA_OK;
}

// Device side of a call: current device, layouts uploaded, head table filled.
int prepare_device(sa_layout* const* distinct, int nl, HeadTable* ht, int* dev_out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    for (int a = 0; a < nl; ++a) {
        int st = device_layout(distinct[a], dev, &ht->lay[a]);
        if (st != SA_OK) return st;
    }
    for (int a = nl; a < kMaxLayouts; ++a) ht->lay[a] = ht->lay[0];
    *dev_out = dev;
    return SA_OK;
}

}  // namespace
}  // namespace sa

using namespace sa;

extern "C" {

int sa_layout_build(int pattern, int64_t n, int64_t l, int64_t c, int32_t block, sa_layout_t** out)
{
    return build_layout(pattern, n, l, c, block, out);
}

int sa_layout_info(const sa_layout_t* lay, int64_t* nqb, int64_t* nnz, int64_t* n_masks, int64_t* allowed_pairs)
{
    if (!lay) return fail(SA_ERR_INVALID_ARG, "sa_layout_info: layout is NULL");
    if (nqb) *nqb = lay->nqb;
    if (nnz) *nnz = lay->nnz;
    if (n_masks) *n_masks = lay->n_masks;
    if (allowed_pairs) *allowed_pairs = lay->allowed;
    return SA_OK;
}

int sa_layout_export(const sa_layout_t* lay, int32_t* row_ptr, int32_t* col_idx, int32_t* mask_id,
                     uint64_t* mask_words, int32_t* col_ptr, int32_t* row_idx, int32_t* csr_pos)
{
    if (!lay) return fail(SA_ERR_INVALID_ARG, "sa_layout_export: layout is NULL");
    auto cp = [](void* dst, const void* src, size_t bytes) {
        if (dst && bytes) memcpy(dst, src, bytes);
    };
    cp(row_ptr, lay->row_ptr.data(), lay->row_ptr.size() * 4);
    cp(col_idx, lay->col_idx.data(), lay->col_idx.size() * 4);
    cp(mask_id, lay->mask_id.data(), lay->mask_id.size() * 4);
    cp(mask_words, lay->masks.data(), lay->masks.size() * 8);
    cp(col_ptr, lay->col_ptr.data(), lay->col_ptr.size() * 4);
    cp(row_idx, lay->row_idx.data(), lay->row_idx.size() * 4);
    cp(csr_pos, lay->csr_pos.data(), lay->csr_pos.size() * 4);
    return SA_OK;
}

namespace {
void drop_view(sa_layout_t* lay)
{
    if (lay->view) sa_layout_destroy(lay->view);
    lay->view = nullptr;
    lay->view_kind = 0;
}
}  // namespace

int sa_layout_set_residue_view(sa_layout_t* lay, int enable)
{
    if (!lay) return fail(SA_ERR_INVALID_ARG, "sa_layout_set_residue_view: layout is NULL");
    if (!enable) {
        if (lay->view_kind == 1) drop_view(lay);
        return SA_OK;
    }
    if (lay->pattern != SA_STRIDED_B)
        return fail(SA_ERR_UNSUPPORTED, "sa_layout_set_residue_view: only strided B layouts have a residue view");
    if (lay->T != 64)
        return fail(SA_ERR_UNSUPPORTED, "sa_layout_set_residue_view: needs block 64 (the bf16 kernels)");
    if (lay->n % lay->l != 0)
        return fail(SA_ERR_UNSUPPORTED, "sa_layout_set_residue_view: n = %lld is not a multiple of l = %lld",
                    (long long)lay->n, (long long)lay->l);
    if (lay->view_kind == 1) return SA_OK;
    const int64_t m = lay->n / lay->l, m_pad = (m + 63) / 64 * 64;
    sa_layout* rv = nullptr;
    int st = build_layout(SA_DENSE_CAUSAL, m_pad, 1, 0, 64, &rv);
    if (st != SA_OK) return st;
    rv->view_l = lay->l;
    rv->view_m = m;
    rv->key_m = m;
    lay->view = rv;
    lay->view_kind = 1;
    return SA_OK;
}

int sa_layout_set_compact_view(sa_layout_t* lay, int enable)
{
    if (!lay) return fail(SA_ERR_INVALID_ARG, "sa_layout_set_compact_view: layout is NULL");
    if (!enable) {
        if (lay->view_kind == 2) drop_view(lay);
        return SA_OK;
    }
    if (lay->pattern != SA_FIXED_B)
        return fail(SA_ERR_UNSUPPORTED, "sa_layout_set_compact_view: only fixed B layouts have a compact view");
    if (lay->T != 64)
        return fail(SA_ERR_UNSUPPORTED, "sa_layout_set_compact_view: needs block 64 (the bf16 kernels)");
    if (lay->n % lay->l != 0)
        return fail(SA_ERR_UNSUPPORTED, "sa_layout_set_compact_view: n = %lld is not a multiple of l = %lld",
                    (long long)lay->n, (long long)lay->l);
    if ((lay->c & (lay->c - 1)) != 0)
        return fail(SA_ERR_UNSUPPORTED, "sa_layout_set_compact_view: c = %lld is not a power of two",
                    (long long)lay->c);
    if (lay->view_kind == 2) return SA_OK;
    sa_layout* cv = nullptr;
    int st = build_compact_view(lay->n, lay->l, lay->c, &cv);
    if (st != SA_OK) return st;
    lay->view = cv;
    lay->view_kind = 2;
    return SA_OK;
}

int sa_layout_view_info(const sa_layout_t* lay, int* kind, int64_t* nqb, int64_t* nkb, int64_t* nnz,
                        int64_t* allowed_pairs)
{
    if (!lay) return fail(SA_ERR_INVALID_ARG, "sa_layout_view_info: layout is NULL");
    const sa_layout* v = lay->view ? lay->view : lay;
    if (kind) *kind = lay->view_kind;
    if (nqb) *nqb = v->nqb;
    if (nkb) *nkb = v->nkb;
    if (nnz) *nnz = v->nnz;
    if (allowed_pairs) *allowed_pairs = v->allowed;
    return SA_OK;
}

void sa_layout_destroy(sa_layout_t* lay)
{
    if (!lay) return;
    release_plans(lay->serial);
    if (lay->view) sa_layout_destroy(lay->view);
    for (auto& kv : lay->dev_mem) {
        int cur = 0;
        if (hipGetDevice(&cur) == hipSuccess && hipSetDevice(kv.first) == hipSuccess) {
            (void)hipFree(kv.second);
            (void)hipSetDevice(cur);
        }
    }
    delete lay;
}

int sa_fwd(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d, int dtype,
           float scale, const void* q, const void* k, const void* v, void* o, float* lse, void* stream)
{
    HeadTable ht;
    int dev = 0, nl = 0;
    std::vector<sa_layout*> hl;
    sa_layout* distinct[kMaxLayouts];
    int st = common_checks("sa_fwd", head_layout, B, H, n, d, dtype, scale, false, true, &ht, &hl, distinct, &nl);
    if (st != SA_OK) return st;
    if (!q || !k || !v || !o || !lse) return fail(SA_ERR_INVALID_ARG, "sa_fwd: NULL tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3))
        return fail(SA_ERR_INVALID_ARG, "sa_fwd: q, k, v, o must be 16-byte aligned, lse 4-byte aligned");
    st = prepare_device(distinct, nl, &ht, &dev);
    if (st != SA_OK) return st;
    Plan plan;
    st = get_plan(dtype == SA_BF16 ? kByQueryPair : kByQuery, dev, B, H, hl.data(), &plan);
    if (st != SA_OK) return st;
    FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.n = n;
    a.H = H;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.items = plan.items;
    a.heads = ht;
    // The paired form when most of the walk's wave-steps have both halves
    // live (full blocks: dense layouts, residue views, wide strided A).
    int64_t pair_steps = 0, half_steps = 0;
    for (int32_t h = 0; h < H; ++h) {
        pair_steps += hl[h]->fwd_pair_steps;
        half_steps += hl[h]->fwd_half_steps;
    }
    hipError_t e = dtype == SA_BF16
                       ? launch_fwd_bf16_t64(d, a, plan.count, pair_steps > half_steps, (hipStream_t)stream)
                       : launch_fwd_f32_t16(d, a, plan.count, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "sa_fwd: kernel launch");
    return SA_OK;
}

size_t sa_bwd_workspace_size(int32_t B, int32_t H, int64_t n, int32_t d)
{
    (void)d;
    if (B < 1 || H < 1 || n < 1) return 0;
    return ((2 * (size_t)B * H * n * sizeof(float)) + 255) & ~(size_t)255;
}

}  // extern "C"

namespace {

// kStageDqRowTerms: the dQ kernel that also forms the row terms; it runs
// first and the dK/dV kernel after it (sa_bwd).
enum BwdStage { kStageRowTerms = 1, kStageDkDv = 2, kStageDq = 4, kStageDqRowTerms = 8 };

int bwd_call(const char* fn, int stages, const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n,
             int32_t d, int dtype, float scale, const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
             void* stream)
{
    HeadTable ht, htk;  // htk: for the dK/dV kernel (no compact views)
    int dev = 0, nl = 0, nlk = 0;
    std::vector<sa_layout*> hl, hlk;
    sa_layout* distinct[kMaxLayouts];
    sa_layout* distinct_k[kMaxLayouts];
    int st = common_checks(fn, head_layout, B, H, n, d, dtype, scale, true, true, &ht, &hl, distinct, &nl);
    if (st != SA_OK) return st;
    st = common_checks(fn, head_layout, B, H, n, d, dtype, scale, true, false, &htk, &hlk, distinct_k, &nlk);
    if (st != SA_OK) return st;
    // Pointers each stage reads or writes.
    const bool rt = stages & kStageRowTerms, kv = stages & kStageDkDv, dqs = stages & (kStageDq | kStageDqRowTerms);
    const bool dq_rt = stages & kStageDqRowTerms;
    std::vector<const void*> need = {workspace};
    if (rt || dq_rt) need.insert(need.end(), {o, dout, (const void*)lse});
    if (kv || dqs) need.insert(need.end(), {q, k, v, dout});
    for (const void* p : need)
        if (!p) return fail(SA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if ((kv && (!dk || !dv)) || (dqs && !dq)) return fail(SA_ERR_INVALID_ARG, "%s: NULL gradient pointer", fn);
    const void* al16[] = {q, k, v, o, dout, dq, dk, dv, workspace};
    for (const void* p : al16)
        if (p && !aligned16(p))
            return fail(SA_ERR_INVALID_ARG, "%s: tensors and workspace must be 16-byte aligned", fn);
    if ((uintptr_t)lse & 3) return fail(SA_ERR_INVALID_ARG, "%s: lse must be 4-byte aligned", fn);
    if (ws_bytes < sa_bwd_workspace_size(B, H, n, d))
        return fail(SA_ERR_INVALID_ARG, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes,
                    sa_bwd_workspace_size(B, H, n, d));
    st = prepare_device(distinct, nl, &ht, &dev);
    if (st != SA_OK) return st;
    st = prepare_device(distinct_k, nlk, &htk, &dev);
    if (st != SA_OK) return st;
    Plan pk{nullptr, 0}, pq{nullptr, 0};
    if (kv) {
        st = get_plan(kByKeyPair, dev, B, H, hlk.data(), &pk);
        if (st != SA_OK) return st;
    }
    if (dqs) {
        st = get_plan(kByQueryPair, dev, B, H, hl.data(), &pq);
        if (st != SA_OK) return st;
    }
    BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.dout = dout;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.ndelta = (float*)workspace;
    a.nl2 = (float*)workspace + (size_t)B * H * n;
    a.n = n;
    a.H = H;
    a.BH = B * H;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.heads = ht;
    a.items = nullptr;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    // The dQ kernel's one-element form pays off where such quadrants occur
    // (strided B); elsewhere the plain form keeps its grouped operand reads.
    bool one = false;
    for (int x = 0; x < nl; ++x) one = one || distinct[x]->one_quads;
    if (dq_rt) {
        a.items = pq.items;
        a.heads = ht;
        e = launch_bwd_dq_bf16_t64(d, a, pq.count, true, one, s);
        if (e != hipSuccess) return hip_fail(e, "sa_bwd: dQ kernel launch");
    }
    if (rt) {
        e = launch_bwd_rowterms_bf16(d, a, (int64_t)B * H * n, s);
        if (e != hipSuccess) return hip_fail(e, "sa_bwd: row-term kernel launch");
    }
    if (kv) {
        a.items = pk.items;
        a.heads = htk;
        e = launch_bwd_dkdv_bf16_t64(d, a, pk.count, s);
        if (e != hipSuccess) return hip_fail(e, "sa_bwd: dK/dV kernel launch");
    }
    if (dqs && !dq_rt) {
        a.items = pq.items;
        a.heads = ht;
        e = launch_bwd_dq_bf16_t64(d, a, pq.count, false, false, s);
        if (e != hipSuccess) return hip_fail(e, "sa_bwd: dQ kernel launch");
    }
    return SA_OK;
}

}  // namespace

extern "C" {

int sa_bwd(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d, int dtype, float scale,
           const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, void* workspace, size_t ws_bytes, void* stream)
{
    return bwd_call("sa_bwd", kStageDqRowTerms | kStageDkDv, head_layout, B, H, n, d, dtype, scale, q, k, v, o, lse, dout, dq, dk, dv,
                    workspace, ws_bytes, stream);
}

int sa_bwd_rowterms(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d, int dtype,
                    float scale, const void* o, const float* lse, const void* dout, void* workspace, size_t ws_bytes,
                    void* stream)
{
    return bwd_call("sa_bwd_rowterms", kStageRowTerms, head_layout, B, H, n, d, dtype, scale, nullptr, nullptr,
                    nullptr, o, lse, dout, nullptr, nullptr, nullptr, workspace, ws_bytes, stream);
}

int sa_bwd_dkdv(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d, int dtype,
                float scale, const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                const void* workspace, size_t ws_bytes, void* stream)
{
    return bwd_call("sa_bwd_dkdv", kStageDkDv, head_layout, B, H, n, d, dtype, scale, q, k, v, nullptr, nullptr, dout,
                    nullptr, dk, dv, const_cast<void*>(workspace), ws_bytes, stream);
}

int sa_bwd_dq_rowterms(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d, int dtype,
                       float scale, const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* workspace, size_t ws_bytes, void* stream)
{
    return bwd_call("sa_bwd_dq_rowterms", kStageDqRowTerms, head_layout, B, H, n, d, dtype, scale, q, k, v, o, lse,
                    dout, dq, nullptr, nullptr, workspace, ws_bytes, stream);
}

int sa_bwd_dq(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d, int dtype,
              float scale, const void* q, const void* k, const void* v, const void* dout, void* dq,
              const void* workspace, size_t ws_bytes, void* stream)
{
    return bwd_call("sa_bwd_dq", kStageDq, head_layout, B, H, n, d, dtype, scale, q, k, v, nullptr, nullptr, dout, dq,
                    nullptr, nullptr, const_cast<void*>(workspace), ws_bytes, stream);
}

const char* sa_status_string(int status)
{
    switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported combination";
    case SA_ERR_HIP: return "HIP runtime error";
    case SA_ERR_ALLOC: return "allocation failed";
    default: return "unknown status";
    }
}

const char* sa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
