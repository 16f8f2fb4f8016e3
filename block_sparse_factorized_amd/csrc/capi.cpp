// capi.cpp -- the extern "C" entry points of libsa: argument checks, layout
// upload, work lists, kernel dispatch and error reporting.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <string_view>
#include <vector>

#include "kernel_args.h"
#include "pack.h"
#include "sa_internal.h"

namespace sa {

namespace {
// sa_set_fwd_form: 0 chosen per call, 1 per-half form, 2 two-half form.
std::atomic<int> g_fwd_form{0};
// sa_set_one_paths: 1 the one-exponential paths are used, 0 never.
std::atomic<int> g_one_paths{1};
}

namespace {

int hip_fail(hipError_t e, const char* what)
{
    return fail(SA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// Upload a layout to the current device once; later calls return the view.
// upload = false: only look it up (no allocation); SA_ERR_UNSUPPORTED when
// it is not on the device yet.
int device_layout(sa_layout* L, int dev, DevLayout* out, bool upload)
{
    std::lock_guard<std::mutex> g(L->mu);
    auto it = L->dev.find(dev);
    if (it != L->dev.end()) {
        *out = it->second;
        return SA_OK;
    }
    if (!upload)
        return fail(SA_ERR_UNSUPPORTED, "a layout is not on device %d yet (one call of sa_fwd or sa_bwd with it "
                    "uploads it)", dev);
    LayoutImage img;
    int st = pack_layout(L, &img);
    if (st != SA_OK) return st;
    const size_t total = img.host.size();
    void* mem = nullptr;
    hipError_t e = hipMalloc(&mem, total);
    if (e != hipSuccess) return fail(SA_ERR_ALLOC, "layout upload: hipMalloc(%zu): %s", total, hipGetErrorString(e));
    e = hipMemcpy(mem, img.host.data(), total, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(mem);
        return hip_fail(e, "layout upload: hipMemcpy");
    }
    const DevLayout v = place_layout(img, L, (const unsigned char*)mem);
    L->dev_mem[dev] = mem;
    L->dev[dev] = v;
    *out = v;
    return SA_OK;
}

// ---------------------------------------------------------------------------
// Work lists (build_work_items), uploaded once and cached per (kind, device,
// B, H, d, layouts, chunking).

// Steps per chunk of a compact view's query list in the dK/dV kernel: long
// enough to amortise a chunk's partial sums, short enough that the first
// key-block pairs (listed by nearly every query block) do not set the
// launch time.  Measured on text (n = 12288, l = 128, c = 32, lists of up to
// 192 steps): dK/dV with its summing pass 232 us at 64 steps, 217 at 96,
// 233 at 128, 293 unsplit, against 226 on the raster layout.
constexpr int32_t kChunkSteps = 96;

struct Plan {
    Item* items;
    int count;
    int dev;
    void* mem;  // the one allocation behind items and the tables below
    // Chunks (see Split): the slot table, the chunked lists of plain layouts
    // (combining pass) and the compact views' summing-pass tables (dK/dV).
    const int2* chunk_tab;
    const int4* groups;
    int n_groups;
    const int2* cheads;
    int n_cheads;
    const int2* cgroups;
    size_t part_bytes;  // the chunks' partial results: slots x slot size
    float* partials;    // the buffer of the call's stream (get_plan)
};

// A cached work list and the partial-result buffers of the streams that
// have run it: calls on one stream are ordered, so they may share a buffer;
// calls on different streams may overlap, so each stream gets its own.
struct PlanEntry {
    Plan plan;
    std::map<void*, void*> parts;  // stream -> partial buffer
};

std::mutex g_plan_mu;
std::map<std::string, PlanEntry, std::less<>> g_plans;  // looked up by string_view: no allocation
// layout serial -> keys of the cached work lists that name it; destroying the
// layout frees them (sa_layout_destroy), so a process that keeps building and
// destroying layouts does not accumulate work lists.
std::map<uint64_t, std::vector<std::string>> g_plan_keys;

// sa_set_split: 0 chunk lengths by the rule below, -1 no chunks of plain
// layouts' lists, k > 0 every plain list longer than k in chunks of <= k.
std::atomic<int> g_split{0};

// The cache key of a work list, written into buf (no allocation); returns its length.
size_t plan_key(char* buf, size_t cap, ListKind kind, int dev, int32_t B, int32_t H, int32_t d, int split,
                sa_layout* const* hl)
{
    size_t len = (size_t)snprintf(buf, cap, "%d:%d:%d:%d:%d:%d", (int)kind, dev, B, H, d, split);
    for (int32_t h = 0; h < H && len < cap; ++h)
        len += (size_t)snprintf(buf + len, cap - len, ":%llu", (unsigned long long)hl[h]->serial);
    return std::min(len, cap - 1);
}

// Chunk length for the lists of plain layouts, and the length a list must
// exceed to be cut (*min_len).  The workgroups of a compute unit share its
// SIMDs, so a unit's time follows the steps it is given, not the number of
// its workgroups: as long as every unit holds several times the longest
// list, the longest-first order leaves their loads even and chunks only add
// work (their partial results and the combining pass).  Chunks pay where one
// list is longer than the other units' whole loads -- few heads and a batch
// of one, where some units would idle.  Lists are cut into chunks of about
// the average load of a unit (at least 16 steps): in a call with at most
// 1.25 lists per unit every list longer than that, else only lists longer
// than twice the average.  Measured (one box, fwd + dQ + dK/dV, chunk
// lengths forced): B = 1, two strided heads, n = 8192 (128 lists): 149 us
// whole, 86 at 16 steps, 107 at 32; B = 1, two fixed heads, n = 16384 (256
// lists): 381 us whole, 138 at 32, 187 at 64 -- the best lengths are the
// average loads (9 and 33 steps, 16 at least); img32 (384 lists, the longest
// 1.9 times the average) 118 us whole, 125-130 with chunks of 12-16; the
// five workloads get no chunks (2-35 % slower with chunks forced on).
int32_t plain_chunk(ListKind kind, int dev, int32_t B, int32_t H, sa_layout* const* hl, int split, int32_t* min_len)
{
    *min_len = 0;
    if (kind == kByQuery || split < 0) return 0;
    if (split > 0) {
        *min_len = split;
        return split;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
    int64_t total = 0, lists = 0;
    for (int32_t h = 0; h < H; ++h) {
        const std::vector<int32_t>& ptr = kind == kByKeyPair ? hl[h]->kgroups.ptr : hl[h]->qgroups.ptr;
        if (ptr.empty()) continue;
        total += (int64_t)(ptr.back() - ptr.front()) * hl[h]->view_l;
        lists += (int64_t)(ptr.size() - 1) * hl[h]->view_l;
    }
    total *= B;
    lists *= B;
    const double avg = (double)total / (double)cus;
    const double cs = std::max(16.0, std::ceil(avg));
    const double over = 4 * lists <= 5 * (int64_t)cus ? cs : std::max(cs, std::ceil(2.0 * avg));
    if (over > (double)(1 << 30)) return 0;
    *min_len = (int32_t)over;
    return (int32_t)cs;
}

// The work list of a call, built and uploaded on first use, with the
// partial-result buffer of `stream`.  create = false (nothing may be
// allocated: sa_bwd_noalloc, or a stream being captured into a graph): only
// look them up; SA_ERR_UNSUPPORTED when the list is not cached.  A stream
// with no buffer of its own gets one, unless create = false: then a buffer
// made for another stream serves (calls that share it must not overlap),
// and SA_ERR_UNSUPPORTED when there is none.
int get_plan(ListKind kind, int dev, int32_t B, int32_t H, int32_t d, sa_layout* const* hl, void* stream, Plan* out,
             bool create)
{
    const int split = g_split.load(std::memory_order_relaxed);
    char kbuf[64 + 21 * kMaxHeads];  // "kind:dev:B:H:d:split" + ":serial" per head
    const size_t klen = plan_key(kbuf, sizeof kbuf, kind, dev, B, H, d, split, hl);
    std::lock_guard<std::mutex> g(g_plan_mu);
    auto it = g_plans.find(std::string_view(kbuf, klen));
    if (it == g_plans.end()) {
        if (!create)
            return fail(SA_ERR_UNSUPPORTED, "no cached work list for this (B, H, layouts) on device %d (one "
                        "uncaptured call of the same kind with the same arguments caches it)", dev);
        const std::string key(kbuf, klen);
        int32_t min_len = 0;
        const int32_t cs = plain_chunk(kind, dev, B, H, hl, split, &min_len);
        std::vector<Item> sorted;
        Split sp;
        build_work_items(kind, B, H, hl, kind == kByKeyPair ? kChunkSteps : 0, cs, min_len, &sorted, &sp);
        const int64_t count = (int64_t)sorted.size();
        // One allocation: items, then the chunk tables, each 256-byte aligned.
        auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
        const size_t off_tab = al(sorted.size() * sizeof(Item));
        const size_t off_groups = al(off_tab + sp.chunk_tab.size() * sizeof(int2));
        const size_t off_cheads = al(off_groups + sp.groups.size() * sizeof(int4));
        const size_t off_cgroups = al(off_cheads + sp.cheads.size() * sizeof(int2));
        const size_t total = al(off_cgroups + sp.cgroups.size() * sizeof(int2));
        std::vector<unsigned char> host(total, 0);
        auto put = [&](size_t off, const void* src, size_t bytes) {
            if (bytes) memcpy(host.data() + off, src, bytes);
        };
        put(0, sorted.data(), sorted.size() * sizeof(Item));
        put(off_tab, sp.chunk_tab.data(), sp.chunk_tab.size() * sizeof(int2));
        put(off_groups, sp.groups.data(), sp.groups.size() * sizeof(int4));
        put(off_cheads, sp.cheads.data(), sp.cheads.size() * sizeof(int2));
        put(off_cgroups, sp.cgroups.data(), sp.cgroups.size() * sizeof(int2));
        void* mem = nullptr;
        hipError_t e = hipMalloc(&mem, std::max<size_t>(total, 256));
        if (e != hipSuccess) return fail(SA_ERR_ALLOC, "work list: hipMalloc(%zu): %s", total, hipGetErrorString(e));
        e = hipMemcpy(mem, host.data(), total, hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            (void)hipFree(mem);
            return hip_fail(e, "work list: hipMemcpy");
        }
        const int64_t slot_floats = kind == kByKeyPair ? kSlotFloats(d) : kind == kByQueryPairDq ? kDqSlotFloats(d)
                                                                                                  : kFwdSlotFloats(d);
        unsigned char* base = (unsigned char*)mem;
        Plan p{};
        p.items = (Item*)mem;
        p.count = (int)count;
        p.dev = dev;
        p.mem = mem;
        p.chunk_tab = (const int2*)(base + off_tab);
        p.groups = (const int4*)(base + off_groups);
        p.n_groups = (int)sp.groups.size();
        p.cheads = (const int2*)(base + off_cheads);
        p.n_cheads = (int)sp.cheads.size();
        p.cgroups = (const int2*)(base + off_cgroups);
        p.part_bytes = (size_t)sp.slots * (size_t)slot_floats * sizeof(float);
        p.partials = nullptr;
        it = g_plans.emplace(key, PlanEntry{p, {}}).first;
        for (int32_t h = 0; h < H; ++h) {
            std::vector<std::string>& keys = g_plan_keys[hl[h]->serial];
            if (keys.empty() || keys.back() != key) keys.push_back(key);
        }
    }
    PlanEntry& pe = it->second;
    *out = pe.plan;
    if (pe.plan.part_bytes) {
        auto b = pe.parts.find(stream);
        if (b == pe.parts.end()) {
            if (!create) {
                if (pe.parts.empty())
                    return fail(SA_ERR_UNSUPPORTED, "no partial-result buffer for this work list on device %d yet "
                                "(one uncaptured call on the device makes it)", dev);
                b = pe.parts.begin();
            } else {
                void* buf = nullptr;
                hipError_t e = hipMalloc(&buf, pe.plan.part_bytes);
                if (e != hipSuccess)
                    return fail(SA_ERR_ALLOC, "partial results: hipMalloc(%zu): %s", pe.plan.part_bytes,
                                hipGetErrorString(e));
                b = pe.parts.emplace(stream, buf).first;
            }
        }
        out->partials = (float*)b->second;
    }
    return SA_OK;
}

// Frees the cached work lists that name layout `serial`, with their
// partial-result buffers.
void release_plans(uint64_t serial)
{
    std::lock_guard<std::mutex> g(g_plan_mu);
    auto it = g_plan_keys.find(serial);
    if (it == g_plan_keys.end()) return;
    for (const std::string& key : it->second) {
        auto p = g_plans.find(key);
        if (p == g_plans.end()) continue;
        int cur = 0;
        if (hipGetDevice(&cur) == hipSuccess && hipSetDevice(p->second.plan.dev) == hipSuccess) {
            (void)hipFree(p->second.plan.mem);
            for (auto& kv : p->second.parts) (void)hipFree(kv.second);
            (void)hipSetDevice(cur);
        }
        g_plans.erase(p);
    }
    g_plan_keys.erase(it);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Whether `stream` is being captured into a graph: a captured call must not
// allocate or copy synchronously, so it only looks up what an earlier
// uncaptured call left on the device.
bool capturing(void* stream)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing((hipStream_t)stream, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

// Checks shared by sa_fwd and sa_bwd; fills the head table with the layouts
// the kernels walk (a layout's view when it has one).
int common_checks(const char* fn, const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n,
                  int32_t d, int dtype, float scale, bool backward, HeadTable* ht,
                  sa_layout** hl /* [kMaxHeads] */, sa_layout** distinct_out, int* n_distinct)
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
        if (L->view) L = L->view;  // the kernels walk the view
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
        hl[h] = L;
    }
    int64_t max_items = 0;
    for (int32_t h = 0; h < H; ++h) max_items += hl[h]->nqb * hl[h]->view_l;
    if ((int64_t)B * max_items > (int64_t)1 << 30)
        return fail(SA_ERR_UNSUPPORTED, "%s: %lld work items is too many for one launch", fn,
                    (long long)((int64_t)B * max_items));
    *n_distinct = nl;
    for (int a = 0; a < nl; ++a) distinct_out[a] = distinct[a];
    return SA_OK;
}

// Device side of a call: current device, layouts uploaded (upload = false:
// already there), head table filled.
int prepare_device(sa_layout* const* distinct, int nl, HeadTable* ht, int* dev_out, bool upload)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    for (int a = 0; a < nl; ++a) {
        int st = device_layout(distinct[a], dev, &ht->lay[a], upload);
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
    sa_layout* rv = nullptr;
    int st = build_residue_view(lay->n, lay->l, &rv);
    if (st != SA_OK) return st;
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
    sa_layout* hl[kMaxHeads];
    sa_layout* distinct[kMaxLayouts];
    int st = common_checks("sa_fwd", head_layout, B, H, n, d, dtype, scale, false, &ht, hl, distinct, &nl);
    if (st != SA_OK) return st;
    if (!q || !k || !v || !o || !lse) return fail(SA_ERR_INVALID_ARG, "sa_fwd: NULL tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3))
        return fail(SA_ERR_INVALID_ARG, "sa_fwd: q, k, v, o must be 16-byte aligned, lse 4-byte aligned");
    const bool alloc = !capturing(stream);
    st = prepare_device(distinct, nl, &ht, &dev, alloc);
    if (st != SA_OK) return st;
    Plan plan;
    st = get_plan(dtype == SA_BF16 ? kByQueryPair : kByQuery, dev, B, H, d, hl, stream, &plan, alloc);
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
    a.chunk_tab = plan.chunk_tab;
    a.partials = plan.partials;
    a.one_bits = g_one_paths.load(std::memory_order_relaxed) ? 3u : 0u;
    // The paired form when most of the walk's wave-steps have both halves
    // live (full blocks: dense layouts, residue views, wide strided A).  A
    // residue view's layout is walked once per residue class, view_l times
    // per head; every head is walked B times, which does not change the
    // comparison.
    int64_t pair_steps = 0, half_steps = 0;
    for (int32_t h = 0; h < H; ++h) {
        pair_steps += hl[h]->fwd_pair_steps * hl[h]->view_l;
        half_steps += hl[h]->fwd_half_steps * hl[h]->view_l;
    }
    const int form = g_fwd_form.load(std::memory_order_relaxed);
    const bool paired = form == 0 ? pair_steps > half_steps : form == 2;
    hipError_t e = dtype == SA_BF16
                       ? launch_fwd_bf16_t64(d, a, plan.count, paired, (hipStream_t)stream)
                       : launch_fwd_f32_t16(d, a, plan.count, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "sa_fwd: kernel launch");
    if (plan.n_groups > 0) {
        // the chunks of long lists: combined in list order
        CombineArgs c{};
        c.out0 = o;
        c.lse = lse;
        c.partials = plan.partials;
        c.groups = plan.groups;
        c.n = n;
        c.H = H;
        c.scale = scale;
        c.scale_log2 = a.scale_log2;
        c.heads = ht;
        e = launch_fwd_combine_bf16(d, c, plan.n_groups, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "sa_fwd: combining launch");
    }
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

// alloc = false (sa_bwd_noalloc): the layouts and work lists must already be
// on the device; nothing is allocated (a missing one is an error).
int bwd_call(const char* fn, int stages, const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n,
             int32_t d, int dtype, float scale, const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
             void* stream, bool alloc = true)
{
    HeadTable ht;
    int dev = 0, nl = 0;
    sa_layout* hl[kMaxHeads];
    sa_layout* distinct[kMaxLayouts];
    int st = common_checks(fn, head_layout, B, H, n, d, dtype, scale, true, &ht, hl, distinct, &nl);
    if (st != SA_OK) return st;
    // Pointers each stage reads or writes.
    const bool rt = stages & kStageRowTerms, kv = stages & kStageDkDv, dqs = stages & (kStageDq | kStageDqRowTerms);
    const bool dq_rt = stages & kStageDqRowTerms;
    if (!workspace) return fail(SA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if ((rt || dq_rt) && (!o || !dout || !lse)) return fail(SA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if ((kv || dqs) && (!q || !k || !v || !dout)) return fail(SA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if ((kv && (!dk || !dv)) || (dqs && !dq)) return fail(SA_ERR_INVALID_ARG, "%s: NULL gradient pointer", fn);
    const void* al16[] = {q, k, v, o, dout, dq, dk, dv, workspace};
    for (const void* p : al16)
        if (p && !aligned16(p))
            return fail(SA_ERR_INVALID_ARG, "%s: tensors and workspace must be 16-byte aligned", fn);
    if ((uintptr_t)lse & 3) return fail(SA_ERR_INVALID_ARG, "%s: lse must be 4-byte aligned", fn);
    if (ws_bytes < sa_bwd_workspace_size(B, H, n, d))
        return fail(SA_ERR_INVALID_ARG, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes,
                    sa_bwd_workspace_size(B, H, n, d));
    alloc = alloc && !capturing(stream);
    st = prepare_device(distinct, nl, &ht, &dev, alloc);
    if (st != SA_OK) return st;
    Plan pk{}, pq{};
    if (kv) {
        st = get_plan(kByKeyPair, dev, B, H, d, hl, stream, &pk, alloc);
        if (st != SA_OK) return st;
    }
    if (dqs) {
        st = get_plan(kByQueryPairDq, dev, B, H, d, hl, stream, &pq, alloc);
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
    a.chunk_tab = nullptr;
    a.partials = nullptr;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    // The combining pass of a plan's chunked plain lists.
    auto combine = [&](const Plan& p, bool dkdv) -> hipError_t {
        CombineArgs c{};
        c.out0 = dkdv ? dk : dq;
        c.out1 = dv;
        c.partials = p.partials;
        c.groups = p.groups;
        c.n = n;
        c.H = H;
        c.scale = scale;
        c.scale_log2 = a.scale_log2;
        c.heads = ht;
        return dkdv ? launch_dkdv_combine_bf16(d, c, p.n_groups, s) : launch_dq_combine_bf16(d, c, p.n_groups, s);
    };
    // The dQ kernel's one-element form pays off where such quadrants occur
    // (strided B); elsewhere the plain form keeps its grouped operand reads.
    bool one = false;
    for (int x = 0; x < nl; ++x) one = one || distinct[x]->one_quads;
    if (!g_one_paths.load(std::memory_order_relaxed)) one = false;
    if (dq_rt) {
        a.items = pq.items;
        a.chunk_tab = pq.chunk_tab;
        a.partials = pq.partials;
        e = launch_bwd_dq_bf16_t64(d, a, pq.count, true, one, s);
        if (e != hipSuccess) return hip_fail(e, "sa_bwd: dQ kernel launch");
        if (pq.n_groups > 0) {
            e = combine(pq, false);
            if (e != hipSuccess) return hip_fail(e, "sa_bwd: dQ combining launch");
        }
    }
    if (rt) {
        e = launch_bwd_rowterms_bf16(d, a, (int64_t)B * H * n, s);
        if (e != hipSuccess) return hip_fail(e, "sa_bwd: row-term kernel launch");
    }
    if (kv) {
        a.items = pk.items;
        a.chunk_tab = pk.chunk_tab;
        a.partials = pk.partials;
        e = launch_bwd_dkdv_bf16_t64(d, a, pk.count, s);
        if (e != hipSuccess) return hip_fail(e, "sa_bwd: dK/dV kernel launch");
        if (pk.n_cheads > 0) {
            // compact views: sum each key-block pair's chunks in order
            ReduceArgs r;
            r.dk = dk;
            r.dv = dv;
            r.partials = pk.partials;
            r.heads_tab = pk.cheads;
            r.groups = pk.cgroups;
            r.n = n;
            r.H = H;
            r.scale = scale;
            r.heads = ht;
            e = launch_bwd_dkdv_reduce_bf16(d, r, pk.n_cheads, n, s);
            if (e != hipSuccess) return hip_fail(e, "sa_bwd: dK/dV summing launch");
        }
        if (pk.n_groups > 0) {
            e = combine(pk, true);
            if (e != hipSuccess) return hip_fail(e, "sa_bwd: dK/dV combining launch");
        }
    }
    if (dqs && !dq_rt) {
        a.items = pq.items;
        a.chunk_tab = pq.chunk_tab;
        a.partials = pq.partials;
        e = launch_bwd_dq_bf16_t64(d, a, pq.count, false, false, s);
        if (e != hipSuccess) return hip_fail(e, "sa_bwd: dQ kernel launch");
        if (pq.n_groups > 0) {
            e = combine(pq, false);
            if (e != hipSuccess) return hip_fail(e, "sa_bwd: dQ combining launch");
        }
    }
    return SA_OK;
}

// Row-term scratch of sa_bwd_noalloc, one copy per device for the life of
// the process: two fp32 per row, the layout sa_bwd's workspace has.
constexpr size_t kScratchRows = (size_t)1 << 21;
constexpr size_t kScratchBytes = 2 * kScratchRows * sizeof(float);  // 16 MiB
static __device__ __align__(256) float scratch[2 * kScratchRows];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (set on first use)

// The device address of this device's scratch array.  The array's name is
// a host-side stand-in, not a device address: kernels get this pointer.
int scratch_on(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices) return fail(SA_ERR_UNSUPPORTED, "sa_bwd_noalloc: device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "sa_bwd_noalloc: hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SA_OK;
}

}  // namespace

extern "C" {

int sa_bwd_noalloc(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d, int dtype,
                   float scale, const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, void* stream)
{
    if (B >= 1 && H >= 1 && n >= 1 && (size_t)B * (size_t)H * (size_t)n > kScratchRows)
        return fail(SA_ERR_INVALID_ARG, "sa_bwd_noalloc: B*H*n = %lld rows exceeds the scratch limit of %zu rows",
                    (long long)B * H * n, kScratchRows);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "sa_bwd_noalloc: hipGetDevice");
    void* ws = nullptr;
    int st = scratch_on(dev, &ws);
    if (st != SA_OK) return st;
    return bwd_call("sa_bwd_noalloc", kStageDqRowTerms | kStageDkDv, head_layout, B, H, n, d, dtype, scale, q, k, v,
                    o, lse, dout, dq, dk, dv, ws, kScratchBytes, stream, false);
}

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

int sa_set_fwd_form(int form)
{
    if (form < 0 || form > 2) return fail(SA_ERR_INVALID_ARG, "sa_set_fwd_form: form %d is not 0, 1 or 2", form);
    return g_fwd_form.exchange(form);
}

int sa_set_one_paths(int enable, int* previous)
{
    if (enable != 0 && enable != 1) return fail(SA_ERR_INVALID_ARG, "sa_set_one_paths: enable %d is not 0 or 1", enable);
    const int prev = g_one_paths.exchange(enable);
    if (previous) *previous = prev;
    return SA_OK;
}

int sa_set_split(int steps, int* previous)
{
    if (steps < -1) return fail(SA_ERR_INVALID_ARG, "sa_set_split: steps %d is below -1", steps);
    const int prev = g_split.exchange(steps);
    if (previous) *previous = prev;
    return SA_OK;
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

const char* sa_last_error(void) { return last_error(); }

}  // extern "C"
