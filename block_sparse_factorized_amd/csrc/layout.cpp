// layout.cpp -- host builder of block layouts for the factorized patterns.
//
// "OpenAI Sparse Transformer" (agentlenshq.com), "Implementation and
// Limitations", and pcnews.ru, "Релиз кода": sparse attention is executed by
// slicing the query and key matrices into blocks and computing only the
// blocks that hold allowed pairs.  The patterns ("Factorized Attention
// Patterns"; pcnews.ru, "Разреженное внимание") are, for key j <= query i:
//   strided A  0 <= i-j < l           strided B  (i-j) mod l == 0
//   fixed A    floor(j/l) == floor(i/l)   fixed B  j mod l >= l-c
//   dense causal: every j <= i.
//
// For a block row (query rows i0..i0+T-1) each row's allowed keys inside a
// key block are a run of intervals (strided A, fixed A, fixed B, dense) or an
// arithmetic progression with step l (strided B), so a block's mask is
// written row by row without testing every element.  Key blocks that cannot
// hold a pair are skipped by a per-pattern range or test first.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>

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

const char* last_error() { return g_last_error.c_str(); }

namespace {

struct Params {
    int pattern;
    int64_t l, c, T;
};

inline void set_bits(uint64_t* w, int64_t e0, int64_t e1)  // bits [e0, e1]
{
    while (e0 <= e1) {
        int64_t word = e0 >> 6, b0 = e0 & 63;
        int64_t b1 = std::min<int64_t>(63, b0 + (e1 - e0));
        int64_t len = b1 - b0 + 1;
        uint64_t m = (len == 64) ? ~0ull : (((1ull << len) - 1) << b0);
        w[word] |= m;
        e0 += len;
    }
}

// Allowed keys of query i inside [j0, j1] (j1 <= i), as bits of tile row r.
// Returns the number of allowed keys.
int64_t row_bits(const Params& p, int64_t i, int64_t j0, int64_t j1, int64_t r, uint64_t* w)
{
    const int64_t base = r * p.T - j0;  // element index of key j is base + j
    int64_t cnt = 0;
    auto run = [&](int64_t a, int64_t b) {
        if (a > b) return;
        set_bits(w, base + a, base + b);
        cnt += b - a + 1;
    };
    switch (p.pattern) {
    case SA_STRIDED_A: run(std::max(j0, i - p.l + 1), j1); break;
    case SA_STRIDED_B: {
        int64_t r0 = (i - j1) % p.l;
        for (int64_t j = j1 - (p.l - r0) % p.l; j >= j0; j -= p.l) run(j, j);
        break;
    }
    case SA_FIXED_A: run(std::max(j0, p.l * (i / p.l)), j1); break;
    case SA_FIXED_B:
        for (int64_t m = j0 / p.l; m <= j1 / p.l; ++m)
            run(std::max(j0, m * p.l + p.l - p.c), std::min(j1, m * p.l + p.l - 1));
        break;
    default: run(j0, j1); break;
    }
    return cnt;
}

// Could key block kb hold a pair for query block qb?  (A cheap filter; the
// row pass below is exact.)
bool may_hold(const Params& p, int64_t qb, int64_t kb)
{
    const int64_t T = p.T;
    switch (p.pattern) {
    case SA_STRIDED_B: {
        int64_t lo = std::max<int64_t>(0, (qb - kb) * T - (T - 1));
        int64_t hi = (qb - kb) * T + (T - 1);
        return (hi / p.l) * p.l >= lo;
    }
    case SA_FIXED_B: {
        int64_t j0 = kb * T, j1 = std::min(kb * T + T - 1, qb * T + T - 1);
        int64_t off = j0 % p.l;
        int64_t first = off >= p.l - p.c ? j0 : j0 + (p.l - p.c - off);
        return first <= j1;
    }
    default: return true;
    }
}

int64_t first_key_block(const Params& p, int64_t qb)
{
    const int64_t i0 = qb * p.T;
    switch (p.pattern) {
    case SA_STRIDED_A: return std::max<int64_t>(0, i0 - (p.l - 1)) / p.T;
    case SA_FIXED_A: return (p.l * (i0 / p.l)) / p.T;
    default: return 0;
    }
}

struct VecHash {
    size_t operator()(const std::vector<uint64_t>& v) const
    {
        uint64_t h = 1469598103934665603ull;
        for (uint64_t x : v) {
            h ^= x + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2);
            h *= 1099511628211ull;
        }
        return (size_t)h;
    }
};

uint64_t next_serial()
{
    static std::mutex mu;
    static uint64_t s = 0;
    std::lock_guard<std::mutex> g(mu);
    return ++s;
}

// From the listing by query block (row_ptr, col_idx, mask_id) and nkb: the
// listing by key block and the two pair lists.
void finish_layout(sa_layout* L)
{
    const int64_t nqb = L->nqb, nkb = L->nkb;
    L->nnz = (int64_t)L->col_idx.size();
    // Transpose: per key block, its query blocks in ascending order.
    L->col_ptr.assign(nkb + 1, 0);
    for (int32_t kb : L->col_idx) L->col_ptr[kb + 1]++;
    for (int64_t kb = 0; kb < nkb; ++kb) L->col_ptr[kb + 1] += L->col_ptr[kb];
    L->row_idx.assign(L->nnz, 0);
    L->csr_pos.assign(L->nnz, 0);
    std::vector<int32_t> fillp(L->col_ptr.begin(), L->col_ptr.end() - 1);
    for (int64_t qb = 0; qb < nqb; ++qb)
        for (int32_t a = L->row_ptr[qb]; a < L->row_ptr[qb + 1]; ++a) {
            int32_t kb = L->col_idx[a];
            int32_t slot = fillp[kb]++;
            L->row_idx[slot] = (int32_t)qb;
            L->csr_pos[slot] = a;
        }
    L->qgroups = pair_blocks(L->row_ptr, L->col_idx, L->mask_id);
    std::vector<int32_t> col_mask(L->nnz);
    for (int64_t a = 0; a < L->nnz; ++a) col_mask[a] = L->mask_id[L->csr_pos[a]];
    L->kgroups = pair_blocks(L->col_ptr, L->row_idx, col_mask);
}

}  // namespace

// Greedy pairing: each block, in ascending order, takes the unpaired block
// among the next four whose list has the largest Jaccard similarity with its
// own, if that is at least 1/2 (two empty lists count as similar).  Strided
// B with l = 2T pairs qb with qb+2, dense and fixed patterns pair neighbours.
Groups pair_blocks(const std::vector<int32_t>& ptr, const std::vector<int32_t>& idx,
                   const std::vector<int32_t>& mask)
{
    const int64_t nb = (int64_t)ptr.size() - 1;
    auto jac = [&](int64_t x, int64_t y) {
        int32_t i = ptr[x], j = ptr[y], ie = ptr[x + 1], je = ptr[y + 1];
        if (ie == i && je == j) return 1.0;
        int64_t inter = 0, uni = 0;
        while (i < ie || j < je) {
            if (j >= je || (i < ie && idx[i] < idx[j])) ++i;
            else if (i >= ie || idx[j] < idx[i]) ++j;
            else { ++i; ++j; ++inter; }
            ++uni;
        }
        return (double)inter / (double)uni;
    };
    Groups g;
    std::vector<char> used(nb, 0);
    g.ptr.push_back(0);
    for (int64_t x = 0; x < nb; ++x) {
        if (used[x]) continue;
        int64_t best = -1;
        double bj = 0.5;
        for (int64_t y = x + 1; y < std::min<int64_t>(nb, x + 5); ++y) {
            if (used[y]) continue;
            double jv = jac(x, y);
            if (jv >= bj) {
                if (best < 0 || jv > bj) { best = y; bj = jv; }
            }
        }
        used[x] = 1;
        if (best >= 0) used[best] = 1;
        g.blk.push_back((int32_t)x);
        g.blk.push_back((int32_t)best);
        int32_t i = ptr[x], ie = ptr[x + 1];
        int32_t j = best >= 0 ? ptr[best] : 0, je = best >= 0 ? ptr[best + 1] : 0;
        while (i < ie || j < je) {
            int32_t o, ma = -2, mb = -2;
            if (j >= je || (i < ie && idx[i] < idx[j])) { o = idx[i]; ma = mask[i]; ++i; }
            else if (i >= ie || idx[j] < idx[i]) { o = idx[j]; mb = mask[j]; ++j; }
            else { o = idx[i]; ma = mask[i]; mb = mask[j]; ++i; ++j; }
            g.step.insert(g.step.end(), {o, ma, mb, 0});
        }
        g.ptr.push_back((int32_t)(g.step.size() / 4));
    }
    return g;
}

int build_layout(int pattern, int64_t n, int64_t l, int64_t c, int32_t block, sa_layout** out)
{
    if (!out) return fail(SA_ERR_INVALID_ARG, "sa_layout_build: out is NULL");
    *out = nullptr;
    if (pattern < SA_STRIDED_A || pattern > SA_DENSE_CAUSAL)
        return fail(SA_ERR_INVALID_ARG, "sa_layout_build: unknown pattern %d", pattern);
    if (block != 8 && block != 16 && block != 32 && block != 64 && block != 128)
        return fail(SA_ERR_INVALID_ARG, "sa_layout_build: block %d not in {8,16,32,64,128}", block);
    if (n < 1) return fail(SA_ERR_INVALID_ARG, "sa_layout_build: n = %lld < 1", (long long)n);
    if (n % block != 0)
        return fail(SA_ERR_INVALID_ARG, "sa_layout_build: n = %lld is not a multiple of block %d",
                    (long long)n, block);
    if (l < 1) return fail(SA_ERR_INVALID_ARG, "sa_layout_build: l = %lld < 1", (long long)l);
    if (pattern == SA_FIXED_B && (c < 1 || c > l))
        return fail(SA_ERR_INVALID_ARG, "sa_layout_build: fixed B needs 1 <= c <= l (c = %lld, l = %lld)",
                    (long long)c, (long long)l);
    const int64_t nqb = n / block;
    if (nqb > 46340)  // nqb*nqb must fit in int32 block indices
        return fail(SA_ERR_INVALID_ARG, "sa_layout_build: %lld query blocks is too many", (long long)nqb);

    sa_layout* L = new (std::nothrow) sa_layout();
    if (!L) return fail(SA_ERR_ALLOC, "sa_layout_build: out of host memory");
    try {
        L->serial = next_serial();
        L->pattern = pattern;
        L->n = n;
        L->view_l = 1;
        L->view_m = n;
        L->l = l;
        L->c = pattern == SA_FIXED_B ? c : 0;
        L->T = block;
        L->nqb = nqb;
        L->nkb = nqb;
        L->key_m = n;
        const Params p{pattern, l, L->c, block};
        const int64_t T = block, nw = T * T / 64;

        std::unordered_map<std::vector<uint64_t>, int32_t, VecHash> ids;
        std::vector<uint64_t> tile(nw);
        L->row_ptr.assign(nqb + 1, 0);
        int64_t allowed = 0;
        for (int64_t qb = 0; qb < nqb; ++qb) {
            for (int64_t kb = first_key_block(p, qb); kb <= qb; ++kb) {
                if (!may_hold(p, qb, kb)) continue;
                std::fill(tile.begin(), tile.end(), 0ull);
                int64_t pop = 0;
                for (int64_t r = 0; r < T; ++r) {
                    int64_t i = qb * T + r, j0 = kb * T, j1 = std::min(kb * T + T - 1, i);
                    if (j1 < j0) continue;
                    pop += row_bits(p, i, j0, j1, r, tile.data());
                }
                if (pop == 0) continue;
                allowed += pop;
                int32_t id = -1;
                if (pop != T * T) {
                    auto it = ids.find(tile);
                    if (it == ids.end()) {
                        id = (int32_t)ids.size();
                        ids.emplace(tile, id);
                        L->masks.insert(L->masks.end(), tile.begin(), tile.end());
                    } else {
                        id = it->second;
                    }
                }
                L->col_idx.push_back((int32_t)kb);
                L->mask_id.push_back(id);
            }
            L->row_ptr[qb + 1] = (int32_t)L->col_idx.size();
        }
        L->n_masks = (int64_t)ids.size();
        L->allowed = allowed;
        finish_layout(L);
    } catch (const std::bad_alloc&) {
        delete L;
        return fail(SA_ERR_ALLOC, "sa_layout_build: out of host memory");
    }
    *out = L;
    return SA_OK;
}

// Residue view of strided B with stride l (n % l == 0, block 64): position
// i attends exactly the earlier positions of its residue class i mod l
// (pcnews.ru, "Разреженное внимание": attention along a column is attention
// along a row of the transposed matrix), so the kernels walk one dense
// causal layout over m = n / l rows (rounded up to blocks), once per residue
// class, reading rows l apart.
int build_residue_view(int64_t n, int64_t l, sa_layout** out)
{
    *out = nullptr;
    if (l < 1 || n % l != 0)
        return fail(SA_ERR_UNSUPPORTED, "residue view: needs n %% l == 0");
    const int64_t m = n / l, m_pad = (m + 63) / 64 * 64;
    sa_layout* rv = nullptr;
    int st = build_layout(SA_DENSE_CAUSAL, m_pad, 1, 0, 64, &rv);
    if (st != SA_OK) return st;
    rv->view_l = l;
    rv->view_m = m;
    rv->key_m = m;
    *out = rv;
    return SA_OK;
}

// Compact view of fixed B.  Fixed B lets query i see exactly the summary
// positions (the last c of every l-block) at or before i ("OpenAI Sparse
// Transformer", "Factorized Attention Patterns": a fixed set of columns;
// pcnews.ru, "Разреженное внимание").  Numbered consecutively, the summary
// positions are keys t = 0 .. (n/l) c - 1 at sequence row
// (t / c) l + (l - c) + t mod c, increasing in t, so the keys query i sees
// are a prefix: t < cnt(i), cnt(i) = floor((i+1)/l) c + max(0, (i+1) mod l
// - (l - c)).  The view lists every query block against the 64-key blocks of
// that prefix: a staircase of full blocks plus one partial block per query
// block, the same allowed pairs as the fixed-B layout in about half as many
// blocks of twice the density.
int build_compact_view(int64_t n, int64_t l, int64_t c, sa_layout** out)
{
    *out = nullptr;
    constexpr int64_t T = 64;
    int kcl = 0;
    while (((int64_t)1 << kcl) < c) ++kcl;
    if (c < 1 || c > l || ((int64_t)1 << kcl) != c || n % l != 0 || n % T != 0)
        return fail(SA_ERR_UNSUPPORTED, "compact view: needs n %% l == 0, n %% 64 == 0 and c a power of two <= l");
    const int64_t nqb = n / T, nk = (n / l) * c, nkb = (nk + T - 1) / T;
    if (l > ((int64_t)1 << 30) || nk > ((int64_t)1 << 30))
        return fail(SA_ERR_UNSUPPORTED, "compact view: l or the key count does not fit 32 bits");
    sa_layout* L = new (std::nothrow) sa_layout();
    if (!L) return fail(SA_ERR_ALLOC, "compact view: out of host memory");
    try {
        L->serial = next_serial();
        L->pattern = SA_FIXED_B;
        L->n = n;
        L->l = l;
        L->c = c;
        L->T = (int32_t)T;
        L->nqb = nqb;
        L->nkb = nkb;
        L->view_l = 1;
        L->view_m = n;
        L->key_cl = kcl;
        L->key_gl = (int32_t)l;
        L->key_off = (int32_t)(l - c);
        L->key_m = nk;
        auto cnt = [&](int64_t i) { return (i + 1) / l * c + std::max<int64_t>(0, (i + 1) % l - (l - c)); };
        std::unordered_map<std::vector<uint64_t>, int32_t, VecHash> ids;
        std::vector<uint64_t> tile(T * T / 64);
        L->row_ptr.assign(nqb + 1, 0);
        int64_t allowed = 0;
        for (int64_t qb = 0; qb < nqb; ++qb) {
            const int64_t cmax = cnt(qb * T + T - 1);  // the widest row of the block
            for (int64_t kb = 0; kb * T < cmax; ++kb) {
                std::fill(tile.begin(), tile.end(), 0ull);
                int64_t pop = 0;
                for (int64_t r = 0; r < T; ++r) {
                    const int64_t p = std::min<int64_t>(T, std::max<int64_t>(0, cnt(qb * T + r) - kb * T));
                    if (p > 0) set_bits(tile.data(), r * T, r * T + p - 1);
                    pop += p;
                }
                allowed += pop;
                int32_t id = -1;
                if (pop != T * T) {
                    auto it = ids.find(tile);
                    if (it == ids.end()) {
                        id = (int32_t)ids.size();
                        ids.emplace(tile, id);
                        L->masks.insert(L->masks.end(), tile.begin(), tile.end());
                    } else {
                        id = it->second;
                    }
                }
                L->col_idx.push_back((int32_t)kb);
                L->mask_id.push_back(id);
            }
            L->row_ptr[qb + 1] = (int32_t)L->col_idx.size();
        }
        L->n_masks = (int64_t)ids.size();
        L->allowed = allowed;
        finish_layout(L);
    } catch (const std::bad_alloc&) {
        delete L;
        return fail(SA_ERR_ALLOC, "compact view: out of host memory");
    }
    *out = L;
    return SA_OK;
}

}  // namespace sa
