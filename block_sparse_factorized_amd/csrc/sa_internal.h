// sa_internal.h -- shared host/device declarations of libsa (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/sa.h"

namespace sa {

constexpr int kMaxLayouts = 8;   // distinct layouts per call
constexpr int kMaxHeads = 256;   // heads per call

// Device view of one layout: one allocation, several arrays.
struct DevLayout {
    const int32_t* row_ptr;   // [nqb+1]   listing by query block
    const int32_t* col_idx;   // [nnz]     key blocks, ascending per query block
    const int32_t* mask_id;   // [nnz]     -1 = full block
    const uint64_t* masks;    // [n_masks][T*T/64]  element (r, s): bit r*T+s
    const uint64_t* masks_t;  // [n_masks][T*T/64]  the same masks transposed:
                              //                    element (r, s): bit s*T+r
    // Block size 64 only: the masks as 64-bit lane masks ("planes") of the
    // 32x32 MFMA accumulator layout, [1 + n_masks][wave w = 0, 1][register
    // 0..31]; set 0 is all ones (a full block), mask m is set m + 1.
    //   planes:   bit L of register 16*t + i = element (row 32w + L%32,
    //             key 32t + 8(i/4) + 4(L/32) + i%4)   (lane = query row)
    //   planes_t: bit L of register 16*t + i = element (row 32t + 8(i/4) +
    //             4(L/32) + i%4, key 32w + L%32)       (lane = key column)
    const uint64_t* planes;
    const uint64_t* planes_t;
    const int32_t* col_ptr;   // [nkb+1]   listing by key block
    const int32_t* row_idx;   // [nnz]     query blocks, ascending per key block
    const int32_t* col_mask;  // [nnz]     mask id of each transposed entry
    // Pairs of blocks with nearly the same list, walked together by one
    // workgroup (qgrp: query blocks over their key lists; kgrp: key blocks
    // over their query lists).  Group g has members grp_blk[g] = {a, b}
    // (b = -1 for a single block) and steps grp_ptr[g] .. grp_ptr[g+1]-1;
    // step = {other block, mask of a, mask of b, quadrants}, mask -1 = full
    // block, -2 = that member does not list this block.  quadrants: bits 0-3
    // for a, 4-7 for b; bit 2*rh + ch is set when the member's mask has an
    // allowed element with query row in half rh and key in half ch of the
    // 64 x 64 block (all four for a full block, none for -2); bits 8-11 (a)
    // and 12-15 (b) the same for quadrants whose every element is allowed;
    // bits 16-19 (a) and 20-23 (b) for partial quadrants where each lane of
    // the forward's score layout holds at most one allowed element (a lane
    // holds keys 32*ch + 8*g + 4*hh + e, g, e < 4, of one query).
    const int32_t* qgrp_ptr;
    const int2* qgrp_blk;
    const int4* qgrp_step;
    const int32_t* kgrp_ptr;
    const int2* kgrp_blk;
    const int4* kgrp_step;
    // Per key-block pair, 2 bits per member (a: bits 0-1, b: bits 2-3): 0, or
    // 1 + h when the member's whole query list has allowed elements only in
    // its 32-key half h.
    const int32_t* kgrp_mode;
    // Per key block: {its key-block pair, member (0 or 1)}.
    const int2* kblk_grp;
    // Sequence view.  Row m of the sequence a work item walks is position
    // r + vl * m of its (batch, head), r the item's residue; rows m >= vm
    // (a ragged last block) are read clamped and never written.  A plain
    // layout: vl = 1, vm = n.  The residue view of a strided-B layout
    // (stride l): vl = l, vm = n / l, walking a dense causal layout.
    int32_t vl;
    int32_t vm;
    // Key rows.  Key t of the layout is sequence row key_pos(t) =
    // (t >> kcl) * kgl + koff + (t & (2^kcl - 1)), and km keys are valid.
    // Plain and residue views: kcl = 30, kgl = koff = 0 (key_pos(t) = t),
    // km = vm.  The compact view of fixed B (c = 2^kcl summary columns at
    // the end of every l = kgl positions): koff = l - c, km = (n / l) c, so
    // the c summary keys of every l-block are consecutive keys.  Only the
    // kernels that stream key tiles (forward, dQ) walk compact views.
    int32_t kcl;
    int32_t kgl;
    int32_t koff;
    int32_t km;
};

// Host-side pairing of one listing (see DevLayout).
struct Groups {
    std::vector<int32_t> ptr;
    std::vector<int32_t> blk;   // 2 per group
    std::vector<int32_t> step;  // 4 per step
};
Groups pair_blocks(const std::vector<int32_t>& ptr, const std::vector<int32_t>& idx,
                   const std::vector<int32_t>& mask);

}  // namespace sa

struct sa_layout {
    uint64_t serial;  // unique per build, keys the work-list cache
    int pattern;
    int64_t n, l, c;
    int32_t T;
    int64_t nqb, nkb, nnz, n_masks, allowed;  // nkb: key blocks (nqb but in a compact view)
    std::vector<int32_t> row_ptr, col_idx, mask_id;
    std::vector<uint64_t> masks;
    std::vector<int32_t> col_ptr, row_idx, csr_pos;
    sa::Groups qgroups, kgroups;  // pairs by query block / by key block
    // Sequence view of this layout when walked by the kernels (see
    // DevLayout): view_l = 1, view_m = n for a plain layout; the internal
    // dense causal layout behind a residue view has view_l = l, view_m = n/l.
    int64_t view_l = 1, view_m = 0;
    // Key rows of this layout when walked (see DevLayout): key_cl = 30,
    // key_gl = key_off = 0, key_m = view_m unless this is a compact view.
    int32_t key_cl = 30, key_gl = 0, key_off = 0;
    int64_t key_m = 0;
    // An alternate view the kernels walk instead of this layout, with the
    // same results:
    //  * residue view (strided B): the heads run as l dense causal attentions
    //    over the residue classes mod l; `view` is a dense causal layout on
    //    n/l rounded up to blocks, with view_l = l, view_m = n/l;
    //  * compact view (fixed B): the keys are the c summary columns of every
    //    l-block, consecutive; `view` lists query blocks against blocks of
    //    those (n/l) c keys.
    sa_layout* view = nullptr;
    int view_kind = 0;  // 0 none, 1 residue, 2 compact
    // Some partial quadrant leaves each lane of the forward's score layout
    // at most one allowed element (set when the layout is first uploaded).
    bool one_quads = false;
    // Wave-steps of the forward's walk with both 32-key halves live (not both
    // of one element per lane) and with one live half (set at upload).
    int64_t fwd_pair_steps = 0, fwd_half_steps = 0;

    std::mutex mu;                       // guards dev
    std::map<int, void*> dev_mem;        // device id -> allocation
    std::map<int, sa::DevLayout> dev;    // device id -> view
};

namespace sa {

// Layout builder (host only, layout.cpp).
int build_layout(int pattern, int64_t n, int64_t l, int64_t c, int32_t block, sa_layout** out);
// The residue view of strided B (block 64; n % l == 0) and the compact view
// of fixed B (block 64; n % l == 0, c a power of two).
int build_residue_view(int64_t n, int64_t l, sa_layout** out);
int build_compact_view(int64_t n, int64_t l, int64_t c, sa_layout** out);

// Error reporting (layout.cpp): records the message for sa_last_error and
// returns `status`; last_error() is the calling thread's last message.
int fail(int status, const char* fmt, ...);
const char* last_error();

}  // namespace sa
