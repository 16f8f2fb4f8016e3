// pack.h -- host side of what libsa uploads: the device image of a layout
// and the work lists of a call, built in host memory with no HIP calls (so
// that they can also be built and checked on the CPU alone).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "kernel_args.h"
#include "sa_internal.h"

namespace sa {

// A layout's device copy as one host buffer of 256-byte aligned sections,
// and where each section starts (see DevLayout for what they hold).
struct LayoutImage {
    std::vector<unsigned char> host;
    size_t off_masks, off_masks_t, off_planes, off_planes_t;
    size_t off_row_ptr, off_col_idx, off_mask_id, off_col_ptr, off_row_idx, off_col_mask;
    size_t off_gptr[2], off_gblk[2], off_gstep[2];
    size_t off_kmode, off_kblk;
    bool has_planes;  // block 64: lane-mask planes present
};

// Builds the image of L (and sets L's upload-time summaries: one_quads,
// fwd_pair_steps, fwd_half_steps).  Returns SA_OK.
int pack_layout(sa_layout* L, LayoutImage* img);

// The device view of an image copied to device address `base`.
DevLayout place_layout(const LayoutImage& img, const sa_layout* L, const unsigned char* base);

// What a work list's items walk: query blocks (fp32 forward), query-block
// pairs (bf16 forward; dQ, a list of its own since its chunks differ) or
// key-block pairs (dK/dV).
enum ListKind { kByQuery = 0, kByQueryPair = 1, kByKeyPair = 2, kByQueryPairDq = 3 };

// A compact view of fixed B (its keys are the summary positions).
inline bool is_compact(const sa_layout* L) { return L->key_gl != 0; }

// The chunks of a work list's long lists and what their combining passes
// read.  Every chunk has a slot: chunk_tab[slot] = {first step, steps} of
// its part of the list, and the kernel leaves its partial results in that
// slot.  groups: each chunked list of a layout walked as itself (not a
// compact view), {bh, pair index, first slot, chunks}, for the combining
// pass of its kernel.  cheads / cgroups: the dK/dV summing pass of compact
// views (see ReduceArgs): per compact (batch, head) {bh, offset into
// cgroups}; per key-block pair {first slot, chunks}.
struct Split {
    std::vector<int2> chunk_tab;
    std::vector<int4> groups;
    std::vector<int2> cheads;
    std::vector<int2> cgroups;
    int64_t slots = 0;
};

// The work items of a call over B batches and H heads (layout hl[h] for
// head h): one per (batch*head, block or pair, residue class), longest list
// first, so the heaviest items start early and the tail is made of short
// ones.  Chunking (the pair kinds; residue views never):
//   compact_steps > 0 (kByKeyPair): every key-block pair of a compact view
//     is walked in chunks of at most compact_steps steps, in list order;
//   plain_steps > 0: a list of any other layout longer than both plain_min
//     and plain_steps steps is cut into ceil(len / plain_steps) chunks of
//     near-equal length.
// split (if not null) receives the chunks' description.
void build_work_items(ListKind kind, int32_t B, int32_t H, sa_layout* const* hl, int32_t compact_steps,
                      int32_t plain_steps, int32_t plain_min, std::vector<Item>* out, Split* split = nullptr);

}  // namespace sa
