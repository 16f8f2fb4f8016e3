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
// pairs (bf16 forward, dQ) or key-block pairs (dK/dV).
enum ListKind { kByQuery = 0, kByQueryPair = 1, kByKeyPair = 2 };

// A compact view of fixed B (its keys are the summary positions).
inline bool is_compact(const sa_layout* L) { return L->key_gl != 0; }

// What the dK/dV kernel's chunks of compact views write and the summing
// pass reads (see ReduceArgs): per compact (batch, head) {bh, offset into
// groups}; per key-block pair {first slot, chunks}; the number of slots.
struct DkdvSplit {
    std::vector<int2> heads;
    std::vector<int2> groups;
    int64_t slots = 0;
};

// The work items of a call over B batches and H heads (layout hl[h] for
// head h): one per (batch*head, block or pair, residue class), longest list
// first, so the heaviest items start early and the tail is made of short
// ones.  With kind kByKeyPair and chunk_steps > 0, compact views' key-block
// pairs become one item per chunk of at most chunk_steps steps of their
// query lists, and split (if not null) receives their slots.
void build_work_items(ListKind kind, int32_t B, int32_t H, sa_layout* const* hl, int32_t chunk_steps,
                      std::vector<Item>* out, DkdvSplit* split = nullptr);

}  // namespace sa
