// kernel_args.h -- argument blocks passed by value to the libsa kernels and
// the host-side launchers (defined in the .hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_internal.h"

namespace sa {

// One (batch*H + head, block, residue) work item.  blk is a query block for
// the fp32 forward kernel, and an index into the layout's pair lists
// (query-block pairs for the bf16 forward and dQ kernels, key-block pairs for
// the dK/dV kernel) otherwise; r is the residue class of a residue view.
// A compact view's key-block pair is walked by the dK/dV kernel in chunks
// of its query list: then r is the chunk's first step and slot (>= 0) the
// partial-sum slot the chunk writes; slot is -1 for every other item.
struct Item {
    int32_t bh;
    int32_t blk;
    int32_t r;     // residue class (0 for a plain layout), or a chunk's first step
    int32_t slot;  // partial-sum slot of a compact view's chunk, else -1
};

// Sequence row of key t of a layout (DevLayout: key rows); t itself but in
// the compact view of fixed B.
__device__ inline int key_pos(const DevLayout& L, int t)
{
    return (t >> L.kcl) * L.kgl + L.koff + (t & ((1 << L.kcl) - 1));
}

struct HeadTable {
    DevLayout lay[kMaxLayouts];
    uint8_t head_lay[kMaxHeads];  // head -> index into lay
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int64_t n;
    int32_t H;
    float scale;       // score scale
    float scale_log2;  // scale * log2(e)
    const Item* items;
    HeadTable heads;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* ndelta;  // workspace: -D_i = -sum_t dO_it * O_it, fp32 [B*H*n]
    float* nl2;    // workspace: -lse_i * log2(e) (-inf for an empty row), fp32 [B*H*n]
    int64_t n;
    int32_t H;
    int32_t BH;
    float scale;
    float scale_log2;
    const Item* items;  // work list of the launch
    HeadTable heads;
    // dK/dV of compact views: each chunk's fp32 partial sums, kSlotFloats(D)
    // floats per slot laid out [dK, dV][member][64 keys][D], and the steps
    // per chunk.
    float* partials;
    int32_t chunk_steps;
};

// Floats of one partial-sum slot: dK and dV of a pair of 64-key blocks.
constexpr int64_t kSlotFloats(int d) { return 2 * 2 * 64 * (int64_t)d; }

// The summing pass of a compact view's dK/dV: one entry per (batch, head)
// walked in a compact view, {bh, offset of its groups' entries in groups}.
// groups[offset + g] = {first slot, chunks} of key-block pair g.
struct ReduceArgs {
    void* dk;
    void* dv;
    const float* partials;
    const int2* heads_tab;  // [n_heads] {bh, offset}
    const int2* groups;
    int64_t n;
    int32_t H;
    float scale;
    HeadTable heads;
};

// Launchers: enqueue one kernel on `stream`, return hipGetLastError().
// paired: the forward form that scores a step's two live halves together.
hipError_t launch_fwd_bf16_t64(int d, const FwdArgs& a, int n_items, bool paired, hipStream_t stream);
hipError_t launch_fwd_f32_t16(int d, const FwdArgs& a, int n_items, hipStream_t stream);
hipError_t launch_bwd_rowterms_bf16(int d, const BwdArgs& a, int64_t rows, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16_t64(int d, const BwdArgs& a, int n_items, hipStream_t stream);
// The summing pass after the dK/dV kernel when compact views are walked:
// every row of each of the n_heads (batch, head) pairs, n rows each.
hipError_t launch_bwd_dkdv_reduce_bf16(int d, const ReduceArgs& a, int n_heads, int64_t n, hipStream_t stream);
// rowterms: the dQ kernel also forms the row terms of its rows and writes
// them to the workspace (no row-term launch before it).  one (with
// rowterms): the form with a one-exponential path for quadrants whose lanes
// hold at most one allowed element each.
hipError_t launch_bwd_dq_bf16_t64(int d, const BwdArgs& a, int n_items, bool rowterms, bool one,
                                  hipStream_t stream);

}  // namespace sa
