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
// A long list is walked in chunks (see Split in pack.h): then slot (>= 0) is
// the chunk's partial-result slot, chunk_tab[slot] = {first step, steps}
// gives its part of the list, and r is 0; slot is -1 for every other item.
struct Item {
    int32_t bh;
    int32_t blk;
    int32_t r;     // residue class (0 for a plain layout or a chunk)
    int32_t slot;  // partial-result slot of a chunk, else -1
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
    // Chunks of long lists: {first step, steps} per slot, and the fp32
    // partial results, kFwdSlotFloats(D) floats per slot (see fwd.hip).
    const int2* chunk_tab;
    float* partials;
    // 3: one-element halves take the one-exponential path; 0: never.
    uint32_t one_bits;
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
    // Chunks of long lists: {first step, steps} per slot, and the fp32
    // partial results: for the dK/dV kernel kSlotFloats(D) floats per slot
    // laid out [dK, dV][member][64 keys][D]; for the dQ kernel
    // kDqSlotFloats(D), per wave its dQ registers, lane-major.
    const int2* chunk_tab;
    float* partials;
};

// Floats of one partial-sum slot of the dK/dV kernel: dK and dV of a pair of
// 64-key blocks.
constexpr int64_t kSlotFloats(int d) { return 2 * 2 * 64 * (int64_t)d; }
// Floats of one slot of the dQ kernel: 4 waves x (d/32 x 16 registers) x 64 lanes.
constexpr int64_t kDqSlotFloats(int d) { return 4 * (int64_t)(d / 32) * 16 * 64; }
// Floats of one slot of the bf16 forward: 4 waves x (d/32 x 16 accumulator
// registers, the row reference m_ref and the row sum) x 64 lanes.
constexpr int64_t kFwdSlotFloats(int d) { return 4 * (int64_t)((d / 32) * 16 + 2) * 64; }

// The combining pass of chunked lists: groups[g] = {bh, pair index, first
// slot, chunks} of every chunked list of a plain layout; one workgroup per
// group adds the chunks' partial results in chunk order and writes the
// pair's rows (forward: O and lse; dQ: dQ; dK/dV: dK and dV).
struct CombineArgs {
    void* out0;    // o, dq or dk
    void* out1;    // dv (dK/dV)
    float* lse;    // forward
    const float* partials;
    const int4* groups;
    int64_t n;
    int32_t H;
    float scale;
    float scale_log2;
    HeadTable heads;
};

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
// The combining passes take n_groups (> 0) groups.
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
hipError_t launch_fwd_combine_bf16(int d, const CombineArgs& a, int n_groups, hipStream_t stream);
hipError_t launch_dq_combine_bf16(int d, const CombineArgs& a, int n_groups, hipStream_t stream);
hipError_t launch_dkdv_combine_bf16(int d, const CombineArgs& a, int n_groups, hipStream_t stream);

}  // namespace sa
