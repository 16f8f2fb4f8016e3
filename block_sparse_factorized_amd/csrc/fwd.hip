// fwd.hip -- block-sparse causal attention forward for gfx950.
//
// What is computed ("OpenAI Sparse Transformer", "Sparse Attention and
// Algorithmic Complexity" and "Implementation and Limitations"; "희소 어텐션
// (Sparse Attention)" for the softmax): for every query block the kernel
// walks the key blocks its layout lists, forms the score tile on the matrix
// cores, masks the disallowed elements of partial blocks, and folds the tile
// into an online softmax (running row max m, running row sum l, rescaled
// output accumulator).  At the end O = acc / l and lse = scale*m + ln l.
// Only O and lse leave the kernel; no score matrix is stored ("[논문 리뷰]
// Generating Long Sequences with Sparse Transformers", ABSTRACT (b)).
//
// bf16 kernel (block 64, d in {64, 128}), one workgroup of four waves per
// pair of query blocks of one (batch, head) whose key lists (nearly)
// coincide; waves 2m and 2m+1 own query rows 0..31 and 32..63 of member m,
// and the K/V tiles of the merged list are loaded once for both members.
//   * The score tile is computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: lane (hh = lane/32, n = lane%32) then holds
//     16 keys of query n per 32-key half, so the row max and row sum are
//     in-lane reductions plus one exchange with lane n+32 (v_permlane32_swap).
//   * The output is accumulated transposed too, O^T = V^T P^T, so the
//     softmax rescale factor of query n is in the lane that owns its output
//     column.  The score accumulators are already the B operand of that
//     product once each 16-key chunk's keys are taken in the order
//     {0-3, 8-11} (lanes 0-31) and {4-7, 12-15} (lanes 32-63); the matching
//     V^T operand comes straight from the row-major V tile through the
//     transposing LDS read (ds_read_b64_tr_b16).
//   * K and V tiles go from HBM straight into LDS (global_load_lds_dwordx4)
//     in a bank-conflict-free swizzled layout, double buffered: the next
//     tile's loads run under the current tile's work.
//   * Partial blocks are masked with 64-bit lane masks held in SGPRs (one
//     v_cndmask per element).  A 32 x 32 quadrant of the block (this wave's
//     32 rows, one 32-key half) with no allowed element is skipped: no score
//     products, softmax or output products for it; one whose every element
//     is allowed skips its masks; one where each lane holds at most one
//     allowed element takes one exponential per lane.
//   * Each live half is folded in on its own.  The running reference moves
//     only when a weight against it would exceed 2^8 (the half's row max is
//     more than 8 above it in log2 units), so the accumulator rescale is
//     rare.
//   * Work-list metadata is read with scalar loads, so waiting for it never
//     waits for tiles in flight.
//
// f32 kernel (block 16, d 64), one wave per (batch, head, query block), the
// same transposed structure on v_mfma_f32_16x16x4_f32.
#include <hip/hip_runtime.h>

#include "kernel_args.h"
#include "tiles.h"

namespace sa {
namespace {

// PAIRED: a step's two live halves are scored together and checked once (the
// better form when most steps have both halves live: full blocks); else each
// live half is folded in on its own (steps with one live half, or one
// allowed element per lane).
template <int D, bool PAIRED>
__global__ __launch_bounds__(256) void fwd_bf16_t64_kernel(const FwdArgs a)
{
    constexpr int T = 64;
    typedef Tile64<D, 4> TL;
    constexpr int NI = TL::kLoads;  // direct-to-LDS loads per wave per tensor
    // Two K/V buffers as separate objects: the loop below is unrolled by two
    // so that every step reads one buffer and fills the other with statically
    // known addresses, which lets the compiler see that the LDS reads of the
    // current tile do not wait for the tile in flight to the other buffer.
    __shared__ __attribute__((aligned(1024))) unsigned char kbuf0[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char vbuf0[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char kbuf1[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char vbuf1[TL::kBytes];

    // Work item: a pair of query blocks of one (batch, head) with nearly the
    // same key list; waves 0-1 own the rows of the first block, waves 2-3 the
    // rows of the second.  The K/V tiles of the merged list are shared.
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int member = w >> 1, wr = w & 1;
    const int n32 = lane & 31, hh = lane >> 5;
    const Item item = ld_uniform(&a.items[blockIdx.x]);
    const int bh = item.bh, grp = item.blk;
    // A chunk of a long list (slot >= 0) walks part of it and leaves partial
    // results in its slot for the combining pass.
    const bool chunk = item.slot >= 0;
    const DevLayout L = a.heads.lay[a.heads.head_lay[bh % a.H]];
    const int2 pair = ld_uniform(&L.qgrp_blk[grp]);
    const int qb = member ? pair.y : pair.x;  // -1: this wave has no rows
    // The walked sequence: row m is position r + vl*m of the head (vl = 1,
    // r = 0 for a plain layout), rs elements apart; rows >= vm are read
    // clamped and never written.  Key t is row key_pos(t) of it; keys >= km
    // are read clamped (and masked out).
    const int vl = L.vl, vm = L.vm, km = L.km;
    const int rs = vl * D;
    const int res = chunk ? 0 : item.r;
    const int64_t head = (int64_t)bh * a.n * D + (int64_t)res * D;
    const int64_t lrow0 = (int64_t)bh * a.n + res;  // lse index of row 0
    const unsigned short* Q = (const unsigned short*)a.q + head;
    const unsigned short* K = (const unsigned short*)a.k + head;
    const unsigned short* V = (const unsigned short*)a.v + head;
    const int q_local = 32 * wr + n32;
    const int q_row = (qb < 0 ? 0 : qb) * T + q_local;
    // this wave has rows that are not padding of a ragged last block
    const bool rows_live = qb >= 0 && qb * T + 32 * wr < vm;

    // Q^T as the B operand of S^T = K Q^T: lane (hh, n) holds d = 16c + 8hh .. +7 of query n.
    bf16x8 qop[D / 16];
    {
        const unsigned short* Qr = Q + (uint32_t)(min(q_row, vm - 1) * rs);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) qop[c] = *(const bf16x8*)(Qr + 16 * c + 8 * hh);
    }

    // Per-thread byte offsets of the direct-to-LDS loads from the tile's
    // first row (the same for every tile but a ragged last one).
    uint32_t goff[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u)
        goff[u] = 2u * (uint32_t)((key_pos(L, TL::load_row(u, w, lane)) - L.koff) * rs + TL::load_col(u, w, lane));
    // LDS byte offsets of this lane's K reads (A operand of S^T) and V transposing reads.
    int koff[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) koff[c] = TL::off(n32, 2 * c + hh);
    int voff[2][D / 32];
#pragma unroll
    for (int j4 = 0; j4 < 2; ++j4)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) voff[j4][dt] = TL::tr_off(lane, j4, dt);

    int p0 = ld_uniform(&L.qgrp_ptr[grp]);
    int nblk = ld_uniform(&L.qgrp_ptr[grp + 1]) - p0;
    if (chunk) {
        const int2 ct = ld_uniform(&a.chunk_tab[item.slot]);  // {first step, steps}
        p0 += ct.x;
        nblk = ct.y;
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    // Running reference m_ref (at most 8 / c2 below the row max seen so
    // far), mc = m_ref * c2, running sum l_run.  Per-half form: while a row
    // has no allowed key yet, m_ref = -inf and mc = -3e38, so its first
    // finite score moves the reference and its weights of -inf scores stay
    // 0.  PAIRED form: mc = 0 while m_ref = -inf, and no_ref tells that some
    // row of the wave has no reference yet.
    float m_ref = -INFINITY, mc = PAIRED ? 0.f : -3.0e38f, l_run = 0.f;
    bool no_ref = true;
    const float c2 = a.scale_log2;

    auto issue = [&](int kb, unsigned char* kd, unsigned char* vd) {
        const int64_t kr = (int64_t)key_pos(L, kb * T) * rs;
        const unsigned short* Kt = K + kr;
        const unsigned short* Vt = V + kr;
        const int last = km - 1 - kb * T;  // last valid key of the tile
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            uint32_t o = goff[u];
            if (last < T - 1) {  // ragged: clamp the key
                const int ln = opaque(lane);
                o = 2u * (uint32_t)((key_pos(L, min(TL::load_row(u, w, ln), last)) - L.koff) * rs +
                                    TL::load_col(u, w, ln));
            }
            __builtin_amdgcn_global_load_lds((glb_void*)sgpr_base_plus(Kt, o), (lds_void*)(kd + TL::load_dst(u, w)), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((glb_void*)sgpr_base_plus(Vt, o), (lds_void*)(vd + TL::load_dst(u, w)), 16, 0, 0);
        }
    };

    int4 st_cur = {0, 0, 0, 0}, st_nxt = {0, 0, 0, 0};
    if (nblk > 0) {
        st_cur = ld_uniform(&L.qgrp_step[p0]);
        st_nxt = ld_uniform(&L.qgrp_step[p0 + min(1, nblk - 1)]);
    }

    // One step: start the loads of tile t + 1 into (kn, vn), fold the tile
    // in (kc, vc) into the online softmax, then wait for tile t + 1.
    auto step_tile = [&](int t, const unsigned char* kc, const unsigned char* vc, unsigned char* kn,
                         unsigned char* vn) {
        // Step records are loaded two steps ahead, so no list read is waited
        // for in the step that uses it.
        const int4 step = st_cur;
        if (t + 1 < nblk) issue(st_nxt.x, kn, vn);
        st_cur = st_nxt;
        st_nxt = ld_uniform(&L.qgrp_step[p0 + min(t + 2, nblk - 1)]);
        const int mid = member ? step.z : step.y;  // -2: not in this block's list
        if (rows_live && mid != -2) {
            // Lane masks of every score register, one 64-bit plane each (a full
            // block reads plane set 0, all ones); the constant address space makes
            // these wave-uniform loads scalar loads.
            const_u64* pl = (const_u64*)(L.planes + ((int64_t)(mid + 1) * 2 + wr) * 32);
            // A 32-key half with no allowed element in this wave's rows (quadrant
            // (query half wr, key half kt) of the mask empty) has only zero
            // weights: its scores, softmax and products are skipped, since they
            // would only add zeros to the output.  Bit kt of lv: half kt is live.
            const unsigned lv = ((unsigned)step.w >> (4 * member + 2 * wr)) & 3u;
            // Bit kt of fl: every element of half kt is allowed, so its lane
            // masks are not applied.
            const unsigned fl = ((unsigned)step.w >> (8 + 4 * member + 2 * wr)) & 3u;
            // Bit kt of o1: each lane has at most one allowed element in half kt.
            const unsigned o1 = ((unsigned)step.w >> (16 + 4 * member + 2 * wr)) & a.one_bits;

            if constexpr (PAIRED) {
                // Both halves of the step together: their score products
                // back to back, then one lazy check over the step.

                // S^T = K Q^T: register i of s[kt] holds key 32*kt + 8*(i/4) + 4*hh + i%4 of query n.
                // A live half's operand reads first, then its products; then the
                // disallowed elements of a partial block to -inf.
                f32x16 s[2];
                auto scores = [&]() {
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
                        if ((lv >> kt) & 1u) {
                            // this half's 16 planes into SGPRs first, so the loads
                            // overlap the products
                            uint64_t pln[16];
                            const bool partial = mid >= 0 && !((fl >> kt) & 1u);
                            if (partial) {
#pragma unroll
                                for (int r = 0; r < 16; ++r) pln[r] = pl[16 * kt + r];
                            }
                            bf16x8 kop[D / 16];
#pragma unroll
                            for (int c = 0; c < D / 16; ++c) kop[c] = *(const bf16x8*)(kc + koff[c] + kt * 32 * TL::kRow);
#pragma unroll
                            for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
                            for (int c = 0; c < D / 16; ++c)
                                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[c], qop[c], s[kt], 0, 0, 0);
                            if (partial) {
#pragma unroll
                                for (int i = 0; i < 16; ++i)
                                    s[kt][i] = __builtin_amdgcn_inverse_ballot_w64(pln[i]) ? s[kt][i] : -INFINITY;
                            }
                        }
                };
                // Weights p = exp2(c2 s - mc) of the live halves, in place; returns
                // this lane's sum of them.
                auto weights = [&]() {
                    float lsum = 0.f;
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
                        if ((lv >> kt) & 1u) {
#pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][i], c2, -mc));
                                s[kt][i] = p;
                                lsum += p;
                            }
                        }
                    return lsum;
                };
                scores();

                // Lazy reference max.  Once every row of the wave has a reference,
                // the tile's max is not computed: the weights are taken against the
                // reference directly, and a per-lane sum of at most 2^8 shows that
                // no weight exceeds 2^8 (the bound the reference is kept to).  Else
                // (no reference yet, or a larger sum: some row's max moved up) the
                // scores are formed again and the exact path below moves the
                // reference to the row max, rescaling the accumulator.
                bool exact = no_ref;
                if (!exact) {
                    const float lsum = weights();
                    exact = __builtin_amdgcn_ballot_w64(!(lsum <= 256.f)) != 0;  // also catches inf
                    if (exact)
                        scores();
                    else
                        l_run += lsum;
                }
                if (exact) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
                        if ((lv >> kt) & 1u) {
#pragma unroll
                            for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, s[kt][i]);
                        }
                    mx = half_max(mx);
                    const float m_new = __builtin_fmaxf(m_ref, mx);
                    if (__builtin_amdgcn_ballot_w64(m_new > m_ref)) {
                        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_ref - m_new) * c2);
                        l_run *= alpha;
#pragma unroll
                        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                            for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
                        m_ref = m_new;
                        mc = m_ref == -INFINITY ? 0.f : m_ref * c2;
                    }
                    no_ref = __builtin_amdgcn_ballot_w64(m_ref == -INFINITY) != 0;
                    l_run += weights();
                }

                // P^T (chunk cc of P^T is registers 8*(cc%2)..+7 of s[cc/2]), then
                // O^T += V^T P^T, one live 32-key half at a time.
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    if ((lv >> kt) & 1u) {
                        bf16x8 vop[2][D / 32];
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int dt = 0; dt < D / 32; ++dt) {
                                const int cc = 2 * kt + h;
                                vop[h][dt] = lds_read_tr8(vc + voff[0][dt] + cc * 16 * TL::kRow,
                                                          vc + voff[1][dt] + cc * 16 * TL::kRow);
                            }
                        const bf16x8 pb[2] = {pack8(s[kt], 0), pack8(s[kt], 8)};
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int dt = 0; dt < D / 32; ++dt)
                                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[h][dt], pb[h], oacc[dt], 0, 0, 0);
                    }
            } else {
                // Each live half is folded in on its own: S^T = K Q^T, weights,
                // O^T += V^T P^T.  Register i of s holds key 32*kt + 8*(i/4) + 4*hh
                // + i%4 of query n.
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    if ((lv >> kt) & 1u) {
                        f32x16 s;
                        const bool partial = mid >= 0 && !((fl >> kt) & 1u);
                        const bool one = (o1 >> kt) & 1u;  // (implies partial)
                        // The half's 16 planes into SGPRs first, so the loads overlap
                        // the products; then S^T = K Q^T.
                        uint64_t pln[16];
                        if (partial) {
#pragma unroll
                            for (int r = 0; r < 16; ++r) pln[r] = pl[16 * kt + r];
                        }
                        {
                            bf16x8 kop[D / 16];
#pragma unroll
                            for (int c = 0; c < D / 16; ++c) kop[c] = *(const bf16x8*)(kc + koff[c] + kt * 32 * TL::kRow);
#pragma unroll
                            for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
                            for (int c = 0; c < D / 16; ++c)
                                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[c], qop[c], s, 0, 0, 0);
                        }
                        // Weights p = exp2(c2 s - mc), in place; returns this
                        // lane's sum of them.
                        auto weights = [&]() {
                            float lsum = 0.f;
#pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -mc));
                                s[i] = p;
                                lsum += p;
                            }
                            return lsum;
                        };
                        // O^T += V^T P^T (chunk h of this half's P^T is registers
                        // 8h..8h+7 of s).
                        auto products = [&]() {
                            bf16x8 vop[2][D / 32];
#pragma unroll
                            for (int h = 0; h < 2; ++h)
#pragma unroll
                                for (int dt = 0; dt < D / 32; ++dt) {
                                    const int cc = 2 * kt + h;
                                    vop[h][dt] = lds_read_tr8(vc + voff[0][dt] + cc * 16 * TL::kRow,
                                                              vc + voff[1][dt] + cc * 16 * TL::kRow);
                                }
                            const bf16x8 pb[2] = {pack8(s, 0), pack8(s, 8)};
#pragma unroll
                            for (int h = 0; h < 2; ++h)
#pragma unroll
                                for (int dt = 0; dt < D / 32; ++dt)
                                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[h][dt], pb[h], oacc[dt], 0, 0, 0);
                        };
                        // Lazy reference: the row max of the half is taken, but the
                        // reference m_ref (and with it the accumulator's scale) only
                        // moves when some weight against it would exceed 2^8, or when
                        // the row had no reference yet.  A half where each lane has at
                        // most one allowed element (strided B's diagonal blocks) takes
                        // that element's score x alone (-inf if the lane has none):
                        // one exponential per lane instead of sixteen.  Otherwise the
                        // disallowed elements of a partial half go to -inf first.
                        float mx = -INFINITY, x = -INFINITY;
                        if (one) {
#pragma unroll
                            for (int i = 0; i < 16; ++i) x = __builtin_amdgcn_inverse_ballot_w64(pln[i]) ? s[i] : x;
                            mx = x;
                        } else {
                            if (partial) {
#pragma unroll
                                for (int i = 0; i < 16; ++i)
                                    s[i] = __builtin_amdgcn_inverse_ballot_w64(pln[i]) ? s[i] : -INFINITY;
                            }
#pragma unroll
                            for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, s[i]);
                        }
                        mx = half_max(mx);
                        const bool move = fmaf(mx, c2, -mc) > 8.f;
                        if (__builtin_amdgcn_ballot_w64(move)) {
                            // (0 for a row's first reference: nothing is summed yet)
                            const float alpha = move ? __builtin_amdgcn_exp2f((m_ref - mx) * c2) : 1.f;
                            l_run *= alpha;
#pragma unroll
                            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                                for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
                            if (move) {
                                m_ref = mx;
                                mc = mx * c2;
                            }
                        }
                        if (one) {
                            const float p = __builtin_amdgcn_exp2f(fmaf(x, c2, -mc));
                            l_run += p;
#pragma unroll
                            for (int i = 0; i < 16; ++i) s[i] = __builtin_amdgcn_inverse_ballot_w64(pln[i]) ? p : 0.f;
                        } else {
                            l_run += weights();
                        }
                        products();
                    }
            }
        }  // this wave's block lists the key block
        wait_vmem();      // tile t + 1 has landed ...
        __syncthreads();  // ... for every wave, and every wave is done with tile t
    };

    if (nblk > 0) issue(st_cur.x, kbuf0, vbuf0);
    wait_vmem();
    __syncthreads();
    for (int t = 0; t < nblk; t += 2) {
        step_tile(t, kbuf0, vbuf0, kbuf1, vbuf1);
        if (t + 1 < nblk) step_tile(t + 1, kbuf1, vbuf1, kbuf0, vbuf0);
    }

    if (qb < 0) return;
    const float l_tot = l_run + swap_halves(l_run);
    if (chunk) {
        // This chunk's accumulator, row reference and row sum, each register
        // 64 lanes wide, for the combining pass.
        float* P = a.partials + (int64_t)item.slot * kFwdSlotFloats(D) + (int64_t)w * ((D / 32) * 16 + 2) * 64 + lane;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) P[(dt * 16 + i) * 64] = oacc[dt][i];
        P[((D / 32) * 16) * 64] = m_ref;
        P[((D / 32) * 16 + 1) * 64] = l_tot;
        return;
    }
    if (q_row >= vm) return;  // a ragged block's padding row
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    unsigned short* O = (unsigned short*)a.o + head + (uint32_t)(q_row * rs);
    // Register i of oacc[dt] holds d = 32*dt + 8*(i/4) + 4*hh + i%4 of query q_row.
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 u;
            u[0] = bf16_pair(oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv);
            u[1] = bf16_pair(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
            *(u32x2*)(O + 32 * dt + 8 * g + 4 * hh) = u;
        }
    if (hh == 0) a.lse[lrow0 + (uint32_t)(vl * q_row)] = l_tot > 0.f ? m_ref * a.scale + logf(l_tot) : -INFINITY;
}

// ---------------------------------------------------------------------------
// Combining pass of the chunks of long lists.  A chunk c of a row leaves its
// accumulator O_c = sum_j p_j v_j and row sum l_c, with weights p_j =
// exp2(c2 s_j - c2 m_c) against its own reference m_c.  With M the largest
// c2 m_c among the chunks that have weight (l_c > 0), the row's results are
// those of one pass over the whole list: O = sum_c f_c O_c / sum_c f_c l_c
// and lse = m* scale + log(sum_c f_c l_c), f_c = exp2(c2 m_c - M), m* the
// reference that gives M; the chunks are added in list order, so the result
// does not depend on which chunk ran first.  A row with no weight anywhere
// gets O = 0, lse = -inf, as in the forward.  Workgroup = one chunked pair,
// wave and lane as in the forward (wave 2m + wr: rows 32 wr .. of member m).
template <int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(const CombineArgs a)
{
    constexpr int T = 64, NR = (D / 32) * 16;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int member = w >> 1, wr = w & 1;
    const int n32 = lane & 31, hh = lane >> 5;
    const int4 g = ld_uniform(&a.groups[blockIdx.x]);  // {bh, pair, first slot, chunks}
    const DevLayout L = a.heads.lay[a.heads.head_lay[g.x % a.H]];
    const int2 pair = ld_uniform(&L.qgrp_blk[g.y]);
    const int qb = member ? pair.y : pair.x;
    if (qb < 0) return;
    const int q_row = qb * T + 32 * wr + n32;
    if (q_row >= L.vm) return;  // a ragged block's padding row
    const float c2 = a.scale_log2;
    const float* P0 = a.partials + (int64_t)g.z * kFwdSlotFloats(D) + (int64_t)w * (NR + 2) * 64 + lane;
    float mx = -INFINITY, m_best = -INFINITY;
    for (int c = 0; c < g.w; ++c) {
        const float* P = P0 + (int64_t)c * kFwdSlotFloats(D);
        const float m = P[NR * 64], l = P[(NR + 1) * 64];
        if (l > 0.f && m * c2 > mx) {
            mx = m * c2;
            m_best = m;
        }
    }
    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    float l_tot = 0.f;
    for (int c = 0; c < g.w; ++c) {
        const float* P = P0 + (int64_t)c * kFwdSlotFloats(D);
        const float l = P[(NR + 1) * 64];
        if (!(l > 0.f)) continue;
        const float f = __builtin_amdgcn_exp2f(P[NR * 64] * c2 - mx);
        l_tot += f * l;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dt][i] += f * P[(dt * 16 + i) * 64];
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t head = (int64_t)g.x * a.n * D;
    unsigned short* O = (unsigned short*)a.out0 + head + (uint32_t)(q_row * L.vl * D);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            u32x2 u;
            u[0] = bf16_pair(o[dt][4 * gg + 0] * inv, o[dt][4 * gg + 1] * inv);
            u[1] = bf16_pair(o[dt][4 * gg + 2] * inv, o[dt][4 * gg + 3] * inv);
            *(u32x2*)(O + 32 * dt + 8 * gg + 4 * hh) = u;
        }
    if (hh == 0)
        a.lse[(int64_t)g.x * a.n + (uint32_t)(L.vl * q_row)] = l_tot > 0.f ? m_best * a.scale + logf(l_tot) : -INFINITY;
}

__global__ __launch_bounds__(64) void fwd_f32_t16_d64_kernel(const FwdArgs a)
{
    constexpr int T = 16, D = 64, P = D + 4;
    __shared__ __attribute__((aligned(16))) float ks[T * P];
    __shared__ __attribute__((aligned(16))) float vs[T * P];

    const int lane = threadIdx.x, g = lane >> 4, n16 = lane & 15;
    const Item item = a.items[blockIdx.x];
    const int bh = item.bh, qb = item.blk;
    const DevLayout L = a.heads.lay[a.heads.head_lay[bh % a.H]];
    const int64_t head = (int64_t)bh * a.n * D;
    const float* Q = (const float*)a.q + head;
    const float* K = (const float*)a.k + head;
    const float* V = (const float*)a.v + head;
    const int64_t q_row = (int64_t)qb * T + n16;

    float qop[D / 4];
#pragma unroll
    for (int c = 0; c < D / 4; ++c) qop[c] = Q[q_row * D + 4 * c + g];

    const int p0 = L.row_ptr[qb];
    const int nblk = L.row_ptr[qb + 1] - p0;
    f32x4 oacc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float c2 = a.scale_log2;

    for (int t = 0; t < nblk; ++t) {
        const int kb = L.col_idx[p0 + t];
        const int mid = L.mask_id[p0 + t];
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int idx = lane + 64 * u, row = idx / (D / 4), c4 = idx % (D / 4);
            *(f32x4*)&ks[row * P + 4 * c4] = *(const f32x4*)(K + ((int64_t)kb * T + row) * D + 4 * c4);
            *(f32x4*)&vs[row * P + 4 * c4] = *(const f32x4*)(V + ((int64_t)kb * T + row) * D + 4 * c4);
        }
        __syncthreads();

        // S^T = K Q^T: register i holds key 4*g + i of query n16.
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 4; ++c)
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(ks[n16 * P + 4 * c + g], qop[c], s, 0, 0, 0);
        if (mid >= 0) {
            // Row n16 of a 16x16 mask is bits (n16%4)*16 .. +15 of word n16/4.
            uint64_t word = L.masks[(int64_t)mid * (T * T / 64) + n16 / 4];
            unsigned bits = (unsigned)(word >> ((n16 % 4) * 16 + 4 * g));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (!((bits >> i) & 1u)) s[i] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
        const float mc = m_use * c2;
        float lsum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -mc));
            lsum += s[i];
        }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            oacc[dt] *= alpha;
            // O^T += V^T P^T, one key per lane group and step: key 4*g + i.
#pragma unroll
            for (int i = 0; i < 4; ++i)
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vs[(4 * g + i) * P + 16 * dt + n16], s[i],
                                                               oacc[dt], 0, 0, 0);
        }
    }

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot = l_tot + __shfl_xor(l_tot, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* O = (float*)a.o + head + q_row * D;
    // Register i of oacc[dt] holds d = 16*dt + 4*g + i of query q_row.
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) *(f32x4*)(O + 16 * dt + 4 * g) = oacc[dt] * inv;
    if (g == 0)
        a.lse[(int64_t)bh * a.n + q_row] = l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY;
}

}  // namespace

hipError_t launch_fwd_bf16_t64(int d, const FwdArgs& a, int n_items, bool paired, hipStream_t stream)
{
    const dim3 g(n_items), b(256);
    if (d == 64 && paired)
        hipLaunchKernelGGL((fwd_bf16_t64_kernel<64, true>), g, b, 0, stream, a);
    else if (d == 64)
        hipLaunchKernelGGL((fwd_bf16_t64_kernel<64, false>), g, b, 0, stream, a);
    else if (paired)
        hipLaunchKernelGGL((fwd_bf16_t64_kernel<128, true>), g, b, 0, stream, a);
    else
        hipLaunchKernelGGL((fwd_bf16_t64_kernel<128, false>), g, b, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fwd_combine_bf16(int d, const CombineArgs& a, int n_groups, hipStream_t stream)
{
    if (d == 64)
        hipLaunchKernelGGL((fwd_combine_kernel<64>), dim3(n_groups), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((fwd_combine_kernel<128>), dim3(n_groups), dim3(256), 0, stream, a);
    return hipGetLastError();
}


hipError_t launch_fwd_f32_t16(int d, const FwdArgs& a, int n_items, hipStream_t stream)
{
    (void)d;
    hipLaunchKernelGGL(fwd_f32_t16_d64_kernel, dim3(n_items), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sa
