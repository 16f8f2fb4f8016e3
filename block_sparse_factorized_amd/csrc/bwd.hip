// bwd.hip -- recompute-style backward of block-sparse causal attention, gfx950.
//
// "[논문 리뷰] Generating Long Sequences with Sparse Transformers" (nubint.ai),
// ABSTRACT item (b) and "제안 방법"; pcnews.ru, "Глубокое внимание": the
// attention matrix is recomputed during backpropagation instead of stored.
// Only O and lse come from the forward pass.  With c = scale:
//     P_ij  = exp(c s_ij - lse_i)        (recomputed per block)
//     D_i   = sum_t dO_it O_it           (formed by the dQ kernel, or by
//                                          the row-term kernel alone)
//     dP_ij = dO_i . v_j,   dS_ij = P_ij (dP_ij - D_i)
//     dQ_i  = c sum_j dS_ij k_j                             (dQ kernel, one
//             workgroup per pair of query blocks, walking their merged
//             key-block lists; runs first)
//     dV_j  = sum_i P_ij dO_i,  dK_j = c sum_i dS_ij q_i   (dK/dV kernel,
//             one workgroup per pair of key blocks, walking their merged
//             query-block lists; runs second, reading the row terms)
// Both kernels write their outputs once, with no atomics, so results are
// deterministic.
//
// Both follow the forward kernel's scheme: 32x32x16 bf16 MFMA tiles, the
// 64-row tiles that stream through the loop go straight from HBM to a
// swizzled LDS layout (double buffered), operands that must run along the
// sequence axis are read with the transposing LDS load, the sequence index of
// each 16-long reduction chunk is taken in the order {0-3, 8-11} (lanes 0-31)
// and {4-7, 12-15} (lanes 32-63) so that accumulator registers feed the next
// MFMA directly, partial-block masks are 64-bit lane masks in SGPRs, and a
// 32 x 32 quadrant of a block with no allowed element is skipped (it would
// only add zeros).
#include <hip/hip_runtime.h>

#include "kernel_args.h"
#include "tiles.h"

namespace sa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float bf16_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline void zero(f32x16& x)
{
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.f;
}

// ---------------------------------------------------------------------------
// Row terms, D/8 threads per row:  -D_i = -sum_t dO_it O_it  and
// nl2_i = -lse_i * log2(e)  (-inf for an empty row, whose P is all zero).
template <int D>
__global__ __launch_bounds__(256) void bwd_rowterms_kernel(const BwdArgs a, int64_t rows)
{
    constexpr int TPR = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / TPR;
    const int part = (int)(gid % TPR);
    float acc = 0.f;
    if (row < rows) {
        u32x4 x = *(const u32x4*)((const unsigned short*)a.o + row * D + part * 8);
        u32x4 y = *(const u32x4*)((const unsigned short*)a.dout + row * D + part * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += bf16_lo(x[e]) * bf16_lo(y[e]) + bf16_hi(x[e]) * bf16_hi(y[e]);
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off);
    if (row < rows && part == 0) {
        a.ndelta[row] = -acc;
        const float l = a.lse[row];
        a.nl2[row] = l == -INFINITY ? -INFINITY : -l * kLog2e;
    }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = a pair of key blocks of one (batch, head) with nearly
// the same query list (waves 0-1: keys of the first, waves 2-3: keys of the
// second), walking the merged query list with shared, double-buffered Q/dO
// tiles and row terms.  Lane (hh, n) of wave w holds key 32*(w%2) + n.
//   S    = Q K^T     C[q][key]  A = Q rows (LDS)          B = K^T (registers)
//   dP   = dO V^T    C[q][key]  A = dO rows (LDS)         B = V^T (registers)
//   dV^T += dO^T P   C[d][key]  A = dO^T (transposing LDS read)  B = P
//   dK^T += Q^T dS   C[d][key]  A = Q^T (transposing LDS read)   B = dS
// Register i of an S or dP tile qt holds query 32*qt + 8*(i/4) + 4*hh + i%4.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(const BwdArgs a)
{
    constexpr int T = 64;
    typedef Tile64<D, 4> TL;
    constexpr int NI = TL::kLoads;
    // Two sets of Q/dO/row-term buffers as separate objects, used alternately
    // by a loop unrolled by two, so that the LDS reads of the current tile
    // are seen not to depend on the loads in flight to the other set.
    __shared__ __attribute__((aligned(1024))) unsigned char qbuf0[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char obuf0[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char qbuf1[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char obuf1[TL::kBytes];
    __shared__ __attribute__((aligned(16))) float rbuf0[2 * T];  // nl2[64], then -D[64]
    __shared__ __attribute__((aligned(16))) float rbuf1[2 * T];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int member = w >> 1, wr = w & 1;
    const int n32 = lane & 31, hh = lane >> 5;
    const Item item = ld_uniform(&a.items[blockIdx.x]);
    const int bh = item.bh, grp = item.blk;
    // A chunk of a long query list (slot >= 0: chunk_tab[slot] = {first
    // step, steps}) leaves fp32 partial sums in its slot for a summing pass.
    const bool chunk = item.slot >= 0;
    const int res = chunk ? 0 : item.r;
    const DevLayout L = a.heads.lay[a.heads.head_lay[bh % a.H]];
    const int2 pair = ld_uniform(&L.kgrp_blk[grp]);
    const int kb = member ? pair.y : pair.x;  // -1: this wave has no keys
    // Key half this wave holds and the query halves it takes: normally its
    // own half (wr) against both query halves; when the member's whole list
    // only has allowed elements in one key half, both waves hold that half
    // and wave wr takes query half wr (their partial dK, dV are summed at
    // the end), so neither wave idles.
    const int modes = ld_uniform(&L.kgrp_mode[grp]);
    const int kmode = (modes >> (2 * member)) & 3;
    const int kh = kmode ? kmode - 1 : wr;
    const unsigned qsel = kmode ? 1u << wr : 3u;
    // The walked sequence: row m is position r + vl*m of the head (vl = 1,
    // r = 0 for a plain layout), rs elements apart; rows >= vm are read
    // clamped, get zero weight and are never written.  Key t is row
    // key_pos(t) of it (the compact view's summary keys), km keys valid.
    const int vl = L.vl, vm = L.vm, km = L.km;
    const int rs = vl * D;
    const int64_t head = (int64_t)bh * a.n * D + (int64_t)res * D;
    const int64_t lrow0 = (int64_t)bh * a.n + res;  // row-term index of row 0
    const unsigned short* Q = (const unsigned short*)a.q + head;
    const unsigned short* dO = (const unsigned short*)a.dout + head;
    const float* nl2g = a.nl2 + lrow0;
    const float* dlg = a.ndelta + lrow0;
    const int k_local = 32 * kh + n32;
    const int k_row = (kb < 0 ? 0 : kb) * T + k_local;
    // this wave holds keys that are not padding of a ragged last block
    const bool keys_live = kb >= 0 && kb * T + 32 * kh < km;

    bf16x8 kop[D / 16], vop[D / 16];
    {
        const uint32_t kr = (uint32_t)(key_pos(L, min(k_row, km - 1)) * rs);
        const unsigned short* K = (const unsigned short*)a.k + head + kr;
        const unsigned short* V = (const unsigned short*)a.v + head + kr;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            kop[c] = *(const bf16x8*)(K + 16 * c + 8 * hh);
            vop[c] = *(const bf16x8*)(V + 16 * c + 8 * hh);
        }
    }
    // Byte offsets of the direct-to-LDS loads from the tile's first row (the
    // same for every tile but a ragged last one).
    uint32_t goff[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u)
        goff[u] = 2u * (uint32_t)(TL::load_row(u, w, lane) * rs + TL::load_col(u, w, lane));
    int aoff[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) aoff[c] = TL::off(n32, 2 * c + hh);
    int toff[2][D / 32];
#pragma unroll
    for (int j4 = 0; j4 < 2; ++j4)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) toff[j4][dt] = TL::tr_off(lane, j4, dt);

    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        zero(dk[dt]);
        zero(dv[dt]);
    }
    const int g0 = ld_uniform(&L.kgrp_ptr[grp]);
    const int glen = ld_uniform(&L.kgrp_ptr[grp + 1]) - g0;
    int p0 = g0, nblk = glen;
    if (chunk) {
        const int2 ct = ld_uniform(&a.chunk_tab[item.slot]);
        p0 += ct.x;
        nblk = ct.y;
    }
    const float c2 = a.scale_log2;

    // Starts the loads of query tile qb into (qd, od) and returns this lane's
    // row term for it (wave 0: nl2, wave 1: -D; a padding row gets nl2 =
    // -inf, so zero weight, and -D = 0), which the caller stores to LDS.
    auto issue = [&](int qb, unsigned char* qd, unsigned char* od) {
        const unsigned short* Qt = Q + (int64_t)qb * T * rs;
        const unsigned short* Ot = dO + (int64_t)qb * T * rs;
        const int last = vm - 1 - qb * T;  // last valid row of the tile
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            uint32_t o = goff[u];
            if (last < T - 1) {  // ragged: clamp the row
                const int ln = opaque(lane);
                o = 2u * (uint32_t)(min(TL::load_row(u, w, ln), last) * rs + TL::load_col(u, w, ln));
            }
            __builtin_amdgcn_global_load_lds((glb_void*)sgpr_base_plus(Qt, o), (lds_void*)(qd + TL::load_dst(u, w)), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((glb_void*)sgpr_base_plus(Ot, o), (lds_void*)(od + TL::load_dst(u, w)), 16, 0, 0);
        }
        float rt = 0.f;
        if (w < 2) {
            const int m = qb * T + lane;
            if (m < vm)
                rt = (w == 0 ? nl2g : dlg)[(uint32_t)(vl * m)];
            else
                rt = w == 0 ? -INFINITY : 0.f;
        }
        return rt;
    };

    int4 st_cur = {0, 0, 0, 0}, st_nxt = {0, 0, 0, 0};
    if (nblk > 0) {
        st_cur = ld_uniform(&L.kgrp_step[p0]);
        st_nxt = ld_uniform(&L.kgrp_step[p0 + min(1, nblk - 1)]);
    }

    // One step: start the next tile's loads into (qn, on, rn), accumulate the
    // tile in (qc, oc, rc), then wait for the next tile.
    auto step_tile = [&](int t, const unsigned char* qc, const unsigned char* oc, const float* rc,
                         unsigned char* qn, unsigned char* on, float* rn) {
        // Step records are loaded two steps ahead, so no list read is waited
        // for in the step that uses it.
        const int4 step = st_cur;
        float rt_next = 0.f;
        if (t + 1 < nblk) rt_next = issue(st_nxt.x, qn, on);
        st_cur = st_nxt;
        st_nxt = ld_uniform(&L.kgrp_step[p0 + min(t + 2, nblk - 1)]);
        const int mid = member ? step.z : step.y;  // -2: this key block is not listed
        if (keys_live && mid != -2) {
            // Transposed lane-mask planes (set 0, all ones, for a full block).
            // A 32-query half is live when the mask has an allowed element in
            // quadrant (query half qt, key half kh).
            const_u64* pl = (const_u64*)(L.planes_t + ((int64_t)(mid + 1) * 2 + kh) * 32);
            const unsigned quad = (unsigned)step.w >> (4 * member);
            bool live[2];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) live[qt] = ((quad >> (2 * qt + kh)) & (qsel >> qt) & 1u) != 0;

            // One 32-query half at a time; a half with no allowed element for
            // this wave's keys is skipped entirely (it would only add zeros).
            // Masked elements get s = -inf, hence P = exp2(c2 s - lse log2 e)
            // = 0 and dS = P (dP - D) = 0.  The half is one straight-line
            // block: its planes (scalar loads) and every LDS operand it needs
            // are requested first, then the products, so the wave waits for
            // memory once per half rather than once per product.
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
                if (live[qt]) {
                    // (a half whose every element is allowed skips its lane masks)
                    const bool partial = ((quad >> (8 + 2 * qt + kh)) & 1u) == 0;
                    uint64_t pln[16];
                    if (partial) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) pln[r] = pl[16 * qt + r];
                    }
                    bf16x8 qa[D / 16], oa[D / 16];
#pragma unroll
                    for (int c = 0; c < D / 16; ++c) {
                        qa[c] = *(const bf16x8*)(qc + aoff[c] + qt * 32 * TL::kRow);
                        oa[c] = *(const bf16x8*)(oc + aoff[c] + qt * 32 * TL::kRow);
                    }
                    // dP starts from -D of its query rows, so the product gives dP - D.
                    f32x16 s, dp;
                    f32x4 nl[4];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 nd = *(const f32x4*)&rc[T + 32 * qt + 8 * g + 4 * hh];
#pragma unroll
                        for (int e = 0; e < 4; ++e) dp[4 * g + e] = nd[e];
                        nl[g] = *(const f32x4*)&rc[32 * qt + 8 * g + 4 * hh];
                    }
                    bf16x8 ot[2][D / 32], qt8[2][D / 32];
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int dt = 0; dt < D / 32; ++dt) {
                            const int cc = 2 * qt + h;
                            ot[h][dt] = lds_read_tr8(oc + toff[0][dt] + cc * 16 * TL::kRow, oc + toff[1][dt] + cc * 16 * TL::kRow);
                            qt8[h][dt] = lds_read_tr8(qc + toff[0][dt] + cc * 16 * TL::kRow, qc + toff[1][dt] + cc * 16 * TL::kRow);
                        }
                    zero(s);
#pragma unroll
                    for (int c = 0; c < D / 16; ++c) {
                        s = mfma(qa[c], kop[c], s);
                        dp = mfma(oa[c], vop[c], dp);
                    }
                    // all LDS reads first, then the S and dP products
                    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 16) + 8 + 8 * (D / 32), 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2 * (D / 16), 0);
                    if (partial) {
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            s[i] = __builtin_amdgcn_inverse_ballot_w64(pln[i]) ? s[i] : -INFINITY;
                    }
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int i = 4 * g + e;
                            const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c2, nl[g][e]));
                            s[i] = p;
                            dp[i] = p * dp[i];
                        }
                    }
                    const bf16x8 pb[2] = {pack8(s, 0), pack8(s, 8)};
                    const bf16x8 db[2] = {pack8(dp, 0), pack8(dp, 8)};
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int dt = 0; dt < D / 32; ++dt) {
                            dv[dt] = mfma(ot[h][dt], pb[h], dv[dt]);
                            dk[dt] = mfma(qt8[h][dt], db[h], dk[dt]);
                        }
                }
        }  // this wave's key block is listed by the query block
        if (w < 2 && t + 1 < nblk) rn[T * w + lane] = rt_next;
        wait_vmem();
        __syncthreads();
    };

    if (nblk > 0) {
        const float rt0 = issue(st_cur.x, qbuf0, obuf0);
        if (w < 2) rbuf0[T * w + lane] = rt0;
    }
    wait_vmem();
    __syncthreads();
    for (int t = 0; t < nblk; t += 2) {
        step_tile(t, qbuf0, obuf0, rbuf0, qbuf1, obuf1, rbuf1);
        if (t + 1 < nblk) step_tile(t + 1, qbuf1, obuf1, rbuf1, qbuf0, obuf0, rbuf0);
    }

    // Shared-half members: wave 1 hands its partial sums to wave 0 through
    // the (now idle) tile buffers, laid out [dt][i][lane].
    if (modes != 0) {
        float* rk = (float*)(member ? qbuf1 : qbuf0);
        float* rv = (float*)(member ? obuf1 : obuf0);
        if (kmode && wr == 1) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    rk[(dt * 16 + i) * 64 + lane] = dk[dt][i];
                    rv[(dt * 16 + i) * 64 + lane] = dv[dt][i];
                }
        }
        __syncthreads();
        if (kmode && wr == 0) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    dk[dt][i] += rk[(dt * 16 + i) * 64 + lane];
                    dv[dt][i] += rv[(dt * 16 + i) * 64 + lane];
                }
        }
    }
    if (kb < 0) return;
    // Each wave writes one 32-key half of its block (its valid rows).  In a shared-half member
    // wave 0 writes the shared half, wave 1 the other half, whose keys no
    // query reaches: zeros.
    int out_local = k_local;
    if (kmode && wr == 1) {
        out_local = 32 * (1 - kh) + n32;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            zero(dk[dt]);
            zero(dv[dt]);
        }
    }
    if (chunk) {
        // The chunk's fp32 partial sums (dK unscaled), [dK, dV][member][key][d]:
        // the summing pass adds the chunks of each pair in order.
        float* P = a.partials + (int64_t)item.slot * kSlotFloats(D) + (int64_t)(member * 64 + out_local) * D;
        float* PV = P + 2 * 64 * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = 32 * dt + 8 * g + 4 * hh;
                *(f32x4*)(P + c) = f32x4{dk[dt][4 * g], dk[dt][4 * g + 1], dk[dt][4 * g + 2], dk[dt][4 * g + 3]};
                *(f32x4*)(PV + c) = f32x4{dv[dt][4 * g], dv[dt][4 * g + 1], dv[dt][4 * g + 2], dv[dt][4 * g + 3]};
            }
        return;
    }
    const int out_row = kb * T + out_local;
    if (out_row >= vm) return;  // a ragged block's padding row
    // Register i of dk[dt]/dv[dt]: d = 32*dt + 8*(i/4) + 4*hh + i%4 of key out_row.
    unsigned short* DK = (unsigned short*)a.dk + head + (uint32_t)(out_row * rs);
    unsigned short* DV = (unsigned short*)a.dv + head + (uint32_t)(out_row * rs);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 uk, uv;
            uk[0] = bf16_pair(dk[dt][4 * g] * a.scale, dk[dt][4 * g + 1] * a.scale);
            uk[1] = bf16_pair(dk[dt][4 * g + 2] * a.scale, dk[dt][4 * g + 3] * a.scale);
            uv[0] = bf16_pair(dv[dt][4 * g], dv[dt][4 * g + 1]);
            uv[1] = bf16_pair(dv[dt][4 * g + 2], dv[dt][4 * g + 3]);
            *(u32x2*)(DK + 32 * dt + 8 * g + 4 * hh) = uk;
            *(u32x2*)(DV + 32 * dt + 8 * g + 4 * hh) = uv;
        }
}

// ---------------------------------------------------------------------------
// Summing pass of a compact view's dK/dV (fixed B): the dK/dV kernel walks
// each key-block pair of summary keys in chunks of its query list and leaves
// one fp32 partial sum per chunk; here every row of the head is written
// once: a summary row (position j with j mod l >= l - c, key t = (j / l) c +
// j mod l - (l - c)) gets the sum of its pair's chunks taken in chunk order,
// dK scaled, both rounded to bf16; every other row, which no query
// reaches, gets zeros.  One workgroup per 64 rows of one head, D/8 threads
// per row, 8 consecutive elements each.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(const ReduceArgs a)
{
    constexpr int TPR = D / 8, RPP = 256 / TPR;  // threads per row, rows per pass
    const int64_t nrb = (a.n + 63) / 64;
    const int hx = (int)(blockIdx.x / nrb);
    const int64_t r0 = (int64_t)(blockIdx.x % nrb) * 64;
    const int2 ht = ld_uniform(&a.heads_tab[hx]);  // {bh, offset into groups}
    const DevLayout L = a.heads.lay[a.heads.head_lay[ht.x % a.H]];
    const int l = L.kgl, c = 1 << L.kcl, off = L.koff;
    const int part = threadIdx.x % TPR;
    for (int pass = 0; pass < 64 / RPP; ++pass) {
        const int64_t j = r0 + pass * RPP + threadIdx.x / TPR;
        if (j >= a.n) break;
        f32x4 k0 = {0.f, 0.f, 0.f, 0.f}, k1 = k0, v0 = k0, v1 = k0;
        const int jm = (int)(j % l);
        if (jm >= off) {
            const int t = (int)(j / l) * c + (jm - off);
            const int2 gm = L.kblk_grp[t >> 6];  // {pair, member}
            if (gm.x >= 0) {
                const int2 gs = a.groups[ht.y + gm.x];  // {first slot, chunks}
                const int64_t e = (int64_t)(gm.y * 64 + (t & 63)) * D + 8 * part;
                for (int ch = 0; ch < gs.y; ++ch) {
                    const float* P = a.partials + (int64_t)(gs.x + ch) * kSlotFloats(D) + e;
                    k0 += *(const f32x4*)P;
                    k1 += *(const f32x4*)(P + 4);
                    v0 += *(const f32x4*)(P + 2 * 64 * D);
                    v1 += *(const f32x4*)(P + 2 * 64 * D + 4);
                }
            }
        }
        const int64_t o = ((int64_t)ht.x * a.n + j) * D + 8 * part;
        u32x4 uk, uv;
        uk[0] = bf16_pair(k0[0] * a.scale, k0[1] * a.scale);
        uk[1] = bf16_pair(k0[2] * a.scale, k0[3] * a.scale);
        uk[2] = bf16_pair(k1[0] * a.scale, k1[1] * a.scale);
        uk[3] = bf16_pair(k1[2] * a.scale, k1[3] * a.scale);
        uv[0] = bf16_pair(v0[0], v0[1]);
        uv[1] = bf16_pair(v0[2], v0[3]);
        uv[2] = bf16_pair(v1[0], v1[1]);
        uv[3] = bf16_pair(v1[2], v1[3]);
        *(u32x4*)((unsigned short*)a.dk + o) = uk;
        *(u32x4*)((unsigned short*)a.dv + o) = uv;
    }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = a pair of query blocks of one (batch, head) with nearly the
// same key list (waves 0-1: rows of the first, waves 2-3: rows of the
// second), walking the merged key list with shared, double-buffered K/V
// tiles.  Lane (hh, n) of wave w holds query 32*(w%2) + n of its block.
//   S^T  = K Q^T      C[key][q]  A = K rows (LDS)          B = Q^T (registers)
//   dP^T = V dO^T     C[key][q]  A = V rows (LDS)          B = dO^T (registers)
//   dQ^T += K^T dS^T  C[d][q]    A = K^T (transposing LDS read)  B = dS^T
// With d = 64 the kernel fits four waves per SIMD (the ONE form spills one
// value, used only after the loop).  ROWTERMS: the kernel forms the row
// terms of its rows from O, dO and lse itself and writes them to the
// workspace, so that no row-term launch precedes it (the dK/dV kernel then
// runs after it).  ONE: quadrants whose lanes hold at most one allowed
// element each take the one-exponential path.
template <int D, bool ROWTERMS, bool ONE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 1))) void bwd_dq_kernel(
    const BwdArgs a)
{
    constexpr int T = 64;
    typedef Tile64<D, 4> TL;
    constexpr int NI = TL::kLoads;
    // Two K/V buffer pairs as separate objects, used alternately by a loop
    // unrolled by two (see the dK/dV kernel).
    __shared__ __attribute__((aligned(1024))) unsigned char kbuf0[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char vbuf0[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char kbuf1[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char vbuf1[TL::kBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int member = w >> 1, wr = w & 1;
    const int n32 = lane & 31, hh = lane >> 5;
    const Item item = ld_uniform(&a.items[blockIdx.x]);
    const int bh = item.bh, grp = item.blk;
    // A chunk of a long key list (slot >= 0: chunk_tab[slot] = {first step,
    // steps}) leaves its fp32 dQ in its slot for the combining pass.
    const bool chunk = item.slot >= 0;
    const int2 ct = chunk ? ld_uniform(&a.chunk_tab[item.slot]) : make_int2(0, 0);
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
    const int64_t lrow0 = (int64_t)bh * a.n + res;  // row-term index of row 0
    const unsigned short* K = (const unsigned short*)a.k + head;
    const unsigned short* V = (const unsigned short*)a.v + head;
    const int q_local = 32 * wr + n32;
    const int q_row = (qb < 0 ? 0 : qb) * T + q_local;
    const int q_rc = min(q_row, vm - 1);  // clamped for reads
    // this wave has rows that are not padding of a ragged last block
    const bool rows_live = qb >= 0 && qb * T + 32 * wr < vm;

    bf16x8 qop[D / 16], dop[D / 16];
    {
        const unsigned short* Qr = (const unsigned short*)a.q + head + (uint32_t)(q_rc * rs);
        const unsigned short* Or = (const unsigned short*)a.dout + head + (uint32_t)(q_rc * rs);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            qop[c] = *(const bf16x8*)(Qr + 16 * c + 8 * hh);
            dop[c] = *(const bf16x8*)(Or + 16 * c + 8 * hh);
        }
    }
    float nl2, nd_i;
    const uint32_t trow = (uint32_t)(vl * q_rc);  // row-term index from lrow0
    if constexpr (ROWTERMS) {
        // The row terms of this wave's rows, as the row-term kernel forms
        // them: -D_i = -sum_t dO_it O_it (lane hh holds d = 16c + 8hh .. +7,
        // the other half comes from lane n + 32) and -lse_i log2(e).  They
        // are written out for the dK/dV kernel, which runs after this one.
        const unsigned short* Xr = (const unsigned short*)a.o + head + (uint32_t)(q_rc * rs);
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            const u32x4 x = *(const u32x4*)(Xr + 16 * c + 8 * hh);
            const u32x4 y = __builtin_bit_cast(u32x4, dop[c]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc += bf16_lo(x[e]) * bf16_lo(y[e]) + bf16_hi(x[e]) * bf16_hi(y[e]);
        }
        nd_i = -(acc + swap_halves(acc));
        const float l = a.lse[lrow0 + trow];
        nl2 = l == -INFINITY ? -INFINITY : -l * kLog2e;
        // (every chunk of a list forms the same row terms; its first writes them)
        if (hh == 0 && qb >= 0 && q_row < vm && ct.x == 0) {
            a.ndelta[lrow0 + trow] = nd_i;
            a.nl2[lrow0 + trow] = nl2;
        }
    } else {
        nl2 = a.nl2[lrow0 + trow];
        nd_i = a.ndelta[lrow0 + trow];
    }
    // Byte offsets of the direct-to-LDS loads from the tile's first row (the
    // same for every tile but a ragged last one).
    uint32_t goff[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u)
        goff[u] = 2u * (uint32_t)((key_pos(L, TL::load_row(u, w, lane)) - L.koff) * rs + TL::load_col(u, w, lane));
    int aoff[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) aoff[c] = TL::off(n32, 2 * c + hh);
    int toff[2][D / 32];
#pragma unroll
    for (int j4 = 0; j4 < 2; ++j4)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) toff[j4][dt] = TL::tr_off(lane, j4, dt);

    f32x16 dq[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) zero(dq[dt]);
    int p0 = ld_uniform(&L.qgrp_ptr[grp]);
    int nblk = ld_uniform(&L.qgrp_ptr[grp + 1]) - p0;
    if (chunk) {
        p0 += ct.x;
        nblk = ct.y;
    }
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

    // One step: start the next tile's loads into (kn, vn), accumulate the
    // tile in (kc, vc), then wait for the next tile.
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
            // Lane-mask planes (set 0, all ones, for a full block) first, so the
            // scalar loads overlap the products.  A 32-key half is live when
            // the mask has an allowed element in quadrant (query half wr, key
            // half kt).
            const_u64* pl = (const_u64*)(L.planes + ((int64_t)(mid + 1) * 2 + wr) * 32);
            uint64_t pln[32];
#pragma unroll
            for (int r = 0; r < 32; ++r) pln[r] = pl[r];
            const unsigned quad = (unsigned)step.w >> (4 * member);
            bool live[2], partial[2], one[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                live[kt] = (quad >> (2 * wr + kt)) & 1u;
                // (a half whose every element is allowed skips its lane masks)
                partial[kt] = mid >= 0 && !((quad >> (8 + 2 * wr + kt)) & 1u);
                // at most one allowed element per lane (used by the ONE form)
                one[kt] = ONE && ((quad >> (16 + 2 * wr + kt)) & 1u);
            }

            // One 32-key half at a time; a half with no allowed element for
            // this wave's rows is skipped entirely (it would only add zeros).
            // Register i of a half's tile: key 32*kt + 8*(i/4) + 4*hh + i%4
            // of query q_local.  Masked elements get s = -inf, so P^T and
            // dS^T = P^T (dP^T - D) are zero there.
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                if (live[kt]) {
                    f32x16 s, dp;
                    bf16x8 kop[2][D / 32];
                    // transposed K, the A operand of dQ^T += K^T dS^T
                    auto read_kop = [&]() {
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int dt = 0; dt < D / 32; ++dt) {
                                const int cc = 2 * kt + h;
                                kop[h][dt] = lds_read_tr8(kc + toff[0][dt] + cc * 16 * TL::kRow, kc + toff[1][dt] + cc * 16 * TL::kRow);
                            }
                    };
                    zero(s);
                    zero(dp);
                    if constexpr (ONE) {
                        // operands read per product (the registers the
                        // one-element path needs)
#pragma unroll
                        for (int c = 0; c < D / 16; ++c) {
                            const bf16x8 ka = *(const bf16x8*)(kc + aoff[c] + kt * 32 * TL::kRow);
                            const bf16x8 va = *(const bf16x8*)(vc + aoff[c] + kt * 32 * TL::kRow);
                            s = mfma(ka, qop[c], s);
                            dp = mfma(va, dop[c], dp);
                        }
                    } else {
                        bf16x8 ka[D / 16], va[D / 16];
#pragma unroll
                        for (int c = 0; c < D / 16; ++c) {
                            ka[c] = *(const bf16x8*)(kc + aoff[c] + kt * 32 * TL::kRow);
                            va[c] = *(const bf16x8*)(vc + aoff[c] + kt * 32 * TL::kRow);
                        }
#pragma unroll
                        for (int c = 0; c < D / 16; ++c) {
                            s = mfma(ka[c], qop[c], s);
                            dp = mfma(va[c], dop[c], dp);
                        }
                    }
                    if (one[kt]) {
                        // At most one allowed element per lane (strided B's
                        // diagonal blocks): its P and dS alone, one
                        // exponential instead of sixteen, then dS scattered
                        // back (zero elsewhere).
                        float x = -INFINITY, y = 0.f;
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const bool b = __builtin_amdgcn_inverse_ballot_w64(pln[16 * kt + i]);
                            x = b ? s[i] : x;
                            y = b ? dp[i] : y;
                        }
                        const float ds = __builtin_amdgcn_exp2f(fmaf(x, c2, nl2)) * (y + nd_i);
#pragma unroll
                        for (int i = 0; i < 16; ++i) dp[i] = __builtin_amdgcn_inverse_ballot_w64(pln[16 * kt + i]) ? ds : 0.f;
                    } else {
                        if (partial[kt]) {
#pragma unroll
                            for (int i = 0; i < 16; ++i)
                                s[i] = __builtin_amdgcn_inverse_ballot_w64(pln[16 * kt + i]) ? s[i] : -INFINITY;
                        }
                        if constexpr (!ONE) read_kop();
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c2, nl2));
                            dp[i] = p * (dp[i] + nd_i);
                        }
                    }
                    if constexpr (ONE) read_kop();
                    const bf16x8 db[2] = {pack8(dp, 0), pack8(dp, 8)};
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int dt = 0; dt < D / 32; ++dt) dq[dt] = mfma(kop[h][dt], db[h], dq[dt]);
                }
        }  // this wave's block lists the key block
        wait_vmem();
        __syncthreads();
    };

    if (nblk > 0) issue(st_cur.x, kbuf0, vbuf0);
    wait_vmem();
    __syncthreads();
    for (int t = 0; t < nblk; t += 2) {
        step_tile(t, kbuf0, vbuf0, kbuf1, vbuf1);
        if (t + 1 < nblk) step_tile(t + 1, kbuf1, vbuf1, kbuf0, vbuf0);
    }

    if (qb < 0) return;  // no rows
    if (chunk) {
        // this chunk's (unscaled) dQ registers, 64 lanes wide, for the combining pass
        float* P = a.partials + (int64_t)item.slot * kDqSlotFloats(D) + (int64_t)w * (D / 32) * 16 * 64 + lane;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) P[(dt * 16 + i) * 64] = dq[dt][i];
        return;
    }
    if (q_row >= vm) return;  // a ragged block's padding row
    unsigned short* DQ = (unsigned short*)a.dq + head + (uint32_t)(q_row * rs);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 u;
            u[0] = bf16_pair(dq[dt][4 * g] * a.scale, dq[dt][4 * g + 1] * a.scale);
            u[1] = bf16_pair(dq[dt][4 * g + 2] * a.scale, dq[dt][4 * g + 3] * a.scale);
            *(u32x2*)(DQ + 32 * dt + 8 * g + 4 * hh) = u;
        }
}

// ---------------------------------------------------------------------------
// Combining pass of the dQ kernel's chunks: each chunked query-block pair's
// rows get the sum of its chunks' fp32 dQ, taken in list order, scaled and
// rounded to bf16 (what one pass over the whole list writes, up to the
// order of the sum).  Wave and lane as in the dQ kernel.
template <int D>
__global__ __launch_bounds__(256) void dq_combine_kernel(const CombineArgs a)
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
    if (q_row >= L.vm) return;
    const float* P0 = a.partials + (int64_t)g.z * kDqSlotFloats(D) + (int64_t)w * NR * 64 + lane;
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) zero(acc[dt]);
    for (int c = 0; c < g.w; ++c) {
        const float* P = P0 + (int64_t)c * kDqSlotFloats(D);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[dt][i] += P[(dt * 16 + i) * 64];
    }
    unsigned short* DQ = (unsigned short*)a.out0 + (int64_t)g.x * a.n * D + (uint32_t)(q_row * L.vl * D);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            u32x2 u;
            u[0] = bf16_pair(acc[dt][4 * gg] * a.scale, acc[dt][4 * gg + 1] * a.scale);
            u[1] = bf16_pair(acc[dt][4 * gg + 2] * a.scale, acc[dt][4 * gg + 3] * a.scale);
            *(u32x2*)(DQ + 32 * dt + 8 * gg + 4 * hh) = u;
        }
}

// Combining pass of the dK/dV kernel's chunks of plain layouts: each chunked
// key-block pair's rows (both members, the valid rows of a ragged last
// block) get the sums of its chunks' fp32 partials ([dK, dV][member][key][d]
// per slot), taken in list order; dK scaled; both rounded to bf16.  D/8
// threads per row, 8 consecutive elements each.
template <int D>
__global__ __launch_bounds__(256) void dkdv_combine_kernel(const CombineArgs a)
{
    constexpr int TPR = D / 8, RPP = 256 / TPR;  // threads per row, rows per pass
    const int4 g = ld_uniform(&a.groups[blockIdx.x]);  // {bh, pair, first slot, chunks}
    const DevLayout L = a.heads.lay[a.heads.head_lay[g.x % a.H]];
    const int2 pair = ld_uniform(&L.kgrp_blk[g.y]);
    const int part = threadIdx.x % TPR;
    for (int pass = 0; pass < 128 / RPP; ++pass) {
        const int rr = pass * RPP + threadIdx.x / TPR;  // member * 64 + key
        const int member = rr >> 6, key = rr & 63;
        const int kb = member ? pair.y : pair.x;
        if (kb < 0) continue;
        const int row = kb * 64 + key;
        if (row >= L.vm) continue;
        f32x4 k0 = {0.f, 0.f, 0.f, 0.f}, k1 = k0, v0 = k0, v1 = k0;
        const int64_t e = (int64_t)rr * D + 8 * part;
        for (int c = 0; c < g.w; ++c) {
            const float* P = a.partials + (int64_t)(g.z + c) * kSlotFloats(D) + e;
            k0 += *(const f32x4*)P;
            k1 += *(const f32x4*)(P + 4);
            v0 += *(const f32x4*)(P + 2 * 64 * D);
            v1 += *(const f32x4*)(P + 2 * 64 * D + 4);
        }
        const int64_t o = (int64_t)g.x * a.n * D + (int64_t)row * L.vl * D + 8 * part;
        u32x4 uk, uv;
        uk[0] = bf16_pair(k0[0] * a.scale, k0[1] * a.scale);
        uk[1] = bf16_pair(k0[2] * a.scale, k0[3] * a.scale);
        uk[2] = bf16_pair(k1[0] * a.scale, k1[1] * a.scale);
        uk[3] = bf16_pair(k1[2] * a.scale, k1[3] * a.scale);
        uv[0] = bf16_pair(v0[0], v0[1]);
        uv[1] = bf16_pair(v0[2], v0[3]);
        uv[2] = bf16_pair(v1[0], v1[1]);
        uv[3] = bf16_pair(v1[2], v1[3]);
        *(u32x4*)((unsigned short*)a.out0 + o) = uk;
        *(u32x4*)((unsigned short*)a.out1 + o) = uv;
    }
}

}  // namespace

hipError_t launch_bwd_rowterms_bf16(int d, const BwdArgs& a, int64_t rows, hipStream_t stream)
{
    const int64_t threads = rows * (d / 8);
    const unsigned grid = (unsigned)((threads + 255) / 256);
    if (d == 64)
        hipLaunchKernelGGL(bwd_rowterms_kernel<64>, dim3(grid), dim3(256), 0, stream, a, rows);
    else
        hipLaunchKernelGGL(bwd_rowterms_kernel<128>, dim3(grid), dim3(256), 0, stream, a, rows);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16_t64(int d, const BwdArgs& a, int n_items, hipStream_t stream)
{
    if (d == 64)
        hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3(n_items), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3(n_items), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv_reduce_bf16(int d, const ReduceArgs& a, int n_heads, int64_t n, hipStream_t stream)
{
    const dim3 g((unsigned)(n_heads * ((n + 63) / 64))), b(256);
    if (d == 64)
        hipLaunchKernelGGL(bwd_dkdv_reduce_kernel<64>, g, b, 0, stream, a);
    else
        hipLaunchKernelGGL(bwd_dkdv_reduce_kernel<128>, g, b, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16_t64(int d, const BwdArgs& a, int n_items, bool rowterms, bool one, hipStream_t stream)
{
    const dim3 g(n_items), b(256);
    if (d == 64 && rowterms && one)
        hipLaunchKernelGGL((bwd_dq_kernel<64, true, true>), g, b, 0, stream, a);
    else if (d == 64 && rowterms)
        hipLaunchKernelGGL((bwd_dq_kernel<64, true, false>), g, b, 0, stream, a);
    else if (d == 64)
        hipLaunchKernelGGL((bwd_dq_kernel<64, false, false>), g, b, 0, stream, a);
    else if (rowterms && one)
        hipLaunchKernelGGL((bwd_dq_kernel<128, true, true>), g, b, 0, stream, a);
    else if (rowterms)
        hipLaunchKernelGGL((bwd_dq_kernel<128, true, false>), g, b, 0, stream, a);
    else
        hipLaunchKernelGGL((bwd_dq_kernel<128, false, false>), g, b, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_dq_combine_bf16(int d, const CombineArgs& a, int n_groups, hipStream_t stream)
{
    if (d == 64)
        hipLaunchKernelGGL(dq_combine_kernel<64>, dim3(n_groups), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(dq_combine_kernel<128>, dim3(n_groups), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_dkdv_combine_bf16(int d, const CombineArgs& a, int n_groups, hipStream_t stream)
{
    if (d == 64)
        hipLaunchKernelGGL(dkdv_combine_kernel<64>, dim3(n_groups), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(dkdv_combine_kernel<128>, dim3(n_groups), dim3(256), 0, stream, a);
    return hipGetLastError();
}



}  // namespace sa
