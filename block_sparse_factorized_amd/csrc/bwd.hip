// bwd.hip -- recompute-style backward of block-sparse causal attention, gfx950.
//
// "[논문 리뷰] Generating Long Sequences with Sparse Transformers" (nubint.ai),
// ABSTRACT item (b) and "제안 방법"; pcnews.ru, "Глубокое внимание": the
// attention matrix is recomputed during backpropagation instead of stored.
// Only O and lse come from the forward pass.  With c = scale:
//     P_ij  = exp(c s_ij - lse_i)        (recomputed per block)
//     D_i   = sum_t dO_it O_it           (row-term kernel)
//     dP_ij = dO_i . v_j,   dS_ij = P_ij (dP_ij - D_i)
//     dV_j  = sum_i P_ij dO_i,  dK_j = c sum_i dS_ij q_i   (dK/dV kernel,
//             one workgroup per key block, walking its query blocks)
//     dQ_i  = c sum_j dS_ij k_j                             (dQ kernel, one
//             workgroup per query block, walking its key blocks)
// Both kernels write their outputs once, with no atomics, so results are
// deterministic.
//
// Both follow the forward kernel's scheme: 32x32x16 bf16 MFMA tiles, the
// 64-row tiles that stream through the loop go straight from HBM to a
// swizzled LDS layout (double buffered), operands that must run along the
// sequence axis are read with the transposing LDS load, the sequence index of
// each 16-long reduction chunk is taken in the order {0-3, 8-11} (lanes 0-31)
// and {4-7, 12-15} (lanes 32-63) so that accumulator registers feed the next
// MFMA directly, and partial-block masks are 64-bit lane masks in SGPRs.
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
// Row terms, D/8 threads per row:  D_i = sum_t dO_it O_it  and
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
        a.delta[row] = acc;
        const float l = a.lse[row];
        a.nl2[row] = l == -INFINITY ? -INFINITY : -l * kLog2e;
    }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = key block (bh, kb), wave w owns keys 32w..32w+31 and
// walks the query blocks that list kb.  Lane (hh, n) holds key 32w + n.
//   S    = Q K^T     C[q][key]  A = Q rows (LDS)          B = K^T (registers)
//   dP   = dO V^T    C[q][key]  A = dO rows (LDS)         B = V^T (registers)
//   dV^T += dO^T P   C[d][key]  A = dO^T (transposing LDS read)  B = P
//   dK^T += Q^T dS   C[d][key]  A = Q^T (transposing LDS read)   B = dS
// Register i of an S or dP tile qt holds query 32*qt + 8*(i/4) + 4*hh + i%4.
template <int D>
__global__ __launch_bounds__(128) void bwd_dkdv_kernel(const BwdArgs a)
{
    constexpr int T = 64;
    typedef Tile64<D> TL;
    constexpr int NI = TL::kBytes / 2048;
    __shared__ __attribute__((aligned(1024))) unsigned char qbuf0[TL::kBytes], qbuf1[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char obuf0[TL::kBytes], obuf1[TL::kBytes];
    __shared__ __attribute__((aligned(16))) float rbuf0[2 * T], rbuf1[2 * T];  // nl2[64], then D[64]

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n32 = lane & 31, hh = lane >> 5;
    const Item item = a.items[blockIdx.x];
    const int bh = item.bh, kb = item.blk;
    const DevLayout L = a.heads.lay[a.heads.head_lay[bh % a.H]];
    const int64_t head = (int64_t)bh * a.n * D;
    const unsigned short* Q = (const unsigned short*)a.q + head;
    const unsigned short* dO = (const unsigned short*)a.dout + head;
    const float* nl2g = a.nl2 + (int64_t)bh * a.n;
    const float* dlg = a.delta + (int64_t)bh * a.n;
    const int k_local = 32 * w + n32;
    const int64_t k_row = (int64_t)kb * T + k_local;

    bf16x8 kop[D / 16], vop[D / 16];
    {
        const unsigned short* K = (const unsigned short*)a.k + head + k_row * D;
        const unsigned short* V = (const unsigned short*)a.v + head + k_row * D;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            kop[c] = *(const bf16x8*)(K + 16 * c + 8 * hh);
            vop[c] = *(const bf16x8*)(V + 16 * c + 8 * hh);
        }
    }
    int goff[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) goff[u] = TL::load_src(u, w, lane);
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
    const int p0 = L.col_ptr[kb];
    const int nblk = L.col_ptr[kb + 1] - p0;
    const float c2 = a.scale_log2;
    const bf16x8 zero8 = __builtin_bit_cast(bf16x8, (u32x4){0u, 0u, 0u, 0u});

    auto issue = [&](int qb, unsigned char* qd, unsigned char* od, float* rd) {
        const unsigned short* Qt = Q + (int64_t)qb * T * D;
        const unsigned short* Ot = dO + (int64_t)qb * T * D;
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            __builtin_amdgcn_global_load_lds((glb_void*)(Qt + goff[u]), (lds_void*)(qd + TL::load_dst(u, w)), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((glb_void*)(Ot + goff[u]), (lds_void*)(od + TL::load_dst(u, w)), 16, 0, 0);
        }
        const float* src = (w == 0 ? nl2g : dlg) + (int64_t)qb * T + lane;
        __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)(rd + T * w), 4, 0, 0);
    };

    if (nblk > 0) issue(L.row_idx[p0], qbuf0, obuf0, rbuf0);
    wait_vmem();
    __syncthreads();

    for (int t = 0; t < nblk; ++t) {
        const bool odd = t & 1;
        const unsigned char* qc = odd ? qbuf1 : qbuf0;
        const unsigned char* oc = odd ? obuf1 : obuf0;
        const float* rc = odd ? rbuf1 : rbuf0;
        if (t + 1 < nblk) issue(L.row_idx[p0 + t + 1], odd ? qbuf0 : qbuf1, odd ? obuf0 : obuf1, odd ? rbuf0 : rbuf1);
        const int mid = L.col_mask[p0 + t];

        f32x16 s[2], dp[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            zero(s[qt]);
            zero(dp[qt]);
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const bf16x8 qa = *(const bf16x8*)(qc + aoff[c] + qt * 32 * TL::kRow);
                const bf16x8 oa = *(const bf16x8*)(oc + aoff[c] + qt * 32 * TL::kRow);
                s[qt] = mfma(qa, kop[c], s[qt]);
                dp[qt] = mfma(oa, vop[c], dp[qt]);
            }
        }
        // Masked elements get s = -inf, hence P = exp2(c2 s - lse log2 e) = 0 and
        // dS = P (dP - D) = 0.  A 32-query half with no allowed element for
        // this wave's keys has zero P and dS: its elementwise work is skipped,
        // its products still run.
        bool live[2] = {true, true};
        if (mid >= 0) {
            const_u64* pl = (const_u64*)(L.planes_t + ((int64_t)mid * 2 + w) * 32);
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                uint64_t any = 0;
#pragma unroll
                for (int i = 0; i < 16; ++i) any |= pl[16 * qt + i];
                live[qt] = any != 0;
                if (live[qt]) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        s[qt][i] = __builtin_amdgcn_inverse_ballot_w64(pl[16 * qt + i]) ? s[qt][i] : -INFINITY;
                }
            }
        }
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            bf16x8 pb[2] = {zero8, zero8}, db[2] = {zero8, zero8};
            if (live[qt]) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 nl = *(const f32x4*)&rc[32 * qt + 8 * g + 4 * hh];
                    const f32x4 dd = *(const f32x4*)&rc[T + 32 * qt + 8 * g + 4 * hh];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 4 * g + e;
                        const float p = __builtin_amdgcn_exp2f(fmaf(s[qt][i], c2, nl[e]));
                        s[qt][i] = p;
                        dp[qt][i] = p * (dp[qt][i] - dd[e]);
                    }
                }
                pb[0] = pack8(s[qt], 0);
                pb[1] = pack8(s[qt], 8);
                db[0] = pack8(dp[qt], 0);
                db[1] = pack8(dp[qt], 8);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    const int cc = 2 * qt + h;
                    const bf16x8 ot = lds_read_tr8(oc + toff[0][dt] + cc * 16 * TL::kRow, oc + toff[1][dt] + cc * 16 * TL::kRow);
                    const bf16x8 qt8 = lds_read_tr8(qc + toff[0][dt] + cc * 16 * TL::kRow, qc + toff[1][dt] + cc * 16 * TL::kRow);
                    dv[dt] = mfma(ot, pb[h], dv[dt]);
                    dk[dt] = mfma(qt8, db[h], dk[dt]);
                }
        }
        wait_vmem();
        __syncthreads();
    }

    // Register i of dk[dt]/dv[dt]: d = 32*dt + 8*(i/4) + 4*hh + i%4 of key k_row.
    unsigned short* DK = (unsigned short*)a.dk + head + k_row * D;
    unsigned short* DV = (unsigned short*)a.dv + head + k_row * D;
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
// dQ: workgroup = query block (bh, qb), wave w owns queries 32w..32w+31 and
// walks the key blocks of the query block.  Lane (hh, n) holds query 32w + n.
//   S^T  = K Q^T      C[key][q]  A = K rows (LDS)          B = Q^T (registers)
//   dP^T = V dO^T     C[key][q]  A = V rows (LDS)          B = dO^T (registers)
//   dQ^T += K^T dS^T  C[d][q]    A = K^T (transposing LDS read)  B = dS^T
template <int D>
__global__ __launch_bounds__(128) void bwd_dq_kernel(const BwdArgs a)
{
    constexpr int T = 64;
    typedef Tile64<D> TL;
    constexpr int NI = TL::kBytes / 2048;
    __shared__ __attribute__((aligned(1024))) unsigned char kbuf0[TL::kBytes], kbuf1[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char vbuf0[TL::kBytes], vbuf1[TL::kBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n32 = lane & 31, hh = lane >> 5;
    const Item item = a.items[blockIdx.x];
    const int bh = item.bh, qb = item.blk;
    const DevLayout L = a.heads.lay[a.heads.head_lay[bh % a.H]];
    const int64_t head = (int64_t)bh * a.n * D;
    const unsigned short* K = (const unsigned short*)a.k + head;
    const unsigned short* V = (const unsigned short*)a.v + head;
    const int q_local = 32 * w + n32;
    const int64_t q_row = (int64_t)qb * T + q_local;

    bf16x8 qop[D / 16], dop[D / 16];
    {
        const unsigned short* Qr = (const unsigned short*)a.q + head + q_row * D;
        const unsigned short* Or = (const unsigned short*)a.dout + head + q_row * D;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            qop[c] = *(const bf16x8*)(Qr + 16 * c + 8 * hh);
            dop[c] = *(const bf16x8*)(Or + 16 * c + 8 * hh);
        }
    }
    const float nl2 = a.nl2[(int64_t)bh * a.n + q_row];
    const float d_i = a.delta[(int64_t)bh * a.n + q_row];
    int goff[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) goff[u] = TL::load_src(u, w, lane);
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
    const int p0 = L.row_ptr[qb];
    const int nblk = L.row_ptr[qb + 1] - p0;
    const float c2 = a.scale_log2;
    const bf16x8 zero8 = __builtin_bit_cast(bf16x8, (u32x4){0u, 0u, 0u, 0u});

    auto issue = [&](int kb, unsigned char* kd, unsigned char* vd) {
        const unsigned short* Kt = K + (int64_t)kb * T * D;
        const unsigned short* Vt = V + (int64_t)kb * T * D;
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            __builtin_amdgcn_global_load_lds((glb_void*)(Kt + goff[u]), (lds_void*)(kd + TL::load_dst(u, w)), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((glb_void*)(Vt + goff[u]), (lds_void*)(vd + TL::load_dst(u, w)), 16, 0, 0);
        }
    };

    if (nblk > 0) issue(L.col_idx[p0], kbuf0, vbuf0);
    wait_vmem();
    __syncthreads();

    for (int t = 0; t < nblk; ++t) {
        const bool odd = t & 1;
        const unsigned char* kc = odd ? kbuf1 : kbuf0;
        const unsigned char* vc = odd ? vbuf1 : vbuf0;
        if (t + 1 < nblk) issue(L.col_idx[p0 + t + 1], odd ? kbuf0 : kbuf1, odd ? vbuf0 : vbuf1);
        const int mid = L.mask_id[p0 + t];

        f32x16 s[2], dp[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            zero(s[kt]);
            zero(dp[kt]);
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const bf16x8 ka = *(const bf16x8*)(kc + aoff[c] + kt * 32 * TL::kRow);
                const bf16x8 va = *(const bf16x8*)(vc + aoff[c] + kt * 32 * TL::kRow);
                s[kt] = mfma(ka, qop[c], s[kt]);
                dp[kt] = mfma(va, dop[c], dp[kt]);
            }
        }
        // Register i of tile kt: key 32*kt + 8*(i/4) + 4*hh + i%4 of query
        // q_local.  Masked elements get s = -inf, so P^T and dS^T = P^T (dP^T -
        // D) are zero there; a 32-key half with no allowed element for this
        // wave's queries is skipped.
        bool live[2] = {true, true};
        if (mid >= 0) {
            const_u64* pl = (const_u64*)(L.planes + ((int64_t)mid * 2 + w) * 32);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                uint64_t any = 0;
#pragma unroll
                for (int i = 0; i < 16; ++i) any |= pl[16 * kt + i];
                live[kt] = any != 0;
                if (live[kt]) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        s[kt][i] = __builtin_amdgcn_inverse_ballot_w64(pl[16 * kt + i]) ? s[kt][i] : -INFINITY;
                }
            }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            bf16x8 db[2] = {zero8, zero8};
            if (live[kt]) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][i], c2, nl2));
                    dp[kt][i] = p * (dp[kt][i] - d_i);
                }
                db[0] = pack8(dp[kt], 0);
                db[1] = pack8(dp[kt], 8);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    const int cc = 2 * kt + h;
                    const bf16x8 kt8 = lds_read_tr8(kc + toff[0][dt] + cc * 16 * TL::kRow, kc + toff[1][dt] + cc * 16 * TL::kRow);
                    dq[dt] = mfma(kt8, db[h], dq[dt]);
                }
        }
        wait_vmem();
        __syncthreads();
    }

    unsigned short* DQ = (unsigned short*)a.dq + head + q_row * D;
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
        hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3(n_items), dim3(128), 0, stream, a);
    else
        hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3(n_items), dim3(128), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16_t64(int d, const BwdArgs& a, int n_items, hipStream_t stream)
{
    if (d == 64)
        hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3(n_items), dim3(128), 0, stream, a);
    else
        hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3(n_items), dim3(128), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sa
