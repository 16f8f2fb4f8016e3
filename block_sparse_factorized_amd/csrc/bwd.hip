// bwd.hip -- recompute-style backward of block-sparse causal attention, gfx950.
//
// "[논문 리뷰] Generating Long Sequences with Sparse Transformers" (nubint.ai),
// ABSTRACT item (b) and "제안 방법"; pcnews.ru, "Глубокое внимание": the
// attention matrix is recomputed during backpropagation instead of stored.
// Only O and lse come from the forward pass.  With c = scale:
//     P_ij  = exp(c s_ij - lse_i)        (recomputed per block)
//     D_i   = sum_t dO_it O_it           (delta kernel)
//     dP_ij = dO_i . v_j,   dS_ij = P_ij (dP_ij - D_i)
//     dV_j  = sum_i P_ij dO_i,  dK_j = c sum_i dS_ij q_i   (dK/dV kernel,
//             one workgroup per key block, walking its query blocks)
//     dQ_i  = c sum_j dS_ij k_j                             (dQ kernel, one
//             workgroup per query block, walking its key blocks)
// Both kernels write their outputs once, with no atomics, so results are
// deterministic.
//
// Operand layouts follow the forward kernel: 32x32x16 bf16 MFMA tiles, the
// key (or query) index of each 16-long reduction chunk taken in the order
// {0-3, 8-11} for lanes 0-31 and {4-7, 12-15} for lanes 32-63, and tiles
// that must be read along the sequence axis stored transposed in LDS with
// bits 2 and 3 of the sequence index swapped.
#include <hip/hip_runtime.h>

#include "kernel_args.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline int swap_bits23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }
__device__ inline unsigned pack_lo(unsigned a, unsigned b) { return (a & 0xffffu) | (b << 16); }
__device__ inline unsigned pack_hi(unsigned a, unsigned b) { return (a >> 16) | (b & 0xffff0000u); }

__device__ inline unsigned bf16_pair(float x, float y)
{
    __bf16 a = (__bf16)x, b = (__bf16)y;
    return (unsigned)__builtin_bit_cast(unsigned short, a) | ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
}

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

// Pack registers 8*(cc%2)..+7 of x[cc/2] into a bf16 operand.
__device__ inline bf16x8 pack_chunk(const f32x16* x, int cc)
{
    u32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = bf16_pair(x[cc / 2][8 * (cc % 2) + 2 * e], x[cc / 2][8 * (cc % 2) + 2 * e + 1]);
    return __builtin_bit_cast(bf16x8, u);
}

// A 64 x D bf16 tile staged by 128 threads as 4x8 blocks: each thread loads
// 4 rows x 8 columns and can store them row-major and/or transposed.
template <int D>
struct TileStager {
    static constexpr int NB = (64 / 4) * (D / 8) / 128;  // blocks per thread
    u32x4 r[NB][4];
    __device__ inline void load(const unsigned short* src, int tid)
    {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            int idx = tid + 128 * b, kg = idx / (D / 8), dc = idx % (D / 8);
#pragma unroll
            for (int a = 0; a < 4; ++a) r[b][a] = *(const u32x4*)(src + (4 * kg + a) * D + dc * 8);
        }
    }
    // Row-major store, row pitch P elements.
    template <int P>
    __device__ inline void store_rows(unsigned short* dst, int tid) const
    {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            int idx = tid + 128 * b, kg = idx / (D / 8), dc = idx % (D / 8);
#pragma unroll
            for (int a = 0; a < 4; ++a) *(u32x4*)&dst[(4 * kg + a) * P + dc * 8] = r[b][a];
        }
    }
    // Transposed store: dst[col][swap_bits23(row)], row pitch P elements.
    template <int P>
    __device__ inline void store_cols(unsigned short* dst, int tid) const
    {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            int idx = tid + 128 * b, kg = idx / (D / 8), dc = idx % (D / 8);
            int pos = swap_bits23(4 * kg);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u32x2 lo, hi;
                lo[0] = pack_lo(r[b][0][e], r[b][1][e]);
                lo[1] = pack_lo(r[b][2][e], r[b][3][e]);
                hi[0] = pack_hi(r[b][0][e], r[b][1][e]);
                hi[1] = pack_hi(r[b][2][e], r[b][3][e]);
                *(u32x2*)&dst[(dc * 8 + 2 * e) * P + pos] = lo;
                *(u32x2*)&dst[(dc * 8 + 2 * e + 1) * P + pos] = hi;
            }
        }
    }
};

// ---------------------------------------------------------------------------
// D_i = sum_t dO_it O_it, D/8 threads per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const BwdArgs a, int64_t rows)
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
    if (row < rows && part == 0) a.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = key block (bh, kb), wave w owns keys 32w..32w+31 and
// walks the query blocks that list kb.  Lane (hh, n) holds key 32w + n.
//   S   = Q K^T      C[q][key]   A = Q (LDS, rows)    B = K^T (registers)
//   dP  = dO V^T     C[q][key]   A = dO (LDS, rows)   B = V^T (registers)
//   dV^T += dO^T P   C[d][key]   A = dO^T (LDS, cols) B = P   (registers)
//   dK^T += Q^T dS   C[d][key]   A = Q^T (LDS, cols)  B = dS  (registers)
template <int D, int NBUF>
__global__ __launch_bounds__(128) void bwd_dkdv_kernel(const BwdArgs a)
{
    constexpr int T = 64;
    constexpr int RP = D + 8;  // row-major pitch
    constexpr int CP = T + 8;  // transposed pitch
    struct Buf {
        unsigned short q[T * RP];
        unsigned short qt[D * CP];
        unsigned short d_o[T * RP];
        unsigned short dot[D * CP];
        float nl2[T];    // -lse * log2(e)  (-inf for an empty row)
        float delta[T];  // D_i
    };
    __shared__ __attribute__((aligned(16))) Buf sm[NBUF];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n32 = lane & 31, hh = lane >> 5;
    const Item item = a.items[blockIdx.x];
    const int bh = item.bh, kb = item.blk;
    const DevLayout L = a.heads.lay[a.heads.head_lay[bh % a.H]];
    const int64_t head = (int64_t)bh * a.n * D;
    const unsigned short* Q = (const unsigned short*)a.q + head;
    const unsigned short* K = (const unsigned short*)a.k + head;
    const unsigned short* V = (const unsigned short*)a.v + head;
    const unsigned short* dO = (const unsigned short*)a.dout + head;
    const float* lse = a.lse + (int64_t)bh * a.n;
    const float* dl = a.delta + (int64_t)bh * a.n;
    const int k_local = 32 * w + n32;
    const int64_t k_row = (int64_t)kb * T + k_local;

    bf16x8 kop[D / 16], vop[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        kop[c] = *(const bf16x8*)(K + k_row * D + 16 * c + 8 * hh);
        vop[c] = *(const bf16x8*)(V + k_row * D + 16 * c + 8 * hh);
    }
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        zero(dk[dt]);
        zero(dv[dt]);
    }

    const int p0 = L.col_ptr[kb];
    const int nblk = L.col_ptr[kb + 1] - p0;
    const float c2 = a.scale_log2;

    TileStager<D> sq, sdo;
    float pre_l = 0.f, pre_d = 0.f;
    auto gload = [&](int qb) {
        sq.load(Q + (int64_t)qb * T * D, tid);
        sdo.load(dO + (int64_t)qb * T * D, tid);
        if (tid < T) {
            pre_l = lse[(int64_t)qb * T + tid];
            pre_d = dl[(int64_t)qb * T + tid];
        }
    };
    auto sstore = [&](Buf& b) {
        sq.template store_rows<RP>(b.q, tid);
        sq.template store_cols<CP>(b.qt, tid);
        sdo.template store_rows<RP>(b.d_o, tid);
        sdo.template store_cols<CP>(b.dot, tid);
        if (tid < T) {
            b.nl2[tid] = pre_l == -INFINITY ? -INFINITY : -pre_l * kLog2e;
            b.delta[tid] = pre_d;
        }
    };

    if (nblk > 0) {
        gload(L.row_idx[p0]);
        sstore(sm[0]);
    }
    __syncthreads();

    for (int t = 0; t < nblk; ++t) {
        Buf& b = sm[NBUF == 2 ? (t & 1) : 0];
        if (NBUF == 2 && t + 1 < nblk) gload(L.row_idx[p0 + t + 1]);
        const int mid = L.col_mask[p0 + t];

        f32x16 s[2], dp[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            zero(s[qt]);
            zero(dp[qt]);
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                bf16x8 qa = *(const bf16x8*)&b.q[(32 * qt + n32) * RP + 16 * c + 8 * hh];
                bf16x8 da = *(const bf16x8*)&b.d_o[(32 * qt + n32) * RP + 16 * c + 8 * hh];
                s[qt] = mfma(qa, kop[c], s[qt]);
                dp[qt] = mfma(da, vop[c], dp[qt]);
            }
        }
        // Register i of tile qt: query 32*qt + 8*(i/4) + 4*hh + i%4, key k_local.
        unsigned mlo = ~0u, mhi = ~0u;
        if (mid >= 0) {
            // Column k_local of the block's mask, as 64 query bits.
            uint64_t word = L.masks_t[(int64_t)mid * (T * T / 64) + k_local] >> (4 * hh);
            mlo = (unsigned)word;
            mhi = (unsigned)(word >> 32);
        }
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const unsigned bits = qt ? mhi : mlo;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 nl = *(const f32x4*)&b.nl2[32 * qt + 8 * g + 4 * hh];
                const f32x4 dd = *(const f32x4*)&b.delta[32 * qt + 8 * g + 4 * hh];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * g + e;
                    float p = __builtin_amdgcn_exp2f(fmaf(s[qt][i], c2, nl[e]));
                    if (!((bits >> (8 * g + e)) & 1u)) p = 0.f;
                    s[qt][i] = p;
                    dp[qt][i] = p * (dp[qt][i] - dd[e]);
                }
            }
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const bf16x8 pb = pack_chunk(s, cc);
            const bf16x8 db = pack_chunk(dp, cc);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                bf16x8 oa = *(const bf16x8*)&b.dot[(32 * dt + n32) * CP + 16 * cc + 8 * hh];
                bf16x8 qa = *(const bf16x8*)&b.qt[(32 * dt + n32) * CP + 16 * cc + 8 * hh];
                dv[dt] = mfma(oa, pb, dv[dt]);
                dk[dt] = mfma(qa, db, dk[dt]);
            }
        }

        if (NBUF == 2) {
            if (t + 1 < nblk) sstore(sm[(t + 1) & 1]);
            __syncthreads();
        } else if (t + 1 < nblk) {
            gload(L.row_idx[p0 + t + 1]);
            __syncthreads();
            sstore(sm[0]);
            __syncthreads();
        }
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
//   S^T  = K Q^T      C[key][q]   A = K (LDS, rows)    B = Q^T (registers)
//   dP^T = V dO^T     C[key][q]   A = V (LDS, rows)    B = dO^T (registers)
//   dQ^T += K^T dS^T  C[d][q]     A = K^T (LDS, cols)  B = dS^T (registers)
template <int D, int NBUF>
__global__ __launch_bounds__(128) void bwd_dq_kernel(const BwdArgs a)
{
    constexpr int T = 64;
    constexpr int RP = D + 8;
    constexpr int CP = T + 8;
    struct Buf {
        unsigned short k[T * RP];
        unsigned short kt[D * CP];
        unsigned short v[T * RP];
    };
    __shared__ __attribute__((aligned(16))) Buf sm[NBUF];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n32 = lane & 31, hh = lane >> 5;
    const Item item = a.items[blockIdx.x];
    const int bh = item.bh, qb = item.blk;
    const DevLayout L = a.heads.lay[a.heads.head_lay[bh % a.H]];
    const int64_t head = (int64_t)bh * a.n * D;
    const unsigned short* Q = (const unsigned short*)a.q + head;
    const unsigned short* K = (const unsigned short*)a.k + head;
    const unsigned short* V = (const unsigned short*)a.v + head;
    const unsigned short* dO = (const unsigned short*)a.dout + head;
    const int q_local = 32 * w + n32;
    const int64_t q_row = (int64_t)qb * T + q_local;

    bf16x8 qop[D / 16], dop[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        qop[c] = *(const bf16x8*)(Q + q_row * D + 16 * c + 8 * hh);
        dop[c] = *(const bf16x8*)(dO + q_row * D + 16 * c + 8 * hh);
    }
    const float lse_i = a.lse[(int64_t)bh * a.n + q_row];
    const float nl2 = lse_i == -INFINITY ? -INFINITY : -lse_i * kLog2e;
    const float d_i = a.delta[(int64_t)bh * a.n + q_row];
    f32x16 dq[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) zero(dq[dt]);

    const int p0 = L.row_ptr[qb];
    const int nblk = L.row_ptr[qb + 1] - p0;
    const float c2 = a.scale_log2;

    TileStager<D> sk, sv;
    auto gload = [&](int kb) {
        sk.load(K + (int64_t)kb * T * D, tid);
        sv.load(V + (int64_t)kb * T * D, tid);
    };
    auto sstore = [&](Buf& b) {
        sk.template store_rows<RP>(b.k, tid);
        sk.template store_cols<CP>(b.kt, tid);
        sv.template store_rows<RP>(b.v, tid);
    };

    if (nblk > 0) {
        gload(L.col_idx[p0]);
        sstore(sm[0]);
    }
    __syncthreads();

    for (int t = 0; t < nblk; ++t) {
        Buf& b = sm[NBUF == 2 ? (t & 1) : 0];
        if (NBUF == 2 && t + 1 < nblk) gload(L.col_idx[p0 + t + 1]);
        const int mid = L.mask_id[p0 + t];

        f32x16 s[2], dp[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            zero(s[kt]);
            zero(dp[kt]);
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                bf16x8 ka = *(const bf16x8*)&b.k[(32 * kt + n32) * RP + 16 * c + 8 * hh];
                bf16x8 va = *(const bf16x8*)&b.v[(32 * kt + n32) * RP + 16 * c + 8 * hh];
                s[kt] = mfma(ka, qop[c], s[kt]);
                dp[kt] = mfma(va, dop[c], dp[kt]);
            }
        }
        unsigned mlo = ~0u, mhi = ~0u;
        if (mid >= 0) {
            uint64_t word = L.masks[(int64_t)mid * (T * T / 64) + q_local] >> (4 * hh);
            mlo = (unsigned)word;
            mhi = (unsigned)(word >> 32);
        }
        // Register i of tile kt: key 32*kt + 8*(i/4) + 4*hh + i%4, query q_local.
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const unsigned bits = kt ? mhi : mlo;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float p = __builtin_amdgcn_exp2f(fmaf(s[kt][i], c2, nl2));
                if (!((bits >> (8 * (i / 4) + (i % 4))) & 1u)) p = 0.f;
                dp[kt][i] = p * (dp[kt][i] - d_i);
            }
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const bf16x8 db = pack_chunk(dp, cc);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                bf16x8 ka = *(const bf16x8*)&b.kt[(32 * dt + n32) * CP + 16 * cc + 8 * hh];
                dq[dt] = mfma(ka, db, dq[dt]);
            }
        }

        if (NBUF == 2) {
            if (t + 1 < nblk) sstore(sm[(t + 1) & 1]);
            __syncthreads();
        } else if (t + 1 < nblk) {
            gload(L.col_idx[p0 + t + 1]);
            __syncthreads();
            sstore(sm[0]);
            __syncthreads();
        }
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

hipError_t launch_bwd_delta_bf16(int d, const BwdArgs& a, int64_t rows, hipStream_t stream)
{
    const int64_t threads = rows * (d / 8);
    const unsigned grid = (unsigned)((threads + 255) / 256);
    if (d == 64)
        hipLaunchKernelGGL(bwd_delta_kernel<64>, dim3(grid), dim3(256), 0, stream, a, rows);
    else
        hipLaunchKernelGGL(bwd_delta_kernel<128>, dim3(grid), dim3(256), 0, stream, a, rows);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16_t64(int d, const BwdArgs& a, int n_items, hipStream_t stream)
{
    if (d == 64)
        hipLaunchKernelGGL((bwd_dkdv_kernel<64, 2>), dim3(n_items), dim3(128), 0, stream, a);
    else
        hipLaunchKernelGGL((bwd_dkdv_kernel<128, 1>), dim3(n_items), dim3(128), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16_t64(int d, const BwdArgs& a, int n_items, hipStream_t stream)
{
    if (d == 64)
        hipLaunchKernelGGL((bwd_dq_kernel<64, 2>), dim3(n_items), dim3(128), 0, stream, a);
    else
        hipLaunchKernelGGL((bwd_dq_kernel<128, 1>), dim3(n_items), dim3(128), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sa
