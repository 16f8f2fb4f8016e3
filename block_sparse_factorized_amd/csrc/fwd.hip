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
// bf16 kernel (block 64, d in {64, 128}), one workgroup of two waves per
// (batch, head, query block); wave w owns query rows 32w..32w+31.
//   * The score tile is computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: lane (hh = lane/32, n = lane%32) then holds
//     16 keys of query n per 32-key tile, so the row max and row sum are
//     in-lane reductions plus one exchange with lane n+32.
//   * The output is accumulated transposed too, O^T = V^T P^T, so the
//     softmax rescale factor of query n is in the lane that owns its output
//     column.  P^T leaves the score accumulators already in the B-operand
//     layout, with the keys of each 16-key chunk taken in the order
//     c*16 + {0-3, 8-11} (lanes 0-31) and {4-7, 12-15} (lanes 32-63); V is
//     stored transposed in LDS with bits 2 and 3 of the key index swapped so
//     that each lane reads its 8 keys with one 16-byte LDS load.
//   * K and V tiles go global -> registers -> LDS with 16-byte loads, double
//     buffered: the next tile's loads are in flight while the matrix cores
//     work on the current one, one barrier per tile.
//
// f32 kernel (block 16, d 64), one wave per (batch, head, query block), the
// same structure on v_mfma_f32_16x16x4_f32.
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
    unsigned short ua = __builtin_bit_cast(unsigned short, a);
    unsigned short ub = __builtin_bit_cast(unsigned short, b);
    return (unsigned)ua | ((unsigned)ub << 16);
}

template <int D>
__global__ __launch_bounds__(128) void fwd_bf16_t64_kernel(const FwdArgs a)
{
    constexpr int T = 64;
    constexpr int KP = D + 8;  // K tile row pitch (elements)
    constexpr int VP = T + 8;  // V^T tile row pitch (elements)
    constexpr int KCH = T * D / 8 / 128;          // 16-byte K chunks per thread
    constexpr int VBL = (T / 4) * (D / 8) / 128;  // 4x8 V blocks per thread
    __shared__ __attribute__((aligned(16))) unsigned short ks[2][T * KP];
    __shared__ __attribute__((aligned(16))) unsigned short vts[2][D * VP];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n32 = lane & 31, hh = lane >> 5;
    const Item item = a.items[blockIdx.x];
    const int bh = item.bh, qb = item.blk;
    const DevLayout L = a.heads.lay[a.heads.head_lay[bh % a.H]];
    const int64_t head = (int64_t)bh * a.n * D;
    const unsigned short* Q = (const unsigned short*)a.q + head;
    const unsigned short* K = (const unsigned short*)a.k + head;
    const unsigned short* V = (const unsigned short*)a.v + head;
    const int q_local = 32 * w + n32;
    const int64_t q_row = (int64_t)qb * T + q_local;

    bf16x8 qop[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qop[c] = *(const bf16x8*)(Q + q_row * D + 16 * c + 8 * hh);

    const int p0 = L.row_ptr[qb];
    const int nblk = L.row_ptr[qb + 1] - p0;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float c2 = a.scale_log2;

    u32x4 kreg[KCH];
    u32x4 vreg[VBL][4];
    auto gload = [&](int kb) {
        const unsigned short* Kt = K + (int64_t)kb * T * D;
        const unsigned short* Vt = V + (int64_t)kb * T * D;
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            int idx = tid + 128 * u, row = idx / (D / 8), c8 = idx % (D / 8);
            kreg[u] = *(const u32x4*)(Kt + row * D + c8 * 8);
        }
#pragma unroll
        for (int b = 0; b < VBL; ++b) {
            int idx = tid + 128 * b, kg = idx / (D / 8), dc = idx % (D / 8);
#pragma unroll
            for (int r = 0; r < 4; ++r) vreg[b][r] = *(const u32x4*)(Vt + (4 * kg + r) * D + dc * 8);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            int idx = tid + 128 * u, row = idx / (D / 8), c8 = idx % (D / 8);
            *(u32x4*)&ks[buf][row * KP + c8 * 8] = kreg[u];
        }
#pragma unroll
        for (int b = 0; b < VBL; ++b) {
            int idx = tid + 128 * b, kg = idx / (D / 8), dc = idx % (D / 8);
            int pos = swap_bits23(4 * kg);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u32x2 lo, hi;
                lo[0] = pack_lo(vreg[b][0][e], vreg[b][1][e]);
                lo[1] = pack_lo(vreg[b][2][e], vreg[b][3][e]);
                hi[0] = pack_hi(vreg[b][0][e], vreg[b][1][e]);
                hi[1] = pack_hi(vreg[b][2][e], vreg[b][3][e]);
                *(u32x2*)&vts[buf][(dc * 8 + 2 * e) * VP + pos] = lo;
                *(u32x2*)&vts[buf][(dc * 8 + 2 * e + 1) * VP + pos] = hi;
            }
        }
    };

    if (nblk > 0) {
        gload(L.col_idx[p0]);
        sstore(0);
    }
    __syncthreads();

    for (int t = 0; t < nblk; ++t) {
        const int buf = t & 1;
        if (t + 1 < nblk) gload(L.col_idx[p0 + t + 1]);
        const int mid = L.mask_id[p0 + t];

        // S^T = K Q^T for keys 0-31 (kt = 0) and 32-63 (kt = 1).
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                bf16x8 kop = *(const bf16x8*)&ks[buf][(32 * kt + n32) * KP + 16 * c + 8 * hh];
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[c], s[kt], 0, 0, 0);
            }
        }
        // Register i of tile kt holds key 32*kt + 8*(i/4) + 4*hh + i%4.
        if (mid >= 0) {
            uint64_t word = L.masks[(int64_t)mid * (T * T / 64) + q_local] >> (4 * hh);
            unsigned wl = (unsigned)word, wh = (unsigned)(word >> 32);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                unsigned bits = kt ? wh : wl;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (!((bits >> (8 * (i / 4) + (i % 4))) & 1u)) s[kt][i] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
        const float mc = m_use * c2;
        float lsum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float p = __builtin_amdgcn_exp2f(fmaf(s[kt][i], c2, -mc));
                s[kt][i] = p;
                lsum += p;
            }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;

        // P^T as the B operand: chunk cc holds registers 8*(cc%2)..+7 of tile cc/2.
        bf16x8 pb[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            u32x4 u;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                u[e] = bf16_pair(s[cc / 2][8 * (cc % 2) + 2 * e], s[cc / 2][8 * (cc % 2) + 2 * e + 1]);
            pb[cc] = __builtin_bit_cast(bf16x8, u);
        }
        // O^T += V^T P^T.
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                bf16x8 vop = *(const bf16x8*)&vts[buf][(32 * dt + n32) * VP + 16 * cc + 8 * hh];
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[cc], oacc[dt], 0, 0, 0);
            }

        if (t + 1 < nblk) sstore(buf ^ 1);
        __syncthreads();
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    unsigned short* O = (unsigned short*)a.o + head + q_row * D;
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
    if (hh == 0)
        a.lse[(int64_t)bh * a.n + q_row] = l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY;
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

hipError_t launch_fwd_bf16_t64(int d, const FwdArgs& a, int n_items, hipStream_t stream)
{
    if (d == 64)
        hipLaunchKernelGGL(fwd_bf16_t64_kernel<64>, dim3(n_items), dim3(128), 0, stream, a);
    else
        hipLaunchKernelGGL(fwd_bf16_t64_kernel<128>, dim3(n_items), dim3(128), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fwd_f32_t16(int d, const FwdArgs& a, int n_items, hipStream_t stream)
{
    (void)d;
    hipLaunchKernelGGL(fwd_f32_t16_d64_kernel, dim3(n_items), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sa
