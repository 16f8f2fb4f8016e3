// tiles.h -- device helpers shared by the gfx950 kernels of libsa: vector
// types, bf16 packing, lane-pair exchanges, transposing LDS reads and the
// swizzled 64-row LDS tile filled by direct global-to-LDS loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>


namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const uint64_t const_u64;
typedef __attribute__((address_space(4))) const int32_t const_i32;

// Read-only, wave-uniform data read through the constant address space, so
// that it becomes a scalar load: scalar loads are counted by lgkmcnt, and a
// wait for them does not also wait for tiles in flight to LDS (vmcnt).
// The value is read as 32-bit words (the HIP vector types' copy constructors
// would take a generic reference and turn it back into a vector load).
template <class T>
__device__ static inline T ld_uniform(const T* p)
{
    static_assert(sizeof(T) % 4 == 0, "ld_uniform reads whole 32-bit words");
    int32_t w[sizeof(T) / 4];
#pragma unroll
    for (unsigned i = 0; i < sizeof(T) / 4; ++i) w[i] = ((const_i32*)p)[i];
    T r;
    __builtin_memcpy(&r, w, sizeof(T));
    return r;
}

__device__ static inline unsigned bf16_pair(float x, float y)
{
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x, y}, bf16x2));
}

// Registers first..first+7 of x as eight bf16 (round to nearest even).
__device__ static inline bf16x8 pack8(const f32x16& x, int first)
{
    u32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = bf16_pair(x[first + 2 * e], x[first + 2 * e + 1]);
    return __builtin_bit_cast(bf16x8, u);
}

// Max of x over lanes n and n+32 (lane pairs that hold the same query row).
__device__ static inline float half_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The value lane n+32 (or n-32) holds.
__device__ static inline float swap_halves(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((__lane_id() < 32) ? r[1] : r[0]);
}

__device__ static inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// s_waitcnt vmcnt(N), other counters not waited on (gfx9 encoding).
template <int N>
__device__ static inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Global address of byte offset off from a wave-uniform base, in the form
// the loads encode as base (SGPRs) + 32-bit offset (VGPR).  The empty asm
// keeps the compiler from hoisting the offset's 64-bit extension out of the
// loop, which would turn every load's address into a 64-bit vector add.
__device__ static inline const void* sgpr_base_plus(const void* base, uint32_t off)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the constraint names a GPU register class
    asm volatile("" : "+v"(off));
#endif
    return (const unsigned char*)base + off;
}

// x, hidden from the optimiser: arithmetic on the result stays where it is
// written instead of being hoisted out of a loop (and holding registers).
__device__ static inline int opaque(int x)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the constraint names a GPU register class
    asm volatile("" : "+v"(x));
#endif
    return x;
}

// Two transposing 8-byte LDS reads (ds_read_b64_tr_b16) forming one 8 x bf16 operand.
__device__ static inline bf16x8 lds_read_tr8(const unsigned char* p0, const unsigned char* p1)
{
    i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(lds_void*)p0);
    i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(lds_void*)p1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A 64 x D bf16 tile in LDS: rows unpadded (2*D bytes), each row's 16-byte
// chunks stored at position chunk ^ swz(row), which spreads the rows that
// one MFMA operand read touches over all LDS banks.  Filled by direct
// global-to-LDS loads shared by the NW waves of a workgroup: load u of wave w
// writes 1 KB of consecutive slots, lane l the 16 bytes at slot l.
template <int D, int NW = 2>
struct Tile64 {
    static constexpr int kRow = 2 * D;
    static constexpr int kBytes = 64 * kRow;
    static constexpr int kLoads = kBytes / (1024 * NW);  // direct-to-LDS loads per wave
    // Row swizzle, for the 64-bank LDS (256 bytes per bank cycle): with d = 64
    // a row is half a bank cycle, so 16 rows of one chunk (a 16-byte MFMA
    // operand read, 16 lanes per cycle) need distinct positions within each
    // row parity, and the 4-row x 32-byte footprints of a transposing read
    // (32 lanes per cycle) need rows r and r+2 in different aligned 4-chunk
    // groups: the bit-reversed (r/2) mod 8 gives both.  With d = 128 a row is
    // a full bank cycle: 16 consecutive rows need distinct positions and any
    // 4 consecutive rows distinct aligned 4-chunk groups.  Both depend only on
    // r mod 16, so tile rows 16 apart share offsets.
    __device__ static inline int swz(int r)
    {
        if (D == 64) return ((r >> 1) & 1) << 2 | ((r >> 2) & 1) << 1 | ((r >> 3) & 1);
        return ((r & 3) << 2) | ((r >> 2) & 3);
    }
    __device__ static inline int off(int r, int chunk) { return r * kRow + ((chunk ^ swz(r)) << 4); }
    __device__ static inline int load_dst(int u, int w) { return (NW * u + w) * 1024; }
    // Element offset in the global tile of the 16 bytes lane `lane` loads in load u of wave w.
    __device__ static inline int load_src(int u, int w, int lane)
    {
        return load_row(u, w, lane) * D + load_col(u, w, lane);
    }
    // Its tile row and its first element in that row.
    __device__ static inline int load_row(int u, int w, int lane) { return (load_dst(u, w) + 16 * lane) / kRow; }
    __device__ static inline int load_col(int u, int w, int lane)
    {
        const int byte = load_dst(u, w) + 16 * lane;
        const int r = byte / kRow, pos = (byte % kRow) >> 4;
        return (pos ^ swz(r)) << 3;
    }
    // Byte offset of this lane's half (j4 = 0, 1) of a transposing read that
    // yields the 32x32x16 A operand [d = 32*dt + lane%32][sequence index
    // 8*(lane/32) + j] of a 16-row chunk at row 0: lane a of each 16-lane
    // group addresses row 8*j4 + 4*(group/2) + a/4, columns 32*dt +
    // 16*(group%2) + 4*(a%4) .. +3, and receives one column of 4 rows.  Add
    // 16*kRow per further chunk (the swizzle does not depend on it).
    __device__ static inline int tr_off(int lane, int j4, int dt)
    {
        const int g = lane >> 4, al = lane & 15;
        const int row = 8 * j4 + 4 * (g >> 1) + (al >> 2);
        const int col = 32 * dt + 16 * (g & 1) + 4 * (al & 3);
        return off(row, col >> 3) + ((col & 4) << 1);
    }
};


}  // namespace sa
