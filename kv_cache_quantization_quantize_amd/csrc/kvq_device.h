// kvq_device.h -- device building blocks shared by the gfx950 kernels: the
// register-resident Walsh-Hadamard transform and quad reductions.
//
// Lane layout.  A head vector of D fp16 values is held by the 4 lanes of one
// quad (lanes 4s..4s+3 of a wavefront hold vector s, 16 vectors per wave).
// Lane q of the quad holds the coordinates
//     c = j*32 + q*8 + e,   j in [0, D/32), e in [0, 8)
// in register r = j*8 + e.  Each (j, q) chunk of 8 coordinates is one
// 16-byte global load, so a quad reads 64 contiguous bytes per load and a
// wave 16 such runs.  Coordinate bits 0-2 (e) and 5.. (j) are register bits;
// bits 3-4 (q) are lane bits.
//
// Walsh-Hadamard transform (Sylvester order: H[i][j] = (-1)^popcount(i&j),
// the butterfly sends the bit-0 element a and bit-1 element b to a+b at bit 0
// and a-b at bit 1 -- the "fast Walsh-Hadamard" of the VecInfer blog, "What
// VecInfer does").  The log2(D) butterfly stages act on different index bits
// and commute, so they may run in any order: register-bit stages are plain
// add/sub pairs; the two lane-bit stages use one v_fmac_f32 with a DPP
// quad_perm source per value:
//     v <- partner * c + v
// With per-lane sign bookkeeping (each lane stores sigma * true value, sigma
// in {+1,-1} the same for all its registers), c = +1 on the bit-0 lane and
// c = -1 on the bit-1 lane realises the butterfly for both lanes in one
// instruction: the bit-0 lane gets sigma*(a+b), the bit-1 lane gets
// (-sigma)*(a-b).  Starting from sigma = +1, after both lane stages
// sigma(q) = (-1)^popcount(q); consumers fold that sign into their per-lane
// multipliers (abs-max does not see it and round-half-even is odd-symmetric).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float lo_half(uint32_t w) { return (float)__builtin_bit_cast(half2_t, w).x; }
__device__ __forceinline__ float hi_half(uint32_t w) { return (float)__builtin_bit_cast(half2_t, w).y; }

// Round two floats to fp16 (round to nearest even) and pack them, the first
// in the low half.
__device__ __forceinline__ uint32_t pack_half2(float a, float b)
{
    half2_t h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// Butterfly on register bit B of every lane's N values.
template <int B, int N>
__device__ __forceinline__ void bfly_reg(float (&v)[N])
{
#pragma unroll
    for (int r = 0; r < N; r++) {
        if (r & (1 << B)) continue;
        const float a = v[r], b = v[r | (1 << B)];
        v[r] = a + b;
        v[r | (1 << B)] = a - b;
    }
}

// One v_fmac_f32_dpp per value on 8 consecutive values; the leading s_nop
// covers the two wait states a DPP read needs after a VALU write.
#define KVQ_FMAC8(PERM)                                                             \
    asm("s_nop 1\n\t"                                                               \
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t" \
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t" \
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t" \
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t" \
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t" \
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t" \
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t" \
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf"     \
        : "+v"(v[i]), "+v"(v[i + 1]), "+v"(v[i + 2]), "+v"(v[i + 3]),               \
          "+v"(v[i + 4]), "+v"(v[i + 5]), "+v"(v[i + 6]), "+v"(v[i + 7])             \
        : "v"(c))

// Butterfly on lane bit 0 of the quad (coordinate bit 3).  c = +1 on lanes
// with q&1 == 0, -1 otherwise.
template <int N>
__device__ __forceinline__ void bfly_quad1(float (&v)[N], float c)
{
    static_assert(N % 8 == 0, "values per lane must be a multiple of 8");
#pragma unroll
    for (int i = 0; i < N; i += 8) KVQ_FMAC8("[1,0,3,2]");
}

// Butterfly on lane bit 1 of the quad (coordinate bit 4).  c = +1 on lanes
// with q&2 == 0, -1 otherwise.
template <int N>
__device__ __forceinline__ void bfly_quad2(float (&v)[N], float c)
{
    static_assert(N % 8 == 0, "values per lane must be a multiple of 8");
#pragma unroll
    for (int i = 0; i < N; i += 8) KVQ_FMAC8("[2,3,0,1]");
}
#undef KVQ_FMAC8

// Full in-register transform of N = 8*NJ values per lane (both lane stages
// included).  Stage "register bit 0" is expected to have been applied by the
// caller (it is fused with the load/scale step).
template <int N>
__device__ __forceinline__ void fwht_rest(float (&v)[N], float c1, float c2)
{
    bfly_reg<1>(v);
    bfly_reg<2>(v);
    if constexpr (N >= 16) bfly_reg<3>(v);
    if constexpr (N >= 32) bfly_reg<4>(v);
    if constexpr (N >= 64) bfly_reg<5>(v);
    bfly_quad1(v, c1);
    bfly_quad2(v, c2);
}

// max over the quad partner at lane xor 1 (and xor 2) for 1..4 values.
__device__ __forceinline__ void quad_max_x1(float& a)
{
    asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "+v"(a));
}
__device__ __forceinline__ void quad_max_x2(float& a)
{
    asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
        : "+v"(a));
}

// Wave-uniform value as an SGPR (the compiler cannot prove threadIdx.x >> 6
// uniform on its own).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace kvq
