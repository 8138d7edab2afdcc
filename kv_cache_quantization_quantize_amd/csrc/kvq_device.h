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

// One v_fmac_f32_dpp per value on 16 consecutive values v[i..i+15]; the
// leading s_nop covers the two wait states a DPP read needs after a VALU
// write of the same register.
#define KVQ_F(n, P) "v_fmac_f32_dpp %" #n ", %" #n ", %16 quad_perm:" P " row_mask:0xf bank_mask:0xf\n\t"
#define KVQ_FMAC16(P)                                                                          \
    asm("s_nop 1\n\t" KVQ_F(0, P) KVQ_F(1, P) KVQ_F(2, P) KVQ_F(3, P) KVQ_F(4, P) KVQ_F(5, P)   \
        KVQ_F(6, P) KVQ_F(7, P) KVQ_F(8, P) KVQ_F(9, P) KVQ_F(10, P) KVQ_F(11, P) KVQ_F(12, P)  \
        KVQ_F(13, P) KVQ_F(14, P) KVQ_F(15, P)                                                 \
        : "+v"(v[i]), "+v"(v[i + 1]), "+v"(v[i + 2]), "+v"(v[i + 3]), "+v"(v[i + 4]),          \
          "+v"(v[i + 5]), "+v"(v[i + 6]), "+v"(v[i + 7]), "+v"(v[i + 8]), "+v"(v[i + 9]),      \
          "+v"(v[i + 10]), "+v"(v[i + 11]), "+v"(v[i + 12]), "+v"(v[i + 13]),                  \
          "+v"(v[i + 14]), "+v"(v[i + 15])                                                     \
        : "v"(c))

// Butterfly on lane bit 0 of the quad (coordinate bit 3).  c = +1 on lanes
// with q&1 == 0, -1 otherwise.
template <int N>
__device__ __forceinline__ void bfly_quad1(float (&v)[N], float c)
{
    static_assert(N % 16 == 0, "values per lane must be a multiple of 16");
#pragma unroll
    for (int i = 0; i < N; i += 16) KVQ_FMAC16("[1,0,3,2]");
}

// Butterfly on lane bit 1 of the quad (coordinate bit 4).  c = +1 on lanes
// with q&2 == 0, -1 otherwise.
template <int N>
__device__ __forceinline__ void bfly_quad2(float (&v)[N], float c)
{
    static_assert(N % 16 == 0, "values per lane must be a multiple of 16");
#pragma unroll
    for (int i = 0; i < N; i += 16) KVQ_FMAC16("[2,3,0,1]");
}
#undef KVQ_FMAC16
#undef KVQ_F

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

// In-place max with the quad partner at lane xor 1 (X2 = false) or xor 2
// (X2 = true) of n <= 8 values, one asm block so that one s_nop serves all.
#define KVQ_M(n, P) "v_max_f32_dpp %" #n ", %" #n ", %" #n " quad_perm:" P " row_mask:0xf bank_mask:0xf\n\t"
template <bool X2, int N>
__device__ __forceinline__ void quad_max(float (&a)[N])
{
    static_assert(N == 1 || N == 2 || N == 4 || N == 8, "1, 2, 4 or 8 values");
    if constexpr (N == 1) {
        if constexpr (X2) asm("s_nop 1\n\t" KVQ_M(0, "[2,3,0,1]") : "+v"(a[0]));
        else asm("s_nop 1\n\t" KVQ_M(0, "[1,0,3,2]") : "+v"(a[0]));
    } else if constexpr (N == 2) {
        if constexpr (X2) asm("s_nop 1\n\t" KVQ_M(0, "[2,3,0,1]") KVQ_M(1, "[2,3,0,1]") : "+v"(a[0]), "+v"(a[1]));
        else asm("s_nop 1\n\t" KVQ_M(0, "[1,0,3,2]") KVQ_M(1, "[1,0,3,2]") : "+v"(a[0]), "+v"(a[1]));
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            if constexpr (X2)
                asm("s_nop 1\n\t" KVQ_M(0, "[2,3,0,1]") KVQ_M(1, "[2,3,0,1]") KVQ_M(2, "[2,3,0,1]")
                    KVQ_M(3, "[2,3,0,1]") : "+v"(a[i]), "+v"(a[i + 1]), "+v"(a[i + 2]), "+v"(a[i + 3]));
            else
                asm("s_nop 1\n\t" KVQ_M(0, "[1,0,3,2]") KVQ_M(1, "[1,0,3,2]") KVQ_M(2, "[1,0,3,2]")
                    KVQ_M(3, "[1,0,3,2]") : "+v"(a[i]), "+v"(a[i + 1]), "+v"(a[i + 2]), "+v"(a[i + 3]));
        }
    }
}
#undef KVQ_M

// 1/sqrt(D) and sqrt(D) for the supported head dims.
template <int D>
struct RsqrtD;
template <> struct RsqrtD<64> { static constexpr float v = 0.125f; };
template <> struct RsqrtD<128> { static constexpr float v = 0.0883883476483184405f; };
template <> struct RsqrtD<256> { static constexpr float v = 0.0625f; };
template <int D>
struct SqrtD;
template <> struct SqrtD<64> { static constexpr float v = 8.0f; };
template <> struct SqrtD<128> { static constexpr float v = 11.3137084989847604f; };
template <> struct SqrtD<256> { static constexpr float v = 16.0f; };

// Lane's register multipliers for the forward rotation (lane q of a quad,
// coordinates j*32 + q*8 + e): s_c * lambda_c / sqrt(D).
template <int D>
__device__ __forceinline__ void load_fwd_mult(const float* lam_lh, const int8_t* signs, int q,
                                              float (&m)[D / 4])
{
#pragma unroll
    for (int j = 0; j < D / 32; j++) {
        const int c0 = j * 32 + q * 8;
        const float4 l0 = *reinterpret_cast<const float4*>(lam_lh + c0);
        const float4 l1 = *reinterpret_cast<const float4*>(lam_lh + c0 + 4);
        const uint2 sg = *reinterpret_cast<const uint2*>(signs + c0);
        const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const uint32_t word = e < 4 ? sg.x : sg.y;
            const int sv = (int)(int8_t)((word >> (8 * (e & 3))) & 0xff);
            m[j * 8 + e] = (sv < 0 ? -lv[e] : lv[e]) * RsqrtD<D>::v;
        }
    }
}

// Inverse multipliers s_c / (lambda_c * sqrt(D)), times the lane's final
// transform sign.
template <int D>
__device__ __forceinline__ void load_inv_mult(const float* lam_lh, const int8_t* signs, int q,
                                              float lane_sign, float (&m)[D / 4])
{
#pragma unroll
    for (int j = 0; j < D / 32; j++) {
        const int c0 = j * 32 + q * 8;
        const float4 l0 = *reinterpret_cast<const float4*>(lam_lh + c0);
        const float4 l1 = *reinterpret_cast<const float4*>(lam_lh + c0 + 4);
        const uint2 sg = *reinterpret_cast<const uint2*>(signs + c0);
        const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const uint32_t word = e < 4 ? sg.x : sg.y;
            const int sv = (int)(int8_t)((word >> (8 * (e & 3))) & 0xff);
            const float sgn = (sv < 0) ? -lane_sign : lane_sign;
            m[j * 8 + e] = sgn / (lv[e] * SqrtD<D>::v);
        }
    }
}

// Forces v to be computed here: no instruction producing v may sink below
// this point, and no load or store may move across it (empty asm with a
// memory clobber).  Used to place the wait for an item's loads before the
// next item's loads are issued.
template <int N>
__device__ __forceinline__ void pin(float (&v)[N])
{
#pragma unroll
    for (int i = 0; i < N; i++) asm volatile("" : "+v"(v[i]) : : "memory");
}

// Wave-uniform value as an SGPR (the compiler cannot prove threadIdx.x >> 6
// uniform on its own).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

}  // namespace kvq
