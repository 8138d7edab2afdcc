// kvq_int4.hip -- fused rotate + int4 quantize and its mirror dequantize for
// gfx950 (MI355X).
//
// Quantize, per fp16 head vector x of one (layer l, head h):
//   1. y = D^-1/2 * Hd * diag(s) * diag(lambda[l,h]) * x   (fp32, registers)
//   2. per group of G consecutive rotated coordinates: amax, fp16 scale
//      = rne(amax / 7), code = rne(y / scale) in [-7, 7] (0 if scale == 0)
//   3. two codes per byte (element 2k in the low nibble), fp16 scales
// This is the step list of the fused kernel in the gist.science explanation
// of arXiv 2605.05699 ("Methodologie" s.2: signs in registers, transform,
// lambda, group abs-max, signed int4 rounding, nibble pack), with the
// Walsh-Hadamard transform the abstract of "When Quantization Is Free" finds
// equivalent to the FFT, and lambda applied before the rotation as in the
// VecInfer blog ("What VecInfer does": smooth scale, then rotation).
// Dequantize is the mirror ("The kernel toggle": dequantize, inverse
// transform, unscale).
//
// Work decomposition.  An item is 16 consecutive tokens of one (l, h) pair;
// one wavefront owns a run of consecutive items, so lambda's per-lane
// multipliers stay in registers while (l, h) is unchanged, and the next
// item's loads are issued before the current item is computed.  The kernel
// is HBM-bound: per vector it moves 2D + D/2 + 2D/G bytes and does about
// 2.9 VALU operations per coordinate.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr float kMagic8 = 12582920.0f;  // 1.5 * 2^23 + 8: fma(y, 1/scale, kMagic8)
                                        // leaves 8 + rne(y/scale) in the low bits
constexpr float kInv7 = 0.142857142857142857f;

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

// Per-item coordinates shared by both kernels.
struct ItemPos {
    int lh, tile;
};

__device__ __forceinline__ ItemPos item_pos(int item, int tiles_per_lh)
{
    ItemPos p;
    p.lh = item / tiles_per_lh;
    p.tile = item - p.lh * tiles_per_lh;
    return p;
}

// Lane's register multipliers for the forward rotation: s_c * lambda_c / sqrt(D).
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

// Byte k of the result = low byte of a_k (k = 0..3).
__device__ __forceinline__ uint32_t gather_low_bytes(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3)
{
    const uint32_t lo = __builtin_amdgcn_perm(a1, a0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(a3, a2, 0x04000c0cu);
    return lo | hi;
}

}  // namespace

// ---------------------------------------------------------------------------
// Quantize
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(64 * kWavesPerBlock) void quantize_kernel(Int4Args a)
{
    constexpr int NJ = D / 32;              // 16-byte chunks per lane
    constexpr int N = NJ * 8;               // coordinates per lane
    constexpr int NG = D / G;               // groups per vector
    // Groups that one lane's registers touch: all NG when a group spans the
    // quad (G >= 32), else one per chunk.
    constexpr int LG = (G >= 32) ? NG : NJ;
    constexpr int CH_PER_G = (G >= 32) ? G / 32 : 1;

    const int lane = threadIdx.x & 63;
    const int q = lane & 3;
    const int slot = lane >> 2;
    const int wave = uniform((int)(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)));
    int item = wave * a.items_per_wave;
    const int item_end = min((int64_t)item + a.items_per_wave, a.n_items);
    if (item >= item_end) return;

    const float c1 = (q & 1) ? -1.0f : 1.0f;
    const float c2 = (q & 2) ? -1.0f : 1.0f;
    const float lane_sign = (__builtin_popcount(q) & 1) ? -1.0f : 1.0f;

    const _Float16* __restrict__ xg = static_cast<const _Float16*>(a.x.data);
    uint8_t* __restrict__ cg = static_cast<uint8_t*>(a.codes.data);
    uint16_t* __restrict__ sg = static_cast<uint16_t*>(a.scales.data);

    const int64_t x_lane = (int64_t)slot * a.x.st + q * 8;
    const int64_t c_lane = (int64_t)slot * a.codes.st + q * 4;
    const int64_t s_lane = (int64_t)slot * a.scales.st;

    float m[N];
    int cur_lh = -1;
    const _Float16* xbase = nullptr;
    uint8_t* cbase = nullptr;
    uint16_t* sbase = nullptr;

    auto bases = [&](int lh) {
        const int l = lh / a.H, h = lh - (lh / a.H) * a.H;
        xbase = xg + (int64_t)l * a.x.sl + (int64_t)h * a.x.sh;
        cbase = cg + (int64_t)l * a.codes.sl + (int64_t)h * a.codes.sh;
        sbase = sg + (int64_t)l * a.scales.sl + (int64_t)h * a.scales.sh;
    };

    auto load_x = [&](int it, uint4 (&raw)[NJ]) {
        const ItemPos p = item_pos(it, a.tiles_per_lh);
        const int l = p.lh / a.H, h = p.lh - l * a.H;
        const int t = p.tile * kTokensPerTile + slot;
        const _Float16* ptr = xg + (int64_t)l * a.x.sl + (int64_t)h * a.x.sh +
                              (int64_t)p.tile * kTokensPerTile * a.x.st + x_lane;
        if (t < a.T) {
#pragma unroll
            for (int j = 0; j < NJ; j++) raw[j] = *reinterpret_cast<const uint4*>(ptr + j * 32);
        } else {
#pragma unroll
            for (int j = 0; j < NJ; j++) raw[j] = make_uint4(0, 0, 0, 0);
        }
    };

    uint4 nxt[NJ];
    load_x(item, nxt);

    for (; item < item_end; ++item) {
        const ItemPos p = item_pos(item, a.tiles_per_lh);
        if (p.lh != cur_lh) {
            cur_lh = p.lh;
            bases(p.lh);
            load_fwd_mult<D>(a.lambda + (int64_t)p.lh * D, a.signs, q, m);
        }
        uint4 cur[NJ];
#pragma unroll
        for (int j = 0; j < NJ; j++) cur[j] = nxt[j];
        if (item + 1 < item_end) load_x(item + 1, nxt);

        // --- load/scale fused with the butterfly on register bit 0 ---------
        float v[N];
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const uint32_t w[4] = {cur[j].x, cur[j].y, cur[j].z, cur[j].w};
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const int r = j * 8 + 2 * k;
                const float b = hi_half(w[k]) * m[r + 1];
                v[r] = fmaf(lo_half(w[k]), m[r], b);
                v[r + 1] = fmaf(lo_half(w[k]), m[r], -b);
            }
        }
        fwht_rest(v, c1, c2);

        // --- group abs-max --------------------------------------------------
        float amax[LG];
#pragma unroll
        for (int u = 0; u < LG; u++) amax[u] = 0.0f;
#pragma unroll
        for (int r = 0; r < N; r++) {
            const int u = (r / 8) / CH_PER_G;
            amax[u] = fmaxf(amax[u], fabsf(v[r]));
        }
        if constexpr (G >= 16) {
#pragma unroll
            for (int u = 0; u < LG; u++) quad_max_x1(amax[u]);
        }
        if constexpr (G >= 32) {
#pragma unroll
            for (int u = 0; u < LG; u++) quad_max_x2(amax[u]);
        }

        // --- scales ---------------------------------------------------------
        uint16_t s16[LG];
        float inv[LG];
#pragma unroll
        for (int u = 0; u < LG; u++) {
            const _Float16 h = (_Float16)(amax[u] * kInv7);
            const float sc = (float)h;
            s16[u] = __builtin_bit_cast(uint16_t, h);
            inv[u] = sc > 0.0f ? lane_sign * __builtin_amdgcn_rcpf(sc) : 0.0f;
        }

        // --- codes and nibble packing ----------------------------------------
        uint32_t word[NJ];
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const int u = j / CH_PER_G;
            uint32_t t[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                float f = fmaf(v[j * 8 + e], inv[u], kMagic8);
                f = __builtin_amdgcn_fmed3f(f, kMagic8 - 7.0f, kMagic8 + 7.0f);
                t[e] = __float_as_uint(f);
            }
            const uint32_t even = gather_low_bytes(t[0], t[2], t[4], t[6]);
            const uint32_t odd = gather_low_bytes(t[1], t[3], t[5], t[7]);
            word[j] = ((odd << 4) | even) ^ 0x88888888u;
        }

        // --- stores -----------------------------------------------------------
        const int t = p.tile * kTokensPerTile + slot;
        if (t < a.T) {
            const int64_t toff = (int64_t)p.tile * kTokensPerTile;
            uint8_t* cp = cbase + toff * a.codes.st + c_lane;
#pragma unroll
            for (int j = 0; j < NJ; j++) *reinterpret_cast<uint32_t*>(cp + j * 16) = word[j];
            uint16_t* sp = sbase + toff * a.scales.st + s_lane;
            if constexpr (G >= 32) {
                // every lane holds all NG scales; lane q writes groups q, q+4, ...
#pragma unroll
                for (int g0 = 0; g0 < NG; g0 += 4) {
                    uint16_t val = s16[g0];
#pragma unroll
                    for (int k = 1; k < 4; k++)
                        if (g0 + k < NG && q == k) val = s16[g0 + k];
                    if (g0 + q < NG) sp[g0 + q] = val;
                }
            } else if constexpr (G == 16) {
                // lanes q and q^1 share group 2j + (q >> 1); the even lane writes
                if ((q & 1) == 0) {
#pragma unroll
                    for (int j = 0; j < NJ; j++) sp[2 * j + (q >> 1)] = s16[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < NJ; j++) sp[4 * j + q] = s16[j];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Dequantize
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(64 * kWavesPerBlock) void dequantize_kernel(Int4Args a)
{
    constexpr int NJ = D / 32;
    constexpr int N = NJ * 8;

    const int lane = threadIdx.x & 63;
    const int q = lane & 3;
    const int slot = lane >> 2;
    const int wave = uniform((int)(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)));
    int item = wave * a.items_per_wave;
    const int item_end = min((int64_t)item + a.items_per_wave, a.n_items);
    if (item >= item_end) return;

    const float c1 = (q & 1) ? -1.0f : 1.0f;
    const float c2 = (q & 2) ? -1.0f : 1.0f;
    const float lane_sign = (__builtin_popcount(q) & 1) ? -1.0f : 1.0f;

    _Float16* __restrict__ og = static_cast<_Float16*>(a.x.data);
    const uint8_t* __restrict__ cg = static_cast<const uint8_t*>(a.codes.data);
    const uint16_t* __restrict__ sg = static_cast<const uint16_t*>(a.scales.data);

    const int64_t o_lane = (int64_t)slot * a.x.st + q * 8;
    const int64_t c_lane = (int64_t)slot * a.codes.st + q * 4;
    const int64_t s_lane = (int64_t)slot * a.scales.st;

    float m[N];
    int cur_lh = -1;

    struct Raw {
        uint32_t w[NJ];
        uint16_t s[NJ];
    };
    auto load_in = [&](int it, Raw& raw) {
        const ItemPos p = item_pos(it, a.tiles_per_lh);
        const int l = p.lh / a.H, h = p.lh - l * a.H;
        const int t = p.tile * kTokensPerTile + slot;
        const int64_t toff = (int64_t)p.tile * kTokensPerTile;
        const uint8_t* cp = cg + (int64_t)l * a.codes.sl + (int64_t)h * a.codes.sh +
                            toff * a.codes.st + c_lane;
        const uint16_t* sp = sg + (int64_t)l * a.scales.sl + (int64_t)h * a.scales.sh +
                             toff * a.scales.st + s_lane;
        if (t < a.T) {
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                raw.w[j] = *reinterpret_cast<const uint32_t*>(cp + j * 16);
                raw.s[j] = sp[(j * 32 + q * 8) / G];
            }
        } else {
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                raw.w[j] = 0x88888888u;   // codes 8 ^ 8 = 0 after unbiasing; decodes to zeros
                raw.s[j] = 0;
            }
        }
    };

    Raw nxt;
    load_in(item, nxt);

    for (; item < item_end; ++item) {
        const ItemPos p = item_pos(item, a.tiles_per_lh);
        if (p.lh != cur_lh) {
            cur_lh = p.lh;
            load_inv_mult<D>(a.lambda + (int64_t)p.lh * D, a.signs, q, lane_sign, m);
        }
        Raw cur = nxt;
        if (item + 1 < item_end) load_in(item + 1, nxt);

        // --- unpack fused with the butterfly on register bit 0 ---------------
        // Offset-binary nibbles n = q + 8 of the pair (2k, 2k+1), which share a
        // scale sc:  yhat_2k + yhat_2k+1 = sc * (n0 + n1 - 16),
        //            yhat_2k - yhat_2k+1 = sc * (n0 - n1 + 16 - 16).
        float v[N];
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const float sc = (float)__builtin_bit_cast(_Float16, cur.s[j]);
            const float off = -16.0f * sc;
            const uint32_t wb = cur.w[j] ^ 0x88888888u;
            const uint32_t lo = wb & 0x0f0f0f0fu;            // n of elements 0,2,4,6
            const uint32_t hi = (wb >> 4) & 0x0f0f0f0fu;     // n of elements 1,3,5,7
            const uint32_t sum = lo + hi;                    // bytewise, <= 30
            const uint32_t dif = (lo | 0x10101010u) - hi;    // bytewise, 1..31
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const float fs = (float)((sum >> (8 * k)) & 0xffu);
                const float fd = (float)((dif >> (8 * k)) & 0xffu);
                v[j * 8 + 2 * k] = fmaf(fs, sc, off);
                v[j * 8 + 2 * k + 1] = fmaf(fd, sc, off);
            }
        }
        fwht_rest(v, c1, c2);

        // --- unscale, round to fp16, store -----------------------------------
        const int t = p.tile * kTokensPerTile + slot;
        if (t < a.T) {
            const int l = p.lh / a.H, h = p.lh - l * a.H;
            _Float16* op = og + (int64_t)l * a.x.sl + (int64_t)h * a.x.sh +
                           (int64_t)p.tile * kTokensPerTile * a.x.st + o_lane;
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                uint4 o;
                o.x = pack_half2(v[j * 8 + 0] * m[j * 8 + 0], v[j * 8 + 1] * m[j * 8 + 1]);
                o.y = pack_half2(v[j * 8 + 2] * m[j * 8 + 2], v[j * 8 + 3] * m[j * 8 + 3]);
                o.z = pack_half2(v[j * 8 + 4] * m[j * 8 + 4], v[j * 8 + 5] * m[j * 8 + 5]);
                o.w = pack_half2(v[j * 8 + 6] * m[j * 8 + 6], v[j * 8 + 7] * m[j * 8 + 7]);
                *reinterpret_cast<uint4*>(op + j * 32) = o;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {

template <template <int, int> class K>
struct Dummy;

template <int D, int G>
hipError_t launch_q(const Int4Args& a, hipStream_t s, bool inverse)
{
    const int64_t waves = (a.n_items + a.items_per_wave - 1) / a.items_per_wave;
    const dim3 grid((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock));
    const dim3 block(64 * kWavesPerBlock);
    if (inverse)
        hipLaunchKernelGGL((dequantize_kernel<D, G>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((quantize_kernel<D, G>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_g(const Int4Args& a, hipStream_t s, bool inverse)
{
    switch (a.G) {
        case 8: return launch_q<D, 8>(a, s, inverse);
        case 16: return launch_q<D, 16>(a, s, inverse);
        case 32: return launch_q<D, 32>(a, s, inverse);
        case 64: return launch_q<D, 64>(a, s, inverse);
        case 128: if constexpr (D >= 128) return launch_q<D, 128>(a, s, inverse); break;
        case 256: if constexpr (D >= 256) return launch_q<D, 256>(a, s, inverse); break;
        default: break;
    }
    return hipErrorInvalidValue;
}

hipError_t dispatch(const Int4Args& a, hipStream_t s, bool inverse)
{
    switch (a.D) {
        case 64: return dispatch_g<64>(a, s, inverse);
        case 128: return dispatch_g<128>(a, s, inverse);
        case 256: return dispatch_g<256>(a, s, inverse);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_quantize(const Int4Args& a, hipStream_t s) { return dispatch(a, s, false); }
hipError_t launch_dequantize(const Int4Args& a, hipStream_t s) { return dispatch(a, s, true); }

}  // namespace kvq
