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
// transform, unscale).  With FT the rotation is the sign-randomized real
// Fourier transform instead (same gist, "Methodologie" s.1: the SRFT), whose
// register layout and sign conventions match the Walsh-Hadamard path's.
//
// Work decomposition.  An item is 16 head vectors, one per quad of a
// wavefront.  When the head count divides 16 the item is 16 consecutive
// (token, head) vectors of one layer -- a contiguous 4 KB run of a [L, T, H,
// 128] cache -- and each lane keeps one head for the whole layer; otherwise
// it is 16 consecutive tokens of one (layer, head).  Either way a wavefront
// owns a run of consecutive items, lambda's per-lane multipliers stay in
// registers until the layer (or head) changes, and the next item's loads are
// issued before the current item is computed.  The kernel
// is HBM-bound: per vector it moves 2D + D/2 + 2D/G bytes and does about
// 2.9 VALU operations per coordinate.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_srft.h"

namespace kvq {

namespace {

// fma(y, 1/scale, kMagic) with kMagic = 1.5 * 2^23 + Z leaves Z + rne(y/scale)
// in the low bits (Z = 8 for int4 codes, 128 for int8 codes).
template <int BITS>
struct CodeFmt;
template <>
struct CodeFmt<4> {
    static constexpr float kMagic = 12582920.0f;     // 1.5 * 2^23 + 8
    static constexpr float kQmax = 7.0f;
    static constexpr float kInvQmax = 0.142857142857142857f;
    static constexpr uint32_t kFlip = 0x88888888u;   // offset binary <-> two's complement
};
template <>
struct CodeFmt<8> {
    static constexpr float kMagic = 12583040.0f;     // 1.5 * 2^23 + 128
    static constexpr float kQmax = 127.0f;
    static constexpr float kInvQmax = 0.00787401574803149606f;
    static constexpr uint32_t kFlip = 0x80808080u;
};

// Byte k of the result = low byte of a_k (k = 0..3).
__device__ __forceinline__ uint32_t gather_low_bytes(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3)
{
    const uint32_t lo = __builtin_amdgcn_perm(a1, a0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(a3, a2, 0x04000c0cu);
    return lo | hi;
}

}  // namespace

// ---------------------------------------------------------------------------
// Work items
// ---------------------------------------------------------------------------
namespace {

// Scalar position of an item: layer, head (head-major items only), first
// token, whether all its vectors exist (then loads and stores need no lane
// mask), and the key its lambda multipliers depend on (layer for
// token-major items, (layer, head) for head-major ones).
struct Item {
    int l, h, t0, key;
    bool full;
};

template <bool TM>
__device__ __forceinline__ Item decode_item(int item, const Int4Args& a)
{
    Item it;
    const int grp = uniform(item / a.items_per_group);
    const int k = item - grp * a.items_per_group;
    it.t0 = uniform(k * a.tok_per_item);
    it.full = it.t0 + a.tok_per_item <= a.T;
    it.key = grp;
    if constexpr (TM) {
        it.l = grp;
        it.h = 0;
    } else {
        it.l = uniform(grp / a.H);
        it.h = grp - it.l * a.H;
    }
    return it;
}

// Element offset of the item's first vector in a view (wave-uniform).
__device__ __forceinline__ int64_t outer_offset(const Tensor4& t, const Item& it)
{
    return uniform64((int64_t)it.l * t.sl + (int64_t)it.h * t.sh + (int64_t)it.t0 * t.st);
}

// Per-lane part of an item: token offset and head of the lane's vector.
struct LaneMap {
    int tok, head;
};

template <bool TM>
__device__ __forceinline__ LaneMap lane_map(int slot, const Int4Args& a)
{
    if constexpr (TM) return LaneMap{slot >> a.h_shift, slot & (a.H - 1)};
    else return LaneMap{slot, 0};
}

// lambda row of the lane's vector for the item's key.
template <bool TM>
__device__ __forceinline__ int64_t lambda_row(const Item& it, const LaneMap& lm, const Int4Args& a)
{
    if constexpr (TM) return ((int64_t)it.l * a.H + lm.head) * a.D;
    else return (int64_t)it.key * a.D;
}

// The lane's NG fp16 scales packed four per 64-bit word; returns scale g.
template <int NG>
__device__ __forceinline__ uint16_t pick_scale(const uint16_t (&s)[NG], int g)
{
    uint64_t w[(NG + 3) / 4] = {};
#pragma unroll
    for (int i = 0; i < NG; i++) w[i / 4] |= (uint64_t)s[i] << (16 * (i % 4));
    uint64_t sel = w[0];
#pragma unroll
    for (int i = 1; i < (NG + 3) / 4; i++)
        if (g / 4 == i) sel = w[i];
    return (uint16_t)(sel >> (16 * (g % 4)));
}

}  // namespace

// Quantizer outputs (codes and scales) are stored with the nontemporal hint:
// they are not read again by the launch, and keeping them out of the caches'
// normal replacement leaves more room for the input stream.  Measured on
// MI355X: Qwen3-8B-shaped int4 quantize 4.59 -> 4.38 ms, MXFP4 4.47 -> 4.27,
// int8 5.37 -> 5.35, Gemma-shaped head_dim 256 0.882 -> 0.837 ms.  The same
// hint on the loads (4.56 -> 4.67 ms) or on the dequantizers' fp16 stores
// made them slower.
__device__ __forceinline__ void store_nt(void* p, uint4 v)
{
    typedef uint32_t u4nt __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u4nt{v.x, v.y, v.z, v.w}, reinterpret_cast<u4nt*>(p));
}

// A scale store takes the hint only when an item's scales fill whole
// 128-byte lines (at least 8 bytes of scales per vector, 16 vectors per
// item); smaller rows are left to the cache to merge: MXFP4 at head_dim 128
// (4 bytes per vector) 4.31 -> 4.23 ms with plain scale stores.
template <bool NT, typename T>
__device__ __forceinline__ void store_scale(T* p, T v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// ---------------------------------------------------------------------------
// Quantize
// ---------------------------------------------------------------------------
template <int D, int G>
struct QuantShape {
    static constexpr int NJ = D / 32;            // 16-byte chunks per lane
    static constexpr int N = NJ * 8;             // coordinates per lane
    static constexpr int NG = D / G;             // groups per vector
    // groups one lane's registers touch: all NG when a group spans the quad
    // (G >= 32), else one per chunk
    static constexpr int LG = (G >= 32) ? NG : NJ;
    static constexpr int CH_PER_G = (G >= 32) ? G / 32 : 1;
};

// Item loop shared by both kernels (see the comment below).  With PREFETCH
// the next item's loads are issued before the current item is finished, into
// the item's one register buffer as soon as the first stage has consumed it
// (a second buffer, with the loop unrolled by two, took 12 to 41 more VGPRs:
// a wave per SIMD less for the quantizers and the SRFT dequantizer).
// Without it (the token-major head_dim-256 dequantizers and the head_dim-256
// SRFT kernels, where a prefetch buffer would pass 256 VGPRs and cost a wave
// per SIMD) each item's loads are issued right before its first stage, and
// only the stores are deferred.
template <typename Buf, typename Out, int N, bool PREFETCH, typename Load, typename First, typename Store,
          typename Finish>
__device__ __forceinline__ void run_pipeline(int begin, int end, Load&& load, First&& first_stage,
                                             Store&& store, Finish&& finish)
{
    Out prev;
    int prev_item = -1;
    if constexpr (PREFETCH) {
        Buf buf;
        load(begin, buf);
        for (int item = begin; item < end; ++item) {
            float v[N];
            first_stage(item, buf, v);
            pin(v);
            if (prev_item >= 0) store(prev_item, prev);
            if (item + 1 < end) load(item + 1, buf);
            __builtin_amdgcn_sched_barrier(0);
            finish(v, prev);
            prev_item = item;
        }
    } else {
        for (int item = begin; item < end; ++item) {
            Buf buf;
            load(item, buf);
            float v[N];
            first_stage(item, buf, v);
            pin(v);
            if (prev_item >= 0) store(prev_item, prev);
            __builtin_amdgcn_sched_barrier(0);
            finish(v, prev);
            prev_item = item;
        }
    }
    store(prev_item, prev);
}

// Software pipeline shared by both kernels.  gfx9 counts loads and stores on
// one counter (vmcnt), so consuming a load while any store is outstanding
// waits for everything issued so far.  Each iteration therefore
//   1. consumes the current item's loaded registers (the wait covers loads
//      and stores issued one full item of compute earlier),
//   2. issues the previous item's stores and the next item's loads,
//   3. computes the rest of the current item,
// and a scheduling barrier keeps step 2 between steps 1 and 3.
// The head_dim-128 SRFT quantizer, VALU-bound, is held to three wavefronts
// per SIMD (168 VGPRs; it needs 153 with its twiddles read from LDS per item):
// 6.60 -> 6.20 ms for the Qwen3-8B-shaped K cache against two wavefronts with
// the twiddles in registers.
template <int D, int G, bool TM, int BITS, bool MX, bool FT>
__global__ __launch_bounds__(64 * kWavesPerBlock, (FT && D == 128) ? 3 : 1) void quantize_kernel(Int4Args a)
{
    static_assert(!MX || (BITS == 4 && G == 32), "MXFP4: 4-bit codes in blocks of 32");
    static_assert(!FT || (BITS == 4 && !MX), "SRFT: int4 codes");
    using S = QuantShape<D, G>;
    using F = CodeFmt<BITS>;
    constexpr int WPJ = BITS / 4;        // code dwords per 8-coordinate chunk
    constexpr int NJ = S::NJ, N = S::N, NG = S::NG, LG = S::LG, CH_PER_G = S::CH_PER_G;
    // scale values a lane stores per vector
    constexpr int NSV = (G >= 32) ? (NG + 3) / 4 : NJ;
    constexpr bool SNT = (MX ? NG : 2 * NG) >= 8;     // scale bytes per vector fill lines

    const int lane = threadIdx.x & 63;
    const int q = lane & 3;
    const int slot = lane >> 2;
    const int wave = uniform((int)(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)));
    const int begin = wave * a.items_per_wave;
    const int end = (int)min((int64_t)begin + a.items_per_wave, a.n_items);
    if (begin >= end) return;

    const float c1 = (q & 1) ? -1.0f : 1.0f;
    const float c2 = (q & 2) ? -1.0f : 1.0f;
    const float lane_sign = (__builtin_popcount(q) & 1) ? -1.0f : 1.0f;

    const _Float16* __restrict__ xg = static_cast<const _Float16*>(a.x.data);
    uint8_t* __restrict__ cg = static_cast<uint8_t*>(a.codes.data);
    uint16_t* __restrict__ sg = static_cast<uint16_t*>(a.scales.data);
    uint8_t* __restrict__ sg8 = static_cast<uint8_t*>(a.scales.data);      // MXFP4: E8M0 bytes
    const LaneMap lm = lane_map<TM>(slot, a);
    const int64_t x_lane = (int64_t)lm.tok * a.x.st + (int64_t)lm.head * a.x.sh + q * 8;
    // this lane stores code chunks q, q + 4, ... (16 bytes each) of its vector
    const int64_t c_lane_chunk = (int64_t)lm.tok * a.codes.st + (int64_t)lm.head * a.codes.sh + q * 16;
    const int64_t s_lane = (int64_t)lm.tok * a.scales.st + (int64_t)lm.head * a.scales.sh;

    float m[N];
    int cur_key = -1;
    // SRFT: one LDS row of D/2 complex points (+1 against bank conflicts) per quad
    __shared__ float2 lds_fft[FT ? kWavesPerBlock * 16 * (D / 2 + 1) : 1];
    float2* fft_row = lds_fft + (FT ? ((threadIdx.x >> 6) * 16 + slot) * (D / 2 + 1) : 0);
    // SRFT: at head_dim 128 the wavefront's twiddle rows (one per quad lane),
    // read back per item; otherwise the twiddles stay in registers
    constexpr bool TW_LDS = FT && D == 128;
    __shared__ float2 lds_tw[TW_LDS ? kWavesPerBlock * 4 * srft::TwRow<D>::N : 1];
    float2* tw_rows = lds_tw + (TW_LDS ? (threadIdx.x >> 6) * 4 * srft::TwRow<D>::N : 0);
    if constexpr (TW_LDS) srft::write_twiddle_row<D>(tw_rows + q * srft::TwRow<D>::N, q);
    srft::Tw<D, -1> tw;
    if constexpr (FT && !TW_LDS) tw = srft::make_twiddles<D, -1>(q);

    struct Out {
        uint32_t word[NJ * WPJ];
        uint16_t sv[NSV];
    };

    // In a partial item the lanes past the last token load the last token's
    // vector: every vector is computed on its own quad and theirs are never
    // stored, so the loads stay unconditional (masked loads cost the
    // register zeroing on every item).
    auto load = [&](int item, uint4(&buf)[NJ]) {
        const Item it = decode_item<TM>(item, a);
        int64_t off = outer_offset(a.x, it) + x_lane;
        if (!it.full) off += (int64_t)(min(lm.tok, a.T - 1 - it.t0) - lm.tok) * a.x.st;
        const _Float16* p = xg + off;
#pragma unroll
        for (int j = 0; j < NJ; j++) buf[j] = *reinterpret_cast<const uint4*>(p + j * 32);
    };

    // Code bytes are transposed within each quad through a wave-private LDS
    // tile so that every lane stores whole 16-byte chunks: code chunk c of a
    // vector (bytes 16c..16c+15) goes to lane c % 4.  int4: chunk j is word j
    // of lanes q = 0..3, and word j of lane (v, q) sits at
    // v*D/8 + ((j ^ (v >> 2)) % NJ)*4 + q, which spreads a wave's 64 dword
    // writes over distinct banks.  int8: lane q's 8 bytes of chunk position
    // j are bytes 32j + 8q .. of the vector, i.e. half (q & 1) of 16-byte
    // chunk 2j + (q >> 1); chunk c of vector v sits at v*CV8 + (c ^ (v % CV8)).
    constexpr int CV8 = D / 16;                                   // int8 chunks per vector
    constexpr int ROWW = BITS == 4 ? D / 8 : D / 4;               // code dwords per vector
    __shared__ uint32_t lds_codes[kWavesPerBlock][16 * ROWW];
    uint32_t* my_codes = lds_codes[threadIdx.x >> 6];
    constexpr int NCH = BITS == 4 ? NJ : CV8;                     // 16-byte code chunks per vector
    constexpr int CPL = (NCH + 3) / 4;                            // chunks each lane stores
    auto chunk_pos = [&](int v, int c) {                          // dword index of chunk c of vector v
        if constexpr (BITS == 4) return v * ROWW + ((c ^ (v >> 2)) % NJ) * 4;
        else return v * ROWW + (c ^ (v % CV8)) * 4;
    };

    // int8: NCH lanes cover one vector's code row, VPI = 64 / NCH vectors per
    // store instruction, so each instruction writes whole rows (1 KB
    // contiguous for a token-major item) and no nontemporal store covers
    // half a line (with four lanes per vector the int8 quantizer wrote 5.1%
    // more than its code bytes; Qwen3-8B-shaped K: 5.35 -> 5.12 ms).  Vector
    // k*VPI + r sits at the offset of vector k*VPI (wavefront-uniform) plus
    // that of vector r.
    constexpr int VPI = 64 / NCH;
    const int r8 = lane / NCH, c8 = lane % NCH;
    const LaneMap rm8 = lane_map<TM>(r8, a);
    const int64_t c8_lane = (int64_t)rm8.tok * a.codes.st + (int64_t)rm8.head * a.codes.sh + c8 * 16;
    auto store = [&](int item, const Out& o) {
        const Item it = decode_item<TM>(item, a);
        uint8_t* cp = cg + outer_offset(a.codes, it) + c_lane_chunk;
        uint16_t* sp = sg + outer_offset(a.scales, it) + s_lane;
        if constexpr (BITS == 4) {
#pragma unroll
            for (int j = 0; j < NJ; j++) my_codes[chunk_pos(slot, j) + q] = o.word[j];
        } else {
#pragma unroll
            for (int j = 0; j < NJ; j++)
                *reinterpret_cast<uint2*>(&my_codes[chunk_pos(slot, 2 * j + (q >> 1)) + 2 * (q & 1)]) =
                    make_uint2(o.word[2 * j], o.word[2 * j + 1]);
        }
        const bool ok = it.full || it.t0 + lm.tok < a.T;
        if constexpr (BITS == 8) {
            uint8_t* cb8 = cg + outer_offset(a.codes, it);
#pragma unroll
            for (int k = 0; k < CPL; k++) {
                const uint4 chunk = *reinterpret_cast<const uint4*>(&my_codes[chunk_pos(k * VPI + r8, c8)]);
                const LaneMap km = lane_map<TM>(k * VPI, a);
                const int64_t off = uniform64((int64_t)km.tok * a.codes.st + (int64_t)km.head * a.codes.sh) + c8_lane;
                if (it.full || it.t0 + km.tok + rm8.tok < a.T) store_nt(cb8 + off, chunk);
            }
        } else {
#pragma unroll
            for (int k = 0; k < CPL; k++) {
                // lanes with q + 4k >= NCH (int4, head_dim 64 only) read a valid slot and do not store
                const int c = q + 4 * k;
                const uint4 chunk = *reinterpret_cast<const uint4*>(&my_codes[chunk_pos(slot, c % NCH)]);
                if (ok && c < NCH) store_nt(cp + 64 * k, chunk);
            }
        }
        if (ok) {
            if constexpr (MX) {
                uint8_t* sp8 = sg8 + outer_offset(a.scales, it) + s_lane;
#pragma unroll
                for (int k = 0; k < NSV; k++)
                    if (4 * k + q < NG) store_scale<SNT>(sp8 + 4 * k + q, (uint8_t)o.sv[k]);
            } else if constexpr (G >= 32) {
                // lane q writes groups q, q+4, ...
#pragma unroll
                for (int k = 0; k < NSV; k++)
                    if (4 * k + q < NG) store_scale<SNT>(sp + 4 * k + q, o.sv[k]);
            } else if constexpr (G == 16) {
                // lanes q and q^1 share group 2j + (q >> 1); the even lane writes
                if ((q & 1) == 0) {
#pragma unroll
                    for (int j = 0; j < NJ; j++) store_scale<SNT>(sp + 2 * j + (q >> 1), o.sv[j]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < NJ; j++) store_scale<SNT>(sp + 4 * j + q, o.sv[j]);
            }
        }
    };

    // step 1: lambda/sign scaling fused with the butterfly on register bit 0
    // (SRFT: the scaling alone)
    auto first_stage = [&](int item, const uint4(&buf)[NJ], float(&v)[N]) {
        const Item it = decode_item<TM>(item, a);
        if (it.key != cur_key) {
            cur_key = it.key;
            load_fwd_mult<D>(a.lambda + lambda_row<TM>(it, lm, a), a.signs, q, m);
            if constexpr (FT) {
#pragma unroll
                for (int i = 0; i < N; i++) m[i] *= 0.70710678118654752440f;   // the SRFT's 1/sqrt2
            }
        }
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const uint32_t w[4] = {buf[j].x, buf[j].y, buf[j].z, buf[j].w};
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const int r = j * 8 + 2 * k;
                if constexpr (FT) {
                    v[r] = fmaf(lo_half(w[k]), m[r], 0.0f);           // one v_fma_mix each
                    v[r + 1] = fmaf(hi_half(w[k]), m[r + 1], 0.0f);
                } else {
                    const float b = fmaf(hi_half(w[k]), m[r + 1], 0.0f);   // one v_fma_mix
                    v[r] = fmaf(lo_half(w[k]), m[r], b);
                    v[r + 1] = fmaf(lo_half(w[k]), m[r], -b);
                }
            }
        }
    };

    // step 3: rest of the transform, scales, codes, packing
    auto finish = [&](float(&v)[N], Out& o) {
        if constexpr (TW_LDS) {
            // an offset the compiler cannot see as loop-invariant, so the row is
            // read per item and not held in registers across items
            int qo = q * srft::TwRow<D>::N;
            asm volatile("" : "+v"(qo));
            srft::forward<D>(v, fft_row, q, static_cast<const float2*>(tw_rows + qo));
        } else if constexpr (FT) {
            srft::forward<D>(v, fft_row, q, tw);
        }
        else fwht_rest(v, c1, c2);

        float amax[LG];
#pragma unroll
        for (int u = 0; u < LG; u++) amax[u] = 0.0f;
#pragma unroll
        for (int r = 0; r < N; r++) {
            const int u = (r / 8) / CH_PER_G;
            amax[u] = fmaxf(amax[u], fabsf(v[r]));
        }
        if constexpr (G >= 16) quad_max<false>(amax);
        if constexpr (G >= 32) quad_max<true>(amax);

        if constexpr (MX) {
            // Block exponent e = floor(log2 amax) - 2, clamped at -127, stored
            // as the E8M0 byte e + 127 = max(biased exponent of amax - 2, 0).
            // The E2M1 conversion (round to nearest even, saturating at 6,
            // sign kept) runs on y * 2^-e, an exact power-of-two scaling.
            uint16_t sb[LG];
            float inv[LG];
#pragma unroll
            for (int u = 0; u < LG; u++) {
                const uint32_t eb = (__float_as_uint(amax[u]) >> 23) & 0xffu;
                const uint32_t byte = eb > 2u ? eb - 2u : 0u;
                sb[u] = (uint16_t)byte;
                inv[u] = lane_sign * __uint_as_float((254u - byte) << 23);
            }
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                const float f = inv[j];
                uint32_t w = 0u;
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * j + 0] * f, v[8 * j + 1] * f, 1.0f, 0);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * j + 2] * f, v[8 * j + 3] * f, 1.0f, 1);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * j + 4] * f, v[8 * j + 5] * f, 1.0f, 2);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * j + 6] * f, v[8 * j + 7] * f, 1.0f, 3);
                o.word[j] = w;
            }
#pragma unroll
            for (int k = 0; k < NSV; k++) o.sv[k] = pick_scale<NG>(sb, (4 * k + q) % NG);
            return;
        }

        uint16_t s16[LG];
        float inv[LG];
        bool overflow = false;
#pragma unroll
        for (int u = 0; u < LG; u++) {
            const _Float16 h = (_Float16)(amax[u] * F::kInvQmax);
            const float sc = (float)h;
            s16[u] = __builtin_bit_cast(uint16_t, h);
            const float r = sc > 0.0f ? __builtin_amdgcn_rcpf(sc) : 0.0f;
            inv[u] = lane_sign * r;
            // only a subnormal scale can let |y|/scale reach qmax + 1/2
            overflow |= amax[u] * r >= F::kQmax + 0.5f;
        }

        // codes: Z + rne(y/scale) lands in the low byte of t; then nibble
        // pack (int4) or byte pack (int8), back to two's complement
        auto encode = [&](auto clamp) {
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                const int u = j / CH_PER_G;
                uint32_t t[8];
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    float f = fmaf(v[j * 8 + e], inv[u], F::kMagic);
                    if constexpr (decltype(clamp)::value)
                        f = __builtin_amdgcn_fmed3f(f, F::kMagic - F::kQmax, F::kMagic + F::kQmax);
                    t[e] = __float_as_uint(f);
                }
                if constexpr (BITS == 4) {
                    const uint32_t even = gather_low_bytes(t[0], t[2], t[4], t[6]);
                    const uint32_t odd = gather_low_bytes(t[1], t[3], t[5], t[7]);
                    o.word[j] = ((odd << 4) | even) ^ F::kFlip;
                } else {
                    o.word[2 * j] = gather_low_bytes(t[0], t[1], t[2], t[3]) ^ F::kFlip;
                    o.word[2 * j + 1] = gather_low_bytes(t[4], t[5], t[6], t[7]) ^ F::kFlip;
                }
            }
        };
        if (__builtin_amdgcn_ballot_w64(overflow))
            encode(std::true_type{});
        else
            encode(std::false_type{});

        if constexpr (G >= 32) {
#pragma unroll
            for (int k = 0; k < NSV; k++) o.sv[k] = pick_scale<NG>(s16, (4 * k + q) % NG);
        } else {
#pragma unroll
            for (int j = 0; j < NJ; j++) o.sv[j] = s16[j];
        }
    };

    // the head_dim-256 quantizers prefetch too (two waves per SIMD either
    // way), except SRFT, which would drop to one
    run_pipeline<uint4[NJ], Out, N, (D <= 128 || !FT)>(begin, end, load, first_stage, store, finish);
}

// ---------------------------------------------------------------------------
// Dequantize
// ---------------------------------------------------------------------------
template <int D, int G, bool TM, int BITS, bool MX, bool FT>
__global__ __launch_bounds__(64 * kWavesPerBlock) void dequantize_kernel(Int4Args a)
{
    static_assert(!MX || (BITS == 4 && G == 32), "MXFP4: 4-bit codes in blocks of 32");
    static_assert(!FT || (BITS == 4 && !MX), "SRFT: int4 codes");
    constexpr int WPJ = BITS / 4;        // code dwords per 8-coordinate chunk
    constexpr int NJ = D / 32;
    constexpr int N = NJ * 8;
    constexpr int NG = D / G;
    constexpr int NW = (NG + 1) / 2;

    const int lane = threadIdx.x & 63;
    const int q = lane & 3;
    const int slot = lane >> 2;
    const int wave = uniform((int)(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)));
    const int begin = wave * a.items_per_wave;
    const int end = (int)min((int64_t)begin + a.items_per_wave, a.n_items);
    if (begin >= end) return;

    const float c1 = (q & 1) ? -1.0f : 1.0f;
    const float c2 = (q & 2) ? -1.0f : 1.0f;
    const float lane_sign = (__builtin_popcount(q) & 1) ? -1.0f : 1.0f;

    _Float16* __restrict__ og = static_cast<_Float16*>(a.x.data);
    const uint8_t* __restrict__ cg = static_cast<const uint8_t*>(a.codes.data);
    const uint16_t* __restrict__ sg = static_cast<const uint16_t*>(a.scales.data);
    const LaneMap lm = lane_map<TM>(slot, a);
    const int64_t c_lane = (int64_t)lm.tok * a.codes.st + (int64_t)lm.head * a.codes.sh + q * 4 * WPJ;
    const int64_t s_lane = (int64_t)lm.tok * a.scales.st + (int64_t)lm.head * a.scales.sh;

    float m[N];
    int cur_key = -1;
    __shared__ float2 lds_fft[FT ? kWavesPerBlock * 16 * (D / 2 + 1) : 1];
    float2* fft_row = lds_fft + (FT ? ((threadIdx.x >> 6) * 16 + slot) * (D / 2 + 1) : 0);
    srft::Tw<D, 1> tw;
    if constexpr (FT) tw = srft::make_twiddles<D, 1>(q);

    // Raw inputs of one item: the lane's NJ code words and its vector's whole
    // scale row as packed 32-bit words.
    struct Raw {
        uint32_t w[NJ * WPJ];
        uint32_t sw[MX ? NG : NW];      // MXFP4: one E8M0 byte per block
    };
    struct Out {
        uint4 o[NJ];
    };

    // Lanes past the last token of a partial item load the last token's
    // codes and scales (their outputs are never stored), so the loads stay
    // unconditional.
    auto load = [&](int item, Raw& raw) {
        const Item it = decode_item<TM>(item, a);
        int64_t coff = outer_offset(a.codes, it) + c_lane, soff = outer_offset(a.scales, it) + s_lane;
        if (!it.full) {
            const int dt = min(lm.tok, a.T - 1 - it.t0) - lm.tok;
            coff += (int64_t)dt * a.codes.st;
            soff += (int64_t)dt * a.scales.st;
        }
        const uint8_t* cp = cg + coff;
        const uint16_t* sp = sg + soff;
        auto ld = [&]() {
            if constexpr (BITS == 4) {
#pragma unroll
                for (int j = 0; j < NJ; j++) raw.w[j] = *reinterpret_cast<const uint32_t*>(cp + j * 16);
            } else {
#pragma unroll
                for (int j = 0; j < NJ; j++) {
                    const uint2 d = *reinterpret_cast<const uint2*>(cp + j * 32);
                    raw.w[2 * j] = d.x;
                    raw.w[2 * j + 1] = d.y;
                }
            }
            if constexpr (MX) {
                const uint8_t* sp8 = reinterpret_cast<const uint8_t*>(sg) + soff;
#pragma unroll
                for (int g = 0; g < NG; g++) raw.sw[g] = sp8[g];
            } else if constexpr (NG == 1) {
                raw.sw[0] = sp[0];
            } else {
                // scale rows are only 2-byte aligned; gfx950 serves unaligned
                // dword loads from global memory
                typedef uint32_t u32_a2 __attribute__((aligned(2)));
#pragma unroll
                for (int i = 0; i < NW; i++) raw.sw[i] = reinterpret_cast<const u32_a2*>(sp)[i];
            }
        };
        ld();
    };

    // The item's 16 output vectors (16 * 2D bytes) are staged through a
    // wave-private LDS tile so that each global store instruction writes 1 KB
    // of consecutive vectors instead of 64-byte pieces at a vector stride.
    // 16-byte chunk c of vector v sits at chunk slot v*CV + (c ^ ((4v) % CV)),
    // which keeps both the chunk writes and the row reads bank-conflict free.
    constexpr int CV = D / 8;                  // 16-byte chunks per vector
    constexpr int VPK = 1024 / (2 * D);        // vectors per 1 KB store row
    __shared__ uint4 lds_out[kWavesPerBlock][16 * CV];
    uint4* my_out = lds_out[threadIdx.x >> 6];
    // store row k: lane covers vector v = k*VPK + lane / CV, chunk lane % CV.
    // Vector k*VPK + r of an item sits at the offset of vector k*VPK (the
    // same for the whole wavefront) plus that of vector r (fixed per lane):
    // VPK and H are powers of two, so the token and head of the sum never
    // carry into each other.  Keeping one lane offset instead of one per row
    // takes the token-major head_dim-128 dequantizers from 148-154 to
    // 114-120 VGPRs (four waves per SIMD instead of three).  Measured on
    // MI355X (Qwen3-8B-shaped K cache): MXFP4 4.88 -> 4.67 ms, SRFT 6.72 ->
    // 6.62, int4 unchanged, int8 5.65 -> 5.81; int8 therefore keeps per-row
    // offsets and three waves per SIMD.
    const int row_c = lane % CV;
    const LaneMap rm = lane_map<TM>(lane / CV, a);
    const int64_t row_lane = (int64_t)rm.tok * a.x.st + (int64_t)rm.head * a.x.sh + row_c * 8;
    auto store = [&](int item, const Out& o) {
        const Item it = decode_item<TM>(item, a);
        _Float16* ob = og + outer_offset(a.x, it);
#pragma unroll
        for (int j = 0; j < NJ; j++) my_out[slot * CV + ((4 * j + q) ^ ((4 * slot) % CV))] = o.o[j];
        uint4 row[NJ];
#pragma unroll
        for (int k = 0; k < NJ; k++) {
            const int v = k * VPK + lane / CV;
            row[k] = my_out[v * CV + (row_c ^ ((4 * v) % CV))];
        }
#pragma unroll
        for (int k = 0; k < NJ; k++) {
            if constexpr (BITS == 8) {
                const LaneMap vm = lane_map<TM>(k * VPK + lane / CV, a);
                const int64_t off = (int64_t)vm.tok * a.x.st + (int64_t)vm.head * a.x.sh + row_c * 8;
                if (it.full || it.t0 + vm.tok < a.T) *reinterpret_cast<uint4*>(ob + off) = row[k];
            } else {
                const LaneMap km = lane_map<TM>(k * VPK, a);
                const int64_t off = uniform64((int64_t)km.tok * a.x.st + (int64_t)km.head * a.x.sh) + row_lane;
                if (it.full || it.t0 + km.tok + rm.tok < a.T) *reinterpret_cast<uint4*>(ob + off) = row[k];
            }
        }
    };

    // scale of chunk j: group (j*32 + q*8) / G of the row
    auto chunk_scale = [&](const Raw& raw, int j) -> float {
        uint32_t h;
        if constexpr (G >= 32) {
            const int g = (j * 32) / G;
            h = raw.sw[g / 2] >> (16 * (g % 2));
        } else if constexpr (G == 16) {
            h = raw.sw[j] >> ((q & 2) * 8);                         // group 2j + (q >> 1)
        } else {
            // group 4j + q: word 2j + (q >> 1), selected without an indexed
            // access (which would force the row into scratch memory)
            const uint32_t lo = raw.sw[2 * j], hi = raw.sw[2 * j + 1];
            const uint32_t wsel = lo ^ ((lo ^ hi) & (0u - (uint32_t)((q >> 1) & 1)));
            h = wsel >> ((q & 1) * 16);
        }
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
    };

    // step 1: unpack fused with the butterfly on register bit 0.  With
    // offset-binary nibbles n = q + 8 of the pair (2k, 2k+1), which share the
    // scale sc:  yhat_2k + yhat_2k+1 = sc * (n0 + n1 - 16) and
    //            yhat_2k - yhat_2k+1 = sc * ((n0 - n1 + 16) - 16).
    auto first_stage = [&](int item, const Raw& raw, float(&v)[N]) {
        const Item it = decode_item<TM>(item, a);
        if (it.key != cur_key) {
            cur_key = it.key;
            load_inv_mult<D>(a.lambda + lambda_row<TM>(it, lm, a), a.signs, q, lane_sign, m);
            if constexpr (FT) {
#pragma unroll
                for (int i = 0; i < N; i++) m[i] *= 0.70710678118654752440f;   // the SRFT's 1/sqrt2
            }
        }
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            if constexpr (MX) {
                // E2M1 pairs straight to f32 (exact), times the block's 2^(b - 127)
                const float X = __builtin_amdgcn_ldexpf(1.0f, (int)raw.sw[j] - 127);
                typedef float f2_t __attribute__((ext_vector_type(2)));
                const f2_t p[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(raw.w[j], 1.0f, 0),
                                   __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(raw.w[j], 1.0f, 1),
                                   __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(raw.w[j], 1.0f, 2),
                                   __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(raw.w[j], 1.0f, 3)};
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    const float t = p[k].y * X;
                    v[j * 8 + 2 * k] = fmaf(p[k].x, X, t);
                    v[j * 8 + 2 * k + 1] = fmaf(p[k].x, X, -t);
                }
                continue;
            }
            const float sc = chunk_scale(raw, j);
            if constexpr (BITS == 8) {
                // offset-binary bytes u = q + 128 of the pair (2k, 2k+1):
                // yhat_2k + yhat_2k+1 = sc * (u0 + u1 - 256), difference sc * (u0 - u1)
                const float off8 = -256.0f * sc;
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const uint32_t wb = raw.w[2 * j + h] ^ 0x80808080u;
#pragma unroll
                    for (int k = 0; k < 2; k++) {
                        const float u0 = (float)((wb >> (16 * k)) & 0xffu);
                        const float u1 = (float)((wb >> (16 * k + 8)) & 0xffu);
                        v[j * 8 + 4 * h + 2 * k] = fmaf(u0 + u1, sc, off8);
                        v[j * 8 + 4 * h + 2 * k + 1] = (u0 - u1) * sc;
                    }
                }
                continue;
            }
            const float off = -16.0f * sc;
            const uint32_t wb = raw.w[j] ^ 0x88888888u;
            const uint32_t lo = wb & 0x0f0f0f0fu;            // n of elements 0,2,4,6
            const uint32_t hi = (wb >> 4) & 0x0f0f0f0fu;     // n of elements 1,3,5,7
            if constexpr (FT) {
                // the plain values yhat = (n - 8) * sc.  With lo and hi opaque,
                // each byte converts with one v_cvt_f32_ubyte<k> (the compiler
                // would otherwise extract every nibble with a v_bfe first)
                uint32_t lo8 = lo, hi8 = hi;
                asm volatile("" : "+v"(lo8), "+v"(hi8));
                const float off8 = -8.0f * sc;
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    v[j * 8 + 2 * k] = fmaf((float)((lo8 >> (8 * k)) & 0xffu), sc, off8);
                    v[j * 8 + 2 * k + 1] = fmaf((float)((hi8 >> (8 * k)) & 0xffu), sc, off8);
                }
                continue;
            }
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
    };

    // step 3: rest of the inverse transform, unscale, round to fp16
    auto finish = [&](float(&v)[N], Out& o) {
        if constexpr (FT) srft::inverse<D>(v, fft_row, q, tw);
        else fwht_rest(v, c1, c2);
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            o.o[j].x = pack_half2(v[j * 8 + 0] * m[j * 8 + 0], v[j * 8 + 1] * m[j * 8 + 1]);
            o.o[j].y = pack_half2(v[j * 8 + 2] * m[j * 8 + 2], v[j * 8 + 3] * m[j * 8 + 3]);
            o.o[j].z = pack_half2(v[j * 8 + 4] * m[j * 8 + 4], v[j * 8 + 5] * m[j * 8 + 5]);
            o.o[j].w = pack_half2(v[j * 8 + 6] * m[j * 8 + 6], v[j * 8 + 7] * m[j * 8 + 7]);
        }
    };

    run_pipeline<Raw, Out, N, (D <= 128 || (!TM && !FT))>(begin, end, load, first_stage, store, finish);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {

template <int D, int G, int BITS, bool MX = false, bool FT = false>
hipError_t launch_qb(const Int4Args& a, hipStream_t s, bool inverse)
{
    const int64_t waves = (a.n_items + a.items_per_wave - 1) / a.items_per_wave;
    const dim3 grid((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock));
    const dim3 block(64 * kWavesPerBlock);
    if (inverse) {
        if (a.token_major) hipLaunchKernelGGL((dequantize_kernel<D, G, true, BITS, MX, FT>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((dequantize_kernel<D, G, false, BITS, MX, FT>), grid, block, 0, s, a);
    } else {
        if (a.token_major) hipLaunchKernelGGL((quantize_kernel<D, G, true, BITS, MX, FT>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((quantize_kernel<D, G, false, BITS, MX, FT>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

template <int D, int G>
hipError_t launch_q(const Int4Args& a, hipStream_t s, bool inverse)
{
    if (a.fourier) return launch_qb<D, G, 4, false, true>(a, s, inverse);
    if constexpr (G == 32)
        if (a.mx) return launch_qb<D, 32, 4, true>(a, s, inverse);
    return a.bits == 8 ? launch_qb<D, G, 8>(a, s, inverse) : launch_qb<D, G, 4>(a, s, inverse);
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
