// kvq_attend.hip -- single-query decode attention straight from the int4
// cache, for gfx950 (MI355X).
//
// The operation (VeloxQuant-MLX package description, "Fused group-affine
// (KIVI-style) attention"): one decode step of softmax attention whose keys
// and values are rebuilt from their codes in registers inside a
// flash-decoding online softmax accumulated in fp32; no dequantized cache is
// ever written.  Here the codes are those of the rotated int4 quantizer
// ("When Quantization Is Free", abstract; gist.science summary,
// "Methodologie" s.1-2), and the attention runs in the rotated domain: the
// rotation is orthogonal and the smooth scale and signs are diagonal, so with
//   qt = H (s * q / lambda_K) / sqrt(D)
//   q . khat_t = qt . yhat_t,            yhat_t,c = code_t,c * scale_t,g(c)
//   sum_t p_t vhat_t = s / (lambda_V sqrt(D)) * H (sum_t p_t yhatV_t).
// Each query is rotated once, keys are never inverse-transformed, and the
// value sum is inverse-transformed once per query.
//
// Partial kernel.  Block = one (outer index, KV head), one token range (a
// split) and up to RP query heads of that KV head.  Lanes: LPT = D/16 lanes
// per token hold 16 coordinates each; a wavefront has TS = 64/LPT token
// slots, and each slot keeps its own online-softmax state over the tokens
// t = slot, slot + TS, ... of the wavefront's range.  Scores are in the
// log2 domain (log2 e is folded into the rotated query).  The codes are
// offset-binary after an xor with 0x88888888; the -8 offset is folded into a
// per-lane query sum (keys) and a running sum of p * scale (values).  Each
// slot writes one partial (max, sum of weights, weighted value sum in the
// rotated domain) to the workspace.
//
// Combine kernel.  One quad per (outer index, query head): merges the
// partials, normalises, applies the inverse rotation and unscale, writes fp16.
#include <algorithm>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

// DPP lane exchanges within rows of 16 (hazards are left to the compiler).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    // every control used here is a full permutation, so no lane keeps an old
    // value (an old operand of 0 would cost a v_mov per use)
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16

// Sum over the LPT consecutive lanes of a token slot; every lane of the slot
// receives the total.
template <int LPT>
__device__ __forceinline__ float slot_sum(float v)
{
    v += dpp_mov<kDppXor1>(v);
    v += dpp_mov<kDppXor2>(v);
    if constexpr (LPT >= 8) v += dpp_mov<kDppHalfMirror>(v);
    if constexpr (LPT >= 16) v += dpp_mov<kDppMirror>(v);
    return v;
}

// Bytes 0..3 of x as floats (one v_cvt_f32_ubyteN each).
__device__ __forceinline__ void bytes_to_f32(uint32_t x, float& a, float& b, float& c, float& d)
{
    asm("v_cvt_f32_ubyte0 %0, %4\n\tv_cvt_f32_ubyte1 %1, %4\n\tv_cvt_f32_ubyte2 %2, %4\n\tv_cvt_f32_ubyte3 %3, %4"
        : "=&v"(a), "=&v"(b), "=&v"(c), "=v"(d)
        : "v"(x));
}

// 16 offset-binary codes (code + 8) of a lane as floats, coordinate order.
__device__ __forceinline__ void unpack16(uint2 w, float (&u)[16])
{
    const uint32_t x[2] = {w.x ^ 0x88888888u, w.y ^ 0x88888888u};
#pragma unroll
    for (int d = 0; d < 2; d++) {
        const uint32_t lo = x[d] & 0x0F0F0F0Fu, hi = (x[d] >> 4) & 0x0F0F0F0Fu;
        bytes_to_f32(lo, u[8 * d + 0], u[8 * d + 2], u[8 * d + 4], u[8 * d + 6]);
        bytes_to_f32(hi, u[8 * d + 1], u[8 * d + 3], u[8 * d + 5], u[8 * d + 7]);
    }
}

}  // namespace

template <int D, int RP, bool SPLIT>
__global__ __launch_bounds__(64 * kAttnWaves) void attend_partial_kernel(AttnArgs a)
{
    constexpr int LPT = D / 16;          // lanes per token
    constexpr int TS = 64 / LPT;         // token slots per wavefront
    constexpr int NJ = D / 32;
    constexpr int N = D / 4;

    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    // Block -> (outer index l, split, KV head h).  The heads of one (l, split)
    // read interleaved rows of the same cache lines ([T, H, D/2] codes,
    // [T, H, D/G] scales), so when the (l, split) count is a multiple of the
    // 8 XCDs (blocks go to XCDs round-robin by index) they are given
    // consecutive block indices of one XCD and share its L2.
    int l, h, split;
    {
        const int b = blockIdx.x;
        int u;
        if (a.xcd_map) {
            const int k = b >> 3;
            u = ((k / a.H) << 3) + (b & 7);
            h = k - (k / a.H) * a.H;
        } else {
            u = b / a.H;
            h = b - u * a.H;
        }
        l = uniform(u / a.S);
        split = u - l * a.S;
        h = uniform(h);
    }
    const int lh = l * a.H + h;
    const int r0 = blockIdx.y * RP;
    const int n = a.lengths ? min(max(a.lengths[l], 0), a.T) : a.T;

    // ---- rotate the pass's queries into LDS (quad r: query r0 + r) ---------
    __shared__ float qt[RP][D];
    if (wid == 0) {
        const int qd = lane >> 2, qq = lane & 3;
        const int rr = min(qd, RP - 1);
        const int qi = min(r0 + rr, a.R - 1);
        const _Float16* qp = a.q + (((int64_t)l * a.H + h) * a.R + qi) * D;
        const float* lk = a.lam_k + ((int64_t)l * a.H + h) * D;
        float v[N];
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const int c0 = 32 * j + 8 * qq;
            const uint4 qw = *reinterpret_cast<const uint4*>(qp + c0);
            const float4 l0 = *reinterpret_cast<const float4*>(lk + c0);
            const float4 l1 = *reinterpret_cast<const float4*>(lk + c0 + 4);
            const uint2 sg = *reinterpret_cast<const uint2*>(a.signs + c0);
            const uint32_t w[4] = {qw.x, qw.y, qw.z, qw.w};
            const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const uint32_t word = e < 4 ? sg.x : sg.y;
                const int sv = (int)(int8_t)((word >> (8 * (e & 3))) & 0xff);
                const float qv = (e & 1) ? hi_half(w[e / 2]) : lo_half(w[e / 2]);
                x[e] = (sv < 0 ? -qv : qv) / (lv[e] * SqrtD<D>::v);
            }
#pragma unroll
            for (int k = 0; k < 4; k++) {
                v[8 * j + 2 * k] = x[2 * k] + x[2 * k + 1];
                v[8 * j + 2 * k + 1] = x[2 * k] - x[2 * k + 1];
            }
        }
        fwht_rest(v, (qq & 1) ? -1.0f : 1.0f, (qq & 2) ? -1.0f : 1.0f);
        const float f = ((__builtin_popcount(qq) & 1) ? -1.0f : 1.0f) * a.qscale;
        if (qd < RP) {
#pragma unroll
            for (int j = 0; j < NJ; j++)
#pragma unroll
                for (int e = 0; e < 8; e++) qt[rr][32 * j + 8 * qq + e] = v[8 * j + e] * f;
        }
    }
    __syncthreads();

    const int slot = lane / LPT;
    const int ck = lane % LPT;           // this lane's coordinates: 16 ck .. 16 ck + 15
    float qv[RP][16], qs0[RP], qs1[RP];
#pragma unroll
    for (int r = 0; r < RP; r++) {
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
            const float4 t4 = *reinterpret_cast<const float4*>(&qt[r][16 * ck + i]);
            qv[r][i] = t4.x; qv[r][i + 1] = t4.y; qv[r][i + 2] = t4.z; qv[r][i + 3] = t4.w;
        }
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++) { s0 += qv[r][i]; s1 += qv[r][8 + i]; }
        qs0[r] = -8.0f * s0;
        qs1[r] = -8.0f * s1;
    }

    // ---- this wavefront's token range --------------------------------------
    const int cb = split * a.chunk;
    const int ce = min(cb + a.chunk, n);
    const int per_wave = ((a.chunk + kAttnWaves * TS - 1) / (kAttnWaves * TS)) * TS;
    const int wb = cb + wid * per_wave;
    const int we = min(wb + per_wave, ce);
    const int nfull = we > wb ? (we - wb) / TS : 0;       // steps where every slot has a token
    const int rem = we > wb ? (we - wb) - nfull * TS : 0; // slots with a token in the last step

    const uint8_t* kcg = static_cast<const uint8_t*>(a.kc.data) + (int64_t)l * a.kc.sl + (int64_t)h * a.kc.sh + 8 * ck;
    const uint8_t* vcg = static_cast<const uint8_t*>(a.vc.data) + (int64_t)l * a.vc.sl + (int64_t)h * a.vc.sh + 8 * ck;
    const int g0 = (16 * ck) >> a.g_shift;
    const uint16_t* ksg = static_cast<const uint16_t*>(a.ks.data) + (int64_t)l * a.ks.sl + (int64_t)h * a.ks.sh + g0;
    const uint16_t* vsg = static_cast<const uint16_t*>(a.vs.data) + (int64_t)l * a.vs.sl + (int64_t)h * a.vs.sh + g0;

    struct Buf {
        uint2 kw, vw;
        uint16_t k0, k1, v0, v1;
    };
    // Pointers of this lane's token; a step advances them by TS tokens.
    struct Ptr {
        const uint8_t* k;
        const uint8_t* v;
        const uint16_t* ks;
        const uint16_t* vs;
    };
    auto at = [&](int t) {
        return Ptr{kcg + (int64_t)t * a.kc.st, vcg + (int64_t)t * a.vc.st, ksg + (int64_t)t * a.ks.st,
                   vsg + (int64_t)t * a.vs.st};
    };
    const int64_t dk = (int64_t)TS * a.kc.st, dv = (int64_t)TS * a.vc.st;
    const int64_t dks = (int64_t)TS * a.ks.st, dvs = (int64_t)TS * a.vs.st;
    auto load = [&](const Ptr& p, Buf& b) {
        b.kw = *reinterpret_cast<const uint2*>(p.k);
        b.vw = *reinterpret_cast<const uint2*>(p.v);
        b.k0 = p.ks[0];
        b.v0 = p.vs[0];
        if constexpr (SPLIT) {     // group 8: the lane's second 8 coordinates have their own scale
            b.k1 = p.ks[1];
            b.v1 = p.vs[1];
        } else {
            b.k1 = b.k0;
            b.v1 = b.v0;
        }
    };
    // advance by one step when `more` (a wave-uniform flag), else stay
    auto advance = [&](Ptr& p, bool more) {
        p.k += more ? dk : 0;
        p.v += more ? dv : 0;
        p.ks += more ? dks : 0;
        p.vs += more ? dvs : 0;
    };

    float m[RP], lsum[RP], acc[RP][16], vs0[RP], vs1[RP];
#pragma unroll
    for (int r = 0; r < RP; r++) {
        m[r] = -__builtin_inff();
        lsum[r] = 0.0f;
        vs0[r] = 0.0f;
        vs1[r] = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++) acc[r][i] = 0.0f;
    }

    // scores of one step (log2 domain); -inf for a slot without a token
    auto scores = [&](const Buf& b, bool valid, float (&s)[RP]) {
        float u[16];
        unpack16(b.kw, u);
        const float sk0 = (float)__builtin_bit_cast(_Float16, b.k0), sk1 = (float)__builtin_bit_cast(_Float16, b.k1);
#pragma unroll
        for (int r = 0; r < RP; r++) {
            float d0 = qs0[r], d1 = qs1[r];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                d0 = fmaf(qv[r][i], u[i], d0);
                d1 = fmaf(qv[r][8 + i], u[8 + i], d1);
            }
            s[r] = slot_sum<LPT>(fmaf(sk0, d0, sk1 * d1));
            s[r] = valid ? s[r] : -__builtin_inff();
        }
    };
    // online softmax: a new maximum rescales what the slot has so far
    auto rescale = [&](const float (&smax)[RP]) {
#pragma unroll
        for (int r = 0; r < RP; r++) {
            const float c = (smax[r] > m[r]) ? __builtin_amdgcn_exp2f(m[r] - smax[r]) : 1.0f;
            m[r] = fmaxf(m[r], smax[r]);
            lsum[r] *= c;
            vs0[r] *= c;
            vs1[r] *= c;
#pragma unroll
            for (int i = 0; i < 16; i++) acc[r][i] *= c;
        }
    };
    // weights and value accumulation of one step (after rescale)
    auto accumulate = [&](const Buf& b, const float (&s)[RP]) {
        float u[16];
        unpack16(b.vw, u);
        const float sv0 = (float)__builtin_bit_cast(_Float16, b.v0), sv1 = (float)__builtin_bit_cast(_Float16, b.v1);
#pragma unroll
        for (int r = 0; r < RP; r++) {
            // exp2(-inf) = 0 for a slot without a token (m is finite once any
            // token has been seen; before that every weight is 0 anyway)
            const float p = (s[r] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(s[r] - m[r]);
            lsum[r] += p;
            const float p0 = p * sv0, p1 = p * sv1;
            vs0[r] += p0;
            vs1[r] += p1;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                acc[r][i] = fmaf(p0, u[i], acc[r][i]);
                acc[r][8 + i] = fmaf(p1, u[8 + i], acc[r][8 + i]);
            }
        }
    };
    // two steps share one rescale
    auto pair = [&](const Buf& b0, const Buf& b1, bool valid1) {
        float s0[RP], s1[RP], sm[RP];
        scores(b0, true, s0);
        scores(b1, valid1, s1);
#pragma unroll
        for (int r = 0; r < RP; r++) sm[r] = fmaxf(s0[r], s1[r]);
        rescale(sm);
        accumulate(b0, s0);
        accumulate(b1, s1);
    };

    // ---- full steps in pairs, the next pair's loads in flight --------------
    if (nfull > 0) {
        Ptr p = at(wb + slot);
        Buf A, B, C, E;
        load(p, A);
        advance(p, 1 < nfull);
        load(p, B);
        for (int i = 0;; i += 4) {
            // a step past the last full step reloads the last one (in range)
            advance(p, i + 2 < nfull);
            load(p, C);
            advance(p, i + 3 < nfull);
            load(p, E);
            pair(A, B, i + 1 < nfull);
            if (i + 2 >= nfull) break;
            advance(p, i + 4 < nfull);
            load(p, A);
            advance(p, i + 5 < nfull);
            load(p, B);
            pair(C, E, i + 3 < nfull);
            if (i + 4 >= nfull) break;
        }
    }
    // ---- last, partial step: slots past the range read the first token ---
    if (rem > 0) {
        const bool valid = slot < rem;
        Buf b;
        load(at(valid ? wb + nfull * TS + slot : wb), b);
        float s1[RP];
        scores(b, valid, s1);
        rescale(s1);
        accumulate(b, s1);
    }

    // ---- write this slot's partial: [max, weight sum, 2 pad, acc[D]] -------
    const int part = (split * kAttnWaves + wid) * TS + slot;
#pragma unroll
    for (int r = 0; r < RP; r++) {
        if (r0 + r >= a.R) break;
        float* P = a.ws + ((((int64_t)lh * a.R + r0 + r) * a.parts) + part) * (D + 4);
        if (ck == 0) *reinterpret_cast<float2*>(P) = make_float2(m[r], lsum[r]);
        float o[16];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            o[i] = acc[r][i] - 8.0f * vs0[r];
            o[8 + i] = acc[r][8 + i] - 8.0f * vs1[r];
        }
#pragma unroll
        for (int i = 0; i < 16; i += 4)
            *reinterpret_cast<float4*>(P + 4 + 16 * ck + i) = make_float4(o[i], o[i + 1], o[i + 2], o[i + 3]);
    }
}

// ---------------------------------------------------------------------------
// Matrix-core partial kernel: head_dim 128 with groups of 32, head_dim 256
// with groups of 64
// ---------------------------------------------------------------------------
// Same query rotation, log2-domain online softmax and partial format as
// attend_partial_kernel, with both contractions on
// v_mfma_f32_16x16x32_f16 (A 16x32, B 32x16, fp32 accumulate; lane l holds
// A row l%16 / B column l%16 and k-slice l/16, eight k per slice; the result
// holds rows 4*(l/16)..+3 of column l%16).  A block is eight wavefronts: the
// KV heads of a head group times sub-ranges of one token split, so the heads
// that share cache lines read them together.  A wavefront takes 32 tokens
// per step and writes one partial.
//
// Codes enter both contractions as biased fp16 values, two per dword from one
// v_bitop3_b32 that masks two nibbles and, in the same operation, turns them
// to offset binary (c + 8) and ors in an fp16 exponent: nibbles in bits 0-3 of
// each half become the low mantissa bits of 1024.0 (value 1032 + c), nibbles
// in bits 4-7 those of 64.0 (value 72 + c).  Even coordinates take the first
// form and odd ones the second, so a dword of eight codes costs one shift and
// four v_bitop3_b32.  The constant parts are removed from the results: from
// each score through the accumulator's initial value, minus the bias-weighted
// group sum of the query; from each value row through a running sum of its
// weight operand (one more MFMA against a tile of ones), subtracted every
// eight steps so that the accumulators never carry more than eight steps of
// the large bias.  The biased operands are exact in fp16, so the results stay
// fp32 accurate.
//
// Scores.  Rows are 16 tokens; columns are (group g, query r) = 4r + g; the
// k-slice of lane row-slice sl is group sl, so B column (g, r) is the rotated
// query r restricted to group g (zero on the other slices) and the result is
// the per-group partial dot products, which the group scales then weight and
// a reduce-scatter over the quad of a query's four groups sums, leaving one
// token's score per lane for the softmax.  The query is split into fp16
// hi + lo halves (two MFMAs), so the dot products are fp32 accurate.  A
// lane's G/2 code bytes of group sl feed G/8 MFMAs, one dword each (four at
// head_dim 128, eight at 256).
//
// Values.  Rows are (group g', query r) = 4g' + r, k is the 32 tokens, and
// columns are coordinates: tile (h, m), column j is coordinate
// 128h + 8j + m (h = 0 only at head_dim 128).  A row (g', r) is
// p_r * vscale_g' over the tokens (hi + lo halves), so the result's row
// (g(c), r) is query r's weighted sum of coordinate c; the other rows are
// discarded.  A lane loads one dword (coordinates 128h + 8j .. + 7) of each of
// its slice's 8 tokens and regroups nibbles with v_perm.
//
// Within every 8-element operand the k order is (0,4,1,5,2,6,3,7), the order
// in which nibble pairs come out of a masked dword; A and B use the same order.
// Scores, weights and scales cross between the two layouts through small
// wave-private LDS tiles.
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kPermK[8] = {0, 4, 1, 5, 2, 6, 3, 7};

// fp16 operand words of the code nibbles (see above).  f(a, b, c) = (a & b) ^ c
// is truth table 0x6A of v_bitop3_b32; the xor flips the nibble's top bit
// (two's complement -> offset binary) and sets the exponent bits, which the
// mask has cleared.
constexpr uint32_t kMaskLo = 0x000F000Fu;     // nibbles in bits 0-3 of each half
constexpr uint32_t kMaskHi = 0x00F000F0u;     // nibbles in bits 4-7 of each half
constexpr uint32_t kXorLo = 0x64086408u;      // fp16 1024 | 8: value 1032 + c
constexpr uint32_t kXorHi = 0x54805480u;      // fp16 64 | 8 << 4: value 72 + c
constexpr float kBiasLo = 1032.0f, kBiasHi = 72.0f;

__device__ __forceinline__ uint32_t nib2(uint32_t x, uint32_t mask, uint32_t k)
{
    return __builtin_amdgcn_bitop3_b32(x, mask, k, (unsigned char)0x6A);
}

// Eight two's-complement codes of a dword (nibble e = element e) in the order
// (0,4,1,5,2,6,3,7): even elements as 1032 + c, odd ones as 72 + c.
__device__ __forceinline__ h8_t codes8(uint32_t w, uint32_t klo, uint32_t khi)
{
    const uint32_t y = w >> 8;
    const uint4 o = make_uint4(nib2(w, kMaskLo, klo), nib2(w, kMaskHi, khi), nib2(y, kMaskLo, klo),
                               nib2(y, kMaskHi, khi));
    return __builtin_bit_cast(h8_t, o);
}

// max(a, b) without the quieting copies the compiler adds to fmaxf for
// operands it cannot prove canonical (lane moves); scores are never NaN.
__device__ __forceinline__ float vmax(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// max over lanes l, l ^ 16, l ^ 32, l ^ 48 with the gfx950 lane swaps:
// v_permlane16_swap_b32 (x, y) returns rows (x0, y0, x2, y2) and (x1, y1, x3,
// y3), so with y = x the larger of the two is the pair max across l ^ 16;
// v_permlane32_swap_b32 does the same across halves.  The optimizer must not
// see that both operands are one value (it would take the two results as
// equal and drop the max).
__device__ __forceinline__ float vmax_xor16_32(float m)
{
    uint32_t a = __builtin_bit_cast(uint32_t, m), b = a;
    asm volatile("" : "+v"(b));
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    m = vmax(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
    a = __builtin_bit_cast(uint32_t, m);
    b = a;
    asm volatile("" : "+v"(b));
    const auto t = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    return vmax(__builtin_bit_cast(float, (uint32_t)t[0]), __builtin_bit_cast(float, (uint32_t)t[1]));
}

// max(v, v of lane l ^ 1) and max(v, v of lane l ^ 2): a DPP max; the s_nop
// covers the wait states a DPP read needs after a VALU write of its source.
__device__ __forceinline__ float vmax_xor1(float v)
{
    float r;
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1"
        : "=v"(r) : "v"(v));
    return r;
}
__device__ __forceinline__ float vmax_xor2(float v)
{
    float r;
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1"
        : "=v"(r) : "v"(v));
    return r;
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, h2_t{(_Float16)a, (_Float16)b});
}

}  // namespace

template <int D, int RP>
__device__ __forceinline__ void rotate_queries(const AttnArgs& a, int l, int h, int r0, int lane, float (&qt)[RP][D])
{
    constexpr int NJ = D / 32;
    constexpr int N = D / 4;
    const int qd = lane >> 2, qq = lane & 3;
    const int rr = min(qd, RP - 1);
    const int qi = min(r0 + rr, a.R - 1);
    const _Float16* qp = a.q + (((int64_t)l * a.H + h) * a.R + qi) * D;
    const float* lk = a.lam_k + ((int64_t)l * a.H + h) * D;
    float v[N];
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        const int c0 = 32 * j + 8 * qq;
        const uint4 qw = *reinterpret_cast<const uint4*>(qp + c0);
        const float4 l0 = *reinterpret_cast<const float4*>(lk + c0);
        const float4 l1 = *reinterpret_cast<const float4*>(lk + c0 + 4);
        const uint2 sg = *reinterpret_cast<const uint2*>(a.signs + c0);
        const uint32_t w[4] = {qw.x, qw.y, qw.z, qw.w};
        const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const uint32_t word = e < 4 ? sg.x : sg.y;
            const int sv = (int)(int8_t)((word >> (8 * (e & 3))) & 0xff);
            const float qv = (e & 1) ? hi_half(w[e / 2]) : lo_half(w[e / 2]);
            x[e] = (sv < 0 ? -qv : qv) / (lv[e] * SqrtD<D>::v);
        }
#pragma unroll
        for (int k = 0; k < 4; k++) {
            v[8 * j + 2 * k] = x[2 * k] + x[2 * k + 1];
            v[8 * j + 2 * k + 1] = x[2 * k] - x[2 * k + 1];
        }
    }
    fwht_rest(v, (qq & 1) ? -1.0f : 1.0f, (qq & 2) ? -1.0f : 1.0f);
    const float f = ((__builtin_popcount(qq) & 1) ? -1.0f : 1.0f) * a.qscale;
    if (qd < RP) {
#pragma unroll
        for (int j = 0; j < NJ; j++)
#pragma unroll
            for (int e = 0; e < 8; e++) qt[rr][32 * j + 8 * qq + e] = v[8 * j + e] * f;
    }
}

template <int D>
__global__ __launch_bounds__(64 * kAttnMfmaWaves) void attend_partial_mfma_kernel(AttnArgs a)
{
    // D = 128 with groups of 32 or D = 256 with groups of 64: four groups per
    // vector either way.  NM MFMAs of k = 32 per group, KW 16-byte code loads
    // per (token, group), NVD value dwords per (token, lane).
    constexpr int RP = 4, STEP = 32, W = kAttnMfmaWaves;
    constexpr int G = D / 4, NM = G / 8, KW = G / 32, NVD = D / 128;
    static_assert(D == 128 || D == 256, "head_dim 128 or 256");
    const int lane = threadIdx.x & 63;
    const int wid = uniform(threadIdx.x >> 6);
    // Block -> (outer index l, head group, split); wavefront -> (head of the
    // group, sub-range of the split).  The heads of a group read interleaved
    // rows of the same cache lines ([T, H, D/2] codes, [T, H, D/G] scales),
    // and its wavefronts walk the same tokens together, so each line is
    // fetched once.
    const int hb = a.hb, nsub = W / hb;
    int l, h, split, sub;
    {
        int b = blockIdx.x;
        split = b % a.S;
        b /= a.S;
        const int ng = a.H / hb;
        l = uniform(b / ng);
        h = uniform((b - l * ng) * hb + (wid & (hb - 1)));
        split = uniform(split);
        sub = uniform(wid / hb);
    }
    const int lh = l * a.H + h;
    const int r0 = blockIdx.y * RP;
    const int n = a.lengths ? min(max(a.lengths[l], 0), a.T) : a.T;

    __shared__ float qt[W][RP][D];
    rotate_queries<D, RP>(a, l, h, r0, lane, qt[wid]);
    __builtin_amdgcn_wave_barrier();

    const int j16 = lane & 15;   // MFMA row (A) / column (B, result)
    const int sl = lane >> 4;    // MFMA k-slice; result row block

    // The rotated queries enter the MFMAs as fp16 hi + lo halves, scaled by
    // 2^-qe so that the largest stays below 2^14 (qe = 0 unless the queries
    // are huge; the scaling is exact), and each score is multiplied back by
    // 2^qe.
    int qe;
    {
        float qm = 0.0f;
        const float* qf = &qt[wid][0][0] + (RP * D / 64) * lane;
#pragma unroll
        for (int i = 0; i < RP * D / 64; i++) qm = fmaxf(qm, fabsf(qf[i]));
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) qm = fmaxf(qm, __shfl_xor(qm, o));
        qe = uniform(qm > 0.0f ? max(0, ilogbf(qm) - 13) : 0);
    }
    const float sfac = ldexpf(1.0f, qe);

    // Score B operands of the wavefront's head: column (g, r) = 4r + g of
    // k-slice sl holds query r's coordinates of group g when g == sl, zeros
    // otherwise.  The 16 non-zero columns of each MFMA are kept in LDS,
    // [hi/lo][MFMA m][column], and read at each use; a lane whose column is
    // zero in its slice reads a block of zeros laid out the same way.
    __shared__ uint4 bqL[W][2][NM][16];
    __shared__ uint4 bqZero[2][NM][16];
    for (int i = threadIdx.x; i < 2 * NM * 16; i += 64 * W) (&bqZero[0][0][0])[i] = make_uint4(0, 0, 0, 0);
    const bool bq_on = (j16 & 3) == sl;
    if (bq_on) {
        const int r = j16 >> 2, g = j16 & 3;
#pragma unroll
        for (int m = 0; m < NM; m++) {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const float v0 = ldexpf(qt[wid][r][G * g + 8 * m + kPermK[2 * k]], -qe);
                const float v1 = ldexpf(qt[wid][r][G * g + 8 * m + kPermK[2 * k + 1]], -qe);
                const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
                hw[k] = __builtin_bit_cast(uint32_t, h2_t{h0, h1});
                lw[k] = pack_h2(v0 - (float)h0, v1 - (float)h1);
            }
            bqL[wid][0][m][j16] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            bqL[wid][1][m][j16] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
    }
    __syncthreads();     // the zero block is shared by the block's wavefronts
    const uint4* bqp = bq_on ? &bqL[wid][0][0][j16] : &bqZero[0][0][j16];

    // The codes enter the MFMAs biased (1032 + c at even coordinates, 72 + c
    // at odd ones): the score column (g, r) starts from minus the bias-weighted
    // sum of query r over group g, taken over the same fp16 hi + lo halves the
    // MFMAs multiply (their sum is exact in fp32).
    float kb;
    {
        const int r = j16 >> 2, g = j16 & 3;
        float sq = 0.0f;
#pragma unroll 8
        for (int c = 0; c < G; c++) {
            const float v = ldexpf(qt[wid][r][G * g + c], -qe);
            const _Float16 hv = (_Float16)v;
            const float q2 = (float)hv + (float)(_Float16)(v - (float)hv);
            sq = fmaf(q2, (c & 1) ? kBiasHi : kBiasLo, sq);
        }
        kb = sq;
    }
    // head_dim 128 starts the score accumulators at -kb; head_dim 256, short
    // of registers, starts them at zero and subtracts kb in the softmax
    const f4_t kinit = NVD == 1 ? f4_t{-kb, -kb, -kb, -kb} : f4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const float kb_late = NVD == 1 ? 0.0f : kb;

    // wave-private exchange tiles
    __shared__ _Float16 ksT[W][4][STEP], vsT[W][4][STEP];
    __shared__ float pL[W][RP][STEP];
    __shared__ float aL[W][RP];

    const int cb = split * a.chunk;
    const int ce = min(cb + a.chunk, n);
    const int per_wave = ((a.chunk + nsub * STEP - 1) / (nsub * STEP)) * STEP;
    const int wb = cb + sub * per_wave;
    const int we = min(wb + per_wave, ce);
    const int nsteps = we > wb ? (we - wb + STEP - 1) / STEP : 0;

    const uint8_t* kcg = static_cast<const uint8_t*>(a.kc.data) + (int64_t)l * a.kc.sl + (int64_t)h * a.kc.sh;
    const uint8_t* vcg = static_cast<const uint8_t*>(a.vc.data) + (int64_t)l * a.vc.sl + (int64_t)h * a.vc.sh;
    const uint16_t* ksg = static_cast<const uint16_t*>(a.ks.data) + (int64_t)l * a.ks.sl + (int64_t)h * a.ks.sh;
    const uint16_t* vsg = static_cast<const uint16_t*>(a.vs.data) + (int64_t)l * a.vs.sl + (int64_t)h * a.vs.sh;
    // Loads are split by what consumes them: the key codes of a step feed its
    // score MFMAs one step before its values and scales are needed.
    struct KBuf {
        uint4 k[2][KW];   // token 16 tau + j16, group sl: G codes
    };
    struct VBuf {
        uint32_t v[NVD][8];   // token 8 sl + t', coordinates 128 hv + 8 j16 .. + 7
        uint32_t ks, vs;      // token lane / 2, groups 2 (lane & 1), +1
    };
    // Loads are raw buffer loads: each stream's resource starts at the step's
    // first token (scalar arithmetic), each lane keeps one fixed 32-bit offset
    // per stream, and the per-load parts are scalar offsets, so a step's
    // addressing costs no vector instructions (the host guarantees 32 token
    // rows span less than 2^31 bytes).  In the wave's last step, rows past
    // its range are clamped to its last token, so every load stays in the
    // cache.
    const uint32_t kst = (uint32_t)a.kc.st, vst = (uint32_t)a.vc.st;
    const uint32_t kss = 2u * (uint32_t)a.ks.st, vss = 2u * (uint32_t)a.vs.st;
    constexpr int kRawBufferFlags = 0x00020000;     // gfx9 descriptor word 3 for raw dword access
    auto rsrc = [](const void* p) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, 0x7fffffff, kRawBufferFlags);
    };
    const uint32_t klane = (uint32_t)j16 * kst + 16u * (uint32_t)(KW * sl);
    const uint32_t vlane = (uint32_t)(8 * sl) * vst + 4u * (uint32_t)j16;
    const uint32_t kslane = (uint32_t)(lane >> 1) * kss + 4u * (uint32_t)(lane & 1);
    const uint32_t vslane = (uint32_t)(lane >> 1) * vss + 4u * (uint32_t)(lane & 1);
    auto load_k = [&](int step, KBuf& b) {
        const int tb = wb + step * STEP;
        const auto r = rsrc(kcg + (int64_t)tb * a.kc.st);
        if (tb + STEP > we) {
            const int lim = we - 1 - tb;
#pragma unroll
            for (int tau = 0; tau < 2; tau++)
#pragma unroll
                for (int kw = 0; kw < KW; kw++)
                    b.k[tau][kw] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                        r, (uint32_t)min(16 * tau + j16, lim) * kst + 16u * (uint32_t)(KW * sl + kw), 0, 0));
        } else {
#pragma unroll
            for (int tau = 0; tau < 2; tau++)
#pragma unroll
                for (int kw = 0; kw < KW; kw++)
                    b.k[tau][kw] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                        r, klane, 16u * (uint32_t)tau * kst + 16u * (uint32_t)kw, 0));
        }
    };
    auto load_v = [&](int step, VBuf& b) {
        const int tb = wb + step * STEP;
        const auto rv = rsrc(vcg + (int64_t)tb * a.vc.st);
        const auto rks = rsrc(ksg + (int64_t)tb * a.ks.st);
        const auto rvs = rsrc(vsg + (int64_t)tb * a.vs.st);
        if (tb + STEP > we) {
            const int lim = we - 1 - tb;
#pragma unroll
            for (int hv = 0; hv < NVD; hv++)
#pragma unroll
                for (int tp = 0; tp < 8; tp++)
                    b.v[hv][tp] = __builtin_amdgcn_raw_buffer_load_b32(
                        rv, (uint32_t)min(8 * sl + tp, lim) * vst + 4u * (uint32_t)j16 + 64u * (uint32_t)hv, 0, 0);
            const uint32_t ts = (uint32_t)min(lane >> 1, lim);
            b.ks = __builtin_amdgcn_raw_buffer_load_b32(rks, ts * kss + 4u * (uint32_t)(lane & 1), 0, 0);
            b.vs = __builtin_amdgcn_raw_buffer_load_b32(rvs, ts * vss + 4u * (uint32_t)(lane & 1), 0, 0);
        } else {
#pragma unroll
            for (int hv = 0; hv < NVD; hv++)
#pragma unroll
                for (int tp = 0; tp < 8; tp++)
                    b.v[hv][tp] = __builtin_amdgcn_raw_buffer_load_b32(rv, vlane, (uint32_t)tp * vst + 64u * (uint32_t)hv, 0);
            b.ks = __builtin_amdgcn_raw_buffer_load_b32(rks, kslane, 0, 0);
            b.vs = __builtin_amdgcn_raw_buffer_load_b32(rvs, vslane, 0, 0);
        }
    };

    uint32_t klo = kXorLo, khi = kXorHi;      // kept in VGPRs (v_bitop3_b32 takes one scalar)
    asm volatile("" : "+v"(klo), "+v"(khi));
    float m_run = -__builtin_inff();   // running max of query j16 & 3 (log2 domain)
    float l_run = 0.0f;                // this lane's share of the weight sum
    f4_t acc[NVD][8];
    f4_t wsum = f4_t{0.0f, 0.0f, 0.0f, 0.0f};   // rows' weight-operand sums since the last bias removal
#pragma unroll
    for (int hv = 0; hv < NVD; hv++)
#pragma unroll
        for (int mt = 0; mt < 8; mt++) acc[hv][mt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // value sums minus their code biases (tile mt holds coordinates of parity mt)
    auto remove_bias = [&]() {
#pragma unroll
        for (int hv = 0; hv < NVD; hv++)
#pragma unroll
            for (int mt = 0; mt < 8; mt++)
#pragma unroll
                for (int v = 0; v < 4; v++)
                    acc[hv][mt][v] = fmaf((mt & 1) ? -kBiasHi : -kBiasLo, wsum[v], acc[hv][mt][v]);
        wsum = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
    };

    // per-group partial scores of a step's 2 x 16 tokens
    auto scores = [&](const KBuf& b, f4_t (&c)[2]) {
#pragma unroll
        for (int tau = 0; tau < 2; tau++) {
            c[tau] = kinit;
#pragma unroll
            for (int kq = 0; kq < KW; kq++) {
                const uint32_t kw[4] = {b.k[tau][kq].x, b.k[tau][kq].y, b.k[tau][kq].z, b.k[tau][kq].w};
#pragma unroll
                for (int d = 0; d < 4; d++) {
                    const int m = 4 * kq + d;
                    const h8_t am = codes8(kw[d], klo, khi);
                    const h8_t bh = __builtin_bit_cast(h8_t, bqp[m * 16]);
                    const h8_t bl = __builtin_bit_cast(h8_t, bqp[(NM + m) * 16]);
                    c[tau] = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, bh, c[tau], 0, 0, 0);
                    c[tau] = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, bl, c[tau], 0, 0, 0);
                }
            }
        }
    };

    // The value operand of a step: A row (g', r') = (j16 >> 2, j16 & 3) holds
    // p * vscale of query r', group g' over tokens 8 sl + (0,4,1,5,...), as
    // fp16 hi and lo halves.
    struct PBuf {
        h8_t hi, lo;
    };
    const int gS = j16 & 3, rS = j16 >> 2;     // score column: group, query
    const int gV = j16 >> 2, rV = j16 & 3;     // value-operand row: group, query
    const bool h1 = (gS & 1) != 0, h2 = (gS & 2) != 0;
    // Softmax of a step from its partial scores, without branches: moves the
    // reference max when needed (l_run is rescaled here; the factor of each
    // query goes to aL for the accumulators, which the caller rescales when
    // the returned flag is set) and builds the step's value operand.  Tokens
    // at or past the wave's end, including every token of a step past the
    // last one, get weight 0 and leave the state unchanged.
    auto softmax = [&](int step, const VBuf& b, const f4_t (&c)[2], PBuf& pb) -> bool {
        const int tb = wb + step * STEP;
        // scale tiles, transposed to [group][token]
        {
            const int tl = lane >> 1, g0 = 2 * (lane & 1);
            ksT[wid][g0][tl] = __builtin_bit_cast(_Float16, (uint16_t)(b.ks & 0xffffu));
            ksT[wid][g0 + 1][tl] = __builtin_bit_cast(_Float16, (uint16_t)(b.ks >> 16));
            vsT[wid][g0][tl] = __builtin_bit_cast(_Float16, (uint16_t)(b.vs & 0xffffu));
            vsT[wid][g0 + 1][tl] = __builtin_bit_cast(_Float16, (uint16_t)(b.vs >> 16));
        }
        __builtin_amdgcn_wave_barrier();
        // Weight by the group scales and sum over the 4 groups, which are the
        // four lanes of a quad (columns 4r + g): a reduce-scatter leaves lane
        // g with the score of token 4 sl + g, so each lane carries on with
        // one score per 16 tokens.
        float sc[2];
#pragma unroll
        for (int tau = 0; tau < 2; tau++) {
            const uint2 kq = *reinterpret_cast<const uint2*>(&ksT[wid][gS][16 * tau + 4 * sl]);
            const h2_t k01 = __builtin_bit_cast(h2_t, kq.x), k23 = __builtin_bit_cast(h2_t, kq.y);
            float x[4];
            x[0] = fmaf(c[tau][0] - kb_late, (float)k01.x, 0.0f);
            x[1] = fmaf(c[tau][1] - kb_late, (float)k01.y, 0.0f);
            x[2] = fmaf(c[tau][2] - kb_late, (float)k23.x, 0.0f);
            x[3] = fmaf(c[tau][3] - kb_late, (float)k23.y, 0.0f);
            // keep tokens 2 (g >> 1) + {0, 1}, add the partner's (lane g ^ 2)
            const float y0 = (h2 ? x[2] : x[0]) + dpp_mov<kDppXor2>(h2 ? x[0] : x[2]);
            const float y1 = (h2 ? x[3] : x[1]) + dpp_mov<kDppXor2>(h2 ? x[1] : x[3]);
            // keep token g, add lane g ^ 1's
            const float sv = ((h1 ? y1 : y0) + dpp_mov<kDppXor1>(h1 ? y0 : y1)) * sfac;
            sc[tau] = tb + 16 * tau + 4 * sl + gS < we ? sv : -__builtin_inff();
        }
        float smax = vmax(sc[0], sc[1]);
        smax = vmax_xor1(smax);
        smax = vmax_xor2(smax);
        smax = vmax_xor16_32(smax);
        // The weights are taken relative to a reference max that moves only
        // when a score exceeds it by more than 2^8 (weights stay below 256),
        // so the accumulators are rescaled a few times per wave rather than
        // every step.  The value operand p * vscale must stay finite in fp16:
        // in a step with a value scale of 128 (0x5800) or more the reference
        // moves to the step's max, so that p <= 1.  Adding 0x2800 to each
        // magnitude half carries into its bit 15 exactly when it is >= 0x5800.
        const bool big = __builtin_amdgcn_ballot_w64((((b.vs & 0x7fff7fffu) + 0x28002800u) & 0x80008000u) != 0) != 0;
        const bool moved = __builtin_amdgcn_ballot_w64(smax > m_run + (big ? 0.0f : 8.0f)) != 0;
        const float m_new = moved ? fmaxf(m_run, smax) : m_run;
        const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
        aL[wid][rS] = alpha;    // the 16 lanes of a query store the same value
        // m_run is finite here for a step in range (every such step has a
        // token in range for each query), so a masked score gives
        // exp2(-inf) = 0; a step past the end leaves m_run as it was
#pragma unroll
        for (int tau = 0; tau < 2; tau++) {
            const float pv = __builtin_amdgcn_exp2f(sc[tau] - m_run);
            l_run += pv;
            pL[wid][rS][16 * tau + 4 * sl + gS] = pv;
        }
        __builtin_amdgcn_wave_barrier();
        {
            const float4 p0 = *reinterpret_cast<const float4*>(&pL[wid][rV][8 * sl]);
            const float4 p1 = *reinterpret_cast<const float4*>(&pL[wid][rV][8 * sl + 4]);
            const uint4 vq = *reinterpret_cast<const uint4*>(&vsT[wid][gV][8 * sl]);
            const float pp[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            const h2_t v2[4] = {__builtin_bit_cast(h2_t, vq.x), __builtin_bit_cast(h2_t, vq.y),
                                __builtin_bit_cast(h2_t, vq.z), __builtin_bit_cast(h2_t, vq.w)};
            const _Float16 vv[8] = {v2[0].x, v2[0].y, v2[1].x, v2[1].y, v2[2].x, v2[2].y, v2[3].x, v2[3].y};
            h2_t hw[4], lw[4];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                // fp16 hi and lo halves of p * vscale (tokens k and k + 4)
                const _Float16 e0 = (_Float16)fmaf(pp[k], (float)vv[k], 0.0f);
                const _Float16 e1 = (_Float16)fmaf(pp[k + 4], (float)vv[k + 4], 0.0f);
                hw[k] = h2_t{e0, e1};
                lw[k] = h2_t{(_Float16)fmaf(pp[k], (float)vv[k], -(float)e0),
                             (_Float16)fmaf(pp[k + 4], (float)vv[k + 4], -(float)e1)};
            }
            pb.hi = __builtin_bit_cast(h8_t, hw);
            pb.lo = __builtin_bit_cast(h8_t, lw);
        }
        return moved;
    };
    // the accumulators follow a moved reference: row 4 sl + v is query v
    auto rescale = [&]() {
        __builtin_amdgcn_wave_barrier();
        const float4 al = *reinterpret_cast<const float4*>(&aL[wid][0]);
        const float av[4] = {al.x, al.y, al.z, al.w};
#pragma unroll
        for (int v = 0; v < 4; v++) wsum[v] *= av[v];
#pragma unroll
        for (int hv = 0; hv < NVD; hv++)
#pragma unroll
            for (int mt = 0; mt < 8; mt++)
#pragma unroll
                for (int v = 0; v < 4; v++) acc[hv][mt][v] *= av[v];
    };
    // value B operands of tile (hv, 2 q' / 2 q' + 1) from byte q' of the 8
    // tokens' dwords of part hv
    auto value_operands = [&](const VBuf& b, int hv, h8_t (&bv)[8]) {
#pragma unroll
        for (int qb = 0; qb < 4; qb++) {
            const uint32_t sel = (uint32_t)qb | (0x0cu << 8) | ((uint32_t)(4 + qb) << 16) | (0x0cu << 24);
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint32_t w = __builtin_amdgcn_perm(b.v[hv][k + 4], b.v[hv][k], sel);
                lo[k] = nib2(w, kMaskLo, klo);
                hi[k] = nib2(w, kMaskHi, khi);
            }
            bv[2 * qb] = __builtin_bit_cast(h8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
            bv[2 * qb + 1] = __builtin_bit_cast(h8_t, make_uint4(hi[0], hi[1], hi[2], hi[3]));
        }
    };
    auto accumulate = [&](const PBuf& pb, int hv, const h8_t (&bv)[8]) {
        if (hv == 0) {
            const h8_t ones = __builtin_bit_cast(h8_t, make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));
            wsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(pb.hi, ones, wsum, 0, 0, 0);
            wsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(pb.lo, ones, wsum, 0, 0, 0);
        }
#pragma unroll
        for (int mt = 0; mt < 8; mt++) {
            acc[hv][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pb.hi, bv[mt], acc[hv][mt], 0, 0, 0);
            acc[hv][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pb.lo, bv[mt], acc[hv][mt], 0, 0, 0);
        }
    };

    // The two wavefronts that share a SIMD (w and w + 4) trade the higher
    // issue priority every 16 steps.  Otherwise the older one of each pair
    // runs ahead for the whole range, and the block's wavefronts, which read
    // interleaved parts of the same lines (the scale rows hold every head's
    // scales), drift apart by more than the lines stay in L2: 8-9% of the
    // bytes were fetched twice.  Trading priority keeps the drift bounded.
    auto share_issue = [&](int st) {
        if ((((st >> 4) & 1) ^ ((wid >> 2) & 1)) != 0) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
    };
    if (nsteps > 0) {
        if constexpr (NVD == 1) {
            // Software pipeline over two steps: one iteration converts step
            // st's value codes and issues its value MFMAs while the softmax of
            // step st + 1 runs on the VALU and the score MFMAs of step st + 2
            // run; the values of step st + 2 and the keys of step st + 3 are
            // in flight.  The accumulators take step st + 1's rescale after
            // step st's values.  Steps past the last one repeat its data (in
            // range) and are masked by the softmax.
            KBuf Ka, Kb;
            VBuf Va, Vb;
            f4_t ca[2], cb[2];
            PBuf Pa, Pb;
            const int last = nsteps - 1;
            load_k(0, Ka);
            load_v(0, Va);
            load_k(min(1, last), Kb);
            load_v(min(1, last), Vb);
            scores(Ka, ca);
            load_k(min(2, last), Ka);
            scores(Kb, cb);
            softmax(0, Va, ca, Pa);     // the accumulators are still zero
            for (int st = 0;; st += 2) {
                share_issue(st);
                h8_t bv[8];
                value_operands(Va, 0, bv);
                load_v(min(st + 2, last), Va);
                load_k(min(st + 3, last), Kb);
                scores(Ka, ca);
                bool moved = softmax(st + 1, Vb, cb, Pb);
                accumulate(Pa, 0, bv);
                if ((st & 7) == 7) remove_bias();
                if (st + 1 >= nsteps) break;
                if (moved) rescale();
                value_operands(Vb, 0, bv);
                load_v(min(st + 3, last), Vb);
                load_k(min(st + 4, last), Ka);
                scores(Kb, cb);
                moved = softmax(st + 2, Va, ca, Pa);
                accumulate(Pb, 0, bv);
                if (((st + 1) & 7) == 7) remove_bias();
                if (st + 2 >= nsteps) break;
                if (moved) rescale();
            }
        } else {
            // head_dim 256: the values of step st + 1 and keys of step st + 2
            // are in flight and the score MFMAs of step st + 1 run while step
            // st is finished (the registers hold no more)
            KBuf K;
            VBuf V0, V1;
            f4_t c0[2], c1[2];
            PBuf P;
            auto finish = [&](int step, const VBuf& b, const f4_t (&c)[2]) {
                if (softmax(step, b, c, P)) rescale();
                h8_t ones = __builtin_bit_cast(h8_t, make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));
                asm volatile("" : "+v"(ones));
                wsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(P.hi, ones, wsum, 0, 0, 0);
                wsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(P.lo, ones, wsum, 0, 0, 0);
                // each pair of value tiles is built right before its MFMAs
#pragma unroll
                for (int hv = 0; hv < NVD; hv++) {
#pragma unroll
                    for (int qb = 0; qb < 4; qb++) {
                        const uint32_t sel = (uint32_t)qb | (0x0cu << 8) | ((uint32_t)(4 + qb) << 16) | (0x0cu << 24);
                        uint32_t lo[4], hi[4];
#pragma unroll
                        for (int k = 0; k < 4; k++) {
                            const uint32_t w = __builtin_amdgcn_perm(b.v[hv][k + 4], b.v[hv][k], sel);
                            lo[k] = nib2(w, kMaskLo, klo);
                            hi[k] = nib2(w, kMaskHi, khi);
                        }
                        const h8_t bl = __builtin_bit_cast(h8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
                        const h8_t bh = __builtin_bit_cast(h8_t, make_uint4(hi[0], hi[1], hi[2], hi[3]));
                        f4_t& a0 = acc[hv][2 * qb];
                        f4_t& a1 = acc[hv][2 * qb + 1];
                        a0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(P.hi, bl, a0, 0, 0, 0);
                        a0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(P.lo, bl, a0, 0, 0, 0);
                        a1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(P.hi, bh, a1, 0, 0, 0);
                        a1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(P.lo, bh, a1, 0, 0, 0);
                    }
                }
                if ((step & 7) == 7) remove_bias();
            };
            load_k(0, K);
            load_v(0, V0);
            scores(K, c0);
            load_k(min(1, nsteps - 1), K);
            for (int st = 0;; st += 2) {
                share_issue(st);
                load_v(min(st + 1, nsteps - 1), V1);
                scores(K, c1);
                load_k(min(st + 2, nsteps - 1), K);
                finish(st, V0, c0);
                if (st + 1 >= nsteps) break;
                load_v(min(st + 2, nsteps - 1), V0);
                scores(K, c0);
                load_k(min(st + 3, nsteps - 1), K);
                finish(st + 1, V1, c1);
                if (st + 2 >= nsteps) break;
            }
        }
    }

    // ---- partial: one per wavefront ------------------------------------------
    l_run += dpp_mov<kDppXor1>(l_run);
    l_run += dpp_mov<kDppXor2>(l_run);
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    const int part0 = split * nsub + sub;
    const int nr = min(RP, a.R - r0);
    {
        const int rS = j16 >> 2, gS = j16 & 3;     // score-column lanes hold query rS's state
        if (gS == 0 && sl == 0 && rS < nr) {
            float* P = a.ws + ((((int64_t)lh * a.R + r0 + rS) * a.parts) + part0) * (D + 4);
            *reinterpret_cast<float2*>(P) = make_float2(m_run, l_run);
        }
    }
    // result rows 4 sl + v = (group sl, query v); column j16 of tile (hv, mt)
    // is coordinate 128 hv + 8 j16 + mt, of group (128 hv + 8 j16) / G.
    remove_bias();
#pragma unroll
    for (int hv = 0; hv < NVD; hv++) {
        if (sl == (128 * hv + 8 * j16) / G) {
#pragma unroll
            for (int v = 0; v < RP; v++) {
                if (v >= nr) break;
                float* P = a.ws + ((((int64_t)lh * a.R + r0 + v) * a.parts) + part0) * (D + 4) + 4 + 128 * hv + 8 * j16;
                *reinterpret_cast<float4*>(P) =
                    make_float4(acc[hv][0][v], acc[hv][1][v], acc[hv][2][v], acc[hv][3][v]);
                *reinterpret_cast<float4*>(P + 4) =
                    make_float4(acc[hv][4][v], acc[hv][5][v], acc[hv][6][v], acc[hv][7][v]);
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(64 * kAttnWaves) void attend_combine_kernel(AttnArgs a)
{
    constexpr int NJ = D / 32;
    constexpr int N = D / 4;
    const int lane = threadIdx.x & 63;
    const int q = lane & 3;
    const int64_t nvec = (int64_t)a.L * a.H * a.R;
    const int64_t vraw = ((int64_t)blockIdx.x * kAttnWaves + (threadIdx.x >> 6)) * 16 + (lane >> 2);
    const bool live = vraw < nvec;
    const int64_t vec = live ? vraw : nvec - 1;
    const int l = (int)(vec / ((int64_t)a.H * a.R));
    const int rest = (int)(vec - (int64_t)l * a.H * a.R);
    const int h = rest / a.R;
    const int r = rest - h * a.R;
    const float* P = a.ws + (((int64_t)l * a.H + h) * a.R + r) * a.parts * (D + 4);

    // merge the partials: running max M, weight sum L, value sum y (lane's
    // coordinates 32 j + 8 q + e)
    float M = -__builtin_inff(), Ls = 0.0f, y[N];
#pragma unroll
    for (int i = 0; i < N; i++) y[i] = 0.0f;
    for (int p = 0; p < a.parts; p++, P += D + 4) {
        const float2 ml = *reinterpret_cast<const float2*>(P);
        if (ml.x == -__builtin_inff()) continue;
        if (ml.x > M) {
            const float c = exp2f(M - ml.x);
            Ls *= c;
#pragma unroll
            for (int i = 0; i < N; i++) y[i] *= c;
            M = ml.x;
        }
        const float w = exp2f(ml.x - M);
        Ls = fmaf(w, ml.y, Ls);
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const float4 a0 = *reinterpret_cast<const float4*>(P + 4 + 32 * j + 8 * q);
            const float4 a1 = *reinterpret_cast<const float4*>(P + 4 + 32 * j + 8 * q + 4);
            const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
            for (int e = 0; e < 8; e++) y[8 * j + e] = fmaf(w, av[e], y[8 * j + e]);
        }
    }
    const float inv = (Ls > 0.0f) ? 1.0f / Ls : 0.0f;

    // inverse rotation and unscale: x = s / (lambda_V sqrt(D)) * H (y / L)
    float v[N];
#pragma unroll
    for (int k = 0; k < N; k += 2) {
        v[k] = (y[k] + y[k + 1]) * inv;
        v[k + 1] = (y[k] - y[k + 1]) * inv;
    }
    fwht_rest(v, (q & 1) ? -1.0f : 1.0f, (q & 2) ? -1.0f : 1.0f);
    float mi[N];
    load_inv_mult<D>(a.lam_v + ((int64_t)l * a.H + h) * D, a.signs, q,
                     (__builtin_popcount(q) & 1) ? -1.0f : 1.0f, mi);
    if (live) {
        _Float16* o = a.out + vec * D;
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            uint4 w;
            w.x = pack_half2(v[8 * j + 0] * mi[8 * j + 0], v[8 * j + 1] * mi[8 * j + 1]);
            w.y = pack_half2(v[8 * j + 2] * mi[8 * j + 2], v[8 * j + 3] * mi[8 * j + 3]);
            w.z = pack_half2(v[8 * j + 4] * mi[8 * j + 4], v[8 * j + 5] * mi[8 * j + 5]);
            w.w = pack_half2(v[8 * j + 6] * mi[8 * j + 6], v[8 * j + 7] * mi[8 * j + 7]);
            *reinterpret_cast<uint4*>(o + 32 * j + 8 * q) = w;
        }
    }
}

namespace {

template <int D, int RP>
hipError_t launch_part(const AttnArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)((int64_t)a.L * a.H * a.S), (unsigned)((a.R + RP - 1) / RP));
    if constexpr (D == 128 || D == 256) {
        if (a.mfma) {
            const dim3 mgrid((unsigned)((int64_t)a.L * (a.H / a.hb) * a.S), (unsigned)((a.R + 3) / 4));
            hipLaunchKernelGGL((attend_partial_mfma_kernel<D>), mgrid, dim3(64 * kAttnMfmaWaves), 0, s, a);
            return hipGetLastError();
        }
    }
    if (a.g_shift == 3) hipLaunchKernelGGL((attend_partial_kernel<D, RP, true>), grid, dim3(64 * kAttnWaves), 0, s, a);
    else hipLaunchKernelGGL((attend_partial_kernel<D, RP, false>), grid, dim3(64 * kAttnWaves), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t s)
{
    hipError_t e;
    if (a.rp == 1) e = launch_part<D, 1>(a, s);
    else if (a.rp == 2) e = launch_part<D, 2>(a, s);
    else e = launch_part<D, 4>(a, s);
    if (e != hipSuccess) return e;
    const int64_t nvec = (int64_t)a.L * a.H * a.R;
    const dim3 grid((unsigned)((nvec + 16 * kAttnWaves - 1) / (16 * kAttnWaves)));
    hipLaunchKernelGGL((attend_combine_kernel<D>), grid, dim3(64 * kAttnWaves), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_decode(const AttnArgs& a, hipStream_t s)
{
    switch (a.D) {
        case 64: return launch_d<64>(a, s);
        case 128: return launch_d<128>(a, s);
        case 256: return launch_d<256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
