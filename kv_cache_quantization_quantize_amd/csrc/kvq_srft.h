// kvq_srft.h -- the sign-randomized real Fourier rotation (SRFT) in the
// quad-per-vector register layout of the int4 kernels.
//
// The rotation (gist.science explanation of arXiv 2605.05699, "Methodologie"
// s.1 and s.2): y = pack(F diag(s) diag(lambda) x), F the unitary DFT of
// length D, and pack keeps one copy of each conjugate pair of the real
// input's spectrum as [X_0, X_{D/2}, sqrt2 Re X_1, sqrt2 Im X_1, ...], which
// is an orthonormal map.  As in that kernel, the length-D real transform is a
// length-N = D/2 complex FFT of z_m = v_2m + i v_2m+1 (radix-2 stages),
// followed by the Hermitian unpacking that turns it into X_0 .. X_{D/2}.
//
// Layout.  Lane q of a quad holds real coordinates c = 32j + 8q + e (the
// int4 kernels' layout), i.e. the complex points m = 16j + 4q + f with
// f = e / 2.  A lane's P = D/8 complex values sit in c[0, P) (real parts)
// and c[P, 2P) (imaginary parts), index i = 4j + f.
//
// FFT.  Decimation in time needs its input in bit-reversed order; the quad
// writes its points to a wave-private LDS row in natural order and reads them
// back bit-reversed (the only data movement through memory).  Stages on the
// point-index bits held in registers (bits 0-1: f, bits 4..: j) are plain
// butterflies with twiddles; the two stages on lane bits (2-3: q) use one
// v_fmac_f32 with a DPP quad_perm source per value, as the Walsh-Hadamard
// code does: each lane first multiplies its own value by the twiddle if it is
// the upper element of its pair (1 otherwise), then v <- partner * c + v with
// c = -1 on the upper lane, so that the upper lane holds minus its true
// value.  After both lane stages every lane's values carry the sign
// sigma(q) = (-1)^popcount(q), which the consumers fold into their per-lane
// multipliers exactly as for the Walsh-Hadamard transform.  The FFT output
// is in natural order.
//
// Hermitian unpacking needs Z_{N-k} next to Z_k.  For k = 16j + 4q + f the
// partner N - k sits in lane 3 - q, register (NJ-1-j, 4-f) when f != 0, and
// for f = 0 in lane (4 - q) mod 4, register (NJ-1-j, 0), or (NJ - j) mod NJ
// for q = 0: both are quad permutations of a fixed register (DPP), plus one
// select for the q = 0 lane.  Lanes 1 and 3 exchange f = 0 partners with a
// lane of the other sign, which one multiply by -1 corrects.
//
// Twiddles that depend only on register indices are compile-time constants
// (a constexpr sin/cos of 2 pi t / n: range reduction to a quarter turn and
// a 14-term Taylor series in double, rounded once to float); those that also
// depend on the lane are one of four such constants, selected by q.
#pragma once

#include <type_traits>

#include "kvq_device.h"

namespace kvq {
namespace srft {

constexpr double kPi = 3.14159265358979323846;

constexpr double sin_taylor(double x)
{
    double t = x, s = x;
    for (int i = 1; i < 14; i++) {
        t *= -x * x / ((2.0 * i) * (2.0 * i + 1.0));
        s += t;
    }
    return s;
}

constexpr double cos_taylor(double x)
{
    double t = 1.0, s = 1.0;
    for (int i = 1; i < 14; i++) {
        t *= -x * x / ((2.0 * i - 1.0) * (2.0 * i));
        s += t;
    }
    return s;
}

// cos and sin of 2 pi t / n for integers t, n > 0.
constexpr double cos2pi(long t, long n)
{
    t %= n;
    if (t < 0) t += n;
    const long quarter = (4 * t) / n;
    const double x = (double)(4 * t - quarter * n) / (double)n * (kPi / 2);   // [0, pi/2)
    const double s = sin_taylor(x), c = cos_taylor(x);
    return quarter == 0 ? c : quarter == 1 ? -s : quarter == 2 ? -c : s;
}
constexpr double sin2pi(long t, long n)
{
    t %= n;
    if (t < 0) t += n;
    const long quarter = (4 * t) / n;
    const double x = (double)(4 * t - quarter * n) / (double)n * (kPi / 2);
    const double s = sin_taylor(x), c = cos_taylor(x);
    return quarter == 0 ? s : quarter == 1 ? c : quarter == 2 ? -s : -c;
}

template <int I, int E, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (I < E) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, E>(f);
    }
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

constexpr int bitrev(int x, int bits)
{
    int r = 0;
    for (int i = 0; i < bits; i++) r |= ((x >> i) & 1) << (bits - 1 - i);
    return r;
}

// One of four compile-time constants, by lane.
__device__ __forceinline__ float by_lane(int q, float a0, float a1, float a2, float a3)
{
    const float lo = (q & 1) ? a1 : a0;
    const float hi = (q & 1) ? a3 : a2;
    return (q & 2) ? hi : lo;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    // every lane has a source under a quad permutation, so no old value is
    // needed (an old operand of 0 would cost a v_mov per use)
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
constexpr int kQuadReverse = 0x1b;    // quad_perm [3, 2, 1, 0]
constexpr int kQuadNegate = 0x6c;     // quad_perm [0, 3, 2, 1]: lane (4 - q) mod 4

// (xr, xi) *= (wr, wi)
__device__ __forceinline__ void cmul(float& xr, float& xi, float wr, float wi)
{
    const float r = fmaf(xr, wr, -xi * wi);
    xi = fmaf(xr, wi, xi * wr);
    xr = r;
}

// (xr, xi) *= SIGN * i where `on`, else unchanged: a select per part, exact.
template <int SIGN>
__device__ __forceinline__ void times_i_where(float& xr, float& xi, bool on)
{
    const float r = on ? (SIGN < 0 ? xi : -xi) : xr;
    const float i = on ? (SIGN < 0 ? -xr : xr) : xi;
    xr = r;
    xi = i;
}

// Natural order -> bit-reversed order through the quad's LDS row (N entries).
template <int D>
__device__ __forceinline__ void to_bit_reversed(float (&c)[D / 4], float2* row, int q)
{
    constexpr int P = D / 8, LOGN = ilog2(D / 2);
#pragma unroll
    for (int i = 0; i < P; i++) row[16 * (i / 4) + 4 * q + (i % 4)] = make_float2(c[i], c[P + i]);
    // bit-reversal of p = 16j + 4q + f: the lane bits 2, 3 land on bits
    // LOGN-3, LOGN-4 and the register bits elsewhere
    const int lane_off = ((q & 1) << (LOGN - 3)) | ((q >> 1) << (LOGN - 4));
    static_for<0, P>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        constexpr int reg = bitrev(16 * (i / 4) + (i % 4), LOGN);
        const float2 t = row[reg | lane_off];
        c[i] = t.x;
        c[P + i] = t.y;
    });
}

// The lane-dependent twiddles of the FFT stages, computed once per kernel
// and kept in registers (they depend only on the lane and on compile-time
// register indices): the two lane-bit stages' factors (1 on the lower lane of
// a pair) and the register-bit stages' twiddles omega^((f + 16 (j mod hj))
// step + 4 q step).  SIGN as in fft_dit.
template <int D, int SIGN>
struct Tw {
    static constexpr int N = D / 2, LOGN = ilog2(N);
    static constexpr int NJT = LOGN > 4 ? 4 * ((1 << (LOGN - 4)) - 1) : 0;
    float l0r[2], l0i[2];            // lane bit 0 stage, f = 1 and 3
    float l1r[3], l1i[3];            // lane bit 1 stage, f = 1..3
    float jr[NJT > 0 ? NJT : 1], ji[NJT > 0 ? NJT : 1];
};

// the first twiddle of register-bit stage b in Tw::jr / Tw::ji
constexpr int tw_j_base(int b) { return 4 * ((1 << (b - 4)) - 1); }

template <int D, int SIGN>
__device__ __forceinline__ Tw<D, SIGN> make_twiddles(int q)
{
    using T = Tw<D, SIGN>;
    constexpr int N = T::N, LOGN = T::LOGN;
    T t;
    const bool up0 = (q & 1) != 0, up1 = (q & 2) != 0, odd = (q & 1) != 0;
    // f = 2 of the lane bit 0 stage and f = 0 of the lane bit 1 stage
    // multiply by SIGN * i or 1 (times_i_where), so they need no registers
    static_for<0, 2>([&](auto kk) {
        constexpr int e = (2 * decltype(kk)::value + 1) * (N / 8);
        t.l0r[decltype(kk)::value] = up0 ? (float)cos2pi(e, N) : 1.0f;
        t.l0i[decltype(kk)::value] = up0 ? (float)(SIGN * sin2pi(e, N)) : 0.0f;
    });
    static_for<1, 4>([&](auto kk) {
        constexpr int k = decltype(kk)::value;
        constexpr int e0 = k * (N / 16), e1 = (k + 4) * (N / 16);
        t.l1r[k - 1] = up1 ? (odd ? (float)cos2pi(e1, N) : (float)cos2pi(e0, N)) : 1.0f;
        t.l1i[k - 1] = up1 ? (odd ? (float)(SIGN * sin2pi(e1, N)) : (float)(SIGN * sin2pi(e0, N))) : 0.0f;
    });
    static_for<4, LOGN>([&](auto bb) {
        constexpr int b = decltype(bb)::value;
        constexpr int hj = 1 << (b - 4);
        constexpr int step = N >> (b + 1);
        const float lr = by_lane(q, 1.0f, (float)cos2pi(4 * step, N), (float)cos2pi(8 * step, N),
                                 (float)cos2pi(12 * step, N));
        const float li = by_lane(q, 0.0f, (float)(SIGN * sin2pi(4 * step, N)), (float)(SIGN * sin2pi(8 * step, N)),
                                 (float)(SIGN * sin2pi(12 * step, N)));
        static_for<0, 4 * hj>([&](auto xx) {
            constexpr int x = decltype(xx)::value;
            constexpr int e = (x % 4 + 16 * (x / 4)) * step;
            const float cr = (float)cos2pi(e, N), ci = (float)(SIGN * sin2pi(e, N));
            t.jr[tw_j_base(b) + x] = fmaf(lr, cr, -li * ci);
            t.ji[tw_j_base(b) + x] = fmaf(lr, ci, li * cr);
        });
    });
    // opaque to the optimiser, so that the values stay in registers across
    // the caller's loop instead of being rebuilt from constants per use
#pragma unroll
    for (int k = 0; k < 2; k++) asm volatile("" : "+v"(t.l0r[k]), "+v"(t.l0i[k]));
#pragma unroll
    for (int k = 0; k < 3; k++) asm volatile("" : "+v"(t.l1r[k]), "+v"(t.l1i[k]));
#pragma unroll
    for (int k = 0; k < T::NJT; k++) asm volatile("" : "+v"(t.jr[k]), "+v"(t.ji[k]));
    return t;
}

// Radix-2 decimation-in-time FFT of N = D/2 points held by a quad, from
// bit-reversed order to natural order, times sigma(q).  SIGN = -1: forward
// (omega = exp(-2 pi i / N)); +1: inverse without the 1/N.
template <int D, int SIGN>
__device__ __forceinline__ void fft_dit(float (&c)[D / 4], int q, const Tw<D, SIGN>& tw)
{
    constexpr int P = D / 8, N = D / 2, NJ = D / 32, LOGN = ilog2(N);
    // stage on point bit 0 (f bit 0): twiddle 1
#pragma unroll
    for (int i = 0; i < P; i += 2) {
        const float ar = c[i], ai = c[P + i], br = c[i + 1], bi = c[P + i + 1];
        c[i] = ar + br; c[P + i] = ai + bi;
        c[i + 1] = ar - br; c[P + i + 1] = ai - bi;
    }
    // point bit 1 (f bit 1): twiddle 1 for f = 0, SIGN * i for f = 1
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        {
            const int a = 4 * j, b = 4 * j + 2;
            const float ar = c[a], ai = c[P + a], br = c[b], bi = c[P + b];
            c[a] = ar + br; c[P + a] = ai + bi;
            c[b] = ar - br; c[P + b] = ai - bi;
        }
        {
            const int a = 4 * j + 1, b = 4 * j + 3;
            // t = (SIGN i) * x_b = (-SIGN xi, SIGN xr)
            const float tr = -SIGN * c[P + b], ti = SIGN * c[b];
            const float ar = c[a], ai = c[P + a];
            c[a] = ar + tr; c[P + a] = ai + ti;
            c[b] = ar - tr; c[P + b] = ai - ti;
        }
    }
    // point bit 2 (lane bit 0): upper lanes (q & 1) multiply by omega^(f N/8);
    // omega^(N/4) = SIGN i
    {
        static_for<0, P>([&](auto ii) {
            constexpr int i = decltype(ii)::value;
            if constexpr (i % 4 == 2) times_i_where<SIGN>(c[i], c[P + i], (q & 1) != 0);
            else if constexpr (i % 4 != 0) cmul(c[i], c[P + i], tw.l0r[i % 4 / 2], tw.l0i[i % 4 / 2]);
        });
        bfly_quad1(c, (q & 1) ? -1.0f : 1.0f);
    }
    // point bit 3 (lane bit 1): upper lanes (q & 2) multiply by
    // omega^((f + 4 (q & 1)) N / 16), which for f = 0 is 1 or SIGN i
    {
        static_for<0, P>([&](auto ii) {
            constexpr int i = decltype(ii)::value;
            if constexpr (i % 4 == 0) times_i_where<SIGN>(c[i], c[P + i], q == 3);
            else cmul(c[i], c[P + i], tw.l1r[i % 4 - 1], tw.l1i[i % 4 - 1]);
        });
        bfly_quad2(c, (q & 2) ? -1.0f : 1.0f);
    }
    // point bits 4 .. LOGN-1 (register j bits)
    static_for<4, LOGN>([&](auto bb) {
        constexpr int b = decltype(bb)::value;
        constexpr int hj = 1 << (b - 4);          // pair distance in j
        // twiddle omega^((f + 16 (j mod hj)) step + 4 q step), step = N / 2^(b+1)
        static_for<0, P>([&](auto ii) {
            constexpr int i = decltype(ii)::value;
            constexpr int j = i / 4, f = i % 4;
            if constexpr ((j & hj) == 0) {
                // a + w b by two fmas per part, then a - w b = 2a - (a + w b):
                // six operations instead of a complex multiply and four adds
                constexpr int ib = i + 4 * hj;
                constexpr int x = tw_j_base(b) + f + 4 * (j % hj);
                const float wr = tw.jr[x], wi = tw.ji[x];
                const float ar = c[i], ai = c[P + i], br = c[ib], bi = c[P + ib];
                const float yr = fmaf(-wi, bi, fmaf(wr, br, ar));
                const float yi = fmaf(wi, br, fmaf(wr, bi, ai));
                c[i] = yr; c[P + i] = yi;
                c[ib] = fmaf(2.0f, ar, -yr); c[P + ib] = fmaf(2.0f, ai, -yi);
            }
        });
    });
}

// Fetch, for every register i of this lane (point k = 16j + 4q + f), the
// value of point N - k from the quad (both parts).  For values carrying
// sigma(q), the f = 0 partners of lanes 1 and 3 come from a lane of the other
// sign: the caller multiplies them by -1 there.
template <int D>
__device__ __forceinline__ void hermitian_partners(const float (&c)[D / 4], float (&pc)[D / 4], int q)
{
    constexpr int P = D / 8, NJ = D / 32;
    const bool q0 = q == 0;
    static_for<0, P>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        constexpr int j = i / 4, f = i % 4;
        if constexpr (f != 0) {
            constexpr int src = 4 * (NJ - 1 - j) + (4 - f);
            pc[i] = dpp<kQuadReverse>(c[src]);
            pc[P + i] = dpp<kQuadReverse>(c[P + src]);
        } else {
            constexpr int s1 = 4 * (NJ - 1 - j), s0 = 4 * ((NJ - j) % NJ);
            const float r1 = dpp<kQuadNegate>(c[s1]), i1 = dpp<kQuadNegate>(c[P + s1]);
            const float r0 = dpp<kQuadNegate>(c[s0]), i0 = dpp<kQuadNegate>(c[P + s0]);
            pc[i] = q0 ? r0 : r1;
            pc[P + i] = q0 ? i0 : i1;
        }
    });
}

// cos and sin of 2 pi k / D for k = 16j + 4q + f (register i = 4j + f), times `scale`.
template <int D, int I>
__device__ __forceinline__ void unpack_twiddle(int q, float scale, float& cw, float& sw)
{
    constexpr int j = I / 4, f = I % 4;
    constexpr int e = 16 * j + f;
    const float lc = by_lane(q, 1.0f, (float)cos2pi(4, D), (float)cos2pi(8, D), (float)cos2pi(12, D));
    const float ls = by_lane(q, 0.0f, (float)sin2pi(4, D), (float)sin2pi(8, D), (float)sin2pi(12, D));
    const float cc = (float)cos2pi(e, D) * scale, cs = (float)sin2pi(e, D) * scale;
    cw = fmaf(cc, lc, -cs * ls);
    sw = fmaf(cs, lc, cc * ls);
}

// The forward transform's twiddles as a table row in LDS: the FFT twiddles
// of Tw (l0, l1, j), then the Hermitian unpacking's (cos, sin) pair of every
// register.  A wavefront keeps one row per quad lane q, and the quantizer
// reads its row back per item instead of holding 50 values in registers
// across items: that takes the head_dim-128 SRFT quantizer from 201 to 153
// VGPRs, three wavefronts per SIMD instead of two.  (At head_dim 256 it
// would go from 326 to 232 VGPRs, two wavefronts instead of one, but
// measured 2.5% slower; that quantizer keeps its twiddles in registers.)
template <int D>
struct TwRow {
    using T = Tw<D, -1>;
    static constexpr int L0 = 0, L1 = 2, J = 5, U = 5 + T::NJT, N = U + D / 8;
};

template <int D>
__device__ __forceinline__ void write_twiddle_row(float2* row, int q)
{
    using R = TwRow<D>;
    const Tw<D, -1> t = make_twiddles<D, -1>(q);
#pragma unroll
    for (int k = 0; k < 2; k++) row[R::L0 + k] = make_float2(t.l0r[k], t.l0i[k]);
#pragma unroll
    for (int k = 0; k < 3; k++) row[R::L1 + k] = make_float2(t.l1r[k], t.l1i[k]);
#pragma unroll
    for (int k = 0; k < Tw<D, -1>::NJT; k++) row[R::J + k] = make_float2(t.jr[k], t.ji[k]);
    static_for<0, D / 8>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        float cw, sw;
        unpack_twiddle<D, i>(q, 1.0f, cw, sw);
        row[R::U + i] = make_float2(cw, sw);
    });
}

template <int D>
__device__ __forceinline__ Tw<D, -1> read_twiddles(const float2* row)
{
    using R = TwRow<D>;
    Tw<D, -1> t;
#pragma unroll
    for (int k = 0; k < 2; k++) { const float2 w = row[R::L0 + k]; t.l0r[k] = w.x; t.l0i[k] = w.y; }
#pragma unroll
    for (int k = 0; k < 3; k++) { const float2 w = row[R::L1 + k]; t.l1r[k] = w.x; t.l1i[k] = w.y; }
#pragma unroll
    for (int k = 0; k < Tw<D, -1>::NJT; k++) { const float2 w = row[R::J + k]; t.jr[k] = w.x; t.ji[k] = w.y; }
    return t;
}

// Forward SRFT of the quad's vector, in place on v (natural layout, values
// already multiplied by s * lambda / sqrt(D), and by 1/sqrt2, which the
// unpacking's weights would otherwise apply): afterwards v holds y times
// sigma(q).  row: the quad's LDS row of N float2; tw: the FFT twiddles;
// utw(integral_constant i): the unpacking's (cos, sin) pair of register i.
template <int D, typename UnpackTw>
__device__ __forceinline__ void forward(float (&v)[D / 4], float2* row, int q, const Tw<D, -1>& tw,
                                        UnpackTw&& utw)
{
    constexpr int P = D / 8;
    float c[D / 4];
#pragma unroll
    for (int i = 0; i < P; i++) {
        c[i] = v[8 * (i / 4) + 2 * (i % 4)];
        c[P + i] = v[8 * (i / 4) + 2 * (i % 4) + 1];
    }
    to_bit_reversed<D>(c, row, q);
    fft_dit<D, -1>(c, q, tw);
    float pc[D / 4];
    hermitian_partners<D>(c, pc, q);
    const float fix = (q & 1) ? -1.0f : 1.0f;      // f = 0 partners' sign
    constexpr float sqrt2 = 1.41421356237309504880f;
    static_for<0, P>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        const float2 u = utw(ii);
        const float cw = u.x, sw = u.y;
        const float a = c[i], b = c[P + i], cc = pc[i], d = pc[P + i];
        float s1, d1, s2, d2;
        if constexpr (i % 4 == 0) {
            s1 = fmaf(fix, cc, a); d1 = fmaf(-fix, cc, a);
            s2 = fmaf(fix, d, b); d2 = fmaf(-fix, d, b);
        } else {
            s1 = a + cc; d1 = a - cc; s2 = b + d; d2 = b - d;
        }
        float y0 = fmaf(cw, s2, fmaf(-sw, d1, s1));
        float y1 = fmaf(-cw, d1, fmaf(-sw, s2, d2));
        if constexpr (i == 0) {
            // k = 0 (lane 0): X_0 and X_{D/2} are real, from Z_0 alone
            if (q == 0) {
                y0 = (a + b) * sqrt2;
                y1 = (a - b) * sqrt2;
            }
        }
        v[8 * (i / 4) + 2 * (i % 4)] = y0;
        v[8 * (i / 4) + 2 * (i % 4) + 1] = y1;
    });
}

// forward with every twiddle held in registers (tw built once per kernel)
template <int D>
__device__ __forceinline__ void forward(float (&v)[D / 4], float2* row, int q, const Tw<D, -1>& tw)
{
    forward<D>(v, row, q, tw, [&](auto ii) {
        float cw, sw;
        unpack_twiddle<D, decltype(ii)::value>(q, 1.0f, cw, sw);
        return make_float2(cw, sw);
    });
}

// forward with the twiddles read from the lane's LDS row (TwRow)
template <int D>
__device__ __forceinline__ void forward(float (&v)[D / 4], float2* row, int q, const float2* twrow)
{
    forward<D>(v, row, q, read_twiddles<D>(twrow),
               [&](auto ii) { return twrow[TwRow<D>::U + decltype(ii)::value]; });
}

// Inverse SRFT of the quad's vector, in place on v (natural layout, true
// rotated-domain values): afterwards v holds sqrt(2 D) times the unscaled
// vector s * lambda * xhat, times sigma(q); the consumer multiplies by
// s / (lambda sqrt(2 D)) and sigma(q).
template <int D>
__device__ __forceinline__ void inverse(float (&v)[D / 4], float2* row, int q, const Tw<D, 1>& tw)
{
    constexpr int P = D / 8;
    float y[D / 4];
#pragma unroll
    for (int i = 0; i < P; i++) {
        y[i] = v[8 * (i / 4) + 2 * (i % 4)];
        y[P + i] = v[8 * (i / 4) + 2 * (i % 4) + 1];
    }
    float py[D / 4];
    hermitian_partners<D>(y, py, q);
    constexpr float sqrt2 = 1.41421356237309504880f;
    float c[D / 4];
    static_for<0, P>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        float cw, sw;
        unpack_twiddle<D, i>(q, 1.0f, cw, sw);
        const float p = y[i], rr = y[P + i], u = py[i], w = py[P + i];
        const float sp = p + u, dp = p - u, sr = rr + w, dr = rr - w;
        float zr = fmaf(-sw, dp, fmaf(-cw, sr, sp));
        float zi = fmaf(cw, dp, fmaf(-sw, sr, dr));
        if constexpr (i == 0) {
            if (q == 0) {
                zr = (p + rr) * sqrt2;
                zi = (p - rr) * sqrt2;
            }
        }
        c[i] = zr;
        c[P + i] = zi;
    });
    to_bit_reversed<D>(c, row, q);
    fft_dit<D, 1>(c, q, tw);
#pragma unroll
    for (int i = 0; i < P; i++) {
        v[8 * (i / 4) + 2 * (i % 4)] = c[i];
        v[8 * (i / 4) + 2 * (i % 4) + 1] = c[P + i];
    }
}

}  // namespace srft
}  // namespace kvq
