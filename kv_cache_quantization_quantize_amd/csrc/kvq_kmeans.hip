// kvq_kmeans.hip -- codebook training for the product VQ: the update half of
// one Lloyd (k-means) iteration on gfx950 (MI355X).
//
// The method (VecInfer blog, "What VecInfer does, and the calibration caveat
// up front"): codebooks are trained k-means style on synthetic samples shaped
// like the keys and values.  One iteration assigns every rotated sub-vector to
// its nearest centroid -- the product-VQ encoder does that, writing the
// assignments -- and then moves each centroid to the mean of the sub-vectors
// assigned to it; a centroid with none keeps its place.
//
// Accumulate.  The training vectors of one head (all layers) are cut into
// ranges of (layer, 16-token tile) rows; two blocks per (head, range), one
// for coordinates 0-3 and one for 4-7 of the sub-vectors, rotate the range's
// vectors exactly as the encoder does (4 lanes per vector, Walsh-Hadamard in
// registers), read each sub-vector's assignment and add its coordinates into
// per-centroid sums in LDS, plus a count (first block only).  The sums are
// fixed point: each coordinate is rounded to a multiple of 2^-24 and added
// as a 64-bit integer with ds_add_u64 (4 x 8 bytes per centroid and block,
// at most 4096 centroids: 128 KB, with the counts 144 KB).  Integer LDS
// atomics cost about 13 cycles per wavefront instruction on this GPU against
// about 200 for ds_add_f32, and integer sums are exact, so the result does
// not depend on the order of the additions.  The sums are stored
// coordinate-major, [4][K]: the 64 lanes of one atomic instruction add
// coordinate e of their own centroids, which spread over the banks.  Each
// block writes its sums (and counts) to the range's workspace slot.  As in
// the decoder, the H blocks of one range are dispatched to the same XCD (and
// the two blocks of a (head, range) one after the other) so that shared
// cache lines are fetched from HBM once.
//
// Finalize.  One thread per (head, centroid) adds the ranges' integer sums
// (exact), scales to fp64, divides by the count and rounds the mean to fp16
// (round to odd into fp32, then round to nearest even into fp16, which is the
// correctly rounded fp16 of the fp64 mean).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

template <int D>
struct KmCfg {
    static constexpr int WAVES = (D == 256) ? 8 : 16;
};

// round(y * 2^24) as a 64-bit integer, exactly (|y| < 2^23): the product is
// exact, its part above 2^16 converts through a truncation, and the
// remainder below 2^16 is exact in fp32 and rounds to nearest even.
__device__ __forceinline__ int64_t to_fixed24(float y)
{
    const float t = y * 16777216.0f;
    const float th = __builtin_truncf(t * (1.0f / 65536.0f));
    const float tl = fmaf(th, -65536.0f, t);
    return (int64_t)(int32_t)th * 65536 + (int64_t)(int32_t)__builtin_rintf(tl);
}

// fp64 -> fp16 with one rounding: round to odd into fp32 (24 significant
// bits, more than 11 + 2), then the hardware's round to nearest even.
__device__ __forceinline__ uint16_t f64_to_f16_bits(double d)
{
    float f = (float)d;
    if ((double)f != d && !__builtin_isinf(f)) {
        uint32_t u = __float_as_uint(f);
        if (!(u & 1u)) u = (fabs(d) > fabs((double)f)) ? u + 1 : u - 1;
        f = __uint_as_float(u);
    }
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

}  // namespace

template <int D>
__global__ __launch_bounds__(64 * KmCfg<D>::WAVES) void kmeans_accum_kernel(KmArgs a)
{
    constexpr int WAVES = KmCfg<D>::WAVES;
    constexpr int NJ = D / 32;
    constexpr int N = D / 4;

    __shared__ unsigned long long sums[4 * kKmMaxCentroids];   // [4][K], fixed point
    __shared__ uint32_t cnts[kKmMaxCentroids];

    const int lane = threadIdx.x & 63;
    const int q = lane & 3;
    const int slot = lane >> 2;
    const int wid = uniform(threadIdx.x >> 6);
    const float c1 = (q & 1) ? -1.0f : 1.0f;
    const float c2 = (q & 2) ? -1.0f : 1.0f;
    const float lane_sign = (__builtin_popcount(q) & 1) ? -1.0f : 1.0f;
    const uint32_t kmax = (uint32_t)(a.K - 1);

    // block b runs on XCD b % 8; coordinate half (b / 8) % 2, head
    // (b / 16) % H, range ((b / 16) / H) * 8 + b % 8
    const int xcd = blockIdx.x & 7;
    const int half = (blockIdx.x >> 3) & 1;
    const int kx = blockIdx.x >> 4;
    const int grp = kx / a.H;
    const int h = kx - grp * a.H;
    const int range = grp * 8 + xcd;
    const int ranges = 8 * a.range_groups;
    const int64_t rows = (int64_t)a.L * a.tiles;
    const int64_t r0 = (int64_t)range * a.rows_per_range;
    const int64_t r1 = min(r0 + a.rows_per_range, rows);

    for (int i = threadIdx.x; i < a.K * 4; i += 64 * WAVES) sums[i] = 0ull;
    for (int i = threadIdx.x; i < a.K; i += 64 * WAVES) cnts[i] = 0u;
    __syncthreads();

    const _Float16* __restrict__ xg = static_cast<const _Float16*>(a.x.data);
    const uint16_t* __restrict__ ig = static_cast<const uint16_t*>(a.idx.data);
    int cur_l = -1;
    float m[N];
    for (int64_t g = r0 + wid; g < r1; g += WAVES) {
        const int l = uniform((int)(g / a.tiles));
        const int tile = (int)(g - (int64_t)l * a.tiles);
        if (l != cur_l) {
            load_fwd_mult<D>(a.lambda + ((int64_t)l * a.H + h) * D, a.signs, q, m);
            cur_l = l;
        }
        // a quad's four lanes share one token; tokens past the end load the
        // last token and add nothing
        const int t = tile * kTokensPerTile + slot;
        const bool valid = t < a.T;
        const int tl = min(t, a.T - 1);
        const _Float16* p = xg + (int64_t)l * a.x.sl + (int64_t)h * a.x.sh + (int64_t)tl * a.x.st + q * 8;
        const uint16_t* ip = ig + (int64_t)l * a.idx.sl + (int64_t)h * a.idx.sh + (int64_t)tl * a.idx.st;
        uint4 raw[NJ];
        uint32_t kk[NJ];
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            raw[j] = *reinterpret_cast<const uint4*>(p + j * 32);
            kk[j] = min((uint32_t)ip[4 * j + q], kmax);        // lane q holds sub-vectors 4j + q
        }
        float v[N];
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const int r = j * 8 + 2 * k;
                const float b = fmaf(hi_half(w[k]), m[r + 1], 0.0f);
                v[r] = fmaf(lo_half(w[k]), m[r], b);
                v[r + 1] = fmaf(lo_half(w[k]), m[r], -b);
            }
        }
        fwht_rest(v, c1, c2);
        if (valid) {
#pragma unroll
            for (int j = 0; j < NJ; j++) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    // coordinate 4 half + e of the sub-vector (half is wave-uniform)
                    const float y = (half ? v[j * 8 + 4 + e] : v[j * 8 + e]) * lane_sign;
                    atomicAdd(sums + e * a.K + kk[j], (unsigned long long)to_fixed24(y));
                }
                if (half == 0) atomicAdd(cnts + kk[j], 1u);
            }
        }
    }
    __syncthreads();

    const int64_t slot_base = (int64_t)h * ranges + range;
    int64_t* ps = a.part_sums + (slot_base * 8 + 4 * half) * a.K;
    for (int i = threadIdx.x; i < a.K * 4; i += 64 * WAVES) ps[i] = (int64_t)sums[i];
    if (half == 0) {
        uint32_t* pc = a.part_counts + slot_base * a.K;
        for (int i = threadIdx.x; i < a.K; i += 64 * WAVES) pc[i] = cnts[i];
    }
}

__global__ __launch_bounds__(256) void kmeans_finalize_kernel(KmArgs a)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (head, centroid)
    if (i >= (int64_t)a.H * a.K) return;
    const int h = (int)(i / a.K);
    const int k = (int)(i - (int64_t)h * a.K);
    const int ranges = 8 * a.range_groups;
    int64_t si[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint64_t n = 0;
    for (int r = 0; r < ranges; r++) {
        const int64_t sl = (int64_t)h * ranges + r;
        const int64_t* ps = a.part_sums + sl * a.K * 8 + k;   // [8][K] per slot
#pragma unroll
        for (int e = 0; e < 8; e++) si[e] += ps[(int64_t)e * a.K];
        n += a.part_counts[sl * a.K + k];
    }
    double s[8];
#pragma unroll
    for (int e = 0; e < 8; e++) s[e] = (double)si[e] * (1.0 / 16777216.0);
    a.counts[i] = (uint32_t)n;
    uint4 o;
    if (n == 0) {
        o = *reinterpret_cast<const uint4*>(a.codebook + i * 8);
    } else {
        const double dn = (double)n;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; e++)
            w[e] = (uint32_t)f64_to_f16_bits(s[2 * e] / dn) | ((uint32_t)f64_to_f16_bits(s[2 * e + 1] / dn) << 16);
        o = make_uint4(w[0], w[1], w[2], w[3]);
    }
    *reinterpret_cast<uint4*>(a.new_codebook + i * 8) = o;
}

namespace {

template <int D>
hipError_t launch_km(const KmArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)(16 * a.H * a.range_groups));
    hipLaunchKernelGGL((kmeans_accum_kernel<D>), grid, dim3(64 * KmCfg<D>::WAVES), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)a.H * a.K;
    hipLaunchKernelGGL(kmeans_finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kmeans_update(const KmArgs& a, hipStream_t s)
{
    switch (a.D) {
        case 64: return launch_km<64>(a, s);
        case 128: return launch_km<128>(a, s);
        case 256: return launch_km<256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
