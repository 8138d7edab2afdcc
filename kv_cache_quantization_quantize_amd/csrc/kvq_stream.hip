// kvq_stream.hip -- streaming kernels that measure the practical HBM
// bandwidth of the GPU for the read/write mixes of the quantizer's kernels
// (libkvq_stream.so, loaded only by the benchmark).
//
// A work unit is RD 16-byte chunks read and WR 16-byte chunks written: a
// wavefront reads 64*RD contiguous chunks (lane l takes chunks l, l+64, ..)
// and writes 64*WR contiguous chunks the same way, so every instruction
// moves 1 KB of consecutive bytes, as the product kernels' stores do.  The
// written values depend on every loaded value (an xor), so no load can be
// dropped.  With no writes the wavefront xors its loads into one dword per
// lane, stored only if it equals a key the data never produces.  NT: the
// loads and stores carry the nontemporal hint.  Units per wavefront: runs of
// consecutive units, like the quantizer's items.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <bool NT>
__device__ __forceinline__ uint4 ld(const uint4* p)
{
    if constexpr (NT) {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}

template <bool NT>
__device__ __forceinline__ void st(uint4* p, uint4 v)
{
    if constexpr (NT) {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(u4{v.x, v.y, v.z, v.w}, reinterpret_cast<u4*>(p));
    } else {
        *p = v;
    }
}

template <int RD, int WR, bool NT>
__global__ __launch_bounds__(256) void stream_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                     int64_t n_units, int units_per_wave, uint32_t key,
                                                     uint32_t* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t u0 = wave * units_per_wave;
    const int64_t u1 = u0 + units_per_wave < n_units ? u0 + units_per_wave : n_units;
    uint32_t acc = 0;
    for (int64_t u = u0; u < u1; ++u) {
        uint4 r[RD];
#pragma unroll
        for (int k = 0; k < RD; k++) r[k] = ld<NT>(src + u * 64 * RD + k * 64 + lane);
        uint4 x = r[0];
#pragma unroll
        for (int k = 1; k < RD; k++) {
            x.x ^= r[k].x;
            x.y ^= r[k].y;
            x.z ^= r[k].z;
            x.w ^= r[k].w;
        }
        if constexpr (WR > 0) {
#pragma unroll
            for (int k = 0; k < WR; k++)
                st<NT>(dst + u * 64 * WR + k * 64 + lane, make_uint4(x.x + k, x.y, x.z, x.w));
        } else {
            acc ^= x.x ^ x.y ^ x.z ^ x.w;
        }
    }
    if constexpr (WR == 0)
        if (acc == key) sink[lane] = acc;
}

template <int RD, int WR>
hipError_t launch(const void* src, void* dst, int64_t n_units, int units_per_wave, int nt, uint32_t* sink,
                  hipStream_t s)
{
    const int64_t waves = (n_units + units_per_wave - 1) / units_per_wave;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (nt)
        hipLaunchKernelGGL((stream_kernel<RD, WR, true>), grid, block, 0, s, static_cast<const uint4*>(src),
                           static_cast<uint4*>(dst), n_units, units_per_wave, 0x9E3779B9u, sink);
    else
        hipLaunchKernelGGL((stream_kernel<RD, WR, false>), grid, block, 0, s, static_cast<const uint4*>(src),
                           static_cast<uint4*>(dst), n_units, units_per_wave, 0x9E3779B9u, sink);
    return hipGetLastError();
}

}  // namespace

extern "C" {

// mode 0: read only (4 chunks per lane and unit); 1: 4 read, 1 written (80/20,
// the quantizer's mix); 2: 1 read, 4 written (20/80, the dequantizer's);
// 3: 1 read, 1 written (copy).  src must hold n_units * 64 * RD chunks and
// dst n_units * 64 * WR; sink at least 64 dwords.  Returns a hipError_t.
int kvq_stream_run(int mode, const void* src, void* dst, int64_t n_units, int units_per_wave, int nontemporal,
                   void* sink, void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t* sk = static_cast<uint32_t*>(sink);
    if (n_units <= 0 || units_per_wave <= 0) return (int)hipErrorInvalidValue;
    switch (mode) {
        case 0: return (int)launch<4, 0>(src, dst, n_units, units_per_wave, nontemporal, sk, s);
        case 1: return (int)launch<4, 1>(src, dst, n_units, units_per_wave, nontemporal, sk, s);
        case 2: return (int)launch<1, 4>(src, dst, n_units, units_per_wave, nontemporal, sk, s);
        case 3: return (int)launch<1, 1>(src, dst, n_units, units_per_wave, nontemporal, sk, s);
        default: return (int)hipErrorInvalidValue;
    }
}

}  // extern "C"
