// kvq_api.cpp -- the C ABI of libkvq.so: host-side validation, work
// decomposition and kernel dispatch.  Validation makes no HIP call, so every
// error path can be exercised on a machine without a GPU.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "../../include/kvq.h"
#include "kvq_internal.h"

namespace {

thread_local char g_err[512];

kvq_status fail(kvq_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

bool aligned(const void* p, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

kvq_status check_shape(const kvq_shape& s)
{
    if (s.layers < 0 || s.tokens < 0 || s.heads < 0)
        return fail(KVQ_ERR_SHAPE, "negative size: layers=%lld tokens=%lld heads=%lld",
                    (long long)s.layers, (long long)s.tokens, (long long)s.heads);
    if (s.head_dim != 64 && s.head_dim != 128 && s.head_dim != 256)
        return fail(KVQ_ERR_UNSUPPORTED, "head_dim=%lld; supported: 64, 128, 256", (long long)s.head_dim);
    if (s.layers > INT32_MAX || s.tokens > INT32_MAX || s.heads > INT32_MAX)
        return fail(KVQ_ERR_SHAPE, "a dimension exceeds 2^31-1");
    const int64_t tiles = (s.tokens + kvq::kTokensPerTile - 1) / kvq::kTokensPerTile;
    // items = layers*heads*tiles must stay below 2^31 (with room for one more wave's run)
    if (s.layers > 0 && s.heads > 0 && tiles > 0 &&
        (double)s.layers * (double)s.heads * (double)tiles > (double)(INT32_MAX - 1024))
        return fail(KVQ_ERR_SHAPE, "layers*heads*ceil(tokens/16) exceeds 2^31");
    return KVQ_OK;
}

bool empty(const kvq_shape& s) { return s.layers == 0 || s.tokens == 0 || s.heads == 0; }

// A view whose rows are `row_bytes` long and must be `align`-byte aligned.
kvq_status check_view(const char* name, const kvq_view& v, int elem_bytes, int64_t row_elems,
                      int align, const kvq_shape& s)
{
    if (!v.data) return fail(KVQ_ERR_NULL, "%s.data is NULL", name);
    if (!aligned(v.data, align))
        return fail(KVQ_ERR_ALIGN, "%s.data must be %d-byte aligned", name, align);
    const int64_t st[3] = {v.stride_layer, v.stride_token, v.stride_head};
    const char* sn[3] = {"stride_layer", "stride_token", "stride_head"};
    const int64_t ext[3] = {s.layers, s.tokens, s.heads};
    for (int i = 0; i < 3; i++) {
        if (st[i] < 0) return fail(KVQ_ERR_SHAPE, "%s.%s is negative", name, sn[i]);
        if ((st[i] * elem_bytes) % align)
            return fail(KVQ_ERR_ALIGN, "%s.%s*%d bytes must be a multiple of %d", name, sn[i], elem_bytes, align);
        if (ext[i] > 1 && st[i] < row_elems && st[i] != 0)
            return fail(KVQ_ERR_SHAPE, "%s.%s=%lld is smaller than a row (%lld elements)", name, sn[i],
                        (long long)st[i], (long long)row_elems);
        if (ext[i] > 1 && st[i] == 0)
            return fail(KVQ_ERR_SHAPE, "%s.%s is 0 for an extent > 1 (outputs would alias)", name, sn[i]);
    }
    return KVQ_OK;
}

kvq_status check_group(int32_t g, int64_t D)
{
    if (g < 8 || g > D || (g & (g - 1)))
        return fail(KVQ_ERR_UNSUPPORTED, "group=%d; must be a power of two with 8 <= group <= head_dim (%lld)",
                    g, (long long)D);
    return KVQ_OK;
}

kvq_status check_params(const float* lambda, const int8_t* signs)
{
    if (!lambda) return fail(KVQ_ERR_NULL, "lambda is NULL");
    if (!signs) return fail(KVQ_ERR_NULL, "signs is NULL");
    if (!aligned(lambda, 16)) return fail(KVQ_ERR_ALIGN, "lambda must be 16-byte aligned");
    if (!aligned(signs, 8)) return fail(KVQ_ERR_ALIGN, "signs must be 8-byte aligned");
    return KVQ_OK;
}

kvq::Tensor4 t4(const kvq_view& v) { return kvq::Tensor4{v.data, v.stride_layer, v.stride_token, v.stride_head}; }

// Consecutive items per wavefront: about 2048 wavefronts (half of what the
// 256 CUs hold at once) for small launches, so that every wavefront runs
// several items and overlaps the next item's loads with the current item's
// work; for large launches at most `cap` per wavefront.  Measured on MI355X
// (19 GB Qwen3-8B-shaped tensors, head_dim 128): the Walsh-Hadamard
// quantizers are fastest with runs of 2 (4.96 -> 4.55 ms against 16; short
// runs keep more loads in flight across the chip, and their per-wavefront
// set-up is a few multiplies), while the dequantizers and the SRFT kernels,
// whose set-up (reciprocal multipliers, twiddles) costs more, are fastest
// with 16 (2 costs 47% more); the head_dim-256 quantizer with 8.  The Qwen2.5-1.5B-shaped K cache dequantize went from
// 38.6 to 28.4 us against one item per wavefront.
int32_t items_per_wave(int64_t n_items, int64_t cap = 16)
{
    int64_t ipw = (n_items + 2047) / 2048;
    if (ipw < 1) ipw = 1;
    if (ipw > cap) ipw = cap;
    return (int32_t)ipw;
}

// Run cap of the quantize / dequantize kernels (see items_per_wave).
int64_t int4_run_cap(int64_t D, bool inverse, bool fourier)
{
    if (inverse || fourier) return 16;
    return D <= 128 ? 2 : 8;
}

// Work items of the 4-lanes-per-vector kernels: token-major (16 consecutive
// (token, head) vectors of a layer) when the head count (above one) divides
// 16, else head-major (16 consecutive tokens of one (layer, head)).  With one
// head both orders give the same items; the head-major kernels keep fewer
// per-lane store offsets (at head_dim 256: 230 VGPRs with the next item's
// loads prefetched, against 268 token-major, which would halve the waves per
// SIMD).  Measured on MI355X, [26, 262144, 1, 256] with groups of 64:
// dequantize 1.047 -> 0.921 ms, quantize 0.894 -> 0.866 ms.
void set_items(const kvq_shape& s, int32_t& token_major, int32_t& h_shift, int32_t& items_per_group,
               int32_t& tok_per_item, int32_t& ipw, int64_t& n_items, int64_t cap = 16)
{
    token_major = s.heads > 1 && (kvq::kTokensPerTile % s.heads) == 0;
    h_shift = 0;
    while ((int64_t(1) << h_shift) < s.heads) h_shift++;
    if (token_major) {
        tok_per_item = (int32_t)(kvq::kTokensPerTile / s.heads);
        items_per_group = (int32_t)((s.tokens + tok_per_item - 1) / tok_per_item);
        n_items = s.layers * (int64_t)items_per_group;
    } else {
        tok_per_item = kvq::kTokensPerTile;
        items_per_group = (int32_t)((s.tokens + kvq::kTokensPerTile - 1) / kvq::kTokensPerTile);
        n_items = s.layers * s.heads * (int64_t)items_per_group;
    }
    ipw = items_per_wave(n_items, cap);
}

// Compute units of the current device (cached per device).
int device_cus()
{
    static thread_local int cached_dev = -1, cached_cus = 256;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return cached_cus;
    if (dev != cached_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            cached_cus = cus;
        cached_dev = dev;
    }
    return cached_cus;
}

kvq_status hip_status(hipError_t e, const char* what)
{
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return KVQ_OK;
}

#define KVQ_TRY(expr)                          \
    do {                                       \
        kvq_status _st = (expr);               \
        if (_st != KVQ_OK) return _st;         \
    } while (0)

kvq_status int4_common(const kvq_shape& shape, const kvq_view& x, const float* lambda,
                       const int8_t* signs, int32_t group, const kvq_view& codes,
                       const kvq_view& scales, kvq::Int4Args& a, bool x_is_output, int bits = 4,
                       bool mx = false, bool fourier = false)
{
    KVQ_TRY(check_shape(shape));
    KVQ_TRY(check_group(group, shape.head_dim));
    if (empty(shape)) return KVQ_OK;
    KVQ_TRY(check_params(lambda, signs));
    const int64_t D = shape.head_dim;
    KVQ_TRY(check_view(x_is_output ? "out_f16" : "x_f16", x, 2, D, 16, shape));
    KVQ_TRY(check_view(bits == 4 ? "codes_u8" : "codes_i8", codes, 1, bits == 4 ? D / 2 : D, 16, shape));
    if (mx) KVQ_TRY(check_view("scales_e8m0", scales, 1, D / group, 1, shape));
    else KVQ_TRY(check_view("scales_f16", scales, 2, D / group, 2, shape));
    a.L = (int32_t)shape.layers;
    a.T = (int32_t)shape.tokens;
    a.H = (int32_t)shape.heads;
    a.D = (int32_t)D;
    a.G = group;
    a.bits = bits;
    a.mx = mx ? 1 : 0;
    a.fourier = fourier ? 1 : 0;
    a.x = t4(x);
    a.codes = t4(codes);
    a.scales = t4(scales);
    a.lambda = lambda;
    a.signs = signs;
    set_items(shape, a.token_major, a.h_shift, a.items_per_group, a.tok_per_item, a.items_per_wave, a.n_items,
              int4_run_cap(D, x_is_output, fourier));
    return KVQ_OK;
}

kvq_status vq_common(const kvq_shape& shape, const kvq_view& x, const float* lambda, const int8_t* signs,
                     const void* codebook, int64_t cb_layer_stride, int32_t K, int32_t sub,
                     const kvq_view& idx, kvq::VqArgs& a, bool x_is_output, bool idx8 = false)
{
    KVQ_TRY(check_shape(shape));
    if (K < 1 || K > 65536) return fail(KVQ_ERR_SHAPE, "n_centroids=%d; must be in 1..65536", K);
    if (idx8 && K > 256) return fail(KVQ_ERR_SHAPE, "n_centroids=%d; one-byte indices need at most 256", K);
    if (sub <= 0 || shape.head_dim % sub) return fail(KVQ_ERR_SHAPE, "sub_dim=%d must divide head_dim", sub);
    if (sub != 8) return fail(KVQ_ERR_UNSUPPORTED, "sub_dim=%d; only 8 is instantiated", sub);
    if (empty(shape)) return KVQ_OK;
    KVQ_TRY(check_params(lambda, signs));
    if (!codebook) return fail(KVQ_ERR_NULL, "codebook is NULL");
    if (!aligned(codebook, 16)) return fail(KVQ_ERR_ALIGN, "codebook must be 16-byte aligned");
    if (cb_layer_stride < 0) return fail(KVQ_ERR_SHAPE, "codebook_layer_stride is negative");
    if ((cb_layer_stride * 2) % 16) return fail(KVQ_ERR_ALIGN, "codebook_layer_stride*2 bytes must be a multiple of 16");
    const int64_t D = shape.head_dim;
    KVQ_TRY(check_view(x_is_output ? "out_f16" : "x_f16", x, 2, D, 16, shape));
    KVQ_TRY(check_view(idx8 ? "idx_u8" : "idx_u16", idx, idx8 ? 1 : 2, D / sub, 4, shape));
    a.idx8 = idx8 ? 1 : 0;
    a.L = (int32_t)shape.layers;
    a.T = (int32_t)shape.tokens;
    a.H = (int32_t)shape.heads;
    a.D = (int32_t)D;
    a.sub = sub;
    a.K = K;
    a.x = t4(x);
    a.idx = t4(idx);
    a.lambda = lambda;
    a.signs = signs;
    a.codebook = static_cast<const uint16_t*>(codebook);
    a.cb_layer_stride = cb_layer_stride;
    set_items(shape, a.token_major, a.h_shift, a.items_per_group, a.tok_per_item, a.items_per_wave, a.n_items);
    a.dec_waves_per_group = (a.items_per_group + a.items_per_wave - 1) / a.items_per_wave;
    a.dec_n_waves = (a.n_items / a.items_per_group) * a.dec_waves_per_group;
    const int64_t tpu = 16 * kvq::vq_encode_waves((int)D, idx8);
    a.enc_units_per_lh = (int32_t)((shape.tokens + tpu - 1) / tpu);
    a.enc_n_units = shape.layers * shape.heads * (int64_t)a.enc_units_per_lh;
    a.enc_units_per_block = 1;
    return KVQ_OK;
}

// Split plan of the decode-attention kernels: query heads per pass, token
// splits per (outer index, KV head), tokens per split (a multiple of the
// block's token slots) and partial states per (outer index, query head).
// A deterministic function of the shape and the current device, so that the
// workspace query and the call agree.
struct AttnPlan {
    int32_t rp, S, chunk, parts;
};

AttnPlan attn_plan(const kvq_shape& s, int32_t R)
{
    AttnPlan p;
    const int64_t ts = 1024 / s.head_dim;                  // token slots per wavefront
    const int64_t step = kvq::kAttnWaves * ts;             // tokens per block step
    p.rp = R == 1 ? 1 : (R == 2 ? 2 : 4);
    const int64_t passes = (R + p.rp - 1) / p.rp;
    const int64_t base = std::max<int64_t>(1, s.layers * s.heads * passes);
    const int64_t target = 4LL * device_cus();             // blocks wanted in flight
    int64_t S = (target + base - 1) / base;
    S = std::min<int64_t>(S, std::max<int64_t>(1, (s.tokens + 4 * step - 1) / (4 * step)));
    int64_t chunk = std::max<int64_t>(1, (s.tokens + S - 1) / S);
    chunk = (chunk + step - 1) / step * step;
    S = std::max<int64_t>(1, (s.tokens + chunk - 1) / chunk);
    p.S = (int32_t)S;
    p.chunk = (int32_t)chunk;
    p.parts = (int32_t)(S * kvq::kAttnWaves * ts);
    return p;
}

// Plan of the matrix-core kernel (head_dim 128 or 256, four groups).  A block is one
// (outer index, split) and a group of hb KV heads, hb the largest of 8, 4, 2,
// 1 that divides H; its eight wavefronts are the hb heads times 8 / hb
// consecutive sub-ranges of the split.  The heads of a group read
// interleaved rows of the same 128-byte lines (two heads' codes, all heads'
// scales), so one block reads each line once.  One block fills a CU; the
// splits give about eight blocks per CU, with at least four 32-token steps
// per wavefront.  parts = splits x sub-ranges, one partial per wavefront.
struct MfmaPlan {
    int32_t hb, S, chunk, parts;
};

MfmaPlan attn_plan_mfma(const kvq_shape& s, int32_t R)
{
    MfmaPlan p;
    p.hb = s.heads % 8 == 0 ? 8 : (s.heads % 4 == 0 ? 4 : (s.heads % 2 == 0 ? 2 : 1));
    const int64_t nsub = kvq::kAttnMfmaWaves / p.hb;
    const int64_t step = nsub * 32;                        // tokens per block step
    const int64_t passes = (R + 3) / 4;
    const int64_t base = std::max<int64_t>(1, s.layers * (s.heads / p.hb) * passes);
    const int64_t target = 8LL * device_cus();
    int64_t S = (target + base - 1) / base;
    S = std::min<int64_t>(S, std::max<int64_t>(1, (s.tokens + 4 * step - 1) / (4 * step)));
    int64_t chunk = std::max<int64_t>(1, (s.tokens + S - 1) / S);
    chunk = (chunk + step - 1) / step * step;
    S = std::max<int64_t>(1, (s.tokens + chunk - 1) / chunk);
    p.S = (int32_t)S;
    p.chunk = (int32_t)chunk;
    p.parts = (int32_t)(S * nsub);
    return p;
}

// Partial states per (outer index, query head) the workspace holds: enough
// for whichever kernel the call picks.
int64_t attn_parts_capacity(const kvq_shape& s, int32_t R)
{
    int64_t parts = attn_plan(s, R).parts;
    if (s.head_dim == 128 || s.head_dim == 256) parts = std::max<int64_t>(parts, attn_plan_mfma(s, R).parts);
    return parts;
}

int64_t attn_workspace_bytes(const kvq_shape& s, int32_t R)
{
    return s.layers * s.heads * (int64_t)R * attn_parts_capacity(s, R) * (s.head_dim + 4) * (int64_t)sizeof(float);
}

kvq_status attn_check(const kvq_shape& shape, int32_t R)
{
    KVQ_TRY(check_shape(shape));
    if (R < 1 || R > 1024) return fail(KVQ_ERR_SHAPE, "q_per_kv=%d; must be in 1..1024", R);
    if ((double)shape.layers * shape.heads * R > (double)(INT32_MAX / 2))
        return fail(KVQ_ERR_SHAPE, "layers*heads*q_per_kv exceeds 2^30");
    return KVQ_OK;
}

}  // namespace

namespace {

kvq_status vq_encode_any(kvq_shape shape, kvq_view x_f16, const float* lambda, const int8_t* signs,
                         const void* codebook_f16, int64_t codebook_layer_stride, int32_t n_centroids,
                         int32_t sub_dim, kvq_view idx, void* stream, bool idx8)
{
    g_err[0] = 0;
    kvq::VqArgs a;
    KVQ_TRY(vq_common(shape, x_f16, lambda, signs, codebook_f16, codebook_layer_stride, n_centroids, sub_dim,
                      idx, a, false, idx8));
    if (empty(shape)) return KVQ_OK;
    // one block per CU holds the 144 KB of LDS (three four-wavefront blocks
    // per CU for one-byte indices); four rounds of resident blocks' worth of
    // units per CU balance the tail
    const int64_t blocks = std::min<int64_t>(a.enc_n_units, (idx8 ? 12 : 4) * (int64_t)device_cus());
    a.enc_units_per_block = (int32_t)((a.enc_n_units + blocks - 1) / blocks);
    return hip_status(kvq::launch_vq_encode(a, static_cast<hipStream_t>(stream)), "kvq_vq_encode launch");
}

kvq_status vq_decode_any(kvq_shape shape, kvq_view idx, const void* codebook_f16,
                         int64_t codebook_layer_stride, int32_t n_centroids, int32_t sub_dim,
                         const float* lambda, const int8_t* signs, kvq_view out_f16, void* stream, bool idx8)
{
    g_err[0] = 0;
    kvq::VqArgs a;
    KVQ_TRY(vq_common(shape, out_f16, lambda, signs, codebook_f16, codebook_layer_stride, n_centroids, sub_dim,
                      idx, a, true, idx8));
    if (empty(shape)) return KVQ_OK;
    a.dec_rows_per_range = 0;
    a.dec_range_groups = 0;
    if (n_centroids <= kvq::kVqChunk && shape.tokens >= kvq::kTokensPerTile) {
        // codebook in LDS: one block per CU.  The (layer, 16-token tile) rows
        // are cut into ranges; each range is decoded by H blocks, one per
        // head, placed on the same XCD so that the heads' indices of a token,
        // which share cache lines, are fetched from HBM once.
        a.token_major = 0;
        a.tok_per_item = kvq::kTokensPerTile;
        a.items_per_group = (int32_t)((shape.tokens + kvq::kTokensPerTile - 1) / kvq::kTokensPerTile);
        a.n_items = shape.layers * shape.heads * (int64_t)a.items_per_group;
        const int64_t rows = shape.layers * (int64_t)a.items_per_group;
        a.dec_range_groups = (int32_t)std::max<int64_t>(1, device_cus() / (8 * shape.heads));
        const int64_t ranges = 8 * (int64_t)a.dec_range_groups;
        a.dec_rows_per_range = (rows + ranges - 1) / ranges;
    }
    return hip_status(kvq::launch_vq_decode(a, static_cast<hipStream_t>(stream)), "kvq_vq_decode launch");
}

// Work split of the k-means update: per head, 8 * range_groups ranges of
// (layer, 16-token tile) rows, two blocks per (head, range) (coordinates
// 0-3 and 4-7 of the sub-vectors).  A function of
// the shape and the current device only, so that the workspace query and the
// call agree.
struct KmPlan {
    int32_t tiles, range_groups;
    int64_t rows_per_range;
};

KmPlan km_plan(const kvq_shape& s)
{
    KmPlan p;
    p.tiles = (int32_t)((s.tokens + kvq::kTokensPerTile - 1) / kvq::kTokensPerTile);
    p.range_groups = (int32_t)std::max<int64_t>(1, device_cus() / (8 * std::max<int64_t>(1, s.heads)));
    const int64_t rows = s.layers * (int64_t)p.tiles;
    const int64_t ranges = 8 * (int64_t)p.range_groups;
    p.rows_per_range = (rows + ranges - 1) / ranges;
    return p;
}

int64_t km_workspace_bytes(const kvq_shape& s, int32_t K, const KmPlan& p)
{
    // int64 fixed-point sums (8 per centroid) and a u32 count per centroid,
    // per (head, range)
    return s.heads * 8 * (int64_t)p.range_groups * (int64_t)K * 68;
}

kvq_status km_check(const kvq_shape& s, int32_t K, int32_t sub)
{
    KVQ_TRY(check_shape(s));
    if (K < 1 || K > kvq::kKmMaxCentroids)
        return fail(KVQ_ERR_SHAPE, "n_centroids=%d; k-means update supports 1..%d", K, kvq::kKmMaxCentroids);
    if (sub <= 0 || s.head_dim % sub) return fail(KVQ_ERR_SHAPE, "sub_dim=%d must divide head_dim", sub);
    if (sub != 8) return fail(KVQ_ERR_UNSUPPORTED, "sub_dim=%d; only 8 is instantiated", sub);
    return KVQ_OK;
}

// Static scratch of kvq_attend_decode_noalloc: the split partial states of
// decode attention, for callers that cannot allocate.  Every GPU the library
// runs on holds its own copy until the process ends.  In host code the name
// `scratch` is only a host-side stand-in; the device address comes from
// hipGetSymbolAddress, once per device (with that device current), and only
// that address is ever handed to a kernel.  Calls on one device share the
// array, so calls that overlap on one device race; its contents on entry do
// not matter (every partial a call reads, it has written).
constexpr int64_t kAttnScratchBytes = 64ll << 20;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kAttnScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

kvq_status scratch_pointer(void** ptr)
{
    int dev = 0;
    KVQ_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
    if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        KVQ_TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
        if (!p) return fail(KVQ_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_quantize(kvq_shape shape, kvq_view x_f16, const float* lambda, const int8_t* signs,
                        int32_t group, kvq_view codes_u8, kvq_view scales_f16, void* stream)
{
    g_err[0] = 0;
    kvq::Int4Args a;
    KVQ_TRY(int4_common(shape, x_f16, lambda, signs, group, codes_u8, scales_f16, a, false));
    if (empty(shape)) return KVQ_OK;
    return hip_status(kvq::launch_quantize(a, static_cast<hipStream_t>(stream)), "kvq_quantize launch");
}

kvq_status kvq_dequantize(kvq_shape shape, kvq_view codes_u8, kvq_view scales_f16, const float* lambda,
                          const int8_t* signs, int32_t group, kvq_view out_f16, void* stream)
{
    g_err[0] = 0;
    kvq::Int4Args a;
    KVQ_TRY(int4_common(shape, out_f16, lambda, signs, group, codes_u8, scales_f16, a, true));
    if (empty(shape)) return KVQ_OK;
    return hip_status(kvq::launch_dequantize(a, static_cast<hipStream_t>(stream)), "kvq_dequantize launch");
}

kvq_status kvq_quantize_srft(kvq_shape shape, kvq_view x_f16, const float* lambda, const int8_t* signs,
                             int32_t group, kvq_view codes_u8, kvq_view scales_f16, void* stream)
{
    g_err[0] = 0;
    kvq::Int4Args a;
    KVQ_TRY(int4_common(shape, x_f16, lambda, signs, group, codes_u8, scales_f16, a, false, 4, false, true));
    if (empty(shape)) return KVQ_OK;
    return hip_status(kvq::launch_quantize(a, static_cast<hipStream_t>(stream)), "kvq_quantize_srft launch");
}

kvq_status kvq_dequantize_srft(kvq_shape shape, kvq_view codes_u8, kvq_view scales_f16, const float* lambda,
                               const int8_t* signs, int32_t group, kvq_view out_f16, void* stream)
{
    g_err[0] = 0;
    kvq::Int4Args a;
    KVQ_TRY(int4_common(shape, out_f16, lambda, signs, group, codes_u8, scales_f16, a, true, 4, false, true));
    if (empty(shape)) return KVQ_OK;
    return hip_status(kvq::launch_dequantize(a, static_cast<hipStream_t>(stream)), "kvq_dequantize_srft launch");
}

kvq_status kvq_quantize_int8(kvq_shape shape, kvq_view x_f16, const float* lambda, const int8_t* signs,
                             int32_t group, kvq_view codes_i8, kvq_view scales_f16, void* stream)
{
    g_err[0] = 0;
    kvq::Int4Args a;
    KVQ_TRY(int4_common(shape, x_f16, lambda, signs, group, codes_i8, scales_f16, a, false, 8));
    if (empty(shape)) return KVQ_OK;
    return hip_status(kvq::launch_quantize(a, static_cast<hipStream_t>(stream)), "kvq_quantize_int8 launch");
}

kvq_status kvq_dequantize_int8(kvq_shape shape, kvq_view codes_i8, kvq_view scales_f16, const float* lambda,
                               const int8_t* signs, int32_t group, kvq_view out_f16, void* stream)
{
    g_err[0] = 0;
    kvq::Int4Args a;
    KVQ_TRY(int4_common(shape, out_f16, lambda, signs, group, codes_i8, scales_f16, a, true, 8));
    if (empty(shape)) return KVQ_OK;
    return hip_status(kvq::launch_dequantize(a, static_cast<hipStream_t>(stream)), "kvq_dequantize_int8 launch");
}

kvq_status kvq_quantize_mxfp4(kvq_shape shape, kvq_view x_f16, const float* lambda, const int8_t* signs,
                              kvq_view codes_u8, kvq_view scales_e8m0, void* stream)
{
    g_err[0] = 0;
    kvq::Int4Args a;
    KVQ_TRY(int4_common(shape, x_f16, lambda, signs, 32, codes_u8, scales_e8m0, a, false, 4, true));
    if (empty(shape)) return KVQ_OK;
    return hip_status(kvq::launch_quantize(a, static_cast<hipStream_t>(stream)), "kvq_quantize_mxfp4 launch");
}

kvq_status kvq_dequantize_mxfp4(kvq_shape shape, kvq_view codes_u8, kvq_view scales_e8m0, const float* lambda,
                                const int8_t* signs, kvq_view out_f16, void* stream)
{
    g_err[0] = 0;
    kvq::Int4Args a;
    KVQ_TRY(int4_common(shape, out_f16, lambda, signs, 32, codes_u8, scales_e8m0, a, true, 4, true));
    if (empty(shape)) return KVQ_OK;
    return hip_status(kvq::launch_dequantize(a, static_cast<hipStream_t>(stream)), "kvq_dequantize_mxfp4 launch");
}


kvq_status kvq_vq_encode(kvq_shape shape, kvq_view x_f16, const float* lambda, const int8_t* signs,
                         const void* codebook_f16, int64_t codebook_layer_stride, int32_t n_centroids,
                         int32_t sub_dim, kvq_view idx_u16, void* stream)
{
    return vq_encode_any(shape, x_f16, lambda, signs, codebook_f16, codebook_layer_stride, n_centroids, sub_dim,
                         idx_u16, stream, false);
}

kvq_status kvq_vq_decode(kvq_shape shape, kvq_view idx_u16, const void* codebook_f16,
                         int64_t codebook_layer_stride, int32_t n_centroids, int32_t sub_dim,
                         const float* lambda, const int8_t* signs, kvq_view out_f16, void* stream)
{
    return vq_decode_any(shape, idx_u16, codebook_f16, codebook_layer_stride, n_centroids, sub_dim, lambda, signs,
                         out_f16, stream, false);
}

kvq_status kvq_vq_encode_u8(kvq_shape shape, kvq_view x_f16, const float* lambda, const int8_t* signs,
                            const void* codebook_f16, int64_t codebook_layer_stride, int32_t n_centroids,
                            int32_t sub_dim, kvq_view idx_u8, void* stream)
{
    return vq_encode_any(shape, x_f16, lambda, signs, codebook_f16, codebook_layer_stride, n_centroids, sub_dim,
                         idx_u8, stream, true);
}

kvq_status kvq_vq_decode_u8(kvq_shape shape, kvq_view idx_u8, const void* codebook_f16,
                            int64_t codebook_layer_stride, int32_t n_centroids, int32_t sub_dim,
                            const float* lambda, const int8_t* signs, kvq_view out_f16, void* stream)
{
    return vq_decode_any(shape, idx_u8, codebook_f16, codebook_layer_stride, n_centroids, sub_dim, lambda, signs,
                         out_f16, stream, true);
}

kvq_status kvq_kmeans_step_workspace(kvq_shape shape, int32_t n_centroids, int32_t sub_dim, int64_t* bytes)
{
    g_err[0] = 0;
    if (!bytes) return fail(KVQ_ERR_NULL, "bytes is NULL");
    *bytes = 0;
    KVQ_TRY(km_check(shape, n_centroids, sub_dim));
    *bytes = km_workspace_bytes(shape, n_centroids, km_plan(shape));
    return KVQ_OK;
}

kvq_status kvq_kmeans_step(kvq_shape shape, kvq_view x_f16, const float* lambda, const int8_t* signs,
                           const void* codebook_f16, int32_t n_centroids, int32_t sub_dim, kvq_view idx_u16,
                           void* new_codebook_f16, uint32_t* counts, void* workspace, int64_t workspace_bytes,
                           void* stream)
{
    g_err[0] = 0;
    KVQ_TRY(km_check(shape, n_centroids, sub_dim));
    if (shape.heads == 0) return KVQ_OK;
    if (!codebook_f16) return fail(KVQ_ERR_NULL, "codebook is NULL");
    if (!new_codebook_f16) return fail(KVQ_ERR_NULL, "new_codebook is NULL");
    if (!counts) return fail(KVQ_ERR_NULL, "counts is NULL");
    if (!aligned(codebook_f16, 16) || !aligned(new_codebook_f16, 16))
        return fail(KVQ_ERR_ALIGN, "codebook and new_codebook must be 16-byte aligned");
    if (!aligned(counts, 4)) return fail(KVQ_ERR_ALIGN, "counts must be 4-byte aligned");
    const KmPlan p = km_plan(shape);
    const int64_t need = km_workspace_bytes(shape, n_centroids, p);
    if (!workspace) return fail(KVQ_ERR_NULL, "workspace is NULL (%lld bytes needed)", (long long)need);
    if (!aligned(workspace, 16)) return fail(KVQ_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
        return fail(KVQ_ERR_SHAPE, "workspace_bytes=%lld; %lld needed", (long long)workspace_bytes, (long long)need);
    if (!empty(shape)) {
        // assignment: the product-VQ encoder against the current codebook
        KVQ_TRY(vq_encode_any(shape, x_f16, lambda, signs, codebook_f16, 0, n_centroids, sub_dim, idx_u16, stream,
                              false));
    }
    kvq::KmArgs a;
    a.L = (int32_t)shape.layers;
    a.T = (int32_t)shape.tokens;
    a.H = (int32_t)shape.heads;
    a.D = (int32_t)shape.head_dim;
    a.K = n_centroids;
    a.x = t4(x_f16);
    a.idx = t4(idx_u16);
    a.lambda = lambda;
    a.signs = signs;
    a.codebook = static_cast<const uint16_t*>(codebook_f16);
    a.new_codebook = static_cast<uint16_t*>(new_codebook_f16);
    a.counts = counts;
    const int64_t slots = shape.heads * 8 * (int64_t)p.range_groups * n_centroids;
    a.part_sums = static_cast<int64_t*>(workspace);
    a.part_counts = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + slots * 64);
    a.tiles = p.tiles;
    a.range_groups = p.range_groups;
    a.rows_per_range = p.rows_per_range;
    return hip_status(kvq::launch_kmeans_update(a, static_cast<hipStream_t>(stream)), "kvq_kmeans_step launch");
}

kvq_status kvq_item_plan(kvq_shape shape, int32_t inverse, int32_t fourier, int32_t* token_major,
                         int64_t* n_items, int32_t* items_per_wave)
{
    g_err[0] = 0;
    if (!token_major || !n_items || !items_per_wave)
        return fail(KVQ_ERR_NULL, "token_major, n_items and items_per_wave must not be NULL");
    *token_major = 0;
    *n_items = 0;
    *items_per_wave = 0;
    KVQ_TRY(check_shape(shape));
    if (empty(shape)) return KVQ_OK;
    int32_t h_shift, items_per_group, tok_per_item;
    set_items(shape, *token_major, h_shift, items_per_group, tok_per_item, *items_per_wave, *n_items,
              int4_run_cap(shape.head_dim, inverse != 0, fourier != 0));
    return KVQ_OK;
}

kvq_status kvq_attend_decode_workspace(kvq_shape shape, int32_t q_per_kv, int64_t* bytes)
{
    g_err[0] = 0;
    if (!bytes) return fail(KVQ_ERR_NULL, "bytes is NULL");
    *bytes = 0;
    KVQ_TRY(attn_check(shape, q_per_kv));
    if (shape.layers == 0 || shape.heads == 0) return KVQ_OK;
    *bytes = attn_workspace_bytes(shape, q_per_kv);
    return KVQ_OK;
}

}  // extern "C"

namespace {

// Everything kvq_attend_decode does.  workspace == nullptr with
// use_scratch: the partial states go to this device's static scratch array
// (kvq_attend_decode_noalloc), whose size is checked against the need first.
kvq_status attend_any(kvq_shape shape, int32_t q_per_kv, const void* q_f16, kvq_view k_codes_u8,
                      kvq_view k_scales_f16, kvq_view v_codes_u8, kvq_view v_scales_f16, const float* lambda_k,
                      const float* lambda_v, const int8_t* signs, int32_t group, const int32_t* lengths,
                      float softmax_scale, void* out_f16, void* workspace, int64_t workspace_bytes, void* stream,
                      bool use_scratch)
{
    KVQ_TRY(attn_check(shape, q_per_kv));
    KVQ_TRY(check_group(group, shape.head_dim));
    if (shape.layers == 0 || shape.heads == 0) return KVQ_OK;
    if (!q_f16) return fail(KVQ_ERR_NULL, "q_f16 is NULL");
    if (!out_f16) return fail(KVQ_ERR_NULL, "out_f16 is NULL");
    if (!aligned(q_f16, 16) || !aligned(out_f16, 16)) return fail(KVQ_ERR_ALIGN, "q_f16 and out_f16 must be 16-byte aligned");
    KVQ_TRY(check_params(lambda_k, signs));
    KVQ_TRY(check_params(lambda_v, signs));
    if (!std::isfinite(softmax_scale)) return fail(KVQ_ERR_SHAPE, "softmax_scale is not finite");
    const int64_t D = shape.head_dim;
    if (shape.tokens > 0) {
        KVQ_TRY(check_view("k_codes_u8", k_codes_u8, 1, D / 2, 16, shape));
        KVQ_TRY(check_view("k_scales_f16", k_scales_f16, 2, D / group, 2, shape));
        KVQ_TRY(check_view("v_codes_u8", v_codes_u8, 1, D / 2, 16, shape));
        KVQ_TRY(check_view("v_scales_f16", v_scales_f16, 2, D / group, 2, shape));
    }
    const int64_t need = attn_workspace_bytes(shape, q_per_kv);
    if (!use_scratch) {
        if (!workspace) return fail(KVQ_ERR_NULL, "workspace is NULL (%lld bytes needed)", (long long)need);
        if (!aligned(workspace, 16)) return fail(KVQ_ERR_ALIGN, "workspace must be 16-byte aligned");
        if (workspace_bytes < need)
            return fail(KVQ_ERR_SHAPE, "workspace_bytes=%lld; %lld needed", (long long)workspace_bytes,
                        (long long)need);
    }
    kvq::AttnArgs a;
    a.L = (int32_t)shape.layers;
    a.T = (int32_t)shape.tokens;
    a.H = (int32_t)shape.heads;
    a.D = (int32_t)D;
    a.R = q_per_kv;
    a.g_shift = 0;
    while ((1 << a.g_shift) < group) a.g_shift++;
    // The matrix-core kernel serves head_dim 128 with groups of 32 and
    // head_dim 256 with groups of 64 (four groups per vector), where 32 token
    // rows of every view span less than 2^31 bytes (it addresses a step's
    // loads with 32-bit offsets); the VALU kernel serves the rest.
    const int64_t row = std::max(std::max(k_codes_u8.stride_token, v_codes_u8.stride_token),
                                 2 * std::max(k_scales_f16.stride_token, v_scales_f16.stride_token));
    a.mfma = ((D == 128 && group == 32) || (D == 256 && group == 64)) && 32 * row + 64 < ((int64_t)1 << 31);
    if (a.mfma) {
        const MfmaPlan p = attn_plan_mfma(shape, q_per_kv);
        a.rp = 4;
        a.hb = p.hb;
        a.S = p.S;
        a.chunk = p.chunk;
        a.parts = p.parts;
        a.xcd_map = 0;
    } else {
        const AttnPlan p = attn_plan(shape, q_per_kv);
        a.rp = p.rp;
        a.hb = 1;
        a.S = p.S;
        a.chunk = p.chunk;
        a.parts = p.parts;
        a.xcd_map = ((int64_t)a.L * a.S) % 8 == 0;
    }
    if (use_scratch) {
        // the partial states of the kernel this call runs (at most the
        // workspace query's bound, which covers either kernel)
        const int64_t used = shape.layers * shape.heads * (int64_t)q_per_kv * a.parts * (D + 4) * (int64_t)sizeof(float);
        if (used > kAttnScratchBytes)
            return fail(KVQ_ERR_SHAPE,
                        "this call needs %lld bytes of partial states; the static scratch holds %lld "
                        "(call kvq_attend_decode with a workspace, or split the call)",
                        (long long)used, (long long)kAttnScratchBytes);
        KVQ_TRY(scratch_pointer(&workspace));
    }
    a.q = static_cast<const _Float16*>(q_f16);
    a.out = static_cast<_Float16*>(out_f16);
    a.kc = t4(k_codes_u8);
    a.ks = t4(k_scales_f16);
    a.vc = t4(v_codes_u8);
    a.vs = t4(v_scales_f16);
    a.lam_k = lambda_k;
    a.lam_v = lambda_v;
    a.signs = signs;
    a.lengths = lengths;
    a.qscale = softmax_scale * 1.4426950408889634f;
    a.ws = static_cast<float*>(workspace);
    return hip_status(kvq::launch_attend_decode(a, static_cast<hipStream_t>(stream)), "kvq_attend_decode launch");
}

}  // namespace

extern "C" {

kvq_status kvq_attend_decode(kvq_shape shape, int32_t q_per_kv, const void* q_f16, kvq_view k_codes_u8,
                             kvq_view k_scales_f16, kvq_view v_codes_u8, kvq_view v_scales_f16,
                             const float* lambda_k, const float* lambda_v, const int8_t* signs, int32_t group,
                             const int32_t* lengths, float softmax_scale, void* out_f16, void* workspace,
                             int64_t workspace_bytes, void* stream)
{
    g_err[0] = 0;
    return attend_any(shape, q_per_kv, q_f16, k_codes_u8, k_scales_f16, v_codes_u8, v_scales_f16, lambda_k,
                      lambda_v, signs, group, lengths, softmax_scale, out_f16, workspace, workspace_bytes, stream,
                      false);
}

kvq_status kvq_attend_decode_noalloc(kvq_shape shape, int32_t q_per_kv, const void* q_f16, kvq_view k_codes_u8,
                                     kvq_view k_scales_f16, kvq_view v_codes_u8, kvq_view v_scales_f16,
                                     const float* lambda_k, const float* lambda_v, const int8_t* signs,
                                     int32_t group, const int32_t* lengths, float softmax_scale, void* out_f16,
                                     void* stream)
{
    g_err[0] = 0;
    return attend_any(shape, q_per_kv, q_f16, k_codes_u8, k_scales_f16, v_codes_u8, v_scales_f16, lambda_k,
                      lambda_v, signs, group, lengths, softmax_scale, out_f16, nullptr, 0, stream, true);
}

const char* kvq_status_string(kvq_status st)
{
    switch (st) {
        case KVQ_OK: return "KVQ_OK";
        case KVQ_ERR_NULL: return "KVQ_ERR_NULL";
        case KVQ_ERR_SHAPE: return "KVQ_ERR_SHAPE";
        case KVQ_ERR_ALIGN: return "KVQ_ERR_ALIGN";
        case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED";
        case KVQ_ERR_HIP: return "KVQ_ERR_HIP";
    }
    return "KVQ_ERR_UNKNOWN";
}

const char* kvq_last_error(void) { return g_err; }

int32_t kvq_version(void) { return 100; }

}  // extern "C"
