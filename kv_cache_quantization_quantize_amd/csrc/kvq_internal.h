// kvq_internal.h -- host-side launch interface between the C ABI layer
// (kvq_api.cpp) and the kernel translation units.  Not installed, not part of
// the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Vectors of one (layer, head) pair are processed 16 tokens at a time by one
// 64-lane wavefront: 4 lanes per vector, each lane holding D/4 coordinates.
constexpr int kTokensPerTile = 16;
constexpr int kWavesPerBlock = 4;

struct Tensor4 {            // strided view, strides in elements
    void* data;
    int64_t sl, st, sh;
};

struct Int4Args {
    int32_t L, T, H, D, G;
    int32_t bits;           // code width: 4 (nibbles) or 8 (bytes)
    int32_t mx;             // 1: block-scaled E2M1 codes with E8M0 byte scales (group 32)
    int32_t fourier;        // 1: SRFT rotation instead of Walsh-Hadamard (int4 codes)
    Tensor4 x;              // fp16 input (quantize) / fp16 output (dequantize)
    Tensor4 codes;          // u8, D/2 per vector
    Tensor4 scales;         // fp16, D/G per vector
    const float* lambda;    // [L, H, D]
    const int8_t* signs;    // [D]
    // Work items.  Token-major (H divides 16): an item is 16 consecutive
    // (token, head) vectors of one layer -- 16/H tokens x all H heads, one
    // contiguous run in a contiguous cache -- and lane slot s always holds
    // head s % H.  Head-major (other H): an item is 16 consecutive tokens of
    // one (layer, head) pair.
    int32_t token_major;
    int32_t h_shift;         // log2(H) when token-major (H is then a power of two)
    int32_t items_per_group; // items per layer (token-major) or per (layer, head)
    int32_t tok_per_item;    // 16/H (token-major) or 16
    int32_t items_per_wave;  // consecutive items per wavefront
    int64_t n_items;
};

struct VqArgs {
    int32_t L, T, H, D, sub, K;
    Tensor4 x;              // fp16 keys (encode) / fp16 output (decode)
    Tensor4 idx;            // u16 (or u8 when idx8), D/sub per vector
    int32_t idx8;           // one-byte indices (K <= 256)
    const float* lambda;    // [L, H, D]
    const int8_t* signs;    // [D]
    const uint16_t* codebook;   // fp16 bits, [H, K, sub] per layer
    int64_t cb_layer_stride;    // elements; 0 = shared
    // decode work items: as Int4Args
    int32_t token_major, h_shift, items_per_group, tok_per_item, items_per_wave;
    int64_t n_items;
    // decode: each wavefront takes up to items_per_wave items of one group
    // ((layer) or (layer, head)), so it loads one set of multipliers
    int32_t dec_waves_per_group;
    int64_t dec_n_waves;
    // decode with the codebook in LDS (K <= kVqChunk): the (layer, 16-token
    // tile) rows are cut into 8 * dec_range_groups ranges of this many rows;
    // the H blocks of one range run on one XCD.  0 selects the other path
    int64_t dec_rows_per_range;
    int32_t dec_range_groups;
    // encode units: (layer, head, 16*waves-token chunk), ordered head-major
    // when one codebook serves all layers so that a block rarely re-stages it
    int32_t enc_units_per_lh;
    int32_t enc_units_per_block;
    int64_t enc_n_units;
};

// Decode attention over the int4 cache.
struct AttnArgs {
    int32_t L, T, H, D, R;          // R query heads per KV head
    int32_t g_shift;                // log2(group)
    int32_t rp;                     // query heads per partial-kernel pass (1, 2 or 4)
    int32_t S;                      // token splits per (outer index, KV head)
    int32_t chunk;                  // tokens per split
    int32_t parts;                  // partial states per (outer index, query head)
    int32_t xcd_map;                // (L*S) % 8 == 0: heads of one (l, split) on one XCD
    int32_t mfma;                   // use the matrix-core kernel (D 128, group 32)
    int32_t hb;                     // matrix-core kernel: KV heads per block
    const _Float16* q;              // [L, H*R, D]
    _Float16* out;                  // [L, H*R, D]
    Tensor4 kc, ks, vc, vs;         // codes u8 (D/2), scales fp16 (D/G)
    const float* lam_k;             // [L, H, D]
    const float* lam_v;
    const int8_t* signs;            // [D]
    const int32_t* lengths;         // [L] or null
    float qscale;                   // softmax scale * log2(e)
    float* ws;                      // partials: [L*H][R][parts][D + 4] floats
};
constexpr int kAttnWaves = 4;       // wavefronts per attention block
constexpr int kAttnMfmaWaves = 8;   // wavefronts per matrix-core attention block

// Centroids staged in LDS at a time by the VQ encoder (64 KB of fp16).
constexpr int kVqChunk = 4096;

// One Lloyd (k-means) update of per-head codebooks [H, K, 8] shared by all
// layers: per-block sums of the rotated sub-vectors assigned to each
// centroid, then a fixed-order reduction of the blocks' partials.
struct KmArgs {
    int32_t L, T, H, D, K;
    Tensor4 x;                      // fp16 samples [L, T, H, D]
    Tensor4 idx;                    // u16 assignments, D/8 per vector
    const float* lambda;            // [L, H, D]
    const int8_t* signs;            // [D]
    const uint16_t* codebook;       // fp16 bits [H, K, 8] (input)
    uint16_t* new_codebook;         // fp16 bits [H, K, 8] (output, may alias codebook)
    uint32_t* counts;               // [H, K]
    int64_t* part_sums;             // [H, ranges, 8, K], fixed point (2^24 per unit)
    uint32_t* part_counts;          // [H, ranges, K]
    int32_t tiles;                  // 16-token tiles per layer
    int32_t range_groups;           // ranges per head = 8 * range_groups (two blocks each)
    int64_t rows_per_range;         // (layer, tile) rows per range
};
constexpr int kKmMaxCentroids = 4096;   // LDS: 36 bytes per centroid

// Wavefronts per VQ-encode block for a head dim (each stages 16 keys).
int vq_encode_waves(int D, bool idx8);

// Launchers: enqueue on `stream`, return the launch status.  Arguments have
// been validated by the caller.
hipError_t launch_quantize(const Int4Args& a, hipStream_t stream);
hipError_t launch_dequantize(const Int4Args& a, hipStream_t stream);
hipError_t launch_vq_encode(const VqArgs& a, hipStream_t stream);
hipError_t launch_vq_decode(const VqArgs& a, hipStream_t stream);
hipError_t launch_attend_decode(const AttnArgs& a, hipStream_t stream);
hipError_t launch_kmeans_update(const KmArgs& a, hipStream_t stream);

}  // namespace kvq
