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
    Tensor4 x;              // fp16 input (quantize) / fp16 output (dequantize)
    Tensor4 codes;          // u8, D/2 per vector
    Tensor4 scales;         // fp16, D/G per vector
    const float* lambda;    // [L, H, D]
    const int8_t* signs;    // [D]
    int32_t tiles_per_lh;   // ceil(T / 16)
    int32_t items_per_wave; // consecutive (layer, head, token-tile) items per wave
    int64_t n_items;        // L * H * tiles_per_lh
};

struct VqArgs {
    int32_t L, T, H, D, sub, K;
    Tensor4 x;              // fp16 keys (encode) / fp16 output (decode)
    Tensor4 idx;            // u16, D/sub per vector
    const float* lambda;    // [L, H, D]
    const int8_t* signs;    // [D]
    const uint16_t* codebook;   // fp16 bits, [H, K, sub] per layer
    int64_t cb_layer_stride;    // elements; 0 = shared
    int32_t tiles_per_lh;
    int32_t items_per_wave;
    int64_t n_items;
};

// Launchers: enqueue on `stream`, return the launch status.  Arguments have
// been validated by the caller.
hipError_t launch_quantize(const Int4Args& a, hipStream_t stream);
hipError_t launch_dequantize(const Int4Args& a, hipStream_t stream);
hipError_t launch_vq_encode(const VqArgs& a, hipStream_t stream);
hipError_t launch_vq_decode(const VqArgs& a, hipStream_t stream);

}  // namespace kvq
