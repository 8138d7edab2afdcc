/*
 * kvq.h -- C ABI of libkvq.so, a fused per-vector KV-cache quantizer for AMD
 * Instinct MI355X (gfx950).
 *
 * The operations follow these pages (cited by title and section):
 *  - "When Quantization Is Free: An int4 KV Cache That Outruns fp16 on Apple
 *    Silicon" (arXiv 2605.05699), abstract: one fused kernel doing a
 *    sign-randomized transform, a per-channel smooth scale lambda, per-group
 *    abs-max and int4 nibble packing of the KV cache;
 *  - gist.science explanation of the same paper, "Methodologie" s.1 (the
 *    transform is diag(sign) then a unitary transform), s.2 (the fused
 *    kernel's step list: signs in registers, transform, lambda, group
 *    abs-max, signed int4 rounding, two codes per byte), s.3 (per-channel
 *    plus per-group scaling);
 *  - "The Kernel That Finally Did Something -- And Didn't Quite Agree With
 *    Itself" (VeloxQuant-MLX blog, VecInfer): "What VecInfer does" (smooth
 *    scale and Walsh-Hadamard rotation of keys, encoding against a trained
 *    codebook, immediate dequantization), "The kernel toggle" (one fused
 *    dispatch: smooth scale, Hadamard, quantize, dequantize, inverse
 *    transform, unscale);
 *  - VeloxQuant-MLX 0.52.0 package description, "Metal kernels"
 *    (quantize_vq: nearest centroid search with the argmin kept in registers,
 *    no [N, n_centroids, sub_dim] difference tensor).
 *
 * Definitions (the readings the library implements):
 *   D = head_dim in {64, 128, 256}; Hd = the Sylvester-order Walsh-Hadamard
 *   matrix, Hd[i][j] = (-1)^popcount(i & j); s = sign vector in {-1,+1}^D;
 *   lambda = smooth scale, one fp32 per (layer, head, channel).
 *   rotate:    y = D^-1/2 * Hd * diag(s) * diag(lambda[l,h,:]) * x
 *   int4:      for each group g of G consecutive rotated coordinates,
 *              scale_g = fp16_rne(max|y_i| / 7),
 *              q_i = 0 if scale_g == 0 else clamp(rne(y_i / scale_g), -7, 7)
 *              byte k of a vector = (q_2k & 0xF) | (q_2k+1 & 0xF) << 4
 *   dequant:   yhat_i = q_i * scale_g;
 *              xhat = fp16_rne(diag(s / lambda[l,h,:]) * Hd * yhat * D^-1/2)
 *   VQ encode: y as above, split into D/sub_dim contiguous sub-vectors;
 *              idx_j = lowest k minimising ||y_j - c_k||^2 over the head's
 *              codebook c[0..n_centroids) (fp16, sub_dim values each)
 *   VQ decode: yhat = concatenation of c[idx_j]; xhat as in dequant.
 * GPU arithmetic is fp32; results agree with an fp64 evaluation of these
 * definitions up to fp32 rounding (a code may differ by one where the exact
 * y/scale lies within 1e-4 of a rounding boundary, a scale by one fp16 ulp,
 * a VQ index where two distances differ by less than 1e-4 relative).
 *
 * Tensors.  A KV tensor is [layers, tokens, heads, head_dim] with the last
 * dimension contiguous; a kvq_view gives its base pointer and its three outer
 * strides, in ELEMENTS of the view's own type (fp16 = 2 bytes, codes = bytes,
 * scales = fp16, VQ indices = uint16).  Code rows hold D/2 bytes, scale rows
 * D/G fp16 values, index rows D/sub_dim uint16 values.  A decode-time append
 * of token t is a call with tokens = 1 and views whose data point at slot t.
 *
 * Memory and ownership.  Every data pointer (x, out, codes, scales, indices,
 * lambda, signs, codebook) is DEVICE memory owned by the caller; the library
 * allocates nothing, keeps no state except a thread-local error message, and
 * never synchronises.  Each call validates its arguments on the host, then
 * enqueues its kernel on `stream` (a hipStream_t passed as void*; NULL is the
 * default stream) and returns.  Faults inside a kernel surface at the
 * caller's next synchronisation.  Calls on different streams may run
 * concurrently when their outputs do not overlap.
 *
 * Errors.  A non-OK status means nothing was enqueued (except KVQ_ERR_HIP,
 * returned when the launch itself failed).  kvq_last_error() then describes
 * the failing argument.  Device-side preconditions that are NOT checked:
 * every sign is +-1; lambda is finite and > 0; inputs are finite and small
 * enough that max|y|/7 fits fp16 (otherwise the outputs of that vector are
 * unspecified, but no out-of-bounds access happens); VQ indices passed to
 * decode are < n_centroids (larger ones are clamped to n_centroids - 1).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_ERR_NULL = 1,         /* a required pointer is NULL */
    KVQ_ERR_SHAPE = 2,        /* negative or inconsistent sizes */
    KVQ_ERR_ALIGN = 3,        /* pointer or stride not aligned as required */
    KVQ_ERR_UNSUPPORTED = 4,  /* valid but not instantiated (head_dim, group, sub_dim) */
    KVQ_ERR_HIP = 5           /* the HIP launch failed */
} kvq_status;

/* Logical shape of a KV tensor: [layers, tokens, heads, head_dim].  Any of
   layers, tokens, heads may be 0: the call then checks only head_dim, group,
   n_centroids and sub_dim (pointers and strides of an empty tensor are not
   looked at) and returns KVQ_OK without enqueuing anything.  head_dim must be
   64, 128 or 256. */
typedef struct kvq_shape {
    int64_t layers, tokens, heads, head_dim;
} kvq_shape;

/* A strided view: element (l, t, h, i) lives at
   data + l*stride_layer + t*stride_token + h*stride_head + i
   (pointer arithmetic in elements of the view's type). */
typedef struct kvq_view {
    void* data;
    int64_t stride_layer, stride_token, stride_head;
} kvq_view;

/* Fused rotate + int4 quantize (sign-randomized Walsh-Hadamard with smooth
 * scale, per-group abs-max, nibble packing) -- the fused kernel of the
 * "When Quantization Is Free" abstract with the Walsh-Hadamard transform in
 * place of the FFT (the paper finds the two indistinguishable for KV quality).
 *   x_f16      fp16 input view, 16-byte aligned data, strides multiples of 8.
 *   lambda     fp32 [layers, heads, head_dim] contiguous, for the layers of
 *              this call (offset it for a single-layer append).
 *   signs      int8 [head_dim], each +1 or -1.
 *   group      G, a power of two with 8 <= G <= head_dim.
 *   codes_u8   output view of D/2-byte rows; 16-byte aligned data and strides.
 *   scales_f16 output view of D/G-element fp16 rows; 2-byte aligned.
 * Heads are independent, so a layer's K and V can go through one call: with
 * the cache laid out [layers, tokens, 2*heads, .] (K in heads 0..H-1, V in
 * heads H..2H-1) and lambda [layers, 2*heads, head_dim], one decode-time
 * append per layer replaces two; kvq_attend_decode takes the two halves as
 * views with the same strides.
 */
kvq_status kvq_quantize(kvq_shape shape, kvq_view x_f16, const float* lambda,
                        const int8_t* signs, int32_t group, kvq_view codes_u8,
                        kvq_view scales_f16, void* stream);

/* Mirror of kvq_quantize: unpack codes, multiply by the group scale, inverse
 * Walsh-Hadamard, divide by lambda and apply the signs, round to fp16
 * (VecInfer blog, "The kernel toggle": dequantize, inverse transform,
 * unscale).  Views and alignment as for kvq_quantize; out_f16 is the fp16
 * output view (16-byte aligned, strides multiples of 8). */
kvq_status kvq_dequantize(kvq_shape shape, kvq_view codes_u8, kvq_view scales_f16,
                          const float* lambda, const int8_t* signs, int32_t group,
                          kvq_view out_f16, void* stream);

/* SRFT variant of kvq_quantize (gist.science summary, "Methodologie" s.1:
 * the sign-randomized Fourier transform as the rotation): the same group
 * quantizer and formats on
 *   y = pack(F diag(s) diag(lambda) x),  F the unitary DFT of length D,
 *   pack = [X_0, X_{D/2}, sqrt2 Re X_1, sqrt2 Im X_1, ..., sqrt2 Im X_{D/2-1}],
 * an orthonormal real representation of the real input's half spectrum.
 * Computed as a D/2-point complex radix-2 FFT of (v_2m + i v_2m+1) and its
 * Hermitian unpacking.  Shapes, views, lambda, signs, group and errors as
 * for kvq_quantize. */
kvq_status kvq_quantize_srft(kvq_shape shape, kvq_view x_f16, const float* lambda,
                             const int8_t* signs, int32_t group, kvq_view codes_u8,
                             kvq_view scales_f16, void* stream);

/* Mirror of kvq_quantize_srft: unpack, scale, inverse SRFT, unscale, fp16.
 * Arguments as for kvq_dequantize. */
kvq_status kvq_dequantize_srft(kvq_shape shape, kvq_view codes_u8, kvq_view scales_f16,
                               const float* lambda, const int8_t* signs, int32_t group,
                               kvq_view out_f16, void* stream);

/* int8 variant of kvq_quantize (gist.science summary, "Methodologie" s.2:
 * the fused kernel rounds to signed int4 or int8): the same rotation and
 * groups, scale = fp16_rne(amax / 127), q = clamp(rne(y / scale), -127, 127)
 * with the stored scale, one two's-complement byte per coordinate (element i
 * in byte i of the row).
 *   codes_i8   output view of D-byte rows; 16-byte aligned data and strides.
 * Everything else (shapes, lambda, signs, group, scales, errors) as for
 * kvq_quantize. */
kvq_status kvq_quantize_int8(kvq_shape shape, kvq_view x_f16, const float* lambda,
                             const int8_t* signs, int32_t group, kvq_view codes_i8,
                             kvq_view scales_f16, void* stream);

/* Mirror of kvq_quantize_int8: code times its group scale, inverse
 * Walsh-Hadamard, unscale, fp16.  Views as for kvq_dequantize, with D-byte
 * code rows. */
kvq_status kvq_dequantize_int8(kvq_shape shape, kvq_view codes_i8, kvq_view scales_f16,
                               const float* lambda, const int8_t* signs, int32_t group,
                               kvq_view out_f16, void* stream);

/* Block-scaled E2M1 variant of kvq_quantize (the PolarQuant/block-FP4
 * abstract names block-scaled E2M1 FP4 as a KV-cache format; the format is
 * the OCP Microscaling MXFP4 one): the same rotation, then blocks of 32
 * rotated coordinates, each with a power-of-two scale X = 2^e, e =
 * floor(log2(amax)) - 2 clamped to [-127, 127] (-127 for an all-zero block),
 * stored as the E8M0 byte e + 127, and E2M1 elements = y / X rounded to
 * nearest (ties to the even code), saturating at +-6, sign bit kept.
 *   codes_u8     output view of D/2-byte rows: element 2k in the low nibble
 *                of byte k; 16-byte aligned data and strides.
 *   scales_e8m0  output view of D/32-byte rows.
 * The E2M1 rounding uses the gfx950 v_cvt_scalef32_pk_fp4_f32 conversion on
 * y * 2^-e.  Other arguments and errors as for kvq_quantize. */
kvq_status kvq_quantize_mxfp4(kvq_shape shape, kvq_view x_f16, const float* lambda,
                              const int8_t* signs, kvq_view codes_u8, kvq_view scales_e8m0,
                              void* stream);

/* Mirror of kvq_quantize_mxfp4: E2M1 value times 2^(scale - 127), inverse
 * Walsh-Hadamard, unscale, fp16.  Views as for kvq_dequantize, with D/32-byte
 * E8M0 scale rows. */
kvq_status kvq_dequantize_mxfp4(kvq_shape shape, kvq_view codes_u8, kvq_view scales_e8m0,
                                const float* lambda, const int8_t* signs, kvq_view out_f16,
                                void* stream);

/* Product-VQ encode (VecInfer blog, "What VecInfer does"; VeloxQuant-MLX
 * package description, "Metal kernels"): rotate as kvq_quantize does (no
 * group quantizer), split into D/sub_dim sub-vectors and store, per
 * sub-vector, the lowest index of a nearest centroid of that head's codebook.
 *   codebook_f16            fp16 [heads, n_centroids, sub_dim] per layer;
 *   codebook_layer_stride   elements between layers' codebooks, 0 = one
 *                           codebook shared by all layers;
 *   n_centroids             1 .. 65536;
 *   sub_dim                 8 (must divide head_dim);
 *   idx_u16                 output view of D/sub_dim uint16 rows; 4-byte
 *                           aligned data, even strides.
 * The codebook must be 16-byte aligned.  Distances use the unrounded fp32
 * rotated key.  Domain: rotated coordinates below 65504 in magnitude and
 * squared centroid norms below 65504 (both enter the matrix cores as fp16
 * hi + lo halves); outside it the indices are unspecified, and no access
 * goes out of bounds. */
kvq_status kvq_vq_encode(kvq_shape shape, kvq_view x_f16, const float* lambda,
                         const int8_t* signs, const void* codebook_f16,
                         int64_t codebook_layer_stride, int32_t n_centroids,
                         int32_t sub_dim, kvq_view idx_u16, void* stream);

/* Product-VQ decode: gather the named centroids, inverse Walsh-Hadamard,
 * unscale, round to fp16 (VecInfer blog, "The kernel toggle").  Arguments as
 * for kvq_vq_encode; idx_u16 is the input view, out_f16 the fp16 output view
 * (16-byte aligned, strides multiples of 8). */
kvq_status kvq_vq_decode(kvq_shape shape, kvq_view idx_u16, const void* codebook_f16,
                         int64_t codebook_layer_stride, int32_t n_centroids,
                         int32_t sub_dim, const float* lambda, const int8_t* signs,
                         kvq_view out_f16, void* stream);

/* Product VQ with one-byte indices, for codebooks of at most 256 centroids
 * (the 8-bit value codebooks of the VecInfer blog, "The numbers":
 * value_codebook_bits = 8).  The same computation as kvq_vq_encode /
 * kvq_vq_decode, including the rotation with the tensor's own lambda;
 * idx_u8 holds D/sub_dim bytes per vector (4-byte aligned data and strides).
 * KVQ_ERR_SHAPE if n_centroids > 256. */
kvq_status kvq_vq_encode_u8(kvq_shape shape, kvq_view x_f16, const float* lambda,
                            const int8_t* signs, const void* codebook_f16,
                            int64_t codebook_layer_stride, int32_t n_centroids,
                            int32_t sub_dim, kvq_view idx_u8, void* stream);
kvq_status kvq_vq_decode_u8(kvq_shape shape, kvq_view idx_u8, const void* codebook_f16,
                            int64_t codebook_layer_stride, int32_t n_centroids,
                            int32_t sub_dim, const float* lambda, const int8_t* signs,
                            kvq_view out_f16, void* stream);

/* Codebook training (VecInfer blog, "What VecInfer does, and the calibration
 * caveat up front": codebooks trained k-means style on synthetic samples):
 * one Lloyd iteration over per-head codebooks [heads, n_centroids, sub_dim]
 * shared by all layers.  Every vector of x (all layers of head h train
 * codebook h) is rotated as kvq_vq_encode does and split into sub-vectors;
 *   1. assignment: idx_u16 receives, per sub-vector, the lowest index of a
 *      nearest centroid of codebook_f16 (exactly kvq_vq_encode's output);
 *   2. update: new_codebook_f16[h, k] = fp16 (round to nearest even) of the
 *      mean of the rotated sub-vectors assigned to centroid k of head h;
 *      a centroid with none keeps its value; counts[h, k] = how many.
 *   n_centroids   1 .. 4096;  sub_dim 8;
 *   new_codebook  16-byte aligned, may be codebook_f16 itself (in place);
 *   counts        uint32 [heads, n_centroids], 4-byte aligned;
 *   workspace     device scratch of at least kvq_kmeans_step_workspace()
 *                 bytes, 16-byte aligned, owned by the caller; no state is
 *                 kept in it between calls.
 * The sums are exact: each rotated coordinate is rounded to a multiple of
 * 2^-24 and added as a 64-bit integer, so the result does not depend on the
 * order of the additions and is the same on every run (|y| * n_k < 2^39 for
 * every centroid, n_k its sample count, keeps the sums in range); each mean
 * is then formed in fp64 and rounded once to fp16.  Views and errors as for
 * kvq_vq_encode; KVQ_ERR_SHAPE for a short workspace. */
kvq_status kvq_kmeans_step_workspace(kvq_shape shape, int32_t n_centroids, int32_t sub_dim,
                                     int64_t* bytes);
kvq_status kvq_kmeans_step(kvq_shape shape, kvq_view x_f16, const float* lambda,
                           const int8_t* signs, const void* codebook_f16, int32_t n_centroids,
                           int32_t sub_dim, kvq_view idx_u16, void* new_codebook_f16,
                           uint32_t* counts, void* workspace, int64_t workspace_bytes,
                           void* stream);

/* Decode attention straight from the int4 cache (VeloxQuant-MLX package
 * description, "Fused group-affine (KIVI-style) attention": one query per
 * head, online softmax accumulated in fp32, codes turned into values in
 * registers, no dequantized cache written).  For every outer index l, KV
 * head h and query head j = h * q_per_kv + r (0 <= r < q_per_kv), over the
 * first n_l tokens (n_l = lengths[l] clamped to [0, tokens], or all tokens
 * when lengths is NULL):
 *   khat_t, vhat_t = the kvq_dequantize values of token t's K and V codes,
 *                    unrounded,
 *   a_t = softmax_scale * (q_j . khat_t),  p = softmax_t(a),
 *   out_j = sum_t p_t vhat_t, rounded to fp16; an outer index with n_l = 0
 *   gets zeros.
 * It runs in the rotated domain: each query is rotated once (by the key
 * cache's lambda and signs), keys are never inverse-transformed, and the
 * weighted value sum is inverse-transformed once per query.  Scores,
 * weights and sums are fp32-accurate: for head_dim 128 with groups of 32 and
 * head_dim 256 with groups of 64 both contractions run on the matrix cores
 * with the query and the weights split into fp16 hi + lo halves and the
 * codes as exact fp16 integers; other shapes run on the vector ALUs in fp32.
 *   shape        layers = outer index (layers, or sequences sharing one
 *                layer), tokens = context capacity T, heads = KV heads,
 *                head_dim = D.
 *   q_per_kv     query heads per KV head, 1 .. 1024.
 *   q_f16        fp16 [layers, heads * q_per_kv, head_dim], contiguous,
 *                16-byte aligned; out_f16 likewise.
 *   k_codes_u8, k_scales_f16, v_codes_u8, v_scales_f16
 *                views as written by kvq_quantize (same alignment rules).
 *   lambda_k, lambda_v
 *                fp32 [layers, heads, head_dim], the lambdas the caches
 *                were quantized with; signs the shared sign vector.
 *   group        the caches' group size.
 *   lengths      device int32 [layers], or NULL.
 *   softmax_scale  finite; usually 1/sqrt(head_dim).
 *   workspace    device memory of at least kvq_attend_decode_workspace()
 *                bytes, 16-byte aligned, owned by the caller; its contents
 *                on entry do not matter and are overwritten.  Calls that
 *                share a workspace must not overlap.
 * Errors: as for kvq_quantize, plus KVQ_ERR_SHAPE when workspace_bytes is
 * smaller than needed.  layers == 0 or heads == 0 is a no-op. */
kvq_status kvq_attend_decode(kvq_shape shape, int32_t q_per_kv, const void* q_f16,
                             kvq_view k_codes_u8, kvq_view k_scales_f16,
                             kvq_view v_codes_u8, kvq_view v_scales_f16,
                             const float* lambda_k, const float* lambda_v,
                             const int8_t* signs, int32_t group, const int32_t* lengths,
                             float softmax_scale, void* out_f16, void* workspace,
                             int64_t workspace_bytes, void* stream);

/* Workspace bytes kvq_attend_decode needs for this shape and q_per_kv on the
 * current device (written to *bytes; 0 for an empty shape). */
kvq_status kvq_attend_decode_workspace(kvq_shape shape, int32_t q_per_kv, int64_t* bytes);

/* kvq_attend_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The partial states go to a static
 * device array of 64 MiB that the library holds on every GPU it runs on
 * until the process ends; nothing is allocated or freed by the call.
 * Arguments, results and errors are kvq_attend_decode's, plus KVQ_ERR_SHAPE
 * when the partial states of the kernel this call runs exceed 64 MiB (split
 * the call, or pass a workspace to kvq_attend_decode; any shape whose
 * kvq_attend_decode_workspace() is at most 64 MiB fits, and so do larger
 * ones on the matrix-core kernel, e.g. 36 layers x 8 sequences of 32K tokens
 * with 8 KV heads of 128 and 4 query heads each), and KVQ_ERR_HIP if the
 * array's device address cannot be looked up (done once per device, on the
 * first call with that device current).  All calls on one device share the
 * array: calls that overlap in time on one device (concurrent streams, or
 * threads) race and must be serialised by the caller; the array needs no
 * clearing between calls. */
kvq_status kvq_attend_decode_noalloc(kvq_shape shape, int32_t q_per_kv, const void* q_f16,
                                     kvq_view k_codes_u8, kvq_view k_scales_f16,
                                     kvq_view v_codes_u8, kvq_view v_scales_f16,
                                     const float* lambda_k, const float* lambda_v,
                                     const int8_t* signs, int32_t group, const int32_t* lengths,
                                     float softmax_scale, void* out_f16, void* stream);

/* Work decomposition of the quantize (inverse = 0) or dequantize
 * (inverse = 1) kernels for a shape, for the Walsh-Hadamard formats (int4,
 * int8, MXFP4; fourier = 0) or SRFT (fourier = 1); host arithmetic only, no
 * HIP call.  An item is 16 head vectors: 16/heads consecutive tokens of one
 * layer (all heads) when heads is above 1 and divides 16 (*token_major =
 * 1), else 16 consecutive tokens of one (layer, head) (*token_major = 0;
 * with one head the two orders give the same items).  Each
 * wavefront runs *items_per_wave consecutive items of the *n_items; the last
 * one may run fewer, and an item past the last token is partial.  Writes
 * zeros for an empty shape.  Errors as for kvq_quantize's shape checks,
 * KVQ_ERR_NULL for a NULL output pointer. */
kvq_status kvq_item_plan(kvq_shape shape, int32_t inverse, int32_t fourier, int32_t* token_major,
                         int64_t* n_items, int32_t* items_per_wave);

/* Static, human-readable name of a status code. */
const char* kvq_status_string(kvq_status status);

/* Detail of this thread's most recent non-OK return ("" if none); the
   pointer stays valid until this thread's next kvq_* call. */
const char* kvq_last_error(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int32_t kvq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
