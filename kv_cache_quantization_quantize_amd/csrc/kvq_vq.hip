// kvq_vq.hip -- product-VQ encode (MFMA nearest-centroid search) and decode
// for gfx950 (MI355X).
//
// The method (VecInfer blog, "What VecInfer does"; VeloxQuant-MLX package
// description, "Metal kernels"): keys are smooth-scaled and Walsh-Hadamard
// rotated, split into sub-vectors of 8, and each sub-vector is replaced by
// the index of its nearest centroid in the head's codebook; the search keeps
// its running argmin in registers and never materialises the [sub-vectors,
// centroids, 8] difference tensor.  Decode gathers the centroids back and
// undoes the rotation and the smooth scale.
//
// Encode.  argmin_k ||y - c_k||^2 = argmax_k (y . c_k - ||c_k||^2 / 2).  The
// dot products of 32 centroids x 32 sub-vectors are one
// v_mfma_f32_32x32x16_f16: A rows are centroids [c | c] (k = 0..15), B
// columns are sub-vectors [y_hi ; y_lo] with y_hi = fp16(y), y_lo =
// fp16(y - y_hi), so A.B = c.(y_hi + y_lo) = c.y to fp32 accuracy without
// rounding the key to fp16.  The accumulator input of those MFMAs is
// -(n_hi + n_lo)/2, the fp16 split of ||c||^2, computed once per centroid
// tile by a 32x32x8 MFMA and shared by every group of sub-vectors.  Each lane then holds the
// scores of 16 centroids for one sub-vector: a max3 tree gives the tile
// maximum, and only the best tile is tracked (strict >, so the earliest tile
// wins ties; with one-byte indices, the best quarter of a tile).  After a
// sweep, the lanes that improved re-score the 16 (4) candidates of their best
// tile (quarter) on VALU to find the position (first maximum, so the lowest
// index wins), and the two lanes that share a sub-vector (rows
// 0-3,8-11,.. and 4-7,12-15,..) merge (value, index) lexicographically.
//
// The codebook (<= 4096 centroids at a time, 64 KB) and its norms live in
// LDS; a block of WAVES wavefronts shares it, each wavefront rotating 16 keys
// of one (layer, head) and sweeping the codebook for GPR (up to 8) groups of
// 32 sub-vectors per pass.  Contraction work per key: D/8 x K x 8 MACs; the
// MFMAs execute 2x that for the hi/lo split plus one half-size norm MFMA per
// tile and GPR groups (2.125x for GPR = 8; in matrix-core time the norm MFMA
// costs as much as a full one, 2.25x).
//
// What bounds the sweep (measured on MI355X with a timing probe of the
// loop): a 32x32x16 f16 MFMA issues every 32 cycles, and the 32x32x8 norm
// MFMA takes as long; v_max3_f32 takes about 8 cycles per wavefront, and
// every score passes through one (16 scores per lane, group and tile, and the
// running best: 8 max3), so with two wavefronts per SIMD the maxima cost
// about as much SIMD time as the nine MFMAs of a tile.  The kernel therefore runs near the
// balance of the two units rather than at the matrix cores' peak.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Encoder shape.  Each wavefront issues a VALU instruction only every 5-6
// clocks, while the SIMD executes one in about two, so VALU-bound work runs
// faster with more wavefronts per SIMD.  The 4096-centroid encoder is bound
// by the matrix pipe during its sweep and keeps eight groups per sweep at two
// wavefronts per SIMD (four groups at three measured slower); the one-byte
// encoder (256 centroids, a short sweep and a longer maxima epilogue per
// tile) is VALU-bound and sweeps four groups at a time in four-wavefront
// blocks, which fit three wavefronts per SIMD (164 VGPRs): 0.917 -> 0.799 ms
// for 2.4 M value vectors on MI355X (two groups at four wavefronts per SIMD
// measured the same).
template <int D, bool IDX8 = false>
struct VqCfg {
    static constexpr int NS = D / 8;               // sub-vectors per key
    static constexpr int NJ = D / 32;              // 16-byte chunks per lane
    static constexpr int N = D / 4;                // coordinates per lane
    static constexpr int NGRP = D / 16;            // groups of 32 sub-vectors per 16 keys
    static constexpr int GMAX = IDX8 ? 4 : 8;
    static constexpr int GPR = NGRP < GMAX ? NGRP : GMAX;   // groups per codebook sweep
    static constexpr int ROUNDS = NGRP / GPR;
    static constexpr int WAVES = (D == 256 || IDX8) ? 4 : 8;  // wavefronts per block (LDS budget)
    static constexpr int MINW = IDX8 ? 3 : 1;      // waves per SIMD the registers must allow
};

// Wavefronts per block of the LDS-codebook decoder (one block per CU:
// 64 KB of codebook plus 16 vectors of output staging per wavefront).
template <int D>
struct VqDecLds {
    static constexpr int WAVES = (D == 256) ? 4 : 16;
};

__device__ __forceinline__ h8_t as_h8(uint4 u) { return __builtin_bit_cast(h8_t, u); }
__device__ __forceinline__ h4_t as_h4(uint2 u) { return __builtin_bit_cast(h4_t, u); }


// LDS slot of centroid k of a codebook chunk: rows are permuted within their
// 32-centroid tile by the tile index, k ^ ((k / 32) % 16).  The sweep reads a
// whole tile (one centroid per lane) and stays conflict-free; the re-score
// gathers the same row of different best tiles across lanes, which without
// the permutation all fall into the same four LDS banks (a 16-byte centroid
// per row, 32 rows per tile): measured on MI355X, 77% of the encoder's LDS
// cycles were bank conflicts.
__device__ __forceinline__ int cb_slot(int k) { return k ^ ((k >> 5) & 15); }

// Swizzled position of 16-byte sub-vector chunk s of key v in a staging row.
template <int NS>
__device__ __forceinline__ int stage_slot(int v, int s) { return v * NS + (s ^ ((4 * v) % NS)); }

}  // namespace

// IDX8: one-byte indices (codebooks of at most 256 centroids), else u16.
template <int D, bool IDX8>
__global__ __launch_bounds__((64 * VqCfg<D, IDX8>::WAVES), (VqCfg<D, IDX8>::MINW)) void vq_encode_kernel(VqArgs a)
{
    typedef typename std::conditional<IDX8, uint8_t, uint16_t>::type idx_t;
    using C = VqCfg<D, IDX8>;
    constexpr int NS = C::NS, NJ = C::NJ, N = C::N, GPR = C::GPR, ROUNDS = C::ROUNDS, WAVES = C::WAVES;

    // one-byte indices imply at most 256 centroids: a small codebook area
    // lets two blocks share a CU
    constexpr int CHUNK = IDX8 ? 256 : kVqChunk;
    // Best-score tracking granularity: sub-blocks of 16 / NSUB of a lane's 16
    // tile scores.  A 256-centroid codebook is eight tiles, so re-scoring all
    // 16 candidates of the best tile would cost more than the sweep; tracking
    // the best 4-score sub-block costs about ten more VALU operations per tile
    // and leaves four candidates (1.45 -> 0.96 ms for 2.4 M keys; sub-blocks
    // of 8 or 2 scores, or single scores, were slower).
    constexpr int NSUB = IDX8 ? 4 : 1, SUBW = 16 / NSUB;
    __shared__ uint4 cb_lds[CHUNK];                    // centroid k: 8 fp16
    __shared__ uint32_t nrm_lds[CHUNK];                // packed (n_hi, n_lo)
    __shared__ float hn_lds[CHUNK];                    // -(n_hi + n_lo) / 2, for the re-score
    __shared__ uint4 stage[WAVES][2][16 * NS];         // [wave][hi/lo][key, sub-vector]

    const int lane = threadIdx.x & 63;
    const int q = lane & 3;
    const int slot = lane >> 2;
    const int wid = uniform(threadIdx.x >> 6);
    const float c1 = (q & 1) ? -1.0f : 1.0f;
    const float c2 = (q & 2) ? -1.0f : 1.0f;
    const float lane_sign = (__builtin_popcount(q) & 1) ? -1.0f : 1.0f;
    const int col = lane & 31;                         // MFMA column (sub-vector in a group)
    const int half = lane >> 5;                        // 0: rows 0-3, 8-11, ..; 1: rows 4-7, ..

    // Norm tile: a 32x32x8 MFMA with A2 rows [n_hi, n_lo, 0, 0] (k = 0..3,
    // and the same words again in k = 4..7) and B2 columns [-1/2, -1/2, 0, 0]
    // in k = 0..3, zero in k = 4..7.
    const uint32_t mhalf2 = 0xB800B800u;               // two fp16 -0.5
    const h4_t b2 = as_h4(make_uint2(half == 0 ? mhalf2 : 0u, 0u));

    const int nchunks = (a.K + CHUNK - 1) / CHUNK;
    const int64_t ubeg = (int64_t)blockIdx.x * a.enc_units_per_block;
    const int64_t uend = min(ubeg + a.enc_units_per_block, a.enc_n_units);
    int cur_cb = -1;

    const _Float16* __restrict__ xg = static_cast<const _Float16*>(a.x.data);
    idx_t* __restrict__ ig = static_cast<idx_t*>(a.idx.data);

    for (int64_t u = ubeg; u < uend; ++u) {
        // ---- unit -> (layer, head, token chunk); codebook-major order ----------
        const int ui = uniform((int)u);
        const int c = ui % a.enc_units_per_lh;
        const int g2 = ui / a.enc_units_per_lh;
        int l, h;
        if (a.cb_layer_stride == 0) { h = uniform(g2 / a.L); l = g2 - h * a.L; }
        else { l = uniform(g2 / a.H); h = g2 - l * a.H; }
        const int lh = l * a.H + h;
        const int cbkey = a.cb_layer_stride == 0 ? h : lh;
        const uint16_t* cbp = a.codebook + (int64_t)l * a.cb_layer_stride + (int64_t)h * a.K * 8;
        float m[N];   // reloaded per unit so that it is not live during the sweeps
        load_fwd_mult<D>(a.lambda + (int64_t)lh * D, a.signs, q, m);

        // ---- rotate this wavefront's 16 keys (4 lanes per key) ---------------
        const int t0 = c * 16 * WAVES + wid * 16;
        const int t = t0 + slot;
        const bool valid = t < a.T;
        uint4 raw[NJ];
        {
            const _Float16* p = xg + (int64_t)l * a.x.sl + (int64_t)h * a.x.sh + (int64_t)t * a.x.st + q * 8;
#pragma unroll
            for (int j = 0; j < NJ; j++) raw[j] = make_uint4(0, 0, 0, 0);
            if (valid) {
#pragma unroll
                for (int j = 0; j < NJ; j++) raw[j] = *reinterpret_cast<const uint4*>(p + j * 32);
            }
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

        // ---- split y = y_hi + y_lo (fp16 each) and stage by sub-vector -------
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const float y0 = v[j * 8 + 2 * k] * lane_sign, y1 = v[j * 8 + 2 * k + 1] * lane_sign;
                const _Float16 h0 = (_Float16)y0, h1 = (_Float16)y1;
                const _Float16 r0 = (_Float16)(y0 - (float)h0), r1 = (_Float16)(y1 - (float)h1);
                hw[k] = __builtin_bit_cast(uint32_t, half2_t{h0, h1});
                lw[k] = __builtin_bit_cast(uint32_t, half2_t{r0, r1});
            }
            const int sl = stage_slot<NS>(slot, 4 * j + q);
            stage[wid][0][sl] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            stage[wid][1][sl] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }

        for (int rd = 0; rd < ROUNDS; rd++) {
            // B operands: group g covers sub-vectors 32g .. 32g+31 of the 16 keys
            h8_t bop[GPR];
#pragma unroll
            for (int gg = 0; gg < GPR; gg++) {
                const int sv = 32 * (rd * GPR + gg) + col;
                bop[gg] = as_h8(stage[wid][half][stage_slot<NS>(sv / NS, sv % NS)]);
            }
            float best_val[GPR];
            int best_idx[GPR];
#pragma unroll
            for (int gg = 0; gg < GPR; gg++) {
                best_val[gg] = -__builtin_inff();
                best_idx[gg] = 0;
            }

            for (int ch = 0; ch < nchunks; ch++) {
                const int kbase = ch * CHUNK;
                const int kc = min(CHUNK, a.K - kbase);
                if (nchunks > 1 || cbkey != cur_cb) {
                    // ---- stage codebook chunk + split norms (whole block) ----------
                    __syncthreads();
                    for (int k = threadIdx.x; k < CHUNK; k += 64 * WAVES) {
                        // Rows past the end of the codebook (only in the last tile of
                        // the last chunk) repeat the chunk's last centroid, K - 1:
                        // they score exactly as it does, so they never beat a real
                        // centroid, and an index they yield is mapped back to K - 1
                        // after the re-score.
                        const int kk = min(k, kc - 1);
                        const uint4 cv = *reinterpret_cast<const uint4*>(cbp + (int64_t)(kbase + kk) * 8);
                        const uint32_t w[4] = {cv.x, cv.y, cv.z, cv.w};
                        float n = 0.0f;
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            n = fmaf(lo_half(w[e]), lo_half(w[e]), n);
                            n = fmaf(hi_half(w[e]), hi_half(w[e]), n);
                        }
                        const _Float16 nh = (_Float16)n;
                        const _Float16 nl = (_Float16)(n - (float)nh);
                        cb_lds[cb_slot(k)] = cv;
                        nrm_lds[cb_slot(k)] = __builtin_bit_cast(uint32_t, half2_t{nh, nl});
                        hn_lds[cb_slot(k)] = -0.5f * ((float)nh + (float)nl);
                    }
                    __syncthreads();
                    cur_cb = nchunks > 1 ? -1 : cbkey;
                }

                // ---- sweep the chunk: 32 centroids per MFMA tile -------------------
                // The norm tile -(n_hi + n_lo)/2 is one MFMA per tile, shared by all
                // GPR groups as their accumulator input.  One accumulator per group:
                // group g's epilogue of tile t-1 runs right before its MFMA of tile t
                // (which overwrites the accumulator), GPR MFMAs after the one that
                // produced it, so the matrix core runs tile t while the VALU takes
                // the maxima of tile t-1.  (A second set of accumulators, with half
                // the groups per sweep, ran 4% slower and needed 64 more VGPRs.)
                const int ntiles = (kc + 31) / 32;
                int best_tile[GPR];
#pragma unroll
                for (int gg = 0; gg < GPR; gg++) best_tile[gg] = -1;
                auto read_a = [&](int tl, h8_t& aop, h4_t& a2) {
                    const int slot = cb_slot(tl * 32 + col);       // centroid tl * 32 + col
                    aop = as_h8(cb_lds[slot]);
                    a2 = as_h4(make_uint2(nrm_lds[slot], 0u));
                };
                auto norm_tile = [&](const h4_t& a2) {
                    const f32x16_t zero = {};
                    return __builtin_amdgcn_mfma_f32_32x32x8f16(a2, b2, zero, 0, 0, 0);
                };
                // Maximum of group gg's 16 tile scores (a max3 tree) against the
                // best so far, and the tile index where the best grew (strict >, so
                // the earliest tile keeps a tie; with one-byte indices, per quarter
                // of the tile's 16 scores).  The tree's temporary, unlike a chain
                // through the running best, lets the running maxima keep their
                // registers (a chain made the compiler rotate them: eight moves per
                // tile).
                // The running best goes into the tree (16 scores and it: eight max3),
                // read from bin and written to bout; with the full-tile tracking the
                // two arrays alternate from tile to tile, so no register is copied to
                // keep the running best in place (eight max3 and a compare and select
                // per group and tile); the sub-block tracking, shorter on registers,
                // updates one array in place.
                auto epilogue = [&](const f32x16_t& acc, int gg, int tl, const float (&bin)[GPR], float (&bout)[GPR]) {
                    if constexpr (NSUB == 1) {
                        float mx = fmaxf(fmaxf(bin[gg], acc[0]), acc[1]);
#pragma unroll
                        for (int r = 2; r < 16; r += 2) mx = fmaxf(fmaxf(mx, acc[r]), acc[r + 1]);
                        best_tile[gg] = mx > bin[gg] ? tl : best_tile[gg];
                        bout[gg] = mx;
                    } else {
                        float b = bin[gg];
#pragma unroll
                        for (int sb = 0; sb < NSUB; sb++) {
                            float nb = fmaxf(b, acc[SUBW * sb]);
#pragma unroll
                            for (int r = 1; r < SUBW; r++) nb = fmaxf(nb, acc[SUBW * sb + r]);
                            best_tile[gg] = nb > b ? tl * NSUB + sb : best_tile[gg];
                            b = nb;
                        }
                        bout[gg] = b;
                    }
                };
                constexpr int EPI_VALU = NSUB == 1 ? 10 : 11;   // VALU operations per group's epilogue
                float best_alt[GPR];
                f32x16_t acc[GPR], nt0, nt1;
                h8_t a_op;
                h4_t a_n2;
                read_a(0, a_op, a_n2);
                nt0 = norm_tile(a_n2);
#pragma unroll
                for (int gg = 0; gg < GPR; gg++)
                    acc[gg] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_op, bop[gg], nt0, 0, 0, 0);
                read_a(min(1, ntiles - 1), a_op, a_n2);
                // tile tl: the maxima of tile tl - 1, then tile tl's MFMAs; the norm
                // tiles alternate between two registers sets (unrolled by two)
                auto step = [&](int tl, f32x16_t& nt, const float (&bin)[GPR], float (&bout)[GPR]) {
                    nt = norm_tile(a_n2);
#pragma unroll
                    for (int gg = 0; gg < GPR; gg++) {
                        epilogue(acc[gg], gg, tl - 1, bin, bout);
                        acc[gg] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_op, bop[gg], nt, 0, 0, 0);
                    }
                    read_a(min(tl + 1, ntiles - 1), a_op, a_n2);
                    // norm MFMA, then each group's maxima right before its MFMA
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
                    for (int gg = 0; gg < GPR; gg++) {
                        __builtin_amdgcn_sched_group_barrier(0x002, EPI_VALU, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    }
                };
                // tile pairs take the running best from best_val to nxt and back
                auto sweep = [&](float (&nxt)[GPR]) {
                    int tl = 1;
                    for (; tl + 1 < ntiles; tl += 2) {
                        step(tl, nt1, best_val, nxt);
                        step(tl + 1, nt0, nxt, best_val);
                    }
                    if (tl < ntiles) {
                        step(tl, nt1, best_val, nxt);
#pragma unroll
                        for (int gg = 0; gg < GPR; gg++) epilogue(acc[gg], gg, ntiles - 1, nxt, best_val);
                    } else {
#pragma unroll
                        for (int gg = 0; gg < GPR; gg++) epilogue(acc[gg], gg, ntiles - 1, best_val, nxt);
#pragma unroll
                        for (int gg = 0; gg < GPR; gg++) best_val[gg] = nxt[gg];
                    }
                };
                if constexpr (NSUB == 1) sweep(best_alt);
                else sweep(best_val);

                // ---- lanes whose best moved into this chunk find its position -------
                // The GPR groups' candidates are scored together, one candidate row
                // of every group at a time, so that their LDS reads are in flight
                // together (scored one group after another, the dependent read ->
                // score chains left this phase latency-bound: a fifth of the
                // kernel's time).  Lanes whose best did not move into this chunk
                // (best_tile < 0) score tile 0 and discard the result.
                {
                    float y[GPR][8], bs[GPR];
                    int bt[GPR], r0[GPR], bk[GPR];
#pragma unroll
                    for (int gg = 0; gg < GPR; gg++) {
                        const int sv = 32 * (rd * GPR + gg) + col;
                        const int ss = stage_slot<NS>(sv / NS, sv % NS);
                        const uint4 yh = stage[wid][0][ss], yl = stage[wid][1][ss];
                        const uint32_t hwv[4] = {yh.x, yh.y, yh.z, yh.w}, lwv[4] = {yl.x, yl.y, yl.z, yl.w};
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            y[gg][2 * e] = lo_half(hwv[e]) + lo_half(lwv[e]);
                            y[gg][2 * e + 1] = hi_half(hwv[e]) + hi_half(lwv[e]);
                        }
                        const int b = max(best_tile[gg], 0);
                        bt[gg] = b / NSUB;
                        r0[gg] = SUBW * (b % NSUB);
                        bs[gg] = -__builtin_inff();
                        bk[gg] = 0;
                    }
#pragma unroll
                    for (int rr = 0; rr < SUBW; rr++) {
                        uint4 cv[GPR];
                        float sc[GPR];
                        int kk[GPR];
#pragma unroll
                        for (int gg = 0; gg < GPR; gg++) {
                            const int r = r0[gg] + rr;
                            kk[gg] = bt[gg] * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                            cv[gg] = cb_lds[cb_slot(kk[gg])];
                            sc[gg] = hn_lds[cb_slot(kk[gg])];
                        }
                        // the groups' dot products step by step, so that their
                        // dependent fma chains interleave
#pragma unroll
                        for (int e = 0; e < 4; e++) {
#pragma unroll
                            for (int gg = 0; gg < GPR; gg++) {
                                const uint32_t w = e == 0 ? cv[gg].x : e == 1 ? cv[gg].y : e == 2 ? cv[gg].z : cv[gg].w;
                                sc[gg] = fmaf(lo_half(w), y[gg][2 * e], sc[gg]);
                                sc[gg] = fmaf(hi_half(w), y[gg][2 * e + 1], sc[gg]);
                            }
                        }
#pragma unroll
                        for (int gg = 0; gg < GPR; gg++) {
                            if (sc[gg] > bs[gg]) {
                                bs[gg] = sc[gg];
                                bk[gg] = kk[gg];
                            }
                        }
                    }
#pragma unroll
                    for (int gg = 0; gg < GPR; gg++)
                        if (best_tile[gg] >= 0) best_idx[gg] = min(kbase + bk[gg], a.K - 1);  // a padded row is centroid K - 1
                }
            }

            // ---- merge the two row halves of each sub-vector, store indices --------
#pragma unroll
            for (int gg = 0; gg < GPR; gg++) {
                const float ov = __shfl_xor(best_val[gg], 32);
                const int oi = __shfl_xor(best_idx[gg], 32);
                int idx = best_idx[gg];
                if (ov > best_val[gg] || (ov == best_val[gg] && oi < idx)) idx = oi;
                const int sv = 32 * (rd * GPR + gg) + col;
                const int key = sv / NS, s = sv % NS;
                const int tk = t0 + key;
                if (half == 0 && tk < a.T)
                    ig[(int64_t)l * a.idx.sl + (int64_t)h * a.idx.sh + (int64_t)tk * a.idx.st + s] = (idx_t)idx;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Decode: indices -> centroids -> inverse transform -> unscale -> fp16
// ---------------------------------------------------------------------------
template <int D, bool TM>
__global__ __launch_bounds__(64 * kWavesPerBlock) void vq_decode_kernel(VqArgs a)
{
    constexpr int NJ = D / 32;          // 16-byte chunks (= sub-vectors) per lane
    constexpr int N = NJ * 8;
    constexpr int CV = D / 8;           // 16-byte chunks per vector
    constexpr int VPK = 1024 / (2 * D); // vectors per 1 KB store row
    constexpr int NIW = D / 64;         // 16-byte words of indices per key

    const int lane = threadIdx.x & 63;
    const int q = lane & 3;
    const int slot = lane >> 2;
    const int wave = uniform((int)(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)));
    if (wave >= a.dec_n_waves) return;
    // the wave's items [begin, end) all lie in group grp
    const int grp = uniform(wave / a.dec_waves_per_group);
    const int begin = (wave - grp * a.dec_waves_per_group) * a.items_per_wave;
    const int end = min(begin + a.items_per_wave, a.items_per_group);
    int l, hbase;
    if constexpr (TM) { l = grp; hbase = 0; }
    else { l = uniform(grp / a.H); hbase = grp - l * a.H; }

    const float c1 = (q & 1) ? -1.0f : 1.0f;
    const float c2 = (q & 2) ? -1.0f : 1.0f;
    const float lane_sign = (__builtin_popcount(q) & 1) ? -1.0f : 1.0f;
    const bool hi_pair = (q & 2) != 0;
    const uint32_t half_shift = (q & 1) * 16;
    const uint32_t kmax = (uint32_t)(a.K - 1);

    _Float16* __restrict__ og = static_cast<_Float16*>(a.x.data);
    const uint16_t* __restrict__ ig = static_cast<const uint16_t*>(a.idx.data);

    // lane's vector within an item: token offset and head (token-major items
    // hold 16/H tokens x H heads, head-major items 16 tokens of one head)
    const int ltok = TM ? (slot >> a.h_shift) : slot;
    const int lhead = TM ? (slot & (a.H - 1)) : 0;

    __shared__ uint4 lds_out[kWavesPerBlock][16 * CV];
    uint4* my_out = lds_out[threadIdx.x >> 6];
    const int row_c = lane % CV;

    // The quad's key index block (D/8 u16); tokens past the end read the last
    // token's block so that every load is in bounds and unconditional.
    typedef uint4 uint4_a4 __attribute__((aligned(4)));
    const uint16_t* ig_lh = ig + (int64_t)l * a.idx.sl + (int64_t)(hbase + lhead) * a.idx.sh;
    auto load_idx = [&](int item, uint4 (&W)[NIW]) {
        const int t = min(item * a.tok_per_item + ltok, a.T - 1);
        const uint16_t* ip = ig_lh + (int64_t)t * a.idx.st;
#pragma unroll
        for (int i = 0; i < NIW; i++) W[i] = *reinterpret_cast<const uint4_a4*>(ip + 8 * i);
    };
    // Lane q holds sub-vectors 4j + q; gather their centroids (clamped index).
    const uint16_t* cbp = a.codebook + (int64_t)l * a.cb_layer_stride + (int64_t)(hbase + lhead) * a.K * 8;
    auto gather = [&](const uint4 (&W)[NIW], uint4 (&cv)[NJ]) {
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const uint4 wd = W[j / 2];
            const uint32_t d = (j & 1) ? (hi_pair ? wd.w : wd.z) : (hi_pair ? wd.y : wd.x);
            const uint32_t ix = min(__builtin_amdgcn_ubfe(d, half_shift, 16), kmax);
            cv[j] = *reinterpret_cast<const uint4*>(cbp + (int64_t)ix * 8);
        }
    };

    float m[N];
    load_inv_mult<D>(a.lambda + ((int64_t)l * a.H + hbase + lhead) * D, a.signs, q, lane_sign, m);
    _Float16* og_l = og + (int64_t)l * a.x.sl + (int64_t)hbase * a.x.sh;
    auto compute_store = [&](int item, const uint4 (&cv)[NJ]) {
        const int t0 = item * a.tok_per_item;
        // first butterfly stage straight from the fp16 centroid values
        float v[N];
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const uint32_t wd[4] = {cv[j].x, cv[j].y, cv[j].z, cv[j].w};
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const float x0 = lo_half(wd[k]), x1 = hi_half(wd[k]);
                v[j * 8 + 2 * k] = x0 + x1;
                v[j * 8 + 2 * k + 1] = x0 - x1;
            }
        }
        fwht_rest(v, c1, c2);
        // stage through LDS so each store instruction writes 1 KB of consecutive vectors
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            uint4 o;
            o.x = pack_half2(v[j * 8 + 0] * m[j * 8 + 0], v[j * 8 + 1] * m[j * 8 + 1]);
            o.y = pack_half2(v[j * 8 + 2] * m[j * 8 + 2], v[j * 8 + 3] * m[j * 8 + 3]);
            o.z = pack_half2(v[j * 8 + 4] * m[j * 8 + 4], v[j * 8 + 5] * m[j * 8 + 5]);
            o.w = pack_half2(v[j * 8 + 6] * m[j * 8 + 6], v[j * 8 + 7] * m[j * 8 + 7]);
            my_out[slot * CV + ((4 * j + q) ^ ((4 * slot) % CV))] = o;
        }
        // A vector past the last token was decoded from the last token's
        // indices (the loads are clamped), so its row is stored over that
        // token's row with identical bytes: every store is unconditional.
        _Float16* ob = og_l + (int64_t)t0 * a.x.st;
        const int last = a.T - 1 - t0;
#pragma unroll
        for (int k = 0; k < NJ; k++) {
            const int vv = k * VPK + lane / CV;
            const uint4 rowv = my_out[vv * CV + (row_c ^ ((4 * vv) % CV))];
            const int vt = min(TM ? (vv >> a.h_shift) : vv, last);
            const int vh = TM ? (vv & (a.H - 1)) : 0;
            const int64_t off = (int64_t)vt * a.x.st + (int64_t)vh * a.x.sh + row_c * 8;
            *reinterpret_cast<uint4*>(ob + off) = rowv;
        }
    };

    // Pipeline: while item i is computed, the centroids of item i + 1 and
    // the indices of item i + 2 are in flight.  All loads are unconditional
    // (items past the wave's range are clamped to its last item) so that the
    // wait before each use is a fixed count; the two centroid buffers
    // alternate by unrolling, never by copying registers that may still be
    // waiting on a load.
    uint4 W[NIW];
    uint4 cvA[NJ], cvB[NJ];
    load_idx(begin, W);
    gather(W, cvA);
    load_idx(min(begin + 1, end - 1), W);
    auto step = [&](int item, const uint4 (&cur)[NJ], uint4 (&nxt)[NJ]) {
        gather(W, nxt);
        load_idx(min(item + 2, end - 1), W);
        __builtin_amdgcn_sched_barrier(0);   // issue the loads before the compute
        compute_store(item, cur);
    };
    // The first step is peeled so that the loop is entered with the same
    // loads and stores in flight as on its back edge.
    step(begin, cvA, cvB);
    for (int item = begin + 1; item < end;) {
        step(item, cvB, cvA);
        if (++item >= end) break;
        step(item, cvA, cvB);
        ++item;
    }
}

// Decode with the head's codebook staged in LDS (n_centroids <= kVqChunk).
// Work items are runs of 16 tokens of one (layer, head).  A block decodes one
// head over a contiguous range of (layer, 16-token tile) rows (one block per
// CU), stages the codebook when it changes, and its wavefronts split each
// layer's part of the range into contiguous runs.  The centroid gathers are
// LDS reads rather than 16-byte pieces of L2 lines.  Each wavefront keeps the
// indices of its next three items in flight.
template <int D, bool IDX8>
__global__ __launch_bounds__(64 * VqDecLds<D>::WAVES) void vq_decode_lds_kernel(VqArgs a)
{
    constexpr int WAVES = VqDecLds<D>::WAVES;
    constexpr int NJ = D / 32;
    constexpr int N = NJ * 8;
    constexpr int CV = D / 8;
    constexpr int VPK = 1024 / (2 * D);
    constexpr int IB = (D / 8) * (IDX8 ? 1 : 2);   // index bytes per key
    constexpr int NIW = (IB + 15) / 16;           // 16-byte loads (8 bytes: one 8-byte load)

    __shared__ uint4 cb_lds[kVqChunk];
    __shared__ uint4 lds_out[WAVES][16 * CV];

    const int lane = threadIdx.x & 63;
    const int q = lane & 3;
    const int slot = lane >> 2;
    const int wid = uniform(threadIdx.x >> 6);

    const float c1 = (q & 1) ? -1.0f : 1.0f;
    const float c2 = (q & 2) ? -1.0f : 1.0f;
    const float lane_sign = (__builtin_popcount(q) & 1) ? -1.0f : 1.0f;
    const bool hi_pair = (q & 2) != 0;
    const uint32_t half_shift = (q & 1) * 16;
    const uint32_t byte_shift = q * 8;
    const uint32_t kmax = (uint32_t)(a.K - 1);

    _Float16* __restrict__ og = static_cast<_Float16*>(a.x.data);
    const uint8_t* __restrict__ ig = static_cast<const uint8_t*>(a.idx.data);
    constexpr int ISZ = IDX8 ? 1 : 2;             // index strides are in elements
    uint4* my_out = lds_out[wid];
    const int row_c = lane % CV;
    typedef uint4 uint4_a4 __attribute__((aligned(4)));
    typedef uint2 uint2_a4 __attribute__((aligned(4)));

    // Block b runs on XCD b % 8.  Its head is (b / 8) % H and its row range
    // is ((b / 8) / H) * 8 + b % 8, so the H blocks of a range share an XCD
    // (and its L2) and run concurrently.
    const int xcd = blockIdx.x & 7;
    const int kx = blockIdx.x >> 3;
    const int grp = kx / a.H;
    const int h = kx - grp * a.H;
    const int64_t rows = (int64_t)a.L * a.items_per_group;
    const int64_t r0 = ((int64_t)grp * 8 + xcd) * a.dec_rows_per_range;
    const int64_t g_end = min(r0 + a.dec_rows_per_range, rows);
    int staged = -1;
    for (int64_t g = r0; g < g_end;) {
        const int l = uniform((int)(g / a.items_per_group));
        const int64_t seg0 = (int64_t)l * a.items_per_group;
        const int i0 = (int)(g - seg0);
        const int i1 = (int)(min(g_end, seg0 + a.items_per_group) - seg0);
        g = seg0 + i1;

        // stage the codebook of (l, h), K centroids of 16 bytes, unless the
        // one in LDS is already it (one codebook for all layers)
        const int cb_l = a.cb_layer_stride ? l : 0;
        if (cb_l != staged) {
            __syncthreads();   // the previous segment's gathers are done
            const uint4* cbg = reinterpret_cast<const uint4*>(a.codebook + (int64_t)cb_l * a.cb_layer_stride +
                                                              (int64_t)h * a.K * 8);
            for (int k = threadIdx.x; k < a.K; k += 64 * WAVES) cb_lds[k] = cbg[k];
            __syncthreads();
            staged = cb_l;
        }

        const int per_wave = (i1 - i0 + WAVES - 1) / WAVES;
        const int begin = i0 + wid * per_wave;
        const int end = min(begin + per_wave, i1);
        if (begin >= end) continue;

        const uint8_t* ig_lh = ig + ((int64_t)l * a.idx.sl + (int64_t)h * a.idx.sh) * ISZ;
        // Per-lane parts of the index and output addresses, fixed for the
        // segment.  The host sends only T >= 16 here, and an item's first
        // token is clamped to T - 16: the last item of a (layer, head) ends at
        // its last token and recomputes (rewrites with the same bytes) the
        // tokens it shares with the item before it, so no load or store is
        // ever masked or clamped per lane.
        const int64_t idx_lane = (int64_t)slot * a.idx.st * ISZ;
        const int64_t out_lane = (int64_t)(lane / CV) * a.x.st + row_c * 8;     // + k * VPK rows
        auto first_token = [&](int item) { return min(item * kTokensPerTile, a.T - kTokensPerTile); };
        // the quad's index row
        auto load_idx = [&](int item, uint4 (&W)[NIW]) {
            const uint8_t* ip = ig_lh + (int64_t)first_token(item) * a.idx.st * ISZ + idx_lane;
            if constexpr (IB >= 16) {
#pragma unroll
                for (int i = 0; i < NIW; i++) W[i] = *reinterpret_cast<const uint4_a4*>(ip + 16 * i);
            } else {
                const uint2 w2 = *reinterpret_cast<const uint2_a4*>(ip);
                W[0] = make_uint4(w2.x, w2.y, 0u, 0u);
            }
        };

        float m[N];
        load_inv_mult<D>(a.lambda + ((int64_t)l * a.H + h) * D, a.signs, q, lane_sign, m);
        _Float16* og_lh = og + (int64_t)l * a.x.sl + (int64_t)h * a.x.sh;

        // One item: centroids from LDS, then the indices of item + 3 into the
        // same buffer, then the inverse transform and the stores.
        auto step = [&](int item, uint4 (&W)[NIW]) {
            item = min(item, end - 1);
            // lane q holds sub-vectors 4j + q
            uint4 cv[NJ];
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                uint32_t k;
                if constexpr (IDX8) {
                    // sub-vector 4j + q is byte q of word j % 4 of 16-byte piece j / 4
                    const uint4 wd = W[j / 4];
                    const uint32_t d = (j & 3) == 0 ? wd.x : (j & 3) == 1 ? wd.y : (j & 3) == 2 ? wd.z : wd.w;
                    k = __builtin_amdgcn_ubfe(d, byte_shift, 8);
                } else {
                    const uint4 wd = W[j / 2];
                    const uint32_t d = (j & 1) ? (hi_pair ? wd.w : wd.z) : (hi_pair ? wd.y : wd.x);
                    k = __builtin_amdgcn_ubfe(d, half_shift, 16);
                }
                cv[j] = cb_lds[min(k, kmax)];
            }
            load_idx(min(item + 3, end - 1), W);
            __builtin_amdgcn_sched_barrier(0);   // issue the indices before the compute
            float v[N];
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                const uint32_t wd[4] = {cv[j].x, cv[j].y, cv[j].z, cv[j].w};
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    const float x0 = lo_half(wd[k]), x1 = hi_half(wd[k]);
                    v[j * 8 + 2 * k] = x0 + x1;
                    v[j * 8 + 2 * k + 1] = x0 - x1;
                }
            }
            fwht_rest(v, c1, c2);
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                uint4 o;
                o.x = pack_half2(v[j * 8 + 0] * m[j * 8 + 0], v[j * 8 + 1] * m[j * 8 + 1]);
                o.y = pack_half2(v[j * 8 + 2] * m[j * 8 + 2], v[j * 8 + 3] * m[j * 8 + 3]);
                o.z = pack_half2(v[j * 8 + 4] * m[j * 8 + 4], v[j * 8 + 5] * m[j * 8 + 5]);
                o.w = pack_half2(v[j * 8 + 6] * m[j * 8 + 6], v[j * 8 + 7] * m[j * 8 + 7]);
                my_out[slot * CV + ((4 * j + q) ^ ((4 * slot) % CV))] = o;
            }
            _Float16* ob = og_lh + (int64_t)first_token(item) * a.x.st;
#pragma unroll
            for (int k = 0; k < NJ; k++) {
                const int vv = k * VPK + lane / CV;
                const uint4 rowv = my_out[vv * CV + (row_c ^ ((4 * vv) % CV))];
                *reinterpret_cast<uint4*>(ob + out_lane + (int64_t)(k * VPK) * a.x.st) = rowv;
            }
        };

        // Three index buffers in rotation.  Steps past the run repeat its
        // last item (same bytes to the same places), so every step is
        // unconditional and the first three, peeled, leave the same loads
        // and stores in flight as the loop's back edge.
        uint4 WA[NIW], WB[NIW], WC[NIW];
        load_idx(begin, WA);
        load_idx(min(begin + 1, end - 1), WB);
        load_idx(min(begin + 2, end - 1), WC);
        step(begin, WA);
        step(begin + 1, WB);
        step(begin + 2, WC);
        for (int item = begin + 3; item < end; item += 3) {
            step(item, WA);
            step(item + 1, WB);
            step(item + 2, WC);
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {

template <int D>
hipError_t launch_enc(const VqArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)((a.enc_n_units + a.enc_units_per_block - 1) / a.enc_units_per_block));
    if (a.idx8) hipLaunchKernelGGL((vq_encode_kernel<D, true>), grid, dim3(64 * VqCfg<D, true>::WAVES), 0, s, a);
    else hipLaunchKernelGGL((vq_encode_kernel<D, false>), grid, dim3(64 * VqCfg<D, false>::WAVES), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dec(const VqArgs& a, hipStream_t s)
{
    if (a.dec_rows_per_range > 0) {
        const dim3 grid((unsigned)(8 * a.H * a.dec_range_groups));
        if (a.idx8) hipLaunchKernelGGL((vq_decode_lds_kernel<D, true>), grid, dim3(64 * VqDecLds<D>::WAVES), 0, s, a);
        else hipLaunchKernelGGL((vq_decode_lds_kernel<D, false>), grid, dim3(64 * VqDecLds<D>::WAVES), 0, s, a);
        return hipGetLastError();
    }
    if (a.idx8) return hipErrorInvalidValue;   // one-byte indices imply K <= 256: the LDS path
    const dim3 grid((unsigned)((a.dec_n_waves + kWavesPerBlock - 1) / kWavesPerBlock));
    if (a.token_major) hipLaunchKernelGGL((vq_decode_kernel<D, true>), grid, dim3(64 * kWavesPerBlock), 0, s, a);
    else hipLaunchKernelGGL((vq_decode_kernel<D, false>), grid, dim3(64 * kWavesPerBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int vq_encode_waves(int D, bool idx8)
{
    if (idx8) return D == 256 ? VqCfg<256, true>::WAVES : VqCfg<128, true>::WAVES;
    return D == 256 ? VqCfg<256>::WAVES : VqCfg<128>::WAVES;
}

hipError_t launch_vq_encode(const VqArgs& a, hipStream_t s)
{
    switch (a.D) {
        case 64: return launch_enc<64>(a, s);
        case 128: return launch_enc<128>(a, s);
        case 256: return launch_enc<256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_vq_decode(const VqArgs& a, hipStream_t s)
{
    switch (a.D) {
        case 64: return launch_dec<64>(a, s);
        case 128: return launch_dec<128>(a, s);
        case 256: return launch_dec<256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
