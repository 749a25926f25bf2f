// Sign flips + blockwise Sylvester Hadamard regularization on gfx950.
//
// Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture
// section 7 (natural-order Sylvester Hadamard normalised by 1/sqrt(B), applied
// per block of B rows on the left and per block of B columns on the right, not
// as one Kronecker transform; decode applies H_l, x su, H_r, x sv) and
// section 8 (per-tile energy for the scale search).
//
//   W_reg = H_l diag(su) W diag(sv) H_r
// evaluated as: sign flips (exact), left fast Walsh-Hadamard transform with
// levels h = 1, 2, ..., B/2 (pairs (p, p+h), p mod 2h < h, become (a+b, a-b)),
// x rn(1/sqrt(B)), the same transform along rows, x rn(1/sqrt(B)).
//
// One workgroup of 2B lanes per B x B block (the blocks are independent):
// coalesced 16-byte loads into LDS, then each column's left transform split
// over a lane pair, the block turned around in LDS, each row's right transform
// split the same way, and a tile-major stage in LDS from which each of the
// block's (B/16)^2 tiles gets its sequential binary32 sum of squares and the
// output is written (tile-major or row-major).  HBM-bound: 6 bytes per element
// for bf16 input (2 in, 4 out).
//
// Tile-major position t of a tile holds the tile's element order[t]
// (element 16 r + c), order being the context's within-tile order (the
// README's tensor-core permutation slot, section 5); without one, element t.
#include "exl3_internal.h"

#include <math.h>

namespace exl3 {
namespace {

__device__ __forceinline__ float load_w(const float *w, size_t i) { return w[i]; }
__device__ __forceinline__ float load_w(const uint16_t *w, size_t i) {
    return __uint_as_float((uint32_t)w[i] << 16);   // bf16 -> fp32 is exact
}

template <int B>
__device__ __forceinline__ void fwht_regs(float (&a)[B]) {
#pragma unroll
    for (int h = 1; h < B; h <<= 1)
#pragma unroll
        for (int p = 0; p < B; ++p)
            if ((p & h) == 0) {
                float u = a[p], w = a[p + h];
                a[p] = u + w;
                a[p + h] = u - w;
            }
}

template <int B>
__device__ __forceinline__ float norm_const() {
    return B == 64 ? 0.125f : __uint_as_float(0x3DB504F3u);   // rn(1/sqrt(128))
}

// One workgroup of 2B lanes per B x B block.  Lane l works as half h = (l >> 5)
// & 1 of index i = (l & 31) + 32 (l >> 6): in the left transform it holds rows
// h B/2 .. h B/2 + B/2 - 1 of column i, in the right transform columns
// h B/2 .. of row i.  The levels h < B/2 of a transform run in registers; the
// last level pairs each value with the same position of the other half, held
// by lane l ^ 32 of the same wave (exchanged with v_permlane32_swap, no LDS).
//
//   1. 16-byte loads of the block's rows (coalesced), signs applied, into LDS
//      (blk_word);
//   2. left transform along columns, x rn(1/sqrt(B)), back to LDS;
//   3. right transform along rows, x rn(1/sqrt(B)) (row-major output written
//      from registers);
//   4. the block in trellis order into a tile-major LDS stage (tile stride
//      274 words, 17 words per tile row: conflict-free stores);
//   5. per-tile sequential sum of squares, one lane per tile;
//   6. tile-major output from the stage, consecutive lanes on consecutive
//      positions.
constexpr int kStageRow = 17;       // LDS words per 16-element tile row in the stage
constexpr int kStageTile = 274;     // LDS words per tile in the stage

__device__ __forceinline__ int stage_word(int t) { return (t >> 4) * kStageRow + (t & 15); }


// The last butterfly level, across the two halves of the wave: one
// v_permlane32_swap of the value with itself leaves the top half's value
// (lanes 0..31) in the first result and the bottom half's (lanes 32..63) in
// the second, in every lane; the lower half keeps top + bottom, the upper half
// top - bottom, as fma(+-1, bottom, top): the product is exact, so the single
// rounding is that of the addition or subtraction.
__device__ __forceinline__ float last_level(float own, float sgn) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(own), __float_as_uint(own),
                                                    false, false);
    return __builtin_fmaf(sgn, __uint_as_float(r[1]), __uint_as_float(r[0]));
}

// LDS word of block element (row, col): rows of B + 1 words, so that the
// column-wise and the row-wise accesses of the transforms hit 32 distinct
// banks per half-wave (the first phase's stores, 8 consecutive columns per
// lane, conflict 4-way; a skew that removes that needs more LDS than two
// workgroups per compute unit leave).
template <int B>
__device__ __forceinline__ int blk_word(int row, int col) { return row * (B + 1) + col; }
template <int B>
constexpr int blk_words() { return B * (B + 1); }

template <typename Tin>
__device__ __forceinline__ void unpack16(const uint4 &u, float (&v)[16 / sizeof(Tin)]);
template <>
__device__ __forceinline__ void unpack16<uint16_t>(const uint4 &u, float (&v)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);             // bf16 -> fp32 is exact
        v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
}
template <>
__device__ __forceinline__ void unpack16<float>(const uint4 &u, float (&v)[4]) {
    v[0] = __uint_as_float(u.x);
    v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z);
    v[3] = __uint_as_float(u.w);
}

// VEC: the weights start on a 16-byte boundary (else one element per load).
template <int B, typename Tin, bool VEC, bool ORDERED>
__global__ void __launch_bounds__(2 * B)
regularize_kernel(const Tin *__restrict__ w, int rows, int cols, const float *__restrict__ su,
                  const float *__restrict__ sv, float *__restrict__ out, int layout,
                  float *__restrict__ tile_sumsq, int *__restrict__ nonfinite,
                  const uint8_t *__restrict__ order) {
    constexpr int H = B / 2;          // values per lane in a transform
    constexpr int TB = B / 16;        // tiles per block side
    constexpr int kWords = blk_words<B>() > TB * TB * kStageTile ? blk_words<B>()
                                                                  : TB * TB * kStageTile;
    __shared__ float smem[kWords];
    __shared__ float sgn[2 * B];      // the block's column signs, then its row signs
    __shared__ uint8_t inv[256];      // element -> trellis position (ORDERED)
    const int l = threadIdx.x;
    const int r0 = blockIdx.y * B, c0 = blockIdx.x * B;
    const int TC = cols / 16;
    const float c = norm_const<B>();
    const int idx = (l & 31) + 32 * (l >> 6), half = (l >> 5) & 1;
    const float sgn_half = half ? -1.0f : 1.0f;

    // 1. load, signs (exact), into LDS
    bool bad = false;
    if constexpr (VEC) {
        constexpr int EPC = 16 / sizeof(Tin);       // elements per 16-byte load
        constexpr int CPR = B / EPC;                // loads per block row
        constexpr int NL = B * CPR / (2 * B);       // loads per lane
        uint4 u[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int q = l + 2 * B * i, rr = q / CPR, cb = (q % CPR) * EPC;
            u[i] = *reinterpret_cast<const uint4 *>(w + (size_t)(r0 + rr) * cols + c0 + cb);
        }
        sgn[l] = l < B ? sv[c0 + l] : su[r0 + l - B];
        if constexpr (ORDERED)
            for (int t = l; t < 256; t += 2 * B) inv[order[t]] = (uint8_t)t;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int q = l + 2 * B * i, rr = q / CPR, cb = (q % CPR) * EPC;
            float v[EPC];
            unpack16<Tin>(u[i], v);
            const float sr = sgn[B + rr];
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                bad |= !isfinite(v[e]);
                smem[blk_word<B>(rr, cb + e)] = (v[e] * sr) * sgn[cb + e];
            }
        }
    } else {
        if constexpr (ORDERED)
            for (int t = l; t < 256; t += 2 * B) inv[order[t]] = (uint8_t)t;
        for (int q = l; q < B * B; q += 2 * B) {
            const int rr = q / B, cc = q % B;
            const float v = load_w(w, (size_t)(r0 + rr) * cols + c0 + cc);
            bad |= !isfinite(v);
            smem[blk_word<B>(rr, cc)] = (v * su[r0 + rr]) * sv[c0 + cc];
        }
    }
    if (bad && nonfinite) *nonfinite = 1;
    __syncthreads();

    // 2. left transform: column idx, rows half * H ..
    float a[H];
#pragma unroll
    for (int r = 0; r < H; ++r) a[r] = smem[blk_word<B>(half * H + r, idx)];
    fwht_regs<H>(a);
#pragma unroll
    for (int r = 0; r < H; ++r) a[r] = last_level(a[r], sgn_half);
#pragma unroll
    for (int r = 0; r < H; ++r) smem[blk_word<B>(half * H + r, idx)] = a[r] * c;
    __syncthreads();

    // 3. right transform: row idx, columns half * H ..
#pragma unroll
    for (int q = 0; q < H; ++q) a[q] = smem[blk_word<B>(idx, half * H + q)];
    fwht_regs<H>(a);
#pragma unroll
    for (int q = 0; q < H; ++q) a[q] = last_level(a[q], sgn_half) * c;
    if (layout != 1) {
        float *dst = out + (size_t)(r0 + idx) * cols + c0 + half * H;
#pragma unroll
        for (int q = 0; q < H; q += 4)
            *reinterpret_cast<float4 *>(dst + q) = make_float4(a[q], a[q + 1], a[q + 2], a[q + 3]);
    }
    if (layout != 1 && !tile_sumsq) return;
    __syncthreads();                  // the block in LDS is read; the stage reuses it

    // 4. trellis order into the tile-major stage
    {
        const int tr = idx >> 4, rin = idx & 15;
#pragma unroll
        for (int q = 0; q < H; ++q) {
            const int cc = half * H + q;
            const int el = 16 * rin + (cc & 15);
            const int t = ORDERED ? inv[el] : el;
            smem[(tr * TB + (cc >> 4)) * kStageTile + stage_word(t)] = a[q];
        }
    }
    __syncthreads();

    // 5. per-tile sequential binary32 sum of squares, trellis order: wave 0,
    // one lane per tile (reads unrolled ahead of the dependent additions)
    if (tile_sumsq && l < 64) {
        if (l < TB * TB) {
            const float *T = smem + l * kStageTile;
            float acc = 0.0f;
#pragma unroll 16
            for (int t = 0; t < 256; ++t) {
                const float v = T[stage_word(t)];
                const float sq = v * v;
                acc = acc + sq;
            }
            tile_sumsq[(size_t)(r0 / 16 + l / TB) * TC + (c0 / 16 + l % TB)] = acc;
        }
        return;
    }

    // 6. tile-major output (the other waves, or all of them without energies):
    // four consecutive positions per lane and store, eight stores' reads issued
    // ahead
    if (layout == 1) {
        const int first = tile_sumsq ? 64 : 0;
        const int nl = 2 * B - first;
        constexpr int kQuads = B * B / 4;
        for (int g0 = l - first; g0 < kQuads; g0 += 8 * nl) {
            float4 v[8];
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int g = g0 + b * nl;
                if (g < kQuads) {
                    const float *T = smem + (g >> 6) * kStageTile;
                    const int t = 4 * (g & 63);
                    v[b] = make_float4(T[stage_word(t)], T[stage_word(t + 1)],
                                       T[stage_word(t + 2)], T[stage_word(t + 3)]);
                }
            }
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int g = g0 + b * nl;
                if (g < kQuads) {
                    const int lt = g >> 6, t = 4 * (g & 63);
                    const size_t tau = (size_t)(r0 / 16 + lt / TB) * TC + (c0 / 16 + lt % TB);
                    *reinterpret_cast<float4 *>(out + tau * 256 + t) = v[b];
                }
            }
        }
    }
}

// Inverse of the regularization (H is symmetric and orthonormal, so its own
// inverse): W = diag(su) H_l W_reg H_r diag(sv), evaluated as left transform,
// x rn(1/sqrt(B)), right transform, x rn(1/sqrt(B)), then x su[row], x sv[col]
// (su, sv may be the folded channel scales, not only +-1).  Input tile-major
// or row-major, output row-major.
template <int B>
__global__ void __launch_bounds__(B)
unregularize_kernel(const float *__restrict__ in, int rows, int cols, int in_layout,
                    const float *__restrict__ su, const float *__restrict__ sv,
                    float *__restrict__ out, const uint8_t *__restrict__ order) {
    __shared__ float blk[B][B + 1];
    const int j = threadIdx.x;
    const int r0 = blockIdx.y * B, c0 = blockIdx.x * B;
    const float c = norm_const<B>();
    const int TC = cols / 16;
    constexpr int TB = B / 16;
    for (int idx = j; idx < B * B; idx += B) {
        int rr, cc;
        size_t src;
        if (in_layout == 1) {
            const int lt = idx >> 8, t = idx & 255, tr = lt / TB, tc = lt % TB;
            const int el = order ? order[t] : t;
            rr = tr * 16 + (el >> 4);
            cc = tc * 16 + (el & 15);
            src = ((size_t)(r0 / 16 + tr) * TC + (c0 / 16 + tc)) * 256 + t;
        } else {
            rr = idx / B;
            cc = idx % B;
            src = (size_t)(r0 + rr) * cols + c0 + cc;
        }
        blk[rr][cc] = in[src];
    }
    __syncthreads();
    float a[B];
#pragma unroll
    for (int r = 0; r < B; ++r) a[r] = blk[r][j];
    fwht_regs<B>(a);
#pragma unroll
    for (int r = 0; r < B; ++r) blk[r][j] = a[r] * c;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < B; ++q) a[q] = blk[j][q];
    fwht_regs<B>(a);
#pragma unroll
    for (int q = 0; q < B; ++q) blk[j][q] = a[q] * c;
    __syncthreads();
    for (int idx = j; idx < B * B; idx += B) {
        const int rr = idx / B, cc = idx % B;
        out[(size_t)(r0 + rr) * cols + c0 + cc] = (blk[rr][cc] * su[r0 + rr]) * sv[c0 + cc];
    }
}

template <int B, typename Tin>
hipError_t launch_reg_t(const void *w, int rows, int cols, const float *su, const float *sv,
                        float *out, int layout, float *tile_sumsq, int *nonfinite,
                        const uint8_t *order, hipStream_t stream) {
    dim3 grid(cols / B, rows / B);
    const Tin *wt = reinterpret_cast<const Tin *>(w);
    const bool vec = reinterpret_cast<uintptr_t>(w) % 16 == 0;
#define EXL3_REG_LAUNCH(V, O)                                                                \
    hipLaunchKernelGGL((regularize_kernel<B, Tin, V, O>), grid, dim3(2 * B), 0, stream, wt,  \
                       rows, cols, su, sv, out, layout, tile_sumsq, nonfinite, order)
    if (vec && order) EXL3_REG_LAUNCH(true, true);
    else if (vec) EXL3_REG_LAUNCH(true, false);
    else if (order) EXL3_REG_LAUNCH(false, true);
    else EXL3_REG_LAUNCH(false, false);
#undef EXL3_REG_LAUNCH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_unregularize(const float *in, int in_layout, int rows, int cols, int had_block,
                               const float *su, const float *sv, float *out,
                               const uint8_t *order, hipStream_t stream) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    if (had_block != 64 && had_block != 128) return hipErrorInvalidValue;
    dim3 grid(cols / had_block, rows / had_block);
    if (had_block == 64)
        hipLaunchKernelGGL(unregularize_kernel<64>, grid, dim3(64), 0, stream, in, rows, cols,
                           in_layout, su, sv, out, order);
    else
        hipLaunchKernelGGL(unregularize_kernel<128>, grid, dim3(128), 0, stream, in, rows, cols,
                           in_layout, su, sv, out, order);
    return hipGetLastError();
}

hipError_t launch_regularize(const void *w, int w_dtype, int rows, int cols, int had_block,
                             const float *su, const float *sv, float *out, int layout,
                             float *tile_sumsq, int *nonfinite, const uint8_t *order,
                             hipStream_t stream) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    if (had_block == 64)
        return w_dtype == 1 ? launch_reg_t<64, uint16_t>(w, rows, cols, su, sv, out, layout,
                                                         tile_sumsq, nonfinite, order, stream)
                            : launch_reg_t<64, float>(w, rows, cols, su, sv, out, layout,
                                                      tile_sumsq, nonfinite, order, stream);
    if (had_block == 128)
        return w_dtype == 1 ? launch_reg_t<128, uint16_t>(w, rows, cols, su, sv, out, layout,
                                                          tile_sumsq, nonfinite, order, stream)
                            : launch_reg_t<128, float>(w, rows, cols, su, sv, out, layout,
                                                       tile_sumsq, nonfinite, order, stream);
    return hipErrorInvalidValue;
}

}  // namespace exl3
