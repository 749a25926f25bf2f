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
// One workgroup of B lanes per B x B block (the blocks are independent).  Lane
// j first holds column j of the block in registers for the left transform,
// the block is turned around in LDS, then lane j holds row j for the right
// transform.  The output is written tile-major (or row-major) and each of the
// block's (B/16)^2 tiles gets its sequential binary32 sum of squares.
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

template <int B, typename Tin>
__global__ void __launch_bounds__(B)
regularize_kernel(const Tin *__restrict__ w, int rows, int cols, const float *__restrict__ su,
                  const float *__restrict__ sv, float *__restrict__ out, int layout,
                  float *__restrict__ tile_sumsq, int *__restrict__ nonfinite,
                  const uint8_t *__restrict__ order) {
    __shared__ float blk[B][B + 1];
    const int j = threadIdx.x;
    const int br = blockIdx.y, bc = blockIdx.x;
    const int r0 = br * B, c0 = bc * B;
    const float c = norm_const<B>();

    float a[B];
    bool bad = false;
    const float svj = sv[c0 + j];
#pragma unroll
    for (int r = 0; r < B; ++r) {
        float val = load_w(w, (size_t)(r0 + r) * cols + c0 + j);
        bad |= !isfinite(val);
        a[r] = (val * su[r0 + r]) * svj;
    }
    if (bad && nonfinite) *nonfinite = 1;

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

    const int TC = cols / 16;
    constexpr int TB = B / 16;        // tiles per block side
    if (layout == 1) {
        for (int idx = j; idx < B * B; idx += B) {
            int lt = idx >> 8, t = idx & 255;
            int tr = lt / TB, tc = lt % TB;
            int el = order ? order[t] : t;
            int rr = tr * 16 + (el >> 4), cc = tc * 16 + (el & 15);
            size_t tau = (size_t)(r0 / 16 + tr) * TC + (c0 / 16 + tc);
            out[tau * 256 + t] = blk[rr][cc];
        }
    } else {
        for (int idx = j; idx < B * B; idx += B) {
            int rr = idx / B, cc = idx % B;
            out[(size_t)(r0 + rr) * cols + c0 + cc] = blk[rr][cc];
        }
    }
    if (tile_sumsq && j < TB * TB) {
        int tr = j / TB, tc = j % TB;
        float acc = 0.0f;
        for (int t = 0; t < 256; ++t) {
            const int el = order ? order[t] : t;
            float val = blk[tr * 16 + (el >> 4)][tc * 16 + (el & 15)];
            float sq = val * val;
            acc = acc + sq;
        }
        tile_sumsq[(size_t)(r0 / 16 + tr) * TC + (c0 / 16 + tc)] = acc;
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
    hipLaunchKernelGGL((regularize_kernel<B, Tin>), grid, dim3(B), 0, stream,
                       reinterpret_cast<const Tin *>(w), rows, cols, su, sv, out, layout,
                       tile_sumsq, nonfinite, order);
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
