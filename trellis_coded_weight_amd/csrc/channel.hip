// Out-channel RMS normalization on gfx950.
//
// Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture
// item 8 (out-channel RMS normalization, sign + scale folding, the zero-channel
// floor and the zero-sign rule for all-zero channels).
//
// The output channels are the rows of W.  Per row i:
//   r_i  = sqrt(sum_j (double)w_ij^2 / cols), j ascending, binary64
//   f_i  = (float)(1.0 / (r_i == 0 ? floor : r_i))
//   w'_ij = rn32(w_ij * f_i),   su'_i = r_i == 0 ? 0 : su_i * (float)r_i
// The binary64 square of a binary32 value is exact, so whether the compiler
// fuses the multiply into the add does not change the sum.
//
// One workgroup of 256 lanes per band of 16 rows.  The band's rows are staged
// through LDS 256 columns at a time with coalesced loads; lane t < 16 then adds
// its row's squares in column order (the chain of dependent binary64 adds is
// the kernel's latency: `cols` adds per row, all rows in parallel).  A second
// sweep reads the band again, one row at a time across all lanes, and writes
// the scaled rows.
#include "exl3.h"
#include "exl3_internal.h"

#include <math.h>

namespace exl3 {
namespace {

constexpr int kBandRows = 16;
constexpr int kChunkCols = 256;

__device__ __forceinline__ float load_w(const float *w, size_t i) { return w[i]; }
__device__ __forceinline__ float load_w(const uint16_t *w, size_t i) {
    return __uint_as_float((uint32_t)w[i] << 16);   // bf16 -> fp32 is exact
}

template <typename Tin>
__global__ void __launch_bounds__(kChunkCols)
channel_normalize_kernel(const Tin *__restrict__ w, int rows, int cols,
                         const float *__restrict__ su, double floor_value,
                         float *__restrict__ w_norm, float *__restrict__ su_folded,
                         double *__restrict__ row_rms) {
    // +1 column of padding: lane t reads row t of the chunk, so the 16 lanes'
    // addresses fall in 16 different banks
    __shared__ float chunk[kBandRows][kChunkCols + 1];
    __shared__ float factor[kBandRows];
    const int t = threadIdx.x;
    const int row0 = blockIdx.x * kBandRows;
    const int nr = min(kBandRows, rows - row0);

    double acc = 0.0;
    for (int c0 = 0; c0 < cols; c0 += kChunkCols) {
        const int nc = min(kChunkCols, cols - c0);
        if (t < nc)
            for (int r = 0; r < nr; ++r)
                chunk[r][t] = load_w(w, (size_t)(row0 + r) * cols + c0 + t);
        __syncthreads();
        if (t < nr)
            for (int c = 0; c < nc; ++c) {
                const double v = (double)chunk[t][c];
                acc = acc + v * v;
            }
        __syncthreads();
    }
    if (t < nr) {
        const int i = row0 + t;
        const double r = sqrt(acc / (double)cols);
        const double r_eff = r == 0.0 ? floor_value : r;
        factor[t] = (float)(1.0 / r_eff);
        su_folded[i] = r == 0.0 ? 0.0f : su[i] * (float)r;
        if (row_rms) row_rms[i] = r;
    }
    __syncthreads();
    for (int r = 0; r < nr; ++r) {
        const float f = factor[r];
        const size_t base = (size_t)(row0 + r) * cols;
        for (int c = t; c < cols; c += kChunkCols) w_norm[base + c] = load_w(w, base + c) * f;
    }
}

}  // namespace

hipError_t launch_channel_normalize(const void *w, int w_dtype, int rows, int cols,
                                    const float *su, double floor_value, float *w_norm,
                                    float *su_folded, double *row_rms, hipStream_t stream) {
    if (rows <= 0 || cols <= 0) return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)((rows + kBandRows - 1) / kBandRows);
    if (w_dtype == EXL3_BF16)
        hipLaunchKernelGGL(channel_normalize_kernel<uint16_t>, dim3(blocks), dim3(kChunkCols), 0,
                           stream, static_cast<const uint16_t *>(w), rows, cols, su, floor_value,
                           w_norm, su_folded, row_rms);
    else
        hipLaunchKernelGGL(channel_normalize_kernel<float>, dim3(blocks), dim3(kChunkCols), 0,
                           stream, static_cast<const float *>(w), rows, cols, su, floor_value,
                           w_norm, su_folded, row_rms);
    return hipGetLastError();
}

}  // namespace exl3
