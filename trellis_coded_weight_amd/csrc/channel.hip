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
// The binary64 square of a binary32 value is exact, so only the additions
// round, in column order.
//
// Both kernels below use one workgroup of 256 lanes per band of 16 rows, in
// which one lane per row adds its row's squares in column order: the chain of
// `cols` dependent binary64 additions per row (all rows in parallel) is the
// kernel's latency.  A second sweep writes the scaled rows.
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
channel_normalize_any_kernel(const Tin *__restrict__ w, int rows, int cols,
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


// The fast form for rows of whole 16-byte groups (cols * sizeof(Tin) and the
// output row a multiple of 16 bytes, both arrays 16-byte aligned).  Workgroup
// of 320 lanes per band of 16 rows.  Wave 0's lanes 0..15 own the band's rows
// and run the sequential binary64 sums; waves 1..4 load the band in chunks of
// kFastCols columns, each lane keeping kFifo chunks of loads in flight in
// registers, and store chunk k into a two-slot LDS ring as binary64 squares
// (the square of a binary32 value is exact in binary64) just before the
// barrier after which wave 0 adds them, one dependent v_add_f64 per element in
// column order.  Then all lanes read the band again with 16-byte loads and
// write the scaled rows with 16-byte stores.  The time is that of the longest
// dependent chain: `cols` additions, each group of 16 waiting for its LDS
// reads, and one barrier per chunk (4096 columns: ~0.07 ms, against 0.013 ms
// for the 100 MB of traffic at the HBM peak).
constexpr int kFastCols = 128;                 // columns per chunk
constexpr int kFifo = 8;                       // chunks of loads in flight per loader lane
constexpr int kLoaders = 256;                  // loader lanes (waves 1..4)
constexpr int kRingStride = kFastCols + 2;     // binary64 words per ring row

template <typename Tin>
__global__ void __launch_bounds__(64 + kLoaders)
channel_normalize_kernel(const Tin *__restrict__ w, int rows, int cols,
                         const float *__restrict__ su, double floor_value,
                         float *__restrict__ w_norm, float *__restrict__ su_folded,
                         double *__restrict__ row_rms) {
    constexpr int EPL = 16 / sizeof(Tin);                  // elements per 16-byte load
    constexpr int LPR = kFastCols / EPL;                   // loads per chunk row
    constexpr int NLD = kBandRows * LPR / kLoaders;        // loads per loader lane per chunk
    static_assert(NLD * kLoaders == kBandRows * LPR, "loads divide over the loader lanes");
    __shared__ double ring[2][kBandRows][kRingStride];
    __shared__ float factor[kBandRows];
    const int t = threadIdx.x;
    const bool loader = t >= 64;
    const int lt = t - 64;
    const int row0 = blockIdx.x * kBandRows;
    const int nr = min(kBandRows, rows - row0);
    const int nchunk = (cols + kFastCols - 1) / kFastCols;

    uint4 fifo[kFifo][NLD];
    auto issue = [&](int k, uint4 (&dst)[NLD]) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int q = lt + kLoaders * i, r = q / LPR, cb = (q % LPR) * EPL;
            if (k < nchunk && r < nr && k * kFastCols + cb < cols)
                dst[i] = *reinterpret_cast<const uint4 *>(w + (size_t)(row0 + r) * cols +
                                                          k * kFastCols + cb);
        }
    };
    auto store = [&](int k, const uint4 (&src)[NLD]) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int q = lt + kLoaders * i, r = q / LPR, cb = (q % LPR) * EPL;
            if (r >= nr || k * kFastCols + cb >= cols) continue;
            const uint32_t wd[4] = {src[i].x, src[i].y, src[i].z, src[i].w};
            double v[EPL];
            if constexpr (EPL == 8) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = (double)__uint_as_float(wd[e] << 16);     // bf16 -> fp32 exact
                    v[2 * e + 1] = (double)__uint_as_float(wd[e] & 0xFFFF0000u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (double)__uint_as_float(wd[e]);
            }
            double *dst = &ring[k & 1][r][cb];
            // the squares (exact in binary64): the row sums only add
#pragma unroll
            for (int e = 0; e < EPL; e += 2)
                *reinterpret_cast<double2 *>(dst + e) =
                    make_double2(v[e] * v[e], v[e + 1] * v[e + 1]);
        }
    };

    if (loader) {
#pragma unroll
        for (int j = 0; j < kFifo; ++j) issue(j, fifo[j]);
    }
    double acc = 0.0;
    for (int k0 = 0; k0 < nchunk; k0 += kFifo) {
#pragma unroll
        for (int j = 0; j < kFifo; ++j) {
            const int k = k0 + j;
            if (loader && k < nchunk) {
                store(k, fifo[j]);
                issue(k + kFifo, fifo[j]);
            }
            __syncthreads();                           // chunk k is in ring slot k & 1
            if (t < nr && k < nchunk) {
                const double *src = ring[k & 1][t];
                const int nc = min(kFastCols, cols - k * kFastCols);
#pragma unroll 16
                for (int c = 0; c < nc; ++c) acc = acc + src[c];
            }
        }
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

    // scaled rows: 16-byte loads (kBatch in flight per lane), 16-byte stores
    constexpr int kBatch = 8;
    constexpr int kLanes = 64 + kLoaders;
    const int gpr = cols / EPL;                        // load groups per row
    const int ng = nr * gpr;
    for (int q0 = t; q0 < ng; q0 += kBatch * kLanes) {
        uint4 ub[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int q = q0 + b * kLanes;
            if (q < ng)
                ub[b] = *reinterpret_cast<const uint4 *>(
                    w + (size_t)(row0 + q / gpr) * cols + (q % gpr) * EPL);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
        const int q = q0 + b * kLanes;
        if (q >= ng) break;
        const int r = q / gpr, cb = (q % gpr) * EPL;
        const size_t base = (size_t)(row0 + r) * cols + cb;
        const uint4 u = ub[b];
        const float f = factor[r];
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
        if constexpr (EPL == 8) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = __uint_as_float(wd[e] << 16) * f;
                v[2 * e + 1] = __uint_as_float(wd[e] & 0xFFFF0000u) * f;
            }
            *reinterpret_cast<float4 *>(w_norm + base) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4 *>(w_norm + base + 4) = make_float4(v[4], v[5], v[6], v[7]);
        } else {
            *reinterpret_cast<float4 *>(w_norm + base) =
                make_float4(__uint_as_float(wd[0]) * f, __uint_as_float(wd[1]) * f,
                            __uint_as_float(wd[2]) * f, __uint_as_float(wd[3]) * f);
        }
        }
    }
}

}  // namespace

hipError_t launch_channel_normalize(const void *w, int w_dtype, int rows, int cols,
                                    const float *su, double floor_value, float *w_norm,
                                    float *su_folded, double *row_rms, hipStream_t stream) {
    if (rows <= 0 || cols <= 0) return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)((rows + kBandRows - 1) / kBandRows);
    const size_t in_bytes = w_dtype == EXL3_BF16 ? 2 : 4;
    const bool fast = reinterpret_cast<uintptr_t>(w) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(w_norm) % 16 == 0 &&
                      ((size_t)cols * in_bytes) % 16 == 0 && ((size_t)cols * 4) % 16 == 0;
    if (w_dtype == EXL3_BF16) {
        const uint16_t *wb = static_cast<const uint16_t *>(w);
        if (fast)
            hipLaunchKernelGGL(channel_normalize_kernel<uint16_t>, dim3(blocks), dim3(64 + kLoaders), 0,
                               stream, wb, rows, cols, su, floor_value, w_norm, su_folded,
                               row_rms);
        else
            hipLaunchKernelGGL(channel_normalize_any_kernel<uint16_t>, dim3(blocks),
                               dim3(kChunkCols), 0, stream, wb, rows, cols, su, floor_value,
                               w_norm, su_folded, row_rms);
    } else {
        const float *wf = static_cast<const float *>(w);
        if (fast)
            hipLaunchKernelGGL(channel_normalize_kernel<float>, dim3(blocks), dim3(64 + kLoaders), 0,
                               stream, wf, rows, cols, su, floor_value, w_norm, su_folded,
                               row_rms);
        else
            hipLaunchKernelGGL(channel_normalize_any_kernel<float>, dim3(blocks),
                               dim3(kChunkCols), 0, stream, wf, rows, cols, su, floor_value,
                               w_norm, su_folded, row_rms);
    }
    return hipGetLastError();
}

}  // namespace exl3
