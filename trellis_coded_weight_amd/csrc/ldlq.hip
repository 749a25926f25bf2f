// LDLQ error feedback around the tile encoder on gfx950.
//
// Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture
// item 3 (one-sided block LDLQ: spans traversed bottom-up, each span's target
// corrected additively from the strictly lower blocks of L, the residual of
// the spans already quantized fed back).
//
// The matrix lives tile-major ([TR*TC][256], tile tr*TC + tc) in the
// context's within-tile order: element 16r + c of a tile sits at position
// inv[16r + c], inv being the inverse of the order (at 16r + c without one).
// The target kernel works in element coordinates and reads and writes tiles
// through inv; the commit kernel is position-wise and needs no table.
// Span j is tile column j: the TR tiles (tr, j).  Its target is
//     T_j = W_j + sum_{i > j} E_i L_ij,      E_i = W_i - What_i,
// accumulated per element in the order i ascending, then t (row of the 16x16
// block L_ij) ascending, each product and each sum a separately rounded
// binary32 operation (this file is built with -ffp-contract=off).  One
// workgroup of 256 lanes per tile row: lane (r, c) owns one element; the
// tile's error blocks E(tr, i) and the factor blocks L_ij of 16 later spans at
// a time are staged in LDS, the next 16 loading while the current ones are
// summed.
#include "exl3_internal.h"

namespace exl3 {
namespace {

constexpr int kBlocksPerChunk = 16;   // later spans staged in LDS per round trip
constexpr int kLtPad = 20;            // row pitch of the transposed factor blocks (16-byte aligned)

// Target of span j for tile row tr = blockIdx.x, lane (r, c) = element 16r + c.
// Chunks of 16 later spans are double-buffered: the global loads of chunk n+1
// are in flight while chunk n is summed from LDS.  The factor blocks are
// stored transposed so that both operands of a lane's 16-term sum are read 4
// at a time (ds_read_b128): the error row E(tr, i)[r][0..15] and the factor
// column L_ij[0..15][c].
__global__ void __launch_bounds__(256)
ldlq_target_kernel(const float *__restrict__ w_tiles, const float *__restrict__ e_tiles,
                   const float *__restrict__ L, int TC, int j, const uint8_t *__restrict__ inv,
                   float *__restrict__ target) {
    __shared__ __attribute__((aligned(16))) float Es[2][kBlocksPerChunk][16][16];
    __shared__ __attribute__((aligned(16))) float Lt[2][kBlocksPerChunk][16][kLtPad];
    const int tr = blockIdx.x;
    const int e = threadIdx.x, r = e >> 4, c = e & 15;
    const int pos = inv ? inv[e] : e;      // position of element (r, c) in a tile
    const size_t C = (size_t)TC * 16;
    float acc = w_tiles[((size_t)tr * TC + j) * 256 + pos];
    // take the load's wait here, once, not at acc's first use inside the loop
    // (where it would also wait for the next chunk's loads)
    asm volatile("" : "+v"(acc));
    const int n_later = TC - 1 - j;
    const int n_chunks = (n_later + kBlocksPerChunk - 1) / kBlocksPerChunk;
    float pe[kBlocksPerChunk], pl[kBlocksPerChunk];
    // loads of chunk n into registers (spans i = j + 1 + 16n + q)
    auto fetch = [&](int n) {
        const int i0 = j + 1 + n * kBlocksPerChunk;
#pragma unroll
        for (int q = 0; q < kBlocksPerChunk; ++q) {
            // past the last span: a valid address whose value is never summed
            const int i = (i0 + q) < TC ? (i0 + q) : (TC - 1);
            pe[q] = e_tiles[((size_t)tr * TC + i) * 256 + pos];        // E[16tr + r][16i + c]
            pl[q] = L[(size_t)(16 * i + r) * C + 16 * (size_t)j + c];  // L_ij[r][c]
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int q = 0; q < kBlocksPerChunk; ++q) {
            Es[buf][q][r][c] = pe[q];
            Lt[buf][q][c][r] = pl[q];
        }
    };
    if (n_chunks > 0) {
        fetch(0);
        stage(0);
        __syncthreads();
    }
    for (int n = 0; n < n_chunks; ++n) {
        const int buf = n & 1;
        if (n + 1 < n_chunks) fetch(n + 1);
        const int nq = (n_later - n * kBlocksPerChunk) < kBlocksPerChunk
                           ? (n_later - n * kBlocksPerChunk) : kBlocksPerChunk;
        for (int q = 0; q < nq; ++q) {
#pragma unroll
            for (int t4 = 0; t4 < 16; t4 += 4) {
                const float4 ev = *reinterpret_cast<const float4 *>(&Es[buf][q][r][t4]);
                const float4 lv = *reinterpret_cast<const float4 *>(&Lt[buf][q][c][t4]);
                acc = acc + ev.x * lv.x;
                acc = acc + ev.y * lv.y;
                acc = acc + ev.z * lv.z;
                acc = acc + ev.w * lv.w;
            }
        }
        if (n + 1 < n_chunks) stage(buf ^ 1);
        __syncthreads();
    }
    target[(size_t)tr * 256 + pos] = acc;
}

// Commit span j: scatter the span's container words, keep its error for the
// spans below, optionally write the dequantized tiles, and the per-tile
// sequential binary32 sum of (W - What)^2.
__global__ void __launch_bounds__(256)
ldlq_commit_kernel(const float *__restrict__ w_tiles, const float *__restrict__ what_span,
                   const uint16_t *__restrict__ packed_span, int TC, int j, int K,
                   uint16_t *__restrict__ packed, float *__restrict__ e_tiles,
                   float *__restrict__ w_hat, float *__restrict__ tile_err) {
    __shared__ float sq[256];
    const int tr = blockIdx.x;
    const int e = threadIdx.x;
    const size_t tile = (size_t)tr * TC + j;
    const float w = w_tiles[tile * 256 + e];
    const float wh = what_span[(size_t)tr * 256 + e];
    const float d = w - wh;
    e_tiles[tile * 256 + e] = d;
    if (w_hat) w_hat[tile * 256 + e] = wh;
    if (e < 16 * K) packed[tile * 16 * K + e] = packed_span[(size_t)tr * 16 * K + e];
    sq[e] = d * d;
    __syncthreads();
    if (e == 0) {
        float acc = 0.0f;
        for (int t = 0; t < 256; ++t) acc = acc + sq[t];
        tile_err[tile] = acc;
    }
}

}  // namespace

hipError_t launch_ldlq_target(const float *w_tiles, const float *e_tiles, const float *L, int TR,
                              int TC, int j, const uint8_t *inv, float *target,
                              hipStream_t stream) {
    if (TR <= 0) return hipSuccess;
    if (j < 0 || j >= TC) return hipErrorInvalidValue;
    hipLaunchKernelGGL(ldlq_target_kernel, dim3((unsigned)TR), dim3(256), 0, stream, w_tiles,
                       e_tiles, L, TC, j, inv, target);
    return hipGetLastError();
}

hipError_t launch_ldlq_commit(const float *w_tiles, const float *what_span,
                              const uint16_t *packed_span, int TR, int TC, int j, int K,
                              uint16_t *packed, float *e_tiles, float *w_hat, float *tile_err,
                              hipStream_t stream) {
    if (TR <= 0) return hipSuccess;
    if (j < 0 || j >= TC || K < 1 || K > 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL(ldlq_commit_kernel, dim3((unsigned)TR), dim3(256), 0, stream, w_tiles,
                       what_span, packed_span, TC, j, K, packed, e_tiles, w_hat, tile_err);
    return hipGetLastError();
}

}  // namespace exl3
