// Traceback, packing and dequantisation of the EXL3 tile encoder on gfx950.
//
// Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture
// section 1 (device-resident circular traceback of the two-pass closure) and
// section 5 (container: the low K bits of each state, MSB-first, 16-bit words,
// then a swap of the two halves of every 32-bit pair; decode by reading the
// 16-bit window that ends at each state's last bit).
//
// Traceback is a chain of dependent reads, one per step, so one lane walks one
// tile; many tiles in flight hide the latency.  The walk uses the predecessor
// rule S_{t-1} = (bp[t-1][S_t >> K] << Kr) | (S_t >> K).
#include "exl3_internal.h"

namespace exl3 {
namespace {

constexpr int kTbThreads = 64;   // tiles per traceback workgroup (one wave)
constexpr int64_t kWaveTbMaxTiles = 1024;   // up to this many tiles: one wave per tile

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// The binary32 and binary16 forward kernels lay their backpointer words out
// differently (same word type and size); H selects the binary16 layout.
template <int K, bool H>
__device__ __forceinline__ uint32_t bp_read(const typename Geo<K>::bp_t *__restrict__ bp_tile,
                                            int slot, uint32_t e) {
    uint32_t lane;
    if (H) {
        // same bytes per step as the binary32 layout; the binary16 kernel
        // writes one 32-bit word per lane (512 lanes at K = 4)
        uint32_t bit[K];
        bp_locate_h<K>(e, lane, bit);
        const uint32_t *bp32 = reinterpret_cast<const uint32_t *>(bp_tile);
        const uint32_t w = bp32[(size_t)slot * GeoH<K>::LANES + lane];
        uint32_t k = 0;
#pragma unroll
        for (int r = 0; r < K; ++r) k |= ((w >> bit[r]) & 1u) << r;
        return k;
    }
    uint32_t bit;
    bp_locate<K>(e, lane, bit);
    const uint32_t w = bp_tile[(size_t)slot * kLanes + lane];
    return (w >> bit) & ((1u << K) - 1u);
}

// Pass 1: from the best final state of the rotated pass back to rotated step
// 127 (original position 255); that state is X.
template <int K, bool H>
__global__ void __launch_bounds__(kTbThreads)
traceback1_kernel(const typename Geo<K>::bp_t *__restrict__ bp, int64_t n,
                  const uint16_t *__restrict__ end_state, uint16_t *__restrict__ X_out) {
    using G = Geo<K>;
    const int64_t b = (int64_t)blockIdx.x * kTbThreads + threadIdx.x;
    if (b >= n) return;
    const typename G::bp_t *bp_tile = bp + (size_t)b * kSlots * kLanes;
    uint32_t s = end_state[b];
    for (int j = kSteps - 1; j >= kSteps / 2; --j) {
        uint32_t e = s >> K;
        uint32_t k = bp_read<K, H>(bp_tile, (j - 1) - 127, e);
        s = (k << G::Kr) | e;
    }
    X_out[b] = (uint16_t)s;
}

// Pass 2: from X at step 255 back to step 0, then pack, and (binary32 mode,
// x given) dequantise and sum the squared error of the tile in step order.
template <int K, bool H>
__global__ void __launch_bounds__(kTbThreads)
traceback2_kernel(const typename Geo<K>::bp_t *__restrict__ bp, int64_t n,
                  const uint16_t *__restrict__ X_in, const float *__restrict__ x,
                  const int32_t *__restrict__ tile_idx, int64_t tile0,
                  const uint16_t *__restrict__ levels, float scale, uint16_t *__restrict__ packed,
                  uint16_t *__restrict__ states_out, float *__restrict__ sse_out,
                  float *__restrict__ w_hat) {
    using G = Geo<K>;
    __shared__ uint16_t S[kTbThreads][kSteps];
    const int lt = threadIdx.x;
    const int64_t b = (int64_t)blockIdx.x * kTbThreads + lt;
    if (b >= n) return;
    const int64_t tile = tile_idx ? (int64_t)tile_idx[b] : tile0 + b;
    const typename G::bp_t *bp_tile = bp + (size_t)b * kSlots * kLanes;

    uint32_t s = X_in[b];
    S[lt][kSteps - 1] = (uint16_t)s;
    for (int t = kSteps - 1; t >= 1; --t) {
        uint32_t e = s >> K;
        uint32_t k = bp_read<K, H>(bp_tile, t - 1, e);
        s = (k << G::Kr) | e;
        S[lt][t - 1] = (uint16_t)s;
    }

    // container: MSB-first stream of the low K bits, 16-bit words, pair swap
    uint16_t *pk = packed + (size_t)tile * (16 * K);
    uint32_t acc = 0;
    int nbits = 0, word = 0;
    for (int t = 0; t < kSteps; ++t) {
        acc = (acc << K) | ((uint32_t)S[lt][t] & ((1u << K) - 1u));
        nbits += K;
        if (nbits >= 16) {
            nbits -= 16;
            pk[word ^ 1] = (uint16_t)(acc >> nbits);
            acc &= (1u << nbits) - 1u;
            ++word;
        }
    }

    if (states_out)
        for (int t = 0; t < kSteps; ++t) states_out[(size_t)tile * kSteps + t] = S[lt][t];
    if (!x) return;

    // dequantise and sequential squared error (equals the search's path cost);
    // the loads of a chunk are issued together, then consumed in step order
    const float *xt = x + (size_t)tile * kSteps;
    float sse = 0.0f;
    constexpr int kChunk = 16;
    for (int t0 = 0; t0 < kSteps; t0 += kChunk) {
        uint16_t c[kChunk];
        float xv[kChunk];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            c[u] = levels[S[lt][t0 + u]];
            xv[u] = xt[t0 + u];
        }
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const float v = scale * half_bits_to_float(c[u]);
            const float d = xv[u] - v;
            const float q = d * d;
            sse = sse + q;
            if (w_hat) w_hat[(size_t)tile * kSteps + t0 + u] = v;
        }
    }
    if (sse_out) sse_out[tile] = sse;
}

// Small batches (a scale-search probe, an LDLQ span): one wave per tile, and
// the walk's chain of dependent reads is shortened by speculation.  Knowing
// S_t, the backpointer of step t-1 is one word; the one of step t-2 is one of
// 2^K words (one per value k1 of the first backpointer), the one of step t-3
// one of 2^2K, and so on.  Lane (d, h) reads the word of step t-1-d under
// hypothesis h = k1 + 2^K k2 + ... (the d backpointers before it), all in one
// round trip; then the wave resolves the D steps in order by reading the lane
// that holds the true hypothesis.  Under h the state at step t-d is
//     (h << (16 - K d)) | (S_t >> (K d)),
// since each step shifts K bits out at the bottom and the backpointer in at
// the top.  In the binary32 layout at K = 1 and 2 the top W bits of a state
// (W = 4 and 2: its butterfly's index among the lane's) only choose the field
// within the word, not the word, so hypotheses that differ only there share
// one load: depth d needs 2^max(0, K d - W) words, and the lanes load whole
// words, the resolution taking the field of the true state.  Look-ahead depth
// D: the largest whose words fit in 64 lanes (K = 1 / 2 / 3 / 4: 9 / 4 / 2 / 2
// in the binary32 layout, 6 / 3 / 2 / 2 in the binary16 one).
template <int K, bool H>
struct Look {
    static constexpr int W = H ? 0 : K == 1 ? 4 : K == 2 ? 2 : 0;
    static constexpr int bits(int d) { return K * d - W > 0 ? K * d - W : 0; }
    static constexpr int offset(int d) {   // first lane of depth d
        int off = 0;
        for (int i = 0; i < d; ++i) off += 1 << bits(i);
        return off;
    }
    static constexpr int depth() {
        int d = 0;
        while (offset(d + 1) <= 64) ++d;
        return d;
    }
    static constexpr int D = depth();
};

// Walk `count` transitions back from state s: the first reads slot `slot0`,
// the next slot0 - 1, ...  If S is given, S[pos0 - 1 - i] receives the state
// after transition i.  Returns the last state (uniform across the wave).
// Every read stays inside slots [slot0 - count + 1, slot0].
template <int K, bool H>
__device__ uint32_t walk_wave(const typename Geo<K>::bp_t *__restrict__ bp_tile, uint32_t s,
                              int slot0, int count, uint16_t *S, int pos0) {
    using G = Geo<K>;
    using L = Look<K, H>;
    constexpr int D = L::D;
    const int lane = threadIdx.x & 63;
    // this lane's depth and the hypothesis bits that choose its word (lanes
    // past the last depth stay idle)
    int d = -1;
    uint32_t hs = 0;
#pragma unroll
    for (int i = 0; i < D; ++i) {
        const int off = L::offset(i);
        if (lane >= off && lane < off + (1 << L::bits(i))) {
            d = i;
            hs = i == 0 ? 0u : (uint32_t)(lane - off) << (16 - K * i);
        }
    }
    const uint32_t shift = d > 0 ? (uint32_t)(K * d) : 0u;
    int done = 0;
    while (done < count) {
        const int r = (count - done) < D ? (count - done) : D;   // steps this round
        uint32_t val = 0;
        if (d >= 0 && d < r) {
            const uint32_t st = hs | (s >> shift);              // state at step t - d
            if constexpr (L::W > 0) {
                // the whole word (the binary32 layout)
                uint32_t wl, wb;
                bp_locate<K>(st >> K, wl, wb);
                val = bp_tile[(size_t)(slot0 - done - d) * kLanes + wl];
            } else {
                val = bp_read<K, H>(bp_tile, slot0 - done - d, st >> K);
            }
        }
        uint32_t hyp = 0;
#pragma unroll
        for (int i = 0; i < D; ++i) {
            if (i < r) {
                const int src = L::offset(i) + (int)(hyp & ((1u << L::bits(i)) - 1u));
                uint32_t k = (uint32_t)__builtin_amdgcn_readlane((int)val, src);
                if constexpr (L::W > 0) {
                    // the field of the true state at step t - i (s, by now)
                    uint32_t wl, wb;
                    bp_locate<K>(s >> K, wl, wb);
                    k = (k >> wb) & ((1u << K) - 1u);
                }
                s = (k << G::Kr) | (s >> K);
                if (S && lane == 0) S[pos0 - 1 - done - i] = (uint16_t)s;
                hyp |= k << (K * i);
            }
        }
        done += r;
    }
    return s;
}

template <int K, bool H>
__global__ void __launch_bounds__(64)
traceback1_wave_kernel(const typename Geo<K>::bp_t *__restrict__ bp, int64_t n,
                       const uint16_t *__restrict__ end_state, uint16_t *__restrict__ X_out) {
    const int64_t b = blockIdx.x;
    const typename Geo<K>::bp_t *bp_tile = bp + (size_t)b * kSlots * kLanes;
    // rotated steps 255 -> 127: 128 transitions, slots 127 .. 0
    const uint32_t X = walk_wave<K, H>(bp_tile, end_state[b], kSteps / 2 - 1, kSteps / 2,
                                       nullptr, 0);
    if (threadIdx.x == 0) X_out[b] = (uint16_t)X;
}

template <int K, bool H>
__global__ void __launch_bounds__(64)
traceback2_wave_kernel(const typename Geo<K>::bp_t *__restrict__ bp, int64_t n,
                       const uint16_t *__restrict__ X_in, const float *__restrict__ x,
                       const int32_t *__restrict__ tile_idx, int64_t tile0,
                       const uint16_t *__restrict__ levels, float scale,
                       uint16_t *__restrict__ packed, uint16_t *__restrict__ states_out,
                       float *__restrict__ sse_out, float *__restrict__ w_hat) {
    __shared__ uint16_t S[kSteps];
    __shared__ float Q[kSteps];
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t tile = tile_idx ? (int64_t)tile_idx[b] : tile0 + b;
    const typename Geo<K>::bp_t *bp_tile = bp + (size_t)b * kSlots * kLanes;

    const uint32_t X = X_in[b];
    if (lane == 0) S[kSteps - 1] = (uint16_t)X;
    walk_wave<K, H>(bp_tile, X, kSlots - 1, kSlots, S, kSteps - 1);
    __syncthreads();

    // container word w: stream bits 16w .. 16w+15, MSB first, pair swap
    if (lane < 16 * K) {
        uint32_t word = 0;
        for (int j = 16 * lane; j < 16 * lane + 16; ++j) {
            const int t = j / K;
            word = (word << 1) | (((uint32_t)S[t] >> (K - 1 - (j - t * K))) & 1u);
        }
        packed[(size_t)tile * (16 * K) + (lane ^ 1)] = (uint16_t)word;
    }
    if (states_out)
        for (int t = lane; t < kSteps; t += 64) states_out[(size_t)tile * kSteps + t] = S[t];
    if (!x) return;

    // dequantise; squared errors summed in step order by one lane
    const float *xt = x + (size_t)tile * kSteps;
    for (int t = lane; t < kSteps; t += 64) {
        const float v = scale * half_bits_to_float(levels[S[t]]);
        const float dd = xt[t] - v;
        Q[t] = dd * dd;
        if (w_hat) w_hat[(size_t)tile * kSteps + t] = v;
    }
    __syncthreads();
    if (lane == 0 && sse_out) {
        float sse = 0.0f;
        for (int t = 0; t < kSteps; ++t) sse = sse + Q[t];
        sse_out[tile] = sse;
    }
}

// Decode: one workgroup of 16 waves per compute unit (as many as the grid
// holds), which copies the level table (65,536 binary16 values, 128 KiB) into
// LDS once and then decodes tiles in turn, one wave per tile and four
// consecutive states per lane; the level lookups, random over the table, are
// LDS reads.  The container stores each pair of 16-bit words swapped, so words
// 2i + 1 and 2i read as one little-endian 32-bit value are stream bits 32i ..
// 32i + 31 with bit 32i as its most significant bit (chunk i).  S_t, the 16
// stream bits ending at bit (t + 1)K - 1 (circularly), is then the top half of
// a funnel shift of two consecutive chunks.  The chunks are assembled from
// 16-bit loads (no alignment needed); the output is one float4 per lane, a
// wave's 1 KiB tile in one store, where it is 16-byte aligned.
constexpr int kDecodeWaves = 16;

__global__ void __launch_bounds__(64 * kDecodeWaves)
decode_kernel(const uint16_t *__restrict__ packed, int64_t n, int K, float scale,
              const uint16_t *__restrict__ levels, float *__restrict__ out, bool out_vec) {
    __shared__ uint4 lut[8192];                        // the level table
    __shared__ uint32_t chunk[kDecodeWaves][64];       // one tile's stream per wave
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint4 *src = reinterpret_cast<const uint4 *>(levels);
    for (int i = threadIdx.x; i < 8192; i += 64 * kDecodeWaves) lut[i] = src[i];
    __syncthreads();
    const uint16_t *lv = reinterpret_cast<const uint16_t *>(lut);
    const int nc = 8 * K;                              // 32-bit chunks per tile (K <= 8)
    const int nbits = 256 * K;
    const int64_t stride = (int64_t)gridDim.x * kDecodeWaves;
    for (int64_t tile = (int64_t)blockIdx.x * kDecodeWaves + wv; tile < n; tile += stride) {
        if (lane < nc) {
            const uint16_t *pw = packed + (size_t)tile * (16 * K) + 2 * lane;
            chunk[wv][lane] = ((uint32_t)pw[1] << 16) | pw[0];
        }
        // the wave's own stores, read back by other lanes of the same wave
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            int p = (4 * lane + k + 1) * K - 16;       // first bit of S_t's window
            if (p < 0) p += nbits;
            const int c = p >> 5;
            const uint32_t hi = chunk[wv][c], lo = chunk[wv][c + 1 == nc ? 0 : c + 1];
            const uint32_t st = __funnelshift_l(lo, hi, (unsigned)(p & 31)) >> 16;
            v[k] = scale * half_bits_to_float(lv[st]);
        }
        float *o = out + (size_t)tile * kSteps + 4 * lane;
        if (out_vec) {
            store_stream(o, v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = v[k];
        }
        // the chunk reads of this tile are done before the next tile's stores
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}

__global__ void __launch_bounds__(256)
gather_tiles_kernel(const float *__restrict__ src, const int32_t *__restrict__ idx,
                    float *__restrict__ dst) {
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    dst[(size_t)b * kSteps + t] = src[(size_t)idx[b] * kSteps + t];
}

// Binary16 encoder inputs: fp16(rn32(w / scale)), all zero at scale 0; tile b
// of the output is tile idx[b] (or b) of the input.
__global__ void __launch_bounds__(256)
to_f16_kernel(const float *__restrict__ src, const int32_t *__restrict__ idx, float scale,
              uint16_t *__restrict__ dst) {
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t tile = idx ? (int64_t)idx[b] : b;
    const float q = scale == 0.0f ? 0.0f : src[(size_t)tile * kSteps + t] / scale;
    dst[(size_t)b * kSteps + t] = __builtin_bit_cast(uint16_t, (_Float16)q);
}

template <int K, bool H>
hipError_t launch_tb_t(int pass, const void *bp, int64_t n, const uint16_t *start_state,
                       uint16_t *X_out, const float *x, const int32_t *tile_idx, int64_t tile0,
                       const uint16_t *levels, float scale, uint16_t *packed, uint16_t *states,
                       float *sse, float *w_hat, hipStream_t stream) {
    using bp_t = typename Geo<K>::bp_t;
    if (n <= kWaveTbMaxTiles) {
        // small batch: one wave per tile with a speculative walk
        if (pass == 1)
            hipLaunchKernelGGL((traceback1_wave_kernel<K, H>), dim3((unsigned)n), dim3(64), 0,
                               stream, reinterpret_cast<const bp_t *>(bp), n, start_state, X_out);
        else
            hipLaunchKernelGGL((traceback2_wave_kernel<K, H>), dim3((unsigned)n), dim3(64), 0,
                               stream, reinterpret_cast<const bp_t *>(bp), n, start_state, x,
                               tile_idx, tile0, levels, scale, packed, states, sse, w_hat);
        return hipGetLastError();
    }
    const unsigned blocks = (unsigned)((n + kTbThreads - 1) / kTbThreads);
    if (pass == 1)
        hipLaunchKernelGGL((traceback1_kernel<K, H>), dim3(blocks), dim3(kTbThreads), 0, stream,
                           reinterpret_cast<const bp_t *>(bp), n, start_state, X_out);
    else
        hipLaunchKernelGGL((traceback2_kernel<K, H>), dim3(blocks), dim3(kTbThreads), 0, stream,
                           reinterpret_cast<const bp_t *>(bp), n, start_state, x, tile_idx,
                           tile0, levels, scale, packed, states, sse, w_hat);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_traceback(int K, int pass, bool f16, const void *bp, int64_t n,
                            const uint16_t *start_state, uint16_t *X_out, const float *x,
                            const int32_t *tile_idx, int64_t tile0, const uint16_t *levels,
                            float scale, uint16_t *packed, uint16_t *states, float *sse,
                            float *w_hat, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
#define EXL3_TB_CASE(KK)                                                                     \
    case KK:                                                                                 \
        return f16 ? launch_tb_t<KK, true>(pass, bp, n, start_state, X_out, x, tile_idx,     \
                                           tile0, levels, scale, packed, states, sse, w_hat, \
                                           stream)                                           \
                   : launch_tb_t<KK, false>(pass, bp, n, start_state, X_out, x, tile_idx,    \
                                            tile0, levels, scale, packed, states, sse,       \
                                            w_hat, stream);
    switch (K) {
        EXL3_TB_CASE(1)
        EXL3_TB_CASE(2)
        EXL3_TB_CASE(3)
        EXL3_TB_CASE(4)
        default:
            return hipErrorInvalidValue;
    }
#undef EXL3_TB_CASE
}

hipError_t launch_decode(const uint16_t *packed, int64_t n, int K, float scale,
                         const uint16_t *levels, float *out, int n_cu, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    if (K < 1 || K > 8) return hipErrorInvalidValue;
    // the level table is read as 16-byte words
    if (reinterpret_cast<uintptr_t>(levels) % 16 != 0) return hipErrorInvalidValue;
    const int64_t need = (n + kDecodeWaves - 1) / kDecodeWaves;
    const int64_t groups = need < n_cu ? need : (n_cu > 0 ? n_cu : 1);
    const bool out_vec = reinterpret_cast<uintptr_t>(out) % 16 == 0;
    hipLaunchKernelGGL(decode_kernel, dim3((unsigned)groups), dim3(64 * kDecodeWaves), 0, stream,
                       packed, n, K, scale, levels, out, out_vec);
    return hipGetLastError();
}

hipError_t launch_to_f16(const float *src, const int32_t *idx, int64_t n, float scale,
                         uint16_t *dst, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(to_f16_kernel, dim3((unsigned)n), dim3(kSteps), 0, stream, src, idx, scale,
                       dst);
    return hipGetLastError();
}

hipError_t launch_gather_tiles(const float *src, const int32_t *idx, int64_t n, float *dst,
                               hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(gather_tiles_kernel, dim3((unsigned)n), dim3(kSteps), 0, stream, src, idx,
                       dst);
    return hipGetLastError();
}

}  // namespace exl3
