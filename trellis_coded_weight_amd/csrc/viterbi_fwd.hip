// Forward add-compare-select pass of the EXL3 tile encoder on gfx950.
//
// Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture
// section 1 (forward dynamic program over the 16-bit bitshift trellis,
// two-pass tail-biting closure) and section 4 (state algebra, lowest-branch
// tie rule).  Arithmetic per state and step, each operation rounded on its own
// (this file must be built with -ffp-contract=off):
//     d = x_t - v[s];  q = d * d;  C[s] = M[s >> K] + q
//     M'[e] = min_k C[(k << Kr) | e],  backpointer = lowest k reaching it.
//
// One workgroup (16 waves) per tile.  The 2^(16-K) tracked minima live in LDS,
// double-buffered (128 / 64 / 32 KiB at K = 2 / 3 / 4), so one barrier per step
// suffices.  Each lane owns 64 states for the whole pass and keeps their
// levels in registers; a step is: read the tracked minima of the lane's
// butterflies, branch metric + add for 64 states, minimum and lowest argmin
// per written tracked state, write the new minima, store one word of
// backpointer bits per lane (coalesced, 4 KiB per step and tile at K = 2).
//
//   pass 1: input rotated by 128, all starting costs 0; backpointers kept for
//           steps 127..254; result: the lowest-cost final state (lowest index
//           on equal costs) -> end_state.
//   pass 2: input in order, only tracked index X & (2^Kr - 1) admitted at the
//           start (cost 0, others +inf); backpointers for steps 0..254;
//           result: C_255[X] -> cost_out (the path's squared error).
#include "exl3_internal.h"

#include <math.h>

namespace exl3 {
namespace {

template <int N>
struct Log2 {
    static constexpr int v = 1 + Log2<N / 2>::v;
};
template <>
struct Log2<1> {
    static constexpr int v = 0;
};

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

template <int K>
__device__ __forceinline__ void lane_butterflies(int g, int (&m)[Geo<K>::GPL], int &b0) {
    using G = Geo<K>;
    if (K == 2) {
#pragma unroll
        for (int i = 0; i < G::GPL; ++i) m[i] = g + kLanes * i;
        b0 = 0;
    } else if (K == 3) {
        m[0] = g;
        b0 = 0;
    } else {
        m[0] = g >> 2;
        b0 = 4 * (g & 3);
    }
}

// Append one bit per lane to acc: acc = 2 * acc + mask[lane] in one VALU op
// (add with carry-in taken from the 64-bit lane mask).
__device__ __forceinline__ uint32_t push_bit(uint32_t acc, uint64_t mask) {
    uint32_t out;
    uint64_t carry_out;
    asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3"
        : "=v"(out), "=s"(carry_out)
        : "v"(acc), "s"(mask));
    return out;
}

// Bits of the lowest index whose match mask is set, most significant first,
// as lane masks.  c[j] = lanes where candidate j equals the minimum; the last
// candidate wins where no earlier one matches, so c[N-1] is never read.
template <int N>
struct FirstMatch {
    static __device__ __forceinline__ void bits(const uint64_t *c, uint64_t *out) {
        uint64_t any_lo = 0;
#pragma unroll
        for (int j = 0; j < N / 2; ++j) any_lo |= c[j];
        const uint64_t hi_half = ~any_lo;
        uint64_t lo_bits[32], hi_bits[32];
        FirstMatch<N / 2>::bits(c, lo_bits);
        FirstMatch<N / 2>::bits(c + N / 2, hi_bits);
        out[0] = hi_half;
#pragma unroll
        for (int j = 0; j + 1 < Log2<N>::v; ++j)
            out[j + 1] = (hi_half & hi_bits[j]) | (~hi_half & lo_bits[j]);
    }
};
template <>
struct FirstMatch<2> {
    static __device__ __forceinline__ void bits(const uint64_t *c, uint64_t *out) {
        out[0] = ~c[0];
    }
};

template <int NB>
__device__ __forceinline__ float tree_min(const float (&a)[NB]) {
    // pairwise then three-way minima (v_min3_f32); exact for non-NaN inputs
    float r[(NB + 2) / 3];
    int n = 0;
#pragma unroll
    for (int j = 0; j + 2 < NB; j += 3) r[n++] = __builtin_fminf(__builtin_fminf(a[j], a[j + 1]), a[j + 2]);
    if (NB % 3 == 2) r[n++] = __builtin_fminf(a[NB - 2], a[NB - 1]);
    if (NB % 3 == 1) r[n++] = a[NB - 1];
    float m = r[0];
#pragma unroll
    for (int j = 1; j < n; ++j) m = __builtin_fminf(m, r[j]);
    return m;
}

// One tracked-state update: minimum over the 2^K candidates and the lowest
// index reaching it; the K index bits are appended to acc, high bit first.
template <int K>
__device__ __forceinline__ float acs(const float (&a)[1 << K], uint32_t &acc) {
    constexpr int NB = 1 << K;
    const float mn = tree_min<NB>(a);
    uint64_t c[NB];
#pragma unroll
    for (int j = 0; j + 1 < NB; ++j) c[j] = __builtin_amdgcn_ballot_w64(a[j] == mn);
    c[NB - 1] = 0;
    uint64_t kb[K];
    FirstMatch<NB>::bits(c, kb);
#pragma unroll
    for (int j = 0; j < K; ++j) acc = push_bit(acc, kb[j]);
    return mn;
}

template <int K, int PASS>
__global__ void __launch_bounds__(kLanes, 1)
viterbi_fwd_kernel(const float *__restrict__ x, const int32_t *__restrict__ tile_idx,
                   int64_t tile0, const uint16_t *__restrict__ levels, float scale,
                   const uint16_t *__restrict__ X_in, typename Geo<K>::bp_t *__restrict__ bp,
                   uint16_t *__restrict__ end_state, float *__restrict__ cost_out) {
    using G = Geo<K>;
    using bp_t = typename G::bp_t;
    __shared__ float Mbuf[2][G::T];
    __shared__ float xs[kSteps];
    __shared__ float red_cost[kLanes / 64];
    __shared__ uint32_t red_state[kLanes / 64];

    const int g = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t tile = tile_idx ? (int64_t)tile_idx[b] : tile0 + b;

    if (g < kSteps) xs[g] = x[tile * kSteps + g];

    int m[G::GPL];
    int b0;
    lane_butterflies<K>(g, m, b0);

    // levels of the lane's 64 states, scaled once per pass
    float v[G::GPL][G::NB][G::BPL];
#pragma unroll
    for (int i = 0; i < G::GPL; ++i)
#pragma unroll
        for (int k = 0; k < G::NB; ++k)
#pragma unroll
            for (int bb = 0; bb < G::BPL; ++bb) {
                uint32_t s = ((uint32_t)k << G::Kr) | ((uint32_t)m[i] << K) | (uint32_t)(b0 + bb);
                v[i][k][bb] = scale * half_bits_to_float(levels[s]);
            }

    const uint32_t xm = (PASS == 1) ? 0u : ((uint32_t)X_in[b] & (uint32_t)(G::T - 1));
    for (int e = g; e < G::T; e += kLanes)
        Mbuf[0][e] = (PASS == 1 || (uint32_t)e == xm) ? 0.0f : INFINITY;
    __syncthreads();

    bp_t *bp_tile = bp + (size_t)b * kSlots * kLanes;

    for (int t = 0; t < kSteps - 1; ++t) {
        const float xt = xs[(PASS == 1) ? ((t + 128) & 255) : t];
        const float *Mc = Mbuf[t & 1];
        float *Mn = Mbuf[(t + 1) & 1];
        uint32_t bits = 0;
#pragma unroll
        for (int i = 0; i < G::GPL; ++i) {
            float Mk[G::NB];
#pragma unroll
            for (int k = 0; k < G::NB; ++k) Mk[k] = Mc[(k << G::MBITS) | m[i]];
            float outv[G::BPL];
#pragma unroll
            for (int bb = 0; bb < G::BPL; ++bb) {
                float a[G::NB];
#pragma unroll
                for (int k = 0; k < G::NB; ++k) {
                    float d = xt - v[i][k][bb];
                    float q = d * d;
                    a[k] = Mk[k] + q;
                }
                outv[bb] = acs<K>(a, bits);
            }
            float *dst = Mn + ((m[i] << K) | b0);
#pragma unroll
            for (int q4 = 0; q4 < G::BPL; q4 += 4)
                *reinterpret_cast<float4 *>(dst + q4) =
                    make_float4(outv[q4], outv[q4 + 1], outv[q4 + 2], outv[q4 + 3]);
        }
        if (PASS == 1) {
            if (t >= 127) bp_tile[(size_t)(t - 127) * kLanes + g] = (bp_t)bits;
        } else {
            bp_tile[(size_t)t * kLanes + g] = (bp_t)bits;
        }
        __syncthreads();
    }

    // last step: costs of all states, no minimum over predecessors
    const float xt = xs[(PASS == 1) ? 127 : 255];
    const float *Mc = Mbuf[(kSteps - 1) & 1];
    if (PASS == 1) {
        float best = 0.0f;
        uint32_t best_s = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < G::GPL; ++i)
#pragma unroll
            for (int k = 0; k < G::NB; ++k) {
                float mk = Mc[(k << G::MBITS) | m[i]];
#pragma unroll
                for (int bb = 0; bb < G::BPL; ++bb) {
                    float d = xt - v[i][k][bb];
                    float q = d * d;
                    float c = mk + q;
                    uint32_t s = ((uint32_t)k << G::Kr) | ((uint32_t)m[i] << K) | (uint32_t)(b0 + bb);
                    bool take = (best_s == 0xFFFFFFFFu) || (c < best) || (c == best && s < best_s);
                    best = take ? c : best;
                    best_s = take ? s : best_s;
                }
            }
        // lexicographic (cost, state) minimum over the wave, then the workgroup
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            float oc = __shfl_xor(best, off, 64);
            uint32_t os = __shfl_xor(best_s, off, 64);
            bool take = (oc < best) || (oc == best && os < best_s);
            best = take ? oc : best;
            best_s = take ? os : best_s;
        }
        if ((g & 63) == 0) {
            red_cost[g >> 6] = best;
            red_state[g >> 6] = best_s;
        }
        __syncthreads();
        if (g == 0) {
            float bc = red_cost[0];
            uint32_t bs = red_state[0];
            for (int w = 1; w < kLanes / 64; ++w) {
                float oc = red_cost[w];
                uint32_t os = red_state[w];
                if ((oc < bc) || (oc == bc && os < bs)) {
                    bc = oc;
                    bs = os;
                }
            }
            end_state[b] = (uint16_t)(bs & 0xFFFFu);
        }
    } else {
        const uint32_t X = X_in[b];
#pragma unroll
        for (int i = 0; i < G::GPL; ++i)
#pragma unroll
            for (int k = 0; k < G::NB; ++k) {
                float mk = Mc[(k << G::MBITS) | m[i]];
#pragma unroll
                for (int bb = 0; bb < G::BPL; ++bb) {
                    uint32_t s = ((uint32_t)k << G::Kr) | ((uint32_t)m[i] << K) | (uint32_t)(b0 + bb);
                    if (s == X) {
                        float d = xt - v[i][k][bb];
                        float q = d * d;
                        cost_out[b] = mk + q;
                    }
                }
            }
    }
}

template <int K, int PASS>
hipError_t launch_fwd_t(const float *x, const int32_t *tile_idx, int64_t tile0, int64_t n,
                        const uint16_t *levels, float scale, const uint16_t *X_in, void *bp,
                        uint16_t *end_state, float *cost_out, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL((viterbi_fwd_kernel<K, PASS>), dim3((unsigned)n), dim3(kLanes), 0, stream,
                       x, tile_idx, tile0, levels, scale, X_in,
                       reinterpret_cast<typename Geo<K>::bp_t *>(bp), end_state, cost_out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_viterbi_fwd(int K, int pass, const float *x, const int32_t *tile_idx,
                              int64_t tile0, int64_t n, const uint16_t *levels, float scale,
                              const uint16_t *X_in, void *bp, uint16_t *end_state,
                              float *cost_out, hipStream_t stream) {
#define EXL3_FWD_CASE(KK)                                                                    \
    case KK:                                                                                 \
        return pass == 1 ? launch_fwd_t<KK, 1>(x, tile_idx, tile0, n, levels, scale, X_in, bp, \
                                                end_state, cost_out, stream)                 \
                         : launch_fwd_t<KK, 2>(x, tile_idx, tile0, n, levels, scale, X_in, bp, \
                                                end_state, cost_out, stream);
    switch (K) {
        EXL3_FWD_CASE(2)
        EXL3_FWD_CASE(3)
        EXL3_FWD_CASE(4)
        default:
            return hipErrorInvalidValue;
    }
#undef EXL3_FWD_CASE
}

}  // namespace exl3
