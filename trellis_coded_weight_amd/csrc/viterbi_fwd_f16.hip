// Forward add-compare-select pass of the EXL3 tile encoder in binary16 on gfx950.
//
// Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture
// section 1 (the search runs in half precision: the branch difference is one
// binary16 subtraction and the path cost one fused multiply-add rounded once
// to binary16) and section 4 (state algebra; among equal costs the first
// branch wins).  Per state and step:
//     d = fp16(x_t - c[s]);  C[s] = fp16(d * d + M[s >> K])   (one rounding)
//     M'[e] = min_k C[(k << Kr) | e],  backpointer = lowest k reaching it.
// Levels are the raw binary16 code values (no scale in this mode).
//
// Same work split and two-pass schedule as the binary32 kernel (one 1024-lane
// workgroup per tile, 64 states per lane with their levels in registers --
// at K = 4 512 lanes of 128 states, so that two tiles share a compute unit --
// tracked minima double-buffered in LDS, half the bytes), but the outputs b
// and b + 1 of a butterfly share one register, so each packed instruction
// (v_pk_add_f16 with a negated operand, v_pk_fma_f16 with the predecessor
// cost broadcast to both halves by op_sel, v_pk_min_f16 / v_pk_minimum3_f16)
// does the work of two.
//
// Index bits without compares.  Costs are non-negative binary16 values or
// +inf, whose bit patterns (at most 0x7C00) order like the values.  For a
// candidate word c and the pair's minimum word m (c >= m in both halves),
//     c - (m + 0x80008001)  mod 2^32  =  (c_hi - m_hi + 0x7FFF) << 16
//                                       + (c_lo - m_lo + 0x7FFF)
// with both digits in [0x7FFF, 0xFBFF] (no carry between the halves), so bit
// 15 is [c_lo > m_lo] and bit 31 is [c_hi > m_hi].  A tournament walk over
// these flag words (v_bitop3_b32 selects) picks the lowest index reaching the
// minimum: at each level the minimum is in the right subtree exactly when the
// left subtree's minimum exceeds it.  v_perm_b32 turns bits 15 and 31 of two
// flag words into four 0x00 / 0xFF bytes, and one v_bitop3_b32 merges them
// into one bit of each byte of the step's backpointer word: two instructions
// per four index bits.
//
// On gfx950 the packed binary16 and min instructions issue at one per
// 4-cycle slot per SIMD, and mixing them with dual-issue-capable 32-bit
// operations was measured not to pair, so the kernel's cost is its
// instruction count: per output pair at K = 2, 4 v_pk_add + 4 v_pk_fma + 2
// minima, and in steps that keep backpointers 5 flag operations + 1 perm +
// 1 merge.
#include "exl3_internal.h"

namespace exl3 {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// bitop3 truth table (operands S0, S1, S2 <-> 0xF0, 0xCC, 0xAA): S2 ? S0 : S1
constexpr unsigned kSel = 0xE4;
// v_perm_b32 selectors 8..11 give a byte of copies of bit 15 / 31 of the low
// source and bit 15 / 31 of the high source
constexpr uint32_t kSignBytes = 0x0B0A0908u;

// flag word of c against the pair minimum (see the header comment)
__device__ __forceinline__ uint32_t flag(h2 c, uint32_t guard) { return u32(c) - guard; }
__device__ __forceinline__ uint32_t guard_of(h2 m) { return u32(m) + 0x80008001u; }

// cond ? a : b, bitwise (for a flag word only bits 15 and 31 of the result
// matter; for a half mask whole halves are selected)
__device__ __forceinline__ uint32_t sel(uint32_t cond, uint32_t a, uint32_t b) {
    return __builtin_amdgcn_bitop3_b32(a, b, cond, kSel);
}

// Flag word -> half mask: each half becomes all ones where its flag bit (15 or
// 31) is set, all zeros otherwise (one v_pk_ashrrev_i16)
__device__ __forceinline__ uint32_t half_mask(uint32_t f) {
    typedef short s2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(s2, f) >> (s2){15, 15});
}

// Four flags -> bit `pos` of each byte of acc: byte 0 / 1 <- bit 15 / 31 of
// lo, byte 2 / 3 <- bit 15 / 31 of hi.
__device__ __forceinline__ void merge(uint32_t &acc, uint32_t hi, uint32_t lo, int pos) {
    const uint32_t bytes = __builtin_amdgcn_perm(hi, lo, kSignBytes);
    acc = __builtin_amdgcn_bitop3_b32(bytes, acc, 0x01010101u << pos, kSel);
}

// Wave priority across a step, stepped down from 3 to 0 (as in the binary32
// kernel): waves that are behind keep priority over the ones finishing.  Used
// at K = 1 only (one workgroup per compute unit: +12 % measured).  At K = 2
// and 3 the kernel must fit 64 registers (two workgroups per compute unit) and
// the priority changes inside the unrolled step made the compiler spill; K = 4
// measured no gain.
__device__ __forceinline__ void step_priority(int e, int n) {
    if (e == 0) __builtin_amdgcn_s_setprio(3);
    if (e == n / 2) __builtin_amdgcn_s_setprio(2);
    if (e == 3 * n / 4) __builtin_amdgcn_s_setprio(1);
    if (e == 7 * n / 8) __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ h2 hmin(h2 a, h2 b) { return __builtin_elementwise_min(a, b); }
__device__ __forceinline__ h2 hmin3(h2 a, h2 b, h2 c) {
    return __builtin_elementwise_minimum(__builtin_elementwise_minimum(a, b), c);
}

// Minimum over the 2^K candidate words of one output pair; with BITS, the
// flag words r[0..K-1] of the lowest index reaching it (r[j] carries index
// bit j of both halves in bits 15 and 31).
template <int K, bool BITS>
struct AcsH;

template <bool BITS>
struct AcsH<1, BITS> {
    static __device__ __forceinline__ h2 run(const h2 (&a)[2], uint32_t (&r)[1]) {
        const h2 m = hmin(a[0], a[1]);
        if (BITS) r[0] = flag(a[0], guard_of(m));                  // index 1
        return m;
    }
};

template <bool BITS>
struct AcsH<2, BITS> {
    static __device__ __forceinline__ h2 run(const h2 (&a)[4], uint32_t (&r)[2]) {
        const h2 m01 = hmin(a[0], a[1]);
        const h2 m = hmin3(m01, a[2], a[3]);
        if (BITS) {
            const uint32_t gd = guard_of(m);
            r[1] = flag(m01, gd);                                     // index in {2, 3}
            r[0] = sel(r[1], flag(a[2], gd), flag(a[0], gd));
        }
        return m;
    }
};

template <bool BITS>
struct AcsH<3, BITS> {
    static __device__ __forceinline__ h2 run(const h2 (&a)[8], uint32_t (&r)[3]) {
        const h2 m01 = hmin(a[0], a[1]);
        const h2 m45 = hmin(a[4], a[5]);
        const h2 m0123 = hmin3(m01, a[2], a[3]);
        const h2 m4567 = hmin3(m45, a[6], a[7]);
        const h2 m = hmin(m0123, m4567);
        if (BITS) {
            // walk down with half masks: select the chosen subtree's left child
            // first, then flag only that one
            const uint32_t gd = guard_of(m);
            r[2] = flag(m0123, gd);                                   // index in 4..7
            const uint32_t k2 = half_mask(r[2]);
            r[1] = flag(as_h2(sel(k2, u32(m45), u32(m01))), gd);
            const uint32_t k1 = half_mask(r[1]);
            const uint32_t e0 = sel(k2, u32(a[4]), u32(a[0]));
            const uint32_t e1 = sel(k2, u32(a[6]), u32(a[2]));
            r[0] = flag(as_h2(sel(k1, e1, e0)), gd);
        }
        return m;
    }
};

template <bool BITS>
struct AcsH<4, BITS> {
    static __device__ __forceinline__ h2 run(const h2 (&a)[16], uint32_t (&r)[4]) {
        const h2 m01 = hmin(a[0], a[1]);
        const h2 m45 = hmin(a[4], a[5]);
        const h2 m89 = hmin(a[8], a[9]);
        const h2 mCD = hmin(a[12], a[13]);
        const h2 m0_3 = hmin3(m01, a[2], a[3]);
        const h2 m4_7 = hmin3(m45, a[6], a[7]);
        const h2 m8_11 = hmin3(m89, a[10], a[11]);
        const h2 m12_15 = hmin3(mCD, a[14], a[15]);
        const h2 m0_7 = hmin(m0_3, m4_7);
        const h2 m = hmin3(m0_7, m8_11, m12_15);
        if (BITS) {
            const uint32_t gd = guard_of(m);
            r[3] = flag(m0_7, gd);                                    // index in 8..15
            const uint32_t k3 = half_mask(r[3]);
            r[2] = flag(as_h2(sel(k3, u32(m8_11), u32(m0_3))), gd);  // left quad of the half
            const uint32_t k2 = half_mask(r[2]);
            const uint32_t plo = sel(k3, u32(m89), u32(m01));
            const uint32_t phi = sel(k3, u32(mCD), u32(m45));
            r[1] = flag(as_h2(sel(k2, phi, plo)), gd);               // left pair of the quad
            const uint32_t k1 = half_mask(r[1]);
            const uint32_t e0 = sel(k3, u32(a[8]), u32(a[0]));
            const uint32_t e1 = sel(k3, u32(a[10]), u32(a[2]));
            const uint32_t e2 = sel(k3, u32(a[12]), u32(a[4]));
            const uint32_t e3 = sel(k3, u32(a[14]), u32(a[6]));
            const uint32_t f0 = sel(k2, e2, e0);
            const uint32_t f1 = sel(k2, e3, e1);
            r[0] = flag(as_h2(sel(k1, f1, f0)), gd);                 // left leaf of the pair
        }
        return m;
    }
};

// Base index (in 16-bit units) of the tracked minima a lane's group i reads
// for branch k, and of the outputs it writes.
template <int K>
__device__ __forceinline__ int read_index(int g, int i, int k) {
    if (K == 1) return (k << 14) | (2 * g + 2048 * i);
    if (K == 2) return (k << 12) | (2 * g + 2048 * i);
    if (K == 3) return (k << 10) | g;
    return (k << 8) | (g >> 1);
}
template <int K>
__device__ __forceinline__ int write_index(int g, int i) {
    if (K <= 2) return (2 * g + 2048 * i) << K;
    if (K == 3) return g << 3;
    return 8 * g;
}
// State of (group i, butterfly j, branch k, pair p, half 0).
template <int K>
__device__ __forceinline__ uint32_t state_of(int g, int i, int j, int k, int p) {
    using G = GeoH<K>;
    uint32_t m, b;
    if (K <= 2) {
        m = 2 * g + j + 2048 * i;
        b = 2 * p;
    } else if (K == 3) {
        m = g;
        b = 2 * p;
    } else {
        m = g >> 1;
        b = 8 * (g & 1) + 2 * p;
    }
    return ((uint32_t)k << G::Kr) | (m << K) | b;
}

// Tracked-minimum words of the lane for branch k (K=2: one word holds the
// group's two adjacent butterflies; K=3, 4: the value sits in the low half).
template <int K>
__device__ __forceinline__ uint32_t read_m(const uint16_t *Mc, int g, int i, int k) {
    if (K <= 2) return *reinterpret_cast<const uint32_t *>(Mc + read_index<K>(g, i, k));
    return Mc[read_index<K>(g, i, k)];
}
template <int K>
__device__ __forceinline__ h2 bcast(uint32_t w, int j) {
    const h2 v = as_h2(w);
    return (K <= 2 && j == 1) ? h2{v.y, v.y} : h2{v.x, v.x};
}

// Backpointer word of a step (layout documented with bp_read_h): the flags of
// the lane's output pairs, merged a byte-bit at a time.
template <int K, bool BITS>
__device__ __forceinline__ uint32_t step_h(
    h2 xt, const uint16_t *__restrict__ Mc, uint16_t *__restrict__ Mn,
    const h2 (&v)[GeoH<K>::NI][GeoH<K>::NJ][GeoH<K>::NB][GeoH<K>::NP], int g) {
    using G = GeoH<K>;
    uint32_t Mw[G::NI][G::NB];
#pragma unroll
    for (int i = 0; i < G::NI; ++i)
#pragma unroll
        for (int k = 0; k < G::NB; ++k) Mw[i][k] = read_m<K>(Mc, g, i, k);
    uint32_t acc = 0;
    uint32_t r2prev = 0;
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
        uint32_t out[G::NJ * G::NP];
#pragma unroll
        for (int j = 0; j < G::NJ; ++j)
#pragma unroll
            for (int p = 0; p < G::NP; ++p) {
                if constexpr (K == 1)
                    step_priority((i * G::NJ + j) * G::NP + p, G::NI * G::NJ * G::NP);
                h2 a[G::NB];
#pragma unroll
                for (int k = 0; k < G::NB; ++k) {
                    const h2 d = xt - v[i][j][k][p];
                    a[k] = __builtin_elementwise_fma(d, d, bcast<K>(Mw[i][k], j));
                }
                uint32_t r[K];
                out[j * G::NP + p] = u32(AcsH<K, BITS>::run(a, r));
                if (BITS) {
                    const int q = (i * G::NJ + j) * G::NP + p;     // pair index in the lane
                    if (K == 1) {
                        if (q & 1)
                            merge(acc, r[0], r2prev, q >> 1);
                        else
                            r2prev = r[0];
                    } else if (K == 2) {
                        merge(acc, r[1 % K], r[0], q);
                    } else if (K == 3) {
                        merge(acc, r[1 % K], r[0], q);
                        if (q & 1)
                            merge(acc, r[2 % K], r2prev, 4 + (q >> 1));
                        else
                            r2prev = r[2 % K];
                    } else {
                        merge(acc, r[1 % K], r[0], 2 * q);
                        merge(acc, r[3 % K], r[2 % K], 2 * q + 1);
                    }
                }
            }
        uint16_t *dst = Mn + write_index<K>(g, i);
        if constexpr (G::NJ * G::NP == 4)
            *reinterpret_cast<uint4 *>(dst) = make_uint4(out[0], out[1], out[2], out[3]);
        else
            *reinterpret_cast<uint2 *>(dst) = make_uint2(out[0], out[1]);
    }
    return acc;
}

// Two tiles' workgroups share a compute unit, so one computes while the
// other waits at its step barrier: at K = 2 and 3 the kernel fits in 64
// registers per lane (two 1024-lane workgroups, 8 waves per SIMD); at K = 4 a
// tile has 512 lanes of 128 states in up to 128 registers (two workgroups, 4
// waves per SIMD).  K = 1's tracked minima (2 x 64 KiB) leave LDS for one
// workgroup.
template <int K>
struct WavesPerSimd {
    static constexpr int v = (K == 2 || K == 3) ? 8 : (K == 4) ? 4 : 1;
};

template <int K, int PASS>
__global__ void __launch_bounds__(GeoH<K>::LANES, WavesPerSimd<K>::v)
viterbi_fwd_f16_kernel(const uint16_t *__restrict__ x, int64_t tile0,
                       const uint16_t *__restrict__ levels, const uint16_t *__restrict__ X_in,
                       typename GeoH<K>::bp_t *__restrict__ bp, uint16_t *__restrict__ end_state,
                       uint16_t *__restrict__ cost_out) {
    using G = GeoH<K>;
    using bp_t = typename G::bp_t;
    __shared__ __attribute__((aligned(16))) uint16_t Mbuf[2][G::T];
    __shared__ uint32_t xs[kSteps];
    __shared__ uint32_t red[G::LANES / 64];

    const int g = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t tile = tile0 + b;

    // the input value twice per word; pass 1 reads position (t + 128) mod 256
    if (g < kSteps) {
        const uint32_t h = x[tile * kSteps + ((PASS == 1) ? ((g + 128) & 255) : g)];
        xs[g] = h | (h << 16);
    }

    // levels of the lane's 64 states: adjacent states, one word per pair
    h2 v[G::NI][G::NJ][G::NB][G::NP];
    const uint32_t *lv32 = reinterpret_cast<const uint32_t *>(levels);
#pragma unroll
    for (int i = 0; i < G::NI; ++i)
#pragma unroll
        for (int j = 0; j < G::NJ; ++j)
#pragma unroll
            for (int k = 0; k < G::NB; ++k)
#pragma unroll
                for (int p = 0; p < G::NP; ++p)
                    v[i][j][k][p] = as_h2(lv32[state_of<K>(g, i, j, k, p) >> 1]);

    const uint32_t xm = (PASS == 1) ? 0u : ((uint32_t)X_in[b] & (uint32_t)(G::T - 1));
    for (int e = g; e < G::T; e += G::LANES)
        Mbuf[0][e] = (PASS == 1 || (uint32_t)e == xm) ? (uint16_t)0 : (uint16_t)0x7C00;
    __syncthreads();

    bp_t *bp_tile = bp + (size_t)b * kSlots * G::LANES;
    constexpr int t_first = (PASS == 1) ? 127 : 0;
    uint16_t *const B0 = Mbuf[0];
    uint16_t *const B1 = Mbuf[1];
    h2 xt = as_h2(xs[0]);
    int t = 0;
    if constexpr (PASS == 1) {
        for (; t + 1 < t_first; t += 2) {           // steps 0..125 in pairs
            const h2 xn = as_h2(xs[t + 1]);
            step_h<K, false>(xt, B0, B1, v, g);
            __syncthreads();
            xt = as_h2(xs[t + 2]);
            step_h<K, false>(xn, B1, B0, v, g);
            __syncthreads();
        }
        {                                           // step 126: B0 -> B1
            const h2 xn = as_h2(xs[t + 1]);
            step_h<K, false>(xt, B0, B1, v, g);
            __syncthreads();
            xt = xn;
            ++t;
        }
        for (; t < kSteps - 1; t += 2) {            // steps 127..254: B1 -> B0 -> B1
            const h2 xn = as_h2(xs[t + 1]);
            uint32_t w = step_h<K, true>(xt, B1, B0, v, g);
            bp_tile[(size_t)(t - t_first) * G::LANES + g] = (bp_t)w;
            __syncthreads();
            xt = xn;
            if (t + 1 < kSteps - 1) {
                xt = as_h2(xs[t + 2]);
                w = step_h<K, true>(xn, B0, B1, v, g);
                bp_tile[(size_t)(t + 1 - t_first) * G::LANES + g] = (bp_t)w;
                __syncthreads();
            }
        }
    } else {
        for (; t < kSteps - 1; t += 2) {            // steps 0..254: B0 -> B1 -> B0
            const h2 xn = as_h2(xs[t + 1]);
            uint32_t w = step_h<K, true>(xt, B0, B1, v, g);
            bp_tile[(size_t)t * G::LANES + g] = (bp_t)w;
            __syncthreads();
            xt = xn;
            if (t + 1 < kSteps - 1) {
                xt = as_h2(xs[t + 2]);
                w = step_h<K, true>(xn, B1, B0, v, g);
                bp_tile[(size_t)(t + 1) * G::LANES + g] = (bp_t)w;
                __syncthreads();
            }
        }
    }

    // last step: costs of all states, no minimum over predecessors
    xt = as_h2(xs[kSteps - 1]);
    const uint16_t *Mc = Mbuf[(kSteps - 1) & 1];
    if (PASS == 1) {
        // lexicographic (cost, state) minimum: cost bits above the state index
        uint32_t best = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < G::NI; ++i)
#pragma unroll
            for (int k = 0; k < G::NB; ++k) {
                const uint32_t w = read_m<K>(Mc, g, i, k);
#pragma unroll
                for (int j = 0; j < G::NJ; ++j)
#pragma unroll
                    for (int p = 0; p < G::NP; ++p) {
                        const h2 d = xt - v[i][j][k][p];
                        const uint32_t c = u32(__builtin_elementwise_fma(d, d, bcast<K>(w, j)));
                        const uint32_t s = state_of<K>(g, i, j, k, p);
                        best = min(best, ((c & 0xFFFFu) << 16) | s);
                        best = min(best, (c & 0xFFFF0000u) | (s + 1u));
                    }
            }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) best = min(best, (uint32_t)__shfl_xor((int)best, off, 64));
        if ((g & 63) == 0) red[g >> 6] = best;
        __syncthreads();
        if (g == 0) {
            uint32_t r = red[0];
            for (int w = 1; w < G::LANES / 64; ++w) r = min(r, red[w]);
            end_state[b] = (uint16_t)(r & 0xFFFFu);
        }
    } else {
        const uint32_t X = X_in[b];
#pragma unroll
        for (int i = 0; i < G::NI; ++i)
#pragma unroll
            for (int k = 0; k < G::NB; ++k)
#pragma unroll
                for (int j = 0; j < G::NJ; ++j)
#pragma unroll
                    for (int p = 0; p < G::NP; ++p) {
                        const uint32_t s = state_of<K>(g, i, j, k, p);
                        if ((X & ~1u) == s) {
                            const uint32_t w = read_m<K>(Mc, g, i, k);
                            const h2 d = xt - v[i][j][k][p];
                            const uint32_t c =
                                u32(__builtin_elementwise_fma(d, d, bcast<K>(w, j)));
                            cost_out[b] = (uint16_t)((X & 1u) ? (c >> 16) : (c & 0xFFFFu));
                        }
                    }
    }
}

template <int K, int PASS>
hipError_t launch_t(const uint16_t *x, int64_t tile0, int64_t n, const uint16_t *levels,
                    const uint16_t *X_in, void *bp, uint16_t *end_state, uint16_t *cost_out,
                    hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL((viterbi_fwd_f16_kernel<K, PASS>), dim3((unsigned)n),
                       dim3(GeoH<K>::LANES), 0,
                       stream, x, tile0, levels, X_in,
                       reinterpret_cast<typename GeoH<K>::bp_t *>(bp), end_state, cost_out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_viterbi_fwd_f16(int K, int pass, const uint16_t *x, int64_t tile0, int64_t n,
                                  const uint16_t *levels, const uint16_t *X_in, void *bp,
                                  uint16_t *end_state, uint16_t *cost_out, hipStream_t stream) {
#define EXL3_FWDH_CASE(KK)                                                                   \
    case KK:                                                                                 \
        return pass == 1 ? launch_t<KK, 1>(x, tile0, n, levels, X_in, bp, end_state,        \
                                           cost_out, stream)                                \
                         : launch_t<KK, 2>(x, tile0, n, levels, X_in, bp, end_state,        \
                                           cost_out, stream);
    switch (K) {
        EXL3_FWDH_CASE(1)
        EXL3_FWDH_CASE(2)
        EXL3_FWDH_CASE(3)
        EXL3_FWDH_CASE(4)
        default:
            return hipErrorInvalidValue;
    }
#undef EXL3_FWDH_CASE
}

}  // namespace exl3
