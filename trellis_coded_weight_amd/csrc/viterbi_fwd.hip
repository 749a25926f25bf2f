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
//   pass 3: pass 2 without backpointers, for callers that need only the path
//           cost (scale-search probes).
#include "exl3_internal.h"

#include <math.h>


namespace exl3 {
namespace {

// Wave priority across a step: 3 from the step's first update, 2 from half of
// its updates, 1 from three quarters, 0 from seven eighths.  The 16 waves of a
// tile meet at a barrier after every step; waves that are behind (their
// predecessor costs arrived late) keep a higher priority than the ones
// finishing, so fewer quad-cycles are left idle before the barrier (A/B on one
// box: 2-4 % shorter forward launches at K = 2).
__device__ __forceinline__ void step_priority(int e, int n) {
    if (e == 0) __builtin_amdgcn_s_setprio(3);
    if (e == n / 2) __builtin_amdgcn_s_setprio(2);
    if (e == 3 * n / 4) __builtin_amdgcn_s_setprio(1);
    if (e == 7 * n / 8) __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

template <int K>
__device__ __forceinline__ void lane_butterflies(int g, int (&m)[Geo<K>::GPL], int &b0) {
    using G = Geo<K>;
    if (K <= 2) {
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

// The scaled levels v = rn(scale * c) of the lane's 64 states, as binary32
// registers for the whole pass.
template <int K>
struct Levels {
    using G = Geo<K>;
    float v[G::GPL][G::NB][G::BPL];
    __device__ __forceinline__ void set(int i, int k, int bb, uint16_t c, float scale) {
        v[i][k][bb] = scale * half_bits_to_float(c);
    }
    __device__ __forceinline__ float at(int i, int k, int bb) const { return v[i][k][bb]; }
};

// Append one bit per lane to acc: acc = 2 * acc + mask[lane] in one VALU op
// (add with carry-in taken from the 64-bit lane mask).
// The carry-outs go to scratch scalar pairs that nothing reads (writing VCC
// here instead was measured to slow the whole loop down markedly); the K
// insertions of one update form a single asm block.
template <int K>
__device__ __forceinline__ void push_bits(uint32_t &acc, const uint64_t (&kb)[K]);
template <>
__device__ __forceinline__ void push_bits<1>(uint32_t &acc, const uint64_t (&kb)[1]) {
    uint64_t c0;
    asm("v_addc_co_u32_e64 %0, %1, %0, %0, %2" : "+v"(acc), "=&s"(c0) : "s"(kb[0]));
}
template <>
__device__ __forceinline__ void push_bits<4>(uint32_t &acc, const uint64_t (&kb)[4]) {
    uint64_t c0, c1, c2, c3;
    asm("v_addc_co_u32_e64 %0, %1, %0, %0, %5\n\t"
        "v_addc_co_u32_e64 %0, %2, %0, %0, %6\n\t"
        "v_addc_co_u32_e64 %0, %3, %0, %0, %7\n\t"
        "v_addc_co_u32_e64 %0, %4, %0, %0, %8"
        : "+v"(acc), "=&s"(c0), "=&s"(c1), "=&s"(c2), "=&s"(c3)
        : "s"(kb[0]), "s"(kb[1]), "s"(kb[2]), "s"(kb[3]));
}

// Lowest-index minimum as one binary64 minimum.  A candidate is the register
// pair {low word: its index k, high word: the bits of its binary32 cost}.
// Costs are non-negative (or +inf) binary32 values, whose bit patterns order
// like the values, and such a pair read as a binary64 number is non-negative
// and never a NaN; binary64 order of these pairs is therefore the
// lexicographic order of (cost, index), and v_min_f64 returns the cheaper
// candidate, the lower index on equal costs -- exactly, since it returns one
// of its operands (double-precision denormals are kept).  The winner's high
// word is the new minimum, its low word the backpointer.
__device__ __forceinline__ double cost_index(float a, uint32_t k) {
    return __builtin_bit_cast(double, ((uint64_t)__float_as_uint(a) << 32) | k);
}
__device__ __forceinline__ double lex_min(double a, double b) {
    double r;
    asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// acc = (acc << K) | k in one instruction (the compiler would otherwise
// re-associate the chain of insertions into shifts and three-way ors)
template <int K>
__device__ __forceinline__ void push_index(uint32_t &acc, uint32_t k) {
    asm("v_lshl_or_b32 %0, %0, %2, %1" : "+v"(acc) : "v"(k), "i"(K));
}

// Minimum of the 2^K candidates and the lowest index reaching it, with the K
// index bits appended to acc (high bit first).
//
// K = 1 and 4, the compare walk: a tournament tree is built bottom-up but only
// the left child of every node on a root-to-leaf path is ever needed: walking
// down from the root, the minimum lies in the right subtree exactly when the
// left child's minimum is larger than the overall minimum (equal values keep
// the left, i.e. lower, index).  Each step of the walk is one compare, whose lane mask is both the
// next index bit (inserted with add-with-carry) and the selector that picks
// the next left child.  No scalar instructions are involved.
template <int K>
struct Acs;

template <>
struct Acs<1> {
    static __device__ __forceinline__ float run(const float (&a)[2], uint32_t &acc) {
        const float m = __builtin_fminf(a[0], a[1]);
        const uint64_t kb[1] = {__builtin_amdgcn_ballot_w64(a[0] > m)};
        push_bits<1>(acc, kb);
        return m;
    }
};

// K = 3: the binary64 lexicographic tournament (seven v_min_f64 and one
// insertion; as many issue slots as the compare walk but no lane-mask
// latencies: 2 % faster measured).
template <>
struct Acs<3> {
    static __device__ __forceinline__ float run(const float (&a)[8], uint32_t &acc) {
        double c[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) c[k] = cost_index(a[k], (uint32_t)k);
        const double t03 = lex_min(lex_min(c[0], c[1]), lex_min(c[2], c[3]));
        const double t47 = lex_min(lex_min(c[4], c[5]), lex_min(c[6], c[7]));
        const uint64_t w = __builtin_bit_cast(uint64_t, lex_min(t03, t47));
        push_index<3>(acc, (uint32_t)w);
        return __uint_as_float((uint32_t)(w >> 32));
    }
};

template <>
struct Acs<4> {
    static __device__ __forceinline__ float run(const float (&a)[16], uint32_t &acc) {
        const float m01 = __builtin_fminf(a[0], a[1]);
        const float m45 = __builtin_fminf(a[4], a[5]);
        const float m89 = __builtin_fminf(a[8], a[9]);
        const float mCD = __builtin_fminf(a[12], a[13]);
        const float m67 = __builtin_fminf(a[6], a[7]);
        const float m0_3 = __builtin_fminf(__builtin_fminf(m01, a[2]), a[3]);
        const float m8_11 = __builtin_fminf(__builtin_fminf(m89, a[10]), a[11]);
        const float m0_7 = __builtin_fminf(__builtin_fminf(m0_3, m45), m67);
        const float m12_15 = __builtin_fminf(__builtin_fminf(mCD, a[14]), a[15]);
        const float m = __builtin_fminf(__builtin_fminf(m0_7, m8_11), m12_15);
        const bool r3 = m0_7 > m;                     // index in 8..15
        const float l2 = r3 ? m8_11 : m0_3;           // left quad of the chosen half
        const bool r2 = l2 > m;
        const float q_lo = r2 ? m45 : m01;            // left pair of the chosen quad
        const float q_hi = r2 ? mCD : m89;
        const float l1 = r3 ? q_hi : q_lo;
        const bool r1 = l1 > m;
        const float p0 = r1 ? a[2] : a[0];            // left leaf of the chosen pair
        const float p1 = r1 ? a[6] : a[4];
        const float p2 = r1 ? a[10] : a[8];
        const float p3 = r1 ? a[14] : a[12];
        const float h0 = r2 ? p1 : p0;
        const float h1 = r2 ? p3 : p2;
        const float l0 = r3 ? h1 : h0;
        const bool r0 = l0 > m;
        const uint64_t kb[4] = {__builtin_amdgcn_ballot_w64(r3), __builtin_amdgcn_ballot_w64(r2),
                                __builtin_amdgcn_ballot_w64(r1), __builtin_amdgcn_ballot_w64(r0)};
        push_bits<4>(acc, kb);
        return m;
    }
};

// Minimum of the 2^K candidates only (steps whose backpointers are not kept).
template <int NB>
__device__ __forceinline__ float min_only(const float (&a)[NB]) {
    if constexpr (NB == 2) return __builtin_fminf(a[0], a[1]);
    float r = __builtin_fminf(__builtin_fminf(a[0], a[1]), a[2]);
#pragma unroll
    for (int j = 3; j + 1 < NB; j += 2) r = __builtin_fminf(__builtin_fminf(r, a[j]), a[j + 1]);
    if (NB % 2 == 0) r = __builtin_fminf(r, a[NB - 1]);
    return r;
}

// K = 1 keeps one copy of its 2^15 tracked minima (128 KiB) plus one spare
// 32 KiB slot: quarter Q (entries 8192 Q ..) lives at its own offset, except
// Q1, which moves between its own slot and the spare every step (steps of
// parity 0 read it at 8192 and write it at 32768, parity 1 the reverse).  A
// lane's butterflies 4..7 produce its part of the new Q1, so they run first,
// before the barrier that lets the others overwrite Q0, Q2, Q3 in place, and
// their work overlaps the step's reads.
constexpr int k1_q1_slot(int par) { return par ? 32768 : 8192; }
constexpr int k1_order(int ii) { return ii < 8 ? (ii ^ 4) : ii; }

// Pass 2 at K = 2 stores tracked minimum e at LDS word (e >> 2) + kSkew2 *
// (e & 3): four planes by the low two bits, each 4096 words, 8 words apart.  A lane's four
// new minima (m << 2) | b then go to words m + kSkew2 * b, consecutive across
// the lanes of a wave for every b, so each one-word store hits 32 distinct
// banks (in the natural order they are four words apart: an 8-way conflict on
// the 32 banks), and the minima of butterflies m and m + 1024 at one b, 1024
// words apart, go out as one two-word store (ds_write2st64, 8 per step instead
// of 16 one-word stores: A/B on one box, pass 2 1.6 % shorter); the reads of
// M[(k << 12) | m] land on words
// (g >> 2) + kSkew2 * (g & 3) + 1024 k + 256 i, where the skew of 8 words per
// plane spreads every 32 consecutive lanes over 32 banks as well.  Offsets stay
// below 64 KiB, so both access kinds use one base register plus immediates.
// Pass 1 and the cost-only pass keep the natural order: their steps without
// backpointers store four adjacent minima with one ds_write_b128, and as
// sixteen one-word stores those steps measured 1 % slower (A/B on one box),
// while pass 2 gained 0.5 %: the conflicts are not what bounds the step.
constexpr int kSkew2 = 4104;
constexpr int kWords2 = 4096 + 3 * kSkew2;   // words per K = 2 buffer (24 unused)

template <int K, int PASS>
constexpr bool skewed() { return K == 2 && PASS == 2; }

template <int K, bool SKEW>
__device__ __forceinline__ uint32_t lds_word(uint32_t e) {
    if constexpr (SKEW) return (e >> 2) + (uint32_t)kSkew2 * (e & 3u);
    else return e;
}
template <int K, bool SKEW>
constexpr int lds_words() { return SKEW ? kWords2 : Geo<K>::T; }

// One trellis step for the lane's 64 states: read the tracked minima of its
// butterflies from Mc, write the new minima to Mn and return the backpointer
// word (BITS) -- or only the minima (!BITS, steps whose backpointers are never
// read).  At K = 2 with bits the lane's 16 updates are software-pipelined so
// that no binary64 minimum is read right after it is written: iteration e
// issues the branch metrics of update e and the two pair minima of its
// candidates, the final minimum (and the store of the new tracked minimum) of
// update e-1, and the index insertion of update e-2.  In the skewed layout
// (pass 2) the updates run butterfly pair by butterfly pair, so that the two
// minima of a two-word store are ready together, and each index goes into its
// own field of the word (the same word as in the natural order).
// Passes 2 and 3 start with one tracked minimum finite (the one X admits), and
// after t steps only 2^(K (t + 1)) of them are: until they fill the tracked set
// most waves read nothing but +inf.  When every candidate of a wave is +inf,
// every new minimum is +inf and the lowest index reaching it is 0 -- exactly
// what the full step would compute -- so such a wave stores those and skips
// the step (a wave-uniform test, SKIP steps only: the first 6 / 4 / 2 at
// K = 2 / 3 / 4; at K = 1 none).
template <int K>
constexpr int skip_steps() { return K == 2 ? 6 : K == 3 ? 4 : K == 4 ? 2 : 0; }

template <int K, bool BITS, int PAR, bool SKEW, bool SKIP = false>
__device__ __forceinline__ uint32_t trellis_step(
    float xt, const float *__restrict__ Mc, float *__restrict__ Mn,
    const Levels<K> &lv, const int (&m)[Geo<K>::GPL], int b0) {
    using G = Geo<K>;
    float Mk[G::GPL][G::NB];
    // K = 1: the LDS offsets of quarter Q1 read and written by a step of parity
    // PAR (see k1_q1_slot)
    [[maybe_unused]] constexpr int q1r = k1_q1_slot(PAR), q1w = k1_q1_slot(PAR ^ 1);
    // K = 1: the lane's 32 reads and 16 writes span 128 KiB, past the 16-bit
    // LDS immediates; with the lane's index opaque to the compiler they are
    // addressed from four base registers plus immediates, not one address
    // register each
    int lb = m[0];
    if constexpr (K == 1) asm volatile("" : "+v"(lb));
    if constexpr (K == 1) {
        // butterflies 4..7 (which write Q1 into the free slot) first
        const float *r0 = Mc + lb, *r0q = Mc + q1r + lb, *r1 = Mc + (1 << G::MBITS) + lb;
#pragma unroll
        for (int ii = 0; ii < G::GPL; ++ii) {
            const int i = k1_order(ii);
            Mk[i][0] = i < 8 ? r0[kLanes * i] : r0q[kLanes * (i - 8)];
            Mk[i][1] = r1[kLanes * i];
        }
    } else if constexpr (SKEW) {
        // M[(k << 12) | m[i]], m[i] = m[0] + 1024 i: one base plus immediates
        const float *r = Mc + lds_word<2, true>((uint32_t)m[0]);
#pragma unroll
        for (int i = 0; i < G::GPL; ++i)
#pragma unroll
            for (int k = 0; k < G::NB; ++k) Mk[i][k] = r[1024 * k + 256 * i];
    } else {
#pragma unroll
        for (int i = 0; i < G::GPL; ++i)
#pragma unroll
            for (int k = 0; k < G::NB; ++k) Mk[i][k] = Mc[(k << G::MBITS) | m[i]];
    }
    if constexpr (SKIP) {
        static_assert(K != 1, "K = 1 steps hold a barrier");
        bool finite = false;
#pragma unroll
        for (int i = 0; i < G::GPL; ++i)
#pragma unroll
            for (int k = 0; k < G::NB; ++k) finite = finite || Mk[i][k] != INFINITY;
        if (__builtin_amdgcn_ballot_w64(finite) == 0) {
            // the same stores as the full step's (see its end)
#pragma unroll
            for (int i = 0; i < G::GPL; ++i) {
                float *dst = Mn + ((m[i] << K) | b0);
                if constexpr (SKEW) {
#pragma unroll
                    for (int bb = 0; bb < G::BPL; ++bb) Mn[m[i] + kSkew2 * bb] = INFINITY;
                } else if constexpr (G::BPL == 2) {
                    *reinterpret_cast<float2 *>(dst) = make_float2(INFINITY, INFINITY);
                } else {
#pragma unroll
                    for (int q4 = 0; q4 < G::BPL; q4 += 4)
                        *reinterpret_cast<float4 *>(dst + q4) =
                            make_float4(INFINITY, INFINITY, INFINITY, INFINITY);
                }
            }
            return 0u;
        }
    }
    uint32_t bits = 0;
    if constexpr (BITS && K == 2 && SKEW) {
        // the updates in the order (p, bb, ii), i = 2p + ii: the new minima of
        // butterflies 2p and 2p + 1 at the same bb are 1024 words apart in the
        // skewed layout, so they go out as one two-word store; each index goes
        // to its fixed field of the backpointer word
        constexpr int NE = 16;
        double T01[2], T23[2];
        uint32_t kk[2];
        float mlo = 0.0f;
#pragma unroll
        for (int e = 0; e < NE + 2; ++e) {
            step_priority(e, NE);
            if (e < NE) {
                const int i = 2 * (e >> 3) + (e & 1), bb = (e >> 1) & 3;
                double c[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    float d = xt - lv.at(i, k, bb);
                    float q = d * d;
                    c[k] = cost_index(Mk[i][k] + q, (uint32_t)k);
                }
                T01[e & 1] = lex_min(c[0], c[1]);
                T23[e & 1] = lex_min(c[2], c[3]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (e >= 1 && e - 1 < NE) {
                const int f = e - 1, i = 2 * (f >> 3) + (f & 1), bb = (f >> 1) & 3;
                const uint64_t w = __builtin_bit_cast(uint64_t, lex_min(T01[f & 1], T23[f & 1]));
                kk[f & 1] = (uint32_t)w;
                const float mv = __uint_as_float((uint32_t)(w >> 32));
                if ((f & 1) == 0) {
                    mlo = mv;
                } else {
                    float *dst = Mn + lds_word<K, SKEW>((uint32_t)((m[i - 1] << K) | (b0 + bb)));
                    dst[0] = mlo;
                    dst[1024] = mv;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (e >= 2) {
                const int f = e - 2, i = 2 * (f >> 3) + (f & 1), bb = (f >> 1) & 3;
                const int sh = 2 * (15 - (4 * i + bb));
                asm("v_lshl_or_b32 %0, %1, %2, %0" : "+v"(bits) : "v"(kk[e & 1]), "i"(sh));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    } else if constexpr (BITS && K == 2) {
        constexpr int NE = G::GPL * G::BPL;
        double T01[2], T23[2];
        uint32_t kk[2];
#pragma unroll
        for (int e = 0; e < NE + 2; ++e) {
            step_priority(e, NE);
            if (e < NE) {
                const int i = e / G::BPL, bb = e % G::BPL;
                double c[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    float d = xt - lv.at(i, k, bb);
                    float q = d * d;
                    c[k] = cost_index(Mk[i][k] + q, (uint32_t)k);
                }
                T01[e & 1] = lex_min(c[0], c[1]);
                T23[e & 1] = lex_min(c[2], c[3]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (e >= 1 && e - 1 < NE) {
                const int f = e - 1, i = f / G::BPL, bb = f % G::BPL;
                const uint64_t w = __builtin_bit_cast(uint64_t, lex_min(T01[f & 1], T23[f & 1]));
                kk[f & 1] = (uint32_t)w;
                // one store per new minimum: the minima are the high halves
                // of register pairs, so a four-wide store would need moves
                __hip_atomic_store(Mn + lds_word<K, SKEW>((uint32_t)((m[i] << K) | (b0 + bb))),
                                   __uint_as_float((uint32_t)(w >> 32)), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (e >= 2) push_index<2>(bits, kk[e & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
#pragma unroll
        for (int ii = 0; ii < G::GPL; ++ii) {
            // K = 1: butterflies 4..7 write quarter Q1 into the free slot; the
            // others overwrite their quarters in place, once every lane has
            // read its predecessors (the barrier after the first four)
            const int i = K == 1 ? k1_order(ii) : ii;
            if (K == 1 && ii == 4) __syncthreads();
            float outv[G::BPL];
#pragma unroll
            for (int bb = 0; bb < G::BPL; ++bb) {
                step_priority(ii * G::BPL + bb, G::GPL * G::BPL);
                float a[G::NB];
#pragma unroll
                for (int k = 0; k < G::NB; ++k) {
                    float d = xt - lv.at(i, k, bb);
                    float q = d * d;
                    a[k] = Mk[i][k] + q;
                }
                if constexpr (BITS) outv[bb] = Acs<K>::run(a, bits);
                else outv[bb] = min_only<G::NB>(a);
            }
            // K = 1 outputs 2m, 2m + 1 of butterfly m = lb + 1024 i: quarter i / 4
            float *dst = Mn + ((m[i] << K) | b0);
            if constexpr (K == 1)
                dst = i < 4   ? Mn + 2 * lb + 2 * kLanes * i
                      : i < 8 ? Mn + q1w + 2 * lb + 2 * kLanes * (i - 4)
                              : Mn + (1 << (G::Kr - 1)) + 2 * lb + 2 * kLanes * (i - 8);
            if constexpr (SKEW) {
                // one word per new minimum into its plane (see kSkew2)
#pragma unroll
                for (int bb = 0; bb < G::BPL; ++bb) Mn[m[i] + kSkew2 * bb] = outv[bb];
            } else if constexpr (G::BPL == 2) {
                *reinterpret_cast<float2 *>(dst) = make_float2(outv[0], outv[1]);
            } else {
#pragma unroll
                for (int q4 = 0; q4 < G::BPL; q4 += 4)
                    *reinterpret_cast<float4 *>(dst + q4) =
                        make_float4(outv[q4], outv[q4 + 1], outv[q4 + 2], outv[q4 + 3]);
            }
        }
    }
    return bits;
}

// K = 2, passes 2 and 3: a quarter of a step, where the rest of it provably
// does not matter.  Both ends of these passes are pinned by X:
//  * in step t <= 5 the finite tracked minima all come from X's low bits and
//    t + 1 new symbols, so the butterflies with finite inputs all have the same
//    index i_t = (X >> (10 - 2t)) & 3 among each lane's four (FIX = 0, V = i_t):
//    the lane runs that butterfly's four updates and stores +inf, the exact
//    result, for the other twelve (every minimum is written, so the two buffers
//    hold exactly what the full steps would leave there);
//  * in step 254 - j, j <= 6, only minima that can lead to the state X read at
//    the end matter, and those all end in the same symbol b = (X >> (2 + 2j))
//    & 3 (FIX = 1, V = b): the lane runs its four updates at position b and
//    leaves the other minima as they were (no later update that matters reads
//    them); the traceback from X reads only these backpointer fields.
// The updates that run are the full step's, operation for operation.
template <bool BITS, bool SKEW, int FIX, int V>
__device__ __forceinline__ uint32_t part_step2_v(float xt, const float *__restrict__ Mc,
                                                 float *__restrict__ Mn, const Levels<2> &lv,
                                                 const int (&m)[4]) {
    float Mk[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (FIX == 1 || i == V)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                Mk[i][k] = Mc[lds_word<2, SKEW>(((uint32_t)k << 12) | (uint32_t)m[i])];
    if constexpr (FIX == 0) {
        bool finite = false;
#pragma unroll
        for (int k = 0; k < 4; ++k) finite = finite || Mk[V][k] != INFINITY;
        const bool live = __builtin_amdgcn_ballot_w64(finite) != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i != V || !live)
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
                    Mn[lds_word<2, SKEW>(((uint32_t)m[i] << 2) | (uint32_t)bb)] = INFINITY;
        if (!live) return 0u;
    }
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            if ((FIX == 0 && i != V) || (FIX == 1 && bb != V)) continue;
            double c[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float d = xt - lv.at(i, k, bb);
                float q = d * d;
                c[k] = cost_index(Mk[i][k] + q, (uint32_t)k);
            }
            const uint64_t w =
                __builtin_bit_cast(uint64_t, lex_min(lex_min(c[0], c[1]), lex_min(c[2], c[3])));
            Mn[lds_word<2, SKEW>(((uint32_t)m[i] << 2) | (uint32_t)bb)] =
                __uint_as_float((uint32_t)(w >> 32));
            if constexpr (BITS) bits |= ((uint32_t)w & 3u) << (2 * (15 - (4 * i + bb)));
        }
    return bits;
}

template <bool BITS, bool SKEW, int FIX>
__device__ __forceinline__ uint32_t part_step2(int v, float xt, const float *__restrict__ Mc,
                                               float *__restrict__ Mn, const Levels<2> &lv,
                                               const int (&m)[4]) {
    switch (v) {
        case 0: return part_step2_v<BITS, SKEW, FIX, 0>(xt, Mc, Mn, lv, m);
        case 1: return part_step2_v<BITS, SKEW, FIX, 1>(xt, Mc, Mn, lv, m);
        case 2: return part_step2_v<BITS, SKEW, FIX, 2>(xt, Mc, Mn, lv, m);
        default: return part_step2_v<BITS, SKEW, FIX, 3>(xt, Mc, Mn, lv, m);
    }
}

constexpr int kPartHead = 6;                   // K = 2: steps 0..5 on one butterfly
constexpr int kPartTail = 7;                   // K = 2: steps 248..254 on one position

template <int K, int PASS>
__global__ void __launch_bounds__(kLanes, 1)
viterbi_fwd_kernel(const float *__restrict__ x, const int32_t *__restrict__ tile_idx,
                   int64_t tile0, const uint16_t *__restrict__ levels, float scale,
                   const float *__restrict__ scale_dev, const uint16_t *__restrict__ X_in,
                   typename Geo<K>::bp_t *__restrict__ bp, uint16_t *__restrict__ end_state,
                   float *__restrict__ cost_out, bool scale_per_tile) {
    using G = Geo<K>;
    using bp_t = typename G::bp_t;
    constexpr bool SKEW = skewed<K, PASS>();
    constexpr int NBUF = (K == 1) ? 1 : 2;          // K = 1: one 128 KiB copy + a spare
    // K = 1 takes the whole 160 KiB of LDS: its inputs are read from global
    // memory each step and the end-of-pass reduction uses the Q1 slot that
    // the last step does not read
    float *Mb, *xs, *red_cost;
    uint32_t *red_state;
    if constexpr (K == 1) {
        __shared__ float smem1[5 * 8192];
        Mb = smem1;
        xs = nullptr;
        red_cost = smem1 + k1_q1_slot(0);
        red_state = reinterpret_cast<uint32_t *>(smem1 + k1_q1_slot(0) + kLanes / 64);
    } else {
        __shared__ float Mbuf[NBUF * lds_words<K, SKEW>()];
        __shared__ float xs_s[kSteps];
        __shared__ float red_cost_s[kLanes / 64];
        __shared__ uint32_t red_state_s[kLanes / 64];
        Mb = Mbuf;
        xs = xs_s;
        red_cost = red_cost_s;
        red_state = red_state_s;
    }

    const int g = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t tile = tile_idx ? (int64_t)tile_idx[b] : tile0 + b;

    // step t reads the input at position (t + 128) mod 256 in pass 1 (rotated)
    const float *x_tile = x + tile * kSteps;
    auto xin = [&](int t) -> float {
        if constexpr (K == 1) return x_tile[(PASS == 1) ? ((t + 128) & 255) : t];
        else return xs[t];
    };
    if constexpr (K != 1)
        if (g < kSteps) xs[g] = x_tile[(PASS == 1) ? ((g + 128) & 255) : g];

    int m[G::GPL];
    int b0;
    lane_butterflies<K>(g, m, b0);

    // levels of the lane's 64 states, scaled once per pass (the scale from
    // device memory when given: a search that chooses it on the device, or one
    // scale per tile for a batch of a search's points)
    if (scale_dev) scale = scale_dev[scale_per_tile ? b : 0];
    Levels<K> lv;
#pragma unroll
    for (int i = 0; i < G::GPL; ++i)
#pragma unroll
        for (int k = 0; k < G::NB; ++k)
#pragma unroll
            for (int bb = 0; bb < G::BPL; ++bb) {
                uint32_t s = ((uint32_t)k << G::Kr) | ((uint32_t)m[i] << K) | (uint32_t)(b0 + bb);
                lv.set(i, k, bb, levels[s], scale);
            }

    const uint32_t xm = (PASS == 1) ? 0u : ((uint32_t)X_in[b] & (uint32_t)(G::T - 1));
    // the first step's buffer, by LDS word (K = 2: unused padding words included)
    const uint32_t xw = lds_word<K, SKEW>(xm);
    for (int w = g; w < lds_words<K, SKEW>(); w += kLanes)
        Mb[w] = (PASS == 1 || (uint32_t)w == xw) ? 0.0f : INFINITY;
    __syncthreads();

    bp_t *bp_tile = bp + (size_t)b * kSlots * kLanes;

    // Steps alternate between the two LDS buffers; the loops advance two steps
    // at a time so both buffer addresses are constants.  Pass 1 keeps
    // backpointers only from step 127 on (odd), pass 2 from step 0.
    constexpr int t_first = (PASS == 1) ? 127 : 0;
    // At K = 2 the second buffer starts 64 KiB in, past the 16-bit immediate
    // offsets of the LDS instructions; with its offset opaque to the compiler
    // both buffers are addressed as one base register plus immediates
    // (ds_read2st64 / ds_write_b128), not one address register per access.
    int b1_off = (NBUF - 1) * lds_words<K, SKEW>();
    if constexpr (NBUF == 2 && lds_words<K, SKEW>() * sizeof(float) >= 65536)
        asm volatile("" : "+v"(b1_off));
    float *const B0 = Mb;
    float *const B1 = Mb + b1_off;
    float xt = xin(0);
    int t = 0;
    if constexpr (PASS == 1) {
        for (; t + 1 < t_first; t += 2) {           // steps 0..125 in pairs
            const float xn = xin(t + 1);
            trellis_step<K, false, 0, SKEW>(xt, B0, B1, lv, m, b0);
            __syncthreads();
            xt = xin(t + 2);
            trellis_step<K, false, 1, SKEW>(xn, B1, B0, lv, m, b0);
            __syncthreads();
        }
        {                                           // step 126: B0 -> B1
            const float xn = xin(t + 1);
            trellis_step<K, false, 0, SKEW>(xt, B0, B1, lv, m, b0);
            __syncthreads();
            xt = xn;
            ++t;
        }
        for (; t < kSteps - 1; t += 2) {            // steps 127..254: B1 -> B0 -> B1
            const float xn = xin(t + 1);
            uint32_t w = trellis_step<K, true, 1, SKEW>(xt, B1, B0, lv, m, b0);
            bp_tile[(size_t)(t - t_first) * kLanes + g] = (bp_t)w;
            __syncthreads();
            xt = xn;
            if (t + 1 < kSteps - 1) {
                xt = xin(t + 2);
                w = trellis_step<K, true, 0, SKEW>(xn, B0, B1, lv, m, b0);
                bp_tile[(size_t)(t + 1 - t_first) * kLanes + g] = (bp_t)w;
                __syncthreads();
            }
        }
    } else if constexpr (PASS == 3 && K == 2) {
        for (; t < kPartHead; t += 2) {             // steps 0..5: one butterfly
            const float xn = xin(t + 1);
            part_step2<false, SKEW, 0>((xm >> (10 - 2 * t)) & 3u, xt, B0, B1, lv, m);
            __syncthreads();
            xt = xin(t + 2);
            part_step2<false, SKEW, 0>((xm >> (8 - 2 * t)) & 3u, xn, B1, B0, lv, m);
            __syncthreads();
        }
        for (; t < kSteps - 1 - kPartTail; t += 2) {   // steps 6..247
            const float xn = xin(t + 1);
            trellis_step<K, false, 0, SKEW>(xt, B0, B1, lv, m, b0);
            __syncthreads();
            xt = xin(t + 2);
            trellis_step<K, false, 1, SKEW>(xn, B1, B0, lv, m, b0);
            __syncthreads();
        }
        const uint32_t Xf = X_in[b];
        for (; t < kSteps - 1; ++t) {               // steps 248..254: one position
            const int j = kSteps - 2 - t;
            const float xn = xin(t + 1);
            part_step2<false, SKEW, 1>((Xf >> (2 + 2 * j)) & 3u, xt, (t & 1) ? B1 : B0,
                                       (t & 1) ? B0 : B1, lv, m);
            __syncthreads();
            xt = xn;
        }
    } else if constexpr (PASS == 3) {
        if constexpr (skip_steps<K>() > 0)
            for (; t < skip_steps<K>(); t += 2) {   // the first steps, unreachable waves skip
                const float xn = xin(t + 1);
                trellis_step<K, false, 0, SKEW, true>(xt, B0, B1, lv, m, b0);
                __syncthreads();
                xt = xin(t + 2);
                trellis_step<K, false, 1, SKEW, true>(xn, B1, B0, lv, m, b0);
                __syncthreads();
            }
        for (; t < kSteps - 1; t += 2) {            // steps 0..254, no backpointers
            const float xn = xin(t + 1);
            trellis_step<K, false, 0, SKEW>(xt, B0, B1, lv, m, b0);
            __syncthreads();
            xt = xn;
            if (t + 1 < kSteps - 1) {
                xt = xin(t + 2);
                trellis_step<K, false, 1, SKEW>(xn, B1, B0, lv, m, b0);
                __syncthreads();
            }
        }
    } else if constexpr (K == 2) {
        for (; t < kPartHead; t += 2) {             // steps 0..5: one butterfly
            const float xn = xin(t + 1);
            uint32_t w = part_step2<true, SKEW, 0>((xm >> (10 - 2 * t)) & 3u, xt, B0, B1, lv, m);
            bp_tile[(size_t)t * kLanes + g] = (bp_t)w;
            __syncthreads();
            xt = xin(t + 2);
            w = part_step2<true, SKEW, 0>((xm >> (8 - 2 * t)) & 3u, xn, B1, B0, lv, m);
            bp_tile[(size_t)(t + 1) * kLanes + g] = (bp_t)w;
            __syncthreads();
        }
        for (; t < kSteps - 1 - kPartTail; t += 2) {   // steps 6..247: B0 -> B1 -> B0
            const float xn = xin(t + 1);
            uint32_t w = trellis_step<K, true, 0, SKEW>(xt, B0, B1, lv, m, b0);
            bp_tile[(size_t)t * kLanes + g] = (bp_t)w;
            __syncthreads();
            xt = xin(t + 2);
            w = trellis_step<K, true, 1, SKEW>(xn, B1, B0, lv, m, b0);
            bp_tile[(size_t)(t + 1) * kLanes + g] = (bp_t)w;
            __syncthreads();
        }
        const uint32_t Xf = X_in[b];
        // the backpointer address afresh (kept from before the loop it would
        // hold two registers through it)
        int gl = g;
        asm volatile("" : "+v"(gl));
        bp_t *const bp_last = bp + (size_t)b * kSlots * kLanes + gl;
        for (; t < kSteps - 1; ++t) {               // steps 248..254: one position
            const int j = kSteps - 2 - t;
            const float xn = xin(t + 1);
            const uint32_t w = part_step2<true, SKEW, 1>((Xf >> (2 + 2 * j)) & 3u, xt,
                                                         (t & 1) ? B1 : B0, (t & 1) ? B0 : B1,
                                                         lv, m);
            bp_last[(size_t)t * kLanes] = (bp_t)w;
            __syncthreads();
            xt = xn;
        }
    } else {
        if constexpr (skip_steps<K>() > 0)
            for (; t < skip_steps<K>(); t += 2) {   // the first steps, unreachable waves skip
                const float xn = xin(t + 1);
                uint32_t w = trellis_step<K, true, 0, SKEW, true>(xt, B0, B1, lv, m, b0);
                bp_tile[(size_t)t * kLanes + g] = (bp_t)w;
                __syncthreads();
                xt = xin(t + 2);
                w = trellis_step<K, true, 1, SKEW, true>(xn, B1, B0, lv, m, b0);
                bp_tile[(size_t)(t + 1) * kLanes + g] = (bp_t)w;
                __syncthreads();
            }
        for (; t < kSteps - 1; t += 2) {            // steps 0..254: B0 -> B1 -> B0
            const float xn = xin(t + 1);
            uint32_t w = trellis_step<K, true, 0, SKEW>(xt, B0, B1, lv, m, b0);
            bp_tile[(size_t)t * kLanes + g] = (bp_t)w;
            __syncthreads();
            xt = xn;
            if (t + 1 < kSteps - 1) {
                xt = xin(t + 2);
                w = trellis_step<K, true, 1, SKEW>(xn, B1, B0, lv, m, b0);
                bp_tile[(size_t)(t + 1) * kLanes + g] = (bp_t)w;
                __syncthreads();
            }
        }
    }

    // last step: costs of all states, no minimum over predecessors
    xt = xin(kSteps - 1);
    const float *Mc = ((kSteps - 1) & 1) && NBUF == 2 ? B1 : B0;
    // tracked index e of the last step's predecessors -> its LDS word (K = 1:
    // quarter Q1 sits in the slot of odd steps)
    auto slot_of = [](uint32_t e) -> uint32_t {
        if constexpr (K == 1)
            return (e >> 13) == 1u ? (uint32_t)k1_q1_slot((kSteps - 1) & 1) + (e & 8191u) : e;
        else
            return lds_word<K, SKEW>(e);
    };
    if (PASS == 1) {
        float best = 0.0f;
        uint32_t best_s = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < G::GPL; ++i)
#pragma unroll
            for (int k = 0; k < G::NB; ++k) {
                float mk = Mc[slot_of(((uint32_t)k << G::MBITS) | (uint32_t)m[i])];
#pragma unroll
                for (int bb = 0; bb < G::BPL; ++bb) {
                    float d = xt - lv.at(i, k, bb);
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
                float mk = Mc[slot_of(((uint32_t)k << G::MBITS) | (uint32_t)m[i])];
#pragma unroll
                for (int bb = 0; bb < G::BPL; ++bb) {
                    uint32_t s = ((uint32_t)k << G::Kr) | ((uint32_t)m[i] << K) | (uint32_t)(b0 + bb);
                    if (s == X) {
                        float d = xt - lv.at(i, k, bb);
                        float q = d * d;
                        cost_out[b] = mk + q;
                    }
                }
            }
    }
}

template <int K, int PASS>
hipError_t launch_fwd_t(const float *x, const int32_t *tile_idx, int64_t tile0, int64_t n,
                        const uint16_t *levels, float scale, const float *scale_dev,
                        const uint16_t *X_in, void *bp, uint16_t *end_state, float *cost_out,
                        hipStream_t stream, bool scale_per_tile) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL((viterbi_fwd_kernel<K, PASS>), dim3((unsigned)n), dim3(kLanes), 0, stream,
                       x, tile_idx, tile0, levels, scale, scale_dev, X_in,
                       reinterpret_cast<typename Geo<K>::bp_t *>(bp), end_state, cost_out,
                       scale_per_tile);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_viterbi_fwd(int K, int pass, const float *x, const int32_t *tile_idx,
                              int64_t tile0, int64_t n, const uint16_t *levels, float scale,
                              const float *scale_dev, const uint16_t *X_in, void *bp,
                              uint16_t *end_state, float *cost_out, hipStream_t stream,
                              bool scale_per_tile) {
#define EXL3_FWD_CASE(KK)                                                                    \
    case KK:                                                                                 \
        return pass == 1   ? launch_fwd_t<KK, 1>(x, tile_idx, tile0, n, levels, scale,       \
                                                  scale_dev, X_in, bp, end_state, cost_out,  \
                                                  stream, scale_per_tile)                    \
               : pass == 2 ? launch_fwd_t<KK, 2>(x, tile_idx, tile0, n, levels, scale,       \
                                                  scale_dev, X_in, bp, end_state, cost_out,  \
                                                  stream, scale_per_tile)                    \
                           : launch_fwd_t<KK, 3>(x, tile_idx, tile0, n, levels, scale,       \
                                                  scale_dev, X_in, bp, end_state, cost_out,  \
                                                  stream, scale_per_tile);
    switch (K) {
        EXL3_FWD_CASE(1)
        EXL3_FWD_CASE(2)
        EXL3_FWD_CASE(3)
        EXL3_FWD_CASE(4)
        default:
            return hipErrorInvalidValue;
    }
#undef EXL3_FWD_CASE
}

}  // namespace exl3
