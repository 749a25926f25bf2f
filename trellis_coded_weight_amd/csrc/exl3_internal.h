// Internal declarations of the gfx950 EXL3 encoder library (not part of the ABI).
//
// Trellis algebra ("EXL3 Intel Arc Quantizer" README, Core Implemented
// Architecture section 4): a 16-bit state shifts K new bits in at the bottom,
// S_t = ((S_{t-1} << K) | b_t) & 0xFFFF.  Kr = 16 - K.  The search keeps one
// running minimum per value e of the low Kr bits (2^Kr "tracked" minima); the
// full states that can precede a state whose top Kr bits are e are
// (k << Kr) | e, k = 0 .. 2^K - 1.
//
// Work split of the forward kernel.  The 2^16 states of a step fall into
// radix-2^K butterflies: for m in [0, 2^(16-2K)) the states
//   sigma(k, m, b) = (k << Kr) | (m << K) | b,   k, b in [0, 2^K)
// read the tracked minima M[(k << (16-2K)) | m] and, after the minimum over k,
// write the new minima M'[(m << K) | b].  A workgroup of 1024 lanes owns one
// tile; every lane owns 64 states for the whole pass, so their levels
// v = rn(scale * c) stay in registers:
//   K=1: 16384 butterflies of 4 states; lane g owns m = g + 1024*i, i < 16
//   K=2: 4096 butterflies of 16 states; lane g owns m = g + 1024*i, i < 4
//   K=3: 1024 butterflies of 64 states; lane g owns m = g
//   K=4:  256 butterflies of 256 states; lane g owns m = g >> 2 and the four
//         values b = 4*(g & 3) + 0..3
// Backpointers (the winning k of every tracked state, K bits) are packed per
// lane per step into one word: 32 bits at K=1 and 2, 24 at K=3 (uint32), 16
// at K=4 (uint16).  The lane appends its tracked states in the order
// n = i * BPL + bb, high bit first (at K = 1 with i = 4..7 before 0..3), so
// state n's k sits at bit K * (GPL * BPL - 1 - n).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exl3 {

constexpr int kLanes = 1024;        // lanes per tile workgroup
constexpr int kSteps = 256;         // trellis steps per tile (16 x 16 weights)
constexpr int kSlots = kSteps - 1;  // steps that produce backpointers

template <int K>
struct Geo {
    static constexpr int Kr = 16 - K;
    static constexpr int T = 1 << Kr;             // tracked minima
    static constexpr int NB = 1 << K;             // branches per tracked state
    static constexpr int MBITS = 16 - 2 * K;      // butterfly index bits
    static constexpr int GPL = (K == 1) ? 16 : (K == 2) ? 4 : 1;  // butterflies per lane
    static constexpr int BPL = (K == 4) ? 4 : NB; // b values per lane per butterfly
    static constexpr int SPL = GPL * NB * BPL;    // states per lane (64)
    using bp_t = typename std::conditional<(K == 4), uint16_t, uint32_t>::type;
    static_assert(SPL == 64, "every lane owns 64 states");
};

// Lane and bit of tracked state e's backpointer inside a step's row of words.
template <int K>
__host__ __device__ inline void bp_locate(uint32_t e, uint32_t &lane, uint32_t &bit) {
    if (K <= 2) {
        constexpr uint32_t bpl = 1u << K, n_e = 32u / K;
        uint32_t m = e >> K, bb = e & (bpl - 1u);
        uint32_t i = m >> 10;
        if (K == 1 && i < 8u) i ^= 4u;   // K = 1 runs butterflies 4..7 first
        lane = m & 1023u;
        bit = K * (n_e - 1u - (bpl * i + bb));
    } else if (K == 3) {
        lane = e >> 3;
        bit = 3u * (7u - (e & 7u));
    } else {
        uint32_t m = e >> 4, b = e & 15u;
        lane = (m << 2) | (b >> 2);
        bit = 4u * (3u - (b & 3u));
    }
}

// Binary16 mode of the forward kernel.  Costs, levels and inputs are IEEE
// binary16; two tracked states share one 32-bit register (low and high half),
// paired as outputs b and b + 1 of one butterfly, so a packed instruction
// serves both.  Ownership (1024 lanes and 64 states per lane at K = 1..3; 512
// lanes and 128 states per lane at K = 4, so that two tiles share a compute
// unit):
//   K=1: lane g owns the butterflies m = 2g + j + 2048 i (i < 8, j < 2)
//   K=2: lane g owns the butterflies m = 2g + j + 2048 i (i, j < 2)
//   K=3: m = g
//   K=4: m = g >> 1 and the outputs b = 8 (g & 1) + 0..7
// The lane's output pairs are numbered q in loop order (i, j, pair p).  Index
// bit r of pair q, half h, comes out as a flag; the step word keeps flags in
// byte-bit positions:
//   K=1: bit 16 (q & 1) + 8h + (q >> 1)
//   K=2: bit 8h + q (r=0), 16 + 8h + q (r=1)
//   K=3: bit 8h + q (r=0), 16 + 8h + q (r=1), 8h + 16 (q & 1) + 4 + (q >> 1) (r=2)
//   K=4: 8h + 2q (r=0), 16 + 8h + 2q (r=1), 8h + 2q + 1 (r=2), 16 + 8h + 2q + 1 (r=3)
template <int K>
struct GeoH {
    static constexpr int Kr = 16 - K;
    static constexpr int T = 1 << Kr;
    static constexpr int NB = 1 << K;
    static constexpr int MBITS = 16 - 2 * K;
    static constexpr int LANES = (K == 4) ? 512 : kLanes;     // lanes per tile
    static constexpr int NI = (K == 1) ? 8 : (K == 2) ? 2 : 1;  // butterfly groups per lane
    static constexpr int NJ = (K <= 2) ? 2 : 1;       // adjacent butterflies per group
    static constexpr int NP = (K == 4) ? 4 : NB / 2;  // output pairs per butterfly and lane
    using bp_t = uint32_t;                            // one word per lane and step
    static_assert(NI * NJ * NP * 2 * NB * LANES == 65536, "the lanes own every state");
};

// Lane and bit positions (index bit 0 first) of tracked state e's
// backpointer in a step's row of words of the binary16 kernel.
template <int K>
__host__ __device__ inline void bp_locate_h(uint32_t e, uint32_t &lane, uint32_t (&bit)[K]) {
    if (K == 1) {
        uint32_t m = e >> 1, h = e & 1u;
        uint32_t q = (m >> 11) * 2u + (m & 1u);
        lane = (m & 2047u) >> 1;
        bit[0] = 16u * (q & 1u) + 8u * h + (q >> 1);
    } else if (K == 2) {
        uint32_t m = e >> 2, b = e & 3u, h = b & 1u;
        uint32_t q = ((m >> 11) * 2u + (m & 1u)) * 2u + (b >> 1);
        lane = (m & 2047u) >> 1;
        bit[0] = 8u * h + q;
        bit[1 % K] = 16u + 8u * h + q;
    } else if (K == 3) {
        uint32_t b = e & 7u, h = b & 1u, q = b >> 1;
        lane = e >> 3;
        bit[0] = 8u * h + q;
        bit[1 % K] = 16u + 8u * h + q;
        bit[2 % K] = 8u * h + 16u * (q & 1u) + 4u + (q >> 1);
    } else {
        uint32_t m = e >> 4, b = e & 15u, bl = b & 7u, h = bl & 1u, q = bl >> 1;
        lane = (m << 1) | (b >> 3);
        bit[0] = 8u * h + 2u * q;
        bit[1 % K] = 16u + 8u * h + 2u * q;
        bit[2 % K] = 8u * h + 2u * q + 1u;
        bit[3 % K] = 16u + 8u * h + 2u * q + 1u;
    }
}

// A 16-byte store (p 16-byte aligned) that does not allocate in the caches:
// for output streams written once, and read, if at all, by a later launch
// from HBM anyway (no cache holds a whole matrix).  Only where a wave's store
// instruction writes whole lines (consecutive lanes on consecutive 16-byte
// pieces): pieces at a stride then reach memory unmerged, several times
// slower than plain stores.
__device__ __forceinline__ void store_stream(float *p, float a, float b, float c, float d) {
    using f4v = float __attribute__((ext_vector_type(4)));
    const f4v v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<f4v *>(p));
}

// Bytes of backpointer scratch per tile in flight.
inline size_t bp_bytes_per_tile(int K) {
    return (size_t)kSlots * kLanes * (K == 4 ? 2 : 4);
}

// ---- kernel launchers (defined in the .hip files) ----
// pass: 1 (rotated, free start, backpointers 127..254, end state), 2 (start
// pinned to X, backpointers 0..254, path cost) or 3 (as 2, path cost only).
// scale_dev: when not null, the levels are scaled by the binary32 value it
// points to (read when the launch runs) instead of `scale`; with
// scale_per_tile, tile b of the launch takes scale_dev[b].
hipError_t launch_viterbi_fwd(int K, int pass, const float *x, const int32_t *tile_idx,
                              int64_t tile0, int64_t n, const uint16_t *levels, float scale,
                              const float *scale_dev, const uint16_t *X_in, void *bp,
                              uint16_t *end_state, float *cost_out, hipStream_t stream,
                              bool scale_per_tile = false);

hipError_t launch_viterbi_fwd_f16(int K, int pass, const uint16_t *x, int64_t tile0, int64_t n,
                                  const uint16_t *levels, const uint16_t *X_in, void *bp,
                                  uint16_t *end_state, uint16_t *cost_out, hipStream_t stream);

// f16 selects the binary16 kernel's backpointer layout; x, sse and w_hat are
// then unused (the path cost comes from the forward pass).
hipError_t launch_traceback(int K, int pass, bool f16, const void *bp, int64_t n,
                            const uint16_t *start_state, uint16_t *X_out, const float *x,
                            const int32_t *tile_idx, int64_t tile0, const uint16_t *levels,
                            float scale, uint16_t *packed, uint16_t *states, float *sse,
                            float *w_hat, hipStream_t stream);

// inv: inverse of the within-tile order (element -> position), or null.
hipError_t launch_ldlq_target(const float *w_tiles, const float *e_tiles, const float *L, int TR,
                              int TC, int j, const uint8_t *inv, float *target,
                              hipStream_t stream);

hipError_t launch_ldlq_commit(const float *w_tiles, const float *what_span,
                              const uint16_t *packed_span, int TR, int TC, int j, int K,
                              uint16_t *packed, float *e_tiles, float *w_hat, float *tile_err,
                              hipStream_t stream);

// order: the within-tile order (position -> element) of tile-major arrays, or
// null for the natural order.  n_cu: compute units of the device (the grid is
// the workgroups resident at once, each taking blocks in turn).
hipError_t launch_regularize(const void *w, int w_dtype, int rows, int cols, int had_block,
                             const float *su, const float *sv, float *out, int layout,
                             float *tile_sumsq, int *nonfinite, const uint8_t *order,
                             int n_cu, hipStream_t stream);

hipError_t launch_unregularize(const float *in, int in_layout, int rows, int cols, int had_block,
                               const float *su, const float *sv, float *out,
                               const uint8_t *order, hipStream_t stream);

hipError_t launch_channel_normalize(const void *w, int w_dtype, int rows, int cols,
                                    const float *su, double floor_value, float *w_norm,
                                    float *su_folded, double *row_rms, hipStream_t stream);

// levels: the device level table (16-byte aligned); n_cu: compute units of
// the device (one workgroup each at most, decoding tiles in turn).
hipError_t launch_decode(const uint16_t *packed, int64_t n, int K, float scale,
                         const uint16_t *levels, float *out, int n_cu, hipStream_t stream);

hipError_t launch_to_f16(const float *src, const int32_t *idx, int64_t n, float scale,
                         uint16_t *dst, hipStream_t stream);

hipError_t launch_gather_tiles(const float *src, const int32_t *idx, int64_t n, float *dst,
                               hipStream_t stream);

// Host-side generators of the level tables (fp16 bit patterns).
void build_mul1_levels(uint16_t *out65536);
void build_mcg_levels(uint16_t *out65536);
void build_3inst_levels(uint16_t *out65536);

}  // namespace exl3
