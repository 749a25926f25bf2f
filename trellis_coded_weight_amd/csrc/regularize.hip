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
// Workgroups of 2B lanes, each taking B x B blocks in turn (the blocks are
// independent): coalesced 16-byte loads into LDS, each column's left transform
// split over a lane pair, the block turned around in LDS, each row's right
// transform split the same way, and a tile-major stage in LDS from which each
// of the block's (B/16)^2 tiles gets its sequential binary32 sum of squares and
// the output is written (tile-major or row-major).  HBM-bound: 6 bytes per
// element for bf16 input (2 in, 4 out).
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

// A workgroup of 2B lanes works on one B x B block at a time.  Lane l works as
// half h = (l >> 5) & 1 of index i = (l & 31) + 32 (l >> 6): in the left
// transform it holds rows
// h B/2 .. h B/2 + B/2 - 1 of column i, in the right transform columns
// h B/2 .. of row i.  The levels h < B/2 of a transform run in registers; the
// last level pairs each value with the same position of the other half, held
// by lane l ^ 32 of the same wave (exchanged with v_permlane32_swap, no LDS).
//
//   1. 16-byte loads of the block's rows (coalesced), signs applied, into LDS
//      (blk_word).  Where the block's signs are all exactly +-1 (as the header
//      requires), each product is its value with the sign bit flipped, so the
//      flips are xors of the raw words (the same result for every finite value
//      and for infinities); other sign values take the two products.  The
//      non-finite test reads the raw exponent fields;
//   2. left transform along columns, x rn(1/sqrt(B)), back to LDS;
//   3. right transform along rows, x rn(1/sqrt(B)) (row-major output written
//      from registers);
//   4. the block in trellis order into a tile-major LDS stage (tile stride
//      274 words, 17 words per tile row: conflict-free stores);
//   5. per-tile sequential sum of squares, one lane per tile, the reads of a
//      tile row in flight while the previous row is summed;
//   6. tile-major output from the stage, one wave per tile, consecutive lanes
//      on consecutive positions.
constexpr int kStageRow = 17;       // LDS words per 16-element tile row in the stage
constexpr int kStageTile = 274;     // LDS words per tile in the stage

__device__ __forceinline__ int stage_word(int t) { return (t >> 4) * kStageRow + (t & 15); }

// The last butterfly level, across the two halves of the wave, for two values
// x, y of every lane (rows or columns r and r + 1 of the lane's half; the pair
// of x in lane t < 32 is x in lane t + 32).  v_permlane32_swap(x, y) swaps the
// upper 32 lanes of x with the lower 32 lanes of y, which gives lane t < 32
// both members (top, bottom) of pair r and lane t + 32 both members of pair
// r + 1; each lane forms top + bottom and top - bottom (one rounding each), and
// a swap of those returns the sums to the top lanes and the differences to the
// bottom lanes, in x (pair r) and y (pair r + 1): 4 instructions per two
// values.
__device__ __forceinline__ void last_level2(float &x, float &y) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y),
                                                    false, false);
    const float top = __uint_as_float(p[0]), bot = __uint_as_float(p[1]);
    const float sum = top + bot, dif = top - bot;
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(dif),
                                                    false, false);
    x = __uint_as_float(q[0]);
    y = __uint_as_float(q[1]);
}

// LDS word of block element (row, col): an odd row pitch P and S words of pad
// after every 32 columns (S = 2 for bf16 input, 1 for fp32).  The transforms'
// accesses (32 lanes on 32 consecutive columns of one row, or on one column of
// 32 consecutive rows) hit 32 distinct banks for any odd P; at B = 128 the
// first phase's stores (EPC consecutive columns per lane, lanes on consecutive
// 16-byte chunks) do too with the pad, which moves every fourth (bf16) or
// eighth (fp32) chunk to the next bank group (at B = 64, bf16, they meet two
// to a bank).
template <int B, typename Tin>
struct BlkPad {
    static constexpr int S = sizeof(Tin) == 2 ? 2 : 1;      // words of pad per 32 columns
    static constexpr int P0 = B + S * (B / 32 - 1);
    static constexpr int P = P0 | 1;                         // odd row pitch
};
template <int B, typename Tin>
__device__ __forceinline__ int blk_word(int row, int col) {
    return row * BlkPad<B, Tin>::P + col + BlkPad<B, Tin>::S * (col >> 5);
}
template <int B, typename Tin>
constexpr int blk_words() { return B * BlkPad<B, Tin>::P; }

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
// Workgroup g takes the blocks g, g + G, g + 2G, ... (G workgroups, as many as
// are resident at once; blocks in row-major order).  When a lane's 16-byte
// loads of a block fit in 32 registers, the next block's are issued as soon as
// the current block is in LDS, and arrive while it is transformed.
template <int B, typename Tin, bool VEC, bool ORDERED>
__global__ void __launch_bounds__(2 * B)
regularize_kernel(const Tin *__restrict__ w, int rows, int cols, const float *__restrict__ su,
                  const float *__restrict__ sv, float *__restrict__ out, int layout,
                  float *__restrict__ tile_sumsq, int *__restrict__ nonfinite,
                  const uint8_t *__restrict__ order) {
    constexpr int H = B / 2;          // values per lane in a transform
    constexpr int TB = B / 16;        // tiles per block side
    constexpr int kWords = blk_words<B, Tin>() > TB * TB * kStageTile ? blk_words<B, Tin>()
                                                                       : TB * TB * kStageTile;
    constexpr int EPC = 16 / sizeof(Tin);       // elements per 16-byte load
    constexpr int CPR = B / EPC;                // loads per block row
    constexpr int NL = B * CPR / (2 * B);       // loads per lane
    constexpr bool kAhead = VEC && NL <= 8;     // the next block's loads issued early
    __shared__ float smem[kWords];
    __shared__ float sgn[2 * B];      // the block's column signs, then its row signs
    __shared__ uint8_t inv[256];      // element -> trellis position (ORDERED)
    __shared__ bool other_sign[2 * B / 64];   // per wave: a staged sign other than +-1
    const int l0 = threadIdx.x;
    const int TC = cols / 16, nbx = cols / B;
    const int nblk = nbx * (rows / B);
    const float c = norm_const<B>();
    if constexpr (ORDERED)
        for (int t = l0; t < 256; t += 2 * B) inv[order[t]] = (uint8_t)t;

    // the lane's 16-byte loads of a block: rows (l + 2B i) / CPR, i < NL, and
    // the same EPC columns cb .. cb + EPC - 1 for every i
    uint4 u[NL];
    float sgv = 0.0f;                 // the lane's sign of the fetched block, loaded with it
    auto fetch = [&](int blk) {
        const int r0 = (blk / nbx) * B, c0 = (blk % nbx) * B, cb = (l0 % CPR) * EPC;
        sgv = l0 < B ? sv[c0 + l0] : su[r0 + l0 - B];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int rr = (l0 + 2 * B * i) / CPR;
            u[i] = *reinterpret_cast<const uint4 *>(w + (size_t)(r0 + rr) * cols + c0 + cb);
        }
    };
    int blk = blockIdx.x;
    if constexpr (kAhead)
        if (blk < nblk) fetch(blk);

    // non-finite input: an exponent field of all ones; with 16-byte loads the
    // largest exponent field of each half-word (bf16) or word (fp32) is kept
    constexpr uint32_t kExp = EPC == 8 ? 0x7F807F80u : 0x7F800000u;
    using u16x2 = unsigned short __attribute__((ext_vector_type(2)));
    u16x2 emax = {0, 0};
    uint32_t emax32 = 0;
    auto track = [&](const uint4 &x) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t wk = (&x.x)[k] & kExp;
            if constexpr (EPC == 8)
                emax = __builtin_elementwise_max(emax, __builtin_bit_cast(u16x2, wk));
            else
                emax32 = emax32 > wk ? emax32 : wk;
        }
    };
    bool bad = false;

    for (; blk < nblk; blk += gridDim.x) {
        // the lane index, opaque to the compiler once per block, so that the LDS
        // addresses derived from it are formed inside the loop instead of being
        // held in registers across it
        int l = l0;
        asm volatile("" : "+v"(l));
        const int idx = (l & 31) + 32 * (l >> 6), half = (l >> 5) & 1;
        const int cb = (l % CPR) * EPC;
        const int r0 = (blk / nbx) * B, c0 = (blk % nbx) * B;
        if constexpr (VEC && !kAhead) fetch(blk);

        // each lane stages one sign; a wave flag records a sign other than +-1
        float sg;
        if constexpr (VEC) sg = sgv;
        else sg = l < B ? sv[c0 + l] : su[r0 + l - B];
        sgn[l] = sg;
        const bool wave_other = __ballot((__float_as_uint(sg) & 0x7FFFFFFFu) != 0x3F800000u) != 0;
        if ((l & 63) == 0) other_sign[l >> 6] = wave_other;
        __syncthreads();              // signs in; the previous block's stage is read

        // 1. signs (exact), into LDS
        if constexpr (VEC) {
            // where every sign of the block is exactly +-1, each product is its
            // value with the sign bit flipped: xors of the raw words; other sign
            // values take the products
            bool pm1 = true;
#pragma unroll
            for (int k = 0; k < 2 * B / 64; ++k) pm1 = pm1 && !other_sign[k];
            if (pm1) {
                uint32_t cm[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    cm[k] = EPC == 8 ? ((__float_as_uint(sgn[cb + 2 * k]) >> 16) & 0x8000u) |
                                           (__float_as_uint(sgn[cb + 2 * k + 1]) & 0x80000000u)
                                     : __float_as_uint(sgn[cb + k]) & 0x80000000u;
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    const int rr = (l + 2 * B * i) / CPR;
                    uint32_t rm = __float_as_uint(sgn[B + rr]) & 0x80000000u;
                    if (EPC == 8) rm |= rm >> 16;
                    track(u[i]);
                    const uint4 x = make_uint4(u[i].x ^ cm[0] ^ rm, u[i].y ^ cm[1] ^ rm,
                                               u[i].z ^ cm[2] ^ rm, u[i].w ^ cm[3] ^ rm);
                    float v[EPC];
                    unpack16<Tin>(x, v);
#pragma unroll
                    for (int e = 0; e < EPC; ++e) smem[blk_word<B, Tin>(rr, cb + e)] = v[e];
                }
            } else {
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    const int rr = (l + 2 * B * i) / CPR;
                    track(u[i]);
                    float v[EPC];
                    unpack16<Tin>(u[i], v);
                    const float sr = sgn[B + rr];
#pragma unroll
                    for (int e = 0; e < EPC; ++e)
                        smem[blk_word<B, Tin>(rr, cb + e)] = (v[e] * sr) * sgn[cb + e];
                }
            }
        } else {
            for (int q = l; q < B * B; q += 2 * B) {
                const int rr = q / B, cc = q % B;
                const float v = load_w(w, (size_t)(r0 + rr) * cols + c0 + cc);
                bad |= !isfinite(v);
                smem[blk_word<B, Tin>(rr, cc)] = (v * sgn[B + rr]) * sgn[cc];
            }
        }
        __syncthreads();
        if constexpr (kAhead)
            if (blk + (int)gridDim.x < nblk) fetch(blk + gridDim.x);

        // 2. left transform: column idx, rows half * H ..
        float a[H];
#pragma unroll
        for (int r = 0; r < H; ++r) a[r] = smem[blk_word<B, Tin>(half * H + r, idx)];
        fwht_regs<H>(a);
#pragma unroll
        for (int r = 0; r < H; r += 2) last_level2(a[r], a[r + 1]);
#pragma unroll
        for (int r = 0; r < H; ++r) smem[blk_word<B, Tin>(half * H + r, idx)] = a[r] * c;
        __syncthreads();

        // 3. right transform: row idx, columns half * H ..
#pragma unroll
        for (int q = 0; q < H; ++q) a[q] = smem[blk_word<B, Tin>(idx, half * H + q)];
        fwht_regs<H>(a);
#pragma unroll
        for (int q = 0; q < H; q += 2) last_level2(a[q], a[q + 1]);
#pragma unroll
        for (int q = 0; q < H; ++q) a[q] = a[q] * c;
        if (layout != 1) {
            // row-major output through LDS: each lane puts back the words it
            // alone read above (no barrier needed before), then consecutive
            // lanes store consecutive 16-byte pieces of a row, so that a wave's
            // store covers whole lines and can stream past the caches
#pragma unroll
            for (int q = 0; q < H; ++q) smem[blk_word<B, Tin>(idx, half * H + q)] = a[q];
            __syncthreads();
            for (int g = l; g < B * B / 4; g += 2 * B) {
                const int row = g / (B / 4), cq = 4 * (g % (B / 4));
                store_stream(out + (size_t)(r0 + row) * cols + c0 + cq,
                             smem[blk_word<B, Tin>(row, cq)], smem[blk_word<B, Tin>(row, cq + 1)],
                             smem[blk_word<B, Tin>(row, cq + 2)],
                             smem[blk_word<B, Tin>(row, cq + 3)]);
            }
        }
        if (layout != 1 && !tile_sumsq) continue;
        __syncthreads();              // the block in LDS is read; the stage reuses it

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

        if (tile_sumsq && l < 64) {
            // 5. per-tile sequential binary32 sum of squares, trellis order: wave
            // 0, one lane per tile, tile rows double-buffered (the reads of row
            // k + 1 in flight while row k is summed)
            if (l < TB * TB) {
                const float *T = smem + l * kStageTile;
                float acc = 0.0f;
                float buf[2][16];
#pragma unroll
                for (int j = 0; j < 16; ++j) buf[0][j] = T[j];
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    if (k + 1 < 16)
#pragma unroll
                        for (int j = 0; j < 16; ++j)
                            buf[(k + 1) & 1][j] = T[(k + 1) * kStageRow + j];
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const float sq = buf[k & 1][j] * buf[k & 1][j];
                        acc = acc + sq;
                    }
                }
                tile_sumsq[(size_t)(r0 / 16 + l / TB) * TC + (c0 / 16 + l % TB)] = acc;
            }
        } else if (layout == 1) {
            // 6. tile-major output (the other waves, or all of them without
            // energies), whole tiles per wave: tile lt is one float4 per lane
            // (positions 4 lane .. 4 lane + 3), the wave's store its 1 KiB; eight
            // tiles' reads are issued ahead, and the tile bound is wave-uniform
            const int first = tile_sumsq ? 1 : 0;
            const int nw = 2 * B / 64 - first, wv = (l >> 6) - first, t = 4 * (l & 63);
            for (int lt0 = wv; lt0 < TB * TB; lt0 += 8 * nw) {
                float4 v[8];
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    const int lt = lt0 + b * nw;
                    if (lt < TB * TB) {
                        const float *T = smem + lt * kStageTile;
                        v[b] = make_float4(T[stage_word(t)], T[stage_word(t + 1)],
                                           T[stage_word(t + 2)], T[stage_word(t + 3)]);
                    }
                }
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    const int lt = lt0 + b * nw;
                    if (lt < TB * TB) {
                        const size_t tau =
                            (size_t)(r0 / 16 + lt / TB) * TC + (c0 / 16 + lt % TB);
                        store_stream(out + tau * 256 + t, v[b].x, v[b].y, v[b].z, v[b].w);
                    }
                }
            }
        }
    }
    if constexpr (VEC) {
        if constexpr (EPC == 8)
            bad = emax.x == 0x7F80u || emax.y == 0x7F80u;
        else
            bad = emax32 == kExp;
    }
    if (bad && nonfinite) *nonfinite = 1;
}

// Inverse of the regularization (H is symmetric and orthonormal, so its own
// inverse): W = diag(su) H_l W_reg H_r diag(sv), evaluated as left transform,
// x rn(1/sqrt(B)), right transform, x rn(1/sqrt(B)), then x su[row], x sv[col]
// (su, sv may be the folded channel scales, not only +-1).  Input tile-major
// or row-major, output row-major.  One workgroup of 2B lanes per block, laid
// out as in the forward kernel: the block in LDS (16-byte loads of tiles or
// rows), each column's transform over a lane pair (the last level by lane
// swaps), each row's the same way, the scaled block back into LDS, and the
// row-major output with consecutive lanes on consecutive 16-byte pieces.
// VEC: input and output start on 16-byte boundaries (else one element per
// access).
template <int B, bool VEC>
__global__ void __launch_bounds__(2 * B)
unregularize_kernel(const float *__restrict__ in, int rows, int cols, int in_layout,
                    const float *__restrict__ su, const float *__restrict__ sv,
                    float *__restrict__ out, const uint8_t *__restrict__ order) {
    constexpr int H = B / 2;
    constexpr int TB = B / 16;
    __shared__ float smem[blk_words<B, float>()];
    __shared__ float srow[B], scol[B];
    __shared__ uint8_t ord[256];      // the within-tile order (tile-major input with one)
    const int l = threadIdx.x;
    const int r0 = blockIdx.y * B, c0 = blockIdx.x * B;
    const int TC = cols / 16;
    const float c = norm_const<B>();
    const int idx = (l & 31) + 32 * (l >> 6), half = (l >> 5) & 1;
    if (l < B) scol[l] = sv[c0 + l];
    else srow[l - B] = su[r0 + l - B];
    const bool ordered = in_layout == 1 && order;
    if (ordered) {
        for (int t = l; t < 256; t += 2 * B) ord[t] = order[t];
        __syncthreads();
    }

    // 1. the block into LDS
    if (in_layout == 1) {
        // tile lt = (tr, tc) of the block: positions 4 q .. 4 q + 3 per access
        for (int g = l; g < B * B / 4; g += 2 * B) {
            const int lt = g >> 6, q = g & 63, tr = lt / TB, tc = lt % TB;
            const size_t tau = (size_t)(r0 / 16 + tr) * TC + (c0 / 16 + tc);
            float v[4];
            if constexpr (VEC) {
                const float4 x = *reinterpret_cast<const float4 *>(in + tau * 256 + 4 * q);
                v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = in[tau * 256 + 4 * q + e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * q + e, el = ordered ? ord[t] : t;
                smem[blk_word<B, float>(16 * tr + (el >> 4), 16 * tc + (el & 15))] = v[e];
            }
        }
    } else {
        for (int g = l; g < B * B / 4; g += 2 * B) {
            const int row = g / (B / 4), cq = 4 * (g % (B / 4));
            const float *src = in + (size_t)(r0 + row) * cols + c0 + cq;
            float v[4];
            if constexpr (VEC) {
                const float4 x = *reinterpret_cast<const float4 *>(src);
                v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = src[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) smem[blk_word<B, float>(row, cq + e)] = v[e];
        }
    }
    __syncthreads();

    // 2. left transform: column idx, rows half * H ..
    float a[H];
#pragma unroll
    for (int r = 0; r < H; ++r) a[r] = smem[blk_word<B, float>(half * H + r, idx)];
    fwht_regs<H>(a);
#pragma unroll
    for (int r = 0; r < H; r += 2) last_level2(a[r], a[r + 1]);
#pragma unroll
    for (int r = 0; r < H; ++r) smem[blk_word<B, float>(half * H + r, idx)] = a[r] * c;
    __syncthreads();

    // 3. right transform: row idx, columns half * H .., then the row and
    // column factors, back into LDS
#pragma unroll
    for (int q = 0; q < H; ++q) a[q] = smem[blk_word<B, float>(idx, half * H + q)];
    fwht_regs<H>(a);
#pragma unroll
    for (int q = 0; q < H; q += 2) last_level2(a[q], a[q + 1]);
    const float fr = srow[idx];
#pragma unroll
    for (int q = 0; q < H; ++q)
        smem[blk_word<B, float>(idx, half * H + q)] = ((a[q] * c) * fr) * scol[half * H + q];
    __syncthreads();

    // 4. row-major output
    for (int g = l; g < B * B / 4; g += 2 * B) {
        const int row = g / (B / 4), cq = 4 * (g % (B / 4));
        float *dst = out + (size_t)(r0 + row) * cols + c0 + cq;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = smem[blk_word<B, float>(row, cq + e)];
        if constexpr (VEC) {
            store_stream(dst, v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e] = v[e];
        }
    }
}

// Workgroups of one instantiation resident per compute unit (queried once).
template <typename Kernel>
int groups_per_cu(Kernel kernel, int threads) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess)
        n = 0;
    return n > 0 ? n : 1;
}

template <int B, typename Tin>
hipError_t launch_reg_t(const void *w, int rows, int cols, const float *su, const float *sv,
                        float *out, int layout, float *tile_sumsq, int *nonfinite,
                        const uint8_t *order, int n_cu, hipStream_t stream) {
    const int nblk = (cols / B) * (rows / B);
    const Tin *wt = reinterpret_cast<const Tin *>(w);
    const bool vec = reinterpret_cast<uintptr_t>(w) % 16 == 0;
#define EXL3_REG_LAUNCH(V, O)                                                                  \
    do {                                                                                       \
        static const int per_cu = groups_per_cu(regularize_kernel<B, Tin, V, O>, 2 * B);       \
        const int groups = nblk < per_cu * n_cu ? nblk : per_cu * n_cu;                        \
        hipLaunchKernelGGL((regularize_kernel<B, Tin, V, O>), dim3((unsigned)groups),          \
                           dim3(2 * B), 0, stream, wt, rows, cols, su, sv, out, layout,        \
                           tile_sumsq, nonfinite, order);                                      \
    } while (0)
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
    const bool vec = reinterpret_cast<uintptr_t>(in) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(out) % 16 == 0;
#define EXL3_UNREG_LAUNCH(BB, V)                                                                \
    hipLaunchKernelGGL((unregularize_kernel<BB, V>), grid, dim3(2 * BB), 0, stream, in, rows,  \
                       cols, in_layout, su, sv, out, order)
    if (had_block == 64) {
        if (vec) EXL3_UNREG_LAUNCH(64, true);
        else EXL3_UNREG_LAUNCH(64, false);
    } else {
        if (vec) EXL3_UNREG_LAUNCH(128, true);
        else EXL3_UNREG_LAUNCH(128, false);
    }
#undef EXL3_UNREG_LAUNCH
    return hipGetLastError();
}

hipError_t launch_regularize(const void *w, int w_dtype, int rows, int cols, int had_block,
                             const float *su, const float *sv, float *out, int layout,
                             float *tile_sumsq, int *nonfinite, const uint8_t *order, int n_cu,
                             hipStream_t stream) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    if (n_cu < 1) n_cu = 1;
    if (had_block == 64)
        return w_dtype == 1
                   ? launch_reg_t<64, uint16_t>(w, rows, cols, su, sv, out, layout, tile_sumsq,
                                                nonfinite, order, n_cu, stream)
                   : launch_reg_t<64, float>(w, rows, cols, su, sv, out, layout, tile_sumsq,
                                             nonfinite, order, n_cu, stream);
    if (had_block == 128)
        return w_dtype == 1
                   ? launch_reg_t<128, uint16_t>(w, rows, cols, su, sv, out, layout, tile_sumsq,
                                                 nonfinite, order, n_cu, stream)
                   : launch_reg_t<128, float>(w, rows, cols, su, sv, out, layout, tile_sumsq,
                                              nonfinite, order, n_cu, stream);
    return hipErrorInvalidValue;
}

}  // namespace exl3
