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
// Three forms, one workgroup per band of rows each: the general one (16 rows,
// any shape) adds a row's squares one at a time in column order, a chain of
// `cols` dependent binary64 additions; the chunked one (4 rows, rows of whole
// 16-byte blocks) adds a group of squares at a time where that is provably
// exact (see below); both then sweep the band again for the scaled rows.  The
// resident-row one (bf16 rows of up to 16 chunks) keeps each row in its wave's
// registers, so it reads the input once, and tests a row's groups in parallel.
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


// Exact shortcut for the row sums.  The squares are exact binary64 values and
// the running sum a is non-negative, so when a and the squares of a block are
// all integer multiples of one power of two u and the exact total
// A = a + s_1 + ... + s_n is below 2^53 u, every partial sum is a multiple of u
// below 2^53 u, hence representable: none of the n additions rounds, and
// a + (s_1 + ... + s_n), with the block's squares summed in any order, is the
// sequential result bit for bit.  Rounding is monotone and 2^53 u is
// representable, so a computed total below 2^53 u implies the exact one is too
// (if some partial sum reached 2^53 u, so would every later computed sum).
// For u the row's lane keeps a lower bound g on the lowest set bit of a: the
// minimum of the lowest set bits of the squares taken since the last block
// that was added one square at a time (a is an exact sum from there on), and
// that block's result's unit in the last place (every binary64 value is a
// multiple of it).  The test is then A < 2^53 min(g, lowest set bit of the
// block's squares).  It is taken for groups of eight blocks at once, with the
// group's squares summed in a tree: every computed partial sum of non-negative
// values is at most the computed total (rounding is monotone), so a total below
// 2^53 u, u now the smallest of the group's and g, again makes every addition
// of the tree exact.  A group that fails is taken again block by block in
// column order; blocks that fail, and blocks with a NaN or infinity (bound 0),
// are added one square at a time.
constexpr int kBig = 1 << 20;          // "no set bit" (a zero)

// 2^(53 + 2 m): the shortcut's bound for squares of values whose lowest set
// bit is at least 2^m; m = kBig (all zero) gives +inf, m = -kBig (a NaN or
// infinity) 0
__device__ __forceinline__ double square_bound(int m) {
    return m == kBig ? (double)INFINITY : m == -kBig ? 0.0 : ldexp(1.0, 53 + 2 * m);
}

// 2^(floor(log2(a)) + 1) for a > 0 (binary64): 2^53 times the unit in the last
// place of a normal a; for a subnormal one at most 2^53 times 2^-1074 (a
// smaller bound than needed, so only stricter)
__device__ __forceinline__ double next_binade(double a) {
    const uint64_t bits = (uint64_t)__double_as_longlong(a);
    const int ex = (int)((bits >> 52) & 0x7FFu);
    const uint64_t mant = bits & 0xFFFFFFFFFFFFFull;
    const int lg = ex ? ex - 1023 : 63 - (int)__builtin_clzll(mant | 1ull) - 1074;
    return ldexp(1.0, lg + 1);
}

// The fast form for rows of whole 16-byte groups (cols * sizeof(Tin) and the
// output row a multiple of 16 bytes, both arrays 16-byte aligned).  Workgroup
// of 256 lanes per band of 4 rows (four workgroups share a compute unit, which
// hides each one's latencies).  All lanes load the band in chunks of
// kChunkBlocks 16-byte blocks per row, one block per lane, keeping kFifo
// chunks of loads in flight in registers (every lane issues every load, from a
// clamped address where it has none, so that the compiler's waits for them
// count exactly); for each block they store into a two-slot LDS ring the sum
// of its squares, the bound of the shortcut above and its raw bits, and per
// group of eight blocks (eight neighbouring lanes, reduced with lane shuffles)
// the sum of their sums and the smallest of their bounds.  The lowest set bit
// of a value is bounded below from its exponent alone (2^(E - p + 1) for p
// significant bits), looser than the bit itself but one comparison per value.
// The kernel's time (4096 x 4096 bf16: 33 us against 49 us for one addition
// per square) is now the VALU work of these summaries and the per-chunk
// barriers, not the additions.  Wave 0's lanes 0..3 also own the band's rows and take
// the groups in column order: one dependent addition and one test per group
// when it passes, block by block (and a failing block's squares one by one)
// when not.  Then all lanes read the band again with 16-byte loads and write
// the scaled rows with 16-byte stores.
constexpr int kFastRows = 4;                   // rows per band of the fast form
constexpr int kChunkBlocks = 64;               // 16-byte blocks per row per chunk
constexpr int kFifo = 4;                       // chunks of loads in flight per lane
constexpr int kFastLanes = 256;                // lanes of the workgroup
constexpr int kRingStride = kChunkBlocks + 1;
constexpr int kGroup = 8;                      // blocks per shortcut group
constexpr int kGroupStride = kChunkBlocks / kGroup + 1;
static_assert(kFastRows * kChunkBlocks == kFastLanes, "one block per lane per chunk");

template <typename Tin>
__device__ __forceinline__ void unpack_block(const uint4 &u, float (&v)[16 / sizeof(Tin)]) {
    const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
    if constexpr (sizeof(Tin) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(wd[e] << 16);             // bf16 -> fp32 is exact
            v[2 * e + 1] = __uint_as_float(wd[e] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(wd[e]);
    }
}

// The shortcut's inputs for one 16-byte block: the sum of its squares (exact
// binary64 squares, added in a tree) and, in m, the exponent of a lower bound on
// the lowest set bit of its values (kBig: all zero; -kBig: a NaN or infinity).
template <typename Tin>
__device__ __forceinline__ double block_summary(const uint4 &u, int &m) {
    constexpr int EPL = 16 / sizeof(Tin);                  // elements per 16-byte block
    constexpr int kSig = sizeof(Tin) == 2 ? 8 : 24;        // significant bits of the input
    float v[EPL];
    unpack_block<Tin>(u, v);
    uint32_t emin = 0x1FFu;                                // smallest exponent field of a nonzero value
    bool bad = false;
    double sq[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const uint32_t bits = __float_as_uint(v[e]);
        const uint32_t ex = (bits >> 23) & 0xFFu;
        bad = bad | (ex == 0xFFu);
        emin = min(emin, (bits & 0x7FFFFFFFu) ? max(ex, 1u) : 0x1FFu);
        const double d = (double)v[e];
        sq[e] = d * d;                                     // exact in binary64
    }
#pragma unroll
    for (int h = 1; h < EPL; h <<= 1)
#pragma unroll
        for (int e = 0; e < EPL; e += 2 * h) sq[e] = sq[e] + sq[e + h];
    m = bad ? -kBig : emin == 0x1FFu ? kBig : (int)emin - 127 - (kSig - 1);
    return sq[0];
}

template <typename Tin>
__global__ void __launch_bounds__(kFastLanes)
channel_normalize_kernel(const Tin *__restrict__ w, int rows, int cols,
                         const float *__restrict__ su, double floor_value,
                         float *__restrict__ w_norm, float *__restrict__ su_folded,
                         double *__restrict__ row_rms) {
    constexpr int EPL = 16 / sizeof(Tin);                  // elements per 16-byte block
    __shared__ double ring_sum[2][kFastRows][kRingStride];
    __shared__ double ring_bound[2][kFastRows][kRingStride];
    __shared__ uint4 ring_raw[2][kFastRows][kRingStride];
    __shared__ double2 ring_group[2][kFastRows][kGroupStride];   // group sum, group bound
    __shared__ float factor[kFastRows];
    const int t = threadIdx.x;
    const int row0 = blockIdx.x * kFastRows;
    const int nr = min(kFastRows, rows - row0);
    const int nblk = cols / EPL;                           // blocks per row
    const int nchunk = (nblk + kChunkBlocks - 1) / kChunkBlocks;
    // the lane's block of each chunk: row r, block b; eight consecutive lanes
    // hold the blocks of a group
    const int r = t / kChunkBlocks, b = t % kChunkBlocks;
    const int rc = min(r, nr - 1);

    uint4 fifo[kFifo];
    auto issue = [&](int k, uint4 &dst) {
        // past the band or the row: a load of the row's last block, unused
        const int bl = min(k * kChunkBlocks + b, nblk - 1);
        dst = *reinterpret_cast<const uint4 *>(w + (size_t)(row0 + rc) * cols + (size_t)bl * EPL);
    };
    auto store = [&](int k, const uint4 &src) {
        const bool valid = r < nr && k < nchunk && k * kChunkBlocks + b < nblk;
        int m;
        const double s_blk = block_summary<Tin>(src, m);
        if (!valid) m = kBig;
        const double s0 = valid ? s_blk : 0.0;
        int mg = m;
        double sg = s0;
#pragma unroll
        for (int x = 1; x < kGroup; x <<= 1) {
            mg = min(mg, __shfl_xor(mg, x));
            sg = sg + __shfl_xor(sg, x);
        }
        if (valid) {
            ring_sum[k & 1][r][b] = s0;
            ring_bound[k & 1][r][b] = square_bound(m);
            ring_raw[k & 1][r][b] = src;
            if (b % kGroup == 0)
                ring_group[k & 1][r][b / kGroup] = make_double2(sg, square_bound(mg));
        }
    };

    double acc = 0.0;
    double gbound = INFINITY;                      // 2^53 x the lower bound g on acc's lowest set bit
    // the first pass of the loop only issues the first kFifo chunks' loads, so
    // that every load is issued by the same instructions into the same
    // registers (the compiler's waits then keep kFifo - 1 chunks in flight)
    for (int k0 = -kFifo; k0 < nchunk; k0 += kFifo) {
#pragma unroll
        for (int j = 0; j < kFifo; ++j) {
            const int k = k0 + j;
            if (k >= 0) store(k, fifo[j]);
            issue(k + kFifo, fifo[j]);
            if (k < 0) continue;
            __syncthreads();                           // chunk k is in ring slot k & 1
            if (t < nr && k < nchunk) {
                const double *S = ring_sum[k & 1][t];
                const double *B = ring_bound[k & 1][t];
                const double2 *G = ring_group[k & 1][t];
                const int nb = min(kChunkBlocks, nblk - k * kChunkBlocks);
                const int ngr = (nb + kGroup - 1) / kGroup;
                double2 gn = G[0];
                for (int gi = 0; gi < ngr; ++gi) {
                    // the group on the shortcut: its blocks' sums summed in a
                    // tree by the loaders, one dependent addition, one test
                    const double2 gc = gn;
                    gn = G[min(gi + 1, kChunkBlocks / kGroup - 1)];
                    const double a = acc + gc.x;
                    if ((a < gbound) & (a < gc.y)) {
                        acc = a;
                        gbound = gc.y < gbound ? gc.y : gbound;
                    } else {
                        // again from the group's start, a block at a time
                        double x = acc, g = gbound;
                        const int b0 = gi * kGroup, ng = min(kGroup, nb - b0);
                        for (int i = 0; i < ng; ++i) {
                            const double A = x + S[b0 + i];
                            const double bb = B[b0 + i];
                            g = bb < g ? bb : g;
                            if (A < g) {
                                x = A;
                            } else {
                                float v[EPL];
                                unpack_block<Tin>(ring_raw[k & 1][t][b0 + i], v);
#pragma unroll
                                for (int e = 0; e < EPL; ++e) {
                                    const double d = (double)v[e];
                                    x = x + d * d;
                                }
                                // x is now a multiple of its unit in the last
                                // place: that alone bounds its lowest set bit
                                g = x > 0.0 ? next_binade(x) : g;
                            }
                        }
                        acc = x;
                        gbound = g;
                    }
                }
            }
        }
    }
    if (t < nr) {
        const int i = row0 + t;
        const double rr = sqrt(acc / (double)cols);
        const double r_eff = rr == 0.0 ? floor_value : rr;
        factor[t] = (float)(1.0 / r_eff);
        su_folded[i] = rr == 0.0 ? 0.0f : su[i] * (float)rr;
        if (row_rms) row_rms[i] = rr;
    }
    __syncthreads();

    // scaled rows: 16-byte loads (kBatch in flight per lane), 16-byte stores
    constexpr int kBatch = 8;
    const int ng = nr * nblk;
    for (int q0 = t; q0 < ng; q0 += kBatch * kFastLanes) {
        uint4 ub[kBatch];
#pragma unroll
        for (int bt = 0; bt < kBatch; ++bt) {
            const int q = min(q0 + bt * kFastLanes, ng - 1);
            ub[bt] = *reinterpret_cast<const uint4 *>(
                w + (size_t)(row0 + q / nblk) * cols + (size_t)(q % nblk) * EPL);
        }
#pragma unroll
        for (int bt = 0; bt < kBatch; ++bt) {
            const int q = q0 + bt * kFastLanes;
            if (q >= ng) break;
            const int rq = q / nblk;
            const size_t base = (size_t)(row0 + rq) * cols + (size_t)(q % nblk) * EPL;
            const float f = factor[rq];
            float v[EPL];
            unpack_block<Tin>(ub[bt], v);
#pragma unroll
            for (int e = 0; e < EPL; e += 4)
                *reinterpret_cast<float4 *>(w_norm + base + e) =
                    make_float4(v[e] * f, v[e + 1] * f, v[e + 2] * f, v[e + 3] * f);
        }
    }
}

// Lane exchanges of the resident-row form inside a wave without the LDS
// crossbar: DPP row operations (lane i of each row of 16 reads lane i - n of
// its row, row_shr:n; rows 1 and 3, or 2 and 3, read lane 15 or 31,
// row_bcast:15 / :31), lanes without a source keeping `id`, and readlane.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v, double id) {
    const uint64_t u = (uint64_t)__double_as_longlong(v), i = (uint64_t)__double_as_longlong(id);
    const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)i, (int)(uint32_t)u, CTRL, ROW_MASK,
                                               0xF, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(i >> 32), (int)(uint32_t)(u >> 32),
                                               CTRL, ROW_MASK, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v, int id) {
    return __builtin_amdgcn_update_dpp(id, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ double lane_f64(double v, int l) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const int hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
// Inclusive scans (sum; minimum) over lanes 0..L-1 of each group of L lanes
// (L = 8 or 64; for L = 8 only lanes 0..7 are exact, the other groups mixing
// with their neighbours, which their callers do not read).
template <int L>
__device__ __forceinline__ void scan_sum_min(double &v, double &m) {
    const double inf = (double)INFINITY;
    v = dpp_f64<kRowShr1, 0xF>(v, 0.0) + v;
    m = fmin(dpp_f64<kRowShr1, 0xF>(m, inf), m);
    v = dpp_f64<kRowShr2, 0xF>(v, 0.0) + v;
    m = fmin(dpp_f64<kRowShr2, 0xF>(m, inf), m);
    v = dpp_f64<kRowShr4, 0xF>(v, 0.0) + v;
    m = fmin(dpp_f64<kRowShr4, 0xF>(m, inf), m);
    if constexpr (L == 64) {
        v = dpp_f64<kRowShr8, 0xF>(v, 0.0) + v;
        m = fmin(dpp_f64<kRowShr8, 0xF>(m, inf), m);
        v = dpp_f64<kRowBcast15, 0xA>(v, 0.0) + v;
        m = fmin(dpp_f64<kRowBcast15, 0xA>(m, inf), m);
        v = dpp_f64<kRowBcast31, 0xC>(v, 0.0) + v;
        m = fmin(dpp_f64<kRowBcast31, 0xC>(m, inf), m);
    }
}

// The resident-row form, for bf16 rows of at most NCH chunks of 64 blocks
// (the rows whose shortcut groups nearly always pass; binary32 rows, whose
// groups fail, keep the form above).  Wave r of the workgroup owns row r of
// the band from start to end: its lanes load all of the row's blocks at once
// and keep them in registers for the scaled row, so the input is read once,
// and store them with the groups' summaries in LDS; the wave then tests the
// row's groups in parallel (see there) and writes the scaled row.  The waves
// share nothing, so a row is written as soon as its own sum is known.  A group
// that fails is taken block by block, each block's summary recomputed from LDS
// by the same code as the loaders', a failing block one square at a time.
template <typename Tin, int NCH>
__global__ void __launch_bounds__(kFastLanes)
channel_normalize_band_kernel(const Tin *__restrict__ w, int rows, int cols,
                              const float *__restrict__ su, double floor_value,
                              float *__restrict__ w_norm, float *__restrict__ su_folded,
                              double *__restrict__ row_rms) {
    constexpr int EPL = 16 / sizeof(Tin);                  // elements per 16-byte block
    constexpr int NB = NCH * kChunkBlocks;                 // blocks per row at most
    __shared__ uint4 raw[kFastRows][NB];
    __shared__ double2 grp[kFastRows][NB / kGroup];        // group sum, group bound
    const int t = threadIdx.x;
    const int row0 = blockIdx.x * kFastRows;
    const int nr = min(kFastRows, rows - row0);
    const int nblk = cols / EPL;                           // blocks per row (<= NB)
    // wave r, lane b: blocks k * 64 + b of row r; eight consecutive lanes hold
    // the blocks of a group
    const int r = t / kChunkBlocks, b = t % kChunkBlocks;
    if (r >= nr) return;                                   // past the last row (whole waves)
    const Tin *wr = w + (size_t)(row0 + r) * cols;

    // every load of the lane at once (past the row: its last block, unused)
    uint4 u[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int bl = min(k * kChunkBlocks + b, nblk - 1);
        u[k] = *reinterpret_cast<const uint4 *>(wr + (size_t)bl * EPL);
    }
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int kb = k * kChunkBlocks + b;
        const bool valid = kb < nblk;
        int m;
        const double s_blk = block_summary<Tin>(u[k], m);
        if (!valid) m = kBig;
        const double s0 = valid ? s_blk : 0.0;
        // the group's sum and smallest exponent reach its last lane (shifts
        // within rows of 16, eight lanes per group)
        int mg = m;
        double sg = s0;
        sg = dpp_f64<kRowShr1, 0xF>(sg, 0.0) + sg;
        mg = min(dpp_i32<kRowShr1>(mg, kBig), mg);
        sg = dpp_f64<kRowShr2, 0xF>(sg, 0.0) + sg;
        mg = min(dpp_i32<kRowShr2>(mg, kBig), mg);
        sg = dpp_f64<kRowShr4, 0xF>(sg, 0.0) + sg;
        mg = min(dpp_i32<kRowShr4>(mg, kBig), mg);
        if (valid) raw[r][kb] = u[k];
        if (b % kGroup == kGroup - 1 && kb - (kGroup - 1) < nblk)
            grp[r][kb / kGroup] = make_double2(sg, square_bound(mg));
    }
    // the row's LDS entries are the wave's own: its stores are done before its
    // reads (no other wave is waited for)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // the rows' sums: wave r takes row r.  A run of groups s..j that all pass
    // the shortcut is exact whatever the order of its additions (the argument
    // above, for the run as one group), so the wave scans the run at once: lane
    // l holds groups l + 64 q, prefix sums P_j = x + sum and prefix bounds
    // min(g, bounds) over 64 lanes, and a ballot of the tests finds the first
    // group the column-order chain would fail (the test's outcome does not
    // depend on the order of the additions either).  Everything before it is
    // added, the failing group is taken block by block, and the scan resumes
    // after it.  The state (x, g) is the column-order chain's, bit for bit.
    float f_row;
    {
        constexpr int GQ = NB / kGroup / 64;               // groups per lane
        const int lane = t & 63;
        const int ngr = (nblk + kGroup - 1) / kGroup;
        double2 gq[GQ];
#pragma unroll
        for (int q = 0; q < GQ; ++q) gq[q] = grp[r][lane + 64 * q];
        double x = 0.0;
        double g = INFINITY;                       // 2^53 x the lower bound on x's lowest set bit
        int s0 = 0;                                // first group not yet added
        while (s0 < ngr) {
            double carry = x, mcarry = g;
            int f = ngr;                           // first failing group (ngr: none)
            double x_f = x, g_f = g;               // the state just before it
#pragma unroll
            for (int q = 0; q < GQ; ++q) {
                const int j = lane + 64 * q;
                const bool in = j >= s0 && j < ngr;
                double v = in ? gq[q].x : 0.0;
                double m = in ? gq[q].y : (double)INFINITY;
                scan_sum_min<64>(v, m);
                const double P = carry + v;
                const double M = mcarry < m ? mcarry : m;
                const uint64_t fails = __ballot(in && !(P < M));
                if (f == ngr && fails) {
                    const int lf = __builtin_ctzll(fails);
                    f = lf + 64 * q;
                    // the state after group f - 1 (or the run's start)
                    const double Pp = lane_f64(P, lf > 0 ? lf - 1 : 0);
                    const double Mp = lane_f64(M, lf > 0 ? lf - 1 : 0);
                    x_f = f > s0 ? (lf > 0 ? Pp : carry) : x;
                    g_f = f > s0 ? (lf > 0 ? Mp : mcarry) : g;
                }
                carry = lane_f64(P, 63);
                mcarry = lane_f64(M, 63);
            }
            if (f == ngr) {                        // every remaining group passed
                x = carry;
                g = mcarry;
                break;
            }
            // group f again from its start, a block at a time, by the same rule
            // one level down: lanes 0..7 (and their copies in every eight
            // lanes) recompute the group's block summaries from LDS, a scan
            // adds each run of passing blocks and finds the first failing one,
            // which is added one square at a time (all lanes alike)
            x = x_f;
            g = g_f;
            const int b0 = f * kGroup, ng = min(kGroup, nblk - b0);
            const int li = lane & (kGroup - 1);
            int mb;
            const double S = block_summary<Tin>(raw[r][b0 + min(li, ng - 1)], mb);
            const double B = square_bound(mb);
            int i0 = 0;
            while (i0 < ng) {
                const bool in = li >= i0 && li < ng;
                double v = in ? S : 0.0;
                double m = in ? B : (double)INFINITY;
                scan_sum_min<kGroup>(v, m);
                const double P = x + v;
                const double M = g < m ? g : m;
                const uint64_t fails = __ballot(in && !(P < M)) & ((1ull << kGroup) - 1);
                if (!fails) {                      // the rest of the group passed
                    x = lane_f64(P, ng - 1);
                    g = lane_f64(M, ng - 1);
                    break;
                }
                const int lf = __builtin_ctzll(fails);
                // the failing block's bound joins g first, as in the column-order
                // chain; then its squares one at a time
                const double Pp = lane_f64(P, lf > 0 ? lf - 1 : 0);
                x = lf > i0 ? Pp : x;
                g = lane_f64(M, lf);
                float vv[EPL];
                unpack_block<Tin>(raw[r][b0 + lf], vv);
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const double d = (double)vv[e];
                    x = x + d * d;
                }
                // x is now a multiple of its unit in the last place: that alone
                // bounds its lowest set bit
                g = x > 0.0 ? next_binade(x) : g;
                i0 = lf + 1;
            }
            s0 = f + 1;
        }
        const double rr = sqrt(x / (double)cols);
        const double r_eff = rr == 0.0 ? floor_value : rr;
        f_row = (float)(1.0 / r_eff);
        if (lane == 0) {
            const int i = row0 + r;
            su_folded[i] = rr == 0.0 ? 0.0f : su[i] * (float)rr;
            if (row_rms) row_rms[i] = rr;
        }
    }

    // the scaled row from the registers, 16-byte stores
    {
        const float f = f_row;
        float *dst = w_norm + (size_t)(row0 + r) * cols;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int kb = k * kChunkBlocks + b;
            if (kb < nblk) {
                float v[EPL];
                unpack_block<Tin>(u[k], v);
#pragma unroll
                for (int e = 0; e < EPL; e += 4)
                    *reinterpret_cast<float4 *>(dst + (size_t)kb * EPL + e) =
                        make_float4(v[e] * f, v[e + 1] * f, v[e + 2] * f, v[e + 3] * f);
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
    const unsigned fast_blocks = (unsigned)((rows + kFastRows - 1) / kFastRows);
    const size_t in_bytes = w_dtype == EXL3_BF16 ? 2 : 4;
    const bool fast = reinterpret_cast<uintptr_t>(w) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(w_norm) % 16 == 0 &&
                      ((size_t)cols * in_bytes) % 16 == 0 && ((size_t)cols * 4) % 16 == 0;
    if (w_dtype == EXL3_BF16) {
        const uint16_t *wb = static_cast<const uint16_t *>(w);
        const int nchunk = (cols / 8 + kChunkBlocks - 1) / kChunkBlocks;
        if (fast && nchunk <= 16) {
            if (nchunk <= 8)
                hipLaunchKernelGGL((channel_normalize_band_kernel<uint16_t, 8>), dim3(fast_blocks),
                                   dim3(kFastLanes), 0, stream, wb, rows, cols, su, floor_value,
                                   w_norm, su_folded, row_rms);
            else
                hipLaunchKernelGGL((channel_normalize_band_kernel<uint16_t, 16>),
                                   dim3(fast_blocks), dim3(kFastLanes), 0, stream, wb, rows, cols,
                                   su, floor_value, w_norm, su_folded, row_rms);
        } else if (fast)
            hipLaunchKernelGGL(channel_normalize_kernel<uint16_t>, dim3(fast_blocks), dim3(kFastLanes), 0,
                               stream, wb, rows, cols, su, floor_value, w_norm, su_folded,
                               row_rms);
        else
            hipLaunchKernelGGL(channel_normalize_any_kernel<uint16_t>, dim3(blocks),
                               dim3(kChunkCols), 0, stream, wb, rows, cols, su, floor_value,
                               w_norm, su_folded, row_rms);
    } else {
        const float *wf = static_cast<const float *>(w);
        if (fast)
            hipLaunchKernelGGL(channel_normalize_kernel<float>, dim3(fast_blocks), dim3(kFastLanes), 0,
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
