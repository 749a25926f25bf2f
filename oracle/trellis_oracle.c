/*
 * Reference CPU trellis search -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is part of the oracle: a plain, slow implementation that the
 * test-suite, the smoke check and the CPU-baseline leg of the benchmark use to
 * judge the GPU library.  Nothing in the product path may link or call it.
 *
 * What it computes (source: "EXL3 Intel Arc Quantizer" README, Core Implemented
 * Architecture, section 1 "SYCL XPU Tile Encoder" -- the add-compare-select
 * dynamic program and the two-pass tail-biting closure -- and section 4
 * "Contract-Conformant CPU Reference Encoder" -- the state algebra):
 *
 *   * a trellis state is a Q-bit word (Q = 16 in production); each step shifts
 *     K new bits in at the bottom: S_t = ((S_{t-1} << K) | b_t) mod 2^Q;
 *   * Kr = Q - K; the dynamic program keeps one running minimum per value of
 *     the low Kr bits ("tracked" states), i.e. 2^Kr numbers;
 *   * the previous full states that can precede a state whose top Kr bits
 *     equal e are (k << Kr) | e for k = 0 .. 2^K - 1;
 *   * branch metric at step t for state s: (x_t - v[s])^2, v = scaled levels.
 *
 * Numeric contract of this part (a reading: the pages' own encoder works in fp16
 * with a fused multiply-add, which the binary16 functions further down follow;
 * here binary32 with every operation rounded on its own, which the file is
 * compiled for with -ffp-contract=off):
 *   d = x_t - v[s];  q = d * d;  C[s] = M[s >> K] + q        (three roundings)
 *   M'[e] = first strict minimum over k ascending of C[(k << Kr) | e]
 *   bp[t][e] = the k that produced it (lowest k among equal costs).
 *
 * The code follows the description step by step; it is deliberately unblocked
 * and unvectorised by hand.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/*
 * Forward pass.  x[0..L-1] are the step inputs, v[0..2^Q-1] the level of every
 * state, M0[0..2^Kr-1] the starting tracked costs.  On return C[0..2^Q-1]
 * holds the costs of every state at the last step.  If bp is not NULL it
 * receives the chosen predecessor k for every step t in [bp_first, L-2] and
 * every tracked state e, at bp[(t - bp_first) * 2^Kr + e].
 */
static void forward_pass(const float *x, int L, int Q, int K, const float *v,
                         const float *M0, float *C, uint8_t *bp, int bp_first,
                         float *M, float *Mnext)
{
    const uint32_t n_states = 1u << Q;
    const int Kr = Q - K;
    const uint32_t n_tracked = 1u << Kr;
    const uint32_t n_branch = 1u << K;

    memcpy(M, M0, n_tracked * sizeof(float));
    for (int t = 0; t < L; t++) {
        const float xt = x[t];
        for (uint32_t s = 0; s < n_states; s++) {
            float d = xt - v[s];
            float q = d * d;
            C[s] = M[s >> K] + q;
        }
        if (t == L - 1)
            break;
        for (uint32_t e = 0; e < n_tracked; e++) {
            float best = C[e];
            uint32_t kbest = 0;
            for (uint32_t k = 1; k < n_branch; k++) {
                float c = C[(k << Kr) | e];
                if (c < best) {
                    best = c;
                    kbest = k;
                }
            }
            Mnext[e] = best;
            if (bp != NULL && t >= bp_first)
                bp[(size_t)(t - bp_first) * n_tracked + e] = (uint8_t)kbest;
        }
        float *tmp = M;
        M = Mnext;
        Mnext = tmp;
    }
}

/* Exported forward pass for tests (brute-force comparison on tiny trellises). */
int oracle_forward(const float *x, int L, int Q, int K, const float *v,
                   const float *M0, float *C_out, uint8_t *bp_out)
{
    if (Q < 2 || Q > 16 || K < 1 || K >= Q || L < 2)
        return -1;
    const size_t n_tracked = (size_t)1 << (Q - K);
    float *M = (float *)malloc(n_tracked * sizeof(float));
    float *Mn = (float *)malloc(n_tracked * sizeof(float));
    if (!M || !Mn) {
        free(M);
        free(Mn);
        return -2;
    }
    forward_pass(x, L, Q, K, v, M0, C_out, bp_out, 0, M, Mn);
    free(M);
    free(Mn);
    return 0;
}

/*
 * Two-pass tail-biting encode of one sequence of L inputs (L even).
 *
 * Pass 1 runs on the input rotated by L/2 from all-zero starting costs, takes
 * the lowest-cost final state (lowest index on equal costs) and walks the
 * predecessors back to rotated step L/2 - 1, which is original position L-1;
 * that state is X.  Pass 2 runs on the input in its own order with only the
 * tracked index X's low Kr bits admitted at the start (cost 0, all others
 * +inf), and the path is read back starting from X at the last step, so the
 * state sequence closes into a ring.
 *
 * Outputs: states[0..L-1] (S_t), *X_out, *cost_out = pass-2 cost of X at the
 * last step (the sequential binary32 sum of the path's branch metrics).
 */
int oracle_encode_seq(const float *x, int L, int Q, int K, const float *v,
                      int32_t *states, int32_t *X_out, float *cost_out)
{
    if (Q < 2 || Q > 16 || K < 1 || K >= Q || L < 2 || (L & 1))
        return -1;
    const int Kr = Q - K;
    const uint32_t n_states = 1u << Q;
    const uint32_t n_tracked = 1u << Kr;
    const uint32_t mask = n_tracked - 1u;
    const int half = L / 2;

    float *xr = (float *)malloc((size_t)L * sizeof(float));
    float *M0 = (float *)malloc(n_tracked * sizeof(float));
    float *M = (float *)malloc(n_tracked * sizeof(float));
    float *Mn = (float *)malloc(n_tracked * sizeof(float));
    float *C = (float *)malloc(n_states * sizeof(float));
    uint8_t *bp = (uint8_t *)malloc((size_t)(L - 1) * n_tracked);
    if (!xr || !M0 || !M || !Mn || !C || !bp) {
        free(xr); free(M0); free(M); free(Mn); free(C); free(bp);
        return -2;
    }

    /* ---- pass 1: rotated input, free start ---- */
    for (int j = 0; j < L; j++)
        xr[j] = x[(j + half) % L];
    for (uint32_t e = 0; e < n_tracked; e++)
        M0[e] = 0.0f;
    /* predecessors are needed for steps half-1 .. L-2 */
    forward_pass(xr, L, Q, K, v, M0, C, bp, half - 1, M, Mn);
    uint32_t s = 0;
    float best = C[0];
    for (uint32_t i = 1; i < n_states; i++) {
        if (C[i] < best) {
            best = C[i];
            s = i;
        }
    }
    for (int j = L - 1; j >= half; j--) {
        uint32_t e = s >> K;
        uint32_t k = bp[(size_t)(j - 1 - (half - 1)) * n_tracked + e];
        s = (k << Kr) | e;
    }
    const uint32_t X = s;

    /* ---- pass 2: original order, start pinned to X's low bits ---- */
    for (uint32_t e = 0; e < n_tracked; e++)
        M0[e] = (e == (X & mask)) ? 0.0f : INFINITY;
    forward_pass(x, L, Q, K, v, M0, C, bp, 0, M, Mn);
    *cost_out = C[X];
    s = X;
    states[L - 1] = (int32_t)s;
    for (int t = L - 1; t >= 1; t--) {
        uint32_t e = s >> K;
        uint32_t k = bp[(size_t)(t - 1) * n_tracked + e];
        s = (k << Kr) | e;
        states[t - 1] = (int32_t)s;
    }
    *X_out = (int32_t)X;

    free(xr); free(M0); free(M); free(Mn); free(C); free(bp);
    return 0;
}

/* Loop of oracle_encode_seq over n sequences stored one after the other. */
int oracle_encode_many(const float *x, int64_t n, int L, int Q, int K,
                       const float *v, int32_t *states, int32_t *X_out,
                       float *cost_out)
{
    for (int64_t i = 0; i < n; i++) {
        int rc = oracle_encode_seq(x + i * L, L, Q, K, v, states + i * L,
                                   X_out + i, cost_out + i);
        if (rc != 0)
            return rc;
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * fp16 mode ("EXL3 Intel Arc Quantizer" README, Core Implemented
 * Architecture section 1 and section 4: the pages' own numeric contract).
 * Inputs, levels and path costs are IEEE binary16 (bit patterns in uint16);
 * per state and step
 *     d = fp16(x_t - c[s])                 (one rounding)
 *     C = fp16(d * d + M[s >> K])          (fused: one rounding of the exact value)
 * and the tracked minimum keeps the first strict minimum over k.  Rounding is
 * to nearest, ties to even, with subnormals; overflow gives +inf.
 *
 * Every binary16 value is an integer multiple of 2^-24 and every product of
 * two is a multiple of 2^-48, so the exact value of d*d + M is an integer
 * multiple of 2^-48; it is held as a 128-bit integer and rounded once.
 * ------------------------------------------------------------------------ */
typedef __int128 i128;

/* binary16 bits -> exact value as a multiple of 2^-24 (signed 64-bit) */
static int64_t f16_to_q24(uint16_t h, int *is_inf)
{
    int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    *is_inf = 0;
    if (e == 31) {
        *is_inf = sign ? -1 : 1;
        return 0;
    }
    int64_t mag = (e == 0) ? (int64_t)f : (int64_t)(1024 + f) << (e - 1);
    return sign ? -mag : mag;
}

/* round n * 2^-frac (exact) to binary16, nearest-even */
static uint16_t round_to_f16(i128 n, int frac)
{
    uint16_t sign = 0;
    if (n < 0) {
        sign = 0x8000;
        n = -n;
    }
    if (n == 0)
        return sign;
    /* express in units of 2^-24 (the binary16 subnormal step) */
    int sh = frac - 24;                 /* >= 0 for our callers */
    i128 q = n >> sh;
    i128 rem = n - (q << sh);
    i128 half = sh > 0 ? ((i128)1 << (sh - 1)) : 0;
    /* find the binary16 quantum for this magnitude: values in [2^(b-1), 2^b)
       units of 2^-24 have 11 significant bits when b > 11 */
    int b = 0;
    for (i128 t = q; t > 0; t >>= 1)
        b++;
    if (b > 11) {
        int s2 = b - 11;                /* extra bits to drop */
        i128 q2 = q >> s2;
        i128 rem2 = ((q - (q2 << s2)) << sh) + rem;   /* remainder in 2^-frac units */
        i128 half2 = (i128)1 << (s2 + sh - 1);
        if (rem2 > half2 || (rem2 == half2 && (q2 & 1)))
            q2 += 1;
        if (q2 == 2048) {
            q2 = 1024;
            s2 += 1;
        }
        int efield = s2 + 1;            /* q2 in [1024, 2048): value = q2 * 2^(s2) * 2^-24 */
        if (efield >= 31)
            return sign | 0x7C00;       /* overflow -> infinity */
        return sign | (uint16_t)(efield << 10) | (uint16_t)(q2 - 1024);
    }
    /* subnormal or smallest normal range: quantum 2^-24 */
    if (sh > 0 && (rem > half || (rem == half && (q & 1))))
        q += 1;
    if (q >= 1024)                      /* rounded up into the normal range */
        return sign | (uint16_t)(1 << 10) | (uint16_t)(q - 1024);
    return sign | (uint16_t)q;
}

uint16_t oracle_f16_sub(uint16_t a, uint16_t b)
{
    int ia, ib;
    int64_t qa = f16_to_q24(a, &ia), qb = f16_to_q24(b, &ib);
    if (ia || ib) {
        if (ia && ib && ia == ib)
            return 0x7E00;              /* inf - inf: NaN (not reached by the encoder) */
        if (ia)
            return ia > 0 ? 0x7C00 : 0xFC00;
        return ib > 0 ? 0xFC00 : 0x7C00;
    }
    return round_to_f16((i128)qa - (i128)qb, 24);
}

/* fp16(d*d + m) with one rounding; m may be +inf */
uint16_t oracle_f16_sqadd(uint16_t d, uint16_t m)
{
    int id, im;
    int64_t qd = f16_to_q24(d, &id), qm = f16_to_q24(m, &im);
    if (id || im)
        return 0x7C00;                  /* +inf (costs are non-negative) */
    i128 n = (i128)qd * qd + ((i128)qm << 24);   /* units of 2^-48 */
    return round_to_f16(n, 48);
}

/* binary16 order for non-negative values and +inf: bit patterns compare as integers */
static int f16_less(uint16_t a, uint16_t b) { return a < b; }

static void forward_pass_f16(const uint16_t *x, int L, int Q, int K, const uint16_t *c,
                             const uint16_t *M0, uint16_t *C, uint8_t *bp, int bp_first,
                             uint16_t *M, uint16_t *Mnext)
{
    const uint32_t n_states = 1u << Q;
    const int Kr = Q - K;
    const uint32_t n_tracked = 1u << Kr;
    const uint32_t n_branch = 1u << K;

    memcpy(M, M0, n_tracked * sizeof(uint16_t));
    for (int t = 0; t < L; t++) {
        for (uint32_t s = 0; s < n_states; s++) {
            uint16_t d = oracle_f16_sub(x[t], c[s]);
            C[s] = oracle_f16_sqadd(d, M[s >> K]);
        }
        if (t == L - 1)
            break;
        for (uint32_t e = 0; e < n_tracked; e++) {
            uint16_t best = C[e];
            uint32_t kbest = 0;
            for (uint32_t k = 1; k < n_branch; k++) {
                uint16_t cc = C[(k << Kr) | e];
                if (f16_less(cc, best)) {
                    best = cc;
                    kbest = k;
                }
            }
            Mnext[e] = best;
            if (bp != NULL && t >= bp_first)
                bp[(size_t)(t - bp_first) * n_tracked + e] = (uint8_t)kbest;
        }
        uint16_t *tmp = M;
        M = Mnext;
        Mnext = tmp;
    }
}

int oracle_forward_f16(const uint16_t *x, int L, int Q, int K, const uint16_t *c,
                       const uint16_t *M0, uint16_t *C_out, uint8_t *bp_out)
{
    if (Q < 2 || Q > 16 || K < 1 || K >= Q || L < 2)
        return -1;
    const size_t n_tracked = (size_t)1 << (Q - K);
    uint16_t *M = (uint16_t *)malloc(n_tracked * sizeof(uint16_t));
    uint16_t *Mn = (uint16_t *)malloc(n_tracked * sizeof(uint16_t));
    if (!M || !Mn) {
        free(M);
        free(Mn);
        return -2;
    }
    forward_pass_f16(x, L, Q, K, c, M0, C_out, bp_out, 0, M, Mn);
    free(M);
    free(Mn);
    return 0;
}

/* Two-pass tail-biting encode in fp16 (same closure as oracle_encode_seq). */
int oracle_encode_seq_f16(const uint16_t *x, int L, int Q, int K, const uint16_t *c,
                          int32_t *states, int32_t *X_out, uint16_t *cost_out)
{
    if (Q < 2 || Q > 16 || K < 1 || K >= Q || L < 2 || (L & 1))
        return -1;
    const int Kr = Q - K;
    const uint32_t n_states = 1u << Q;
    const uint32_t n_tracked = 1u << Kr;
    const uint32_t mask = n_tracked - 1u;
    const int half = L / 2;

    uint16_t *xr = (uint16_t *)malloc((size_t)L * sizeof(uint16_t));
    uint16_t *M0 = (uint16_t *)malloc(n_tracked * sizeof(uint16_t));
    uint16_t *M = (uint16_t *)malloc(n_tracked * sizeof(uint16_t));
    uint16_t *Mn = (uint16_t *)malloc(n_tracked * sizeof(uint16_t));
    uint16_t *C = (uint16_t *)malloc(n_states * sizeof(uint16_t));
    uint8_t *bp = (uint8_t *)malloc((size_t)(L - 1) * n_tracked);
    if (!xr || !M0 || !M || !Mn || !C || !bp) {
        free(xr); free(M0); free(M); free(Mn); free(C); free(bp);
        return -2;
    }
    for (int j = 0; j < L; j++)
        xr[j] = x[(j + half) % L];
    for (uint32_t e = 0; e < n_tracked; e++)
        M0[e] = 0;
    forward_pass_f16(xr, L, Q, K, c, M0, C, bp, half - 1, M, Mn);
    uint32_t s = 0;
    uint16_t best = C[0];
    for (uint32_t i = 1; i < n_states; i++) {
        if (f16_less(C[i], best)) {
            best = C[i];
            s = i;
        }
    }
    for (int j = L - 1; j >= half; j--) {
        uint32_t e = s >> K;
        uint32_t k = bp[(size_t)(j - 1 - (half - 1)) * n_tracked + e];
        s = (k << Kr) | e;
    }
    const uint32_t X = s;
    for (uint32_t e = 0; e < n_tracked; e++)
        M0[e] = (e == (X & mask)) ? 0 : 0x7C00;
    forward_pass_f16(x, L, Q, K, c, M0, C, bp, 0, M, Mn);
    *cost_out = C[X];
    s = X;
    states[L - 1] = (int32_t)s;
    for (int t = L - 1; t >= 1; t--) {
        uint32_t e = s >> K;
        uint32_t k = bp[(size_t)(t - 1) * n_tracked + e];
        s = (k << Kr) | e;
        states[t - 1] = (int32_t)s;
    }
    *X_out = (int32_t)X;
    free(xr); free(M0); free(M); free(Mn); free(C); free(bp);
    return 0;
}

int oracle_encode_many_f16(const uint16_t *x, int64_t n, int L, int Q, int K,
                           const uint16_t *c, int32_t *states, int32_t *X_out,
                           uint16_t *cost_out)
{
    for (int64_t i = 0; i < n; i++) {
        int rc = oracle_encode_seq_f16(x + i * L, L, Q, K, c, states + i * L, X_out + i,
                                       cost_out + i);
        if (rc != 0)
            return rc;
    }
    return 0;
}
