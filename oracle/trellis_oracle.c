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
 * Numeric contract (a reading: the pages' own encoder works in fp16 with a fused
 * multiply-add; this build fixes binary32 with every operation rounded on its
 * own, which the file is compiled for with -ffp-contract=off):
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
