// Host generators of the level tables used by the gfx950 encoder: mul1 (the
// default), mcg and 3INST.
//
// Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture
// section 5 names the mul1 procedural codebook (a level for each 16-bit state;
// the distinct values are fp16 numbers spread over roughly [-3.45, 3.35]) but
// does not define it.  This library's definition (a documented reading, not a
// reproduction of upstream's table):
//   h(s)    = (A * s) mod 2^32 with A = 0x9E3779B1 (odd; golden-ratio hash),
//   beta(s) = sum of the four bytes of h(s),
//   level   = fp16 round-to-nearest-even of (beta - mean) / std,
// where mean and std are over all 2^16 states.  The quotient is formed as
// (2^16 * beta - S1) / sqrt(2^16 * S2 - S1^2) with exact integer sums
// S1 = sum beta, S2 = sum beta^2, so only two correctly rounded binary64
// operations are involved and the table is the same on every IEEE machine.
#include "exl3_internal.h"

#include <cmath>
#include <cstdint>

namespace exl3 {

namespace {

constexpr uint32_t kMul1A = 0x9E3779B1u;

// binary64 -> fp16 bits, round to nearest, ties to even (finite inputs).
uint16_t f64_to_f16_bits(double z) {
    uint16_t sign = std::signbit(z) ? 0x8000u : 0u;
    double a = std::fabs(z);
    if (a == 0.0) return sign;
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);   // rounds to infinity
    int e = 0;
    std::frexp(a, &e);                 // a in [2^(e-1), 2^e)
    int ulp_exp = e - 11;              // 11 significant bits in the normal range
    if (ulp_exp < -24) ulp_exp = -24;  // subnormal spacing
    double q = std::ldexp(a, -ulp_exp);          // exact
    double r = std::nearbyint(q);                // ties to even (default mode)
    long mant = (long)r;
    if (mant >= 2048) {                          // carried into the next binade
        mant >>= 1;
        ulp_exp += 1;
    }
    if (mant < 1024) return (uint16_t)(sign | (uint16_t)mant);   // subnormal
    int efield = ulp_exp + 25;
    return (uint16_t)(sign | (uint16_t)(efield << 10) | (uint16_t)(mant - 1024));
}

}  // namespace

void build_mul1_levels(uint16_t *out) {
    static int beta[65536];
    int64_t s1 = 0, s2 = 0;
    for (uint32_t s = 0; s < 65536u; ++s) {
        uint32_t h = kMul1A * s;       // mod 2^32
        int bsum = (int)(h & 0xFFu) + (int)((h >> 8) & 0xFFu) + (int)((h >> 16) & 0xFFu) +
                   (int)(h >> 24);
        beta[s] = bsum;
        s1 += bsum;
        s2 += (int64_t)bsum * bsum;
    }
    const int64_t n = 65536;
    const double denom = std::sqrt((double)(n * s2 - s1 * s1));
    for (uint32_t s = 0; s < 65536u; ++s) {
        double z = (double)(n * beta[s] - s1) / denom;
        out[s] = f64_to_f16_bits(z);
    }
}

// mcg and 3INST [P1 section 5 names them and prints their counts of distinct
// levels, 10,746 and 10,598].  A state gives a 32-bit word: 3INST is the
// published three-instruction decoder of the QTIP trellis codes (linear
// congruential step w = a*s + b mod 2^32), mcg a multiplicative step
// w = A*s mod 2^32.  The pages give no multiplier; A = 0x9E378FED is the first
// odd number at or above the golden-ratio constant 0x9E3779B1 (the mul1
// reading's multiplier) whose table has exactly the printed 10,746 distinct
// levels, the 2,847th odd number scanned.  Then
// w = (w & 0x8FFF8FFF) ^ 0x3B603B60 leaves each 16-bit half a binary16 number
// of magnitude [1/8, 2) (exponent field 12..15), and the level is the
// binary16 round-to-nearest-even of the sum of the two halves (the binary64
// sum of two such numbers is exact).
namespace {

constexpr uint32_t kInst3A = 89226354u, kInst3B = 64248484u;
constexpr uint32_t kMcgA = 0x9E378FEDu;

double f16_bits_to_double(uint16_t h) {
    const int e = (h >> 10) & 0x1F;
    const int f = h & 0x3FF;
    double v = e == 0 ? std::ldexp((double)f, -24) : std::ldexp((double)(1024 + f), e - 25);
    return (h & 0x8000u) ? -v : v;
}

void build_halves_sum(uint32_t a, uint32_t b, uint16_t *out) {
    for (uint32_t s = 0; s < 65536u; ++s) {
        const uint32_t w = ((a * s + b) & 0x8FFF8FFFu) ^ 0x3B603B60u;
        const double sum = f16_bits_to_double((uint16_t)(w & 0xFFFFu)) +
                           f16_bits_to_double((uint16_t)(w >> 16));
        out[s] = f64_to_f16_bits(sum);
    }
}

}  // namespace

void build_mcg_levels(uint16_t *out) { build_halves_sum(kMcgA, 0u, out); }
void build_3inst_levels(uint16_t *out) { build_halves_sum(kInst3A, kInst3B, out); }

}  // namespace exl3
