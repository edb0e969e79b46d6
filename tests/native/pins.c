/*
 * pins.c -- exhaustive property checks used by the CPU test suite to pin the
 * oracle.  Nothing here computes a split or a GEMM: every function receives
 * the oracle's outputs and checks properties that the split and the BF16
 * products must have.
 *
 * Properties (NVIDIA Technical Blog, "Unlocking Tensor Core Performance for
 * Machine Learning Interatomic Potentials", Fig. 1 caption, and the
 * discuss.pytorch.kr summary, section on BF16x9: x = x0 + 2^-8 x1 + 2^-16 x2,
 * each piece holding 8 significant bits):
 *   P1 exact reconstruction in double for every finite x;
 *   P2 x0 is x rounded toward zero to BF16: same sign, |x0| <= |x| and no
 *      BF16 value lies strictly between |x0| and |x|  (|x| - |x0| < ulp_bf16(x0));
 *   P3 x1 is t = 2^8 (x - x0) rounded toward zero to BF16, checked the same way;
 *   P4 components carry the sign of x (a truncated tiny negative piece is -0)
 *      or are +0;
 *   P5 non-finite x: x0 is the same special class with the same sign, x1 = x2 = +0.
 * Built with -O2 -fno-fast-math -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static double bf(uint16_t h) { return (double)f_of((uint32_t)h << 16); }

/* distance from |v| (a BF16 value) to the next larger BF16 magnitude */
static double bf16_ulp_above(uint16_t h)
{
    uint16_t mag = h & 0x7FFF;
    return bf((uint16_t)(mag + 1)) - bf(mag);
}

static int sign_ok(uint16_t comp, int neg)
{
    if ((comp & 0x7FFF) == 0) return comp == 0 || neg;   /* +0, or -0 for negative x */
    return ((comp >> 15) != 0) == neg;
}

/* Is v (finite double holding a float) truncated to BF16 by h? */
static int is_rz_bf16(double v, uint16_t h)
{
    double a = fabs(v), b = bf(h & 0x7FFF);
    if (b > a) return 0;
    return (a - b) < bf16_ulp_above(h);
}

/*
 * Check the oracle's split of the encodings start .. start+count-1.
 * Returns the number of failing encodings; the first one is stored in *first_bad.
 */
int64_t pin_split_range(uint64_t start, int64_t count, const uint16_t *x0,
                        const uint16_t *x1, const uint16_t *x2, uint64_t *first_bad)
{
    int64_t bad = 0;
    uint64_t first = UINT64_MAX;
    #pragma omp parallel for reduction(+:bad) schedule(static)
    for (int64_t n = 0; n < count; ++n) {
        uint32_t u = (uint32_t)(start + (uint64_t)n);
        float x = f_of(u);
        int ok = 1;
        if (!isfinite(x)) {
            float c0 = f_of((uint32_t)x0[n] << 16);
            ok = x1[n] == 0 && x2[n] == 0 && (signbit(c0) != 0) == (signbit(x) != 0);
            if (isnan(x)) ok = ok && isnan(c0) && (x0[n] & 0x0040);   /* quiet NaN */
            else ok = ok && isinf(c0);
        } else {
            int neg = signbit(x) != 0;
            double X = (double)x;
            double r = bf(x0[n]) + ldexp(bf(x1[n]), -8) + ldexp(bf(x2[n]), -16);
            ok = ok && (r == X);                                         /* P1 */
            if (x != 0.0f) ok = ok && ((x0[n] & 0x7FFF) == 0 || sign_ok(x0[n], neg));
            else ok = ok && (x0[n] == (uint16_t)(u >> 16));              /* +-0 keeps sign */
            ok = ok && is_rz_bf16(X, x0[n]);                             /* P2 */
            double t = ldexp(X - bf(x0[n]), 8);
            ok = ok && is_rz_bf16(t, x1[n]);                             /* P3 */
            ok = ok && sign_ok(x1[n], neg) && sign_ok(x2[n], neg);       /* P4 */
            ok = ok && isfinite(bf(x1[n])) && isfinite(bf(x2[n]));
        }
        if (!ok) {
            bad += 1;
            #pragma omp critical
            { if ((uint64_t)u < first) first = u; }
        }
    }
    *first_bad = first;
    return bad;
}

/*
 * Is h a round-to-nearest-even BF16 of the finite value v (a double holding a
 * float, the split's remainder t, or x itself)?  The two BF16 magnitudes that
 * bracket |v| are found by masking |v|'s FP32 pattern to its high half and
 * stepping once away from zero; h must be the nearer one with v's sign, the
 * one with an even last mantissa bit on a tie, and the lower one when the
 * upper would be Inf (the split never rounds to Inf).  Zero v must give +-0.
 */
static int is_rne_bf16(double v, uint16_t h)
{
    float vf = (float)v;
    if ((double)vf != v) return 0;                       /* v must be exactly a float */
    uint32_t mag = u_of(fabsf(vf)) >> 16;                /* truncated magnitude */
    uint16_t lo = (uint16_t)mag, hi = (uint16_t)(mag + 1);
    double a = fabs(v);
    uint16_t hm = h & 0x7FFF;
    if (a == 0.0) return hm == 0;
    if (hm != lo && hm != hi) return 0;
    if (((h >> 15) != 0) != (v < 0.0)) return 0;         /* same sign as v */
    if ((hi & 0x7F80) == 0x7F80) return hm == lo;        /* upper neighbour is Inf */
    double dl = a - bf(lo), dh = bf(hi) - a;
    if (dl < dh) return hm == lo;
    if (dh < dl) return hm == hi;
    return (hm & 1) == 0;                                /* tie: even mantissa */
}

/*
 * Round-to-nearest split (the ablation's rounding), encodings start ..
 * start+count-1: exact reconstruction, x0 a round-to-nearest-even BF16 of x,
 * x1 of t = 2^8 (x - x0), finite components, special classes as for RZ.
 */
int64_t pin_split_rne_range(uint64_t start, int64_t count, const uint16_t *x0,
                            const uint16_t *x1, const uint16_t *x2, uint64_t *first_bad)
{
    int64_t bad = 0;
    uint64_t first = UINT64_MAX;
    #pragma omp parallel for reduction(+:bad) schedule(static)
    for (int64_t n = 0; n < count; ++n) {
        uint32_t u = (uint32_t)(start + (uint64_t)n);
        float x = f_of(u);
        int ok = 1;
        if (!isfinite(x)) {
            float c0 = f_of((uint32_t)x0[n] << 16);
            ok = x1[n] == 0 && x2[n] == 0 && (signbit(c0) != 0) == (signbit(x) != 0);
            if (isnan(x)) ok = ok && isnan(c0) && (x0[n] & 0x0040);
            else ok = ok && isinf(c0);
        } else {
            double X = (double)x;
            double r = bf(x0[n]) + ldexp(bf(x1[n]), -8) + ldexp(bf(x2[n]), -16);
            ok = ok && (r == X);
            if (x == 0.0f) ok = ok && (x0[n] == (uint16_t)(u >> 16)) && x1[n] == 0 && x2[n] == 0;
            else ok = ok && is_rne_bf16(X, x0[n]);
            double t = ldexp(X - bf(x0[n]), 8);
            if (t != 0.0) ok = ok && is_rne_bf16(t, x1[n]);
            else ok = ok && x1[n] == 0;
            ok = ok && isfinite(bf(x0[n])) && isfinite(bf(x1[n])) && isfinite(bf(x2[n]));
        }
        if (!ok) {
            bad += 1;
            #pragma omp critical
            { if ((uint64_t)u < first) first = u; }
        }
    }
    *first_bad = first;
    return bad;
}

/*
 * BF16 x BF16 products are exact in FP32 when they stay in FP32's normal
 * range: 8 x 8 significant bits give at most 16.  Checks every ordered pair
 * (a, b) with a's pattern in [a_start, a_start + a_count) and every b.
 * Returns the number of failures; *checked counts pairs in range.
 */
int64_t pin_bf16_products(uint32_t a_start, uint32_t a_count, int64_t *checked)
{
    int64_t bad = 0, n = 0;
    #pragma omp parallel for reduction(+:bad,n) schedule(dynamic, 16)
    for (uint32_t ia = 0; ia < a_count; ++ia) {
        float a = f_of((a_start + ia) << 16);
        if (!isfinite(a)) continue;
        for (uint32_t ib = 0; ib < 65536u; ++ib) {
            float b = f_of(ib << 16);
            if (!isfinite(b)) continue;
            double exact = (double)a * (double)b;
            double m = fabs(exact);
            if (m < 0x1p-126 || m > (double)3.4028234663852886e38) continue;
            volatile float p = a * b;
            n += 1;
            if ((double)p != exact) bad += 1;
        }
    }
    *checked = n;
    return bad;
}

/*
 * Band algebra on pairs (a, b) with their oracle splits:
 *   E1 a*b == sum_{p,q} 2^-8(p+q) a_p b_q exactly (in double);
 *   E2 a*b - [a0 b0 + 2^-8 (a0 b1 + a1 b0)]
 *        == 2^-16 (a0 b2 + a1 b1 + a2 b0) + 2^-24 (a1 b2 + a2 b1) + 2^-32 a2 b2;
 *   E3 the mass dropped by keeping bands s < b is below bound_b |a b| for
 *      normal a and b, with bound_4 = 2^-30, bound_3 = 2^-21 + 2^-30,
 *      bound_2 = 2^-13 + 2^-21 + 2^-30, bound_1 = 2^-6 + 2^-13 + 2^-21 + 2^-30.
 * Returns the number of failing pairs.
 */
int64_t pin_band_algebra(int64_t n, const float *a, const float *b,
                         const uint16_t *a0, const uint16_t *a1, const uint16_t *a2,
                         const uint16_t *b0, const uint16_t *b1, const uint16_t *b2)
{
    static const double bound[5] = {0x1p-6 + 0x1p-13 + 0x1p-21 + 0x1p-30,
                                    0x1p-13 + 0x1p-21 + 0x1p-30,
                                    0x1p-21 + 0x1p-30, 0x1p-30, 0.0};
    int64_t bad = 0;
    #pragma omp parallel for reduction(+:bad) schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double A[3] = {bf(a0[i]), bf(a1[i]), bf(a2[i])};
        double B[3] = {bf(b0[i]), bf(b1[i]), bf(b2[i])};
        double exact = (double)a[i] * (double)b[i];
        double band[5] = {0, 0, 0, 0, 0};
        for (int p = 0; p < 3; ++p)
            for (int q = 0; q < 3; ++q) band[p + q] += A[p] * B[q];
        double total = 0.0;
        for (int s = 4; s >= 0; --s) total += ldexp(band[s], -8 * s);
        int ok = total == exact;                                                 /* E1 */
        double kept2 = A[0] * B[0] + ldexp(A[0] * B[1] + A[1] * B[0], -8);
        double dropped = ldexp(A[0] * B[2] + A[1] * B[1] + A[2] * B[0], -16)
                       + ldexp(A[1] * B[2] + A[2] * B[1], -24) + ldexp(A[2] * B[2], -32);
        ok = ok && (exact - kept2 == dropped);                                   /* E2 */
        int normal = fabsf(a[i]) >= 0x1p-126f && fabsf(b[i]) >= 0x1p-126f;
        if (normal) {
            double kept = 0.0;
            for (int nb = 1; nb <= 4; ++nb) {
                kept += ldexp(band[nb - 1], -8 * (nb - 1));
                ok = ok && fabs(exact - kept) < bound[nb - 1] * fabs(exact);      /* E3 */
            }
        }
        if (!ok) bad += 1;
    }
    return bad;
}

/* float bits helper for tests */
uint32_t pin_bits(float f) { return u_of(f); }
