/*
 * hr_oracle.c -- CPU oracle for the FP16 all-reduce combine.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the GPU kernels are checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never links, loads or calls it, and it shares no code,
 * header, table or constant with the HIP sources.
 *
 * What it computes.  The 1Cat-vLLM pull request "[Kernel] Two-rank FP16
 * all-reduce through pinned host memory for GPUs without P2P" (section
 * "Purpose") defines the two-rank result as the FP16 sum of both ranks'
 * values with a single FP16 rounding, commutative, so that both ranks hold
 * the same bits.  For G > 2 contributions the pages fix no order; the SGLang
 * pull request "[SM120] Add optional FlashInfer PCIe-IPC all-reduce for
 * switch-free hosts" (section "Accuracy") shows that the accumulation order
 * changes bits.  The reading taken here is a left fold in increasing rank
 * order, rounding to FP16 after every add:
 *
 *     R = fl16( ... fl16( fl16(x0 + x1) + x2 ) ... + x_{G-1} )
 *
 * Each add is done in IEEE binary64.  For two binary16 operands that add is
 * exact: both are integer multiples of 2^-24 with magnitude below 2^16, so
 * the exact sum needs at most 41 significant bits, fewer than binary64's 53.
 * The one rounding is therefore the explicit round-to-nearest-even below.
 *
 * Binary16 layout (IEEE 754-2008): sign bit 15, exponent field bits 14..10
 * (bias 15), fraction bits 9..0.  Exponent field 0 encodes zero and
 * subnormals m * 2^-24; 31 encodes infinity (fraction 0) or NaN.
 *
 * NaN payloads are not specified by the pages or by IEEE 754 for an add; the
 * oracle returns the quiet NaN 0x7E00 and callers compare NaN by class.
 *
 * No FP environment, no _Float16, no intrinsics, no lookup tables: only
 * frexp/ldexp/floor from <math.h>, which are exact operations.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Value of a binary16 bit pattern, exactly, as a double. */
double hro_decode(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int efield = (h >> 10) & 31;
    int frac = h & 1023;
    double mag;
    if (efield == 0) {
        mag = ldexp((double)frac, -24);             /* zero or subnormal */
    } else if (efield == 31) {
        mag = (frac == 0) ? INFINITY : NAN;
    } else {
        mag = ldexp((double)(1024 + frac), efield - 25); /* (1.f) * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

/* Round a non-negative double to an integer, ties to even.  Valid for
 * 0 <= x < 2^52, where x - floor(x) is exact. */
static double round_half_even(double x)
{
    double lo = floor(x);
    double rest = x - lo;
    if (rest > 0.5)
        return lo + 1.0;
    if (rest < 0.5)
        return lo;
    /* exact midpoint: keep the even neighbour */
    return (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;
}

/* Round a double to the nearest binary16, ties to even (IEEE 754 default
 * rounding), with gradual underflow and overflow to infinity. */
uint16_t hro_round(double v)
{
    if (isnan(v))
        return 0x7E00;
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7C00;
    if (a == 0.0)
        return sign;                                  /* keeps -0 */

    if (a < ldexp(1.0, -14)) {
        /* Subnormal range: the result is q * 2^-24 with q in [0, 1024].
         * q == 1024 is the smallest normal 0x0400, which the bit pattern
         * sign | q already spells. */
        double q = round_half_even(ldexp(a, 24));
        return sign | (uint16_t)q;
    }

    /* Normal range: a = f * 2^ex with f in [0.5, 1).  The binary16 exponent
     * field is efield = ex + 14 (value in [2^(efield-15), 2^(efield-14))),
     * and the significand scaled to an integer is f * 2^11 in [1024, 2048). */
    int ex;
    double f = frexp(a, &ex);
    int efield = ex + 14;
    if (efield >= 31)
        return sign | 0x7C00;                         /* a >= 65536 */
    double q = round_half_even(ldexp(f, 11));
    if (q == 2048.0) {                                /* carry into exponent */
        q = 1024.0;
        efield += 1;
        if (efield >= 31)
            return sign | 0x7C00;                     /* 65520 and above */
    }
    return sign | (uint16_t)(efield << 10) | (uint16_t)((int)q - 1024);
}

/* One FP16 add with a single rounding: fl16(a + b). */
uint16_t hro_add(uint16_t a, uint16_t b)
{
    return hro_round(hro_decode(a) + hro_decode(b));
}

/* Elementwise hro_add over arrays of n patterns. */
void hro_add_vec(const uint16_t *a, const uint16_t *b, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = hro_add(a[i], b[i]);
}

void hro_decode_vec(const uint16_t *h, double *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = hro_decode(h[i]);
}

void hro_round_vec(const double *v, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = hro_round(v[i]);
}

/* Left fold of G contributions in rank order 0..G-1, one rounding per add.
 * x[g] points at n binary16 patterns of rank g; out receives n patterns and
 * may alias any x[g] exactly (each element is read before it is written). */
void hro_fold(const uint16_t *const *x, int G, size_t n, uint16_t *out)
{
    for (size_t i = 0; i < n; ++i) {
        uint16_t acc = x[0][i];
        for (int g = 1; g < G; ++g)
            acc = hro_round(hro_decode(acc) + hro_decode(x[g][i]));
        out[i] = acc;
    }
}

/* The same fold with the element range split over nthreads OpenMP threads.
 * Elements are independent, so the result is identical to hro_fold.
 * Returns the number of threads the parallel region actually ran with. */
int hro_fold_threads(const uint16_t *const *x, int G, size_t n, uint16_t *out,
                     int nthreads)
{
    int used = 1;
#ifdef _OPENMP
    #pragma omp parallel num_threads(nthreads)
    {
        #pragma omp single
        used = omp_get_num_threads();
        #pragma omp for schedule(static)
        for (long long i = 0; i < (long long)n; ++i) {
            uint16_t acc = x[0][i];
            for (int g = 1; g < G; ++g)
                acc = hro_round(hro_decode(acc) + hro_decode(x[g][i]));
            out[i] = acc;
        }
    }
#else
    (void)nthreads;
    hro_fold(x, G, n, out);
#endif
    return used;
}

/* ------------------------------------------------------------------ bf16 --
 *
 * The same combine on bfloat16 operands (the SGLang pull request "[SM120]
 * Add optional FlashInfer PCIe-IPC all-reduce for switch-free hosts" runs
 * its reduction in bf16; section "Accuracy").  bfloat16 layout: sign bit 15,
 * exponent field bits 14..7 (bias 127), fraction bits 6..0.  Exponent field
 * 0 encodes zero and subnormals m * 2^-133; 255 encodes infinity (fraction
 * 0) or NaN.
 *
 * Unlike binary16, the binary64 sum of two bfloat16 values is not always
 * exact (their exponents may differ by up to 254).  One rounding to
 * binary64 followed by one rounding to bfloat16 still equals the single
 * correctly rounded bfloat16 sum, because 53 >= 2 * 8 + 2 (Figueroa's
 * double-rounding condition for +, with 8-bit bfloat16 significands).  Sums
 * whose exponents are close enough to matter in the bfloat16 subnormal range
 * are exact in binary64, so gradual underflow is unaffected.
 */

/* Value of a bfloat16 bit pattern, exactly, as a double. */
double hro_decode_bf16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int efield = (h >> 7) & 255;
    int frac = h & 127;
    double mag;
    if (efield == 0) {
        mag = ldexp((double)frac, -133);            /* zero or subnormal */
    } else if (efield == 255) {
        mag = (frac == 0) ? INFINITY : NAN;
    } else {
        mag = ldexp((double)(128 + frac), efield - 134); /* (1.f) * 2^(e-127) */
    }
    return sign ? -mag : mag;
}

/* Round a double to the nearest bfloat16, ties to even, with gradual
 * underflow and overflow to infinity.  NaN gives the quiet NaN 0x7FC0. */
uint16_t hro_round_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;

    if (a < ldexp(1.0, -126)) {
        /* subnormal range: q * 2^-133, q in [0, 128]; 128 spells the
         * smallest normal 0x0080 */
        double q = round_half_even(ldexp(a, 133));
        return sign | (uint16_t)q;
    }

    /* a = f * 2^ex, f in [0.5, 1): exponent field ex + 126, significand
     * scaled to an integer f * 2^8 in [128, 256) */
    int ex;
    double f = frexp(a, &ex);
    int efield = ex + 126;
    if (efield >= 255)
        return sign | 0x7F80;
    double q = round_half_even(ldexp(f, 8));
    if (q == 256.0) {
        q = 128.0;
        efield += 1;
        if (efield >= 255)
            return sign | 0x7F80;
    }
    return sign | (uint16_t)(efield << 7) | (uint16_t)((int)q - 128);
}

uint16_t hro_add_bf16(uint16_t a, uint16_t b)
{
    return hro_round_bf16(hro_decode_bf16(a) + hro_decode_bf16(b));
}

void hro_add_bf16_vec(const uint16_t *a, const uint16_t *b, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = hro_add_bf16(a[i], b[i]);
}

void hro_decode_bf16_vec(const uint16_t *h, double *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = hro_decode_bf16(h[i]);
}

void hro_round_bf16_vec(const double *v, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = hro_round_bf16(v[i]);
}

/* Left fold of G bfloat16 contributions in rank order, one rounding per add. */
void hro_fold_bf16(const uint16_t *const *x, int G, size_t n, uint16_t *out)
{
    for (size_t i = 0; i < n; ++i) {
        uint16_t acc = x[0][i];
        for (int g = 1; g < G; ++g)
            acc = hro_round_bf16(hro_decode_bf16(acc) + hro_decode_bf16(x[g][i]));
        out[i] = acc;
    }
}
