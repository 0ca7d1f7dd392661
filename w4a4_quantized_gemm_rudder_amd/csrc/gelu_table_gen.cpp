// Build-time generator of the GELU table used by the fused up-projection
// epilogue (rudder_linear_gelu_quant, rudder_gelu_bf16).
//
// GELU stays in BF16 between the MLP projections (SteerQuant, paperlayer.ai
// digest, App. D).  Its input there is a bf16 value, so the function is a
// table over the 65536 bf16 bit patterns.  Each entry is the exact (erf)
// form gelu(x) = x * Phi(x) = 0.5 * x * erfc(-x / sqrt 2) evaluated in
// double precision, rounded to fp32 and then to bf16 (round to nearest even
// both times).  erfc is computed here from first principles -- the
// Maclaurin series of erf below 2, the continued fraction of erfc (modified
// Lentz) above -- not by a math library.  Non-finite inputs: NaN -> quiet NaN
// of the same sign, +inf -> +inf, -inf -> -0.
//
// Usage: gelu_table_gen OUT.inc   (writes 65536 comma-separated hex entries)
#include <cstdint>
#include <cstdio>
#include <cstring>

namespace {

const double kSqrtPi = 1.7724538509055160273;
const double kLn2 = 0.69314718055994530942;

// e^y for y <= 0: y = k ln2 + r, |r| <= ln2 / 2, Taylor series of e^r, then
// scaled by 2^k one halving at a time (subnormal results round once, last).
double exp_nonpositive(double y) {
    if (y < -745.0) return 0.0;
    const double kf = y / kLn2;
    long k = (long)(kf < 0 ? kf - 0.5 : kf + 0.5);
    const double r = y - (double)k * kLn2;
    double term = 1.0, sum = 1.0;
    for (int i = 1; i < 30; ++i) {
        term *= r / i;
        sum += term;
    }
    for (; k < 0; ++k) sum *= 0.5;
    return sum;
}

// erf(z), 0 <= z < 2: 2/sqrt(pi) * sum_n (-1)^n z^(2n+1) / (n! (2n+1)).
double erf_series(double z) {
    const double z2 = z * z;
    double term = z, sum = z;
    for (int n = 1; n < 200; ++n) {
        term *= -z2 / n;
        const double t = term / (2 * n + 1);
        sum += t;
        if (t < 1e-30 && t > -1e-30) break;
    }
    return 2.0 / kSqrtPi * sum;
}

// erfc(z), z >= 2: e^(-z^2)/sqrt(pi) / (z + (1/2)/(z + 1/(z + (3/2)/(z + ...)))).
double erfc_fraction(double z) {
    const double tiny = 1e-300;
    double f = z, C = z, D = 0.0;
    for (int n = 1; n < 5000; ++n) {
        const double a = n * 0.5;
        D = z + a * D;
        if (D < tiny && D > -tiny) D = tiny;
        C = z + a / C;
        if (C < tiny && C > -tiny) C = tiny;
        D = 1.0 / D;
        const double delta = C * D;
        f *= delta;
        const double d1 = delta - 1.0;
        if (d1 < 1e-17 && d1 > -1e-17) break;
    }
    return exp_nonpositive(-z * z) / kSqrtPi / f;
}

double erfc_of(double z) {
    if (z < 0) return 2.0 - erfc_of(-z);
    if (z < 2.0) return 1.0 - erf_series(z);
    return erfc_fraction(z);
}

uint16_t bf16_rne(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

uint16_t gelu_entry(uint16_t h) {
    const uint32_t e = (h >> 7) & 0xFFu;
    const uint16_t sign = h & 0x8000u;
    if (e == 0xFFu) {
        if (h & 0x7Fu) return (uint16_t)(sign | 0x7FC0u);
        return sign ? (uint16_t)0x8000u : (uint16_t)0x7F80u;
    }
    const uint32_t u = (uint32_t)h << 16;
    float xf;
    std::memcpy(&xf, &u, 4);
    const double x = (double)xf;
    const double g = 0.5 * x * erfc_of(-x * 0.70710678118654752440);
    return bf16_rne((float)g);
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 2) {
        std::fprintf(stderr, "usage: %s OUT.inc\n", argv[0]);
        return 2;
    }
    FILE* f = std::fopen(argv[1], "w");
    if (!f) return 1;
    for (int i = 0; i < 65536; ++i)
        std::fprintf(f, "0x%04x,%s", gelu_entry((uint16_t)i), (i % 16 == 15) ? "\n" : "");
    return std::fclose(f) == 0 ? 0 : 1;
}
