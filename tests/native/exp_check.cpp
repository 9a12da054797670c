// Accuracy check of the sampling kernels' fp64 exponential (exp_f64.h),
// compiled for the host: errors in units in the last place against the
// x87 extended-precision expl (64-bit significand, so its own error is far
// below a double's ulp), over the arguments the masses use (z - max z <= 0)
// and the whole finite range, plus the special values. Prints one
// "key value" line per figure.
#define PKV_HOST_DEVICE
#include "exp_f64.h"

#include <cfloat>
#include <cmath>
#include <cstdio>
#include <random>

static double worst = 0.0, worst_x = 0.0;
static long count = 0;

static double worst_np = 0.0;

static double ulp_err(double y, long double ref) {
    const double ulp = std::ldexp(1.0, std::ilogb(static_cast<double>(ref)) - 52);
    return static_cast<double>(fabsl(static_cast<long double>(y) - ref) / ulp);
}

static void check(double x) {
    const double y = pkv::exp_tab(x, pkv::kExp2Frac);
    if (x <= 0.0) {   // the non-positive variant agrees bit for bit where both apply
        const double z = pkv::exp_nonpos(x, pkv::kExp2Frac);
        if (z != y) worst_np = 1e9;
    }
    const long double ref = expl(static_cast<long double>(x));
    if (ref < static_cast<long double>(DBL_MIN) || ref > static_cast<long double>(DBL_MAX)) return;
    const double e = ulp_err(y, ref);
    ++count;
    if (e > worst) {
        worst = e;
        worst_x = x;
    }
}

int main() {
    std::mt19937_64 g(20261202);
    std::uniform_real_distribution<double> masses(-40.0, 0.0), wide(-708.0, 709.7), unit(-1.0, 1.0);
    for (int i = 0; i < 2000000; ++i) check(masses(g));
    for (int i = 0; i < 1000000; ++i) check(wide(g));
    for (int i = 0; i < 200000; ++i) check(unit(g) * 1e-3);
    // either side of the reduction's half-steps, where n changes
    for (int k = -2000; k <= 2000; ++k) {
        const double h = (k + 0.5) * (0.6931471805599453 / 32.0);
        check(h);
        check(std::nextafter(h, 1e9));
        check(std::nextafter(h, -1e9));
    }
    std::printf("checked %ld\n", count);
    std::printf("max_ulp %.4f\n", worst);
    std::printf("max_ulp_at %.17g\n", worst_x);
    const double* t = pkv::kExp2Frac;
    const bool special = pkv::exp_tab(0.0, t) == 1.0 && pkv::exp_tab(-0.0, t) == 1.0 &&
                         std::isnan(pkv::exp_tab(NAN, t)) && pkv::exp_tab(-INFINITY, t) == 0.0 &&
                         pkv::exp_tab(INFINITY, t) == INFINITY && pkv::exp_tab(-746.0, t) == 0.0 &&
                         pkv::exp_tab(709.8001, t) == INFINITY && std::isfinite(pkv::exp_tab(709.78, t)) &&
                         pkv::exp_tab(-745.0, t) > 0.0;
    // the non-positive variant down to the underflow, where exp_tab's select gives 0
    for (double x = -760.0; x <= -700.0; x += 0.0137) {
        const double y = pkv::exp_nonpos(x, t);
        const long double ref = expl(static_cast<long double>(x));
        if (x <= -746.0 ? y != 0.0 : (ref >= static_cast<long double>(DBL_MIN) && ulp_err(y, ref) > 1.5)) worst_np = 1e9;
        if (x > -746.0 && ref < static_cast<long double>(DBL_MIN) &&
            fabsl(static_cast<long double>(y) - ref) > 0x1p-1074L)
            worst_np = 1e9;   // subnormal results within one subnormal step
    }
    const bool special_np = std::isnan(pkv::exp_nonpos(NAN, t)) && pkv::exp_nonpos(-INFINITY, t) == 0.0 &&
                            pkv::exp_nonpos(0.0, t) == 1.0 && pkv::exp_nonpos(-0.0, t) == 1.0;
    std::printf("special %d\n", special && special_np ? 1 : 0);
    std::printf("nonpos_mismatch %d\n", worst_np > 0.0 ? 1 : 0);
    return 0;
}
