// Host check of the table-driven fp64 exp that the bulk FFN quantizer uses for SwiGLU
// (exp_f64_tab in the library's common.hpp) against the host library's exp: prints, for a set
// of special arguments and random ones over the whole domain, the largest error in units of
// the last place and every special case whose result differs in kind (zero, infinity, NaN).
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../bit_gemm_02_amd/csrc/common.hpp"

static double ulps(double got, double want)
{
    if (got == want)
        return 0.0;
    if (!isfinite(want) || want == 0.0)
        return INFINITY;
    return fabs(got - want) / (nextafter(fabs(want), INFINITY) - fabs(want));
}

int main()
{
    double tab[64];
    for (int j = 0; j < 64; ++j)
        tab[j] = exp2(j / 64.0);
    double worst = 0.0, worst_t = 0.0;
    int kind_mismatch = 0;
    const double special[] = {0.0, -0.0, 1e-300, -1e-300, 5e-324, 1e-17, -1e-17, 0.5, -0.5, 1.0,
                              -1.0, 0.0108304, -0.0108304, 0.01083042, 10.0, -10.0, 88.7, -87.3,
                              100.0, -100.0, 700.0, -700.0, 708.39, 709.78, -708.4, -744.4,
                              -745.1, 745.2, 750.0, -750.0, 800.0, -800.0, 1e300, -1e300};
    for (double t : special) {
        const double g = bl::exp_f64_tab(t, tab), w = exp(t);
        const bool same_kind = (isinf(g) == isinf(w)) && ((g == 0.0) == (w == 0.0));
        if (!same_kind) {
            ++kind_mismatch;
            printf("kind t=%.17g got=%.17g want=%.17g\n", t, g, w);
        } else if (isfinite(w) && w >= 2.2250738585072014e-308) {   // normal results
            const double u = ulps(g, w);
            if (u > worst) { worst = u; worst_t = t; }
        }
    }
    if (!isnan(bl::exp_f64_tab(NAN, tab))) {
        ++kind_mismatch;
        printf("kind t=nan not NaN\n");
    }
    uint64_t s = 0x9E3779B97F4A7C15ull;
    for (int i = 0; i < 2000000; ++i) {
        s ^= s << 13; s ^= s >> 7; s ^= s << 17;
        const double t = -708.0 + 1417.0 * ((double)(s >> 11) / 9007199254740992.0);
        const double u = ulps(bl::exp_f64_tab(t, tab), exp(t));
        if (u > worst) { worst = u; worst_t = t; }
    }
    printf("max_ulps %.3f at %.17g\nkind_mismatches %d\n", worst, worst_t, kind_mismatch);
    return 0;
}
