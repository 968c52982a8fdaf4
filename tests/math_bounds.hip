// Host evaluation of the library's fp64 math (the same source the kernels
// inline) against long double references, over seeded samples that span
// every float exponent, the subnormals and the edges of each function's
// range.  Prints one JSON object of worst errors; tests/test_math_bounds.py
// compiles and runs it on the CPU and checks the bounds.
//
//   log2_sig32   error of log2(x) relative to max(1, |log2 x|), x from a
//                float or a uint32
//   exp2_tab     relative error of 2^y (normal results), and the absolute
//                error in units of DBL_MIN where the result is subnormal
//   pow_prio     relative error of p^alpha, the general path (any alpha > 0)
//   pow_prio_fast  the per-workgroup-table path (alpha <= 16); outside the
//                normal range: the absolute error in units of DBL_MIN below
//                it, and above it 0 for +inf, else the relative error
//   exp_row      relative error of e^x, x <= 0 (the row resampler's exp)
#include <cfloat>
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "psamp_device.h"
#include "resample_row.h"

using namespace psamp;

namespace {

// splitmix64: a fixed, seeded stream of 64-bit words
struct Rng {
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    double unit() { return (double)(next() >> 11) * 0x1p-53; }
};

// a positive finite float with a uniformly drawn bit pattern below +inf:
// every exponent (subnormals included) is equally likely
float any_pos_float(Rng& g) {
    for (;;) {
        const uint32_t b = (uint32_t)(g.next() >> 33);     // [0, 2^31)
        if (b != 0 && b < 0x7F800000u) {
            float f;
            std::memcpy(&f, &b, 4);
            return f;
        }
    }
}

long double rel(long double got, long double ref) { return fabsl(got - ref) / fabsl(ref); }

struct Worst {
    long double err = 0;
    double at = 0, at2 = 0;
    long n = 0;
    void add(long double e, double x, double x2 = 0) {
        ++n;
        if (e > err || e != e) {
            err = e;
            at = x;
            at2 = x2;
        }
    }
};

void print(const char* name, const Worst& w, bool last = false) {
    std::printf("  \"%s\": {\"err\": %.6Le, \"at\": %.17g, \"at2\": %.17g, \"n\": %ld}%s\n", name,
                w.err, w.at, w.at2, w.n, last ? "" : ",");
}

}  // namespace

int main(int argc, char** argv) {
    const long N = argc > 1 ? std::atol(argv[1]) : 200000;
    Rng g{0x5EED0001ull};
    static MathLds M;
    math_lds_fill(&M, 0, 1);

    // log2 of doubles converted from floats and from uint32
    Worst lg;
    for (long i = 0; i < N; ++i) {
        const double x = (i & 1) ? (double)any_pos_float(g) : (double)(uint32_t)(g.next() | 1u);
        const long double ref = log2l((long double)x);
        lg.add(fabsl((long double)log2_sig32(x, &M) - ref) / fmaxl(1.0L, fabsl(ref)), x);
    }
    for (uint32_t u = 1; u < 70000; ++u) {        // small integers and the table's edges
        const long double ref = log2l((long double)u);
        lg.add(fabsl((long double)log2_sig32((double)u, &M) - ref) / fmaxl(1.0L, ref), u);
    }

    // 2^y over the whole range, normal and subnormal results apart
    Worst e2, e2s;
    for (long i = 0; i < 2 * N; ++i) {
        double y = -1075.0 + 2099.0 * g.unit();
        if (i % 4 == 1) y = std::nearbyint(y * 64.0) / 64.0 + (g.unit() - 0.5) * 0x1p-20;
        const long double ref = exp2l((long double)y);
        const double r = exp2_tab(y, &M);
        if (ref >= (long double)DBL_MIN && ref <= (long double)DBL_MAX)
            e2.add(rel(r, ref), y);
        else if (ref < (long double)DBL_MIN)
            e2s.add(fabsl((long double)r - ref) / (long double)DBL_MIN, y);
    }

    // p^alpha, the general path and the table path
    const double alphas[] = {0.05, 0.25, 0.4, 0.5, 0.6, 0.7, 1.0, 1.5, 2.0, 3.7, 7.0, 12.5, 16.0};
    Worst pw, pf, pfs;
    static PowLds PL;
    for (double a : alphas) {
        pow_tables_build(&PL, &M, a, 0, 1);
        const PowCoef c = pow_coef(a);
        for (long i = 0; i < N / 4; ++i) {
            const float p = any_pos_float(g);
            const long double ref = powl((long double)p, (long double)a);
            const double f = pow_prio_fast(p, &PL, c);
            if (ref < (long double)DBL_MIN) {            // subnormal or zero results
                pfs.add(fabsl((long double)f - ref) / (long double)DBL_MIN, p, a);
                continue;
            }
            if (ref > (long double)DBL_MAX) {            // +inf, or DBL_MAX within the bound
                pfs.add(f == (double)INFINITY ? 0.0L : rel(f, ref), p, a);
                continue;
            }
            pw.add(rel(pow_prio(p, a, &M), ref), p, a);
            pf.add(rel(f, ref), p, a);
        }
    }

    // p^alpha within a few per cent of DBL_MAX and of DBL_MIN (the table's
    // scaling at both ends)
    for (double a : alphas) {
        pow_tables_build(&PL, &M, a, 0, 1);
        const PowCoef c = pow_coef(a);
        for (int edge = 0; edge < 2; ++edge) {
            const double l2 = edge ? 1024.0 : -1022.0;         // log2 of the edge
            for (long i = 0; i < N / 20; ++i) {
                const double y = (l2 + (g.unit() - 0.5) * 0.2) / a;   // log2 p
                if (y < -149.0 || y >= 128.0) continue;
                const float p = (float)exp2l((long double)y);
                if (!(p > 0.0f) || p == INFINITY) continue;
                const long double ref = powl((long double)p, (long double)a);
                const double f = pow_prio_fast(p, &PL, c);
                if (ref >= (long double)DBL_MIN && ref <= (long double)DBL_MAX)
                    pf.add(rel(f, ref), p, a);
                else if (ref < (long double)DBL_MIN)
                    pfs.add(fabsl((long double)f - ref) / (long double)DBL_MIN, p, a);
                else
                    pfs.add(f == (double)INFINITY ? 0.0L : rel(f, ref), p, a);
            }
        }
    }

    // e^x for x <= 0 (normal results)
    static double etab[256];
    for (int t = 0; t < 256; ++t) etab[t] = exp_row_tab_load(t);
    Worst er, ers;
    for (long i = 0; i < 2 * N; ++i) {
        const double x = (i & 1) ? -745.0 * g.unit() : -40.0 * g.unit() * g.unit();
        const long double ref = expl((long double)x);
        const double r = exp_row(x, etab);
        if (ref >= (long double)DBL_MIN)
            er.add(rel(r, ref), x);
        else
            ers.add(fabsl((long double)r - ref) / (long double)DBL_MIN, x);
    }

    // special values: 1 where every case holds
    const float inf = INFINITY;
    pow_tables_build(&PL, &M, 0.6, 0, 1);
    const PowCoef c6 = pow_coef(0.6);
    int special = 1;
    special &= pow_prio(0.0f, 0.6, &M) == 0.0 && pow_prio_fast(0.0f, &PL, c6) == 0.0;
    special &= pow_prio(inf, 0.6, &M) == (double)inf && pow_prio_fast(inf, &PL, c6) == (double)inf;
    special &= std::isnan(pow_prio(-1.0f, 0.6, &M)) && std::isnan(pow_prio_fast(-1.0f, &PL, c6));
    special &= std::isnan(pow_prio(NAN, 0.6, &M)) && std::isnan(pow_prio_fast(NAN, &PL, c6));
    special &= pow_prio(1.0f, 0.6, &M) == 1.0 && pow_prio_fast(1.0f, &PL, c6) == 1.0;
    special &= exp2_tab(0.0, &M) == 1.0 && exp2_tab(1.0, &M) == 2.0 && exp2_tab(-1.0, &M) == 0.5;
    special &= exp2_tab(1024.0, &M) == (double)inf && exp2_tab(-1076.0, &M) == 0.0;
    special &= std::isnan(exp2_tab(NAN, &M));
    special &= exp_row(0.0, etab) == 1.0 && exp_row(-800.0, etab) == 0.0 &&
               exp_row(-1000.0, etab) == 0.0 && exp_row(-1048576.0, etab) == 0.0;
    special &= std::isnan(exp_row(NAN, etab));

    std::printf("{\n");
    print("log2_sig32", lg);
    print("exp2_tab_rel", e2);
    print("exp2_tab_subnormal_abs", e2s);
    print("pow_prio_rel", pw);
    print("pow_prio_fast_rel", pf);
    print("pow_prio_fast_outside_normal", pfs);
    print("exp_row_rel", er);
    print("exp_row_subnormal_abs", ers);
    std::printf("  \"special\": %d\n}\n", special);
    return 0;
}
