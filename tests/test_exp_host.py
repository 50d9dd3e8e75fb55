"""Host-side accuracy of the sampler's table-driven fp64 exp (csrc/sv_math.h).

The same header the gfx950 kernels include is compiled for the host with g++
and compared against the C library's long-double expl over the whole argument
range the sampler uses (x <= 0).  The sampler's decision margins are 1e-12
relative; the bound checked here is 2e-15.
"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "speculative_decoding_verify_04_amd", "csrc")

PROG = r"""
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include "sv_math.h"
int main() {
    double tab[64];
    for (int j = 0; j < 64; ++j) tab[j] = std::exp2(j / 64.0);
    double worst = 0.0, worst_x = 0.0;
    unsigned long long s = 88172645463325252ull;
    for (long i = 0; i < 4000000; ++i) {
        s ^= s << 13; s ^= s >> 7; s ^= s << 17;
        double u = (s >> 11) * (1.0 / 9007199254740992.0);
        double x = (i & 1) ? -745.0 * u : -40.0 * u * u;   // dense near 0 too
        long double ref = expl((long double)x);
        double got = sv::exp_nonpos(x, tab);
        if (ref == 0.0L) { if (got != 0.0) { printf("FAIL nonzero %g\n", x); return 1; } continue; }
        if (ref < 2.2250738585072014e-308L) continue;            // subnormal results
        double rel = (double)fabsl(((long double)got - ref) / ref);
        if (rel > worst) { worst = rel; worst_x = x; }
    }
    if (sv::exp_nonpos(0.0, tab) != 1.0) { printf("FAIL exp(0)\n"); return 1; }
    if (sv::exp_nonpos(-INFINITY, tab) != 0.0) { printf("FAIL exp(-inf)\n"); return 1; }
    if (sv::exp_nonpos(-800.0, tab) != 0.0) { printf("FAIL underflow\n"); return 1; }
    printf("%.3e %.17g\n", worst, worst_x);
    return 0;
}
"""


def test_exp_nonpos_accuracy(tmp_path):
    src = tmp_path / "t.cpp"
    src.write_text(PROG)
    exe = tmp_path / "t"
    subprocess.check_call(["g++", "-O2", "-std=c++17", f"-I{HDR}", str(src), "-o", str(exe)])
    out = subprocess.check_output([str(exe)], text=True).split()
    worst = float(out[0])
    assert worst < 2e-15, out
