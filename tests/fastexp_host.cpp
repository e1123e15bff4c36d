// Host build of the library's fp64 exponential, for a CPU comparison with numpy.
// stdin: one double per line (as %a hex float); stdout: e^x as %a.
#include <cstdio>
#include "fastexp.hpp"

int main() {
    double x;
    while (std::scanf("%la", &x) == 1) std::printf("%a\n", specverify::exp_nonpos_f64(x));
    return 0;
}
