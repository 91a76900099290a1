// Exhaustive check of the division identity the activation-quantization kernels use.
// For a divisor b and y = RN(1/b): q = RN(a*y), r = fma(-q, b, a) (exact), t = fma(r, y, q).
// Markstein's theorem says t = RN(a/b); this program compares t with the IEEE quotient for
// EVERY fp32 a with a/b in [2^-3, 2^8) (the range where rounding 127x/beta to an integer
// can be decided), for the given number of divisors (fixed hard cases, then random).
// Exit status 0 iff there is no mismatch.  Built with -ffp-contract=off -mfma.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <stdlib.h>
static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
int main(int argc, char** argv) {
    int nb = argc > 1 ? atoi(argv[1]) : 16;
    uint64_t bad = 0, tot = 0;
    srand(12345);
    for (int t = 0; t < nb; ++t) {
        float b;
        if (t == 0) b = 1.0f; else if (t == 1) b = f_of(0x3FFFFFFF); else if (t == 2) b = 3.0f;
        else if (t == 3) b = f_of(0x407FFFFF); else b = (float)(0.3 + 60.0 * rand() / (double)RAND_MAX);
        volatile float one = 1.0f;
        float y = one / b;
        // a ranges over binades so that a/b in [2^-3, 2^8)
        float lo = b * 0.125f, hi = b * 256.0f;
        for (uint32_t u = u_of(lo); u <= u_of(hi); ++u) {
            float a = f_of(u);
            float q = a * y;
            float r = fmaf(-q, b, a);
            float q2 = fmaf(r, y, q);
            volatile float ref = a / b;
            if (u_of(q2) != u_of(ref)) { if (bad < 10) printf("MISMATCH b=%a a=%a q2=%a ref=%a\n", b, a, q2, ref); ++bad; }
            ++tot;
        }
    }
    printf("checked %llu quotients over %d divisors: %llu mismatches\n", (unsigned long long)tot, nb, (unsigned long long)bad);
    return bad != 0;
}
