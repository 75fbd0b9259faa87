/*
 * The oracle's C code run under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_host_sanitizers.py): every entry point on small rows of every
 * storage type, ragged widths, one row and no rows, and the argument errors.
 * Any out-of-bounds access, overflow or other undefined behaviour the
 * sanitizers see ends the run with an error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../oracle/oracle.c"

static uint64_t state = 0x9E3779B97F4A7C15ull;

/* splitmix64: test inputs only */
static uint64_t next_u64(void)
{
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* finite values of moderate size in each storage type */
static void fill(int dtype, void *p, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        uint64_t r = next_u64();
        if (dtype == OR_F32) {
            ((float *)p)[i] = (float)((double)(r >> 11) / 9007199254740992.0 * 8.0 - 4.0);
        } else if (dtype == OR_F16) {
            /* sign, exponent 10..17 (values 2^-5 .. 4), random mantissa */
            ((uint16_t *)p)[i] = (uint16_t)(((r & 1) << 15) | ((10 + (r >> 1) % 8) << 10) | ((r >> 8) & 0x3ff));
        } else {
            /* bf16: exponent 122..129 */
            ((uint16_t *)p)[i] = (uint16_t)(((r & 1) << 15) | ((122 + (r >> 1) % 8) << 7) | ((r >> 8) & 0x7f));
        }
    }
}

int main(void)
{
    const int64_t Ns[] = {1, 2, 3, 7, 8, 64, 65, 257, 781};
    const int64_t Ms[] = {0, 1, 3};
    int bad = 0;
    for (int dtype = 0; dtype < 3; ++dtype) {
        const size_t e = dtype == OR_F32 ? 4 : 2;
        for (size_t a = 0; a < sizeof Ms / sizeof Ms[0]; ++a)
            for (size_t b = 0; b < sizeof Ns / sizeof Ns[0]; ++b) {
                const int64_t M = Ms[a], N = Ns[b], n = M * N;
                void *x = malloc((size_t)(n ? n : 1) * e), *r = malloc((size_t)(n ? n : 1) * e);
                void *g = malloc((size_t)N * e), *bb = malloc((size_t)N * e);
                double *y = malloc((size_t)(n ? n : 1) * sizeof(double));
                double *mu = malloc((size_t)(M ? M : 1) * sizeof(double));
                double *rs = malloc((size_t)(M ? M : 1) * sizeof(double));
                fill(dtype, x, n);
                fill(dtype, r, n);
                fill(dtype, g, N);
                fill(dtype, bb, N);
                bad |= or_decode(n, dtype, x, y);
                bad |= or_softmax(M, N, dtype, x, y);
                bad |= or_layernorm(M, N, dtype, 1e-5f, x, g, bb, y, mu, rs);
                bad |= or_layernorm(M, N, dtype, 1e-5f, x, NULL, NULL, y, NULL, NULL);
                bad |= or_rmsnorm(M, N, dtype, 1e-6f, x, g, y);
                bad |= or_rmsnorm(M, N, dtype, 1e-6f, x, NULL, y);
                bad |= or_add(n, dtype, x, r, y);
                bad |= or_softmax_causal(M, N, dtype, 0.125f, 2, 1, x, y);
                for (int64_t blk = 1; blk <= N; blk *= 4) bad |= or_softmax_online(M, N, dtype, blk, x, y);
                free(x); free(r); free(g); free(bb); free(y); free(mu); free(rs);
            }
    }
    /* argument errors */
    double d;
    float f = 0.f;
    if (or_softmax(-1, 4, OR_F32, &f, &d) == 0 || or_softmax(1, 0, OR_F32, &f, &d) == 0 ||
        or_softmax(1, 1, 7, &f, &d) == 0 || or_softmax_online(1, 1, OR_F32, 0, &f, &d) == 0 ||
        or_softmax_causal(1, 1, OR_F32, 1.f, 0, 0, &f, &d) == 0 || or_decode(-1, OR_F32, &f, &d) == 0) {
        fprintf(stderr, "an argument error was accepted\n");
        return 1;
    }
    if (bad) {
        fprintf(stderr, "an oracle call failed on valid arguments\n");
        return 1;
    }
    printf("ok\n");
    return 0;
}
