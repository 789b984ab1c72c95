/* Plain fp64 triple-loop contraction for the CPU oracle.
 *
 * Test infrastructure only: nothing in the product path links this file.
 *
 *   y[m][n] = sum over k of w[n][k] * x[m][k]        (all fp64)
 *
 * Loops run in the order m, n, k with one accumulator per output, summed in
 * increasing k.  OpenMP splits the n loop across threads; the order of the
 * sum inside one output does not depend on the thread count.  No blocking,
 * no BLAS, no reassociation (build with -O2 -ffp-contract=off).
 */
#include <stdint.h>

void oracle_contract(const double *w, const double *x, double *y,
                     int64_t m, int64_t n, int64_t k, int nthreads)
{
    for (int64_t i = 0; i < m; ++i) {
#pragma omp parallel for num_threads(nthreads) schedule(static)
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int64_t t = 0; t < k; ++t)
                acc += w[j * k + t] * x[i * k + t];
            y[i * n + j] = acc;
        }
    }
}
