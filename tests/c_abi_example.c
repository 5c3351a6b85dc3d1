/*
 * A plain C program that uses the library through its C ABI only: device
 * memory and a stream from the HIP runtime, products from ddgemm.h and
 * qdgemm.h.  Small integer matrices make every product exact (all partial sums
 * are integers far below 2^53), so the expected results are integer matrix
 * products computed here.  Prints "c abi ok" and exits with 0 when every check
 * passes; 1 on a failed check, 2 on a HIP runtime error.
 */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "ddgemm.h"
#include "qdgemm.h"

#define CHECK_HIP(x)                                                                        \
    do {                                                                                    \
        hipError_t e_ = (x);                                                                \
        if (e_ != hipSuccess) {                                                             \
            fprintf(stderr, "line %d: %s\n", __LINE__, hipGetErrorString(e_));              \
            return 2;                                                                       \
        }                                                                                   \
    } while (0)

#define CHECK(c)                                                                            \
    do {                                                                                    \
        if (!(c)) {                                                                         \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);                 \
            return 1;                                                                       \
        }                                                                                   \
    } while (0)

static int64_t a_val(int64_t i, int64_t p) { return (i * 7 + p * 3) % 19 - 9; }
static int64_t b_val(int64_t p, int64_t j) { return (p * 5 + j * 11) % 23 - 11; }

int main(void) {
    const int64_t m = 37, n = 29, k = 45;
    const size_t na = (size_t)(m * k), nb = (size_t)(k * n), nc = (size_t)(m * n);
    double* hA = malloc(na * sizeof(double));
    double* hB = malloc(nb * sizeof(double));
    double* hC = malloc(4 * nc * sizeof(double));
    int64_t* want = malloc(nc * sizeof(int64_t));
    int64_t i, j, p;
    size_t q;
    CHECK(hA && hB && hC && want);
    for (i = 0; i < m; ++i)
        for (p = 0; p < k; ++p) hA[i * k + p] = (double)a_val(i, p);
    for (p = 0; p < k; ++p)
        for (j = 0; j < n; ++j) hB[p * n + j] = (double)b_val(p, j);
    for (i = 0; i < m; ++i)
        for (j = 0; j < n; ++j) {
            int64_t s = 0;
            for (p = 0; p < k; ++p) s += a_val(i, p) * b_val(p, j);
            want[i * n + j] = s;
        }

    double *dA, *dA_lo, *dB, *dC;
    void* ws;
    hipStream_t stream;
    CHECK_HIP(hipMalloc((void**)&dA, na * sizeof(double)));
    CHECK_HIP(hipMalloc((void**)&dA_lo, na * sizeof(double)));
    CHECK_HIP(hipMalloc((void**)&dB, nb * sizeof(double)));
    CHECK_HIP(hipMalloc((void**)&dC, 4 * nc * sizeof(double)));
    CHECK_HIP(hipStreamCreate(&stream));
    CHECK_HIP(hipMemcpy(dA, hA, na * sizeof(double), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(dA_lo, 0, na * sizeof(double)));
    CHECK_HIP(hipMemcpy(dB, hB, nb * sizeof(double), hipMemcpyHostToDevice));

    /* double-double: the allocating entry point (B's lo plane omitted) */
    CHECK(dd_gemm(m, n, k, dA, dA_lo, k, dB, NULL, n, dC, dC + nc, n, stream) == DDGEMM_SUCCESS);
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(hC, dC, 2 * nc * sizeof(double), hipMemcpyDeviceToHost));
    for (q = 0; q < nc; ++q) CHECK(hC[q] == (double)want[q] && hC[nc + q] == 0.0);

    /* the caller's workspace, nine slices per entry */
    {
        const size_t need = dd_gemm_workspace_size_ns(m, n, k, 9);
        CHECK(need > 0);
        CHECK_HIP(hipMalloc(&ws, need));
        CHECK_HIP(hipMemset(dC, 0xFF, 2 * nc * sizeof(double)));
        CHECK(dd_gemm_ws_ns(m, n, k, 9, dA, NULL, k, dB, NULL, n, dC, dC + nc, n, ws, need, stream) ==
              DDGEMM_SUCCESS);
        CHECK_HIP(hipStreamSynchronize(stream));
        CHECK_HIP(hipMemcpy(hC, dC, 2 * nc * sizeof(double), hipMemcpyDeviceToHost));
        for (q = 0; q < nc; ++q) CHECK(hC[q] == (double)want[q] && hC[nc + q] == 0.0);
        CHECK(dd_gemm_ws_ns(m, n, k, 9, dA, NULL, k, dB, NULL, n, dC, dC + nc, n, ws, need - 1, stream) ==
              DDGEMM_ERROR_WORKSPACE);
        CHECK_HIP(hipFree(ws));
    }

    /* quad-double: one component given, the other three NULL */
    {
        const double* A4[4] = {dA, NULL, NULL, NULL};
        const double* B4[4] = {dB, NULL, NULL, NULL};
        double* C4[4] = {dC, dC + nc, dC + 2 * nc, dC + 3 * nc};
        CHECK(qd_gemm(m, n, k, A4, k, B4, n, C4, n, stream) == DDGEMM_SUCCESS);
        CHECK_HIP(hipStreamSynchronize(stream));
        CHECK_HIP(hipMemcpy(hC, dC, 4 * nc * sizeof(double), hipMemcpyDeviceToHost));
        for (q = 0; q < nc; ++q)
            CHECK(hC[q] == (double)want[q] && hC[nc + q] == 0.0 && hC[2 * nc + q] == 0.0 && hC[3 * nc + q] == 0.0);
    }

    /* argument errors come back as status codes, before anything is enqueued */
    CHECK(dd_gemm(m, n, k, dA, NULL, k - 1, dB, NULL, n, dC, dC + nc, n, stream) == DDGEMM_ERROR_INVALID_VALUE);
    CHECK(dd_gemm(m, n, k, dA, NULL, k, dB, NULL, n, dA, dC + nc, n, stream) == DDGEMM_ERROR_INVALID_VALUE);
    CHECK(ddgemm_status_string(DDGEMM_ERROR_INVALID_VALUE) != NULL);

    CHECK_HIP(hipStreamDestroy(stream));
    CHECK_HIP(hipFree(dA));
    CHECK_HIP(hipFree(dA_lo));
    CHECK_HIP(hipFree(dB));
    CHECK_HIP(hipFree(dC));
    free(hA);
    free(hB);
    free(hC);
    free(want);
    printf("c abi ok\n");
    return 0;
}
