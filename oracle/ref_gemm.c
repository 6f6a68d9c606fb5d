/*
 * CPU ORACLE for the dense matrix product -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this file's library.  The GPU library never links, loads or calls it,
 * and it shares no code, header, table or constant with the GPU path.
 *
 * What it computes is the plain definition of C = A @ B from the roofline and
 * tiling notes ("Week-4 notes: Roofline and Tiling", section 1 and section 5.2):
 * every output C[i][j] is the sum over k of A[i][k] * B[k][j], which costs
 * 2*M*N*K floating point operations.  The tiled kernels on the Triton matmul
 * pages accumulate that sum in fp32 ("(1/n) ... persistent kernel", naive tiled
 * matmul listing); the oracle accumulates it in fp64, in ascending k, one term at
 * a time, and also returns S[i][j] = sum_k |A[i][k] * B[k][j]|, the scale used
 * by the acceptance bound.
 *
 * Inputs are the raw 16-bit patterns of IEEE binary16 (dtype 1) or bfloat16
 * (dtype 2) values.  They are decoded here, from the sign / exponent / mantissa
 * fields, into exact fp64 values; every product of two such values is exact in
 * fp64, so the only error of the oracle is fp64 summation (at most
 * K * 2^-53 * S).
 *
 * Element (i, k) of A is A[i*s_am + k*s_ak]; element (k, j) of B is
 * B[k*s_bk + j*s_bn]; strides are in elements, as in the pages' kernels.
 *
 * Build:  gcc -O2 -fopenmp -shared -fPIC ref_gemm.c -o libtsoracle.so -lm
 * (no fast-math: the summation order above must be kept).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F16 1
#define ORACLE_BF16 2

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits. */
static double decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)mant, -24);               /* subnormal: mant * 2^-24 */
    } else if (expo == 31) {
        v = mant ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + mant), expo - 25); /* (1 + mant/2^10) * 2^(expo-15) */
    }
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 mantissa bits. */
static double decode_bf16(uint16_t b) {
    int sign = (b >> 15) & 1;
    int expo = (b >> 7) & 0xff;
    int mant = b & 0x7f;
    double v;
    if (expo == 0) {
        v = ldexp((double)mant, -133);              /* subnormal: mant * 2^-133 */
    } else if (expo == 255) {
        v = mant ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + mant), expo - 134); /* (1 + mant/2^7) * 2^(expo-127) */
    }
    return sign ? -v : v;
}

static double decode(uint16_t bits, int dtype) {
    return dtype == ORACLE_F16 ? decode_f16(bits) : decode_bf16(bits);
}

/* Decode n values; returns 0, or -1 for an unknown dtype. */
int ts_oracle_decode(const uint16_t* in, int64_t n, int dtype, double* out) {
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = decode(in[i], dtype);
    return 0;
}

/* Number of threads the OpenMP runtime would use for a parallel region. */
int ts_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Block of outputs: C[(i-i0)*ldo + (j-j0)] and S[...] for i in [i0,i1), j in [j0,j1).
 * Each C[i][j] is accumulated over k = 0, 1, ..., K-1 in that order.  Rows are
 * independent; with nthreads > 1 they are shared among OpenMP threads, which
 * does not change any element's arithmetic.  K = 0 gives C = 0, S = 0.
 */
int ts_oracle_gemm_block(const uint16_t* A, const uint16_t* B, int dtype,
                         int64_t M, int64_t N, int64_t K,
                         int64_t s_am, int64_t s_ak, int64_t s_bk, int64_t s_bn,
                         int64_t i0, int64_t i1, int64_t j0, int64_t j1,
                         double* C, double* S, int64_t ldo, int nthreads) {
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    if (M < 0 || N < 0 || K < 0 || i0 < 0 || j0 < 0 || i1 > M || j1 > N) return -2;
    if (i1 <= i0 || j1 <= j0) return 0;
    /* every 16-bit pattern decoded once, so that a term costs a table lookup */
    double* table = (double*)malloc(65536 * sizeof(double));
    if (!table) return -3;
    for (int v = 0; v < 65536; ++v) table[v] = decode((uint16_t)v, dtype);
    const int64_t rows = i1 - i0, cols = j1 - j0;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t i = i0 + r;
        double* c = C + r * ldo;
        double* s = S + r * ldo;
        for (int64_t c0 = 0; c0 < cols; ++c0) { c[c0] = 0.0; s[c0] = 0.0; }
        for (int64_t k = 0; k < K; ++k) {
            const double a = table[A[i * s_am + k * s_ak]];
            const uint16_t* brow = B + k * s_bk;
            for (int64_t c0 = 0; c0 < cols; ++c0) {
                const double p = a * table[brow[(j0 + c0) * s_bn]];
                c[c0] += p;
                s[c0] += fabs(p);
            }
        }
    }
    free(table);
    return 0;
}

/*
 * Scattered outputs: for p in [0, npts), C[p] = sum_k A[ii[p]][k] * B[k][jj[p]]
 * (ascending k) and S[p] = sum_k |A[ii[p]][k] * B[k][jj[p]]|.
 */
int ts_oracle_gemm_points(const uint16_t* A, const uint16_t* B, int dtype,
                          int64_t M, int64_t N, int64_t K,
                          int64_t s_am, int64_t s_ak, int64_t s_bk, int64_t s_bn,
                          const int64_t* ii, const int64_t* jj, int64_t npts,
                          double* C, double* S, int nthreads) {
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    if (M < 0 || N < 0 || K < 0) return -2;
    for (int64_t p = 0; p < npts; ++p)
        if (ii[p] < 0 || ii[p] >= M || jj[p] < 0 || jj[p] >= N) return -2;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
    for (int64_t p = 0; p < npts; ++p) {
        const int64_t i = ii[p], j = jj[p];
        double c = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double prod = decode(A[i * s_am + k * s_ak], dtype) *
                                decode(B[k * s_bk + j * s_bn], dtype);
            c += prod;
            s += fabs(prod);
        }
        C[p] = c;
        S[p] = s;
    }
    return 0;
}
