// Per-row statistics of the input for the forward of a binary-quadratic
// (BQQ-form) weight matrix.
//
// The TL;DR of "Binary Quadratic Quantization: Beyond First-Order
// Quantization for Real-Valued Matrix Compression" writes W as a sum of
// scaled products of 0/1 matrices plus rank-one terms:
//   W = Σ_i ( r_i Y_i Z_i + s_i Y_i 1 + t_i 1 Z_i ) + u 1.
// The products go through the DBF kernels (0/1 flavour); the other terms
// reduce, for an input row x, to E[o] * Σ_l x_l + Σ_l γ_l x_l with
// E[o] = Σ_i s_i (row o of Y_i summed) + u and γ_l = Σ_i t_i (column l of
// Z_i summed), both fixed at pack time.  This kernel forms the two sums per
// row; the products' epilogue adds the term before the one rounding.  With
// group-wise scalars the term has rank p + 1 (Σ_i R_i[o] σ_i + κ, runtime.hip)
// and the second kernel forms its p + 1 weighted sums per row.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "bqq_rowstats.h"
#include "dbf_internal.h"

namespace dbf {
namespace {

constexpr int kStatThreads = 256;

// One workgroup per row of x: stats[2r] = Σ_l x[r][l], stats[2r + 1] =
// Σ_l gamma[l] x[r][l] (bqq_rowstats.h).
__global__ __launch_bounds__(kStatThreads) void bqq_rowstats_kernel(const __half *__restrict__ x, int m,
                                                                    const float *__restrict__ gamma,
                                                                    float *__restrict__ stats) {
    __shared__ float sh[2 * kStatThreads];
    const int r = blockIdx.x;
    bqq_rowstats_row<kStatThreads>(x + static_cast<size_t>(r) * m, m, gamma, stats + 2 * r, sh);
}

// Group-wise form, one workgroup per row of x: stats[r * Q + q] = Σ_l
// w[q * m + l] x[r][l], all Q statistics in one pass over the row.
template <int Q>
__global__ __launch_bounds__(kStatThreads) void bqq_rowstats_q_kernel(const __half *__restrict__ x, int m,
                                                                      const float *__restrict__ w,
                                                                      float *__restrict__ stats) {
    __shared__ float sh[Q * kStatThreads];
    const int r = blockIdx.x;
    bqq_rowstats_dotq<kStatThreads, Q>(x + static_cast<size_t>(r) * m, m, w, stats + static_cast<size_t>(r) * Q, sh);
}

}  // namespace

int launch_bqq_rowstats_q(const void *x, int batch, int m, const float *w, int Q, float *stats, void *stream) {
    if (Q < 1 || Q > kMaxStatQ) return static_cast<int>(hipErrorInvalidValue);
    if (batch <= 0) return 0;
    static void (*const kernels[kMaxStatQ])(const __half *, int, const float *, float *) = {
        bqq_rowstats_q_kernel<1>, bqq_rowstats_q_kernel<2>, bqq_rowstats_q_kernel<3>,
        bqq_rowstats_q_kernel<4>, bqq_rowstats_q_kernel<5>, bqq_rowstats_q_kernel<6>,
        bqq_rowstats_q_kernel<7>, bqq_rowstats_q_kernel<8>, bqq_rowstats_q_kernel<9>};
    static_assert(kMaxStatQ == 9, "one kernel per statistic count");
    launch_kernel(kernels[Q - 1], dim3(batch), dim3(kStatThreads), 0, static_cast<hipStream_t>(stream),
                  static_cast<const __half *>(x), m, w, stats);
    return static_cast<int>(hipGetLastError());
}

int launch_bqq_rowstats(const void *x, int batch, int m, const float *gamma, float *stats, void *stream) {
    if (batch <= 0) return 0;
    launch_kernel(bqq_rowstats_kernel, dim3(batch), dim3(kStatThreads), 0, static_cast<hipStream_t>(stream),
                  static_cast<const __half *>(x), m, gamma, stats);
    return static_cast<int>(hipGetLastError());
}

}  // namespace dbf
