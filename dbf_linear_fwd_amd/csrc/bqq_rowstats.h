// Per-row input sums of the BQQ-form layer (device code, shared by the
// standalone kernel and the decode stage-1 kernel).
//
// For one row x of the input (m fp16 values): sigma = Σ_l x_l and
// kappa = Σ_l gamma_l x_l in fp32.  A workgroup of `threads` threads takes
// 8-element chunks c = tid + threads * q, issuing the loads of up to four
// chunks before adding them, then the threads' partial sums meet in a
// fixed-order tree in LDS: every call gives the same bits.

#ifndef DBF_BQQ_ROWSTATS_H_
#define DBF_BQQ_ROWSTATS_H_

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

namespace dbf {

template <int THREADS>
__device__ __forceinline__ void bqq_rowstats_row(const __half *__restrict__ xr, int m,
                                                 const float *__restrict__ gamma, float *__restrict__ out2,
                                                 float *sh /* LDS, 2 * THREADS floats */) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const int tid = threadIdx.x;
    float s = 0.0f, k = 0.0f;
    if ((m & 7) == 0 && (reinterpret_cast<uintptr_t>(xr) & 15) == 0) {
        const int nch = m >> 3;
        for (int c0 = 0; c0 < nch; c0 += 4 * THREADS) {
            h8 xv[4];
            float4 g0[4], g1[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = min(c0 + tid + THREADS * q, nch - 1);  // past the end: a valid chunk, not added
                xv[q] = *reinterpret_cast<const h8 *>(xr + 8 * c);
                g0[q] = *reinterpret_cast<const float4 *>(gamma + 8 * c);
                g1[q] = *reinterpret_cast<const float4 *>(gamma + 8 * c + 4);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (c0 + tid + THREADS * q < nch) {
                    const float gv[8] = {g0[q].x, g0[q].y, g0[q].z, g0[q].w, g1[q].x, g1[q].y, g1[q].z, g1[q].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float v = static_cast<float>(xv[q][e]);
                        s += v;
                        k += gv[e] * v;
                    }
                }
            }
        }
    } else {
        for (int l = tid; l < m; l += THREADS) {
            const float v = __half2float(xr[l]);
            s += v;
            k += gamma[l] * v;
        }
    }
    sh[tid] = s;
    sh[THREADS + tid] = k;
    __syncthreads();
    for (int w = THREADS / 2; w > 0; w >>= 1) {
        if (tid < w) {
            sh[tid] += sh[tid + w];
            sh[THREADS + tid] += sh[THREADS + tid + w];
        }
        __syncthreads();
    }
    if (tid == 0) {
        out2[0] = sh[0];
        out2[1] = sh[THREADS];
    }
}

// For one row x of the input (m fp16 values): out[0] = Σ_l wa[l] x_l and,
// if wb is not null, out[1] = Σ_l wb[l] x_l, in fp32 (one product and one
// add per term), with the chunking and the fixed-order tree of
// bqq_rowstats_row.
template <int THREADS>
__device__ __forceinline__ void bqq_rowstats_dot2(const __half *__restrict__ xr, int m, const float *__restrict__ wa,
                                                  const float *__restrict__ wb, float *__restrict__ out,
                                                  float *sh /* LDS, 2 * THREADS floats */) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const int tid = threadIdx.x;
    const bool two = wb != nullptr;
    float s = 0.0f, k = 0.0f;
    if ((m & 7) == 0 && (reinterpret_cast<uintptr_t>(xr) & 15) == 0) {
        const int nch = m >> 3;
        for (int c0 = 0; c0 < nch; c0 += 4 * THREADS) {
            h8 xv[4];
            float4 a0[4], a1[4], b0[4], b1[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = min(c0 + tid + THREADS * q, nch - 1);  // past the end: a valid chunk, not added
                xv[q] = *reinterpret_cast<const h8 *>(xr + 8 * c);
                a0[q] = *reinterpret_cast<const float4 *>(wa + 8 * c);
                a1[q] = *reinterpret_cast<const float4 *>(wa + 8 * c + 4);
                if (two) {
                    b0[q] = *reinterpret_cast<const float4 *>(wb + 8 * c);
                    b1[q] = *reinterpret_cast<const float4 *>(wb + 8 * c + 4);
                } else {
                    b0[q] = b1[q] = float4{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (c0 + tid + THREADS * q < nch) {
                    const float av[8] = {a0[q].x, a0[q].y, a0[q].z, a0[q].w, a1[q].x, a1[q].y, a1[q].z, a1[q].w};
                    const float bv[8] = {b0[q].x, b0[q].y, b0[q].z, b0[q].w, b1[q].x, b1[q].y, b1[q].z, b1[q].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float v = static_cast<float>(xv[q][e]);
                        s += av[e] * v;
                        k += bv[e] * v;
                    }
                }
            }
        }
    } else {
        for (int l = tid; l < m; l += THREADS) {
            const float v = __half2float(xr[l]);
            s += wa[l] * v;
            if (two) k += wb[l] * v;
        }
    }
    sh[tid] = s;
    sh[THREADS + tid] = k;
    __syncthreads();
    for (int w = THREADS / 2; w > 0; w >>= 1) {
        if (tid < w) {
            sh[tid] += sh[tid + w];
            sh[THREADS + tid] += sh[THREADS + tid + w];
        }
        __syncthreads();
    }
    if (tid == 0) {
        out[0] = sh[0];
        if (two) out[1] = sh[THREADS];
    }
    __syncthreads();  // sh is reused by the next call
}

}  // namespace dbf

#endif  // DBF_BQQ_ROWSTATS_H_
