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

// For one row x of the input (m fp16 values): out[q] = Σ_l w[q * m + l] x_l
// for q < Q, in fp32 (one product and one add per term), all Q sums in one
// pass over the row: every load of a round (x and the Q weight rows) is
// issued before the first add, so the pass waits on memory once per round.
// The chunking and the fixed-order tree are those of bqq_rowstats_row (one
// tree per statistic).
template <int THREADS, int Q>
__device__ __forceinline__ void bqq_rowstats_dotq(const __half *__restrict__ xr, int m, const float *__restrict__ w,
                                                  float *__restrict__ out, float *sh /* LDS, Q * THREADS floats */) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const int tid = threadIdx.x;
    float acc[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) acc[q] = 0.0f;
    if ((m & 7) == 0 && (reinterpret_cast<uintptr_t>(xr) & 15) == 0) {
        const int nch = m >> 3;
        for (int c0 = 0; c0 < nch; c0 += 2 * THREADS) {
            h8 xv[2];
            float4 a[Q][2][2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int c = min(c0 + tid + THREADS * u, nch - 1);  // past the end: a valid chunk, not added
                xv[u] = *reinterpret_cast<const h8 *>(xr + 8 * c);
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const float *wr = w + static_cast<size_t>(q) * m + 8 * c;
                    a[q][u][0] = *reinterpret_cast<const float4 *>(wr);
                    a[q][u][1] = *reinterpret_cast<const float4 *>(wr + 4);
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (c0 + tid + THREADS * u < nch) {
#pragma unroll
                    for (int q = 0; q < Q; ++q) {
                        const float wv[8] = {a[q][u][0].x, a[q][u][0].y, a[q][u][0].z, a[q][u][0].w,
                                             a[q][u][1].x, a[q][u][1].y, a[q][u][1].z, a[q][u][1].w};
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[q] += wv[e] * static_cast<float>(xv[u][e]);
                    }
                }
            }
        }
    } else {
        for (int l = tid; l < m; l += THREADS) {
            const float v = __half2float(xr[l]);
#pragma unroll
            for (int q = 0; q < Q; ++q) acc[q] += w[static_cast<size_t>(q) * m + l] * v;
        }
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) sh[q * THREADS + tid] = acc[q];
    __syncthreads();
    for (int s = THREADS / 2; s > 0; s >>= 1) {
        if (tid < s) {
#pragma unroll
            for (int q = 0; q < Q; ++q) sh[q * THREADS + tid] += sh[q * THREADS + tid + s];
        }
        __syncthreads();
    }
    if (tid < Q) out[tid] = sh[tid * THREADS];
}

}  // namespace dbf

#endif  // DBF_BQQ_ROWSTATS_H_
