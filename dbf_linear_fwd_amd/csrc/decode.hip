// Decode path (batch <= 16) of the DBF linear forward.
//
// §2.1 of the gist.science technical summary of "Addition is almost all you
// need" evaluates X W^T as ((((X ⊙ bᵀ) Bᵀ) ⊙ midᵀ) Aᵀ) ⊙ aᵀ: every product with
// a sign matrix is a sum of activations with their signs flipped where the
// sign is -1.  Here both signed sums run on the vector ALUs in fp32:
//   stage 1: t[r][j] = sum_l B[j][l] * (x[r][l] * b[l])        (j < k)
//   stage 2: s[r][i] = sum_j A[i][j] * (t[r][j] * mid[j])      (i < n)
//   final:   y[r][i] = rne16(s[r][i] * a[i])
// Each stage splits its reduction dimension into chunks of 1024 elements, one
// workgroup per (64-row tile, chunk); partial sums go to the workspace and
// are added in a fixed chunk order, so results are deterministic.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "dbf_internal.h"

namespace dbf {
namespace {

constexpr int kMaxB = kDecodeMaxBatch;
constexpr int kChunkElems = kChunkWords * 32;

// Element index (0..31) inside a 32-element block held by device bit q.
__device__ __forceinline__ int element_of_bit(int q) { return q < 16 ? 2 * q : 2 * (q - 16) + 1; }

__global__ __launch_bounds__(64) void decode_stage1_kernel(const uint32_t *__restrict__ Bt,
                                                           const __half *__restrict__ x,
                                                           const __half *__restrict__ b,
                                                           float *__restrict__ tpart, int batch, int m,
                                                           int Wm, int k_pad) {
    __shared__ float u[kMaxB * kChunkElems];
    const int c = blockIdx.y;
    const int w0 = c * kChunkWords;
    const int w1 = min(w0 + kChunkWords, Wm);
    const int ncols = (w1 - w0) * 32;
    for (int idx = threadIdx.x; idx < batch * ncols; idx += blockDim.x) {
        const int r = idx / ncols;
        const int e = idx - r * ncols;
        const int l = w0 * 32 + e;
        u[r * kChunkElems + e] =
            l < m ? __half2float(x[static_cast<size_t>(r) * m + l]) * __half2float(b[l]) : 0.0f;
    }
    __syncthreads();

    const int j = blockIdx.x * 64 + threadIdx.x;
    float acc[kMaxB];
#pragma unroll
    for (int r = 0; r < kMaxB; ++r) acc[r] = 0.0f;
    for (int w = w0; w < w1; ++w) {
        const uint32_t word = Bt[tiled_index(j, w, Wm)];
        const int base = (w - w0) * 32;
        for (int q = 0; q < 32; ++q) {
            const bool neg = (word >> q) & 1u;
            const int e = base + element_of_bit(q);
#pragma unroll
            for (int r = 0; r < kMaxB; ++r) {
                if (r < batch) {
                    const float v = u[r * kChunkElems + e];
                    acc[r] += neg ? -v : v;
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < kMaxB; ++r) {
        if (r < batch) tpart[(static_cast<size_t>(c) * batch + r) * k_pad + j] = acc[r];
    }
}

__global__ __launch_bounds__(64) void decode_stage2_kernel(const uint32_t *__restrict__ At,
                                                           const float *__restrict__ tpart,
                                                           const __half *__restrict__ mid,
                                                           float *__restrict__ ypart, int batch, int Wk,
                                                           int n_pad, int k_pad, int nchunk_m) {
    __shared__ float v[kMaxB * kChunkElems];
    const int c = blockIdx.y;
    const int w0 = c * kChunkWords;
    const int w1 = min(w0 + kChunkWords, Wk);
    const int ncols = (w1 - w0) * 32;
    for (int idx = threadIdx.x; idx < batch * ncols; idx += blockDim.x) {
        const int r = idx / ncols;
        const int e = idx - r * ncols;
        const int j = w0 * 32 + e;
        float t = 0.0f;
        for (int cm = 0; cm < nchunk_m; ++cm) t += tpart[(static_cast<size_t>(cm) * batch + r) * k_pad + j];
        v[r * kChunkElems + e] = t * __half2float(mid[j]);
    }
    __syncthreads();

    const int i = blockIdx.x * 64 + threadIdx.x;
    float acc[kMaxB];
#pragma unroll
    for (int r = 0; r < kMaxB; ++r) acc[r] = 0.0f;
    for (int w = w0; w < w1; ++w) {
        const uint32_t word = At[tiled_index(i, w, Wk)];
        const int base = (w - w0) * 32;
        for (int q = 0; q < 32; ++q) {
            const bool neg = (word >> q) & 1u;
            const int e = base + element_of_bit(q);
#pragma unroll
            for (int r = 0; r < kMaxB; ++r) {
                if (r < batch) {
                    const float s = v[r * kChunkElems + e];
                    acc[r] += neg ? -s : s;
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < kMaxB; ++r) {
        if (r < batch) ypart[(static_cast<size_t>(c) * batch + r) * n_pad + i] = acc[r];
    }
}

__global__ __launch_bounds__(256) void decode_final_kernel(const float *__restrict__ ypart,
                                                           const __half *__restrict__ a,
                                                           __half *__restrict__ y, int batch, int n,
                                                           int n_pad, int nchunk_k) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= batch * n) return;
    const int r = idx / n;
    const int i = idx - r * n;
    float s = 0.0f;
    for (int c = 0; c < nchunk_k; ++c) s += ypart[(static_cast<size_t>(c) * batch + r) * n_pad + i];
    y[idx] = __float2half_rn(s * __half2float(a[i]));
}

}  // namespace

int launch_decode_stage1(const uint32_t *B_dev, const void *x, const void *b_dev, float *tpart, int batch,
                         int m, int m_pad, int k_pad, int nchunk_m, void *stream) {
    dim3 grid(k_pad / 64, nchunk_m);
    hipLaunchKernelGGL(decode_stage1_kernel, grid, dim3(64), 0, static_cast<hipStream_t>(stream), B_dev,
                       static_cast<const __half *>(x), static_cast<const __half *>(b_dev), tpart, batch, m,
                       m_pad / 32, k_pad);
    return static_cast<int>(hipGetLastError());
}

int launch_decode_stage2(const uint32_t *A_dev, const float *tpart, const void *mid_dev, float *ypart,
                         int batch, int n_pad, int k_pad, int nchunk_m, int nchunk_k, void *stream) {
    dim3 grid(n_pad / 64, nchunk_k);
    hipLaunchKernelGGL(decode_stage2_kernel, grid, dim3(64), 0, static_cast<hipStream_t>(stream), A_dev,
                       tpart, static_cast<const __half *>(mid_dev), ypart, batch, k_pad / 32, n_pad, k_pad,
                       nchunk_m);
    return static_cast<int>(hipGetLastError());
}

int launch_decode_final(const float *ypart, const void *a_dev, void *y, int batch, int n, int n_pad,
                        int nchunk_k, void *stream) {
    const int total = batch * n;
    dim3 grid((total + 255) / 256);
    hipLaunchKernelGGL(decode_final_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), ypart,
                       static_cast<const __half *>(a_dev), static_cast<__half *>(y), batch, n, n_pad,
                       nchunk_k);
    return static_cast<int>(hipGetLastError());
}

}  // namespace dbf
