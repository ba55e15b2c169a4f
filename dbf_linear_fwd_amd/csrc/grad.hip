// Batch sums of the gradients of the DBF linear layer.
//
// The gradients of the scale vectors (da, dmid, db) are sums over the batch
// rows of elementwise products of a product's result with another batch x
// width matrix (the upstream gradient, an intermediate, the input).  The
// product kernels form the sums over each group of 64 rows in their epilogue
// (prefill.hip); this kernel adds the groups of a column in group order, so
// repeated calls give identical bits.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "dbf_internal.h"

namespace dbf {
namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;  // group sums loaded together per thread

__global__ __launch_bounds__(kThreads) void colsum_finish_kernel(const float *__restrict__ partial, int ld,
                                                                 int ngroup, int cols, float *__restrict__ out) {
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c >= cols) return;
    float acc = 0.0f;
    for (int g0 = 0; g0 < ngroup; g0 += kInFlight) {
        float v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            v[u] = g0 + u < ngroup ? partial[static_cast<size_t>(g0 + u) * ld + c] : 0.0f;
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) acc += v[u];  // in group order
    }
    out[c] = acc;
}

}  // namespace

int launch_colsum_finish(const float *partial, int ld, int rows, int cols, float *out, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int ngroup = (rows + kColChunk - 1) / kColChunk;
    launch_kernel(colsum_finish_kernel, dim3((cols + kThreads - 1) / kThreads), dim3(kThreads), 0, s, partial, ld,
                  ngroup, cols, out);
    return static_cast<int>(hipGetLastError());
}

}  // namespace dbf
