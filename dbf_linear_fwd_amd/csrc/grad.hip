// Batch reductions of the gradients of the DBF linear layer.
//
// The gradients of the scale vectors (da, dmid, db) are sums over the batch
// rows of elementwise products of two batch x width matrices (the upstream
// gradient and a forward intermediate, or two intermediates).  They are
// formed here in a fixed order, so that repeated calls give identical bits:
// each thread sums kColChunk rows of one column in row order, then the chunk
// partials of a column are added in chunk order.  Reads are coalesced across
// the threads of a wave (consecutive columns).

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "dbf_internal.h"

namespace dbf {
namespace {

constexpr int kThreads = 256;

template <bool F32>
__device__ __forceinline__ float load_val(const void *p, size_t i) {
    if constexpr (F32) return static_cast<const float *>(p)[i];
    else return __half2float(static_cast<const __half *>(p)[i]);
}

template <bool PF, bool QF>
__global__ __launch_bounds__(kThreads) void colsum_chunk_kernel(const void *__restrict__ P, int ldp,
                                                                const void *__restrict__ Q, int ldq, int rows,
                                                                int cols, float *__restrict__ partial) {
    const int c = blockIdx.x * kThreads + threadIdx.x;
    const int r0 = blockIdx.y * kColChunk;
    if (c >= cols) return;
    const int r1 = min(rows, r0 + kColChunk);
    float acc = 0.0f;
    for (int r = r0; r < r1; ++r)
        acc += load_val<PF>(P, static_cast<size_t>(r) * ldp + c) * load_val<QF>(Q, static_cast<size_t>(r) * ldq + c);
    partial[static_cast<size_t>(blockIdx.y) * cols + c] = acc;
}

__global__ __launch_bounds__(kThreads) void colsum_finish_kernel(const float *__restrict__ partial, int nchunk,
                                                                 int cols, float *__restrict__ out) {
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c >= cols) return;
    float acc = 0.0f;
    for (int q = 0; q < nchunk; ++q) acc += partial[static_cast<size_t>(q) * cols + c];
    out[c] = acc;
}

template <bool PF, bool QF>
void launch_chunks(const void *P, int ldp, const void *Q, int ldq, int rows, int cols, float *partial, int nchunk,
                   hipStream_t s) {
    launch_kernel((colsum_chunk_kernel<PF, QF>), dim3((cols + kThreads - 1) / kThreads, nchunk), dim3(kThreads), 0, s,
                  P, ldp, Q, ldq, rows, cols, partial);
}

}  // namespace

int launch_colsum_chunks(const void *P, int p_f32, int ldp, const void *Q, int q_f32, int ldq, int rows, int cols,
                         float *partial, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int nchunk = (rows + kColChunk - 1) / kColChunk;
    if (p_f32 && q_f32) launch_chunks<true, true>(P, ldp, Q, ldq, rows, cols, partial, nchunk, s);
    else if (p_f32) launch_chunks<true, false>(P, ldp, Q, ldq, rows, cols, partial, nchunk, s);
    else if (q_f32) launch_chunks<false, true>(P, ldp, Q, ldq, rows, cols, partial, nchunk, s);
    else launch_chunks<false, false>(P, ldp, Q, ldq, rows, cols, partial, nchunk, s);
    return static_cast<int>(hipGetLastError());
}

int launch_colsum_finish(const float *partial, int rows, int cols, float *out, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int nchunk = (rows + kColChunk - 1) / kColChunk;
    launch_kernel(colsum_finish_kernel, dim3((cols + kThreads - 1) / kThreads), dim3(kThreads), 0, s, partial, nchunk,
                  cols, out);
    return static_cast<int>(hipGetLastError());
}

}  // namespace dbf
