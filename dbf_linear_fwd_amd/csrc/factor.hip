// DBF factorization on the GPU: W (n x m, fp32) -> a, A, mid, B, b.
//
// The technical summary (gist.science) of "Addition is almost all you need",
// §2.2, names the method's optimizer: alternating minimization of the two
// factors, ADMM for each constrained subproblem, projection onto "sign
// matrix with rank-one scaling" by SVID (OneBit's sign-value-independent
// decomposition), and importance scaling of rows and columns.  Written out:
//   T = diag(d_o) W diag(d_i);  W ~ U V, U = diag(a) A diag(c_u) (n x k),
//   V = diag(c_v) B diag(b) (k x m), mid = c_u ⊙ c_v.
//   Outer iteration: update U with V fixed, then V with U fixed (the same
//   step on the transposed problem T^T ~ V^T U^T).  One step, for
//   min_X ||T' - X F^T||^2 with X (rows x k) scaled-sign and F the other
//   factor (stored rows x k as well: U is n x k, V is kept as V^T, m x k):
//     G = F^T F, rho = rho_rel * trace(G) / k, H = G + rho I,
//     P = T' F (T' = T or T^T), Z = X (feasible), L = 0, inner times:
//       X = (P + rho (Z - L)) H^{-1}
//       Z = SVID(X + L) = sign(X + L) ⊙ sigma u v^T (power method on |X + L|)
//       L = L + X - Z
//   then X := Z.
// Dense products are library GEMMs (rocBLAS, fp32); H^{-1} is formed by the
// Newton-Schulz iteration X <- X (2I - H X) from X = alpha I (GEMMs only;
// alpha from a power-method estimate of H's largest eigenvalue, the step
// count from the resulting bound on the initial error); everything else --
// scaling, the ADMM updates, SVID's power method and sign pattern, the error
// and the output scales -- is in the kernels below, with reductions in a
// fixed order so that a call is reproducible bit for bit.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "dbf.h"
#include "dbf_internal.h"

namespace dbf {
namespace {

constexpr int kT = 256;           // threads of the elementwise and reduction kernels
constexpr int kRedBlocks = 1024;  // blocks of the two-pass reductions

// ---------------------------------------------------------------- elementwise

__global__ __launch_bounds__(kT) void scale_kernel(const float *__restrict__ W, const float *__restrict__ d_o,
                                                   const float *__restrict__ d_i, float *__restrict__ T, int n, int m) {
    const size_t total = static_cast<size_t>(n) * m;
    for (size_t e = blockIdx.x * static_cast<size_t>(kT) + threadIdx.x; e < total; e += static_cast<size_t>(gridDim.x) * kT) {
        const int i = static_cast<int>(e / m), j = static_cast<int>(e - static_cast<size_t>(i) * m);
        float v = W[e];
        if (d_o) v *= d_o[i];
        if (d_i) v *= d_i[j];
        T[e] = v;
    }
}

// R = P + rho (Z - L) (L may be null: zero)
__global__ __launch_bounds__(kT) void combine_kernel(const float *__restrict__ P, const float *__restrict__ Z,
                                                     const float *__restrict__ L, float rho, float *__restrict__ R,
                                                     size_t total) {
    for (size_t e = blockIdx.x * static_cast<size_t>(kT) + threadIdx.x; e < total; e += static_cast<size_t>(gridDim.x) * kT)
        R[e] = P[e] + rho * (Z[e] - (L ? L[e] : 0.0f));
}

// M = X + L
__global__ __launch_bounds__(kT) void add_kernel(const float *__restrict__ X, const float *__restrict__ L,
                                                 float *__restrict__ M, size_t total) {
    for (size_t e = blockIdx.x * static_cast<size_t>(kT) + threadIdx.x; e < total; e += static_cast<size_t>(gridDim.x) * kT)
        M[e] = X[e] + L[e];
}

// H += rho I  and  X0 = alpha I (k x k)
__global__ __launch_bounds__(kT) void diag_kernel(float *__restrict__ H, float rho, float *__restrict__ X0, float alpha,
                                                  int k) {
    const size_t total = static_cast<size_t>(k) * k;
    for (size_t e = blockIdx.x * static_cast<size_t>(kT) + threadIdx.x; e < total; e += static_cast<size_t>(gridDim.x) * kT) {
        const int i = static_cast<int>(e / k), j = static_cast<int>(e - static_cast<size_t>(i) * k);
        if (i == j) H[e] += rho;
        X0[e] = i == j ? alpha : 0.0f;
    }
}

// R = 2I - R (k x k)
__global__ __launch_bounds__(kT) void two_minus_kernel(float *__restrict__ R, int k) {
    const size_t total = static_cast<size_t>(k) * k;
    for (size_t e = blockIdx.x * static_cast<size_t>(kT) + threadIdx.x; e < total; e += static_cast<size_t>(gridDim.x) * kT) {
        const int i = static_cast<int>(e / k), j = static_cast<int>(e - static_cast<size_t>(i) * k);
        R[e] = (i == j ? 2.0f : 0.0f) - R[e];
    }
}

// SVID applied, with the ADMM dual update and the next X step's right-hand
// side fused:  Z = sign(M) ⊙ (sigma u) v^T,  L = M - Z  (= L + X - Z with
// M = X + L),  R = P + rho (Z - L).  sigma u and v come as vectors.
__global__ __launch_bounds__(kT) void svid_apply_kernel(const float *__restrict__ M, const float *__restrict__ su,
                                                        const float *__restrict__ v, const float *__restrict__ P,
                                                        float rho, float *__restrict__ Z, float *__restrict__ L,
                                                        float *__restrict__ R, int rows, int k) {
    const size_t total = static_cast<size_t>(rows) * k;
    for (size_t e = blockIdx.x * static_cast<size_t>(kT) + threadIdx.x; e < total; e += static_cast<size_t>(gridDim.x) * kT) {
        const int i = static_cast<int>(e / k), j = static_cast<int>(e - static_cast<size_t>(i) * k);
        const float mv = M[e];
        const float mag = su[i] * v[j];
        const float z = mv < 0.0f ? -mag : mag;  // sign(0) = +1
        const float l = mv - z;
        Z[e] = z;
        L[e] = l;
        R[e] = P[e] + rho * (z - l);
    }
}

// ---------------------------------------------------------------- reductions (fixed order)

// Block b sums elements b, b + G, b + 2G, ... (G = gridDim.x * kT threads in a
// fixed grid) into part[b]; finish_sum adds the parts in order.
__device__ __forceinline__ float block_sum(float s, float *sh) {
    sh[threadIdx.x] = s;
    __syncthreads();
    for (int w = kT / 2; w > 0; w >>= 1) {
        if (static_cast<int>(threadIdx.x) < w) sh[threadIdx.x] += sh[threadIdx.x + w];
        __syncthreads();
    }
    return sh[0];
}

// part[b] = Σ (T - Q)^2 and part[G + b] = Σ T^2 over this block's elements
__global__ __launch_bounds__(kT) void sqdiff_kernel(const float *__restrict__ T, const float *__restrict__ Q,
                                                    size_t total, float *__restrict__ part) {
    __shared__ float sh[kT];
    float d = 0.0f, t = 0.0f;
    for (size_t e = blockIdx.x * static_cast<size_t>(kT) + threadIdx.x; e < total; e += static_cast<size_t>(gridDim.x) * kT) {
        const float tv = T[e];
        const float dv = tv - Q[e];
        d += dv * dv;
        t += tv * tv;
    }
    const float bd = block_sum(d, sh);
    __syncthreads();
    const float bt = block_sum(t, sh);
    if (threadIdx.x == 0) {
        part[blockIdx.x] = bd;
        part[gridDim.x + blockIdx.x] = bt;
    }
}

// out[0] = sqrt(Σ part[0..G) / Σ part[G..2G)) (one block)
__global__ __launch_bounds__(kT) void rel_err_kernel(const float *__restrict__ part, int G, float *__restrict__ out) {
    __shared__ float sh[kT];
    float d = 0.0f, t = 0.0f;
    for (int b = threadIdx.x; b < G; b += kT) {
        d += part[b];
        t += part[G + b];
    }
    const float sd = block_sum(d, sh);
    __syncthreads();
    const float st = block_sum(t, sh);
    if (threadIdx.x == 0) out[0] = st > 0.0f ? sqrtf(sd / st) : 0.0f;
}

// trace of a k x k matrix (one block)
__global__ __launch_bounds__(kT) void trace_kernel(const float *__restrict__ G, int k, float *__restrict__ out) {
    __shared__ float sh[kT];
    float s = 0.0f;
    for (int i = threadIdx.x; i < k; i += kT) s += G[static_cast<size_t>(i) * k + i];
    const float r = block_sum(s, sh);
    if (threadIdx.x == 0) out[0] = r;
}

// y = op(A) x for a rows x cols row-major A, op = |.| (ABS) or identity,
// one block per output row, x scaled by 1 / xnorm[0] (xnorm may be null).
template <bool ABS>
__global__ __launch_bounds__(kT) void row_matvec_kernel(const float *__restrict__ A, const float *__restrict__ x,
                                                        const float *__restrict__ xnorm, int cols,
                                                        float *__restrict__ y) {
    __shared__ float sh[kT];
    const float *a = A + static_cast<size_t>(blockIdx.x) * cols;
    float s = 0.0f;
    for (int j = threadIdx.x; j < cols; j += kT) s += (ABS ? fabsf(a[j]) : a[j]) * x[j];
    const float r = block_sum(s, sh);
    if (threadIdx.x == 0) y[blockIdx.x] = xnorm ? (xnorm[0] > 0.0f ? r / xnorm[0] : 0.0f) : r;
}

// Column sums y = |A|^T x for a rows x cols row-major A, in two passes:
// block (cb, rb) sums rows [rb * kRows, ...) of columns cb * kT + t into
// part[rb][col]; col_finish adds the row blocks in order and divides by xnorm.
constexpr int kRows = 64;
__global__ __launch_bounds__(kT) void col_matvec_kernel(const float *__restrict__ A, const float *__restrict__ x,
                                                        int rows, int cols, float *__restrict__ part) {
    const int col = blockIdx.x * kT + threadIdx.x;
    const int r0 = blockIdx.y * kRows;
    if (col >= cols) return;
    float s = 0.0f;
    const int r1 = min(rows, r0 + kRows);
    for (int r = r0; r < r1; ++r) s += fabsf(A[static_cast<size_t>(r) * cols + col]) * x[r];
    part[static_cast<size_t>(blockIdx.y) * cols + col] = s;
}
__global__ __launch_bounds__(kT) void col_finish_kernel(const float *__restrict__ part, int nblk, int cols,
                                                        const float *__restrict__ xnorm, float *__restrict__ y) {
    const int col = blockIdx.x * kT + threadIdx.x;
    if (col >= cols) return;
    float s = 0.0f;
    for (int b = 0; b < nblk; ++b) s += part[static_cast<size_t>(b) * cols + col];
    y[col] = xnorm ? (xnorm[0] > 0.0f ? s / xnorm[0] : 0.0f) : s;
}

// dst (cols x rows) = src^T, src rows x cols row-major
__global__ __launch_bounds__(kT) void transpose_kernel(const float *__restrict__ src, int rows, int cols,
                                                       float *__restrict__ dst) {
    const size_t total = static_cast<size_t>(rows) * cols;
    for (size_t e = blockIdx.x * static_cast<size_t>(kT) + threadIdx.x; e < total; e += static_cast<size_t>(gridDim.x) * kT) {
        const int i = static_cast<int>(e / cols), j = static_cast<int>(e - static_cast<size_t>(i) * cols);
        dst[static_cast<size_t>(j) * rows + i] = src[e];
    }
}

// out[0] = ||x|| (one block)
__global__ __launch_bounds__(kT) void norm_kernel(const float *__restrict__ x, int len, float *__restrict__ out) {
    __shared__ float sh[kT];
    float s = 0.0f;
    for (int i = threadIdx.x; i < len; i += kT) s += x[i] * x[i];
    const float r = block_sum(s, sh);
    if (threadIdx.x == 0) out[0] = sqrtf(r);
}

// x[i] = value (fill)
__global__ __launch_bounds__(kT) void fill_kernel(float *__restrict__ x, int len, float value) {
    const int i = blockIdx.x * kT + threadIdx.x;
    if (i < len) x[i] = value;
}

// su = sigma u  from the unnormalized u' (= |M| v) : sigma u = u' exactly
// (sigma = ||u'||, u = u' / sigma); v = v' / ||v'||.  (The power method's
// last half-step leaves u' = |M| v with v normalized.)
__global__ __launch_bounds__(kT) void normalize_kernel(float *__restrict__ v, int len, const float *__restrict__ vnorm) {
    const int i = blockIdx.x * kT + threadIdx.x;
    if (i < len) v[i] = vnorm[0] > 0.0f ? v[i] / vnorm[0] : 0.0f;
}

// ---------------------------------------------------------------- outputs

// A[i][j] = sign(Z[i][j]) (transpose = false) or A[j][i] = sign(Z[i][j])
__global__ __launch_bounds__(kT) void signs_kernel(const float *__restrict__ Z, int rows, int k, bool transpose,
                                                   int8_t *__restrict__ S) {
    const size_t total = static_cast<size_t>(rows) * k;
    for (size_t e = blockIdx.x * static_cast<size_t>(kT) + threadIdx.x; e < total; e += static_cast<size_t>(gridDim.x) * kT) {
        const int i = static_cast<int>(e / k), j = static_cast<int>(e - static_cast<size_t>(i) * k);
        const int8_t sgn = Z[e] < 0.0f ? -1 : 1;
        if (transpose) S[static_cast<size_t>(j) * rows + i] = sgn;
        else S[e] = sgn;
    }
}

// a = su_U / d_o, b = su_V / d_i, mid = v_U ⊙ v_V; a, b divided by their RMS,
// mid multiplied by both; all rounded to fp16 (one block).
__global__ __launch_bounds__(kT) void scales_kernel(const float *__restrict__ suU, const float *__restrict__ vU,
                                                    const float *__restrict__ suV, const float *__restrict__ vV,
                                                    const float *__restrict__ d_o, const float *__restrict__ d_i,
                                                    int n, int m, int k, __half *__restrict__ a,
                                                    __half *__restrict__ mid, __half *__restrict__ b) {
    __shared__ float sh[kT];
    float sa = 0.0f, sb = 0.0f;
    for (int i = threadIdx.x; i < n; i += kT) {
        const float v = d_o ? suU[i] / d_o[i] : suU[i];
        sa += v * v;
    }
    for (int l = threadIdx.x; l < m; l += kT) {
        const float v = d_i ? suV[l] / d_i[l] : suV[l];
        sb += v * v;
    }
    const float ta = block_sum(sa, sh);
    __syncthreads();
    const float tb = block_sum(sb, sh);
    float ra = sqrtf(ta / n), rb = sqrtf(tb / m);
    if (!(ra > 0.0f) || !(rb > 0.0f)) ra = rb = 1.0f;
    for (int i = threadIdx.x; i < n; i += kT) a[i] = __float2half_rn((d_o ? suU[i] / d_o[i] : suU[i]) / ra);
    for (int l = threadIdx.x; l < m; l += kT) b[l] = __float2half_rn((d_i ? suV[l] / d_i[l] : suV[l]) / rb);
    for (int j = threadIdx.x; j < k; j += kT) mid[j] = __float2half_rn(vU[j] * vV[j] * ra * rb);
}

// ---------------------------------------------------------------- host side

unsigned grid_for(size_t total) {
    return static_cast<unsigned>(std::min<size_t>((total + kT - 1) / kT, 8192));
}

struct Buffers {
    std::vector<void *> owned;
    bool ok = true;
    float *alloc(size_t floats) {
        void *p = nullptr;
        if (!ok || hipMalloc(&p, std::max<size_t>(floats, 1) * sizeof(float)) != hipSuccess) {
            ok = false;
            return nullptr;
        }
        owned.push_back(p);
        return static_cast<float *>(p);
    }
    ~Buffers() {
        for (void *p : owned) (void)hipFree(p);
    }
};

struct Ctx {
    rocblas_handle blas = nullptr;
    hipStream_t s = nullptr;
    bool ok = true;
    // row-major C (r x c) = A (r x kk) * B (kk x c); the other forms below
    void gemm_nn(int r, int c, int kk, const float *A, int lda, const float *B, int ldb, float *C, int ldc) {
        const float one = 1.0f, zero = 0.0f;
        // column-major view: C^T (c x r) = B^T (c x kk) * A^T (kk x r)
        if (rocblas_sgemm(blas, rocblas_operation_none, rocblas_operation_none, c, r, kk, &one, B, ldb, A, lda, &zero,
                          C, ldc) != rocblas_status_success)
            ok = false;
    }
    // row-major C (r x c) = A^T * B with A stored kk x r, B stored kk x c
    void gemm_tn(int r, int c, int kk, const float *A, int lda, const float *B, int ldb, float *C, int ldc) {
        const float one = 1.0f, zero = 0.0f;
        // C^T (c x r) = B^T (c x kk) * A (kk x r): column-major B^T is B stored, A is A stored transposed
        if (rocblas_sgemm(blas, rocblas_operation_none, rocblas_operation_transpose, c, r, kk, &one, B, ldb, A, lda,
                          &zero, C, ldc) != rocblas_status_success)
            ok = false;
    }
    // row-major C (r x c) = A * B^T with A stored r x kk, B stored c x kk
    void gemm_nt(int r, int c, int kk, const float *A, int lda, const float *B, int ldb, float *C, int ldc) {
        const float one = 1.0f, zero = 0.0f;
        // C^T (c x r) = B (c x kk) * A^T (kk x r)
        if (rocblas_sgemm(blas, rocblas_operation_transpose, rocblas_operation_none, c, r, kk, &one, B, ldb, A, lda,
                          &zero, C, ldc) != rocblas_status_success)
            ok = false;
    }
};

float read_scalar(const float *d, hipStream_t s, bool &ok) {
    float h = 0.0f;
    if (hipMemcpyAsync(&h, d, sizeof(float), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        ok = false;
    return h;
}

struct StepBufs {
    float *P, *R, *X, *Z, *L, *M;  // rows x k
    float *G, *Hinv, *N1, *N2;     // k x k
    float *su, *v, *part;          // vectors, reduction parts
    float *scal;                   // device scalars
};

// SVID of M (rows x k): su = sigma u, v (power method, `iters` steps from u = 1/sqrt(rows))
void svid_power(Ctx &c, const StepBufs &b, const float *M, int rows, int k, int iters) {
    float *u = b.su;  // u and su share storage: the last step leaves su = |M| v
    hipLaunchKernelGGL(fill_kernel, dim3((rows + kT - 1) / kT), dim3(kT), 0, c.s, u, rows, 1.0f / std::sqrt(float(rows)));
    const int nblk = (rows + kRows - 1) / kRows;
    float *unorm = b.scal + 4;  // ||u|| of the previous step (1 for the start vector)
    hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(kT), 0, c.s, unorm, 1, 1.0f);
    for (int it = 0; it < iters; ++it) {
        // v' = |M|^T (u / ||u||), v = v' / ||v'||
        hipLaunchKernelGGL(col_matvec_kernel, dim3((k + kT - 1) / kT, nblk), dim3(kT), 0, c.s, M, u, rows, k, b.part);
        hipLaunchKernelGGL(col_finish_kernel, dim3((k + kT - 1) / kT), dim3(kT), 0, c.s, b.part, nblk, k, unorm, b.v);
        hipLaunchKernelGGL(norm_kernel, dim3(1), dim3(kT), 0, c.s, b.v, k, b.scal + 5);
        hipLaunchKernelGGL(normalize_kernel, dim3((k + kT - 1) / kT), dim3(kT), 0, c.s, b.v, k, b.scal + 5);
        // u' = |M| v  (sigma u = u' after the last step)
        hipLaunchKernelGGL(row_matvec_kernel<true>, dim3(rows), dim3(kT), 0, c.s, M, b.v, nullptr, k, u);
        hipLaunchKernelGGL(norm_kernel, dim3(1), dim3(kT), 0, c.s, u, rows, unorm);
    }
}

// One ADMM step for the factor X (rows x k) with the other factor F (frows x
// k), T' = T (TRANS false: T is rows x frows) or T^T (TRANS true: T is frows x
// rows).  X is updated in place (becomes the final Z); su / v of its SVID
// are left in b.su / b.v.
void admm_step(Ctx &c, const StepBufs &b, const float *T, bool trans, float *X, const float *F, int rows, int frows,
               int k, float rho_rel, int inner, int power_iters) {
    const size_t rk = static_cast<size_t>(rows) * k;
    // G = F^T F (k x k), P = T' F (rows x k)
    c.gemm_tn(k, k, frows, F, k, F, k, b.G, k);
    if (!trans) c.gemm_nn(rows, k, frows, T, frows, F, k, b.P, k);
    else c.gemm_tn(rows, k, frows, T, rows, F, k, b.P, k);
    // rho from trace(G); alpha from a power-method estimate of lambda_max(G)
    hipLaunchKernelGGL(trace_kernel, dim3(1), dim3(kT), 0, c.s, b.G, k, b.scal);
    {
        float *x = b.v, *y = b.su;  // (both at least k long)
        hipLaunchKernelGGL(fill_kernel, dim3((k + kT - 1) / kT), dim3(kT), 0, c.s, x, k, 1.0f / std::sqrt(float(k)));
        for (int it = 0; it < 16; ++it) {
            hipLaunchKernelGGL(row_matvec_kernel<false>, dim3(k), dim3(kT), 0, c.s, b.G, x, nullptr, k, y);
            hipLaunchKernelGGL(norm_kernel, dim3(1), dim3(kT), 0, c.s, y, k, b.scal + 1);  // ||G x||, ||x|| = 1
            hipLaunchKernelGGL(normalize_kernel, dim3((k + kT - 1) / kT), dim3(kT), 0, c.s, y, k, b.scal + 1);
            std::swap(x, y);
        }
    }
    const float trG = read_scalar(b.scal, c.s, c.ok);
    const float lmax = read_scalar(b.scal + 1, c.s, c.ok);
    const float rho = rho_rel * trG / k;
    // H = G + rho I; Newton-Schulz from alpha I, alpha = 1 / (lambda_max bound + rho): the
    // initial error e0 = 1 - alpha * lambda_min <= 1 - rho / (lmax' + rho), e0^(2^j) < 1e-7
    const float lmax_b = std::min(trG, 1.25f * lmax);  // the power method approaches lambda_max from below
    const float alpha = 1.0f / (lmax_b + rho);
    const double q = rho / (double(lmax_b) + rho);
    int ns = static_cast<int>(std::ceil(std::log2(16.2 / std::max(q, 1e-12)))) + 2;
    ns = std::max(4, std::min(ns, 60));
    hipLaunchKernelGGL(diag_kernel, dim3(grid_for(size_t(k) * k)), dim3(kT), 0, c.s, b.G, rho, b.Hinv, alpha, k);
    for (int j = 0; j < ns; ++j) {
        c.gemm_nn(k, k, k, b.G, k, b.Hinv, k, b.N1, k);               // N1 = H X
        hipLaunchKernelGGL(two_minus_kernel, dim3(grid_for(size_t(k) * k)), dim3(kT), 0, c.s, b.N1, k);
        c.gemm_nn(k, k, k, b.Hinv, k, b.N1, k, b.N2, k);              // X (2I - H X)
        (void)hipMemcpyAsync(b.Hinv, b.N2, sizeof(float) * k * k, hipMemcpyDeviceToDevice, c.s);
    }
    // ADMM: Z = X (feasible), L = 0, R = P + rho Z
    (void)hipMemcpyAsync(b.Z, X, sizeof(float) * rk, hipMemcpyDeviceToDevice, c.s);
    hipLaunchKernelGGL(combine_kernel, dim3(grid_for(rk)), dim3(kT), 0, c.s, b.P, b.Z, nullptr, rho, b.R, rk);
    (void)hipMemsetAsync(b.L, 0, sizeof(float) * rk, c.s);
    for (int i = 0; i < inner; ++i) {
        c.gemm_nn(rows, k, k, b.R, k, b.Hinv, k, b.X, k);            // X = R H^{-1}
        hipLaunchKernelGGL(add_kernel, dim3(grid_for(rk)), dim3(kT), 0, c.s, b.X, b.L, b.M, rk);  // M = X + L
        svid_power(c, b, b.M, rows, k, power_iters);
        hipLaunchKernelGGL(svid_apply_kernel, dim3(grid_for(rk)), dim3(kT), 0, c.s, b.M, b.su, b.v, b.P, rho, b.Z,
                           b.L, b.R, rows, k);
    }
    (void)hipMemcpyAsync(X, b.Z, sizeof(float) * rk, hipMemcpyDeviceToDevice, c.s);
}

}  // namespace
}  // namespace dbf

extern "C" dbf_status_t dbf_factorize(const float *W, int32_t n, int32_t m, int32_t k, const float *U0,
                                      const float *V0, const float *d_out, const float *d_in, float rho_rel,
                                      int32_t outer, int32_t inner, int32_t power_iters, int8_t *A, int8_t *B,
                                      uint16_t *a, uint16_t *mid, uint16_t *b, float *err, hipStream_t stream) {
    using namespace dbf;
    if (!W || !U0 || !V0 || !A || !B || !a || !mid || !b) return DBF_ERR_INVALID_ARG;
    if (n < 1 || m < 1 || k < 1 || outer < 1 || inner < 1 || power_iters < 1 || !(rho_rel > 0.0f))
        return DBF_ERR_INVALID_ARG;
    if (int64_t(n) * m > (int64_t(1) << 31) || int64_t(std::max(n, m)) * k > (int64_t(1) << 31) ||
        int64_t(k) * k > (int64_t(1) << 31))
        return DBF_ERR_SHAPE;
    const int rmax = std::max(n, m);
    Buffers mem;
    float *T = mem.alloc(size_t(n) * m);
    float *Q = mem.alloc(size_t(n) * m);          // U V for the error
    float *U = mem.alloc(size_t(n) * k);
    float *Vt = mem.alloc(size_t(m) * k);         // V^T
    StepBufs sb{};
    sb.P = mem.alloc(size_t(rmax) * k);
    sb.R = mem.alloc(size_t(rmax) * k);
    sb.X = mem.alloc(size_t(rmax) * k);
    sb.Z = mem.alloc(size_t(rmax) * k);
    sb.L = mem.alloc(size_t(rmax) * k);
    sb.M = mem.alloc(size_t(rmax) * k);
    sb.G = mem.alloc(size_t(k) * k);
    sb.Hinv = mem.alloc(size_t(k) * k);
    sb.N1 = mem.alloc(size_t(k) * k);
    sb.N2 = mem.alloc(size_t(k) * k);
    sb.su = mem.alloc(size_t(std::max(rmax, k)));
    sb.v = mem.alloc(size_t(std::max(rmax, k)));
    sb.part = mem.alloc(size_t((rmax + kRows - 1) / kRows) * std::max(rmax, k) + 2 * kRedBlocks);
    sb.scal = mem.alloc(16);
    float *suU = mem.alloc(size_t(n)), *vU = mem.alloc(size_t(k));
    float *suV = mem.alloc(size_t(m)), *vV = mem.alloc(size_t(k));
    if (!mem.ok) return DBF_ERR_OOM;
    Ctx c;
    c.s = stream;
    if (rocblas_create_handle(&c.blas) != rocblas_status_success) return DBF_ERR_HIP;
    if (rocblas_set_stream(c.blas, stream) != rocblas_status_success) c.ok = false;
    hipLaunchKernelGGL(scale_kernel, dim3(grid_for(size_t(n) * m)), dim3(kT), 0, stream, W, d_out, d_in, T, n, m);
    (void)hipMemcpyAsync(U, U0, sizeof(float) * n * k, hipMemcpyDeviceToDevice, stream);
    hipLaunchKernelGGL(transpose_kernel, dim3(grid_for(size_t(k) * m)), dim3(kT), 0, stream, V0, k, m, Vt);
    for (int t = 0; t < outer && c.ok; ++t) {
        admm_step(c, sb, T, false, U, Vt, n, m, k, rho_rel, inner, power_iters);
        (void)hipMemcpyAsync(suU, sb.su, sizeof(float) * n, hipMemcpyDeviceToDevice, stream);
        (void)hipMemcpyAsync(vU, sb.v, sizeof(float) * k, hipMemcpyDeviceToDevice, stream);
        admm_step(c, sb, T, true, Vt, U, m, n, k, rho_rel, inner, power_iters);
        (void)hipMemcpyAsync(suV, sb.su, sizeof(float) * m, hipMemcpyDeviceToDevice, stream);
        (void)hipMemcpyAsync(vV, sb.v, sizeof(float) * k, hipMemcpyDeviceToDevice, stream);
        if (err) {
            c.gemm_nt(n, m, k, U, k, Vt, k, Q, m);   // Q = U V = U (V^T)^T
            hipLaunchKernelGGL(sqdiff_kernel, dim3(kRedBlocks), dim3(kT), 0, stream, T, Q, size_t(n) * m, sb.part);
            hipLaunchKernelGGL(rel_err_kernel, dim3(1), dim3(kT), 0, stream, sb.part, kRedBlocks, err + t);
        }
    }
    hipLaunchKernelGGL(signs_kernel, dim3(grid_for(size_t(n) * k)), dim3(kT), 0, stream, U, n, k, false, A);
    hipLaunchKernelGGL(signs_kernel, dim3(grid_for(size_t(m) * k)), dim3(kT), 0, stream, Vt, m, k, true, B);
    hipLaunchKernelGGL(scales_kernel, dim3(1), dim3(kT), 0, stream, suU, vU, suV, vV, d_out, d_in, n, m, k,
                       reinterpret_cast<__half *>(a), reinterpret_cast<__half *>(mid), reinterpret_cast<__half *>(b));
    const bool launched = hipGetLastError() == hipSuccess;
    const bool synced = hipStreamSynchronize(stream) == hipSuccess;  // before the workspace is freed
    (void)rocblas_destroy_handle(c.blas);
    return (c.ok && launched && synced) ? DBF_OK : DBF_ERR_HIP;
}
