// Prefill path (large batch) of the DBF linear forward on the CDNA4 matrix cores.
//
// At large batch both signed sums of §2.1 (gist.science technical summary of
// "Addition is almost all you need") are dense contractions, so they run as
// f16 x f16 -> f32 MFMA products with the sign operand expanded in registers:
//   T = rne16( mid ⊙ (X (B ⊙ bᵀ)ᵀ) )      batch x k   (b folded into the signs:
//                                                       ±b is exact in fp16)
//   Y = rne16( a ⊙ (T Aᵀ) )                 batch x n
// The fp16 rounding of T is the one extra rounding of this path.
//
// A sign word of the device layout holds 32 consecutive elements of a row
// with element 2q at bit q and element 2q+1 at bit 16+q.  A lane that needs
// elements 8g..8g+7 shifts the word once so that the pair (8g+2p, 8g+2p+1)
// sits at bits (15, 31) -- the sign bits of a packed pair of halves -- after
// a further shift by 3-p; the mask is then xor-ed into the scale pair (or
// or-ed into the pattern of +1.0).

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "dbf_internal.h"

namespace dbf {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kSignPair = 0x80008000u;
constexpr uint32_t kOnePair = 0x3C003C00u;  // two fp16 +1.0

// Signs of elements 8g..8g+7 of a 32-element word, times the scale pairs
// `sc` (or +1.0 when HAS_SK is false), as the 8 halves of an MFMA operand.
template <bool HAS_SK>
__device__ __forceinline__ f16x8 expand_signs(uint32_t word, int g, const uint32_t *sc) {
    const uint32_t sh = word << (12 - 4 * g);
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t mask = (sh << (3 - p)) & kSignPair;
        r[p] = HAS_SK ? (sc[p] ^ mask) : (mask | kOnePair);
    }
    return __builtin_bit_cast(f16x8, r);
}

// One workgroup of 4 waves computes a 64 x 64 output tile; each wave a 32 x 32
// quarter as 2 x 2 MFMA 16x16x32 tiles.  One K step is one sign word (32).
template <bool HAS_SK>
__global__ __launch_bounds__(256) void sign_gemm_v1(const __half *__restrict__ P, int ldp, int M, int K,
                                                    const uint32_t *__restrict__ S, int words,
                                                    const __half *__restrict__ sk,
                                                    const __half *__restrict__ sn,
                                                    __half *__restrict__ out, int ldo, int n_out) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int li = lane & 15;
    const int m0 = blockIdx.y * 64 + (wave >> 1) * 32;
    const int n0 = blockIdx.x * 64 + (wave & 1) * 32;

    f32x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint32_t *sk32 = reinterpret_cast<const uint32_t *>(sk);
    for (int w = 0; w < words; ++w) {
        const int kk = w * 32 + 8 * g;  // first of this lane's 8 K indices
        f16x8 af[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row = m0 + t * 16 + li;
            f16x8 v;
            if (row < M && kk + 8 <= K && (ldp & 7) == 0) {
                v = *reinterpret_cast<const f16x8 *>(P + static_cast<size_t>(row) * ldp + kk);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v[e] = (row < M && kk + e < K)
                               ? static_cast<_Float16>(__half2float(P[static_cast<size_t>(row) * ldp + kk + e]))
                               : static_cast<_Float16>(0.0f);
                }
            }
            af[t] = v;
        }
        uint32_t sc[4] = {0u, 0u, 0u, 0u};
        if (HAS_SK) {
#pragma unroll
            for (int p = 0; p < 4; ++p) sc[p] = sk32[(kk >> 1) + p];
        }
        f16x8 bf[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t word = S[tiled_index(n0 + t * 16 + li, w, words)];
            bf[t] = expand_signs<HAS_SK>(word, g, sc);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
    }

    // D layout of the 16x16 MFMA: lane (g, li) holds rows 4g..4g+3 of column li.
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int col = n0 + b * 16 + li;
            if (col >= n_out) continue;
            const float scale = __half2float(sn[col]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + a * 16 + 4 * g + v;
                if (row < M) out[static_cast<size_t>(row) * ldo + col] = __float2half_rn(acc[a][b][v] * scale);
            }
        }
    }
}

}  // namespace

int launch_sign_gemm(const void *P, int ldp, int M, int K, const uint32_t *S, int words, int n_rows_pad,
                     const void *sk, const void *sn, void *out, int ldo, int n_out, void *stream) {
    dim3 grid(n_rows_pad / 64, (M + 63) / 64);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (sk) {
        hipLaunchKernelGGL(sign_gemm_v1<true>, grid, dim3(256), 0, s, static_cast<const __half *>(P), ldp, M, K,
                           S, words, static_cast<const __half *>(sk), static_cast<const __half *>(sn),
                           static_cast<__half *>(out), ldo, n_out);
    } else {
        hipLaunchKernelGGL(sign_gemm_v1<false>, grid, dim3(256), 0, s, static_cast<const __half *>(P), ldp, M,
                           K, S, words, static_cast<const __half *>(nullptr), static_cast<const __half *>(sn),
                           static_cast<__half *>(out), ldo, n_out);
    }
    return static_cast<int>(hipGetLastError());
}

}  // namespace dbf
