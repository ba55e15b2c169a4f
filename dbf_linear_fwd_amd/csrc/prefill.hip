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
// Both are instances of one kernel, C[M x N] = P[M x K] · S'ᵀ with S' the
// sign rows expanded to ±1 (or ±sk[k]) and a per-column epilogue scale.
// Block tile 128 (M) x 256 (N) x 64 (K), four waves of 64 x 128 each, as
// 2 x 4 tiles of the 32x32x16 f16 MFMA.  The P tile goes through LDS, double
// buffered: the global loads of the next K step are in flight while the
// current one is multiplied.  The signs of a K step are one 8-byte word pair
// per sign row (1 bit per element), loaded straight into registers one step
// ahead and expanded there; each expanded fragment feeds two MFMAs.  Blocks
// are ordered so that the blocks resident on one XCD (blockIdx mod 8) share
// rows of P, which then come from that XCD's L2.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "dbf_internal.h"

namespace dbf {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int LDP = BK + 8;          // LDS row stride of the P tile (halves), padded against bank conflicts
constexpr int kThreads = 256;
constexpr int kXcds = 8;             // MI355X: blocks are dispatched round-robin over 8 XCDs

struct ExpandConsts {
    uint32_t mask, one;
};

// The constants of the sign expansion as register values (see expand()).
// Called once at kernel entry, before any MFMA is issued.
__device__ __forceinline__ ExpandConsts expand_consts() {
    ExpandConsts c;
    asm volatile("s_mov_b32 %0, 0x80008000" : "=s"(c.mask));
    asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(c.one));
    return c;
}

// Halves 8g..8g+7 of a 32-element sign word as MFMA operand: ±sc (scale
// pairs, SCALED) or ±1.0.  Element 2q sits at bit q and element 2q+1 at bit
// 16+q; after one shift by 12-4g the pair (8g+2p, 8g+2p+1) is at bits
// (12+p, 28+p) and a further shift by 3-p puts it on the fp16 sign bits.
template <bool SCALED>
__device__ __forceinline__ f16x8 expand(uint32_t word, int g, const u32x4 &sc, ExpandConsts ec) {
    const uint32_t sh = word << (12 - 4 * g);
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t m = (sh << (3 - p)) & ec.mask;
        r[p] = SCALED ? (sc[p] ^ m) : (m | ec.one);
    }
    return __builtin_bit_cast(f16x8, r);
}

// C = P S'ᵀ (see the file comment).  P: fp16 [M][ldp], K valid columns
// (zero beyond).  S: tiled sign rows, `words` per row, n_rows_pad rows.
// sk: fp16 scale per K (zero-padded to words*32) or unused.  sn: fp16 scale
// per output column.  out: fp16 [M][ldo], columns < n_out written.
// PVEC: rows of P are 16-byte aligned (ldp % 8 == 0).
template <bool HAS_SK, bool PVEC>
__global__ __launch_bounds__(kThreads) void sign_gemm_kernel(const __half *__restrict__ P, int ldp, int M, int K,
                                                             const uint32_t *__restrict__ S, int words,
                                                             int n_rows_pad, const __half *__restrict__ sk,
                                                             const __half *__restrict__ sn,
                                                             __half *__restrict__ out, int ldo, int n_out, int nbm,
                                                             int nbn) {
    __shared__ _Float16 Ps[2][BM * LDP];
    __shared__ uint32_t Ss[2][BK / 2];  // sk of the K step, as half pairs

    const ExpandConsts ec = expand_consts();
    // XCD-aware tile order: the blocks of one XCD take consecutive tiles.
    const int G = nbm * nbn;
    const int b = blockIdx.x;
    const int xcd = b % kXcds, slot = b / kXcds, q = G / kXcds, rem = G % kXcds;
    const int tile = xcd * q + min(xcd, rem) + slot;
    const int bm = tile / nbn, bn = tile - (tile / nbn) * nbn;
    const int m0 = bm * BM, n0 = bn * BN;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, kg = lane >> 5;

    const uint2 *S2 = reinterpret_cast<const uint2 *>(S);
    const int nk = words >> 1;  // K steps of 64 = word pairs

    // sign rows of this lane's four N fragments (clamped: rows past the end
    // are loaded but never written out)
    int srow[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) srow[f] = min(n0 + wn * 128 + f * 32 + l32, n_rows_pad - 1);
    auto load_signs = [&](int kt, uint2 (&w)[4]) {
#pragma unroll
        for (int f = 0; f < 4; ++f)
            w[f] = S2[(static_cast<size_t>(srow[f] >> 6) * (words >> 1) + kt) * 64 + (srow[f] & 63)];
    };

    // P tile of a K step: 128 rows x 64 halves = 1024 items of 8 halves, 4 per thread
    u32x4 pv[4];
    u32x4 skv = {0u, 0u, 0u, 0u};
    auto load_p = [&](int kt) {
        const int k0 = kt * BK;
        const bool full = PVEC && (k0 + BK <= K);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int it = tid + kThreads * i;
            const int row = min(m0 + (it >> 3), M - 1);  // rows past M: loaded, never written out
            const int col = k0 + (it & 7) * 8;
            const __half *src = P + static_cast<size_t>(row) * ldp + col;
            if (full) {
                pv[i] = *reinterpret_cast<const u32x4 *>(src);
            } else {
                f16x8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = col + e < K ? static_cast<_Float16>(__half2float(src[e])) : static_cast<_Float16>(0.0f);
                pv[i] = __builtin_bit_cast(u32x4, v);
            }
        }
        if (HAS_SK && tid < BK / 8) skv = *reinterpret_cast<const u32x4 *>(sk + k0 + tid * 8);
    };
    auto store_p = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int it = tid + kThreads * i;
            *reinterpret_cast<u32x4 *>(&Ps[buf][(it >> 3) * LDP + (it & 7) * 8]) = pv[i];
        }
        if (HAS_SK && tid < BK / 8) *reinterpret_cast<u32x4 *>(&Ss[buf][tid * 4]) = skv;
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.0f;

    float snv[4];  // epilogue column scales, fetched early
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int col = n0 + wn * 128 + f * 32 + l32;
        snv[f] = col < n_out ? __half2float(sn[col]) : 0.0f;
    }

    uint2 wcur[4], wnxt[4];
    load_signs(0, wcur);
    load_p(0);
    store_p(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            load_signs(kt + 1, wnxt);
            load_p(kt + 1);
        }
        const _Float16 *pa = &Ps[buf][(wm * 64 + l32) * LDP + 8 * kg];
#pragma unroll
        for (int s = 0; s < 4; ++s) {  // K sub-steps of 16
            f16x8 a0 = *reinterpret_cast<const f16x8 *>(pa + s * 16);
            f16x8 a1 = *reinterpret_cast<const f16x8 *>(pa + 32 * LDP + s * 16);
            u32x4 sc = {0u, 0u, 0u, 0u};
            if (HAS_SK) sc = *reinterpret_cast<const u32x4 *>(&Ss[buf][s * 8 + 4 * kg]);
            const int g = 2 * (s & 1) + kg;  // which 8 elements of the 32-element word
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const f16x8 bf = expand<HAS_SK>(s < 2 ? wcur[f].x : wcur[f].y, g, sc, ec);
                acc[0][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, bf, acc[0][f], 0, 0, 0);
                acc[1][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, bf, acc[1][f], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) {
            store_p(buf ^ 1);
#pragma unroll
            for (int f = 0; f < 4; ++f) wcur[f] = wnxt[f];
        }
        __syncthreads();
    }

    // epilogue: 32x32 MFMA result register v of a lane holds row
    // 8*(v/4) + 4*(lane/32) + v%4 and column lane%32 of its tile
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int col = n0 + wn * 128 + f * 32 + l32;
            if (col >= n_out) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
                if (row < M) out[static_cast<size_t>(row) * ldo + col] = __float2half_rn(acc[i][f][v] * snv[f]);
            }
        }
    }
}

template <bool HAS_SK, bool PVEC>
void launch(const void *P, int ldp, int M, int K, const uint32_t *S, int words, int n_rows_pad, const void *sk,
            const void *sn, void *out, int ldo, int n_out, hipStream_t s) {
    const int nbm = (M + BM - 1) / BM;
    const int nbn = (n_out + BN - 1) / BN;
    launch_kernel((sign_gemm_kernel<HAS_SK, PVEC>), dim3(nbm * nbn), dim3(kThreads), 0, s,
                       static_cast<const __half *>(P), ldp, M, K, S, words, n_rows_pad,
                       static_cast<const __half *>(sk), static_cast<const __half *>(sn), static_cast<__half *>(out),
                       ldo, n_out, nbm, nbn);
}

}  // namespace

int launch_sign_gemm(const void *P, int ldp, int M, int K, const uint32_t *S, int words, int n_rows_pad,
                     const void *sk, const void *sn, void *out, int ldo, int n_out, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool pvec = (ldp & 7) == 0;
    if (sk) {
        if (pvec) launch<true, true>(P, ldp, M, K, S, words, n_rows_pad, sk, sn, out, ldo, n_out, s);
        else launch<true, false>(P, ldp, M, K, S, words, n_rows_pad, sk, sn, out, ldo, n_out, s);
    } else {
        if (pvec) launch<false, true>(P, ldp, M, K, S, words, n_rows_pad, sk, sn, out, ldo, n_out, s);
        else launch<false, false>(P, ldp, M, K, S, words, n_rows_pad, sk, sn, out, ldo, n_out, s);
    }
    return static_cast<int>(hipGetLastError());
}

}  // namespace dbf
