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
// Both are instances of one product, C[M x N] = P[M x K] · S'ᵀ with S' the
// sign rows expanded to ±1 (or ±sk[k]) and a per-column epilogue scale, on
// the 32x32x16 f16 MFMA.  The signs of a K step of 64 are one 8-byte word
// pair per sign row (1 bit per element), expanded in registers right before
// their MFMAs; each expanded fragment feeds every M fragment of its wave.
// Blocks are ordered so that the blocks resident on one XCD (blockIdx mod 8)
// share rows of P, which then come from that XCD's L2.
//
// sign_gemm_dma_kernel (K % 64 == 0, 16-byte aligned rows; the usual case):
// block 128 x 256, eight waves of 64 x 64 (two per SIMD).  The operands of a
// step go from global memory straight into a ring of LDS stages
// (global_load_lds), several steps ahead of the MFMAs.
//
// sign_gemm_kernel (any K, any alignment): block 128 x 256, four waves of
// 64 x 128, P tile staged through registers into a double-buffered LDS tile,
// signs loaded into registers one step ahead.
//
// Split-K: a grid of few tiles (small batch) leaves most CUs idle while each
// workgroup walks the whole K.  Such grids are cut along K into parts that
// run as separate workgroups of the DMA kernel and store unscaled fp32 sums;
// split_finish_kernel adds the parts of each output in part order and
// applies the epilogue.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>

#include "dbf_internal.h"

namespace dbf {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#ifndef DBF_PREFILL_NF
#define DBF_PREFILL_NF 4
#endif
#ifndef DBF_PREFILL_MF
#define DBF_PREFILL_MF 2
#endif
#ifndef DBF_PREFILL_OCC
#define DBF_PREFILL_OCC 1
#endif
constexpr int MF = DBF_PREFILL_MF;   // 32-row M fragments per wave
constexpr int NF = DBF_PREFILL_NF;   // 32-wide N fragments per wave
constexpr int BM = 128, BK = 64;
constexpr int WGM = BM / (32 * MF);  // waves along M
constexpr int WGN = 4 / WGM;         // waves along N
constexpr int BN = 32 * NF * WGN;
constexpr int LDP = BK + 8;          // LDS row stride of the P tile (halves), padded against bank conflicts
constexpr int kThreads = 256;
constexpr int kXcds = 8;             // MI355X: blocks are dispatched round-robin over 8 XCDs

struct ExpandConsts {
    uint32_t mask, one, mask2;
};

// The constants of the sign expansion as register values (see expand()).
// Called once at kernel entry, before any MFMA is issued.
template <bool BIN>
__device__ __forceinline__ ExpandConsts expand_consts() {
    ExpandConsts c;
    asm volatile("s_mov_b32 %0, 0x80008000" : "=s"(c.mask));
    asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(c.one));
    if constexpr (BIN) asm volatile("s_mov_b32 %0, 0x40004000" : "=s"(c.mask2));
    else c.mask2 = 0;
    return c;
}

// Halves 8g..8g+7 of a 32-element sign word as MFMA operand: ±sc (scale
// pairs, SCALED) or ±1.0.  Element 2q sits at bit q and element 2q+1 at bit
// 16+q; after one shift by 12-4g the pair (8g+2p, 8g+2p+1) is at bits
// (12+p, 28+p) and a further shift by 3-p puts it on the fp16 sign bits.
// BIN: the word is a row of a 0/1 matrix and the operand is {0, 2.0}: the
// pair one bit lower, on the top exponent bit of each fp16 (0x4000 = 2.0);
// the factor 2 is folded into the scales.
template <bool SCALED, bool BIN>
__device__ __forceinline__ f16x8 expand(uint32_t word, int g, const u32x4 &sc, ExpandConsts ec) {
    const uint32_t sh = word << (12 - 4 * g);
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        if constexpr (BIN) {
            r[p] = (p < 3 ? sh << (2 - p) : sh >> 1) & ec.mask2;
        } else {
            const uint32_t m = (sh << (3 - p)) & ec.mask;
            r[p] = SCALED ? (sc[p] ^ m) : (m | ec.one);
        }
    }
    return __builtin_bit_cast(f16x8, r);
}

// x as an fp32 value the compiler must materialize.  An epilogue's product
// is rounded to fp32 here and then converted to fp16 (two roundings, in every
// kernel form alike); without this the backend may fuse the product and the
// conversion into one mixed-precision instruction that rounds the exact
// product once -- in some kernel forms and not others, whatever the
// contraction setting.
__device__ __forceinline__ float fp32_value(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Optional affine output term: out[r][c] = rne16(sn[c] * C[r][c] +
// term(r, c)) with
//   term(r, c) = Σ_{q < Q-1} E[q * ldE + c] * stats[r * Q + q] + stats[r * Q + Q - 1]
// (E null: none).  Q = 2 is one row of E and two statistics per row.
struct Affine {
    const float *E = nullptr;
    const float *stats = nullptr;  // [M][Q]
    int Q = 2, ldE = 0;
};

// term(r, c) above in fp32, the products added in q order.
__device__ __forceinline__ float affine_term(const Affine &aff, int row, int col) {
    const float *st = aff.stats + static_cast<size_t>(row) * aff.Q;
    float t = aff.E[col] * st[0];
    for (int q = 1; q < aff.Q - 1; ++q) t = t + aff.E[static_cast<size_t>(q) * aff.ldE + col] * st[q];
    return t + st[aff.Q - 1];
}

// Batch-sum epilogue (gradients): for every output column c, the sum over
// the wave's 64 rows of C[r][c] * Q[r][c], written to part[(r0 / 64) * n_out
// + c]; summing the parts in order gives Σ_r C[r][c] Q[r][c] (grad.hip).
struct DotArgs {
    const void *q;  // fp16 or fp32 (q_f32), row-major, leading dimension ldq
    int q_f32, ldq;
    float *part;    // null: no batch sums
};

// The epilogue of both product kernels.  32x32 MFMA result register v of a
// lane holds row 8*(v/4) + 4*(lane/32) + v%4 and column lane%32 of its tile;
// row0 / col0 are the wave's first row and column.
template <int MF_, int NF_>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[MF_][NF_], const float (&snv)[NF_], int M, int n_out,
                                         int row0, int col0, int l32, int kg, __half *__restrict__ out, int ldo,
                                         float *__restrict__ out32, int ldo32, const DotArgs &dot,
                                         const Affine &aff) {
    static_assert(32 * MF_ == 64, "batch-sum groups are the waves' 64 rows");
#pragma unroll
    for (int i = 0; i < MF_; ++i) {
#pragma unroll
        for (int f = 0; f < NF_; ++f) {
            const int col = col0 + f * 32 + l32;
            if (col >= n_out) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = row0 + i * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
                if (row < M) {
                    if (out) {
                        float val = fp32_value(acc[i][f][v] * snv[f]);
                        if (aff.E) val = fp32_value(val + affine_term(aff, row, col));
                        out[static_cast<size_t>(row) * ldo + col] = __float2half_rn(val);
                    }
                    if (out32) out32[static_cast<size_t>(row) * ldo32 + col] = acc[i][f][v];
                }
            }
        }
    }
    if (dot.part) {
#pragma unroll
        for (int f = 0; f < NF_; ++f) {
            const int col = col0 + f * 32 + l32;
            float sum = 0.0f;
            if (col < n_out) {
#pragma unroll
                for (int i = 0; i < MF_; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int row = row0 + i * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
                        if (row < M) {
                            const size_t qi = static_cast<size_t>(row) * dot.ldq + col;
                            const float qv = dot.q_f32 ? static_cast<const float *>(dot.q)[qi]
                                                       : __half2float(static_cast<const __half *>(dot.q)[qi]);
                            sum += acc[i][f][v] * qv;
                        }
                    }
            }
            sum += __shfl_xor(sum, 32);  // the two halves of the wave hold alternate row quads of the column
            if (kg == 0 && col < n_out && row0 < M) dot.part[static_cast<size_t>(row0 / 64) * n_out + col] = sum;
        }
    }
}

// Split-K parts: the unscaled sums of the tile, part[row * ldw + col].
template <int MF_, int NF_>
__device__ __forceinline__ void store_partial(const f32x16 (&acc)[MF_][NF_], int M, int n_out, int row0, int col0,
                                              int l32, int kg, float *__restrict__ part, int ldw) {
#pragma unroll
    for (int i = 0; i < MF_; ++i)
#pragma unroll
        for (int f = 0; f < NF_; ++f) {
            const int col = col0 + f * 32 + l32;
            if (col >= n_out) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = row0 + i * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
                if (row < M) part[static_cast<size_t>(row) * ldw + col] = acc[i][f][v];
            }
        }
}

// Sum of the split-K parts in part order, scaled and rounded once: one
// thread per four outputs of a row (16-byte loads of each part, eight
// parts' loads in flight at a time, one 8-byte store).
__global__ __launch_bounds__(256) void split_finish_kernel(const float *__restrict__ part, int nsplit, int M,
                                                           int n_out, int ldw, const __half *__restrict__ sn,
                                                           __half *__restrict__ out, int ldo, const Affine aff) {
    const int cq = ldw >> 2;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * cq) return;
    const int row = idx / cq, c0 = (idx - row * cq) * 4;
    const size_t plane = static_cast<size_t>(M) * ldw;
    const float *p = part + static_cast<size_t>(row) * ldw + c0;
    float4 s = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < nsplit; k0 += 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = *reinterpret_cast<const float4 *>(p + static_cast<size_t>(min(k0 + u, nsplit - 1)) * plane);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (k0 + u < nsplit) {
                s.x += v[u].x;
                s.y += v[u].y;
                s.z += v[u].z;
                s.w += v[u].w;
            }
    }
    const float sv[4] = {s.x, s.y, s.z, s.w};
    __half o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int col = min(c0 + e, n_out - 1);
        float val = fp32_value(sv[e] * __half2float(sn[col]));
        if (aff.E) val = fp32_value(val + affine_term(aff, row, col));
        o[e] = __float2half_rn(val);
    }
    __half *dst = out + static_cast<size_t>(row) * ldo + c0;
    if (c0 + 4 <= n_out && ((reinterpret_cast<uintptr_t>(dst) & 7) == 0)) {
        *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(o);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (c0 + e < n_out) dst[e] = o[e];
    }
}

// C = P S'ᵀ (see the file comment).  P: fp16 [M][ldp], K valid columns
// (zero beyond).  S: tiled sign rows, `words` per row, n_rows_pad rows.
// sk: fp16 scale per K (zero-padded to words*32) or unused.  sn: fp16 scale
// per output column.  out: fp16 [M][ldo], columns < n_out written.
// PVEC: rows of P are 16-byte aligned (ldp % 8 == 0).  KFULL: also K % 64
// == 0, so every K step loads whole 16-byte items with no bounds test.
template <bool HAS_SK, bool PVEC, bool KFULL, bool BIN>
__global__ __launch_bounds__(kThreads, DBF_PREFILL_OCC) void sign_gemm_kernel(const __half *__restrict__ P, int ldp, int M, int K,
                                                             const uint32_t *__restrict__ S, int words,
                                                             int n_rows_pad, const __half *__restrict__ sk,
                                                             const __half *__restrict__ sn,
                                                             __half *__restrict__ out, int ldo, int n_out,
                                                             float *__restrict__ out32, int ldo32, const DotArgs dot,
                                                             const Affine aff, int nbm, int nbn) {
    __shared__ _Float16 Ps[2][BM * LDP];
    __shared__ uint32_t Ss[2][BK / 2];  // sk of the K step, as half pairs

    const ExpandConsts ec = expand_consts<BIN>();
    // XCD-aware tile order: the blocks of one XCD take consecutive tiles.
    const int G = nbm * nbn;
    const int b = blockIdx.x;
    const int xcd = b % kXcds, slot = b / kXcds, q = G / kXcds, rem = G % kXcds;
    const int tile = xcd * q + min(xcd, rem) + slot;
    const int bm = tile / nbn, bn = tile - (tile / nbn) * nbn;
    const int m0 = bm * BM, n0 = bn * BN;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WGN, wn = wave % WGN;
    const int l32 = lane & 31, kg = lane >> 5;

    const uint2 *S2 = reinterpret_cast<const uint2 *>(S);
    const int nk = words >> 1;  // K steps of 64 = word pairs

    // sign rows of this lane's four N fragments (clamped: rows past the end
    // are loaded but never written out)
    int srow[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) srow[f] = min(n0 + wn * 32 * NF + f * 32 + l32, n_rows_pad - 1);
    auto load_signs = [&](int kt, uint2 (&w)[NF]) {
#pragma unroll
        for (int f = 0; f < NF; ++f)
            w[f] = S2[(static_cast<size_t>(srow[f] >> 6) * (words >> 1) + kt) * 64 + (srow[f] & 63)];
    };

    // P tile of a K step: 128 rows x 64 halves = 1024 items of 8 halves, 4 per thread
    u32x4 pv[4];
    u32x4 skv = {0u, 0u, 0u, 0u};
    auto load_p = [&](int kt) {
        const int k0 = kt * BK;
        const bool full = KFULL || (PVEC && (k0 + BK <= K));
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

    f32x16 acc[MF][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.0f;

    float snv[NF];  // epilogue column scales, fetched early
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int col = n0 + wn * 32 * NF + f * 32 + l32;
        snv[f] = sn && col < n_out ? __half2float(sn[col]) : 0.0f;
    }

    uint2 wcur[NF], wnxt[NF];
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
        const _Float16 *pa = &Ps[buf][(wm * 32 * MF + l32) * LDP + 8 * kg];
#pragma unroll
        for (int s = 0; s < 4; ++s) {  // K sub-steps of 16
            f16x8 af[MF];
#pragma unroll
            for (int i = 0; i < MF; ++i) af[i] = *reinterpret_cast<const f16x8 *>(pa + i * 32 * LDP + s * 16);
            u32x4 sc = {0u, 0u, 0u, 0u};
            if (HAS_SK) sc = *reinterpret_cast<const u32x4 *>(&Ss[buf][s * 8 + 4 * kg]);
            const int g = 2 * (s & 1) + kg;  // which 8 elements of the 32-element word
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const f16x8 bf = expand<HAS_SK, BIN>(s < 2 ? wcur[f].x : wcur[f].y, g, sc, ec);
#pragma unroll
                for (int i = 0; i < MF; ++i)
                    acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf, acc[i][f], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) {
            store_p(buf ^ 1);
#pragma unroll
            for (int f = 0; f < NF; ++f) wcur[f] = wnxt[f];
        }
        __syncthreads();
    }

    epilogue<MF, NF>(acc, snv, M, n_out, m0 + wm * 32 * MF, n0 + wn * 32 * NF, l32, kg, out, ldo, out32, ldo32, dot,
                     aff);
}

// Host-side arguments of one product launch.
struct GemmLaunch {
    const void *P;
    int ldp, M, K;
    const uint32_t *S;
    int words, n_rows_pad;
    const void *sk, *sn;
    void *out;
    int ldo, n_out;
    float *out32;
    int ldo32;
    DotArgs dot;
    Affine aff;
    int sk_cols = 0, sk_stride = 0;  // per-column-block scales (GemmFlavor)
};

template <bool HAS_SK, bool PVEC, bool KFULL, bool BIN>
void launch(const GemmLaunch &a, hipStream_t s) {
    const int nbm = (a.M + BM - 1) / BM;
    const int nbn = (a.n_out + BN - 1) / BN;
    launch_kernel((sign_gemm_kernel<HAS_SK, PVEC, KFULL, BIN>), dim3(nbm * nbn), dim3(kThreads), 0, s,
                  static_cast<const __half *>(a.P), a.ldp, a.M, a.K, a.S, a.words, a.n_rows_pad,
                  static_cast<const __half *>(a.sk), static_cast<const __half *>(a.sn), static_cast<__half *>(a.out),
                  a.ldo, a.n_out, a.out32, a.ldo32, a.dot, a.aff, nbm, nbn);
}


// ---------------------------------------------------------------------------
// Deep-pipelined form for K % 64 == 0 and 16-byte aligned rows of P.
//
// The operands of a K step go from global memory straight into LDS
// (global_load_lds_dwordx4 / _dword, no register staging) into a ring of
// kStages buffers, so kStages - 1 steps are in flight while one is
// multiplied: the loads have several microseconds of MFMA work to arrive
// instead of one step's.  Per step and wave the loads are uniform (P: 4
// 16-byte loads, signs: 2 dword loads, sk: 1 dword load), so the wait for a
// step is a fixed `s_waitcnt vmcnt`.  The waves meet at one barrier per step;
// the compiler's own barrier would also wait for the younger steps' loads,
// hence the raw s_barrier with explicit counts.
//
// P tile in LDS: 128 rows of 64 halves (8 chunks of 16 bytes), chunk c of row
// r stored at position c ^ (r & 7): the eight rows that one MFMA operand read
// touches then cover all 32 banks once.
#ifndef DBF_PREFILL_DMA_MF
#define DBF_PREFILL_DMA_MF 2
#endif
#ifndef DBF_PREFILL_DMA_NF
#define DBF_PREFILL_DMA_NF 2
#endif
#ifndef DBF_PREFILL_STAGES
#define DBF_PREFILL_STAGES 4
#endif
#ifndef DBF_PREFILL_DMA_WAVES
#define DBF_PREFILL_DMA_WAVES 8
#endif
constexpr int kDWaves = DBF_PREFILL_DMA_WAVES;
constexpr int kDThreads = 64 * kDWaves;
constexpr int DMF = DBF_PREFILL_DMA_MF;
constexpr int DNF = DBF_PREFILL_DMA_NF;
constexpr int DWGM = BM / (32 * DMF);
constexpr int DWGN = kDWaves / DWGM;
constexpr int DBN = 32 * DNF * DWGN;
constexpr int kStages = DBF_PREFILL_STAGES;

// Sizes of one pipeline step of KP word pairs (K = 64 * KP).
template <int KP>
struct DmaStep {
    static constexpr int K = 64 * KP;
    static constexpr int PBytes = BM * K * 2;             // P tile
    static constexpr int SBytes = DBN * 8 * KP;           // KP word pairs per sign row
    static constexpr int KBytes = K * 2;                  // sk of the step
    static constexpr int StageBytes = PBytes + SBytes + KBytes;
    static constexpr size_t Lds = static_cast<size_t>(kStages) * StageBytes;
    static constexpr int Chunks = K / 8;                  // 16-byte chunks per P row
    static constexpr int PI = PBytes / 1024 / kDWaves;    // 1 KiB P loads per wave
    static constexpr int SIP = DBN / 64 * 2;              // 256-byte sign loads per word pair
    static constexpr int SI = SIP * KP / kDWaves;         // 256-byte sign loads per wave
    static_assert(PI * kDWaves * 1024 == PBytes && SI * kDWaves * 256 == SBytes && SI >= 1,
                  "loads of a step divide evenly over the waves");
    static_assert(Lds <= 160 * 1024, "LDS of a CU");
};

#ifndef DBF_PREFILL_PAIRS
#define DBF_PREFILL_PAIRS 2
#endif
constexpr int kDmaPairs = DBF_PREFILL_PAIRS;  // word pairs per pipeline step where K allows

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void *g, char *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)(l), 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, char *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)(l), 4, 0, 0);
}

// Wait until at most n of this wave's loads are outstanding (n constant).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // s_waitcnt: vmcnt bits [3:0] and [15:14]; expcnt [6:4] and lgkmcnt [11:8] left at "no wait"
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until this wave's loads of a step have landed while the loads of its
// `y` younger steps (0 <= y <= Y) may still be in flight; D loads per step.
template <int D, int Y>
__device__ __forceinline__ void wait_step(int y) {
    if constexpr (Y == 0) {
        wait_vm<0>();
    } else {
        if (y >= Y) wait_vm<Y * D>();
        else wait_step<D, Y - 1>(y);
    }
}

// One K step of sign_gemm_dma_kernel: start the loads of step `nxt` into
// stage `dst` (if GO), then multiply the operands in stage `src`.  The two
// stage pointers are restrict-qualified: they never overlap, and the compiler
// then does not hold the LDS reads of `src` back until the loads into `dst`
// have landed (the kernel orders them itself with vmcnt and the barrier).
template <bool HAS_SK, int KP, int D, bool BIN, bool GO, typename IssueOne>
__device__ __forceinline__ void dma_step(int nxt, char *__restrict__ dst, const char *__restrict__ src,
                                         IssueOne &issue_one, f32x16 (&acc)[DMF][DNF], int wm, int wn, int l32,
                                         int kg, ExpandConsts ec) {
    using C = DmaStep<KP>;
    static_assert(D <= 4 * KP, "one load per sub-step");
    const uint2 *sg = reinterpret_cast<const uint2 *>(src + C::PBytes);
    const char *prow = src + (wm * 32 * DMF + l32) * (C::K * 2);
#pragma unroll
    for (int j = 0; j < KP; ++j) {  // word pairs
        uint2 w[DNF];
#pragma unroll
        for (int f = 0; f < DNF; ++f) w[f] = sg[j * DBN + wn * 32 * DNF + f * 32 + l32];
#pragma unroll
        for (int s = 4 * j; s < 4 * j + 4; ++s) {  // K sub-steps of 16
        // the loads of step nxt go out one per sub-step, between the MFMAs,
        // so that the memory pipeline works while the matrix cores do
        if (GO && s < D) issue_one(nxt, dst, s);
        const int pc = ((2 * s + kg) ^ (l32 & 7)) * 16;
        f16x8 af[DMF];
#pragma unroll
        for (int i = 0; i < DMF; ++i) af[i] = *reinterpret_cast<const f16x8 *>(prow + i * 32 * (C::K * 2) + pc);
        u32x4 sc = {0u, 0u, 0u, 0u};
        if (HAS_SK) sc = *reinterpret_cast<const u32x4 *>(src + C::PBytes + C::SBytes + (s * 8 + 4 * kg) * 4);
        const int g = 2 * (s & 1) + kg;
#pragma unroll
        for (int f = 0; f < DNF; ++f) {
            const f16x8 bf = expand<HAS_SK, BIN>((s & 3) < 2 ? w[f].x : w[f].y, g, sc, ec);
#pragma unroll
            for (int i = 0; i < DMF; ++i)
                acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf, acc[i][f], 0, 0, 0);
        }
        }
    }
}

// The product's work for output tile (bm, bn), K part `split` of nsplit.
template <bool HAS_SK, int KP, bool BIN>
__device__ __forceinline__ void dma_tile(char *lds, const __half *__restrict__ P, int ldp, int M,
                                         const uint32_t *__restrict__ S, int words, int n_rows_pad,
                                         const __half *__restrict__ sk, const __half *__restrict__ sn,
                                         __half *__restrict__ out, int ldo, int n_out, float *__restrict__ out32,
                                         int ldo32, const DotArgs &dot, const Affine &aff, int bm, int bn, int split,
                                         float *__restrict__ part, int nsplit, int ldw) {
    using C = DmaStep<KP>;
    constexpr int D = C::PI + C::SI + (HAS_SK ? 1 : 0);  // loads per step and wave

    const ExpandConsts ec = expand_consts<BIN>();
    const int m0 = bm * BM, n0 = bn * DBN;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave / DWGN, wn = wave % DWGN;
    const int l32 = lane & 31, kg = lane >> 5;
    // K steps [kb, kb + nk) of this split
    const int nk_all = words / (2 * KP);
    const int kb = split * nk_all / nsplit;
    const int nk = (split + 1) * nk_all / nsplit - kb;

    // per-lane source offsets of the step loads (a step adds K halves / KP word pairs)
    const __half *psrc[C::PI];
#pragma unroll
    for (int qq = 0; qq < C::PI; ++qq) {
        const int c = (wave * C::PI + qq) * 64 + lane;  // 16-byte chunk of the tile
        const int r = c / C::Chunks, pc = c % C::Chunks;
        const int lc = pc ^ (r & 7);
        psrc[qq] = P + static_cast<size_t>(min(m0 + r, M - 1)) * ldp + lc * 8;
    }
    const uint32_t *ssrc[C::SI];
#pragma unroll
    for (int h = 0; h < C::SI; ++h) {
        const int ii = wave * C::SI + h;  // loads of 256 bytes: word pair x row tile x half
        const int j = ii / C::SIP, rem = ii % C::SIP;
        const int t = min((n0 >> 6) + (rem >> 1), n_rows_pad / 64 - 1);  // tiles past the end: loaded, unused
        ssrc[h] = S + (static_cast<size_t>(t) * (words >> 1) + j) * 128 + (rem & 1) * 64 + lane;
    }
    // load q (0 <= q < D) of this wave for step kt into stage st
    auto issue_one = [&](int kl, char *st, int q) {
        const int kt = kb + kl;
        if (q < C::PI) {
            dma16(psrc[q] + kt * C::K, st + (wave * C::PI + q) * 1024);
        } else if (q < C::PI + C::SI) {
            const int h = q - C::PI;
            dma4(ssrc[h] + kt * KP * 128, st + C::PBytes + (wave * C::SI + h) * 256);
        } else if (HAS_SK) {
            // every wave: the same K * 2 bytes
            if (lane < C::K / 2) dma4(sk + kt * C::K + 2 * lane, st + C::PBytes + C::SBytes);
        }
    };
    auto issue = [&](int kt, char *st) {
#pragma unroll
        for (int q = 0; q < D; ++q) issue_one(kt, st, q);
    };

    f32x16 acc[DMF][DNF];
#pragma unroll
    for (int i = 0; i < DMF; ++i)
#pragma unroll
        for (int f = 0; f < DNF; ++f)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.0f;

    float snv[DNF];
#pragma unroll
    for (int f = 0; f < DNF; ++f) {
        const int col = n0 + wn * 32 * DNF + f * 32 + l32;
        snv[f] = sn && col < n_out ? __half2float(sn[col]) : 0.0f;
    }

#pragma unroll
    for (int s0 = 0; s0 < kStages - 1; ++s0)
        if (s0 < nk) issue(s0, lds + s0 * C::StageBytes);

    // Steps that start the loads of a later step, then the last kStages - 1
    // steps that start none: no branch inside a step's body, so the
    // compiler schedules a whole step as one block (LDS reads of the next K
    // sub-step ahead of the current one's MFMAs; 4096x14336 MLP products
    // 7-9 % faster than with the loads under a per-step condition).
    int kt = 0;
    for (; kt < nk - (kStages - 1); ++kt) {
        // this wave's loads of step kt have landed, those of the kStages - 2
        // younger steps may be in flight; the barrier: every other wave's too,
        // and step kt - 1's buffer is free
        wait_vm<(kStages - 2) * D>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int nxt = kt + kStages - 1;
        dma_step<HAS_SK, KP, D, BIN, true>(nxt, lds + (nxt % kStages) * C::StageBytes,
                                           lds + (kt % kStages) * C::StageBytes, issue_one, acc, wm, wn, l32, kg,
                                           ec);
    }
    for (; kt < nk; ++kt) {
        wait_step<D, kStages - 2>(min(kStages - 2, nk - 1 - kt));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        dma_step<HAS_SK, KP, D, BIN, false>(0, lds, lds + (kt % kStages) * C::StageBytes, issue_one, acc, wm, wn,
                                            l32, kg, ec);
    }

    if (part) {
        store_partial<DMF, DNF>(acc, M, n_out, m0 + wm * 32 * DMF, n0 + wn * 32 * DNF, l32, kg,
                                part + static_cast<size_t>(split) * M * ldw, ldw);
        return;
    }
    epilogue<DMF, DNF>(acc, snv, M, n_out, m0 + wm * 32 * DMF, n0 + wn * 32 * DNF, l32, kg, out, ldo, out32, ldo32,
                       dot, aff);
}

// XCD-aware position of workgroup b among G: the workgroups of one XCD
// (b mod 8) take consecutive indexes, so they share K ranges and rows of P
// in that XCD's L2.
__device__ __forceinline__ int xcd_index(int b, int G) {
    const int xcd = b % kXcds, slot = b / kXcds, q = G / kXcds, rem = G % kXcds;
    return xcd * q + min(xcd, rem) + slot;
}

template <bool HAS_SK, int KP, bool BIN>
__global__ __launch_bounds__(kDThreads) void sign_gemm_dma_kernel(const __half *__restrict__ P, int ldp, int M,
                                                                 const uint32_t *__restrict__ S, int words,
                                                                 int n_rows_pad, const __half *__restrict__ sk,
                                                                 const __half *__restrict__ sn,
                                                                 __half *__restrict__ out, int ldo, int n_out,
                                                                 float *__restrict__ out32, int ldo32, const DotArgs dot,
                                                                 const Affine aff, int nbm, int nbn,
                                                                 float *__restrict__ part, int nsplit, int ldw,
                                                                 int sk_cols, int sk_stride) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    // order over (split, tile), tile fastest
    const int T = nbm * nbn;
    const int idx = xcd_index(blockIdx.x, T * nsplit);
    const int split = idx / T, tile = idx - split * T;
    const int bm = tile / nbn, bn = tile - (tile / nbn) * nbn;
    // stacked products: this tile's columns take the scale of their block
    const __half *skt = sk && sk_cols > 0 ? sk + static_cast<size_t>(bn * DBN / sk_cols) * sk_stride : sk;
    dma_tile<HAS_SK, KP, BIN>(lds, P, ldp, M, S, words, n_rows_pad, skt, sn, out, ldo, n_out, out32, ldo32, dot, aff,
                              bm, bn, split, part, nsplit, ldw);
}

// Several products with the same M, as one launch: product i covers tiles
// [tile0[i], tile0[i + 1]) of the grid, in the order of a product of its own
// (the tiles of one row block consecutive); every tile runs the same body,
// over the whole K.
template <bool HAS_SK, int KP, bool BIN>
__global__ __launch_bounds__(kDThreads) void sign_gemm_dma_group_kernel(const GemmGroup g) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int idx = xcd_index(blockIdx.x, g.tile0[g.count]);
    int i = 0;
    for (int j = 1; j < g.count; ++j)
        if (idx >= g.tile0[j]) i = j;
    const GemmItem &it = g.item[i];
    const int tile = idx - g.tile0[i];
    const int nbn = (it.n_out + DBN - 1) / DBN;
    const int bm = tile / nbn, bn = tile - bm * nbn;
    dma_tile<HAS_SK, KP, BIN>(lds, static_cast<const __half *>(it.P), it.ldp, g.M, it.S, it.words, it.n_rows_pad,
                              static_cast<const __half *>(it.sk), static_cast<const __half *>(it.sn),
                              static_cast<__half *>(it.out), it.ldo, it.n_out, nullptr, 0, DotArgs{}, Affine{}, bm,
                              bn, 0, nullptr, 1, 0);
}

// One product's arguments of dma_tile, with its grid of tiles and its K parts.
struct DmaPart {
    const __half *P;
    int ldp, M;
    const uint32_t *S;
    int words, n_rows_pad;
    const __half *sk, *sn;
    __half *out;
    int ldo, n_out;
    float *out32;
    int ldo32;
    DotArgs dot;
    Affine aff;
    int nbm, nbn;
    float *part;
    int nsplit, ldw;
};

// A head-and-tail product as one launch: workgroup b first runs head tile b
// (its columns [0, c0) over the whole K, as the head grid would place it),
// then, after a barrier that frees the LDS ring, tail piece b (a K part of a
// column tile from c0 on, as the tail grid would place it) into the split-K
// workspace.  The pieces, their K ranges and their XCDs are those of the two
// separate launches, so the results are the same bits; a tail piece starts
// as soon as its own workgroup's head tile is done, instead of after the
// slowest head tile and a launch.
template <bool HAS_SK, bool BIN>
__global__ __launch_bounds__(kDThreads) void sign_gemm_dma_headtail_kernel(const DmaPart head, const DmaPart tail) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int b = blockIdx.x;
    const int TH = head.nbm * head.nbn;
    if (b < TH) {
        const int idx = xcd_index(b, TH);
        const int bm = idx / head.nbn, bn = idx - (idx / head.nbn) * head.nbn;
        dma_tile<HAS_SK, 2, BIN>(lds, head.P, head.ldp, head.M, head.S, head.words, head.n_rows_pad, head.sk,
                                 head.sn, head.out, head.ldo, head.n_out, head.out32, head.ldo32, head.dot, head.aff,
                                 bm, bn, 0, nullptr, 1, 0);
    }
    const int TT = tail.nbm * tail.nbn, GT = TT * tail.nsplit;
    if (b < GT) {
        __syncthreads();  // every wave is done with the head's LDS stages
        const int idx = xcd_index(b, GT);
        const int split = idx / TT, tile = idx - split * TT;
        const int bm = tile / tail.nbn, bn = tile - (tile / tail.nbn) * tail.nbn;
        dma_tile<HAS_SK, 2, BIN>(lds, tail.P, tail.ldp, tail.M, tail.S, tail.words, tail.n_rows_pad, tail.sk,
                                 tail.sn, tail.out, tail.ldo, tail.n_out, tail.out32, tail.ldo32, tail.dot, tail.aff,
                                 bm, bn, split, tail.part, tail.nsplit, tail.ldw);
    }
}

template <bool HAS_SK, int KP, bool BIN>
void launch_dma(const GemmLaunch &a, hipStream_t s, float *part = nullptr, int nsplit = 1, int ldw = 0) {
    using C = DmaStep<KP>;
    static const bool once =
        ((void)hipFuncSetAttribute(reinterpret_cast<const void *>(sign_gemm_dma_kernel<HAS_SK, KP, BIN>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(C::Lds)),
         true);
    (void)once;
    const int nbm = (a.M + BM - 1) / BM;
    const int nbn = (a.n_out + DBN - 1) / DBN;
    launch_kernel((sign_gemm_dma_kernel<HAS_SK, KP, BIN>), dim3(nbm * nbn * nsplit), dim3(kDThreads), C::Lds, s,
                  static_cast<const __half *>(a.P), a.ldp, a.M, a.S, a.words, a.n_rows_pad,
                  static_cast<const __half *>(a.sk), static_cast<const __half *>(a.sn), static_cast<__half *>(a.out),
                  a.ldo, a.n_out, a.out32, a.ldo32, a.dot, a.aff, nbm, nbn, part, nsplit, ldw, a.sk_cols,
                  a.sk_stride);
}

DmaPart dma_part(const GemmLaunch &a, float *part, int nsplit, int ldw) {
    return DmaPart{static_cast<const __half *>(a.P), a.ldp, a.M, a.S, a.words, a.n_rows_pad,
                   static_cast<const __half *>(a.sk), static_cast<const __half *>(a.sn), static_cast<__half *>(a.out),
                   a.ldo, a.n_out, a.out32, a.ldo32, a.dot, a.aff, (a.M + BM - 1) / BM, (a.n_out + DBN - 1) / DBN,
                   part, nsplit, ldw};
}

template <bool HAS_SK, bool BIN>
void launch_headtail(const GemmLaunch &head, const GemmLaunch &tail, hipStream_t s, float *part, int nsplit,
                     int ldw) {
    using C = DmaStep<2>;
    static const bool once =
        ((void)hipFuncSetAttribute(reinterpret_cast<const void *>(sign_gemm_dma_headtail_kernel<HAS_SK, BIN>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(C::Lds)),
         true);
    (void)once;
    const DmaPart h = dma_part(head, nullptr, 1, 0), t = dma_part(tail, part, nsplit, ldw);
    const int grid = std::max(h.nbm * h.nbn, t.nbm * t.nbn * nsplit);
    launch_kernel((sign_gemm_dma_headtail_kernel<HAS_SK, BIN>), dim3(grid), dim3(kDThreads), C::Lds, s, h, t);
}

#ifndef DBF_SPLIT_BELOW
#define DBF_SPLIT_BELOW 129
#endif
#ifndef DBF_SPLIT_TARGET
#define DBF_SPLIT_TARGET 256
#endif
#ifndef DBF_SPLIT_MIN_STEPS
#define DBF_SPLIT_MIN_STEPS 2
#endif

// Word pairs per step of the DMA kernel for this product.
int dma_pairs(int M, int words, int n_out) {
    if constexpr (kDmaPairs == 2) {
        const int tiles = ((M + BM - 1) / BM) * ((n_out + DBN - 1) / DBN);
        if (words % 4 == 0 && tiles <= 256) return 2;
    }
    return 1;
}

// K parts of the split-K form: grids of fewer than DBF_SPLIT_BELOW tiles (at
// most 128: half the CUs or less) are cut along K into about
// DBF_SPLIT_TARGET workgroups in all, each with at least DBF_SPLIT_MIN_STEPS
// steps.
int split_parts(int M, int words, int n_out) {
    const int tiles = ((M + BM - 1) / BM) * ((n_out + DBN - 1) / DBN);
    if (tiles >= DBF_SPLIT_BELOW) return 1;
    const int nk = words / (2 * dma_pairs(M, words, n_out));
    return std::max(1, std::min(DBF_SPLIT_TARGET / tiles, nk / DBF_SPLIT_MIN_STEPS));
}

#ifndef DBF_PREFILL_TAIL
#define DBF_PREFILL_TAIL 1
#endif
#ifndef DBF_PREFILL_FUSED_TAIL
#define DBF_PREFILL_FUSED_TAIL 1
#endif
#ifndef DBF_TAIL_BELOW
#define DBF_TAIL_BELOW 512
#endif

// Head and tail of a grid of 257 to DBF_TAIL_BELOW - 1 tiles (one wave of
// workgroups over the CUs plus a partial one): the first column tiles, at
// most 256 tiles, run whole-K as one wave, and the remaining columns run
// split-K in about DBF_SPLIT_TARGET workgroups instead of as a second,
// mostly empty wave.  Returns the first tail column (0: no head and tail)
// and sets *parts to the tail's part count.  Measured at batch 2048 (304
// tiles in the first product of the k = 4800 MLP layers): 4096x14336
// 406 -> 336 us per forward, 14336x4096 341 -> 335 us.  Grids of 512 tiles
// and more keep K steps of 64 and two workgroups per CU (a head of whole
// waves with a split tail measured no faster there).
int tail_split(int M, int words, int n_out, int *parts) {
    *parts = 1;
    if (!DBF_PREFILL_TAIL || kDmaPairs != 2 || words % 4 != 0) return 0;
    const int nbm = (M + BM - 1) / BM, nbn = (n_out + DBN - 1) / DBN;
    const int tiles = nbm * nbn;
    if (tiles <= 256 || tiles >= DBF_TAIL_BELOW) return 0;
    const int head = 256 / nbm;  // column tiles of the head
    if (head < 1 || head >= nbn) return 0;
    const int tail_tiles = nbm * (nbn - head);
    if (tail_tiles >= DBF_SPLIT_BELOW) return 0;
    const int nk = words / 4;
    *parts = std::max(1, std::min(DBF_SPLIT_TARGET / tail_tiles, nk / DBF_SPLIT_MIN_STEPS));
    if (*parts <= 1) return 0;
    return head * DBN;
}

}  // namespace

size_t sign_gemm_split_elems(int M, int K, int words, int n_out) {
#ifndef DBF_PREFILL_NO_DMA
    if (M <= 0 || K % BK != 0 || K != words * 32) return 0;
    int parts = split_parts(M, words, n_out);
    if (parts > 1) return static_cast<size_t>(parts) * M * ((n_out + 3) & ~3);
    const int col0 = tail_split(M, words, n_out, &parts);
    if (col0 > 0) return static_cast<size_t>(parts) * M * ((n_out - col0 + 3) & ~3);
    return 0;
#else
    (void)M, (void)K, (void)words, (void)n_out;
    return 0;
#endif
}

int launch_split_finish(const SplitK &split, int M, int n_out, const void *sn, void *out, int ldo, void *stream,
                        const float *aff_E, const float *aff_stats, int aff_Q, int aff_ldE) {
    const int items = M * (split.ldw >> 2);
    if (items == 0) return 0;
    const int c0 = split.col0;
    launch_kernel(split_finish_kernel, dim3((items + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                  static_cast<const float *>(split.ws), split.nsplit, M, n_out - c0, split.ldw,
                  static_cast<const __half *>(sn) + c0, static_cast<__half *>(out) + c0, ldo,
                  Affine{aff_E ? aff_E + c0 : nullptr, aff_stats, aff_Q, aff_ldE});
    return static_cast<int>(hipGetLastError());
}

namespace {

template <bool HAS_SK, bool BIN>
void dispatch_dma(const GemmLaunch &a, hipStream_t s, int kp, float *part = nullptr, int nsplit = 1, int ldw = 0) {
    if (kp == 2) launch_dma<HAS_SK, 2, BIN>(a, s, part, nsplit, ldw);
    else launch_dma<HAS_SK, 1, BIN>(a, s, part, nsplit, ldw);
}

template <bool HAS_SK, bool BIN>
int dispatch(const GemmLaunch &a, hipStream_t s, SplitK *split) {
    const bool pvec = (a.ldp & 7) == 0;
    const bool kfull = pvec && (a.K % BK) == 0;
#ifndef DBF_PREFILL_NO_DMA
    if (kfull && (reinterpret_cast<uintptr_t>(a.P) & 15) == 0 && a.K == a.words * 32) {
        const int kp = dma_pairs(a.M, a.words, a.n_out);
        if (split && split->ws && a.out && a.sn && !a.out32 && !a.dot.part) {
            const int parts = split_parts(a.M, a.words, a.n_out);
            const int ldw = (a.n_out + 3) & ~3;
            if (parts > 1 && static_cast<size_t>(parts) * a.M * ldw <= split->cap) {
                split->nsplit = parts;
                split->ldw = ldw;
                dispatch_dma<HAS_SK, BIN>(a, s, kp, split->ws, parts, ldw);
                return static_cast<int>(hipGetLastError());
            }
            int tparts = 1;
            const int c0 = a.sk_cols > 0 ? 0 : tail_split(a.M, a.words, a.n_out, &tparts);
            const int ldt = (a.n_out - c0 + 3) & ~3;
            if (c0 > 0 && static_cast<size_t>(tparts) * a.M * ldt <= split->cap) {
                GemmLaunch head = a;  // columns [0, c0), whole K
                head.n_out = c0;
                GemmLaunch tail = a;  // columns [c0, n_out): sign rows from 64-row tile c0 / 64 on
                tail.S = a.S + static_cast<size_t>(c0 / 64) * (a.words >> 1) * 128;
                tail.n_rows_pad = a.n_rows_pad - c0;
                tail.sn = static_cast<const __half *>(a.sn) + c0;
                tail.out = static_cast<__half *>(a.out) + c0;
                tail.n_out = a.n_out - c0;
                tail.aff.E = a.aff.E ? a.aff.E + c0 : nullptr;
#if DBF_PREFILL_FUSED_TAIL
                launch_headtail<HAS_SK, BIN>(head, tail, s, split->ws, tparts, ldt);
#else
                // timed as one product: the start event on the head, the stop event on the tail
                const LaunchEvents ev = launch_events();
                launch_events() = {ev.start, nullptr};
                dispatch_dma<HAS_SK, BIN>(head, s, 2);
                launch_events() = {nullptr, ev.stop};
                dispatch_dma<HAS_SK, BIN>(tail, s, 2, split->ws, tparts, ldt);
                launch_events() = ev;
#endif
                split->nsplit = tparts;
                split->ldw = ldt;
                split->col0 = c0;
                return static_cast<int>(hipGetLastError());
            }
        }
        // K steps of 128 where K allows and the tiles fit one wave of
        // workgroups over the 256 CUs; else steps of 64, whose 74 KiB of LDS
        // lets two workgroups share a CU (a partial last wave of tiles then
        // runs beside the first instead of after it)
        dispatch_dma<HAS_SK, BIN>(a, s, kp);
        return static_cast<int>(hipGetLastError());
    }
#endif
    if (a.sk_cols > 0) return static_cast<int>(hipErrorInvalidValue);  // stacked scales: the DMA form only
    if (kfull) launch<HAS_SK, true, true, BIN>(a, s);
    else if (pvec) launch<HAS_SK, true, false, BIN>(a, s);
    else launch<HAS_SK, false, false, BIN>(a, s);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_sign_gemm_group(GemmGroup &g, void *stream) {
    if (g.count < 1 || g.count > kMaxGroup || g.M < 1) return static_cast<int>(hipErrorInvalidValue);
    const bool has_sk = g.item[0].sk != nullptr;
    const int nbm = (g.M + BM - 1) / BM;
    int tiles = 0;
    bool pairs2 = kDmaPairs == 2;
    for (int i = 0; i < g.count; ++i) {
        const GemmItem &it = g.item[i];
        // the deep-pipelined form only: K a multiple of 64, whole words, 16-byte aligned rows of P
        if (!it.P || !it.S || !it.sn || !it.out || it.n_out < 1 || it.K % BK != 0 || it.K != it.words * 32 ||
            (it.ldp & 7) != 0 || (reinterpret_cast<uintptr_t>(it.P) & 15) != 0 || (it.sk != nullptr) != has_sk ||
            it.n_rows_pad < it.n_out)
            return static_cast<int>(hipErrorInvalidValue);
        g.tile0[i] = tiles;
        tiles += nbm * ((it.n_out + DBN - 1) / DBN);
        pairs2 = pairs2 && it.words % 4 == 0;
    }
    g.tile0[g.count] = tiles;
    const int kp = pairs2 && tiles <= 256 ? 2 : 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto go = [&](auto kernel, size_t lds) {
        static const bool once = ((void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                                            hipFuncAttributeMaxDynamicSharedMemorySize,
                                                            static_cast<int>(lds)),
                                  true);
        (void)once;
        launch_kernel(kernel, dim3(tiles), dim3(kDThreads), lds, s, g);
    };
    if (has_sk) {
        if (kp == 2) go(sign_gemm_dma_group_kernel<true, 2, false>, DmaStep<2>::Lds);
        else go(sign_gemm_dma_group_kernel<true, 1, false>, DmaStep<1>::Lds);
    } else {
        if (kp == 2) go(sign_gemm_dma_group_kernel<false, 2, false>, DmaStep<2>::Lds);
        else go(sign_gemm_dma_group_kernel<false, 1, false>, DmaStep<1>::Lds);
    }
    return static_cast<int>(hipGetLastError());
}

int launch_sign_gemm(const void *P, int ldp, int M, int K, const uint32_t *S, int words, int n_rows_pad,
                     const void *sk, const void *sn, void *out, int ldo, int n_out, float *out32, int ldo32,
                     const void *dq, int dq_f32, int lddq, float *dpart, void *stream, SplitK *split,
                     const GemmFlavor *flavor) {
    GemmLaunch a{P, ldp, M, K, S, words, n_rows_pad, sk, sn, out, ldo, n_out, out32, ldo32,
                 DotArgs{dq, dq_f32, lddq, dpart},
                 flavor ? Affine{flavor->aff_E, flavor->aff_stats, flavor->aff_Q, flavor->aff_ldE} : Affine{}};
    if (flavor && flavor->sk_cols > 0) {
        if (!sk || flavor->sk_cols % DBN != 0 || flavor->sk_stride < K) return static_cast<int>(hipErrorInvalidValue);
        a.sk_cols = flavor->sk_cols;
        a.sk_stride = flavor->sk_stride;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (split) {
        split->nsplit = 1;
        split->col0 = 0;
    }
    if (flavor && flavor->binary) {
        if (sk) return static_cast<int>(hipErrorInvalidValue);  // 0/1 matrices take no per-K scale
        return dispatch<false, true>(a, s, split);
    }
    if (sk) return dispatch<true, false>(a, s, split);
    return dispatch<false, false>(a, s, split);
}

}  // namespace dbf
