// Decode path (batch 1..16) of the DBF linear forward on the CDNA4 matrix cores.
//
// §2.1 of the gist.science technical summary of "Addition is almost all you
// need" evaluates X W^T as ((((X ⊙ bᵀ) Bᵀ) ⊙ midᵀ) Aᵀ) ⊙ aᵀ.  Both signed sums
// run here as 16x16x32 f16 MFMA products: the sign matrix is the A operand,
// expanded from its bits to ±1.0 in registers, and the activations are the B
// operand with the batch as the (at most 16 wide) N dimension.
// Batch 1:
//   stage 1: u = x ⊙ b is formed in fp32 (exact: a product of two fp16) and
//            split into u_hi = rne16(u) and u_lo = rne16(u - u_hi), which
//            carry about 22 significant bits; t = B u_hi + B u_lo in fp32;
//            the epilogue forms v = t * mid and stores it the same way, as
//            fp16 planes v_hi, v_lo.
//   stage 2: s = A v_hi + A v_lo in fp32; y = rne16(s * a).
//   The hi and lo parts ride in columns r and r + 8 of one MFMA.
// Batch 2..16 (the columns are batch rows): the sign operand of
// stage 1 carries ±b (b's fp16 sign bit flipped, exact), so x enters the
// product as it is and t = (B ⊙ b) x; v = rne16(t * mid) is one fp16 plane
// and s = A v -- the numerics of the prefill path.
//
// Work split.  A workgroup of 8 waves owns 16*RT rows of the sign matrix and
// its whole reduction dimension, taken in rounds that fit LDS (one round for
// the layer shapes of interest at batch <= 4).  Per round it first issues
// every global load it needs -- its block of sign words as coalesced 16-byte
// loads (the rows of one pair are contiguous in the tiled layout), and the
// activations of the round -- then writes them to LDS: the signs as they
// are, the activations as the hi/lo planes above.  Word pair p belongs to
// wave p mod 8, which accumulates in MFMA registers in increasing p; the
// waves reduce through LDS in a fixed order, so every output is summed in
// the same order whatever the batch size.  No partial sums leave the
// workgroup: a forward is two kernel launches.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>

#include "bqq_rowstats.h"
#include "dbf_internal.h"

namespace dbf {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kNW = 8;                      // waves per workgroup
constexpr int kThreads = kNW * 64;
constexpr int kMaxItems = 8;                // 16-byte sign loads per thread in flight per batch
#ifndef DBF_DECODE_TRIM_LOADS
#define DBF_DECODE_TRIM_LOADS 1
#endif
constexpr int kMaxAct = 4;                  // activation items (8 elements) per thread per batch
#ifndef DBF_DECODE_WIDE_ACT_NB
#define DBF_DECODE_WIDE_ACT_NB 8
#endif
#ifndef DBF_DECODE_WIDE_ACT
#define DBF_DECODE_WIDE_ACT 8
#endif
// Activation items per thread per batch at batch NB: twice as many from
// batch 8 on, so that the rounds of the pipelined form are half as many
// (14336-wide reductions at batch 16: 48 -> 43 us per forward for the
// 4096x14336 layer; 207 VGPRs, no spills; 16 items spill).
template <int NB>
__host__ __device__ constexpr int act_slots() {
    return NB >= DBF_DECODE_WIDE_ACT_NB ? DBF_DECODE_WIDE_ACT : kMaxAct;
}
#ifndef DBF_DECODE_LDS_KB
#define DBF_DECODE_LDS_KB 144
#endif
#ifndef DBF_DECODE_ONE_ROUND
#define DBF_DECODE_ONE_ROUND 256
#endif
constexpr size_t kLdsBudget = DBF_DECODE_LDS_KB * 1024;   // LDS of one workgroup (of 160 KiB per CU)
#ifndef DBF_DECODE_READAHEAD
#define DBF_DECODE_READAHEAD 1
#endif
constexpr bool kReadahead = DBF_DECODE_READAHEAD != 0;
constexpr int kCUs = 256;                   // MI355X
constexpr int kReadaheadBatch = 8;          // read-ahead loads in flight per thread
constexpr int kReadaheadMax = 16;           // read-ahead only if it needs at most this many loads per thread
constexpr uint32_t kSignPair = 0x80008000u;
constexpr uint32_t kOnePair = 0x3C003C00u;  // two fp16 +1.0

// Halves 8g..8g+7 of a 32-element sign word as ±1.0 MFMA operand.  Element
// 2q sits at bit q and element 2q+1 at bit 16+q, so after one shift by 12-4g
// the pair (8g+2p, 8g+2p+1) is at bits (12+p, 28+p) and a further shift by
// 3-p puts it on the two fp16 sign bits.  `mask` (the two sign bits) and
// `one` (two fp16 +1.0) are passed in registers so that each register of the
// operand is one v_and_or_b32: this ISA's VOP3 form cannot carry two literal
// constants, and with literals the compiler splits it into an and plus an or.
__device__ __forceinline__ f16x8 expand_pm1(uint32_t word, int g, uint32_t mask, uint32_t one) {
    const uint32_t sh = word << (12 - 4 * g);
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) r[p] = ((sh << (3 - p)) & mask) | one;
    return __builtin_bit_cast(f16x8, r);
}

// Halves 8g..8g+7 of a sign word as the operand ±sc (scale pairs sc[p],
// single-plane stage 1: ±b, exact): each sign pair is XORed onto the fp16
// sign bits of its scale pair.
__device__ __forceinline__ f16x8 expand_scaled(uint32_t word, int g, const u32x4 &sc, uint32_t mask) {
    const uint32_t sh = word << (12 - 4 * g);
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) r[p] = sc[p] ^ ((sh << (3 - p)) & mask);
    return __builtin_bit_cast(f16x8, r);
}

// Halves 8g..8g+7 of a word of a 0/1 matrix as the operand {0, 2.0}: the
// same pair moved one bit lower, onto the top exponent bit of each fp16
// (0x4000 = 2.0).  The factor 2 of each product is folded into the scales.
__device__ __forceinline__ f16x8 expand_01(uint32_t word, int g, uint32_t mask2) {
    const uint32_t sh = word << (12 - 4 * g);
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 3; ++p) r[p] = (sh << (2 - p)) & mask2;
    r[3] = (sh >> 1) & mask2;
    return __builtin_bit_cast(f16x8, r);
}

// The constants of expand_pm1 / expand_01 as register values the compiler
// cannot fold back into literals: the masks in scalar registers, +1.0 pair
// in a vector register.  Called once at kernel entry, before any MFMA has
// been issued, so the vector move cannot collide with an MFMA still reading
// its operands (the hazard recognizer does not see inside inline asm).
struct ExpandConsts {
    uint32_t mask, one, mask2;
};
template <bool BIN>
__device__ __forceinline__ ExpandConsts expand_consts() {
    ExpandConsts c;
    asm volatile("s_mov_b32 %0, 0x80008000" : "=s"(c.mask));
    asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(c.one));
    if constexpr (BIN) asm volatile("s_mov_b32 %0, 0x40004000" : "=s"(c.mask2));
    else c.mask2 = 0;
    return c;
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

__device__ __forceinline__ f16x8 zero8() { return __builtin_bit_cast(f16x8, u32x4{0u, 0u, 0u, 0u}); }

// Operand forms by batch size (NB < DBF_DECODE_SP_MIN: the first form):
//   NB = 1   : hi and lo fp16 planes of u = x ⊙ b (stage 1) and v (stage 2)
//              ride in columns r and r + 8 of one MFMA (kShared);
//   NB 2..16 : one plane (kSP): stage 1 multiplies x itself, with b folded
//              into the expanded signs as ±b (exact, as on the prefill
//              path), and stage 2 multiplies v rounded once to fp16; one
//              MFMA per sign fragment with the batch rows as its columns.
//              (Half the activation bytes: measured 5-25 % faster than the
//              hi/lo form at batch 2-8 on the 4096- and 14336-wide layers.)
#ifndef DBF_DECODE_SP_MIN
#define DBF_DECODE_SP_MIN 2
#endif
template <int NB>
struct Acc {
    static_assert(DBF_DECODE_SP_MIN >= 2 && DBF_DECODE_SP_MIN <= 9, "hi/lo planes need 2 NB <= 16 columns");
    static constexpr bool kSP = NB >= DBF_DECODE_SP_MIN;
    static constexpr bool kShared = !kSP;
    static constexpr int N = 1;
    // activation bytes per word pair in LDS: 2 planes x NB rows x 64 halves;
    // single plane: NB rows + one row of b (stage 1)
    static constexpr int kActPair = kSP ? 128 * NB + 128 : 256 * NB;
};

// LDS layout of one round of PR pairs:
//   signs  [PR][16*RT rows][2 words]           PR * 128 * RT bytes
//   planes [2][NB][64*PR] fp16 (hi, lo)         PR * 256 * NB bytes
//          (single plane: [NB + 1][64*PR], the last row b)
// and, after the last round, over the same bytes:
//   reduce [Acc::N][kNW][RT][64 lanes][4] fp32  Acc::N * kNW * RT * 1 KiB
// followed by kLdsTail bytes for workgroup-wide scalars.
constexpr size_t kLdsTail = 64;
template <int NB, int RT>
__host__ __device__ constexpr size_t lds_round_bytes(int PR) {
    return static_cast<size_t>(PR) * (128 * RT + Acc<NB>::kActPair);
}
template <int NB, int RT>
__host__ __device__ constexpr size_t lds_reduce_bytes() {
    return sizeof(float) * Acc<NB>::N * kNW * RT * 256;
}
template <int NB, int RT>
__host__ __device__ constexpr size_t lds_bytes(int PR) {
    return (lds_round_bytes<NB, RT>(PR) > lds_reduce_bytes<NB, RT>() ? lds_round_bytes<NB, RT>(PR)
                                                                       : lds_reduce_bytes<NB, RT>()) +
           kLdsTail;
}

// Pairs per round that fit the LDS budget.
template <int NB, int RT>
int round_pairs() {
    return static_cast<int>((kLdsBudget - kLdsTail) / (128 * RT + Acc<NB>::kActPair));
}

// Issue the loads of this thread's 16-byte sign items of the round, items
// it = item0 + threadIdx.x + kThreads * q (q < kMaxItems) of the block
// [pairs][rows].  Slots that no thread of the workgroup needs are skipped (a
// uniform branch; measured 2-5 % faster at batch 1 than loading them); in
// the last slot, items past the end load a valid item instead (the index is
// clamped) and are not stored, so the loads stay unconditional per lane and
// are all in flight together.
template <int RT>
__device__ __forceinline__ void load_sign_items(u32x4 (&v)[kMaxItems], const uint32_t *__restrict__ S, int words,
                                                int r0, int pr0, int nitems, int item0) {
    const int tile = r0 >> 6, roff = r0 & 63;
#pragma unroll
    for (int q = 0; q < kMaxItems; ++q) {
#if DBF_DECODE_TRIM_LOADS
        // slots no lane of the workgroup needs are not loaded (a uniform branch)
        if (item0 + kThreads * q >= nitems) break;
#endif
        const int it = min(item0 + static_cast<int>(threadIdx.x) + kThreads * q, nitems - 1);
        const int p = pr0 + it / (8 * RT);
        const int off = (it % (8 * RT)) * 4;  // in words
        v[q] = *reinterpret_cast<const u32x4 *>(S + ((static_cast<size_t>(tile) * (words >> 1) + p) * 64 + roff) * 2 + off);
    }
}

__device__ __forceinline__ void store_sign_items(const u32x4 (&v)[kMaxItems], uint32_t *sgn, int nitems, int item0) {
#pragma unroll
    for (int q = 0; q < kMaxItems; ++q) {
        const int it = item0 + threadIdx.x + kThreads * q;
        if (it < nitems) *reinterpret_cast<u32x4 *>(sgn + 4 * it) = v[q];
    }
}

// One round: pairs [pr0, pr1) of rows r0..r0+16RT-1 from the LDS copies.
template <int NB, int RT, bool STAGE1, bool BIN>
__device__ __forceinline__ void round_mma(f32x4 (&acc)[Acc<NB>::N][RT], const uint32_t *sgn, const _Float16 *act,
                                          int KR, int pr0, int pr1, int wave, int li, int g, ExpandConsts ec) {
    constexpr bool kShared = Acc<NB>::kShared;
    constexpr bool kSP = Acc<NB>::kSP;
    // Activation rows this lane feeds.  Column c of the B operand only
    // reaches output column c, so lanes of unused columns simply repeat a
    // valid row (no branches, no zeroing); those outputs are never read.
    const int r = (li & 7) < NB ? (li & 7) : NB - 1;
    const _Float16 *arow0 = kShared ? act + ((li < 8 ? 0 : NB) + r) * KR : act + (li < NB ? li : NB - 1) * KR;
    const _Float16 *brow = act + NB * KR;  // single plane, stage 1: the b row
    // operands of one word pair from LDS
    struct PairOps {
        uint2 w[RT];
        f16x8 v0[2];
        u32x4 sc[2];  // single-plane stage 1: b of the lane's 8 elements
    };
    auto load_pair = [&](int p, PairOps &o) {
        const int pl = p - pr0;
#pragma unroll
        for (int t = 0; t < RT; ++t) o.w[t] = *reinterpret_cast<const uint2 *>(sgn + (pl * 16 * RT + 16 * t + li) * 2);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int e = 64 * pl + 32 * h + 8 * g;
            o.v0[h] = *reinterpret_cast<const f16x8 *>(arow0 + e);
            if constexpr (kSP && STAGE1 && !BIN) o.sc[h] = *reinterpret_cast<const u32x4 *>(brow + e);
        }
    };
    auto mma_pair = [&](const PairOps &o) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                f16x8 sv;
                if constexpr (BIN) sv = expand_01(h ? o.w[t].y : o.w[t].x, g, ec.mask2);  // (b = 1)
                else if constexpr (kSP && STAGE1) sv = expand_scaled(h ? o.w[t].y : o.w[t].x, g, o.sc[h], ec.mask);
                else sv = expand_pm1(h ? o.w[t].y : o.w[t].x, g, ec.mask, ec.one);
                acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sv, o.v0[h], acc[0][t], 0, 0, 0);
            }
    };
    // Pair p belongs to wave p mod 8 whatever the rounds (the first pair of
    // this round with that residue), so every wave sums the same pairs in the
    // same order however the reduction dimension is cut into rounds.  Two
    // pairs per iteration: the LDS reads of both are issued before either's
    // MFMAs, so their latencies overlap (the pairs are still summed in
    // increasing order).
    int p = pr0 + ((wave - pr0) & (kNW - 1));
    for (; p + kNW < pr1; p += 2 * kNW) {
        PairOps o0, o1;
        load_pair(p, o0);
        load_pair(p + kNW, o1);
        mma_pair(o0);
        mma_pair(o1);
    }
    if (p < pr1) {
        PairOps o0;
        load_pair(p, o0);
        mma_pair(o0);
    }
}

// Direct form of a stage's multiply: all activations of the reduction
// dimension are in LDS (pair p's 64 columns at 64 p), and each wave loads the
// sign words of its own pairs (p = wave, wave + 8, ...) straight from global
// memory into the operand registers, kDirect pairs ahead of the MFMAs -- no
// LDS copy of the signs and no barrier between their arrival and use.  The
// MFMAs run in the same order as in round_mma, so both forms give the same
// bits.  r0: the workgroup's first row (its 16 RT rows lie in one 64-row tile);
// the pairs are p0 .. p0 + npairs - 1 (p0 a multiple of kNW), the activations
// of pair p0 + q at 64 q.
#ifndef DBF_DECODE_DIRECT_DEPTH
#define DBF_DECODE_DIRECT_DEPTH 4
#endif
constexpr int kDirect = DBF_DECODE_DIRECT_DEPTH;
template <int NB, int RT, bool STAGE1, bool BIN>
__device__ __forceinline__ void direct_mma(f32x4 (&acc)[Acc<NB>::N][RT], const uint32_t *__restrict__ S, int words,
                                           int r0, int p0, int npairs, const _Float16 *act, int KR, int wave, int li,
                                           int g, ExpandConsts ec) {
    constexpr bool kShared = Acc<NB>::kShared;
    constexpr bool kSP = Acc<NB>::kSP;
    const int r = (li & 7) < NB ? (li & 7) : NB - 1;
    const _Float16 *arow0 = kShared ? act + ((li < 8 ? 0 : NB) + r) * KR : act + (li < NB ? li : NB - 1) * KR;
    const _Float16 *brow = act + NB * KR;
    // word pair p of row r0 + 16 t + li: uint2 at ((tile * words / 2 + p) * 64 + (r0 & 63) + 16 t + li)
    const uint2 *src = reinterpret_cast<const uint2 *>(S) + static_cast<size_t>(r0 >> 6) * (words >> 1) * 64 +
                       static_cast<size_t>(p0) * 64 + (r0 & 63) + li;
    const int np = npairs > wave ? (npairs - wave + kNW - 1) / kNW : 0;  // this wave's pairs
    if (np == 0) return;
    uint2 wa[kDirect][RT], wb[kDirect][RT];
    auto load_group = [&](uint2 (&w)[kDirect][RT], int i0) {
#pragma unroll
        for (int ii = 0; ii < kDirect; ++ii) {
            const int p = wave + kNW * min(i0 + ii, np - 1);  // past the end: a valid pair, not used
#pragma unroll
            for (int t = 0; t < RT; ++t) w[ii][t] = src[static_cast<size_t>(p) * 64 + 16 * t];
        }
    };
    auto mma_group = [&](const uint2 (&w)[kDirect][RT], int i0) {
#pragma unroll
        for (int ii = 0; ii < kDirect; ++ii) {
            if (i0 + ii >= np) break;
            const int p = wave + kNW * (i0 + ii);
            f16x8 v0[2];
            u32x4 sc[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int e = 64 * p + 32 * h + 8 * g;
                v0[h] = *reinterpret_cast<const f16x8 *>(arow0 + e);
                if constexpr (kSP && STAGE1 && !BIN) sc[h] = *reinterpret_cast<const u32x4 *>(brow + e);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    f16x8 sv;
                    if constexpr (BIN) sv = expand_01(h ? w[ii][t].y : w[ii][t].x, g, ec.mask2);
                    else if constexpr (kSP && STAGE1) sv = expand_scaled(h ? w[ii][t].y : w[ii][t].x, g, sc[h], ec.mask);
                    else sv = expand_pm1(h ? w[ii][t].y : w[ii][t].x, g, ec.mask, ec.one);
                    acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sv, v0[h], acc[0][t], 0, 0, 0);
                }
        }
    };
    load_group(wa, 0);
    for (int i0 = 0; i0 < np; i0 += 2 * kDirect) {
        if (i0 + kDirect < np) load_group(wb, i0 + kDirect);
        mma_group(wa, i0);
        if (i0 + kDirect >= np) break;
        if (i0 + 2 * kDirect < np) load_group(wa, i0 + 2 * kDirect);
        mma_group(wb, i0 + kDirect);
    }
}

// Sum the waves' accumulators through LDS in a fixed wave order; wave 0's
// slots then hold the workgroup totals.
template <int NB, int RT>
__device__ __forceinline__ void reduce_waves(const f32x4 (&acc)[Acc<NB>::N][RT], float *red, int wave, int lane) {
    constexpr int N = Acc<NB>::N;
    __syncthreads();  // every wave is done reading the round buffers that `red` overlays
#pragma unroll
    for (int c = 0; c < N; ++c)
#pragma unroll
        for (int t = 0; t < RT; ++t)
            *reinterpret_cast<f32x4 *>(&red[((c * kNW + wave) * RT + t) * 256 + lane * 4]) = acc[c][t];
    __syncthreads();
    for (int idx = threadIdx.x; idx < N * RT * 256; idx += kThreads) {
        const int c = idx / (RT * 256);
        const int rest = idx - c * RT * 256;
        float s = red[(c * kNW) * RT * 256 + rest];
#pragma unroll
        for (int w = 1; w < kNW; ++w) s += red[((c * kNW + w) * RT) * 256 + rest];
        red[(c * kNW) * RT * 256 + rest] = s;
    }
    __syncthreads();
}

// hi + lo total for (row tile t, this lane's 4 rows, batch column li).
template <int NB, int RT>
__device__ __forceinline__ f32x4 total(const float *red, int t, int lane) {
    const f32x4 dh = *reinterpret_cast<const f32x4 *>(&red[t * 256 + lane * 4]);
    if constexpr (Acc<NB>::kSP) return dh;
    const f32x4 dl = *reinterpret_cast<const f32x4 *>(&red[t * 256 + (lane + 8) * 4]);
    return dh + dl;
}

#ifndef DBF_DECODE_S1_SPLIT_PAIRS
#define DBF_DECODE_S1_SPLIT_PAIRS 160
#endif
#ifndef DBF_DECODE_S1_SPLIT_MIN_NB
#define DBF_DECODE_S1_SPLIT_MIN_NB DBF_DECODE_SP_MIN
#endif

// Reduction parts of stage 1: part `s` of `parts` takes word pairs
// [pb0, pb1) (whole groups of kNW pairs, so pair p still belongs to wave
// p mod kNW) and writes its unscaled sums to part[(s * NB + r) * k_pad + j];
// the last part of a row block to finish (a ticket per row block) adds the
// parts in order s = 0, 1, ... and writes v.  parts == 1: no split.
struct S1Split {
    float *part;
    unsigned *tickets;
    int parts;
};

// Stage 1 for row block `blk` (rows 16*RT*blk ..): v = mid * (B (x ⊙ b)),
// stored as fp16 hi/lo planes [2][NB][k_pad] (single plane: [NB][k_pad]).
template <int NB, int RT, bool BIN>
__device__ __forceinline__ void stage1_body(int blk, char *base, const uint32_t *__restrict__ Bt, int Wm,
                                            const __half *__restrict__ x, int m, const __half *__restrict__ b,
                                            const __half *__restrict__ mid, __half *__restrict__ v16, int k_pad,
                                            int PR, int pipe, const S1Split sp = S1Split{nullptr, nullptr, 1},
                                            int part = 0) {
    const int KR = 64 * PR;
    uint32_t *sgn = reinterpret_cast<uint32_t *>(base);
    _Float16 *act = reinterpret_cast<_Float16 *>(base + static_cast<size_t>(PR) * 128 * RT);
    float *red = reinterpret_cast<float *>(base);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int li = lane & 15;
    const int j0 = blk * 16 * RT;
    const ExpandConsts ec = expand_consts<BIN>();

    float mid_pre[RT][4];  // epilogue scales, fetched early
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) mid_pre[t][v] = __half2float(mid[j0 + 16 * t + 4 * g + v]);

    f32x4 acc[Acc<NB>::N][RT];
#pragma unroll
    for (int c = 0; c < Acc<NB>::N; ++c)
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int npairs = Wm >> 1;
    // this part's word pairs [pb0, pb1) (batches below the parts' threshold
    // never take parts: their code keeps the whole range)
    constexpr bool kParts = NB >= DBF_DECODE_S1_SPLIT_MIN_NB;
    const int ngroups = (npairs + kNW - 1) / kNW;
    const int pb0 = kParts ? min(npairs, part * ngroups / sp.parts * kNW) : 0;
    const int pb1 = kParts ? min(npairs, (part + 1) * ngroups / sp.parts * kNW) : npairs;
    const bool xvec = (m & 7) == 0;
    // the loads of one batch: sign items and the x / b fragments of the round
    struct Batch {
        u32x4 v[kMaxItems];
        f16x8 xv[act_slots<NB>()], bv[act_slots<NB>()];
    };
    auto issue = [&](Batch &B, int pr0, int pr1, int item0, int act0, bool with_signs = true) {
        const int nitems = (pr1 - pr0) * 8 * RT;
        const int k0 = 64 * pr0, len = 64 * (pr1 - pr0);
        const int nact = NB * (len >> 3);  // 8-element activation items
        const int per_row = len >> 3;
        if (with_signs) load_sign_items<RT>(B.v, Bt, Wm, j0, pr0, nitems, item0);
        if (xvec) {
            // rows of x are 16-byte aligned: clamped, unconditional vector loads
#pragma unroll
            for (int q = 0; q < act_slots<NB>(); ++q) {
#if DBF_DECODE_TRIM_LOADS
                if (act0 + kThreads * q >= nact) break;
#endif
                const int it = min(act0 + static_cast<int>(threadIdx.x) + kThreads * q, nact - 1);
                const int r = NB == 1 ? 0 : it / per_row;
                const int l = k0 + (it - r * per_row) * 8;
                // columns past m (zero-padded b) read some valid x instead
                B.xv[q] = *reinterpret_cast<const f16x8 *>(x + static_cast<size_t>(r) * m + min(l, m - 8));
                B.bv[q] = *reinterpret_cast<const f16x8 *>(b + l);  // b is zero-padded to m_pad
            }
        } else {
#pragma unroll
            for (int q = 0; q < act_slots<NB>(); ++q) {
                const int it = min(act0 + static_cast<int>(threadIdx.x) + kThreads * q, nact - 1);
                const int r = NB == 1 ? 0 : it / per_row;
                const int l = k0 + (it - r * per_row) * 8;
                B.xv[q] = zero8();
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (l + e < m) B.xv[q][e] = static_cast<_Float16>(__half2float(x[static_cast<size_t>(r) * m + l + e]));
                B.bv[q] = *reinterpret_cast<const f16x8 *>(b + l);
            }
        }
    };
    auto stash = [&](const Batch &B, uint32_t *sgn_b, _Float16 *act_b, int pr0, int pr1, int item0, int act0,
                     bool with_signs = true) {
        const int nitems = (pr1 - pr0) * 8 * RT;
        const int len = 64 * (pr1 - pr0);
        const int nact = NB * (len >> 3);
        const int per_row = len >> 3;
        if (with_signs) store_sign_items(B.v, sgn_b, nitems, item0);
        if constexpr (Acc<NB>::kSP) {
            // x as it is (b goes into the signs); row 0's items also store b
#pragma unroll
            for (int q = 0; q < act_slots<NB>(); ++q) {
                const int it = act0 + threadIdx.x + kThreads * q;
                if (it < nact) {
                    const int r = it / per_row;
                    const int e = (it - r * per_row) * 8;
                    *reinterpret_cast<f16x8 *>(act_b + r * KR + e) = B.xv[q];
                    if (r == 0) *reinterpret_cast<f16x8 *>(act_b + NB * KR + e) = B.bv[q];
                }
            }
        } else {
            // u = x ⊙ b (exact in fp32) as hi/lo planes
#pragma unroll
            for (int q = 0; q < act_slots<NB>(); ++q) {
                const int it = act0 + threadIdx.x + kThreads * q;
                if (it < nact) {
                    const int r = NB == 1 ? 0 : it / per_row;
                    const int e = (it - r * per_row) * 8;
                    f16x8 hi, lo;
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const float u = static_cast<float>(B.xv[q][c]) * static_cast<float>(B.bv[q][c]);
                        hi[c] = static_cast<_Float16>(u);
                        lo[c] = static_cast<_Float16>(u - static_cast<float>(hi[c]));
                    }
                    *reinterpret_cast<f16x8 *>(act_b + r * KR + e) = hi;
                    *reinterpret_cast<f16x8 *>(act_b + (NB + r) * KR + e) = lo;
                }
            }
        }
    };
    if (pipe == 2) {
        // direct form: the activations of all of m in LDS, the signs straight to registers
        _Float16 *act_all = reinterpret_cast<_Float16 *>(base);
        const int nact = NB * 8 * (pb1 - pb0);
        for (int act0 = 0; act0 < nact; act0 += kThreads * act_slots<NB>()) {
            Batch B;
            issue(B, pb0, pb1, 0, act0, false);
            stash(B, nullptr, act_all, pb0, pb1, 0, act0, false);
        }
        __syncthreads();
        // (rows of act_all at the stride KR = 64 PR the plan sized for the largest part)
        direct_mma<NB, RT, true, BIN>(acc, Bt, Wm, j0, pb0, pb1 - pb0, act_all, KR, wave, li, g, ec);
    } else if (pipe) {
        // Rounds of PR pairs, each one batch, through two LDS buffers: the
        // loads of round r + 1 are in flight while round r is multiplied.
        const size_t RB = lds_round_bytes<NB, RT>(PR);
        const int nr = (pb1 - pb0 + PR - 1) / PR;
        Batch B;
        if (nr > 0) issue(B, pb0, min(pb0 + PR, pb1), 0, 0);
        for (int r = 0; r < nr; ++r) {
            const int pr0 = pb0 + r * PR, pr1 = min(pr0 + PR, pb1);
            char *buf = base + (r & 1) * RB;
            uint32_t *sgn_b = reinterpret_cast<uint32_t *>(buf);
            _Float16 *act_b = reinterpret_cast<_Float16 *>(buf + static_cast<size_t>(PR) * 128 * RT);
            stash(B, sgn_b, act_b, pr0, pr1, 0, 0);
            __syncthreads();  // round r staged; every wave is done with round r - 1's buffer
            if (r + 1 < nr) issue(B, pr1, min(pr1 + PR, pb1), 0, 0);
            round_mma<NB, RT, true, BIN>(acc, sgn_b, act_b, KR, pr0, pr1, wave, li, g, ec);
        }
    } else {
        for (int pr0 = pb0; pr0 < pb1; pr0 += PR) {
            const int pr1 = min(pr0 + PR, pb1);
            const int nitems = (pr1 - pr0) * 8 * RT;
            const int nact = NB * 8 * (pr1 - pr0);
            if (pr0 > pb0) __syncthreads();  // the previous round is done with LDS
            // Every load of a batch (sign items, x and b fragments) is issued
            // before any of it is used; one batch covers the layer shapes of
            // interest, so the workgroup waits for memory once per round.
            for (int item0 = 0, act0 = 0; item0 < nitems || act0 < nact;
                 item0 += kThreads * kMaxItems, act0 += kThreads * act_slots<NB>()) {
                Batch B;
                issue(B, pr0, pr1, item0, act0);
                stash(B, sgn, act, pr0, pr1, item0, act0);
            }
            __syncthreads();
            round_mma<NB, RT, true, BIN>(acc, sgn, act, KR, pr0, pr1, wave, li, g, ec);
        }
    }

    reduce_waves<NB, RT>(acc, red, wave, lane);
    f32x4 dsum[RT];
    if (kParts && sp.parts > 1) {
        // publish this part's sums, take a ticket; the last part of the row
        // block adds all parts in order (the flag overlays the reduction
        // slots, whose totals are read before it is written; a static LDS
        // variable would put the dynamic LDS off its 16-byte alignment)
        int &s_last = *reinterpret_cast<int *>(red);
        // The sums go out as agent-scope atomic stores (written through to
        // memory, where the other XCDs' agent-scope loads read them), and
        // the ticket is taken only after they have completed (vmcnt 0); no
        // release fence, whose write-back of the whole L2 costs microseconds
        // per workgroup on this chip.
        if (wave == 0 && li < NB) {
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const f32x4 d = total<NB, RT>(red, t, lane);
                float *dst = sp.part + (static_cast<size_t>(part) * NB + li) * k_pad + j0 + 16 * t + 4 * g;
#pragma unroll
                for (int v = 0; v < 4; ++v) __hip_atomic_store(dst + v, d[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // every counter: this thread's stores have completed
        __syncthreads();
        if (threadIdx.x == 0)
            s_last = __hip_atomic_fetch_add(&sp.tickets[blk], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     static_cast<unsigned>(sp.parts - 1);
        __syncthreads();
        if (!s_last) return;
        // The last part reads the others' sums.  Ordering: each part's stores
        // are agent-scope atomics, performed at the device's coherence point
        // (not in an XCD's L2), and its ticket is taken only after they have
        // completed (the vmcnt wait above, then the barrier); the ticket
        // itself is an agent-scope atomic at the same point.  So a part that
        // draws the last ticket does so after every part's stores are in
        // memory, and its reads below are agent-scope atomic loads, served at
        // that point too -- no line of its own XCD's caches can stand in for
        // them.  (An acquire fence here would invalidate that XCD's L2 as
        // well, where this launch has read stage 2's sign words ahead: it
        // measured 4-8 us slower on the 14336-wide layers at batch 8-16.)
        if (wave == 0 && li < NB) {
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                dsum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                for (int q = 0; q < sp.parts; ++q) {
                    const float *src = sp.part + (static_cast<size_t>(q) * NB + li) * k_pad + j0 + 16 * t + 4 * g;
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        dsum[t][v] += __hip_atomic_load(src + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        if (threadIdx.x == 0)  // ready for the next call
            __hip_atomic_store(&sp.tickets[blk], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // epilogue (wave 0): D[row 4g+v][col li] of row tile t is t[li][j0 + 16t + 4g + v]
    if (wave == 0 && li < NB) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int row0 = j0 + 16 * t + 4 * g;
            const f32x4 d = kParts && sp.parts > 1 ? dsum[t] : total<NB, RT>(red, t, lane);
            f16x4 hi, lo;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float val = fp32_value(d[v] * mid_pre[t][v]);
                hi[v] = static_cast<_Float16>(val);
                lo[v] = static_cast<_Float16>(val - static_cast<float>(hi[v]));
            }
            *reinterpret_cast<f16x4 *>(v16 + static_cast<size_t>(li) * k_pad + row0) = hi;
            if constexpr (!Acc<NB>::kSP)
                *reinterpret_cast<f16x4 *>(v16 + static_cast<size_t>(NB + li) * k_pad + row0) = lo;
        }
    }
}

// Stage 2 for row block `blk`: y = rne16(a ⊙ (A (v_hi + v_lo))) (single plane: A v).
template <int NB, int RT, bool BIN>
__device__ __forceinline__ void stage2_body(int blk, char *base, const uint32_t *__restrict__ At, int Wk,
                                            const __half *__restrict__ v16, int k_pad, const __half *__restrict__ a,
                                            __half *__restrict__ y, int n, int PR, int pipe,
                                            const float *__restrict__ aff_E, const float *__restrict__ aff_stats) {
    const int KR = 64 * PR;
    uint32_t *sgn = reinterpret_cast<uint32_t *>(base);
    _Float16 *act = reinterpret_cast<_Float16 *>(base + static_cast<size_t>(PR) * 128 * RT);
    float *red = reinterpret_cast<float *>(base);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int li = lane & 15;
    const int i0 = blk * 16 * RT;
    const ExpandConsts ec = expand_consts<BIN>();

    float a_pre[RT][4];  // epilogue scales, fetched early
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = i0 + 16 * t + 4 * g + v;
            a_pre[t][v] = row < n ? __half2float(a[row]) : 0.0f;
        }
    // affine term (if any), fetched early too: E of this lane's rows, the
    // row sums of batch row li
    float e_pre[RT][4];
    float2 st = float2{0.0f, 0.0f};
    if (aff_E) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = i0 + 16 * t + 4 * g + v;
                e_pre[t][v] = row < n ? aff_E[row] : 0.0f;
            }
        if (li < NB) st = *reinterpret_cast<const float2 *>(aff_stats + 2 * li);
    }

    f32x4 acc[Acc<NB>::N][RT];
#pragma unroll
    for (int c = 0; c < Acc<NB>::N; ++c)
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int npairs = Wk >> 1;
    constexpr int kPlanes = Acc<NB>::kSP ? 1 : 2;  // hi and lo rows (one plane in the single-plane form)
    struct Batch {
        u32x4 v[kMaxItems];
        f16x8 av[act_slots<NB>()];
    };
    auto issue = [&](Batch &B, int pr0, int pr1, int item0, int act0, bool with_signs = true) {
        const int nitems = (pr1 - pr0) * 8 * RT;
        const int k0 = 64 * pr0, len = 64 * (pr1 - pr0);
        const int nact = kPlanes * NB * (len >> 3);  // 16-byte plane items: hi rows then lo rows
        const int per_row = len >> 3;
        if (with_signs) load_sign_items<RT>(B.v, At, Wk, i0, pr0, nitems, item0);
#pragma unroll
        for (int q = 0; q < act_slots<NB>(); ++q) {
#if DBF_DECODE_TRIM_LOADS
            if (act0 + kThreads * q >= nact) break;
#endif
            const int it = min(act0 + static_cast<int>(threadIdx.x) + kThreads * q, nact - 1);
            const int r = it / per_row;
            const int e = (it - r * per_row) * 8;
            B.av[q] = *reinterpret_cast<const f16x8 *>(v16 + static_cast<size_t>(r) * k_pad + k0 + e);
        }
    };
    auto stash = [&](const Batch &B, uint32_t *sgn_b, _Float16 *act_b, int pr0, int pr1, int item0, int act0,
                     bool with_signs = true) {
        const int nitems = (pr1 - pr0) * 8 * RT;
        const int len = 64 * (pr1 - pr0);
        const int nact = kPlanes * NB * (len >> 3);
        const int per_row = len >> 3;
        if (with_signs) store_sign_items(B.v, sgn_b, nitems, item0);
#pragma unroll
        for (int q = 0; q < act_slots<NB>(); ++q) {
            const int it = act0 + threadIdx.x + kThreads * q;
            if (it < nact) {
                const int r = it / per_row;
                const int e = (it - r * per_row) * 8;
                *reinterpret_cast<f16x8 *>(act_b + r * KR + e) = B.av[q];
            }
        }
    };
    if (pipe == 2) {
        // direct form: v of all of k in LDS, the signs straight to registers
        _Float16 *act_all = reinterpret_cast<_Float16 *>(base);
        const int nact = kPlanes * NB * 8 * npairs;
        for (int act0 = 0; act0 < nact; act0 += kThreads * act_slots<NB>()) {
            Batch B;
            issue(B, 0, npairs, 0, act0, false);
            stash(B, nullptr, act_all, 0, npairs, 0, act0, false);
        }
        __syncthreads();
        direct_mma<NB, RT, false, BIN>(acc, At, Wk, i0, 0, npairs, act_all, 64 * npairs, wave, li, g, ec);
    } else if (pipe) {
        // two LDS buffers: round r + 1's loads in flight while round r is multiplied
        const size_t RB = lds_round_bytes<NB, RT>(PR);
        const int nr = (npairs + PR - 1) / PR;
        Batch B;
        issue(B, 0, min(PR, npairs), 0, 0);
        for (int r = 0; r < nr; ++r) {
            const int pr0 = r * PR, pr1 = min(pr0 + PR, npairs);
            char *buf = base + (r & 1) * RB;
            uint32_t *sgn_b = reinterpret_cast<uint32_t *>(buf);
            _Float16 *act_b = reinterpret_cast<_Float16 *>(buf + static_cast<size_t>(PR) * 128 * RT);
            stash(B, sgn_b, act_b, pr0, pr1, 0, 0);
            __syncthreads();  // round r staged; every wave is done with round r - 1's buffer
            if (r + 1 < nr) issue(B, pr1, min(pr1 + PR, npairs), 0, 0);
            round_mma<NB, RT, false, BIN>(acc, sgn_b, act_b, KR, pr0, pr1, wave, li, g, ec);
        }
    } else {
        for (int pr0 = 0; pr0 < npairs; pr0 += PR) {
            const int pr1 = min(pr0 + PR, npairs);
            const int nitems = (pr1 - pr0) * 8 * RT;
            const int nact = kPlanes * NB * 8 * (pr1 - pr0);
            if (pr0 > 0) __syncthreads();
            // all loads of a batch (sign items, v_hi / v_lo items) are issued first
            for (int item0 = 0, act0 = 0; item0 < nitems || act0 < nact;
                 item0 += kThreads * kMaxItems, act0 += kThreads * act_slots<NB>()) {
                Batch B;
                issue(B, pr0, pr1, item0, act0);
                stash(B, sgn, act, pr0, pr1, item0, act0);
            }
            __syncthreads();
            round_mma<NB, RT, false, BIN>(acc, sgn, act, KR, pr0, pr1, wave, li, g, ec);
        }
    }

    reduce_waves<NB, RT>(acc, red, wave, lane);
    if (wave == 0 && li < NB) {
        // affine term (if any): E[row] * stats[li].x + stats[li].y, added before the one rounding
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int row0 = i0 + 16 * t + 4 * g;
            const f32x4 d = total<NB, RT>(red, t, lane);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = row0 + v;
                if (row < n) {
                    float val = fp32_value(d[v] * a_pre[t][v]);
                    if (aff_E) val = fp32_value(val + (e_pre[t][v] * st.x + st.y));
                    y[static_cast<size_t>(li) * n + row] = __float2half_rn(val);
                }
            }
        }
    }
}

// Read-ahead of the stage-2 sign words.  Stage 1 of a layer at decode sizes
// leaves CUs idle (k / 16 row blocks); extra workgroups of the stage-1
// launch read the words stage 2 will read, so that stage 2 finds them in a
// cache instead of HBM.  Workgroups are dispatched round-robin over the 8
// XCDs, so read-ahead workgroup number g (XCD g mod 8) reads the rows of the
// stage-2 workgroups on that same XCD, whose L2 then holds them; the
// Infinity Cache, shared by all XCDs, holds them too.
struct Stage2Readahead {
    const uint4 *A;    // tiled sign words of A, as 16-byte items
    int pairs;         // word pairs per row
    int rows_per_wg;   // rows of one stage-2 workgroup (16 * RT)
    int groups;        // stage-2 workgroups
    int per_xcd;       // read-ahead workgroups per XCD
};

__device__ __forceinline__ void readahead_stage2(const Stage2Readahead &ra, int g /* launch-wide block index */,
                                                 int q /* index among this XCD's read-ahead blocks */) {
    const int xcd = g & 7;
    const int half = ra.rows_per_wg >> 1;  // 16-byte items per word pair of one workgroup
    const int per_wg = ra.pairs * half;
    const int nwg = (ra.groups - xcd + 7) >> 3;  // stage-2 workgroups b with b mod 8 == xcd
    const int total = nwg * per_wg;
    if (total == 0) return;
    const int stride = ra.per_xcd * kThreads;
    uint32_t acc = 0;
    // batches of kReadaheadBatch loads in flight; indexes past the end are
    // clamped to the last item (straight-line code, no waits between loads)
    for (int i0 = q * kThreads + static_cast<int>(threadIdx.x); i0 < total; i0 += kReadaheadBatch * stride) {
        uint4 v[kReadaheadBatch];
#pragma unroll
        for (int u = 0; u < kReadaheadBatch; ++u) {
            const int i = min(i0 + u * stride, total - 1);
            const int j = i / per_wg, rem = i - j * per_wg;
            const int row0 = (xcd + 8 * j) * ra.rows_per_wg;
            const int pr = rem / half, e = rem - pr * half;
            v[u] = ra.A[((static_cast<size_t>(row0 >> 6) * ra.pairs + pr) * 64 + (row0 & 63)) / 2 + e];
        }
#pragma unroll
        for (int u = 0; u < kReadaheadBatch; ++u) acc ^= v[u].x ^ v[u].w;
    }
    asm volatile("" ::"v"(acc));  // the loads are the point: keep them
}

// Stage 1; workgroups past the (row block, part) ones read ahead for stage 2.
template <int NB, int RT, bool BIN>
__global__ __launch_bounds__(kThreads) void mfma_stage1_kernel(const uint32_t *__restrict__ Bt, int Wm,
                                                               const __half *__restrict__ x, int m,
                                                               const __half *__restrict__ b,
                                                               const __half *__restrict__ mid,
                                                               __half *__restrict__ v16, int k_pad, int PR, int pipe,
                                                               const Stage2Readahead ra,
                                                               const float *__restrict__ gamma,
                                                               float *__restrict__ stats, const S1Split sp) {
    extern __shared__ float lds[];
    const int G1 = k_pad / (16 * RT);
    const int GC = G1 * sp.parts;  // (row block, part) workgroups, row block fastest
    if (static_cast<int>(blockIdx.x) >= GC) {
        const int extra = blockIdx.x - GC;
        if (BIN && extra >= 8 * ra.per_xcd) {
            // 0/1 layers: one block per batch row forms the row sums of x
            const int r = extra - 8 * ra.per_xcd;
            bqq_rowstats_row<kThreads>(x + static_cast<size_t>(r) * m, m, gamma, stats + 2 * r, lds);
            return;
        }
        readahead_stage2(ra, blockIdx.x, extra >> 3);
        return;
    }
    stage1_body<NB, RT, BIN>(blockIdx.x % G1, reinterpret_cast<char *>(lds), Bt, Wm, x, m, b, mid, v16, k_pad, PR,
                             pipe, sp, blockIdx.x / G1);
}

template <int NB, int RT, bool BIN>
__global__ __launch_bounds__(kThreads) void mfma_stage2_kernel(const uint32_t *__restrict__ At, int Wk,
                                                               const __half *__restrict__ v16, int k_pad,
                                                               const __half *__restrict__ a,
                                                               __half *__restrict__ y, int n, int PR, int pipe,
                                                               const float *__restrict__ aff_E,
                                                               const float *__restrict__ aff_stats) {
    extern __shared__ float lds[];
    stage2_body<NB, RT, BIN>(blockIdx.x, reinterpret_cast<char *>(lds), At, Wk, v16, k_pad, a, y, n, PR, pipe, aff_E,
                             aff_stats);
}

// Grouped form: one launch runs a stage for several layers that share the
// input.  Workgroup b belongs to the last layer whose first block blk0 <= b.
struct GroupStage1Layer {
    const uint32_t *Bt;
    const __half *b, *mid;
    __half *v16;
    int k_pad, blk0;
};
struct GroupStage1Args {
    GroupStage1Layer L[kMaxGroup];
    int count;
    const __half *x;
    int m, Wm, PR, pipe;
};
struct GroupStage2Layer {
    const uint32_t *At;
    const __half *v16, *a;
    __half *y;
    int Wk, k_pad, n, PR, pipe, blk0;
};
struct GroupStage2Args {
    GroupStage2Layer L[kMaxGroup];
    int count;
};

template <typename A>
__device__ __forceinline__ int group_layer(const A &g) {
    int l = 0;
    for (int i = 1; i < g.count; ++i)
        if (static_cast<int>(blockIdx.x) >= g.L[i].blk0) l = i;
    return l;
}

template <int NB, int RT>
__global__ __launch_bounds__(kThreads) void mfma_group_stage1_kernel(const GroupStage1Args g) {
    extern __shared__ float lds[];
    const int l = group_layer(g);
    const GroupStage1Layer &L = g.L[l];
    stage1_body<NB, RT, false>(blockIdx.x - L.blk0, reinterpret_cast<char *>(lds), L.Bt, g.Wm, g.x, g.m, L.b, L.mid,
                               L.v16, L.k_pad, g.PR, g.pipe);
}

template <int NB, int RT>
__global__ __launch_bounds__(kThreads) void mfma_group_stage2_kernel(const GroupStage2Args g) {
    extern __shared__ float lds[];
    const int l = group_layer(g);
    const GroupStage2Layer &L = g.L[l];
    stage2_body<NB, RT, false>(blockIdx.x - L.blk0, reinterpret_cast<char *>(lds), L.At, L.Wk, L.v16, L.k_pad, L.a,
                               L.y, L.n, L.PR, L.pipe, nullptr, nullptr);
}

template <typename K>
void allow_lds(K kernel, size_t bytes) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(bytes));
}

#ifndef DBF_DECODE_PIPE_KB
#define DBF_DECODE_PIPE_KB 16
#endif
#ifndef DBF_DECODE_PIPE_ROUNDS
#define DBF_DECODE_PIPE_ROUNDS 3
#endif

// Rounds of a stage: in the single-plane form a workgroup whose block of sign words
// reaches DBF_DECODE_PIPE_KB takes it in at least DBF_DECODE_PIPE_ROUNDS
// rounds, each one batch of loads, through two LDS buffers (the next round's
// loads fly while the current round is multiplied); otherwise one round when
// LDS allows.  (Measured: at batch 16 the MLP layers gain 6-10 %; in the
// hi/lo form, where a round's MFMA work is shorter than the memory latency,
// the extra round trips cost more than the overlap saves.)  act_rows: activation
// rows staged per word pair.
struct RoundPlan {
    int PR, pipe;
    size_t lds;
};
#ifndef DBF_DECODE_DIRECT
#define DBF_DECODE_DIRECT 1
#endif
#ifndef DBF_DECODE_DIRECT_MIN_NB
#define DBF_DECODE_DIRECT_MIN_NB 2
#endif
template <int NB, int RT>
RoundPlan plan_rounds(int npairs, int act_rows, int lds_rows) {
    RoundPlan p{};
    const int budget = round_pairs<NB, RT>();
    // Direct form at batch >= 2 when the activations of the whole reduction
    // dimension (lds_rows rows of 64 halves per pair) fit LDS.  (Measured:
    // 4096x4096 k = 2048 at batch 16, 19.4 -> 15.1 us per forward, batch 4
    // 11.5 -> 10.9 us; at batch 1 the one-shot staging through LDS is as
    // fast or faster -- 8 times fewer load instructions for the big layers.)
    const size_t act_all = static_cast<size_t>(lds_rows) * 64 * npairs * sizeof(_Float16);
    if (DBF_DECODE_DIRECT && NB >= DBF_DECODE_DIRECT_MIN_NB && act_all + kLdsTail <= kLdsBudget) {
        p.PR = npairs;
        p.pipe = 2;
        p.lds = std::max(act_all, lds_reduce_bytes<NB, RT>()) + kLdsTail;
        return p;
    }
    if (Acc<NB>::kSP && DBF_DECODE_PIPE_KB > 0 &&
        static_cast<size_t>(npairs) * 128 * RT >= size_t(DBF_DECODE_PIPE_KB) * 1024) {
        const int cap = std::min({budget / 2, kThreads * kMaxItems / (8 * RT), kThreads * act_slots<NB>() / (8 * act_rows)});
        if (cap >= 1) {
            const int nr = std::max(DBF_DECODE_PIPE_ROUNDS, (npairs + cap - 1) / cap);
            p.PR = std::min(cap, ((npairs + nr - 1) / nr + kNW - 1) / kNW * kNW);  // whole waves' worth
            p.pipe = 1;
            p.lds = std::max(2 * lds_round_bytes<NB, RT>(p.PR), lds_reduce_bytes<NB, RT>()) + kLdsTail;
            return p;
        }
    }
    p.PR = std::min(npairs, budget);
    p.pipe = 0;
    p.lds = lds_bytes<NB, RT>(p.PR);
    return p;
}

// Rows per workgroup: 16, 32 or 64, the smallest that keeps the grid within
// one workgroup per CU of the 256-CU MI355X.  Every workgroup stages the
// whole activation block, so fewer, taller workgroups also cut that traffic.
int split_rt(int rows) {
    if (rows / 16 <= DBF_DECODE_ONE_ROUND) return 1;
    if (rows / 32 <= DBF_DECODE_ONE_ROUND) return 2;
    return 4;
}

// Stage 1's reduction cut into parts (batch >= 2, signed layers): where m
// spans at least DBF_DECODE_S1_SPLIT_PAIRS word pairs, 3 or else 2 parts
// with the smallest rows per workgroup that keep (row block, part)
// workgroups within the CUs.  At batch 16 the 14336-wide activations (458
// KiB) do not fit LDS and each workgroup streamed all of them in rounds that
// wait on memory; a part streams a third of them, on three times the CUs.

struct S1Plan {
    int rt, parts;
};
S1Plan s1_plan(int m_pad, int k_pad) {
    S1Plan p{split_rt(k_pad), 1};
    if (DBF_DECODE_S1_SPLIT_PAIRS <= 0 || m_pad / 64 < DBF_DECODE_S1_SPLIT_PAIRS) return p;
    for (int parts = 3; parts >= 2; --parts)
        for (int rt = 1; rt <= 4; rt *= 2)
            if ((k_pad / (16 * rt)) * parts <= kCUs) return S1Plan{rt, parts};
    return p;
}

}  // namespace

int mfma_stage1_parts(int m_pad, int k_pad, int batch) {
    if (batch < DBF_DECODE_S1_SPLIT_MIN_NB) return 1;
    return s1_plan(m_pad, k_pad).parts;
}

namespace {

template <int NB, int RT, bool BIN>
int launch_rt(const MfmaDecodeArgs &d, hipStream_t s, int which, int parts = 1) {
    if (which == 1) {
        static const bool once = (allow_lds(mfma_stage1_kernel<NB, RT, BIN>, kLdsBudget), true);
        (void)once;
        // the largest part's word pairs (parts take whole groups of kNW pairs)
        const int npairs = d.m_pad / 64;
        const int part_pairs = std::min(npairs, ((npairs + kNW - 1) / kNW + parts - 1) / parts * kNW);
        const RoundPlan rp = plan_rounds<NB, RT>(part_pairs, NB, Acc<NB>::kSP ? NB + 1 : 2 * NB);
        const int G1 = d.k_pad / (16 * RT);
        const int GC = G1 * parts;
        Stage2Readahead ra{};
        ra.A = reinterpret_cast<const uint4 *>(d.A_dev);
        ra.pairs = d.k_pad / 64;
        const int rt2 = split_rt(d.n_pad);
        ra.rows_per_wg = 16 * rt2;
        ra.groups = d.n_pad / (16 * rt2);
        // 0/1 layers add one block per batch row for the row sums of x
        const int stat_blocks = BIN ? NB : 0;
        // the read-ahead blocks take the CUs stage 1 and the row-sum blocks
        // leave free (a block beyond one per CU would wait for a CU: the
        // kernel's registers allow one block per CU), if there are enough of
        // them to read stage 2's words in a few batches
        ra.per_xcd = kReadahead ? std::max(0, (kCUs - GC - stat_blocks) / 8) : 0;  // none when stage 1 fills the CUs
        if (ra.per_xcd > 0) {
            const size_t items = static_cast<size_t>(d.n_pad) * (d.k_pad / 32) / 4;
            if (items > static_cast<size_t>(kReadaheadMax) * 8 * ra.per_xcd * kThreads) ra.per_xcd = 0;
        }
        // the read-ahead blocks start on XCD GC mod 8; 8 * per_xcd of them cover every XCD equally
        launch_kernel((mfma_stage1_kernel<NB, RT, BIN>), dim3(GC + 8 * ra.per_xcd + stat_blocks), dim3(kThreads),
                      rp.lds, s, d.B_dev, d.m_pad / 32, static_cast<const __half *>(d.x), d.m,
                      static_cast<const __half *>(d.b_dev), static_cast<const __half *>(d.mid_dev),
                      reinterpret_cast<__half *>(d.v16), d.k_pad, rp.PR, rp.pipe, ra, d.gamma, d.stats_out,
                      S1Split{d.s1_part, d.s1_tickets, parts});
    } else {
        static const bool once = (allow_lds(mfma_stage2_kernel<NB, RT, BIN>, kLdsBudget), true);
        (void)once;
        const RoundPlan rp = plan_rounds<NB, RT>(d.k_pad / 64, (Acc<NB>::kSP ? 1 : 2) * NB, (Acc<NB>::kSP ? 1 : 2) * NB);
        launch_kernel((mfma_stage2_kernel<NB, RT, BIN>), dim3(d.n_pad / (16 * RT)), dim3(kThreads), rp.lds, s,
                      d.A_dev, d.k_pad / 32, reinterpret_cast<const __half *>(d.v16), d.k_pad,
                      static_cast<const __half *>(d.a_dev), static_cast<__half *>(d.y), d.n, rp.PR, rp.pipe,
                      d.aff_E, d.aff_stats);
    }
    return static_cast<int>(hipGetLastError());
}

template <int NB>
int launch_nb(const MfmaDecodeArgs &d, hipStream_t s, int which) {
    int rt = split_rt(which == 1 ? d.k_pad : d.n_pad);
    if (which == 1 && !d.binary && mfma_stage1_parts(d.m_pad, d.k_pad, NB) > 1) {
        const S1Plan p = s1_plan(d.m_pad, d.k_pad);
        if (!d.s1_part || !d.s1_tickets || static_cast<size_t>(p.parts) * NB * d.k_pad > d.s1_part_cap ||
            d.k_pad / (16 * p.rt) > d.s1_ntickets)
            return static_cast<int>(hipErrorInvalidValue);  // the handle's workspace is sized for the parts
        if (p.rt == 1) return launch_rt<NB, 1, false>(d, s, which, p.parts);
        if (p.rt == 2) return launch_rt<NB, 2, false>(d, s, which, p.parts);
        return launch_rt<NB, 4, false>(d, s, which, p.parts);
    }
    if (d.binary) {
        if (rt == 2) return launch_rt<NB, 2, true>(d, s, which);
        if (rt == 4) return launch_rt<NB, 4, true>(d, s, which);
        return launch_rt<NB, 1, true>(d, s, which);
    }
    if (rt == 2) return launch_rt<NB, 2, false>(d, s, which);
    if (rt == 4) return launch_rt<NB, 4, false>(d, s, which);
    return launch_rt<NB, 1, false>(d, s, which);
}

template <int NB, int RT>
int launch_group_rt(const MfmaGroupArgs &g, hipStream_t s, int which) {
    if (which == 1) {
        static const bool once = (allow_lds(mfma_group_stage1_kernel<NB, RT>, kLdsBudget), true);
        (void)once;
        GroupStage1Args a{};
        a.count = g.count;
        a.x = static_cast<const __half *>(g.x);
        a.m = g.m;
        a.Wm = g.m_pad / 32;
        const RoundPlan rp = plan_rounds<NB, RT>(g.m_pad / 64, NB, Acc<NB>::kSP ? NB + 1 : 2 * NB);
        a.PR = rp.PR;
        a.pipe = rp.pipe;
        int blocks = 0;
        for (int i = 0; i < g.count; ++i) {
            const MfmaGroupLayer &L = g.L[i];
            a.L[i] = {L.B_dev, static_cast<const __half *>(L.b_dev), static_cast<const __half *>(L.mid_dev),
                      reinterpret_cast<__half *>(L.v16), L.k_pad, blocks};
            blocks += L.k_pad / (16 * RT);
        }
        launch_kernel((mfma_group_stage1_kernel<NB, RT>), dim3(blocks), dim3(kThreads), rp.lds, s, a);
    } else {
        static const bool once = (allow_lds(mfma_group_stage2_kernel<NB, RT>, kLdsBudget), true);
        (void)once;
        GroupStage2Args a{};
        a.count = g.count;
        int blocks = 0;
        size_t lds = 0;
        for (int i = 0; i < g.count; ++i) {
            const MfmaGroupLayer &L = g.L[i];
            const RoundPlan rp =
                plan_rounds<NB, RT>(L.k_pad / 64, (Acc<NB>::kSP ? 1 : 2) * NB, (Acc<NB>::kSP ? 1 : 2) * NB);
            a.L[i] = {L.A_dev, reinterpret_cast<const __half *>(L.v16), static_cast<const __half *>(L.a_dev),
                      static_cast<__half *>(L.y), L.k_pad / 32, L.k_pad, L.n, rp.PR, rp.pipe, blocks};
            blocks += L.n_pad / (16 * RT);
            lds = std::max(lds, rp.lds);
        }
        launch_kernel((mfma_group_stage2_kernel<NB, RT>), dim3(blocks), dim3(kThreads), lds, s, a);
    }
    return static_cast<int>(hipGetLastError());
}

template <int NB>
int launch_group_nb(const MfmaGroupArgs &g, hipStream_t s, int which) {
    int rows = 0;
    for (int i = 0; i < g.count; ++i) rows += which == 1 ? g.L[i].k_pad : g.L[i].n_pad;
    const int rt = split_rt(rows);
    if (rt == 2) return launch_group_rt<NB, 2>(g, s, which);
    if (rt == 4) return launch_group_rt<NB, 4>(g, s, which);
    return launch_group_rt<NB, 1>(g, s, which);
}

}  // namespace

int launch_mfma_decode(const MfmaDecodeArgs &d, void *stream, int which) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (d.batch) {
        case 1: return launch_nb<1>(d, s, which);
        case 2: return launch_nb<2>(d, s, which);
        case 3: return launch_nb<3>(d, s, which);
        case 4: return launch_nb<4>(d, s, which);
        case 5: return launch_nb<5>(d, s, which);
        case 6: return launch_nb<6>(d, s, which);
        case 7: return launch_nb<7>(d, s, which);
        case 8: return launch_nb<8>(d, s, which);
        case 9: return launch_nb<9>(d, s, which);
        case 10: return launch_nb<10>(d, s, which);
        case 11: return launch_nb<11>(d, s, which);
        case 12: return launch_nb<12>(d, s, which);
        case 13: return launch_nb<13>(d, s, which);
        case 14: return launch_nb<14>(d, s, which);
        case 15: return launch_nb<15>(d, s, which);
        case 16: return launch_nb<16>(d, s, which);
        default: return static_cast<int>(hipErrorInvalidValue);
    }
}

int launch_mfma_decode_group(const MfmaGroupArgs &g, void *stream, int which) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (g.count < 1 || g.count > kMaxGroup) return static_cast<int>(hipErrorInvalidValue);
    switch (g.batch) {
        case 1: return launch_group_nb<1>(g, s, which);
        case 2: return launch_group_nb<2>(g, s, which);
        case 3: return launch_group_nb<3>(g, s, which);
        case 4: return launch_group_nb<4>(g, s, which);
        case 5: return launch_group_nb<5>(g, s, which);
        case 6: return launch_group_nb<6>(g, s, which);
        case 7: return launch_group_nb<7>(g, s, which);
        case 8: return launch_group_nb<8>(g, s, which);
        case 9: return launch_group_nb<9>(g, s, which);
        case 10: return launch_group_nb<10>(g, s, which);
        case 11: return launch_group_nb<11>(g, s, which);
        case 12: return launch_group_nb<12>(g, s, which);
        case 13: return launch_group_nb<13>(g, s, which);
        case 14: return launch_group_nb<14>(g, s, which);
        case 15: return launch_group_nb<15>(g, s, which);
        case 16: return launch_group_nb<16>(g, s, which);
        default: return static_cast<int>(hipErrorInvalidValue);
    }
}

}  // namespace dbf
