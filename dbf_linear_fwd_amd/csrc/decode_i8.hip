// Decode path at batch 1 of the DBF linear forward, on the CDNA4 int8 matrix
// cores.
//
// §2.1 of the gist.science technical summary of "Addition is almost all you
// need" evaluates x W^T as ((((x ⊙ bᵀ) Bᵀ) ⊙ midᵀ) Aᵀ) ⊙ aᵀ.  Here that is two
// launches of one kernel: stage 1 forms v = mid ⊙ (B u) with u = x ⊙ b, stage
// 2 forms y = rne16(a ⊙ (A v)).  Each stage is a signed sum of one vector
// (u, or v) per output row.
//
// Numerics: the signed sums are exact integer sums of a fixed-point vector.
//   Each workgroup brings the whole vector to 32-bit fixed point with one
//   exponent S for all of it: q_l = rne(u_l 2^S), S chosen so that
//   2^29 <= max_l |u_l 2^S| < 2^30 (u = x ⊙ b is exact in fp32; so is any
//   power-of-two scaling of it).  Then s_r = Σ_l sign_rl q_l is an exact
//   integer, formed as U - 2 Z_r with U = Σ_l q_l and Z_r = Σ_{bit_rl = 1} q_l
//   (bit 1 means -1), and the stage result s_r 2^-S is exact in fp64
//   (|s_r| < 2^53).  The only roundings: q (2^-31 of the vector's largest
//   entry, at most), v = rne32(t mid) between the stages, and one
//   correctly rounded conversion of a s to fp16 at the end.  The result of a
//   row does not depend on how the reduction is cut among waves or
//   workgroups (every partial sum is exact).
//
// Matrix-core mapping (v_mfma_i32_16x16x64_i8: D 16x16 += A 16x64 * B 64x16).
//   B operand: q as four balanced base-256 digits, q = d0 + 2^8 d1 + 2^16 d2
//   + 2^24 d3 with every d in [-128, 127], in columns c = 0..3 (columns 4..15
//   are not used at batch 1).  A operand: the sign bits as int8 values 0 or
//   2^j.  A 32-bit word of signs AND 0x01010101 << j keeps its bits j, 8+j,
//   16+j, 24+j as four int8 values in {0, 2^j} (j = 7: {0, -128}) -- one VALU
//   instruction per four signs; the layout (pack.cpp, dbf_layout_signs_dec)
//   places the bits so that these are the columns the B operand holds.  One
//   accumulator per j; at the end of a tile Z_c = Σ_j ±acc_j >> j (exact:
//   acc_j is a multiple of 2^j) and Z = Σ_c Z_c 2^(8 c).
//
// Work split.  A workgroup (8 waves) owns a contiguous range of at most 8
// tiles of 16 rows; wave w takes superchunks [w SC / 8, (w+1) SC / 8) of
// every tile (a superchunk is 512 reduction columns, 1 KiB of signs per
// tile).  Each wave streams its sign words straight from global memory into
// registers, two groups of four superchunks in flight, the first group
// issued before the vector prologue; the digits of the whole vector sit in
// LDS.  The waves' partial Z of a tile meet in LDS; the last wave to arrive
// (an LDS counter) finishes the tile.  No barrier after the prologue.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>

#include "bqq_rowstats.h"
#include "dbf_internal.h"

namespace dbf {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kW = 8;                 // waves per workgroup
constexpr int kT = kW * 64;           // threads per workgroup
constexpr int kTilesWG = 8;           // 16-row tiles per workgroup, at most
constexpr int kCUs = 256;             // MI355X
constexpr int kActSC = 2048;          // LDS bytes of digits per superchunk: [8 j][4 g][4 c][16]
constexpr int kPartBytes = kTilesWG * kW * 16 * 4 * 4;  // [tile][wave][row][c] int32
constexpr int kMiscBytes = 128 + 2 * kTilesWG * 16 * 4;  // counters, reduction slots, row scales
constexpr int kPipe = 4;              // superchunks per load group (two groups in flight)

__host__ __device__ constexpr size_t lds_bytes_for(int SC) {
    return static_cast<size_t>(SC) * kActSC + kPartBytes + kMiscBytes;
}

// Raw loads of four consecutive entries base .. base + 3 (base a multiple of
// 4) of the stage's vector: stage 1, x and b (fp16); stage 2, v (fp32).
// Entries at or past K read as 0.  Runs entirely past K load entry 0 (a
// valid address) and are zeroed after the load, so that every load is
// unconditional; when K is not a multiple of 4 (stage 1 only) the entries
// are loaded one by one, each index clamped.
struct Run {
    uint32_t r[4];
};
template <int STAGE, bool K4>
__device__ __forceinline__ Run load_run(const I8Layer &L, int base) {
    Run o;
    const bool in = base < L.K;
    const int bb = in ? base : 0;
    if constexpr (STAGE == 1) {
        const __half *x = static_cast<const __half *>(L.vec);
        if constexpr (K4) {
            const uint2 xv = *reinterpret_cast<const uint2 *>(x + bb);
            const uint2 bv = *reinterpret_cast<const uint2 *>(L.bsc + bb);
            o.r[0] = in ? xv.x : 0u;
            o.r[1] = in ? xv.y : 0u;
            o.r[2] = in ? bv.x : 0u;
            o.r[3] = in ? bv.y : 0u;
        } else {
            const uint16_t *xs = static_cast<const uint16_t *>(L.vec);
            const uint16_t *bs = reinterpret_cast<const uint16_t *>(L.bsc);
            uint32_t xe[4], be[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = base + e < L.K;
                const int idx = ok ? base + e : 0;
                xe[e] = ok ? xs[idx] : 0u;
                be[e] = ok ? bs[idx] : 0u;
            }
            o.r[0] = xe[0] | (xe[1] << 16);
            o.r[1] = xe[2] | (xe[3] << 16);
            o.r[2] = be[0] | (be[1] << 16);
            o.r[3] = be[2] | (be[3] << 16);
        }
    } else {
        const float4 t = *reinterpret_cast<const float4 *>(static_cast<const float *>(L.vec) + bb);
        o.r[0] = in ? __float_as_uint(t.x) : 0u;
        o.r[1] = in ? __float_as_uint(t.y) : 0u;
        o.r[2] = in ? __float_as_uint(t.z) : 0u;
        o.r[3] = in ? __float_as_uint(t.w) : 0u;
    }
    return o;
}

// The four fp32 entries of a run: stage 1, x ⊙ b (exact); stage 2, v.
template <int STAGE>
__device__ __forceinline__ void run_values(const Run &o, float (&u)[4]) {
    if constexpr (STAGE == 1) {
        const __half2 x01 = __builtin_bit_cast(__half2, o.r[0]), x23 = __builtin_bit_cast(__half2, o.r[1]);
        const __half2 b01 = __builtin_bit_cast(__half2, o.r[2]), b23 = __builtin_bit_cast(__half2, o.r[3]);
        u[0] = __low2float(x01) * __low2float(b01);
        u[1] = __high2float(x01) * __high2float(b01);
        u[2] = __low2float(x23) * __low2float(b23);
        u[3] = __high2float(x23) * __high2float(b23);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = __uint_as_float(o.r[e]);
    }
}

// The fp16 value nearest to d (ties to even), without a double rounding:
// d is first cut to fp32 toward zero with a sticky last bit (round to odd),
// which keeps the information the final rounding to 11 bits needs.
__device__ __forceinline__ __half rne16_of(double d) {
    float f = __double2float_rz(d);
    if (static_cast<double>(f) != d) f = __uint_as_float(__float_as_uint(f) | 1u);
    return __float2half_rn(f);
}

template <int STAGE, bool BIN, bool K4, int NBLK>
__global__ __launch_bounds__(kT) void dec_i8_kernel(const I8Args args) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int bid = blockIdx.x;
    if (BIN && bid == args.stat_wg) {
        // 0/1 layers: the per-row input sums of the affine term
        bqq_rowstats_row<kT>(args.stat_x, args.stat_m, args.gamma, args.stats, reinterpret_cast<float *>(lds));
        return;
    }
    int li = 0;
    for (int i = 1; i < args.count; ++i)
        if (bid >= args.L[i].wg0) li = i;
    const I8Layer &L = args.L[li];
    const int wg = bid - L.wg0;
    const int tA = static_cast<int>(static_cast<long long>(wg) * L.ntiles / L.nwg);
    const int nt = static_cast<int>(static_cast<long long>(wg + 1) * L.ntiles / L.nwg) - tA;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int SC = L.SC;
    const int tile_words = 256 * (SC - 1) + 64 * L.wlast;

    char *act = lds;
    int *part = reinterpret_cast<int *>(lds + static_cast<size_t>(SC) * kActSC);
    int *cnt = part + kPartBytes / 4;                       // [kTilesWG]
    float *red_f = reinterpret_cast<float *>(cnt + kTilesWG);  // [kW]
    long long *red_l = reinterpret_cast<long long *>(red_f + kW);  // [kW]
    float *scl = reinterpret_cast<float *>(red_l + kW);  // [2][kTilesWG * 16]: output scale, affine E
    if (tid < kTilesWG) cnt[tid] = 0;

    // this wave's superchunks of every tile
    const int sc0 = w * SC / kW, sc1 = (w + 1) * SC / kW;
    const int upt = sc1 - sc0;
    const int NU = nt * upt;
    const uint32_t *Sb = L.S + static_cast<size_t>(tA) * tile_words;

    // One superchunk of one tile: 4 words per lane (16-byte aligned), or
    // wlast words in a short last superchunk, read as one 16-byte access
    // (dword aligned; the words past wlast belong to the next lane or tile,
    // or to the allocation's 16-byte tail, and are masked off where they
    // are used).  One load instruction either way, so the loads in flight
    // are counted alike; nothing reads a loaded word before its use.
    const int wl = L.wlast;
    auto load_unit = [&](int lt, int s) -> u32x4 {
        const int W = s == SC - 1 ? wl : 4;
        const uint32_t *p = Sb + static_cast<size_t>(lt) * tile_words + 256 * s + W * lane;
        u32x4 r;
        __builtin_memcpy(&r, p, sizeof(r));
        return r;
    };
    // load iterator (clamped at the last unit: loads stay unconditional)
    int ld_lt = 0, ld_s = sc0;
    u32x4 bufA[kPipe], bufB[kPipe];
    auto load_group = [&](u32x4 (&buf)[kPipe], int u0) {
#pragma unroll
        for (int q = 0; q < kPipe; ++q) {
            buf[q] = load_unit(ld_lt, ld_s);
            // next unit (selects, no branches: the loads in flight stay countable)
            const bool adv = u0 + q + 1 < NU;
            const bool wrap = ld_s + 1 == sc1;
            ld_lt += (adv && wrap) ? 1 : 0;
            ld_s = adv ? (wrap ? sc0 : ld_s + 1) : ld_s;
        }
    };
    // ---- vector prologue: fixed-point digits of the whole vector in LDS.
    // The vector's loads are issued first, then the first group of sign
    // loads: a wave waits for its loads in issue order, so the prologue's
    // uses of the vector do not wait for the sign words, which stay in
    // flight through the prologue.
    const int nblk = SC * 32;  // digit blocks (s, j, g) of 16 columns each
    // (NBLK * kT >= nblk blocks; threads past the last block load, and later
    // write, the last block again)
    Run raw[NBLK][4];
#pragma unroll
    for (int bi = 0; bi < NBLK; ++bi) {
        const int d = min(tid + bi * kT, nblk - 1);
        const int s = d >> 5, j = (d >> 2) & 7, g = d & 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[bi][i] = load_run<STAGE, K4>(L, 512 * s + 128 * i + 16 * j + 4 * g);
    }
    // the output scales of the workgroup's rows (and the affine term of a
    // 0/1 layer), so that finishing a tile loads nothing from memory
    float osc_v = 0.0f, affe_v = 0.0f;
    {
        const int row = min(tA * 16 + tid, L.rows - 1);
        osc_v = __half2float(L.osc[row]);
        if (STAGE == 2 && BIN && L.aff_E) affe_v = L.aff_E[row];
    }
    float aff_s0 = 0.0f, aff_s1 = 0.0f;
    if (STAGE == 2 && BIN && L.aff_E) {
        aff_s0 = L.aff_stats[0];
        aff_s1 = L.aff_stats[1];
    }
    // (unconditional: with no units the clamped iterator names superchunk
    // sc0 < SC of the workgroup's first tile, a valid address)
    load_group(bufA, 0);
    float mx = 0.0f;
#pragma unroll
    for (int bi = 0; bi < NBLK; ++bi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float u[4];
            run_values<STAGE>(raw[bi][i], u);
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(u[e]));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) red_f[w] = mx;
    __syncthreads();
    mx = red_f[0];
#pragma unroll
    for (int i = 1; i < kW; ++i) mx = fmaxf(mx, red_f[i]);
    int S = 0;
    if (mx > 0.0f) {
        int E;
        (void)frexpf(mx, &E);  // mx = f 2^E, f in [0.5, 1)
        S = 30 - E;            // mx 2^S in [2^29, 2^30)
    }
    S = __builtin_amdgcn_readfirstlane(S);
    long long usum = 0;
#pragma unroll
    for (int bi = 0; bi < NBLK; ++bi) {
        {
            const bool own = tid + bi * kT < nblk;  // else a copy of the last block
            const int d = min(tid + bi * kT, nblk - 1);
            uint32_t P[4][4];  // [digit plane c][dword i]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float u[4];
                run_values<STAGE>(raw[bi][i], u);
                uint32_t E[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int q = __float2int_rn(ldexpf(u[e], S));
                    usum += own ? q : 0;
                    // balanced base-256 digits: the bytes of (q + 0x808080) ^ 0x808080
                    E[e] = (static_cast<uint32_t>(q) + 0x808080u) ^ 0x808080u;
                }
                // 4x4 byte transpose: P[c][i] = (E[0].c, E[1].c, E[2].c, E[3].c)
                const uint32_t lo01 = __builtin_amdgcn_perm(E[1], E[0], 0x05010400u);
                const uint32_t hi01 = __builtin_amdgcn_perm(E[1], E[0], 0x07030602u);
                const uint32_t lo23 = __builtin_amdgcn_perm(E[3], E[2], 0x05010400u);
                const uint32_t hi23 = __builtin_amdgcn_perm(E[3], E[2], 0x07030602u);
                P[0][i] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
                P[1][i] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
                P[2][i] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
                P[3][i] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
                *reinterpret_cast<u32x4 *>(act + 64 * d + 16 * c) = u32x4{P[c][0], P[c][1], P[c][2], P[c][3]};
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) usum += __shfl_xor(usum, o);
    if (lane == 0) red_l[w] = usum;
    // (last: a wave may wait for all of its loads, sign words included, here)
    if (tid < kTilesWG * 16) {
        scl[tid] = osc_v;
        scl[kTilesWG * 16 + tid] = affe_v;
    }
    __syncthreads();  // digits, scales, counters and the wave sums are in place
    long long U = 0;
#pragma unroll
    for (int i = 0; i < kW; ++i) U += red_l[i];

    // ---- main loop
    i32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = i32x4{0, 0, 0, 0};
    const int c = lane & 15, gq = lane >> 4;

    auto epilogue = [&](int lt) {
        if (lane < 16) {
            const int r = lane;
            long long Z = 0;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                int zc = 0;
#pragma unroll
                for (int ww = 0; ww < kW; ++ww) zc += part[((lt * kW + ww) * 16 + r) * 4 + cc];
                Z += static_cast<long long>(zc) * (1LL << (8 * cc));
            }
            const long long sf = BIN ? 2 * Z : U - 2 * Z;
            const double res = ldexp(static_cast<double>(sf), -S);
            const int row = (tA + lt) * 16 + r;
            if (row < L.rows) {
                const double sc = static_cast<double>(scl[lt * 16 + r]);
                if constexpr (STAGE == 1) {
                    static_cast<float *>(L.out)[row] = static_cast<float>(res * sc);
                } else {
                    double val = res * sc;
                    if (BIN && L.aff_E)
                        val += static_cast<double>(scl[kTilesWG * 16 + lt * 16 + r]) * static_cast<double>(aff_s0) +
                               static_cast<double>(aff_s1);
                    static_cast<__half *>(L.out)[row] = rne16_of(val);
                }
            }
        }
    };
    auto finish_tile = [&](int lt) {
        if (c < 4) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                int z = 0;
#pragma unroll
                for (int j = 0; j < 7; ++j) z += acc[j][v] >> j;
                z -= acc[7][v] >> 7;
                part[((lt * kW + w) * 16 + 4 * gq + v) * 4 + c] = z;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = i32x4{0, 0, 0, 0};
        int old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(&cnt[lt], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        old = __builtin_amdgcn_readfirstlane(old);
        if (old == kW - 1) epilogue(lt);
    };
    // B operand of lane (c, g): 16 bytes of digit plane c (planes >= 4 read
    // neighbouring bytes, never used)
    const char *act_lane = act + 64 * gq + 16 * c;
    auto compute_unit = [&](const u32x4 &wd, int s) {
        const char *ab = act_lane + kActSC * s;
        const int W = s == SC - 1 ? wl : 4;  // words of this superchunk (the rest are masked off)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t msk = 0x01010101u << j;
            const u32x4 m4 = u32x4{msk, W > 1 ? msk : 0u, W > 2 ? msk : 0u, W > 3 ? msk : 0u};
            const i32x4 a = __builtin_bit_cast(i32x4, wd & m4);
            const i32x4 b = *reinterpret_cast<const i32x4 *>(ab + 256 * j);
            acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
        }
    };
    int cp_lt = 0, cp_s = sc0;
    auto compute_group = [&](const u32x4 (&buf)[kPipe], int u0) {
#pragma unroll
        for (int q = 0; q < kPipe; ++q) {
            if (u0 + q >= NU) break;
            compute_unit(buf[q], cp_s);
            if (++cp_s == sc1) {
                finish_tile(cp_lt);
                cp_s = sc0;
                ++cp_lt;
            }
        }
    };
    if (NU > 0) {
        for (int u0 = 0; u0 < NU; u0 += 2 * kPipe) {
            if (u0 + kPipe < NU) load_group(bufB, u0 + kPipe);
            compute_group(bufA, u0);
            if (u0 + kPipe >= NU) break;
            if (u0 + 2 * kPipe < NU) load_group(bufA, u0 + 2 * kPipe);
            compute_group(bufB, u0 + kPipe);
        }
    } else {
        for (int lt = 0; lt < nt; ++lt) finish_tile(lt);  // no superchunks here: zero partials
    }
}

template <typename K>
void allow_lds(K kernel, size_t bytes) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(bytes));
}

}  // namespace

int i8_superchunks(int K) { return (round_up_int(K, 128) + 511) / 512; }

int launch_decode_i8(I8Args &a, int stage, bool bin, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.count < 1 || a.count > kMaxGroup) return static_cast<int>(hipErrorInvalidValue);
    // workgroups: about one per CU, shared among the layers by their work,
    // each with at most kTilesWG tiles
    long long units = 0;
    for (int i = 0; i < a.count; ++i) {
        I8Layer &L = a.L[i];
        if (L.SC < 1 || L.SC > kI8MaxSC || L.wlast < 1 || L.wlast > 4 || L.ntiles < 1)
            return static_cast<int>(hipErrorInvalidValue);
        units += static_cast<long long>(L.ntiles) * L.SC;
    }
    const int target = kCUs - ((bin && a.stat_wg >= 0) ? 1 : 0);
    int wg = 0, maxSC = 1;
    for (int i = 0; i < a.count; ++i) {
        I8Layer &L = a.L[i];
        const long long u = static_cast<long long>(L.ntiles) * L.SC;
        int g = static_cast<int>((target * u + units / 2) / units);
        g = std::max(g, (L.ntiles + kTilesWG - 1) / kTilesWG);
        g = std::max(1, std::min(g, L.ntiles));
        L.wg0 = wg;
        L.nwg = g;
        wg += g;
        maxSC = std::max(maxSC, L.SC);
    }
    if (bin && a.stat_wg >= 0) a.stat_wg = wg++;
    else a.stat_wg = -1;
    const size_t lds = lds_bytes_for(maxSC);
    // stage 1 reads x in runs of four entries when every layer's m allows
    bool k4 = true;
    for (int i = 0; i < a.count; ++i) k4 = k4 && (a.L[i].K % 4 == 0);
    // (stage 2 reads v, k_pad entries: always whole runs); digit blocks per
    // thread NBLK = 1, 2, 4 for up to 16, 32, 64 superchunks
    static void (*const kernels[3][6])(I8Args) = {
#define DBF_I8_ROW(NB)                                                                                        \
    {dec_i8_kernel<1, false, true, NB>, dec_i8_kernel<1, false, false, NB>, dec_i8_kernel<1, true, true, NB>, \
     dec_i8_kernel<1, true, false, NB>, dec_i8_kernel<2, false, true, NB>, dec_i8_kernel<2, true, true, NB>}
        DBF_I8_ROW(1), DBF_I8_ROW(2), DBF_I8_ROW(4)
#undef DBF_I8_ROW
    };
    static bool lds_set[3][6] = {};
    const int ni = maxSC <= 16 ? 0 : maxSC <= 32 ? 1 : 2;
    const int ki = stage == 1 ? (bin ? 2 : 0) + (k4 ? 0 : 1) : 4 + (bin ? 1 : 0);
    if (!lds_set[ni][ki]) {
        allow_lds(kernels[ni][ki], lds_bytes_for(kI8MaxSC));
        lds_set[ni][ki] = true;
    }
    launch_kernel(kernels[ni][ki], dim3(wg), dim3(kT), lds, s, a);
    return static_cast<int>(hipGetLastError());
}

}  // namespace dbf
