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
//   exponent S: q_l = rne(u_l 2^S), S chosen so that 2^29 <= max_l |u_l 2^S|
//   < 2^30 (u = x ⊙ b is exact in fp32; so is any power-of-two scaling of
//   it).  Then s_r = Σ_l sign_rl q_l is an exact integer, formed as U - 2 Z_r
//   with U = Σ_l q_l and Z_r = Σ_{bit_rl = 1} q_l (bit 1 means -1), and the
//   stage result s_r 2^-S is exact in fp64 (|s_r| < 2^53).  The only
//   roundings: q (2^-31 of the vector's largest entry, at most), v =
//   rne32(t mid) between the stages, and one correctly rounded conversion of
//   a s to fp16 at the end.  The result of a row does not depend on how the
//   reduction is cut among waves (every partial sum is exact).
//
// Matrix-core mapping (v_mfma_i32_16x16x64_i8: D 16x16 += A 16x64 * B 64x16).
//   B operand: q as four balanced base-256 digits, q = d0 + 2^8 d1 + 2^16 d2
//   + 2^24 d3 with every d in [-128, 127], in columns c = 0..3 (columns 4..15
//   are not used at batch 1).  A operand: the sign bits as int8 values 0 or
//   2^j.  A 32-bit word of signs AND 0x01010101 << j keeps its bits j, 8+j,
//   16+j, 24+j as four int8 values in {0, 2^j} (j = 7: {0, -128}) -- one VALU
//   instruction per four signs; the layout (pack.cpp, dbf_layout_signs_dec)
//   places the bits so that these are the columns the B operand holds.  One
//   accumulator per j; at the end of a wave's part Z_c = Σ_j ±acc_j >> j
//   (exact: acc_j is a multiple of 2^j) and Z = Σ_c Z_c 2^(8 c).
//
// Work split.  A workgroup (8 waves) owns tpw consecutive tiles of 16 rows;
// each tile's reduction is cut into `parts` ranges of superchunks (512
// columns, 1 KiB of signs per tile), one per wave, so a wave's job is one
// (tile, range) pair.  The host picks the fewest tiles per workgroup, tpw in
// {1, 2, 4, 8}, with which the grid has at most one workgroup per CU, and
// parts = min(8 / tpw, SC).  A wave streams its sign words from global
// memory into a ring of three register sets (the first three issued before
// the vector prologue); the digits of the whole vector sit in LDS.  The waves' partial Z meet in LDS
// and one thread per row finishes it.
//
// Every wave issues at most one instruction per four cycles, so what a wave
// executes between the kernel's start and its last store is the floor of
// the kernel's duration: the kernel keeps that path short -- the layer comes
// from blockIdx.y (no search through the arguments), the loops are rolled,
// and no work is repeated across waves.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>
#include <type_traits>

#include "bqq_rowstats.h"
#include "dbf_internal.h"

namespace dbf {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kW = 8;                 // waves per workgroup
constexpr int kT = kW * 64;           // threads per workgroup
constexpr int kCUs = 256;             // MI355X
constexpr int kMaxTPWc = 8;           // tiles per workgroup, at most
constexpr int kActSC = 2048;          // LDS bytes of digits per superchunk: [8 j][16 slots][16]
constexpr int kPartBytes = kMaxTPWc * 16 * 8;  // [tile][row] int64: Z of the workgroup's rows, per vector
// wave maxima and sums (per vector), row scales (fp32), affine terms of 0/1 layers (fp64)
constexpr int kMiscBytes = kMaxTPWc * 16 * 4 + kMaxTPWc * 16 * 8;
constexpr int kWaveBytes = kW * 4 + kW * 8;
constexpr int kRing = 3;              // superchunks of signs in flight per wave

__host__ __device__ constexpr size_t lds_bytes_for(int SC, int NB = 1) {
    return static_cast<size_t>(NB) * (static_cast<size_t>(SC) * kActSC + kPartBytes + kWaveBytes) + kMiscBytes;
}

// Digits in LDS.  Block (s, j, g) -- the 16 vector entries 512 s + 128 i +
// 16 j + 4 g + b (i, b < 4) -- holds one 16-byte row per digit plane c
// (byte 4 i + b), the B operand of lane (c, g) in the product for bit j of
// superchunk s.  Superchunk s, bit j is a 256-byte chunk of 16 slots; plane
// c of block g sits in slot digit_slot(g, c, j), a permutation under which
// the prologue's writes (lanes over (j, g), one plane) and the operand reads
// (lanes over (c, g), one j) each reach every bank once.
__device__ __forceinline__ int digit_slot(int g, int c, int j) {
    return 8 * (g >> 1) + 4 * (g & 1) + ((c + 2 * (g >> 1) + j) & 3);
}

// Buffer resources: loads through them at offsets past num_records return 0
// without touching memory, so a load never needs a condition or a clamped
// address (raw buffer, 32-bit offsets; the fourth descriptor word of a
// plain raw buffer on this family).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(bytes), 0x00020000);
}
constexpr uint32_t kOff = 0x7FFFFFF0u;  // an offset past every range

// Raw loads of eight consecutive entries base .. base + 7 (base a multiple
// of 8) of the stage's vector: stage 1, x and b (fp16, 16 bytes each);
// stage 2, v (fp32, two 16-byte loads).  Entries at or past K read as 0
// (they lie outside the resources' ranges).  When K is not a multiple of 8
// (stage 1 only) the entries are loaded one by one.
struct Octet {
    uint32_t r[8];
};
template <int STAGE, bool K8>
__device__ __forceinline__ Octet load_octet(__amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rb, int base) {
    Octet o;
    if constexpr (STAGE == 1) {
        if constexpr (K8) {
            const u32x4 xv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, 2 * base, 0, 0));
            const u32x4 bv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, 2 * base, 0, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o.r[e] = xv[e];
                o.r[4 + e] = bv[e];
            }
        } else {
            uint32_t xe[8], be[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                xe[e] = __builtin_amdgcn_raw_buffer_load_b16(rx, 2 * (base + e), 0, 0);
                be[e] = __builtin_amdgcn_raw_buffer_load_b16(rb, 2 * (base + e), 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o.r[e] = xe[2 * e] | (xe[2 * e + 1] << 16);
                o.r[4 + e] = be[2 * e] | (be[2 * e + 1] << 16);
            }
        }
    } else {
        const u32x4 t0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, 4 * base, 0, 0));
        const u32x4 t1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, 4 * base + 16, 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o.r[e] = t0[e];
            o.r[4 + e] = t1[e];
        }
    }
    return o;
}

// The eight fp32 entries of an octet: stage 1, x ⊙ b (exact); stage 2, v.
template <int STAGE>
__device__ __forceinline__ void octet_values(const Octet &o, float (&u)[8]) {
    if constexpr (STAGE == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const __half2 xh = __builtin_bit_cast(__half2, o.r[e]), bh = __builtin_bit_cast(__half2, o.r[4 + e]);
            u[2 * e] = __low2float(xh) * __low2float(bh);
            u[2 * e + 1] = __high2float(xh) * __high2float(bh);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = __uint_as_float(o.r[e]);
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

// Wave-wide reductions through DPP (no LDS round trips): pairs and quads
// (quad_perm), halves and whole rows of 16 lanes (row_half_mirror,
// row_mirror), then rows 1 and 3 take rows 0 and 2 (row_bcast:15) and row 3
// takes lanes 0..31 (row_bcast:31); lane 63 ends with the total.  Lanes a
// step does not write keep the identity 0 as their operand.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_src(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROWS, 0xF, false));
}
// maximum of non-negative floats (their bits order as unsigned integers)
__device__ __forceinline__ float wave_max_nonneg(float x) {
    uint32_t v = __float_as_uint(x);
    v = max(v, dpp_src<0xB1, 0xF>(v));   // quad_perm [1, 0, 3, 2]
    v = max(v, dpp_src<0x4E, 0xF>(v));   // quad_perm [2, 3, 0, 1]
    v = max(v, dpp_src<0x141, 0xF>(v));  // row_half_mirror
    v = max(v, dpp_src<0x140, 0xF>(v));  // row_mirror
    v = max(v, dpp_src<0x142, 0xA>(v));  // row_bcast:15
    v = max(v, dpp_src<0x143, 0x8>(v));  // row_bcast:31
    return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63)));
}
// sum of 32-bit integers (wrapping; callers keep the total in range)
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    v += dpp_src<0xB1, 0xF>(v);
    v += dpp_src<0x4E, 0xF>(v);
    v += dpp_src<0x141, 0xF>(v);
    v += dpp_src<0x140, 0xF>(v);
    v += dpp_src<0x142, 0xA>(v);
    v += dpp_src<0x143, 0x8>(v);
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// NO: octets of the vector per thread in the prologue.  Octet o holds the
// entries 512 s + 128 i + 16 j + 8 gp + (0..7) -- run i of blocks g = 2 gp
// and 2 gp + 1 of (s, j) -- with (s, j, i, gp) = (o >> 6, (o >> 3) & 7,
// (o >> 1) & 3, o & 1); the vector, padded to SC superchunks, has SC * 64
// octets, NO * kT >= that.
// The p + 1 weighted sums of x that the group-wise BQQ form's affine term
// needs (bqq_rowstats.h; the statistic count is a template argument there).
__device__ __forceinline__ void rowstats_q(const I8Args &args, float *sh) {
    switch (args.stat_Q) {
#define DBF_STAT_CASE(Q)                                                                                 \
    case Q:                                                                                              \
        bqq_rowstats_dotq<kT, Q>(args.stat_x, args.stat_m, args.stat_w, args.stats, sh);                \
        break;
        DBF_STAT_CASE(2) DBF_STAT_CASE(3) DBF_STAT_CASE(4) DBF_STAT_CASE(5)
        DBF_STAT_CASE(6) DBF_STAT_CASE(7) DBF_STAT_CASE(8) DBF_STAT_CASE(9)
#undef DBF_STAT_CASE
        default:
            break;
    }
}

// QSTAT: stage 1 of a signed launch whose last grid row (an empty layer
// entry) forms the group-wise BQQ statistics beside it.
// NB: the workgroup takes NB input vectors (batch rows) at once, each with
// its own exponent and its own digits (columns 4 r .. 4 r + 3 of the product
// for row r); rows from args.nrows on read as zero and are not stored.
template <int STAGE, bool BIN, bool K8, int NO, bool QSTAT = false, int NB = 1>
__global__ __launch_bounds__(kT, NO <= 4 ? 2 : 1) void dec_i8_kernel(const I8Args args) {
    static_assert(NB == 1 || (!BIN && !QSTAT && NB * 4 <= 16), "batch rows: signed layers, 16 product columns");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    // Every field of the layer, read at once (one round of scalar loads: the
    // empty asm takes them all as inputs, so none of the loads is sunk into
    // a later branch, where each would cost a round trip of its own)
    const I8Layer L = args.L[blockIdx.y];
    asm volatile("" ::"s"(L.S), "s"(L.vec), "s"(L.bsc), "s"(L.osc), "s"(L.out), "s"(L.aff_E), "s"(L.aff_stats),
                 "s"(L.rows), "s"(L.K), "s"(L.SC), "s"(L.wlast), "s"(L.ntiles), "s"(L.tpw), "s"(L.parts),
                 "s"(L.nwg), "s"(L.job[0]), "s"(L.job[1]), "s"(L.job[2]), "s"(L.job[3]));
    if (BIN && L.SC == 0) {
        // 0/1 layers: the per-row input sums of the affine term (an empty
        // layer entry marks that row of the grid)
        if (blockIdx.x == 0)
            bqq_rowstats_row<kT>(args.stat_x, args.stat_m, args.gamma, args.stats, reinterpret_cast<float *>(lds));
        return;
    }
    if (QSTAT && L.SC == 0) {
        if (blockIdx.x == 0) rowstats_q(args, reinterpret_cast<float *>(lds));
        return;
    }
    const int wg = blockIdx.x;
    if (wg >= L.nwg) return;  // padding of the grid's shorter rows
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int SC = L.SC, wl = L.wlast;
    const int t0 = wg * L.tpw;
    const int nt = min(L.tpw, L.ntiles - t0);  // tiles of this workgroup
    const int tile_words = 256 * (SC - 1) + 64 * wl;
    // this wave's job: tile lt of the workgroup, superchunks [s0, s0 + nu)
    const uint32_t jpair = w < 4 ? (w < 2 ? L.job[0] : L.job[1]) : (w < 6 ? L.job[2] : L.job[3]);
    const uint32_t job = (jpair >> (16 * (w & 1))) & 0xFFFFu;
    const int lt = job & 7, s0 = (job >> 3) & 63;
    const int nu = lt < nt ? static_cast<int>(job >> 9) : 0;

    char *act = lds;  // digits [NB][SC][8 j][4 g][4 c][16]
    long long *zrow = reinterpret_cast<long long *>(lds + static_cast<size_t>(NB) * SC * kActSC);  // [NB][tile][row]
    float *wmax = reinterpret_cast<float *>(zrow + NB * (kPartBytes / 8));  // [NB][kW]
    long long *wU = reinterpret_cast<long long *>(wmax + NB * kW);          // [NB][kW]
    float *scl = reinterpret_cast<float *>(wU + NB * kW);  // [kMaxTPWc * 16] row scales (a or mid)
    double *saff = reinterpret_cast<double *>(scl + kMaxTPWc * 16);  // [kMaxTPWc * 16] affine terms (0/1 layers)

    // ---- loads, in the order their data is used (a wave waits for its
    // loads in issue order): the vector, the row scales, then the first
    // kRing superchunks of signs
    const int noct = SC * 64;
    const uint32_t kb = static_cast<uint32_t>(L.K);
    const __amdgpu_buffer_rsrc_t rb = rsrc(L.bsc, STAGE == 1 ? 2u * kb : 0u);
    const int nrows = NB == 1 ? 1 : args.nrows;
    Octet raw[NB][NO];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        // vector r: row r of the batch (K entries apart); rows past nrows read as zero
        const __amdgpu_buffer_rsrc_t rx =
            rsrc(static_cast<const char *>(L.vec) + static_cast<size_t>(r) * kb * (STAGE == 1 ? 2u : 4u),
                 r < nrows ? kb * (STAGE == 1 ? 2u : 4u) : 0u);
#pragma unroll
        for (int k = 0; k < NO; ++k) {
            const int o = tid + kT * k;
            const int base = 512 * (o >> 6) + 16 * ((o >> 3) & 7) + 128 * ((o >> 1) & 3) + 8 * (o & 1);
            raw[r][k] = load_octet<STAGE, K8>(rx, rb, o < noct ? base : (1 << 27));
        }
    }
    // thread tid < nt * 16 finishes row t0 * 16 + tid
    const int my_row = min(t0 * 16 + tid, L.rows - 1);
    const float osc_v = __half2float(L.osc[my_row]);
    // 0/1 layers: the affine term's E of this row (Q - 1 rows of E) and the
    // Q statistics; loads past them read nothing (zero)
    float aff_e[kI8MaxQ - 1], aff_s[kI8MaxQ];
    if constexpr (STAGE == 2 && BIN) {
        const bool aff = L.aff_E != nullptr;
        const uint32_t Q = static_cast<uint32_t>(args.aff_Q);
        const __amdgpu_buffer_rsrc_t re = rsrc(L.aff_E, aff ? 4u * static_cast<uint32_t>(L.rows) * (Q - 1) : 0u);
        const __amdgpu_buffer_rsrc_t rt = rsrc(L.aff_stats, aff ? 4u * Q : 0u);
#pragma unroll
        for (int q = 0; q < kI8MaxQ - 1; ++q)
            aff_e[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(re, 4 * (q * L.rows + my_row), 0, 0));
#pragma unroll
        for (int q = 0; q < kI8MaxQ; ++q)
            aff_s[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rt, 4 * q, 0, 0));
    }
    // One superchunk of the wave's tile: 4 words per lane (16-byte aligned),
    // or wlast words in a short last superchunk, read as one 16-byte access
    // (dword aligned; the words past wlast belong to the next lane or tile,
    // or to the allocation's 16-byte tail, and are masked off where they are
    // used).  Loads past the job read nothing (offsets past the range), so
    // every path issues the same loads and the waits on them are static.
    const __amdgpu_buffer_rsrc_t rs =
        rsrc(L.S + static_cast<size_t>(t0) * tile_words, 4u * static_cast<uint32_t>(nt * tile_words) + 16u);
    auto unit_off = [&](int i) -> uint32_t {
        const int s = s0 + i;
        const int W = s == SC - 1 ? wl : 4;
        return i < nu ? 4u * static_cast<uint32_t>(lt * tile_words + 256 * s + W * lane) : kOff;
    };
    u32x4 ring[kRing];
#pragma unroll
    for (int q = 0; q < kRing; ++q)
        ring[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, unit_off(q), 0, 0));

    // ---- each vector as fixed-point digits, one exponent per vector for the workgroup
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        float mx = 0.0f;
#pragma unroll
        for (int k = 0; k < NO; ++k) {
            float u[8];
            octet_values<STAGE>(raw[r][k], u);
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(u[e]));
        }
        mx = wave_max_nonneg(mx);
        if (lane == 0) wmax[r * kW + w] = mx;
    }
    __syncthreads();
    int S[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        float mx = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kW; ++ww) mx = fmaxf(mx, wmax[r * kW + ww]);
        S[r] = 0;
        if (mx > 0.0f) {
            int E;
            (void)frexpf(mx, &E);  // mx = f 2^E, f in [0.5, 1)
            S[r] = 30 - E;         // mx 2^S in [2^29, 2^30)
        }
    }
    // the row scales, kept in LDS for the finishing threads (their loads
    // are waited for here, not behind the last sign loads)
    if (tid < nt * 16) {
#pragma unroll
        for (int r = 0; r < NB; ++r) zrow[r * (kPartBytes / 8) + tid] = 0;
        scl[tid] = osc_v;
        if constexpr (STAGE == 2 && BIN) {
            // Σ_{q < Q-1} E_q[row] s_q + s_{Q-1} in fp64 (exact products of fp32 values)
            const int Q = args.aff_Q;
            double t = static_cast<double>(aff_e[0]) * static_cast<double>(aff_s[0]);
            double last = static_cast<double>(aff_s[1]);
#pragma unroll
            for (int q = 1; q < kI8MaxQ - 1; ++q) {
                if (q < Q - 1) t += static_cast<double>(aff_e[q]) * static_cast<double>(aff_s[q]);
                if (q == Q - 1) last = static_cast<double>(aff_s[q]);
            }
            if (Q == kI8MaxQ) last = static_cast<double>(aff_s[kI8MaxQ - 1]);
            saff[tid] = t + last;
        }
    }
#pragma unroll
    for (int r = 0; r < NB; ++r) {
    char *actr = act + static_cast<size_t>(r) * SC * kActSC;
    int dsum[4] = {0, 0, 0, 0};  // Σ of each digit plane over this thread's octets
#pragma unroll
    for (int k = 0; k < NO; ++k) {
        const int o = tid + kT * k;
        if (o < noct) {
            float u[8];
            octet_values<STAGE>(raw[r][k], u);
            const int sj = o >> 3, j = sj & 7, i = (o >> 1) & 3, gp = o & 1;
#pragma unroll
            for (int h = 0; h < 2; ++h) {  // block g = 2 gp + h: entries 4 h .. 4 h + 3
                uint32_t E[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int q = __float2int_rn(ldexpf(u[4 * h + e], S[r]));
                    // balanced base-256 digits: the bytes of (q + 0x808080) ^ 0x808080
                    E[e] = (static_cast<uint32_t>(q) + 0x808080u) ^ 0x808080u;
                }
                // 4x4 byte transpose: plane c = (E[0].c, E[1].c, E[2].c, E[3].c)
                const uint32_t lo01 = __builtin_amdgcn_perm(E[1], E[0], 0x05010400u);
                const uint32_t hi01 = __builtin_amdgcn_perm(E[1], E[0], 0x07030602u);
                const uint32_t lo23 = __builtin_amdgcn_perm(E[3], E[2], 0x05010400u);
                const uint32_t hi23 = __builtin_amdgcn_perm(E[3], E[2], 0x07030602u);
                const uint32_t Pc[4] = {__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),
                                        __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
                                        __builtin_amdgcn_perm(hi23, hi01, 0x05040100u),
                                        __builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
                const int g = 2 * gp + h;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    dsum[c] = __builtin_amdgcn_sdot4(static_cast<int>(Pc[c]), 0x01010101, dsum[c], false);
                    // bytes 4 i .. 4 i + 3 of plane c of block (s, j, g)
                    *reinterpret_cast<uint32_t *>(actr + 256 * sj + 16 * digit_slot(g, c, j) + 4 * i) = Pc[c];
                }
            }
        }
    }
    if constexpr (!BIN) {
        // U = Σ q = Σ_c 256^c (Σ of plane c); each plane's wave sum fits 32 bits
        long long U = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            U += static_cast<long long>(static_cast<int>(wave_sum_u32(static_cast<uint32_t>(dsum[c])))) * (1LL << (8 * c));
        if (lane == 0) wU[r * kW + w] = U;
    }
    }
    __syncthreads();

    // ---- the wave's job
    i32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = i32x4{0, 0, 0, 0};
    const int c = lane & 15, gq = lane >> 4;
    // B operand of lane (c, g): 16 bytes of digit plane c mod 4 of vector
    // c / 4; lanes of the unused columns c >= 4 NB read nothing (their
    // columns of D are not used).  The slot depends on j mod 4.
    int slot_off[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) slot_off[k] = 16 * digit_slot(gq, c & 3, k);
    if (nu > 0) {
        int i0 = 0;
        // one exit, at the bottom; every step issues its load (kRing units
        // ahead), so every path through the body leaves kRing loads in flight
        do {
#pragma unroll
            for (int q = 0; q < kRing; ++q) {
                const int i = i0 + q;
                if (i < nu) {
                    const int s = s0 + i;
                    i32x4 B[8];
                    if (c < 4 * NB) {
                        const char *as = act + kActSC * (static_cast<size_t>(c >> 2) * SC + s);
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            B[j] = *reinterpret_cast<const i32x4 *>(as + slot_off[j & 3] + 256 * j);
                    }
                    u32x4 wd = ring[q];
                    if (s == SC - 1) {  // words past wlast: not this superchunk's
                        wd.y = wl > 1 ? wd.y : 0u;
                        wd.z = wl > 2 ? wd.z : 0u;
                        wd.w = wl > 3 ? wd.w : 0u;
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const i32x4 a = __builtin_bit_cast(i32x4, wd & (0x01010101u << j));
                        acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, B[j], acc[j], 0, 0, 0);
                    }
                }
                ring[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, unit_off(i + kRing), 0, 0));
            }
            i0 += kRing;
        } while (i0 < nu);
        // Z of the job's 16 rows, per digit column: Σ_j ±acc_j >> j, added
        // with its weight 256^c to the row's sum in LDS (exact integers, so
        // the order of the additions does not matter)
        if (c < 4 * NB) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                int f = 0;
#pragma unroll
                for (int j = 0; j < 7; ++j) f += acc[j][v] >> j;
                f -= acc[7][v] >> 7;
                __hip_atomic_fetch_add(&zrow[(c >> 2) * (kPartBytes / 8) + lt * 16 + 4 * gq + v],
                                       static_cast<long long>(f) * (1LL << (8 * (c & 3))), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
    __syncthreads();

    // ---- one thread per (vector, row): the parts' exact sums, then the scales
    // vector and row of the workgroup (kMaxTPWc * 16 = 128 rows per vector)
    const int fr = NB == 1 ? 0 : tid >> 7, fi = NB == 1 ? tid : tid & 127;
    if ((NB == 1 || fr < nrows) && fi < nt * 16) {
        int Sr = S[0];
#pragma unroll
        for (int r = 1; r < NB; ++r) Sr = fr == r ? S[r] : Sr;
        long long sf = 2 * zrow[fr * (kPartBytes / 8) + fi];
        if constexpr (!BIN) {
            long long U = 0;
#pragma unroll
            for (int ww = 0; ww < kW; ++ww) U += wU[fr * kW + ww];
            sf = U - sf;
        }
        const double res = ldexp(static_cast<double>(sf), -Sr) * static_cast<double>(scl[fi]);
        const int row = t0 * 16 + fi;
        if (row < L.rows) {
            // output rows are L.rows apart
            const size_t at = NB == 1 ? static_cast<size_t>(row) : static_cast<size_t>(fr) * L.rows + row;
            if constexpr (STAGE == 1) {
                static_cast<float *>(L.out)[at] = static_cast<float>(res);
            } else {
                double val = res;
                if constexpr (BIN) val += saff[fi];
                static_cast<__half *>(L.out)[at] = rne16_of(val);
            }
        }
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
    if (a.nrows < 1 || a.nrows > kI8MaxRows || (a.nrows > 1 && bin)) return static_cast<int>(hipErrorInvalidValue);
    if (stage == 2 && bin && (a.aff_Q < 2 || a.aff_Q > kI8MaxQ)) return static_cast<int>(hipErrorInvalidValue);
    for (int i = 0; i < a.count; ++i) {
        const I8Layer &L = a.L[i];
        if (L.SC < 1 || L.SC > kI8MaxSC || L.wlast < 1 || L.wlast > 4 || L.ntiles < 1 || L.rows < 1 ||
            L.rows > 16 * L.ntiles)
            return static_cast<int>(hipErrorInvalidValue);
    }
    int maxSC = 1;
    for (int i = 0; i < a.count; ++i) maxSC = std::max(maxSC, a.L[i].SC);
    if (a.nrows > 1 && maxSC > kI8RowsMaxSC) return static_cast<int>(hipErrorInvalidValue);
    // vector octets per thread NO = 1, 2, 4, 8 for up to 8, 16, 32, 64
    // superchunks
    const int ni = maxSC <= 8 ? 0 : maxSC <= 16 ? 1 : maxSC <= 32 ? 2 : 3;
    // tiles per workgroup: the fewest (1, 2, 4, 8) with which the grid has
    // one workgroup per CU at most; the waves of a workgroup are shared out
    // among its tiles as parts of their reductions.  (Every workgroup brings
    // the whole vector to fixed point, so more, smaller workgroups repeat
    // that work: measured on the decoder block, one workgroup per CU beats
    // two, and both beat fewer than one.)
    const int slots = kCUs;
    // (the grid is rectangular: its shorter rows' padding workgroups hold a
    // slot while they start and leave)
    int tpw = kMaxTPWc;
    for (int cand = 1; cand < kMaxTPWc; cand *= 2) {
        long long wmax = 0;
        for (int i = 0; i < a.count; ++i) wmax = std::max<long long>(wmax, (a.L[i].ntiles + cand - 1) / cand);
        if (wmax * a.count <= slots) {
            tpw = cand;
            break;
        }
    }
    int maxwg = 1;
    for (int i = 0; i < a.count; ++i) {
        I8Layer &L = a.L[i];
        const int P = std::min(kW / tpw, L.SC);
        L.tpw = tpw;
        L.parts = P;
        L.nwg = (L.ntiles + tpw - 1) / tpw;
        // wave w: tile w / P of the workgroup, the (w % P)-th of P near-equal
        // superchunk ranges; waves past tpw * P have no job
        for (int q = 0; q < 4; ++q) L.job[q] = 0;
        for (int w = 0; w < kW; ++w) {
            const int lt = w / P, p = w % P;
            const int s0 = p * L.SC / P, nu = lt < tpw ? (p + 1) * L.SC / P - s0 : 0;
            L.job[w >> 1] |= static_cast<uint32_t>(lt | (s0 << 3) | (nu << 9)) << (16 * (w & 1));
        }
        maxwg = std::max(maxwg, L.nwg);
    }
    // stage 1 of a signed launch may carry the group-wise BQQ statistics
    const bool qstat = !bin && stage == 1 && a.stat_wg >= 0 && a.stat_w != nullptr;
    if (qstat && (a.stat_Q < 2 || a.stat_Q > kMaxStatQ)) return static_cast<int>(hipErrorInvalidValue);
    const bool stat = (bin && a.stat_wg >= 0) || qstat;
    if (a.nrows > 1 && stat) return static_cast<int>(hipErrorInvalidValue);
    if (stat && a.count >= kMaxGroup) return static_cast<int>(hipErrorInvalidValue);
    if (tpw > kMaxTPWc) return static_cast<int>(hipErrorInvalidValue);
    a.stat_wg = stat ? 0 : -1;
    if (stat) a.L[a.count] = I8Layer{};  // the row of the row-sum workgroup
    const dim3 grid(maxwg, a.count + (stat ? 1 : 0));
    // batch rows: one kernel form for 2, one for 3 and 4 (rows past nrows read as zero)
    const int NB = a.nrows == 1 ? 1 : a.nrows == 2 ? 2 : 4;
    const size_t lds = lds_bytes_for(maxSC, NB);
    // stage 1 reads x in 16-byte octets when every layer's m allows
    bool k8 = true;
    for (int i = 0; i < a.count; ++i) k8 = k8 && (a.L[i].K % 8 == 0);
    // (stage 2 reads v, k_pad entries: a multiple of 64)
    static void (*const kernels[4][6])(I8Args) = {
#define DBF_I8_ROW(NO)                                                                                        \
    {dec_i8_kernel<1, false, true, NO>, dec_i8_kernel<1, false, false, NO>, dec_i8_kernel<1, true, true, NO>, \
     dec_i8_kernel<1, true, false, NO>, dec_i8_kernel<2, false, true, NO>, dec_i8_kernel<2, true, true, NO>}
        DBF_I8_ROW(1), DBF_I8_ROW(2), DBF_I8_ROW(4), DBF_I8_ROW(8)
#undef DBF_I8_ROW
    };
    static void (*const qstat_kernels[4][2])(I8Args) = {
        {dec_i8_kernel<1, false, true, 1, true>, dec_i8_kernel<1, false, false, 1, true>},
        {dec_i8_kernel<1, false, true, 2, true>, dec_i8_kernel<1, false, false, 2, true>},
        {dec_i8_kernel<1, false, true, 4, true>, dec_i8_kernel<1, false, false, 4, true>},
        {dec_i8_kernel<1, false, true, 8, true>, dec_i8_kernel<1, false, false, 8, true>}};
    static bool lds_set[4][6] = {}, qlds_set[4][2] = {};
    const int ki = stage == 1 ? (bin ? 2 : 0) + (k8 ? 0 : 1) : 4 + (bin ? 1 : 0);
    if (NB > 1) {
        // signed layers only; reductions of at most kI8RowsMaxSC superchunks (NO = 1 or 2)
        static void (*const rkernels[2][2][3])(I8Args) = {
#define DBF_I8_NB_ROW(NB_, NO)                                                                              \
    {dec_i8_kernel<1, false, true, NO, false, NB_>, dec_i8_kernel<1, false, false, NO, false, NB_>,           \
     dec_i8_kernel<2, false, true, NO, false, NB_>}
            {DBF_I8_NB_ROW(2, 1), DBF_I8_NB_ROW(2, 2)},
            {DBF_I8_NB_ROW(4, 1), DBF_I8_NB_ROW(4, 2)}
#undef DBF_I8_NB_ROW
        };
        static bool rlds_set[2][2][3] = {};
        const int bi = NB == 2 ? 0 : 1, ri = stage == 1 ? (k8 ? 0 : 1) : 2;
        if (ni > 1) return static_cast<int>(hipErrorInvalidValue);
        auto k = rkernels[bi][ni][ri];
        if (!rlds_set[bi][ni][ri]) {
            allow_lds(k, lds_bytes_for(kI8RowsMaxSC, NB));
            rlds_set[bi][ni][ri] = true;
        }
        launch_kernel(k, grid, dim3(kT), lds, s, a);
        return static_cast<int>(hipGetLastError());
    }
    if (qstat) {
        // (the statistics row uses kMaxStatQ trees of kT floats of LDS at most)
        const size_t qlds = std::max(lds, static_cast<size_t>(kMaxStatQ) * kT * 4);
        auto k = qstat_kernels[ni][k8 ? 0 : 1];
        if (!qlds_set[ni][k8 ? 0 : 1]) {
            allow_lds(k, lds_bytes_for(kI8MaxSC));
            qlds_set[ni][k8 ? 0 : 1] = true;
        }
        launch_kernel(k, grid, dim3(kT), qlds, s, a);
        return static_cast<int>(hipGetLastError());
    }
    if (!lds_set[ni][ki]) {
        allow_lds(kernels[ni][ki], lds_bytes_for(kI8MaxSC));
        lds_set[ni][ki] = true;
    }
    launch_kernel(kernels[ni][ki], grid, dim3(kT), lds, s, a);
    return static_cast<int>(hipGetLastError());
}

}  // namespace dbf
