// Decode path (batch <= 16) of the DBF linear forward.
//
// §2.1 of the gist.science technical summary of "Addition is almost all you
// need" evaluates X W^T as ((((X ⊙ bᵀ) Bᵀ) ⊙ midᵀ) Aᵀ) ⊙ aᵀ: every product with
// a sign matrix is a sum of activations with their signs flipped where the
// sign is -1.  Both signed sums run on the vector ALUs in fp32:
//   stage 1: t[r][j] = sum_l B[j][l] * (x[r][l] * b[l])        (j < k)
//   stage 2: s[r][i] = sum_j A[i][j] * (t[r][j] * mid[j])      (i < n)
//            y[r][i] = rne16(s[r][i] * a[i])
//
// Work split: a workgroup (4 waves) owns a tile of 64 rows of the sign matrix
// and a chunk of its words along the reduction dimension; each lane owns one
// row, the four waves take interleaved word pairs of the chunk.  Partial sums
// of a chunk go to the workspace and are added in a fixed order, so results
// are deterministic and independent of the other batch rows.
//
// A launch takes up to 4 batch rows (larger batches run as groups of rows)
// and uses lookup tables instead of one add per sign: for every group of 4
// activations that share a nibble of a sign word, the 16 signed sums of
// those 4 values are tabulated in LDS, and a lane adds one table entry per
// nibble of its row's word.  All lanes of a wave read the
// table of the same word at the same time, so a wave's 64 reads touch at most
// 16 distinct LDS words (broadcast, no bank conflicts).
//
// Stage 2 finishes the forward itself: the last workgroup of a row tile to
// finish (a per-tile ticket counter) adds the chunk partials of that tile,
// scales by a and rounds to fp16, so a forward is two kernel launches.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "dbf_internal.h"

namespace dbf {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxPairsPerWave = (kMaxLutChunkWords / 2 + kWaves - 1) / kWaves;

// Element index (0..31) held by device bit q of a sign word.
__device__ __forceinline__ int element_of_bit(int q) { return q < 16 ? 2 * q : 2 * (q - 16) + 1; }

// Element (0..31) of lookup group `r` (nibble r of the word: bits 4r..4r+3), lane i of 4.
__device__ __forceinline__ int element_of_nibble(int r, int i) { return 8 * (r & 3) + 2 * i + (r >> 2); }

// Write the 16 signed sums of (u0..u3) to lut[0..15]; bit i of the entry index
// set means u_i enters with a minus sign (sign bit 1 = -1).
__device__ __forceinline__ void write_group(float *lut, float u0, float u1, float u2, float u3) {
    const float p0 = u0 + u1, p1 = -u0 + u1, p2 = u0 - u1, p3 = -u0 - u1;
    const float q0 = u2 + u3, q1 = -u2 + u3, q2 = u2 - u3, q3 = -u2 - u3;
    float4 *o = reinterpret_cast<float4 *>(lut);
    o[0] = make_float4(p0 + q0, p1 + q0, p2 + q0, p3 + q0);
    o[1] = make_float4(p0 + q1, p1 + q1, p2 + q1, p3 + q1);
    o[2] = make_float4(p0 + q2, p1 + q2, p2 + q2, p3 + q2);
    o[3] = make_float4(p0 + q3, p1 + q3, p2 + q3, p3 + q3);
}

// (a & 60) | c in one VALU instruction: the byte offset of a nibble's table
// entry (a holds the nibble at bits 2..5) merged with the 64-byte aligned
// table base c.  The compiler would otherwise turn the "or" into an add.
__device__ __forceinline__ uint32_t nibble_address(uint32_t a, uint32_t c) {
    uint32_t d;
    asm("v_and_or_b32 %0, %1, 60, %2" : "=v"(d) : "v"(a), "v"(c));
    return d;
}

typedef __attribute__((address_space(3))) const float lds_float;

// 32-bit LDS offset of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_offset(const float *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_float *)(p)));
}

// Load the fp32 table entry at LDS byte offset `addr` + `imm` (imm folds into the instruction).
__device__ __forceinline__ float lds_load(uint32_t addr, int imm) {
    return ((lds_float *)(static_cast<uintptr_t>(addr)))[imm / 4];
}

// Load this lane's words of the chunk: pairs pl = wave, wave + 4, ... of the
// chunk (`npairs` pairs starting at pair p0 of the row).
__device__ __forceinline__ void load_pairs(uint2 (&wd)[kMaxPairsPerWave], const uint32_t *__restrict__ S,
                                           int tile, int row_in_tile, int words, int p0, int npairs, int wave) {
    const uint2 *S2 = reinterpret_cast<const uint2 *>(S);
#pragma unroll
    for (int s = 0; s < kMaxPairsPerWave; ++s) {
        const int pl = wave + kWaves * s;
        wd[s] = make_uint2(0u, 0u);
        if (pl < npairs) {
            const size_t idx = (static_cast<size_t>(tile) * (words >> 1) + (p0 + pl)) * 64 + row_in_tile;
            wd[s] = S2[idx];
        }
    }
}

// Table lookups for this lane's words; acc[rb] += sum over nibbles.  The 16
// reads of a word pair are issued before the adds so their LDS latency overlaps.
template <int NB>
__device__ __forceinline__ void lookup_pairs(float (&acc)[NB], const uint2 (&wd)[kMaxPairsPerWave],
                                             const float *lut, int CW, int npairs, int wave) {
    const uint32_t lut0 = lds_offset(lut);
#pragma unroll
    for (int s = 0; s < kMaxPairsPerWave; ++s) {
        const int pl = wave + kWaves * s;
        if (pl < npairs) {
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                float e[16];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t word = h ? wd[s].y : wd[s].x;
                    // LDS address of this word's 8 tables (512 bytes, 512-byte
                    // aligned, so the low 9 bits are free for the entry offset)
                    const uint32_t base = lut0 + static_cast<uint32_t>((rb * CW + 2 * pl + h) * 512);
                    e[8 * h] = lds_load(nibble_address(word << 2, base), 0);
#pragma unroll
                    for (int r = 1; r < 8; ++r) e[8 * h + r] = lds_load(nibble_address(word >> (4 * r - 2), base), r * 64);
                }
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[rb] += e[q];
            }
        }
    }
}

// Sum the per-wave accumulators of the workgroup (fixed order) into wave 0.
template <int NB>
__device__ __forceinline__ void reduce_waves(float (&acc)[NB], float *red, int wave, int lane) {
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) red[(wave * NB + rb) * 64 + lane] = acc[rb];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            float s = red[rb * 64 + lane];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) s += red[(w * NB + rb) * 64 + lane];
            acc[rb] = s;
        }
    }
}

template <int NB>
__global__ __launch_bounds__(kThreads) void lut_stage1_kernel(const uint32_t *__restrict__ Bt,
                                                              const __half *__restrict__ x,
                                                              const __half *__restrict__ b,
                                                              float *__restrict__ tpart, int m, int Wm,
                                                              int k_pad, int CW) {
    extern __shared__ float lds[];           // no static shared: the table starts at offset 0
    float *lut = lds;                         // [NB][CW][8][16]
    float *red = lds + NB * CW * 128;         // [kWaves][NB][64]
    const int tile = blockIdx.x;
    const int c = blockIdx.y;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int w0 = c * CW;
    const int nw = min(CW, Wm - w0);
    const int npairs = nw >> 1;

    uint2 wd[kMaxPairsPerWave];
    load_pairs(wd, Bt, tile, lane, Wm, w0 >> 1, npairs, wave);

    // table of u = x * b for the chunk's columns
    for (int g = threadIdx.x; g < NB * nw * 8; g += kThreads) {
        const int r = g & 7;
        const int wl = (g >> 3) % nw;
        const int rb = (g >> 3) / nw;
        const int base = 32 * (w0 + wl);
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int l = base + element_of_nibble(r, i);
            u[i] = l < m ? __half2float(x[static_cast<size_t>(rb) * m + l]) * __half2float(b[l]) : 0.0f;
        }
        write_group(lut + ((rb * CW + wl) * 8 + r) * 16, u[0], u[1], u[2], u[3]);
    }
    __syncthreads();

    float acc[NB];
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) acc[rb] = 0.0f;
    lookup_pairs<NB>(acc, wd, lut, CW, npairs, wave);
    reduce_waves<NB>(acc, red, wave, lane);
    if (wave == 0) {
        const int j = tile * 64 + lane;
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) tpart[(static_cast<size_t>(c) * NB + rb) * k_pad + j] = acc[rb];
    }
}

template <int NB>
__global__ __launch_bounds__(kThreads) void lut_stage2_kernel(const uint32_t *__restrict__ At,
                                                              const float *__restrict__ tpart,
                                                              const __half *__restrict__ mid,
                                                              const __half *__restrict__ a,
                                                              float *__restrict__ ypart,
                                                              unsigned *__restrict__ tickets,
                                                              __half *__restrict__ y, int n, int Wk,
                                                              int n_pad, int k_pad, int nchunk_m, int nchunk_k,
                                                              int CW) {
    // No static shared variables here: the table must start at LDS offset 0
    // (512-byte aligned bases, see lookup_pairs).
    extern __shared__ float lds[];
    float *lut = lds;
    float *red = lds + NB * CW * 128;
    int *s_last = reinterpret_cast<int *>(red + kWaves * NB * 64);
    const int tile = blockIdx.x;
    const int c = blockIdx.y;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int w0 = c * CW;
    const int nw = min(CW, Wk - w0);
    const int npairs = nw >> 1;

    uint2 wd[kMaxPairsPerWave];
    load_pairs(wd, At, tile, lane, Wk, w0 >> 1, npairs, wave);

    // table of v = mid * t, t the fixed-order sum of the stage-1 chunk partials
    for (int g = threadIdx.x; g < NB * nw * 8; g += kThreads) {
        const int r = g & 7;
        const int wl = (g >> 3) % nw;
        const int rb = (g >> 3) / nw;
        const int base = 32 * (w0 + wl);
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = base + element_of_nibble(r, i);
            float t = 0.0f;
            for (int cm = 0; cm < nchunk_m; ++cm) t += tpart[(static_cast<size_t>(cm) * NB + rb) * k_pad + j];
            v[i] = t * __half2float(mid[j]);
        }
        write_group(lut + ((rb * CW + wl) * 8 + r) * 16, v[0], v[1], v[2], v[3]);
    }
    __syncthreads();

    float acc[NB];
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) acc[rb] = 0.0f;
    lookup_pairs<NB>(acc, wd, lut, CW, npairs, wave);
    reduce_waves<NB>(acc, red, wave, lane);

    const int i = tile * 64 + lane;
    if (nchunk_k == 1) {
        if (wave == 0 && i < n) {
            const float sa = __half2float(a[i]);
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) y[static_cast<size_t>(rb) * n + i] = __float2half_rn(acc[rb] * sa);
        }
        return;
    }
    if (wave == 0) {
#pragma unroll
        for (int rb = 0; rb < NB; ++rb)
            __hip_atomic_store(&ypart[(static_cast<size_t>(c) * NB + rb) * n_pad + i], acc[rb], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    // Publish the partial (agent-scope atomic stores, written through to
    // memory, completed before the ticket: no release fence, whose write-back
    // of the whole L2 costs microseconds per workgroup), then take a ticket;
    // the last of the tile's chunks adds all partials of the tile in chunk
    // order with agent-scope loads.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&tickets[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = prev == static_cast<unsigned>(nchunk_k - 1);
    }
    __syncthreads();
    if (!*s_last) return;
    if (wave == 0 && i < n) {
        const float sa = __half2float(a[i]);
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            float s = 0.0f;
            for (int cc = 0; cc < nchunk_k; ++cc) {
                s += __hip_atomic_load(&ypart[(static_cast<size_t>(cc) * NB + rb) * n_pad + i], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            y[static_cast<size_t>(rb) * n + i] = __float2half_rn(s * sa);
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(&tickets[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


template <int NB>
size_t lut_lds_bytes(int CW) {
    return sizeof(float) * (static_cast<size_t>(NB) * CW * 128 + kWaves * NB * 64 + 4);
}

template <int NB>
int lut_stage1(const DecodeArgs &d, hipStream_t s) {
    launch_kernel(lut_stage1_kernel<NB>, dim3(d.k_pad / 64, d.nchunk_m), dim3(kThreads),
                       lut_lds_bytes<NB>(d.cw_m), s, d.B_dev, static_cast<const __half *>(d.x),
                       static_cast<const __half *>(d.b_dev), d.tpart, d.m, d.m_pad / 32, d.k_pad, d.cw_m);
    return static_cast<int>(hipGetLastError());
}

template <int NB>
int lut_stage2(const DecodeArgs &d, hipStream_t s) {
    launch_kernel(lut_stage2_kernel<NB>, dim3(d.n_pad / 64, d.nchunk_k), dim3(kThreads),
                       lut_lds_bytes<NB>(d.cw_k), s, d.A_dev, d.tpart, static_cast<const __half *>(d.mid_dev),
                       static_cast<const __half *>(d.a_dev), d.ypart, d.tickets, static_cast<__half *>(d.y), d.n,
                       d.k_pad / 32, d.n_pad, d.k_pad, d.nchunk_m, d.nchunk_k, d.cw_k);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

int lut_max_chunk_words(int nb) {
    // LDS budget of one workgroup: the table (512 bytes per word per batch
    // row) plus the cross-wave reduction buffer stay below 63 KiB.
    const int w = (64512 - 1024 * nb) / (512 * nb);
    return (w < kMaxLutChunkWords ? w : kMaxLutChunkWords) & ~1;
}

int launch_lut_stage1(const DecodeArgs &d, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (d.batch) {
        case 1: return lut_stage1<1>(d, s);
        case 2: return lut_stage1<2>(d, s);
        case 3: return lut_stage1<3>(d, s);
        case 4: return lut_stage1<4>(d, s);
        default: return static_cast<int>(hipErrorInvalidValue);
    }
}

int launch_lut_stage2(const DecodeArgs &d, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (d.batch) {
        case 1: return lut_stage2<1>(d, s);
        case 2: return lut_stage2<2>(d, s);
        case 3: return lut_stage2<3>(d, s);
        case 4: return lut_stage2<4>(d, s);
        default: return static_cast<int>(hipErrorInvalidValue);
    }
}

}  // namespace dbf
