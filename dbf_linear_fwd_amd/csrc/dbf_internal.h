// Internal declarations shared by the runtime and the kernel files.
#ifndef DBF_INTERNAL_H_
#define DBF_INTERNAL_H_

#include <cstddef>
#include <cstdint>

#include "dbf.h"

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <hip/hip_fp16.h>
#define DBF_HD __host__ __device__
#else
#define DBF_HD
struct __half;
#endif

namespace dbf {

// Largest batch served by the decode (signed-sum) kernels.
constexpr int kDecodeMaxBatch = 16;

uint32_t reorder_word(uint32_t canonical);

// Index of word w of row `row` in the tiled device layout (rows in tiles of
// 64, words in pairs); `words` is the (even) number of words per row.
DBF_HD inline size_t tiled_index(int row, int w, int words) {
    return ((static_cast<size_t>(row >> 6) * (words >> 1) + (w >> 1)) * 64 + (row & 63)) * 2 + (w & 1);
}

// ---- batch-1 decode on the int8 matrix cores (decode_i8.hip)

DBF_HD inline int round_up_int(int v, int q) { return (v + q - 1) / q * q; }

// Superchunks (512 reduction columns) of the decode layout: the reduction
// length is padded to a multiple of 128, at most kI8MaxSC superchunks.
constexpr int kI8MaxSC = 64;
int i8_superchunks(int K);

// One layer of a decode stage.  Stage 1: rows = k_pad output rows (v),
// K = m, vec = x (fp16), bsc = b, osc = mid, out = v (fp32).  Stage 2:
// rows = n, K = k_pad, vec = v (fp32), osc = a, out = y (fp16).
struct I8Layer {
    const uint32_t *S = nullptr;   // signs in the dbf_layout_signs_dec layout
    const void *vec = nullptr;
    const __half *bsc = nullptr;
    const __half *osc = nullptr;
    void *out = nullptr;
    const float *aff_E = nullptr;      // stage 2 of a 0/1 layer: y += E[row] * stats[0] + stats[1] (I8Args::aff_Q)
    const float *aff_stats = nullptr;
    int rows = 0, K = 0;
    int SC = 0, wlast = 0;             // superchunks; words per lane of the last one (1..4)
    int ntiles = 0;                    // 16-row tiles
    // set by launch_decode_i8: tiles per workgroup, waves (parts of the
    // reduction) per tile, workgroups of the layer, and each wave's job as
    // 16 bits (tile of the workgroup: 3, first superchunk: 6, superchunks: 7)
    int tpw = 0, parts = 0, nwg = 0;
    uint32_t job[4] = {0, 0, 0, 0};
};
struct I8Args {
    I8Layer L[8];
    int count = 0;
    // stage 1 of a 0/1 layer: one more workgroup forms the row sums of x
    // (stats[0] = Σ x, stats[1] = Σ gamma x); stat_wg >= 0 asks for it
    // (the workgroup at blockIdx = (0, count); count < 8 then)
    const __half *stat_x = nullptr;
    int stat_m = 0;
    const float *gamma = nullptr;
    float *stats = nullptr;
    int stat_wg = -1;
    // stage 1 of the signed launch of a group-wise BQQ layer: the statistics
    // row forms stats[q] = Σ_l stat_w[q * stat_m + l] x[l] for q < stat_Q
    // instead (stat_w not null)
    const float *stat_w = nullptr;
    int stat_Q = 0;
    // stage 2 of a 0/1 layer: the affine term's rank, y += Σ_{q < aff_Q - 1}
    // aff_E[q * rows + row] * aff_stats[q] + aff_stats[aff_Q - 1]
    // (2 <= aff_Q <= kI8MaxQ; the same for every layer of the launch)
    int aff_Q = 2;
    // batch rows (1..kI8MaxRows): vector r is at vec + r * K entries and its
    // result at out + r * rows; more than one row: signed layers, no
    // statistics row, at most kI8RowsMaxSC superchunks
    int nrows = 1;
};
constexpr int kI8MaxRows = 4;
constexpr int kI8RowsMaxSC = 16;
constexpr int kI8MaxQ = 9;
// stage = 1 or 2; bin: 0/1 matrices (Z instead of U - 2 Z, times 2).
int launch_decode_i8(I8Args &a, int stage, bool bin, void *stream);

// Arguments of the matrix-core decode kernels (batch 1..16).
struct MfmaDecodeArgs {
    const uint32_t *A_dev, *B_dev;
    const void *a_dev, *mid_dev, *b_dev;
    const void *x;
    void *y;
    uint16_t *v16;       // [2][batch][k_pad] fp16: v_hi then v_lo planes
    int batch, n, m, n_pad, m_pad, k_pad;
    // 0/1 matrices (bit 1 = 1, bit 0 = 0) instead of signs, expanded as
    // {0, 2} (the factor 2 per product is folded into the scales)
    int binary = 0;
    // optional affine output term: y[r][i] = rne16(a_i s_ri + E[i] * stats[r].x + stats[r].y)
    const float *aff_E = nullptr;
    const float *aff_stats = nullptr;  // [batch][2]
    // 0/1 layers: stage 1 also forms the per-row sums of x the affine term
    // needs, stats_out[2r] = Σ_l x[r][l], stats_out[2r + 1] = Σ_l gamma[l] x[r][l]
    const float *gamma = nullptr;
    float *stats_out = nullptr;
    // stage-1 reduction parts (mfma_stage1_parts): fp32 partials of
    // s1_part_cap floats and s1_ntickets per-row-block tickets, zero between calls
    float *s1_part = nullptr;
    size_t s1_part_cap = 0;
    unsigned *s1_tickets = nullptr;
    int s1_ntickets = 0;
};

// Parts into which the matrix-core decode cuts stage 1's reduction (over m)
// at this batch: a function of the layer's shape and of the batch's numeric
// form only (1: not cut).  Wide reductions at batch >= 2 are cut so that
// more CUs share them; the handle then needs parts * kDecodeMaxBatch * k_pad
// floats of stage-1 partials and k_pad / 16 tickets.
int mfma_stage1_parts(int m_pad, int k_pad, int batch);

// which = 1: stage 1 (writes v16); which = 2: stage 2 (writes y).
int launch_mfma_decode(const MfmaDecodeArgs &d, void *stream, int which);

// Layers that read the same input, decoded together: one launch per stage
// for all of them (workgroups map to (layer, row block)).
constexpr int kMaxGroup = 8;
struct MfmaGroupLayer {
    const uint32_t *A_dev, *B_dev;
    const void *a_dev, *mid_dev, *b_dev;
    void *y;
    uint16_t *v16;
    int n, n_pad, k_pad;
};
struct MfmaGroupArgs {
    MfmaGroupLayer L[kMaxGroup];
    int count;
    const void *x;
    int batch, m, m_pad;
};
int launch_mfma_decode_group(const MfmaGroupArgs &g, void *stream, int which);

// ---- kernel launchers (return hipError_t as int to keep HIP types out of here)

// Events that bracket the next kernel launch when the runtime times kernels
// (null otherwise).  They are handed to the launch itself, so the elapsed time
// between them is the kernel's own execution, without queueing around it.
struct LaunchEvents {
    void *start = nullptr, *stop = nullptr;
};
LaunchEvents &launch_events();

#if defined(__HIPCC__)
// Launch through hipExtLaunchKernel when a launch event is set (start: recorded
// as the kernel starts, stop: as it ends), plainly otherwise.
template <typename K, typename... Args>
inline void launch_kernel(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, Args... args) {
    const LaunchEvents &e = launch_events();
    if (e.start || e.stop)
        hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(lds), s, static_cast<hipEvent_t>(e.start),
                              static_cast<hipEvent_t>(e.stop), 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}
#endif

// Matrix-core product with a sign matrix:
//   out[i][c] = rne16( sn[c] * sum_kk P[i][kk] * S[c][kk] * (sk ? sk[kk] : 1) )
// for i < M, c < n_out.  P is fp16 row-major with leading dimension ldp and
// K valid columns (columns >= K read as 0); S is the tiled sign matrix with
// `words` words per row and at least n_rows_pad >= n_out rows.
//   out (fp16, may be null): rne16(sn[c] * sum); out32 (fp32, may be null):
//   the unscaled sum, out32[i * ldo32 + c]; dpart (may be null): batch sums
//   of sum * Q[i][c] over each group of 64 rows i (Q fp16 or fp32 as dq_f32,
//   leading dimension lddq), dpart[(i / 64) * n_out + c], to be finished by
//   launch_colsum_finish(dpart, M, n_out, ...).
//   split (may be null; fp16 output only, no out32 or dpart): where the
//   grid of output tiles is too small to fill the GPU, the K range is cut
//   into split->nsplit parts that run as separate workgroups and write
//   their unscaled fp32 sums to split->ws[s][M][split->ldw]; the caller then
//   runs launch_split_finish, which adds the parts in order s = 0, 1, ...
//   and writes out.  Where the grid is one wave of workgroups plus a small
//   partial one, only the output columns from split->col0 on (the tail) are
//   split; the columns before it are written directly.  split->nsplit is
//   set to 1 when no split was taken.
struct SplitK {
    float *ws = nullptr;  // workspace of cap floats
    size_t cap = 0;
    int nsplit = 1;       // set by launch_sign_gemm
    int ldw = 0;
    int col0 = 0;         // first output column of the split part (set by launch_sign_gemm)
};
//   flavor (may be null): binary = S holds a 0/1 matrix (bit 1 = 1), the
//   operand is then {0, 2} (callers fold the 2 into sn) and sk must be null;
//   aff_E / aff_stats: out[i][c] = rne16(sn[c] * sum + term(i, c)) with
//   term(i, c) = Σ_{q < Q-1} aff_E[q * aff_ldE + c] * aff_stats[i * Q + q]
//   + aff_stats[i * Q + Q - 1] (fp32, q in order; Q = aff_Q).
//   sk_cols > 0: output columns [j sk_cols, (j + 1) sk_cols) take the per-K
//   scale sk + j sk_stride (several products that share P, stacked along
//   the columns, each with its own scale); sk_cols a multiple of 256 (one
//   scale per output tile), the deep-pipelined product form only (K a
//   multiple of 64, 16-byte aligned rows of P), no split head and tail.
struct GemmFlavor {
    int binary = 0;
    const float *aff_E = nullptr;
    const float *aff_stats = nullptr;
    int aff_Q = 2, aff_ldE = 0;
    int sk_cols = 0, sk_stride = 0;
};
int launch_sign_gemm(const void *P, int ldp, int M, int K, const uint32_t *S, int words, int n_rows_pad,
                     const void *sk, const void *sn, void *out, int ldo, int n_out, float *out32, int ldo32,
                     const void *dq, int dq_f32, int lddq, float *dpart, void *stream, SplitK *split = nullptr,
                     const GemmFlavor *flavor = nullptr);
// Floats of split workspace that launch_sign_gemm would use for this
// product (0: it would not split), assuming 16-byte aligned rows of P.
size_t sign_gemm_split_elems(int M, int K, int words, int n_out);
// out[i][c] = rne16(sn[c] * (ws[0][i][c - col0] + ws[1][i][c - col0] + ...)
//                  [+ term(i, c) of GemmFlavor's affine form]), i < M, split.col0 <= c < n_out.
int launch_split_finish(const SplitK &split, int M, int n_out, const void *sn, void *out, int ldo, void *stream,
                        const float *aff_E = nullptr, const float *aff_stats = nullptr, int aff_Q = 2,
                        int aff_ldE = 0);

// Products of a grouped launch (layers that share their input at large
// batch): out_i = rne16(sn_i ⊙ (P_i (S_i ⊙ sk_i)ᵀ)) for i < count, every
// product with the same M rows, K_i = 32 words_i a multiple of 64, P_i
// 16-byte aligned with ldp_i % 8 == 0, sk present on all or none.  Each
// output tile is summed over its whole K (no split); launch_sign_gemm_group
// fills tile0 and returns hipErrorInvalidValue for any other form.
struct GemmItem {
    const void *P = nullptr;
    int ldp = 0, K = 0;
    const uint32_t *S = nullptr;
    int words = 0, n_rows_pad = 0;
    const void *sk = nullptr, *sn = nullptr;
    void *out = nullptr;
    int ldo = 0, n_out = 0;
};
struct GemmGroup {
    GemmItem item[kMaxGroup];
    int tile0[kMaxGroup + 1] = {};
    int count = 0, M = 0;
};
int launch_sign_gemm_group(GemmGroup &g, void *stream);

// Batch sums of the gradients: out[c] = sum over g < ceil(rows / 64) of
// partial[g * ld + c] for c < cols, added in g order (the partials are
// 64-row sums written by launch_sign_gemm's dpart epilogue).
constexpr int kColChunk = 64;
int launch_colsum_finish(const float *partial, int ld, int rows, int cols, float *out, void *stream);

// BQQ-form layers: stats[2r] = sum of row r of x (fp16, batch x m), stats[2r + 1]
// = Σ_l gamma[l] x[r][l]; fp32, fixed summation order.
int launch_bqq_rowstats(const void *x, int batch, int m, const float *gamma, float *stats, void *stream);
// Group-wise BQQ form: stats[r * Q + q] = Σ_l w[q * m + l] x[r][l] for q < Q
// (Q <= kMaxStatQ); fp32, fixed summation order.
constexpr int kMaxStatQ = 9;
int launch_bqq_rowstats_q(const void *x, int batch, int m, const float *w, int Q, float *stats, void *stream);

}  // namespace dbf

#endif  // DBF_INTERNAL_H_
