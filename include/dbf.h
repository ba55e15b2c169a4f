/*
 * dbf.h -- C ABI of the Double Binary Factorization (DBF) linear forward for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * Source: "Addition is almost all you need: Compressing large language models
 * with double binary factorization", technical summary on gist.science,
 * §2.1 (mathematical formulation), and Figure 1's caption on the
 * sciencestack.ai page of the same paper.
 *
 * A weight matrix W (n x m; n outputs, m inputs) is stored as
 *     W = diag(a) * A * diag(mid) * B * diag(b)
 * with A an n x k matrix of +1/-1, B a k x m matrix of +1/-1 and fp16 scale
 * vectors a (n), mid (k) and b (m).  (The pages name the middle vector "m";
 * it is "mid" here because m is also the input width.)  For an fp16 input X
 * of shape batch x m the layer returns the fp16 matrix Y = X * W^T of shape
 * batch x n, evaluated right to left as §2.1 orders it: scale the input
 * columns by b, take signed sums along m with B, scale by mid, take signed
 * sums along k with A, scale by a.  The products with A and B are additions
 * and sign flips; no dense W is formed.
 *
 * Numerics: fp16 in and out, one round-to-nearest-even to fp16 at the end;
 * no flush-to-zero.  At batch 1 (layers with m and k_pad up to 32768) each
 * signed sum is exact: the vector (u = x * b, then v) is brought to 32-bit
 * fixed point with one power-of-two exponent, summed as integers on the
 * int8 matrix cores, and v = t * mid is kept in fp32; u may exceed the fp16
 * range there.  DBF_PATH_DECODE_EXACT runs the same exact sums at batch 2..4
 * (+/-1 layers with m and k_pad up to 8192), each batch row with its own
 * exponent, so a row's result is the same bits whatever batch it runs in.
 * At decode batch 2..16 otherwise and on the prefill path the sums
 * accumulate in fp32 and v is rounded once to fp16, the operand of 16-bit
 * matrix-core products, so it must stay inside the fp16 range
 * (|v| < 65520); batch 1 on wider layers keeps v as the sum of two fp16
 * numbers (about 22 significant bits), and u = x * b as well, so there
 * |x * b| must stay below 65520 too.
 *
 * Packed sign format (the pages fix none; this is the library's own)
 * ----------------------------------------------------------------------
 * Signs are packed along each matrix's reduction dimension: A along k, B
 * along m.  32 signs per uint32, element 32*w + p of a row in bit p of word w
 * (least significant bit first); bit value 1 means -1, 0 means +1.  Bits past
 * the end of a row are 0.  This is the format dbf_pack_signs() writes.  The
 * device keeps its own tiled copy (see dbf_layout_signs()).
 *
 * Conventions
 * -----------
 * All functions have C linkage and return a status; no C++ exception crosses
 * this boundary.  Host pointers are read during the call and not retained
 * (the caller keeps ownership).  Device pointers stay owned by the caller.
 * Kernel launches are asynchronous on the given stream; a device fault
 * surfaces at the caller's next synchronisation, not in the return value.
 */
#ifndef DBF_H_
#define DBF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP runtime's stream type (identical to its own declaration). */
typedef struct ihipStream_t *hipStream_t;

typedef struct dbf_layer *dbf_handle_t;

typedef enum {
    DBF_OK = 0,
    DBF_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, sign not +/-1, bad batch */
    DBF_ERR_SHAPE = 2,       /* sizes whose byte counts overflow, or exceed the kernels' limits */
    DBF_ERR_OOM = 3,         /* device or host allocation failed; nothing leaks */
    DBF_ERR_HIP = 4,         /* a HIP runtime call failed (includes: no GPU present) */
    DBF_ERR_UNSUPPORTED = 5  /* a valid request this build does not implement */
} dbf_status_t;

/* Kernel-path selection for dbf_linear_forward_ex(). */
typedef enum {
    DBF_PATH_AUTO = 0,         /* batch <= 16: DBF_PATH_DECODE; batch > 16: DBF_PATH_PREFILL */
    DBF_PATH_DECODE = 1,       /* small-batch kernels: exact int8 matrix-core sums with v in fp32
                                  (batch 1), batch as the MFMA N dimension with v rounded once to
                                  fp16 (batch 2..16); batch must be <= 16 */
    DBF_PATH_PREFILL = 2,      /* tiled MFMA products, intermediate rounded once to fp16; any batch */
    DBF_PATH_DECODE_TABLE = 3, /* no longer built (it was slower than the matrix cores at every
                                  measured shape): always DBF_ERR_UNSUPPORTED */
    DBF_PATH_DECODE_EXACT = 4  /* batch 1..4: the exact int8 sums of batch 1, one fixed-point
                                  exponent per batch row, so every output row has the bits of its
                                  own batch-1 forward (batch-invariant results, for callers that
                                  must reproduce a request's output whatever it was batched with);
                                  slower than DBF_PATH_DECODE at batch 3..4.  batch > 4 is
                                  DBF_ERR_INVALID_ARG; 0/1 (BQQ-form) layers, and layers with m
                                  or k_pad above 32768 (batch 1) or above 8192 (batch 2..4), are
                                  DBF_ERR_UNSUPPORTED */
} dbf_path_t;

typedef struct {
    int32_t n, m, k;          /* logical sizes */
    int32_t n_pad, m_pad, k_pad; /* device sizes: each rounded up to a multiple of 64 */
    int32_t max_batch;
    int32_t device;           /* HIP device the handle lives on */
    size_t packed_bytes;      /* device bytes of packed A and B (padding included; with DBF_PACK_BACKWARD
                                 the transposed copies too) */
    size_t scale_bytes;       /* device bytes of a, mid, b (padding included) */
    size_t workspace_bytes;   /* device scratch owned by the handle */
} dbf_info_t;

/*
 * dbf_pack -- build a layer handle from its factors (§2.1: A, B, a, mid, b).
 *   n, m, k     >= 1: output width, input width, middle dimension.
 *   A_signs     host int8, n x k row-major, every entry +1 or -1.
 *   B_signs     host int8, k x m row-major, every entry +1 or -1.
 *   a, mid, b   host fp16 bit patterns (uint16), lengths n, k, m.
 *   max_batch   >= 1: largest batch later passed to dbf_linear_forward.
 *   out         receives the handle.
 * Packs the signs on the CPU, uploads them and the scales to the current HIP
 * device, and allocates the handle's workspace for max_batch.  Arguments are
 * validated before any HIP call.  On failure *out is set to NULL (when out is
 * not NULL) and nothing leaks.  Errors: DBF_ERR_INVALID_ARG, DBF_ERR_SHAPE,
 * DBF_ERR_OOM, DBF_ERR_HIP.
 */
dbf_status_t dbf_pack(int32_t n, int32_t m, int32_t k,
                      const int8_t *A_signs, const int8_t *B_signs,
                      const uint16_t *a, const uint16_t *mid, const uint16_t *b,
                      int32_t max_batch, dbf_handle_t *out);

/*
 * dbf_linear_forward -- Y = X W^T for the layer h (§2.1 evaluation order).
 *   x      device fp16, batch x m row-major (caller-owned, 16-byte aligned).
 *   y      device fp16, batch x n row-major (caller-owned, 16-byte aligned,
 *          must not overlap x).  Fully overwritten.
 *   batch  0 <= batch <= max_batch; 0 returns DBF_OK without launching.
 *   stream HIP stream to launch on (NULL = the null stream).
 * Enqueues the kernels and returns; no host synchronisation.  The current
 * HIP device must be the handle's.  The handle's workspace is shared by its
 * calls: calls on one handle must be ordered (e.g. all on one stream).
 * Errors: DBF_ERR_INVALID_ARG (null handle or pointers, batch out of range,
 * misaligned pointers, wrong device), DBF_ERR_HIP (launch failure).
 */
dbf_status_t dbf_linear_forward(dbf_handle_t h, const void *x, void *y, int32_t batch,
                                hipStream_t stream);

/*
 * dbf_linear_forward_ex -- dbf_linear_forward with an explicit kernel path
 * (dbf_path_t).  DBF_PATH_DECODE with batch > 16 is DBF_ERR_INVALID_ARG.
 * The paths compute the same function; they differ in the fp16 rounding of
 * the intermediate and in the summation (see "Numerics" above).
 */
dbf_status_t dbf_linear_forward_ex(dbf_handle_t h, const void *x, void *y, int32_t batch,
                                   int32_t path, hipStream_t stream);

/*
 * dbf_linear_forward_group -- the forwards of several layers that read the
 * same input (for example the q, k and v projections of an attention block,
 * or the gate and up projections of an MLP, gist.science technical summary
 * §4 runs DBF on every linear layer of such blocks): ys[i] = x W_i^T for
 * i < count, as dbf_linear_forward(hs[i], x, ys[i], batch, ...) computes
 * it (see below for the bits).
 *   hs     count handles (1 <= count <= 8), all with the same input width m,
 *          all on the current device.
 *   x      device fp16, batch x m (shared by all layers, 16-byte aligned).
 *   ys     count device fp16 outputs, ys[i] batch x n_i, 16-byte aligned,
 *          overlapping neither x nor each other.
 *   batch  0 <= batch <= every handle's max_batch; 0 returns DBF_OK.
 * For batch <= 16 all layers share one launch per stage (2 launches in all
 * instead of 2 per layer), and each output is bit-identical to the layer's
 * own forward.  Above batch 16, when m is a multiple of 64, the layers share
 * one launch per product (the tiles of every layer in one grid, each summed
 * over its whole K); a layer's own forward may cut K into parts there, so
 * the two agree within the parity tolerance rather than bit for bit.  Other
 * shapes run each layer's forward in turn.
 * The handles' workspaces are used: calls involving one handle must be
 * ordered.  Errors: DBF_ERR_INVALID_ARG (count out of range, null pointers,
 * differing m, batch out of range, misaligned pointers, wrong device),
 * DBF_ERR_HIP (launch failure).
 */
dbf_status_t dbf_linear_forward_group(const dbf_handle_t *hs, int32_t count, const void *x, void *const *ys,
                                      int32_t batch, hipStream_t stream);

/*
 * dbf_linear_forward_noalloc -- dbf_linear_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and the same results,
 * bit for bit, but their scratch (the intermediate, split-K and stage-1
 * partials, tickets, the row sums of 0/1 layers) lives in a static device
 * array of 64 MiB compiled into the library instead of the handle's
 * workspace.  Each device that runs it holds its own copy of the array until
 * the process ends; the copy's address is resolved on the first call on that
 * device.  No allocation at all: no hipMalloc or hipFree, no library routine
 * that allocates, no timing events (kernel timing of the handle is paused
 * for the call).
 *   Arguments and their ownership are those of dbf_linear_forward.
 *   Every call on a device shares that device's array, which keeps the last
 *   call's contents: calls that overlap on one device (other streams, other
 *   threads) race and must be ordered by the caller.  What must start at
 *   zero is cleared by the call itself (a kernel, not a memset).
 * Errors: as dbf_linear_forward, plus DBF_ERR_SHAPE when this batch needs
 * more scratch than the array holds (decode batches always fit; the
 * batch-2048 products fit for k_pad up to about 16000), and
 * DBF_ERR_UNSUPPORTED for a device index of 64 or more.
 */
dbf_status_t dbf_linear_forward_noalloc(dbf_handle_t h, const void *x, void *y, int32_t batch,
                                        hipStream_t stream);

/*
 * dbf_pack_ex -- dbf_pack with flags.  DBF_PACK_BACKWARD also packs the
 * transposed factors (Aᵀ along n, Bᵀ along k; the transpose of a DBF matrix
 * is the DBF matrix diag(b) Bᵀ diag(mid) Aᵀ diag(a)) and allocates the fp32
 * workspace of the gradients (4 * max_batch * (2 k_pad + n + m) bytes and
 * the reduction partials), for dbf_linear_backward_data and
 * dbf_linear_backward.  Unknown flags are DBF_ERR_INVALID_ARG.
 */
#define DBF_PACK_BACKWARD 1
dbf_status_t dbf_pack_ex(int32_t n, int32_t m, int32_t k,
                         const int8_t *A_signs, const int8_t *B_signs,
                         const uint16_t *a, const uint16_t *mid, const uint16_t *b,
                         int32_t max_batch, int32_t flags, dbf_handle_t *out);

/*
 * dbf_bqq_pack -- a layer whose weight is in the binary-quadratic form of
 * the TL;DR of "Binary Quadratic Quantization: Beyond First-Order
 * Quantization for Real-Valued Matrix Compression" (sciencestack.ai page):
 *   W = Σ_{i<p} ( r_i Y_i Z_i + s_i Y_i 1 + t_i 1 Z_i ) + u 1        (n x m)
 * with Y_i (n x d) and Z_i (d x m) 0/1 matrices and 1 an all-ones matrix of
 * the shape that fits.  The returned handle takes dbf_linear_forward and
 * dbf_linear_forward_ex (paths AUTO, DECODE, PREFILL) with the contract of a
 * DBF layer: y = rne16(x Wᵀ), fp32 accumulation, one final rounding.
 *   Y      host uint8, p x n x d (row-major, term-major), entries 0 or 1.
 *   Z      host uint8, p x d x m, entries 0 or 1.
 *   r,s,t  host fp16 bit patterns, p each; u one fp16 bit pattern.
 * The p products run as one DBF product with middle dimension p*d on the
 * DBF kernels (0/1 operands, mid = r_i per term); the other terms reduce to
 * E[o] * Σx + γ·x with E[o] = Σ_i s_i (row o of Y_i summed) + u and
 * γ[l] = Σ_i t_i (column l of Z_i summed), formed at pack time in double
 * precision and kept in fp32; the per-row sums Σx and γ·x (fp32, one small
 * kernel per forward) enter the output epilogue before its rounding.  The
 * intermediate (batch x p d) follows the DBF path rules (fp32 from exact
 * sums at decode batch 1, else one fp16 rounding, in fp16 range).
 * Errors: DBF_ERR_INVALID_ARG (null pointers, sizes < 1, entries not 0/1),
 * DBF_ERR_SHAPE, DBF_ERR_OOM, DBF_ERR_HIP.  Grouped forwards and gradients
 * return DBF_ERR_UNSUPPORTED for such a handle.
 */
dbf_status_t dbf_bqq_pack(int32_t n, int32_t m, int32_t d, int32_t p,
                          const uint8_t *Y, const uint8_t *Z,
                          const uint16_t *r, const uint16_t *s, const uint16_t *t, uint16_t u,
                          int32_t max_batch, dbf_handle_t *out);

/*
 * dbf_bqq_pack_grouped -- the binary-quadratic form with group-wise scalars.
 * The same TL;DR names group-wise scaling as the way the form keeps its
 * parameter overhead low (and the page's Figure 2 is on weight scaling) but
 * gives no formula; the reading here: the m input columns fall into groups
 * of `group` consecutive columns (the last may be shorter), each with its
 * own scalars, the 0/1 matrices shared.  On the columns l of group h,
 *   W[:, l] = Σ_{i<p} ( r_i[h] Y_i Z_i + s_i[h] Y_i 1 + t_i[h] 1 Z_i )[:, l] + u[h].
 *   Y, Z   as for dbf_bqq_pack.
 *   r,s,t  host fp16 bit patterns, p x ngroups (term-major), ngroups =
 *          ceil(m / group); u host fp16 bit patterns, ngroups.
 * One group (group >= m) is dbf_bqq_pack exactly.  With more groups the
 * layer runs as: p signed first products on the DBF kernels (Z_i as ±1 signs,
 * per-term input scale b_i[l] = r_i[h(l)], mid = 1), the 0/1 product of the
 * Y_i with a = -1/4, and a rank-(p + 1) affine term Σ_i R_i[o] σ_i + κ
 * (R_i[o] the row sums of Y_i; σ_i, κ per input row: fp32 sums of x with
 * weights s_i[h] + r_i[h] / 2 and Σ_i t_i[h] (column sums of Z_i) + u[h],
 * formed at pack time in double precision and kept in fp32) added before
 * the one rounding.  Paths: AUTO runs the int8 decode kernels at batch 1
 * and the prefill products at every other batch; DECODE serves batch 1
 * only (DBF_ERR_UNSUPPORTED otherwise); PREFILL any batch.  The
 * intermediate follows the DBF path rules.
 * Limits: d a multiple of 64 and p <= 8 when there is more than one group
 * (DBF_ERR_SHAPE otherwise).
 * Errors: as dbf_bqq_pack.  Grouped forwards, gradients and
 * dbf_linear_forward_noalloc return DBF_ERR_UNSUPPORTED for such a handle.
 */
dbf_status_t dbf_bqq_pack_grouped(int32_t n, int32_t m, int32_t d, int32_t p, int32_t group,
                                  const uint8_t *Y, const uint8_t *Z,
                                  const uint16_t *r, const uint16_t *s, const uint16_t *t, const uint16_t *u,
                                  int32_t max_batch, dbf_handle_t *out);

/*
 * dbf_factorize -- the DBF factors of a weight matrix W (n x m), the step
 * before packing.  Technical summary (gist.science) of "Addition is almost
 * all you need", §2.2: alternating minimization of the two factors, ADMM
 * for each constrained subproblem, SVID projection onto sign matrices with
 * a rank-one scaling, importance scaling of rows and columns.  With
 * T = diag(d_out) W diag(d_in) and W ~ U V, U = diag(a) A diag(c_u),
 * V = diag(c_v) B diag(b), each of `outer` iterations updates U with V
 * fixed and then V with U fixed by `inner` ADMM iterations:
 *   X = (T' F + rho (Z - L)) (F^T F + rho I)^{-1},  Z = SVID(X + L),
 *   L = L + X - Z,   rho = rho_rel * trace(F^T F) / k,
 * starting from the current factor (Z) and L = 0; SVID(M) = sign(M) times
 * the rank-one approximation of |M| from `power_iters` power-method steps
 * (sign(0) = +1).  mid = c_u * c_v; a and b are divided by their RMS and
 * mid multiplied by both before the one rounding to fp16.
 *   W      device fp32, n x m row-major.
 *   U0, V0 device fp32, n x k and k x m row-major: the starting factors.
 *   d_out, d_in  device fp32 row / column importance (n, m), or NULL (1).
 *   A, B   device int8 outputs, n x k and k x m, entries +1 / -1 (the input
 *          format of dbf_pack).
 *   a, mid, b  device fp16 outputs (n, k, m).
 *   err    device fp32 [outer] or NULL: ||T - U V||_F / ||T||_F after each
 *          outer iteration.
 * fp32 arithmetic: dense products on rocBLAS GEMMs, (F^T F + rho I)^{-1} by
 * Newton-Schulz iteration, the rest in the library's kernels; reductions in
 * a fixed order (repeated calls give identical results).  Allocates its
 * workspace (about 4 n m + 8 max(n, m) k + 4 k^2 floats) and frees it before
 * returning; synchronizes `stream`.
 * Errors: DBF_ERR_INVALID_ARG (null pointers, sizes or counts < 1,
 * rho_rel <= 0), DBF_ERR_SHAPE, DBF_ERR_OOM, DBF_ERR_HIP.
 */
dbf_status_t dbf_factorize(const float *W, int32_t n, int32_t m, int32_t k,
                           const float *U0, const float *V0, const float *d_out, const float *d_in,
                           float rho_rel, int32_t outer, int32_t inner, int32_t power_iters,
                           int8_t *A, int8_t *B, uint16_t *a, uint16_t *mid, uint16_t *b, float *err,
                           hipStream_t stream);

/*
 * dbf_linear_backward_data -- dX = dY W (batch x m, fp16) for an upstream
 * gradient dY (batch x n, fp16): the forward of the transposed layer, with
 * the same kernels and numerics as dbf_linear_forward.  Fine-tuning of the
 * factors is part of the method (gist.science technical summary, §4: tuning
 * of the binary factors; §5: its memory cost as open work).  Needs a handle
 * packed with DBF_PACK_BACKWARD (else DBF_ERR_UNSUPPORTED).  Pointer and
 * batch rules as dbf_linear_forward.
 */
dbf_status_t dbf_linear_backward_data(dbf_handle_t h, const void *dy, void *dx, int32_t batch,
                                      hipStream_t stream);

/*
 * dbf_linear_backward -- gradients of the layer at input x (batch x m, fp16)
 * for the upstream gradient dy (batch x n, fp16):
 *   dx[r,l]  = Σ_i dy[r,i] W[i,l]                        fp16, batch x m
 *   da[i]    = Σ_r dy[r,i] s[r,i],   s = ((x ⊙ b) Bᵀ ⊙ mid) Aᵀ      fp32, n
 *   dmid[j]  = Σ_r g[r,j] t[r,j],    t = (x ⊙ b) Bᵀ, g = (dy ⊙ a) A  fp32, k
 *   db[l]    = Σ_r h[r,l] x[r,l],    h = (g ⊙ mid) B                fp32, m
 * All four products run on the matrix cores (the prefill kernels) with fp32
 * accumulation; t ⊙ mid and g ⊙ mid are rounded once to fp16 as operands of
 * the second products (as on the prefill forward).  Sums over the batch are
 * taken in a fixed order: repeated calls give identical bits.  Any of dx,
 * da, dmid, db may be NULL (not computed).  Device pointers, caller-owned;
 * x, dy, dx 16-byte aligned.  0 <= batch <= max_batch.  Needs
 * DBF_PACK_BACKWARD (else DBF_ERR_UNSUPPORTED).  Calls on one handle must be
 * ordered (the workspace is shared).
 */
dbf_status_t dbf_linear_backward(dbf_handle_t h, const void *x, const void *dy, void *dx, float *da,
                                 float *dmid, float *db, int32_t batch, hipStream_t stream);

/* dbf_free -- release the handle and its device memory.  NULL is a no-op.
 * Synchronises the handle's device first, so pending work on it finishes. */
void dbf_free(dbf_handle_t h);

/* dbf_get_info -- sizes of the handle (host-only; no HIP call). */
dbf_status_t dbf_get_info(dbf_handle_t h, dbf_info_t *info);

/* dbf_status_string -- static English text for a status code. */
const char *dbf_status_string(dbf_status_t s);

/*
 * dbf_pack_signs -- host-only packer into the format described above.
 *   S              host int8, rows x cols row-major, entries +1 or -1.
 *   out            host uint32, rows x words_per_row, fully written
 *                  (words past ceil(cols/32) are written as 0).
 *   words_per_row  >= ceil(cols / 32).
 * Errors: DBF_ERR_INVALID_ARG (null pointer, rows/cols < 1, a sign not +/-1,
 * words_per_row too small).  Needs no GPU.
 */
dbf_status_t dbf_pack_signs(const int8_t *S, int32_t rows, int32_t cols,
                            uint32_t *out, int32_t words_per_row);

/*
 * dbf_layout_signs -- host-only: the device copy's tiling of packed signs.
 *   in         host uint32, rows x words row-major, in the dbf_pack_signs format.
 *   rows       >= 1;  words >= 1 and even.
 *   out        host uint32 of dbf_layout_words(rows, words) entries.
 * Layout: rows are grouped in tiles of 64 (the last tile zero-filled), words
 * in pairs; out[((tile * (words/2) + pair) * 64 + r) * 2 + h] holds word
 * 2*pair + h of row 64*tile + r, so one wavefront reading one row per lane
 * touches 512 contiguous bytes.  Inside each word the bits are reordered so
 * that element 2q of the 32-element block is at bit q and element 2q+1 at
 * bit 16+q (q = 0..15): a pair of neighbouring elements then sits at the two
 * fp16 sign-bit positions after one shift.  Needs no GPU.
 */
dbf_status_t dbf_layout_signs(const uint32_t *in, int32_t rows, int32_t words, uint32_t *out);
size_t dbf_layout_words(int32_t rows, int32_t words);

/*
 * dbf_layout_signs_dec -- host-only: the copy of packed signs that the
 * batch-1 decode kernels read (int8 matrix cores).
 *   in         host uint32, rows x words row-major, in the dbf_pack_signs format
 *              (words >= ceil(cols / 32)).
 *   rows, cols the matrix (>= 1); rows_pad >= rows, a multiple of 16;
 *              cols_pad >= cols, a multiple of 128.
 *   out        host uint32 of dbf_layout_words_dec(rows_pad, cols_pad) entries,
 *              fully written (padding rows and columns hold 0 bits).
 * Layout: rows in tiles of 16, columns in superchunks of 512 (the last one
 * may hold 128, 256 or 384).  In superchunk s of tile T, lane l = r + 16 g
 * (r < 16, g < 4) owns W words (W = 4, or (cols_pad - 512 s) / 128 in a short
 * last superchunk); its word i is out[T * cols_pad / 2 + 256 s + W l + i], and
 * bit 8 b + j of that word (j < 8, b < 4) is the sign bit of column
 * 512 s + 128 i + 16 j + 4 g + b of row 16 T + r.  A word AND 0x01010101 << j
 * then holds four int8 values 0 or 2^j, the operand of an int8 matrix-core
 * product over those four columns.  The entry count includes 4 words of
 * padding after the last tile.  Needs no GPU.
 */
dbf_status_t dbf_layout_signs_dec(const uint32_t *in, int32_t rows, int32_t cols, int32_t words,
                                  int32_t rows_pad, int32_t cols_pad, uint32_t *out);
size_t dbf_layout_words_dec(int32_t rows_pad, int32_t cols_pad);

/*
 * Kernel timing (measurement support).  When enabled on a handle, every
 * kernel the handle launches carries a pair of HIP events on the launch itself
 * (hipExtLaunchKernel), so their elapsed time is that kernel's execution on
 * its stream.  dbf_timing_read() synchronises those events and returns, per
 * kernel name, the number of launches and the summed elapsed time since the
 * last read.  Disabled by default.  dbf_timing_read fills at most `cap`
 * entries and sets *count to the number of distinct kernels seen.
 */
typedef struct {
    char name[48];
    int64_t launches;
    double total_ms;
} dbf_kernel_time_t;

dbf_status_t dbf_timing_enable(dbf_handle_t h, int32_t enable);
dbf_status_t dbf_timing_read(dbf_handle_t h, dbf_kernel_time_t *out, int32_t cap, int32_t *count);

#ifdef __cplusplus
}
#endif

#endif /* DBF_H_ */
