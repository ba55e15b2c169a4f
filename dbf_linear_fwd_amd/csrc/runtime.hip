// Host runtime of the DBF layer: handle, upload, kernel choice and launch.
//
// The layer is W = diag(a) A diag(mid) B diag(b) with ±1 factors A (n x k),
// B (k x m) and fp16 scales ("Addition is almost all you need", gist.science
// technical summary, §2.1; the fp16 formats are from Figure 1's caption on the
// sciencestack.ai page).  This file owns the device copies of the packed
// signs and the zero-padded scales, the workspace, and the choice between
// the decode kernels (batch <= 16) and the matrix-core kernels.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <limits>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "dbf.h"
#include "dbf_internal.h"

struct dbf_layer {
    int32_t n = 0, m = 0, k = 0;
    int32_t n_pad = 0, m_pad = 0, k_pad = 0;
    int32_t max_batch = 0;
    int32_t device = 0;
    int32_t Wk = 0, Wm = 0;  // words per row of A (along k) and of B (along m)
    uint32_t *A_dev = nullptr;
    uint32_t *B_dev = nullptr;
    uint16_t *a_dev = nullptr, *mid_dev = nullptr, *b_dev = nullptr;
    // workspace
    float *tpart = nullptr;   // matrix-core decode stage-1 partials [parts][16][k_pad]
    size_t tpart_cap = 0;     // floats
    int ntickets = 0;
    uint16_t *T = nullptr;    // prefill intermediate    [max_batch][k_pad] fp16
    unsigned *tickets = nullptr;  // per 64-row tile of A or 16-row block of B; zero between calls
    uint16_t *v16 = nullptr;      // matrix-core decode intermediate [2][16][k_pad] fp16
    // batch-1 decode (int8 matrix cores): A and B in the dbf_layout_signs_dec
    // layout (A: round_up(n, 16) rows along k_pad; B: k_pad rows along m) and
    // the fp32 intermediate v [k_pad]
    uint32_t *A_i8 = nullptr, *B_i8 = nullptr;
    float *v32 = nullptr;
    int32_t A_i8_rows = 0;
    bool i8_ok = false;           // m and k_pad within the batch-1 kernels' reduction limit
    float *split = nullptr;       // split-K parts of the prefill products (small grids)
    size_t split_cap = 0;         // floats
    // BQQ-form layer (dbf_bqq_pack): A, B hold 0/1 matrices, and the output
    // gains E[o] * Σx + γ·x (per-row sums in bqq_stats [max_batch][2])
    bool binary = false;
    float *bqq_E = nullptr, *bqq_gamma = nullptr, *bqq_stats = nullptr;
    // group-wise scalars (dbf_bqq_pack_grouped, more than one group): the
    // p products' first stage runs as p signed DBF products with per-term
    // input scales bqq_b [p][m_pad] (fp16); bqq_E holds [p][n] row sums of
    // the Y_i, bqq_gamma the [p + 1][m] weights of the row statistics and
    // bqq_stats [max_batch][p + 1] (bqq_Q = p + 1)
    int32_t bqq_groups = 0, bqq_p = 0, bqq_d = 0, bqq_Q = 2;
    uint16_t *bqq_b = nullptr;
    size_t packed_bytes = 0, scale_bytes = 0, workspace_bytes = 0;
    // backward (dbf_pack_ex with DBF_PACK_BACKWARD): the transposed layer
    // Wᵀ = diag(b) Bᵀ diag(mid) Aᵀ diag(a), and fp32 intermediates of the
    // scale gradients, [max_batch][width] each
    dbf_layer *bwd = nullptr;
    float *t32 = nullptr;     // (X ⊙ b) Bᵀ in fp32          [max_batch][k_pad]
    float *red = nullptr;     // batch-sum partials [ceil(max_batch / 64)][max(n, k_pad, m)]
    // kernel timing
    bool timing = false;
    struct Pending {
        std::string name;
        hipEvent_t start, stop;
    };
    std::vector<Pending> pending;
    std::vector<hipEvent_t> event_pool;
    std::map<std::string, std::pair<int64_t, double>> totals;
};

namespace {

int g_alloc_calls = 0;  // device allocations made by the current dbf_pack call

// Test hook: DBF_TEST_FAIL_ALLOC=N makes the N-th device allocation (1-based)
// of each dbf_pack call fail as if the device were out of memory.
bool injected_alloc_failure() {
    const char *env = std::getenv("DBF_TEST_FAIL_ALLOC");
    ++g_alloc_calls;
    if (!env) return false;
    return std::atoi(env) == g_alloc_calls;
}

dbf_status_t dev_alloc(void **p, size_t bytes) {
    *p = nullptr;
    if (injected_alloc_failure()) return DBF_ERR_OOM;
    hipError_t e = hipMalloc(p, bytes);
    if (e == hipErrorOutOfMemory) return DBF_ERR_OOM;
    if (e != hipSuccess) {
        *p = nullptr;
        return DBF_ERR_HIP;
    }
    return DBF_OK;
}

void release(dbf_layer *h) {
    if (!h) return;
    // (the transposed layer of a backward-capable handle is released with it)
    (void)hipFree(h->A_dev);
    (void)hipFree(h->B_dev);
    (void)hipFree(h->a_dev);
    (void)hipFree(h->mid_dev);
    (void)hipFree(h->b_dev);
    (void)hipFree(h->tpart);
    (void)hipFree(h->T);
    (void)hipFree(h->tickets);
    (void)hipFree(h->v16);
    (void)hipFree(h->A_i8);
    (void)hipFree(h->B_i8);
    (void)hipFree(h->v32);
    (void)hipFree(h->split);
    (void)hipFree(h->bqq_E);
    (void)hipFree(h->bqq_gamma);
    (void)hipFree(h->bqq_stats);
    (void)hipFree(h->bqq_b);
    (void)hipFree(h->t32);
    (void)hipFree(h->red);
    release(h->bwd);
    for (auto &p : h->pending) {
        (void)hipEventDestroy(p.start);
        (void)hipEventDestroy(p.stop);
    }
    for (auto e : h->event_pool) (void)hipEventDestroy(e);
    delete h;
}

int32_t round_up(int32_t v, int32_t q) { return (v + q - 1) / q * q; }

// Pack a +/-1 matrix (rows x cols) along cols and tile it for the device:
// `tiled` in the dbf_layout_signs layout and, when dec_rows > 0, `dec` in the
// dbf_layout_signs_dec layout (dec_rows x dec_cols, padded sizes).
dbf_status_t pack_tiled(const int8_t *S, int32_t rows, int32_t cols, int32_t words,
                        std::vector<uint32_t> &tiled, int32_t dec_rows, int32_t dec_cols,
                        std::vector<uint32_t> &dec) {
    std::vector<uint32_t> canon;
    try {
        canon.assign(static_cast<size_t>(rows) * words, 0u);
        tiled.assign(dbf_layout_words(rows, words), 0u);
        if (dec_rows > 0) dec.assign(dbf_layout_words_dec(dec_rows, dec_cols), 0u);
        else dec.clear();
    } catch (const std::bad_alloc &) {
        return DBF_ERR_OOM;
    }
    dbf_status_t st = dbf_pack_signs(S, rows, cols, canon.data(), words);
    if (st != DBF_OK) return st;
    st = dbf_layout_signs(canon.data(), rows, words, tiled.data());
    if (st != DBF_OK || dec_rows <= 0) return st;
    return dbf_layout_signs_dec(canon.data(), rows, cols, words, dec_rows, dec_cols, dec.data());
}

dbf_status_t upload(void *dst, const void *src, size_t bytes) {
    return hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice) == hipSuccess ? DBF_OK : DBF_ERR_HIP;
}

dbf_status_t upload_scales(uint16_t **dst, const uint16_t *src, int32_t len, int32_t len_pad) {
    std::vector<uint16_t> buf;
    try {
        buf.assign(static_cast<size_t>(len_pad), 0u);  // zero padding: the padded entries are +0.0
    } catch (const std::bad_alloc &) {
        return DBF_ERR_OOM;
    }
    std::memcpy(buf.data(), src, sizeof(uint16_t) * static_cast<size_t>(len));
    dbf_status_t st = dev_alloc(reinterpret_cast<void **>(dst), buf.size() * sizeof(uint16_t));
    if (st != DBF_OK) return st;
    return upload(*dst, buf.data(), buf.size() * sizeof(uint16_t));
}

}  // namespace

namespace dbf {
LaunchEvents &launch_events() {
    static thread_local LaunchEvents ev;
    return ev;
}
}  // namespace dbf

namespace {

hipEvent_t take_event(dbf_layer *h) {
    if (!h->event_pool.empty()) {
        hipEvent_t e = h->event_pool.back();
        h->event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Launch one kernel through `fn`; with timing on, a pair of events rides on
// the launch itself (see launch_kernel) and is kept for dbf_timing_read.
template <typename F>
dbf_status_t timed_launch(dbf_layer *h, const char *name, hipStream_t stream, F fn) {
    (void)stream;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (h->timing) {
        e0 = take_event(h);
        e1 = take_event(h);
        if (e0 && e1) dbf::launch_events() = {e0, e1};
    }
    const int err = fn();
    dbf::launch_events() = {};
    if (e0 && e1) {
        h->pending.push_back({name, e0, e1});
    } else {
        if (e0) h->event_pool.push_back(e0);
        if (e1) h->event_pool.push_back(e1);
    }
    return err == 0 ? DBF_OK : DBF_ERR_HIP;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The value of an fp16 bit pattern, exactly, as a double.
double half_bits_value(uint16_t h) {
    const int ex = (h >> 10) & 31, man = h & 1023;
    double v;
    if (ex == 0) v = std::ldexp(double(man), -24);
    else if (ex == 31) v = man ? std::numeric_limits<double>::quiet_NaN() : std::numeric_limits<double>::infinity();
    else v = std::ldexp(double(man + 1024), ex - 25);
    return (h & 0x8000) ? -v : v;
}

}  // namespace

extern "C" const char *dbf_status_string(dbf_status_t s) {
    switch (s) {
        case DBF_OK: return "success";
        case DBF_ERR_INVALID_ARG: return "invalid argument";
        case DBF_ERR_SHAPE: return "unsupported or overflowing shape";
        case DBF_ERR_OOM: return "out of memory";
        case DBF_ERR_HIP: return "HIP runtime error";
        case DBF_ERR_UNSUPPORTED: return "unsupported request";
    }
    return "unknown status";
}

// The layer handle for (A, B, a, mid, b); arguments are validated first.
static dbf_status_t pack_layer(int32_t n, int32_t m, int32_t k, const int8_t *A_signs, const int8_t *B_signs,
                               const uint16_t *a, const uint16_t *mid, const uint16_t *b, int32_t max_batch,
                               dbf_handle_t *out) {
    if (out) *out = nullptr;
    if (!out || !A_signs || !B_signs || !a || !mid || !b) return DBF_ERR_INVALID_ARG;
    if (n < 1 || m < 1 || k < 1 || max_batch < 1) return DBF_ERR_INVALID_ARG;
    // Padded sizes must stay inside int32 element counts for the kernels.
    const int64_t lim = int64_t(1) << 30;
    if (n > lim || m > lim || k > lim) return DBF_ERR_SHAPE;
    const int32_t n_pad = round_up(n, 64), m_pad = round_up(m, 64), k_pad = round_up(k, 64);
    if (int64_t(n_pad) * k_pad > (int64_t(1) << 40) || int64_t(k_pad) * m_pad > (int64_t(1) << 40) ||
        int64_t(max_batch) * k_pad > (int64_t(1) << 31) || int64_t(max_batch) * n > (int64_t(1) << 31) ||
        int64_t(max_batch) * m > (int64_t(1) << 31))
        return DBF_ERR_SHAPE;
    // Validate every sign before touching the device.
    for (int64_t i = 0; i < int64_t(n) * k; ++i)
        if (A_signs[i] != 1 && A_signs[i] != -1) return DBF_ERR_INVALID_ARG;
    for (int64_t i = 0; i < int64_t(k) * m; ++i)
        if (B_signs[i] != 1 && B_signs[i] != -1) return DBF_ERR_INVALID_ARG;

    dbf_layer *h = new (std::nothrow) dbf_layer();
    if (!h) return DBF_ERR_OOM;
    h->n = n;
    h->m = m;
    h->k = k;
    h->n_pad = n_pad;
    h->m_pad = m_pad;
    h->k_pad = k_pad;
    h->max_batch = max_batch;
    h->Wk = k_pad / 32;
    h->Wm = m_pad / 32;

    dbf_status_t st = DBF_OK;
    if (hipGetDevice(&h->device) != hipSuccess) st = DBF_ERR_HIP;

    // batch-1 decode layouts: reduction lengths (m, k_pad) padded to 128,
    // within the kernels' limit of kI8MaxSC superchunks of 512
    const int32_t m128 = dbf::round_up_int(m, 128), k128 = dbf::round_up_int(k_pad, 128);
    h->i8_ok = m128 <= 512 * dbf::kI8MaxSC && k128 <= 512 * dbf::kI8MaxSC;
    h->A_i8_rows = dbf::round_up_int(n, 16);
    std::vector<uint32_t> tiled, dec;
    if (st == DBF_OK) st = pack_tiled(A_signs, n, k, h->Wk, tiled, h->i8_ok ? h->A_i8_rows : 0, k128, dec);
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->A_dev), tiled.size() * 4);
    if (st == DBF_OK) st = upload(h->A_dev, tiled.data(), tiled.size() * 4);
    if (st == DBF_OK) h->packed_bytes += tiled.size() * 4;
    if (st == DBF_OK && h->i8_ok) st = dev_alloc(reinterpret_cast<void **>(&h->A_i8), dec.size() * 4);
    if (st == DBF_OK && h->i8_ok) st = upload(h->A_i8, dec.data(), dec.size() * 4);
    if (st == DBF_OK) h->packed_bytes += dec.size() * 4;
    if (st == DBF_OK) st = pack_tiled(B_signs, k, m, h->Wm, tiled, h->i8_ok ? k_pad : 0, m128, dec);
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->B_dev), tiled.size() * 4);
    if (st == DBF_OK) st = upload(h->B_dev, tiled.data(), tiled.size() * 4);
    if (st == DBF_OK) h->packed_bytes += tiled.size() * 4;
    if (st == DBF_OK && h->i8_ok) st = dev_alloc(reinterpret_cast<void **>(&h->B_i8), dec.size() * 4);
    if (st == DBF_OK && h->i8_ok) st = upload(h->B_i8, dec.data(), dec.size() * 4);
    if (st == DBF_OK) h->packed_bytes += dec.size() * 4;
    std::vector<uint32_t>().swap(tiled);
    std::vector<uint32_t>().swap(dec);
    if (st == DBF_OK) st = upload_scales(&h->a_dev, a, n, n_pad);
    if (st == DBF_OK) st = upload_scales(&h->mid_dev, mid, k, k_pad);
    if (st == DBF_OK) st = upload_scales(&h->b_dev, b, m, m_pad);
    if (st == DBF_OK) h->scale_bytes = 2 * size_t(n_pad + k_pad + m_pad);

    const int32_t dec_b = max_batch < dbf::kDecodeMaxBatch ? max_batch : dbf::kDecodeMaxBatch;
    size_t tpart_elems = 64;
    // stage-1 reduction parts of the matrix-core decode (wide m, batch >= 2)
    const int s1_parts = dbf::mfma_stage1_parts(m_pad, k_pad, dbf::kDecodeMaxBatch);
    if (s1_parts > 1) tpart_elems = std::max(tpart_elems, size_t(s1_parts) * dbf::kDecodeMaxBatch * k_pad);
    const size_t tpart_bytes = sizeof(float) * tpart_elems;
    const int ntickets = std::max(n_pad / 64, k_pad / 16);
    const size_t ticket_bytes = sizeof(unsigned) * size_t(ntickets);
    const size_t T_bytes = sizeof(uint16_t) * size_t(max_batch) * k_pad;
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->tpart), tpart_bytes);
    if (st == DBF_OK) h->tpart_cap = tpart_elems;
    h->ntickets = ntickets;
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->T), T_bytes);
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->tickets), ticket_bytes);
    if (st == DBF_OK && hipMemset(h->tickets, 0, ticket_bytes) != hipSuccess) st = DBF_ERR_HIP;
    if (st == DBF_OK && hipDeviceSynchronize() != hipSuccess) st = DBF_ERR_HIP;
    const size_t v16_bytes = sizeof(uint16_t) * 2 * size_t(dec_b) * k_pad;
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->v16), v16_bytes);
    // v of the batch-1..4 int8 decode, one row of k_pad per batch row
    const size_t v32_bytes = sizeof(float) * size_t(std::min(max_batch, dbf::kI8MaxRows)) * k_pad;
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->v32), v32_bytes);
    // split-K parts: the most that either prefill product takes at any batch
    // <= max_batch (the part count depends on the batch through its 128-row
    // tiles only, so the largest batch of each tile count is the worst case)
    size_t split_elems = 64;
    for (int32_t mb = 1; st == DBF_OK; mb += 128) {
        const int32_t M = std::min(max_batch, mb + 127);
        split_elems = std::max(split_elems, dbf::sign_gemm_split_elems(M, m, h->Wm, k_pad));
        split_elems = std::max(split_elems, dbf::sign_gemm_split_elems(M, k_pad, h->Wk, n));
        if (M >= max_batch) break;
    }
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->split), sizeof(float) * split_elems);
    if (st == DBF_OK) h->split_cap = split_elems;
    if (st == DBF_OK)
        h->workspace_bytes =
            tpart_bytes + T_bytes + ticket_bytes + v16_bytes + v32_bytes + sizeof(float) * split_elems;

    if (st != DBF_OK) {
        release(h);
        return st;
    }
    *out = h;
    return DBF_OK;
}

extern "C" dbf_status_t dbf_pack(int32_t n, int32_t m, int32_t k, const int8_t *A_signs, const int8_t *B_signs,
                                 const uint16_t *a, const uint16_t *mid, const uint16_t *b, int32_t max_batch,
                                 dbf_handle_t *out) {
    return dbf_pack_ex(n, m, k, A_signs, B_signs, a, mid, b, max_batch, 0, out);
}

extern "C" dbf_status_t dbf_pack_ex(int32_t n, int32_t m, int32_t k, const int8_t *A_signs, const int8_t *B_signs,
                                    const uint16_t *a, const uint16_t *mid, const uint16_t *b, int32_t max_batch,
                                    int32_t flags, dbf_handle_t *out) {
    if (out) *out = nullptr;
    if (!out || (flags & ~DBF_PACK_BACKWARD) != 0) return DBF_ERR_INVALID_ARG;
    g_alloc_calls = 0;
    dbf_layer *h = nullptr;
    dbf_status_t st = pack_layer(n, m, k, A_signs, B_signs, a, mid, b, max_batch, &h);
    if (st != DBF_OK || !(flags & DBF_PACK_BACKWARD)) {
        *out = h;
        return st;
    }
    // transposed signs on the host: Aᵀ (k x n) and Bᵀ (m x k)
    std::vector<int8_t> At, Bt;
    try {
        At.resize(static_cast<size_t>(k) * n);
        Bt.resize(static_cast<size_t>(m) * k);
    } catch (const std::bad_alloc &) {
        release(h);
        return DBF_ERR_OOM;
    }
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < k; ++j) At[j * n + i] = A_signs[i * k + j];
    for (int64_t j = 0; j < k; ++j)
        for (int64_t l = 0; l < m; ++l) Bt[l * k + j] = B_signs[j * m + l];
    st = pack_layer(m, n, k, Bt.data(), At.data(), b, mid, a, max_batch, &h->bwd);
    std::vector<int8_t>().swap(At);
    std::vector<int8_t>().swap(Bt);
    const size_t mb = static_cast<size_t>(max_batch);
    const size_t wmax = static_cast<size_t>(std::max({h->n, h->k_pad, h->m}));
    const size_t nchunk = (mb + dbf::kColChunk - 1) / dbf::kColChunk;
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->t32), 4 * mb * h->k_pad);
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->red), 4 * nchunk * wmax);
    if (st != DBF_OK) {
        release(h);
        return st;
    }
    h->workspace_bytes += 4 * mb * size_t(h->k_pad) + 4 * nchunk * wmax;
    h->packed_bytes += h->bwd->packed_bytes;
    *out = h;
    return DBF_OK;
}

extern "C" dbf_status_t dbf_bqq_pack(int32_t n, int32_t m, int32_t d, int32_t p, const uint8_t *Y,
                                     const uint8_t *Z, const uint16_t *r, const uint16_t *s, const uint16_t *t,
                                     uint16_t u, int32_t max_batch, dbf_handle_t *out) {
    if (out) *out = nullptr;
    if (!out || !Y || !Z || !r || !s || !t) return DBF_ERR_INVALID_ARG;
    if (n < 1 || m < 1 || d < 1 || p < 1 || max_batch < 1) return DBF_ERR_INVALID_ARG;
    const int64_t k = int64_t(p) * d;
    if (k > (int64_t(1) << 30)) return DBF_ERR_SHAPE;
    for (int64_t i = 0; i < int64_t(p) * n * d; ++i)
        if (Y[i] > 1) return DBF_ERR_INVALID_ARG;
    for (int64_t i = 0; i < int64_t(p) * d * m; ++i)
        if (Z[i] > 1) return DBF_ERR_INVALID_ARG;
    g_alloc_calls = 0;
    // The p products as one: Y_0 .. Y_{p-1} side by side (n x p d), Z_i
    // stacked (p d x m), in the packed-sign encoding (bit 1 <-> entry 1,
    // passed as -1).  Both products expand to {0, 2}: mid = r_i and
    // a = 1/4 undo the two factors of 2; b = 1.
    std::vector<int8_t> As, Bs;
    std::vector<uint16_t> a16, mid16, b16;
    std::vector<double> E(static_cast<size_t>(n)), gamma(static_cast<size_t>(m), 0.0);
    try {
        As.resize(static_cast<size_t>(n) * k);
        Bs.resize(static_cast<size_t>(k) * m);
        a16.assign(static_cast<size_t>(n), 0x3400);  // fp16 0.25
        b16.assign(static_cast<size_t>(m), 0x3C00);  // fp16 1.0
        mid16.resize(static_cast<size_t>(k));
    } catch (const std::bad_alloc &) {
        return DBF_ERR_OOM;
    }
    const double uu = half_bits_value(u);
    for (int64_t o = 0; o < n; ++o) E[o] = uu;
    for (int64_t i = 0; i < p; ++i) {
        const double si = half_bits_value(s[i]), ti = half_bits_value(t[i]);
        for (int64_t j = 0; j < d; ++j) mid16[i * d + j] = r[i];
        for (int64_t o = 0; o < n; ++o) {
            const uint8_t *yrow = Y + (i * n + o) * d;
            int64_t deg = 0;
            for (int64_t j = 0; j < d; ++j) {
                As[o * k + i * d + j] = yrow[j] ? -1 : 1;
                deg += yrow[j];
            }
            E[o] += si * double(deg);
        }
        for (int64_t j = 0; j < d; ++j) {
            const uint8_t *zrow = Z + (i * d + j) * m;
            int8_t *brow = Bs.data() + (i * d + j) * m;
            for (int64_t l = 0; l < m; ++l) {
                brow[l] = zrow[l] ? -1 : 1;
                gamma[l] += ti * double(zrow[l]);
            }
        }
    }
    dbf_layer *h = nullptr;
    dbf_status_t st = pack_layer(n, m, static_cast<int32_t>(k), As.data(), Bs.data(), a16.data(), mid16.data(),
                                 b16.data(), max_batch, &h);
    if (st != DBF_OK) return st;
    std::vector<int8_t>().swap(As);
    std::vector<int8_t>().swap(Bs);
    h->binary = true;
    std::vector<float> E32(E.begin(), E.end()), g32(gamma.begin(), gamma.end());
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->bqq_E), sizeof(float) * E32.size());
    if (st == DBF_OK) st = upload(h->bqq_E, E32.data(), sizeof(float) * E32.size());
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->bqq_gamma), sizeof(float) * g32.size());
    if (st == DBF_OK) st = upload(h->bqq_gamma, g32.data(), sizeof(float) * g32.size());
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->bqq_stats), sizeof(float) * 2 * size_t(max_batch));
    if (st == DBF_OK) {
        h->scale_bytes += sizeof(float) * (E32.size() + g32.size());
        h->workspace_bytes += sizeof(float) * 2 * size_t(max_batch);
    }
    if (st != DBF_OK) {
        release(h);
        return st;
    }
    *out = h;
    return DBF_OK;
}

// Group-wise scalars: on the columns l of group h = l / group,
//   W[:, l] = Σ_i ( r_i[h] Y_i Z_i + s_i[h] Y_i 1 + t_i[h] 1 Z_i )[:, l] + u[h].
// With S_i = 1 - 2 Z_i (entries ±1) and b_i[l] = r_i[h(l)],
//   Σ_l (Y_i Z_i)[o, l] r_i[h(l)] x_l = ½ R_i[o] β_i - ½ (Y_i t_i)[o],
// t_i = S_i (b_i ⊙ x) the signed DBF first stage of term i, β_i = b_i·x and
// R_i[o] = Σ_j Y_i[o, j].  So the first stage is p signed products (the DBF
// kernels, per-term b, mid = 1), the second is the 0/1 product of the Y_i
// ({0, 2} operand, a = -1/4), and the rest is the rank-(p + 1) term
//   Σ_i R_i[o] σ_i + κ,  σ_i = Σ_l (s_i[h(l)] + ½ r_i[h(l)]) x_l,
//   κ = Σ_l ( Σ_i t_i[h(l)] C_i[l] + u[h(l)] ) x_l,  C_i[l] = Σ_j Z_i[j, l],
// with the weights formed in double precision and kept in fp32.
extern "C" dbf_status_t dbf_bqq_pack_grouped(int32_t n, int32_t m, int32_t d, int32_t p, int32_t group,
                                             const uint8_t *Y, const uint8_t *Z, const uint16_t *r,
                                             const uint16_t *s, const uint16_t *t, const uint16_t *u,
                                             int32_t max_batch, dbf_handle_t *out) {
    if (out) *out = nullptr;
    if (!out || !Y || !Z || !r || !s || !t || !u) return DBF_ERR_INVALID_ARG;
    if (n < 1 || m < 1 || d < 1 || p < 1 || group < 1 || max_batch < 1) return DBF_ERR_INVALID_ARG;
    const int32_t ng = static_cast<int32_t>((int64_t(m) + group - 1) / group);
    if (ng == 1) return dbf_bqq_pack(n, m, d, p, Y, Z, r, s, t, u[0], max_batch, out);
    // term boundaries on 64-row tiles of the sign layouts; p + 1 statistics per row
    if (d % 64 != 0 || p + 1 > dbf::kMaxStatQ || p > dbf::kMaxGroup) return DBF_ERR_SHAPE;
    const int64_t k = int64_t(p) * d;
    if (k > (int64_t(1) << 30)) return DBF_ERR_SHAPE;
    for (int64_t i = 0; i < int64_t(p) * n * d; ++i)
        if (Y[i] > 1) return DBF_ERR_INVALID_ARG;
    for (int64_t i = 0; i < int64_t(p) * d * m; ++i)
        if (Z[i] > 1) return DBF_ERR_INVALID_ARG;
    g_alloc_calls = 0;
    const int32_t Q = p + 1;
    const int32_t m_pad = round_up(m, 64);
    std::vector<int8_t> As, Bs;
    std::vector<uint16_t> a16, mid16, b16, bt16;
    std::vector<float> E32, w32;
    try {
        As.resize(static_cast<size_t>(n) * k);
        Bs.resize(static_cast<size_t>(k) * m);
        a16.assign(static_cast<size_t>(n), 0xB400);  // fp16 -0.25
        mid16.assign(static_cast<size_t>(k), 0x3C00);
        b16.assign(static_cast<size_t>(m), 0x3C00);  // (the per-term scales below serve instead)
        bt16.assign(static_cast<size_t>(p) * m_pad, 0);
        E32.assign(static_cast<size_t>(p) * n, 0.0f);
        w32.assign(static_cast<size_t>(Q) * m, 0.0f);
    } catch (const std::bad_alloc &) {
        return DBF_ERR_OOM;
    }
    std::vector<double> kappa(static_cast<size_t>(m), 0.0);
    for (int64_t l = 0; l < m; ++l) kappa[l] = half_bits_value(u[l / group]);
    for (int64_t i = 0; i < p; ++i) {
        for (int64_t o = 0; o < n; ++o) {
            const uint8_t *yrow = Y + (i * n + o) * d;
            int64_t deg = 0;
            for (int64_t j = 0; j < d; ++j) {
                As[o * k + i * d + j] = yrow[j] ? -1 : 1;
                deg += yrow[j];
            }
            E32[i * n + o] = static_cast<float>(deg);
        }
        std::vector<int64_t> colsum(static_cast<size_t>(m), 0);
        for (int64_t j = 0; j < d; ++j) {
            const uint8_t *zrow = Z + (i * d + j) * m;
            int8_t *brow = Bs.data() + (i * d + j) * m;
            for (int64_t l = 0; l < m; ++l) {
                brow[l] = zrow[l] ? -1 : 1;
                colsum[l] += zrow[l];
            }
        }
        for (int64_t l = 0; l < m; ++l) {
            const int64_t hg = l / group;
            const double ri = half_bits_value(r[i * ng + hg]), si = half_bits_value(s[i * ng + hg]),
                         ti = half_bits_value(t[i * ng + hg]);
            bt16[i * m_pad + l] = r[i * ng + hg];
            w32[i * m + l] = static_cast<float>(si + 0.5 * ri);
            kappa[l] += ti * double(colsum[l]);
        }
    }
    for (int64_t l = 0; l < m; ++l) w32[int64_t(p) * m + l] = static_cast<float>(kappa[l]);
    dbf_layer *h = nullptr;
    dbf_status_t st = pack_layer(n, m, static_cast<int32_t>(k), As.data(), Bs.data(), a16.data(), mid16.data(),
                                 b16.data(), max_batch, &h);
    if (st != DBF_OK) return st;
    std::vector<int8_t>().swap(As);
    std::vector<int8_t>().swap(Bs);
    h->binary = true;
    h->bqq_groups = ng;
    h->bqq_p = p;
    h->bqq_d = d;
    h->bqq_Q = Q;
    // split-K workspace for the per-term first products (n_out = d)
    size_t split_elems = h->split_cap;
    for (int32_t mb = 1;; mb += 128) {
        const int32_t M = std::min(max_batch, mb + 127);
        split_elems = std::max(split_elems, dbf::sign_gemm_split_elems(M, m, h->Wm, d));
        if (M >= max_batch) break;
    }
    if (split_elems > h->split_cap) {
        (void)hipFree(h->split);
        h->split = nullptr;
        st = dev_alloc(reinterpret_cast<void **>(&h->split), sizeof(float) * split_elems);
        if (st == DBF_OK) {
            h->workspace_bytes += sizeof(float) * (split_elems - h->split_cap);
            h->split_cap = split_elems;
        }
    }
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->bqq_E), sizeof(float) * E32.size());
    if (st == DBF_OK) st = upload(h->bqq_E, E32.data(), sizeof(float) * E32.size());
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->bqq_gamma), sizeof(float) * w32.size());
    if (st == DBF_OK) st = upload(h->bqq_gamma, w32.data(), sizeof(float) * w32.size());
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->bqq_b), sizeof(uint16_t) * bt16.size());
    if (st == DBF_OK) st = upload(h->bqq_b, bt16.data(), sizeof(uint16_t) * bt16.size());
    if (st == DBF_OK) st = dev_alloc(reinterpret_cast<void **>(&h->bqq_stats), sizeof(float) * Q * size_t(max_batch));
    if (st == DBF_OK) {
        h->scale_bytes += sizeof(float) * (E32.size() + w32.size()) + sizeof(uint16_t) * bt16.size();
        h->workspace_bytes += sizeof(float) * Q * size_t(max_batch);
    }
    if (st != DBF_OK) {
        release(h);
        return st;
    }
    *out = h;
    return DBF_OK;
}

extern "C" void dbf_free(dbf_handle_t h) {
    if (!h) return;
    int cur = 0;
    if (hipGetDevice(&cur) == hipSuccess && cur != h->device) {
        (void)hipSetDevice(h->device);
        (void)hipDeviceSynchronize();
        (void)hipSetDevice(cur);
    } else {
        (void)hipDeviceSynchronize();
    }
    release(h);
}

extern "C" dbf_status_t dbf_get_info(dbf_handle_t h, dbf_info_t *info) {
    if (!h || !info) return DBF_ERR_INVALID_ARG;
    info->n = h->n;
    info->m = h->m;
    info->k = h->k;
    info->n_pad = h->n_pad;
    info->m_pad = h->m_pad;
    info->k_pad = h->k_pad;
    info->max_batch = h->max_batch;
    info->device = h->device;
    info->packed_bytes = h->packed_bytes;
    info->scale_bytes = h->scale_bytes;
    info->workspace_bytes = h->workspace_bytes;
    return DBF_OK;
}

// The stage descriptions of one layer for the batch-1 decode kernels.
static void i8_stages(const dbf_layer *h, const void *x, void *y, dbf::I8Layer &s1, dbf::I8Layer &s2) {
    const int m128 = dbf::round_up_int(h->m, 128), k128 = dbf::round_up_int(h->k_pad, 128);
    s1 = dbf::I8Layer{};
    s1.S = h->B_i8;
    s1.vec = x;
    s1.bsc = reinterpret_cast<const __half *>(h->b_dev);
    s1.osc = reinterpret_cast<const __half *>(h->mid_dev);
    s1.out = h->v32;
    s1.rows = h->k_pad;
    s1.K = h->m;
    s1.SC = dbf::i8_superchunks(h->m);
    s1.wlast = (m128 - 512 * (s1.SC - 1)) / 128;
    s1.ntiles = h->k_pad / 16;
    s2 = dbf::I8Layer{};
    s2.S = h->A_i8;
    s2.vec = h->v32;
    s2.osc = reinterpret_cast<const __half *>(h->a_dev);
    s2.out = y;
    s2.rows = h->n;
    s2.K = h->k_pad;
    s2.SC = dbf::i8_superchunks(h->k_pad);
    s2.wlast = (k128 - 512 * (s2.SC - 1)) / 128;
    s2.ntiles = h->A_i8_rows / 16;
    if (h->binary) {
        s2.aff_E = h->bqq_E;
        s2.aff_stats = h->bqq_stats;
    }
}

// Whether the int8 matrix-core kernels can run a forward at this batch:
// batch 1 wherever the layouts exist (m and k_pad within the kernels'
// reduction limit; the default path there); batch 2..4 for signed layers
// whose reductions have at most kI8RowsMaxSC superchunks (m and k_pad up to
// 8192), so that the batch's digit planes fit LDS (DBF_PATH_DECODE_EXACT).
// Each batch row is summed exactly with its own exponent, so its result is
// bit-identical to its batch-1 forward.
static bool i8_rows_ok(const dbf_layer *h, int32_t batch) {
    if (!h->i8_ok || batch < 1 || batch > dbf::kI8MaxRows) return false;
    if (batch == 1) return true;
    return !h->binary && h->bqq_groups == 0 && dbf::i8_superchunks(h->m) <= dbf::kI8RowsMaxSC &&
           dbf::i8_superchunks(h->k_pad) <= dbf::kI8RowsMaxSC;
}

// Batch 1..4: two launches of the int8 matrix-core kernels (decode_i8.hip).
static dbf_status_t forward_decode_i8(dbf_layer *h, const void *x, void *y, int32_t batch, hipStream_t stream) {
    dbf::I8Args a1{}, a2{};
    a1.count = a2.count = 1;
    a1.nrows = a2.nrows = batch;
    i8_stages(h, x, y, a1.L[0], a2.L[0]);
    if (h->binary) {
        a1.stat_x = static_cast<const __half *>(x);
        a1.stat_m = h->m;
        a1.gamma = h->bqq_gamma;
        a1.stats = h->bqq_stats;
        a1.stat_wg = 0;
    }
    dbf_status_t st =
        timed_launch(h, "decode_stage1", stream, [&] { return dbf::launch_decode_i8(a1, 1, h->binary, stream); });
    if (st != DBF_OK) return st;
    return timed_launch(h, "decode_stage2", stream, [&] { return dbf::launch_decode_i8(a2, 2, h->binary, stream); });
}

static dbf_status_t forward_decode_mfma(dbf_layer *h, const void *x, void *y, int32_t batch,
                                        hipStream_t stream) {
    if (batch == 1 && h->i8_ok) return forward_decode_i8(h, x, y, 1, stream);
    dbf::MfmaDecodeArgs d{};
    d.A_dev = h->A_dev;
    d.B_dev = h->B_dev;
    d.a_dev = h->a_dev;
    d.mid_dev = h->mid_dev;
    d.b_dev = h->b_dev;
    d.x = x;
    d.y = y;
    d.v16 = h->v16;
    d.batch = batch;
    d.n = h->n;
    d.m = h->m;
    d.n_pad = h->n_pad;
    d.m_pad = h->m_pad;
    d.k_pad = h->k_pad;
    d.binary = h->binary ? 1 : 0;
    d.aff_E = h->bqq_E;
    d.aff_stats = h->bqq_stats;
    d.gamma = h->bqq_gamma;       // (0/1 layers: stage 1 forms the row sums)
    d.stats_out = h->bqq_stats;
    d.s1_part = h->tpart;
    d.s1_part_cap = h->tpart_cap;
    d.s1_tickets = h->tickets;
    d.s1_ntickets = h->ntickets;
    dbf_status_t st = timed_launch(h, "decode_stage1", stream, [&] { return dbf::launch_mfma_decode(d, stream, 1); });
    if (st != DBF_OK) return st;
    return timed_launch(h, "decode_stage2", stream, [&] { return dbf::launch_mfma_decode(d, stream, 2); });
}

static dbf_status_t forward_prefill(dbf_layer *h, const void *x, void *y, int32_t batch, hipStream_t stream) {
    // T = rne16(mid ⊙ (X (B ⊙ b)ᵀ)), all k_pad columns (padded ones are 0).
    // (BQQ-form layers: 0/1 matrices, b = 1 so no per-K scale, and the
    // affine term in the second product's epilogue)
    dbf::SplitK sp;
    sp.ws = h->split;
    sp.cap = h->split_cap;
    dbf::GemmFlavor f1, f2;
    f1.binary = f2.binary = h->binary ? 1 : 0;
    f2.aff_E = h->bqq_E;
    f2.aff_stats = h->bqq_stats;
    const void *sk = h->binary ? nullptr : h->b_dev;
    dbf_status_t st = timed_launch(h, "prefill_gemm1", stream, [&] {
        return dbf::launch_sign_gemm(x, h->m, batch, h->m, h->B_dev, h->Wm, h->k_pad, sk, h->mid_dev, h->T,
                                     h->k_pad, h->k_pad, nullptr, 0, nullptr, 0, 0, nullptr, stream, &sp, &f1);
    });
    if (st == DBF_OK && sp.nsplit > 1)
        st = timed_launch(h, "prefill_split1", stream, [&] {
            return dbf::launch_split_finish(sp, batch, h->k_pad, h->mid_dev, h->T, h->k_pad, stream);
        });
    if (st != DBF_OK) return st;
    // Y = rne16(a ⊙ (T Aᵀ)).
    st = timed_launch(h, "prefill_gemm2", stream, [&] {
        return dbf::launch_sign_gemm(h->T, h->k_pad, batch, h->k_pad, h->A_dev, h->Wk, h->n_pad, nullptr,
                                     h->a_dev, y, h->n, h->n, nullptr, 0, nullptr, 0, 0, nullptr, stream, &sp, &f2);
    });
    if (st == DBF_OK && sp.nsplit > 1)
        st = timed_launch(h, "prefill_split2", stream, [&] {
            return dbf::launch_split_finish(sp, batch, h->n, h->a_dev, y, h->n, stream, h->bqq_E, h->bqq_stats);
        });
    return st;
}

// Forward of a layer with group-wise BQQ scalars (see dbf_bqq_pack_grouped):
// the row statistics, then the p signed first products (per-term input
// scales) into v / T, then the 0/1 second product with the rank-(p + 1)
// affine term.  Batch 1 runs the int8 decode kernels (the p first products
// as one launch of p layers); other batches run the prefill products.
static dbf_status_t forward_bqq_grouped(dbf_layer *h, const void *x, void *y, int32_t batch, int32_t path,
                                        hipStream_t stream) {
    const int p = h->bqq_p, d = h->bqq_d;
    const bool i8 = path != DBF_PATH_PREFILL && batch == 1 && h->i8_ok;
    if (path == DBF_PATH_DECODE && !i8) return DBF_ERR_UNSUPPORTED;
    // the row statistics: a row of the batch-1 stage-1 launch where the grid
    // has one to spare, else a kernel of their own
    const bool fused_stats = i8 && p < dbf::kMaxGroup;
    dbf_status_t st = DBF_OK;
    if (!fused_stats)
        st = timed_launch(h, "bqq_rowstats", stream, [&] {
            return dbf::launch_bqq_rowstats_q(x, batch, h->m, h->bqq_gamma, h->bqq_Q, h->bqq_stats, stream);
        });
    if (st != DBF_OK) return st;
    if (i8) {
        dbf::I8Args a1{}, a2{};
        dbf::I8Layer s1, s2;
        i8_stages(h, x, y, s1, s2);
        const size_t tile_words = static_cast<size_t>(256 * (s1.SC - 1) + 64 * s1.wlast);
        a1.count = p;
        for (int i = 0; i < p; ++i) {
            dbf::I8Layer L = s1;
            L.S = h->B_i8 + static_cast<size_t>(i) * (d / 16) * tile_words;
            L.bsc = reinterpret_cast<const __half *>(h->bqq_b + static_cast<size_t>(i) * h->m_pad);
            L.osc = reinterpret_cast<const __half *>(h->mid_dev + static_cast<size_t>(i) * d);
            L.out = h->v32 + static_cast<size_t>(i) * d;
            L.rows = d;
            L.ntiles = d / 16;
            a1.L[i] = L;
        }
        if (fused_stats) {
            a1.stat_x = static_cast<const __half *>(x);
            a1.stat_m = h->m;
            a1.stat_w = h->bqq_gamma;
            a1.stat_Q = h->bqq_Q;
            a1.stats = h->bqq_stats;
            a1.stat_wg = 0;
        }
        a2.count = 1;
        a2.L[0] = s2;
        a2.aff_Q = h->bqq_Q;
        st = timed_launch(h, "decode_stage1", stream, [&] { return dbf::launch_decode_i8(a1, 1, false, stream); });
        if (st != DBF_OK) return st;
        return timed_launch(h, "decode_stage2", stream, [&] { return dbf::launch_decode_i8(a2, 2, true, stream); });
    }
    dbf::SplitK sp;
    sp.ws = h->split;
    sp.cap = h->split_cap;
    if (d % 256 == 0 && h->m % 64 == 0) {
        // the p products share x: one product over all p d rows of B (the
        // terms' rows are consecutive), each 256-column output tile taking
        // its term's input scale b_i; T = rne16(S (b_term ⊙ x)) (mid = 1)
        dbf::GemmFlavor f1;
        f1.sk_cols = d;
        f1.sk_stride = h->m_pad;
        st = timed_launch(h, "prefill_gemm1", stream, [&] {
            return dbf::launch_sign_gemm(x, h->m, batch, h->m, h->B_dev, h->Wm, p * d, h->bqq_b, h->mid_dev, h->T,
                                         h->k_pad, p * d, nullptr, 0, nullptr, 0, 0, nullptr, stream, &sp, &f1);
        });
        if (st == DBF_OK && sp.nsplit > 1)
            st = timed_launch(h, "prefill_split1", stream, [&] {
                return dbf::launch_split_finish(sp, batch, p * d, h->mid_dev, h->T, h->k_pad, stream);
            });
    }
    for (int i = 0; i < p && st == DBF_OK && !(d % 256 == 0 && h->m % 64 == 0); ++i) {
        // T[:, i d : (i + 1) d] = rne16(S_i (b_i ⊙ x)) (mid = 1); B's rows of term i from its 64-row tile i d / 64
        const uint32_t *S = h->B_dev + static_cast<size_t>(i) * (d / 64) * (h->Wm >> 1) * 128;
        const uint16_t *bi = h->bqq_b + static_cast<size_t>(i) * h->m_pad;
        const uint16_t *midi = h->mid_dev + static_cast<size_t>(i) * d;
        uint16_t *Ti = h->T + static_cast<size_t>(i) * d;
        st = timed_launch(h, "prefill_gemm1", stream, [&] {
            return dbf::launch_sign_gemm(x, h->m, batch, h->m, S, h->Wm, d, bi, midi, Ti, h->k_pad, d, nullptr, 0,
                                         nullptr, 0, 0, nullptr, stream, &sp, nullptr);
        });
        if (st == DBF_OK && sp.nsplit > 1)
            st = timed_launch(h, "prefill_split1", stream, [&] {
                return dbf::launch_split_finish(sp, batch, d, midi, Ti, h->k_pad, stream);
            });
    }
    if (st != DBF_OK) return st;
    dbf::GemmFlavor f2;
    f2.binary = 1;
    f2.aff_E = h->bqq_E;
    f2.aff_stats = h->bqq_stats;
    f2.aff_Q = h->bqq_Q;
    f2.aff_ldE = h->n;
    st = timed_launch(h, "prefill_gemm2", stream, [&] {
        return dbf::launch_sign_gemm(h->T, h->k_pad, batch, h->k_pad, h->A_dev, h->Wk, h->n_pad, nullptr, h->a_dev,
                                     y, h->n, h->n, nullptr, 0, nullptr, 0, 0, nullptr, stream, &sp, &f2);
    });
    if (st == DBF_OK && sp.nsplit > 1)
        st = timed_launch(h, "prefill_split2", stream, [&] {
            return dbf::launch_split_finish(sp, batch, h->n, h->a_dev, y, h->n, stream, h->bqq_E, h->bqq_stats,
                                            h->bqq_Q, h->n);
        });
    return st;
}

extern "C" dbf_status_t dbf_linear_forward_ex(dbf_handle_t h, const void *x, void *y, int32_t batch, int32_t path,
                                              hipStream_t stream) {
    if (!h) return DBF_ERR_INVALID_ARG;
    if (batch < 0 || batch > h->max_batch) return DBF_ERR_INVALID_ARG;
    if (path != DBF_PATH_AUTO && path != DBF_PATH_DECODE && path != DBF_PATH_PREFILL &&
        path != DBF_PATH_DECODE_TABLE && path != DBF_PATH_DECODE_EXACT)
        return DBF_ERR_INVALID_ARG;
    if (path == DBF_PATH_DECODE && batch > dbf::kDecodeMaxBatch) return DBF_ERR_INVALID_ARG;
    if (path == DBF_PATH_DECODE_EXACT && batch > dbf::kI8MaxRows) return DBF_ERR_INVALID_ARG;
    if (batch == 0) return DBF_OK;
    if (!x || !y || !aligned16(x) || !aligned16(y)) return DBF_ERR_INVALID_ARG;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return DBF_ERR_HIP;
    if (cur != h->device) return DBF_ERR_INVALID_ARG;
    if (path == DBF_PATH_DECODE_TABLE) return DBF_ERR_UNSUPPORTED;  // (removed: slower than the matrix cores)
    if (path == DBF_PATH_DECODE_EXACT) {
        // the exact int8 sums at batch 1..4, every row the bits of its batch-1 forward
        if (!i8_rows_ok(h, batch) || h->binary || h->bqq_groups > 0) return DBF_ERR_UNSUPPORTED;
        return forward_decode_i8(h, x, y, batch, stream);
    }
    if (h->bqq_groups > 0)
        return forward_bqq_grouped(h, x, y, batch, path, stream);
    const bool decode = path == DBF_PATH_DECODE || (path == DBF_PATH_AUTO && batch <= dbf::kDecodeMaxBatch);
    if (h->binary && !decode) {
        // (on the decode path the stage-1 launch forms the row sums itself)
        const dbf_status_t st = timed_launch(h, "bqq_rowstats", stream, [&] {
            return dbf::launch_bqq_rowstats(x, batch, h->m, h->bqq_gamma, h->bqq_stats, stream);
        });
        if (st != DBF_OK) return st;
    }
    return decode ? forward_decode_mfma(h, x, y, batch, stream) : forward_prefill(h, x, y, batch, stream);
}

extern "C" dbf_status_t dbf_linear_forward_group(const dbf_handle_t *hs, int32_t count, const void *x, void *const *ys,
                                                 int32_t batch, hipStream_t stream) {
    if (!hs || !ys || count < 1 || count > dbf::kMaxGroup || batch < 0) return DBF_ERR_INVALID_ARG;
    for (int i = 0; i < count; ++i) {
        if (!hs[i]) return DBF_ERR_INVALID_ARG;
        if (hs[i]->m != hs[0]->m || hs[i]->device != hs[0]->device || batch > hs[i]->max_batch)
            return DBF_ERR_INVALID_ARG;
        if (hs[i]->binary) return DBF_ERR_UNSUPPORTED;
    }
    if (batch == 0) return DBF_OK;
    if (!x || !aligned16(x)) return DBF_ERR_INVALID_ARG;
    for (int i = 0; i < count; ++i)
        if (!ys[i] || !aligned16(ys[i])) return DBF_ERR_INVALID_ARG;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return DBF_ERR_HIP;
    if (cur != hs[0]->device) return DBF_ERR_INVALID_ARG;
    if (batch > dbf::kDecodeMaxBatch) {
        // one launch per product for all the layers (their tiles in one
        // grid), where every product has the deep-pipelined form (m a
        // multiple of 64); otherwise each layer's own forward
        bool grouped = count > 1 && hs[0]->m % 64 == 0;
        dbf::GemmGroup g1{}, g2{};
        g1.count = g2.count = count;
        g1.M = g2.M = batch;
        for (int i = 0; i < count; ++i) {
            const dbf_layer *h = hs[i];
            dbf::GemmItem &a = g1.item[i];
            a.P = x, a.ldp = h->m, a.K = h->m, a.S = h->B_dev, a.words = h->Wm, a.n_rows_pad = h->k_pad;
            a.sk = h->b_dev, a.sn = h->mid_dev, a.out = h->T, a.ldo = h->k_pad, a.n_out = h->k_pad;
            dbf::GemmItem &c = g2.item[i];
            c.P = h->T, c.ldp = h->k_pad, c.K = h->k_pad, c.S = h->A_dev, c.words = h->Wk, c.n_rows_pad = h->n_pad;
            c.sk = nullptr, c.sn = h->a_dev, c.out = ys[i], c.ldo = h->n, c.n_out = h->n;
            grouped = grouped && h->Wm * 32 == h->m && h->Wk * 32 == h->k_pad;
        }
        if (!grouped) {
            for (int i = 0; i < count; ++i) {
                const dbf_status_t st = forward_prefill(hs[i], x, ys[i], batch, stream);
                if (st != DBF_OK) return st;
            }
            return DBF_OK;
        }
        dbf_layer *t = hs[0];  // kernel timing follows the first handle
        dbf_status_t st = timed_launch(t, "prefill_group_gemm1", stream,
                                       [&] { return dbf::launch_sign_gemm_group(g1, stream); });
        if (st != DBF_OK) return st;
        return timed_launch(t, "prefill_group_gemm2", stream, [&] { return dbf::launch_sign_gemm_group(g2, stream); });
    }
    if (batch == 1) {
        int nok = 0;
        for (int i = 0; i < count; ++i) nok += hs[i]->i8_ok ? 1 : 0;
        if (nok > 0 && nok < count) {
            // some layers on the int8 kernels, some not: each layer's own
            // forward, so every output keeps the bits of that forward
            for (int i = 0; i < count; ++i) {
                const dbf_status_t st = forward_decode_mfma(hs[i], x, ys[i], batch, stream);
                if (st != DBF_OK) return st;
            }
            return DBF_OK;
        }
        if (nok == count) {
            dbf::I8Args a1{}, a2{};
            a1.count = a2.count = count;
            a1.nrows = a2.nrows = batch;
            for (int i = 0; i < count; ++i) i8_stages(hs[i], x, ys[i], a1.L[i], a2.L[i]);
            dbf_layer *t = hs[0];  // kernel timing follows the first handle
            dbf_status_t st = timed_launch(t, "decode_group_stage1", stream,
                                           [&] { return dbf::launch_decode_i8(a1, 1, false, stream); });
            if (st != DBF_OK) return st;
            return timed_launch(t, "decode_group_stage2", stream,
                                [&] { return dbf::launch_decode_i8(a2, 2, false, stream); });
        }
    }
    // layers whose stage 1 is cut into reduction parts run their own
    // forwards (the grouped kernels do not cut), so each output keeps the
    // bits of the layer's own forward
    for (int i = 0; i < count; ++i) {
        if (dbf::mfma_stage1_parts(hs[i]->m_pad, hs[i]->k_pad, batch) > 1) {
            for (int j = 0; j < count; ++j) {
                const dbf_status_t st = forward_decode_mfma(hs[j], x, ys[j], batch, stream);
                if (st != DBF_OK) return st;
            }
            return DBF_OK;
        }
    }
    dbf::MfmaGroupArgs g{};
    g.count = count;
    g.x = x;
    g.batch = batch;
    g.m = hs[0]->m;
    g.m_pad = hs[0]->m_pad;
    for (int i = 0; i < count; ++i) {
        const dbf_layer *h = hs[i];
        g.L[i] = {h->A_dev, h->B_dev, h->a_dev, h->mid_dev, h->b_dev, ys[i], h->v16, h->n, h->n_pad, h->k_pad};
    }
    dbf_layer *t = hs[0];  // kernel timing follows the first handle
    dbf_status_t st =
        timed_launch(t, "decode_group_stage1", stream, [&] { return dbf::launch_mfma_decode_group(g, stream, 1); });
    if (st != DBF_OK) return st;
    return timed_launch(t, "decode_group_stage2", stream, [&] { return dbf::launch_mfma_decode_group(g, stream, 2); });
}

extern "C" dbf_status_t dbf_linear_backward_data(dbf_handle_t h, const void *dy, void *dx, int32_t batch,
                                                 hipStream_t stream) {
    if (!h) return DBF_ERR_INVALID_ARG;
    if (!h->bwd) return DBF_ERR_UNSUPPORTED;
    return dbf_linear_forward_ex(h->bwd, dy, dx, batch, DBF_PATH_AUTO, stream);
}

extern "C" dbf_status_t dbf_linear_backward(dbf_handle_t h, const void *x, const void *dy, void *dx, float *da,
                                            float *dmid, float *db, int32_t batch, hipStream_t stream) {
    if (!h) return DBF_ERR_INVALID_ARG;
    if (!h->bwd) return DBF_ERR_UNSUPPORTED;
    if (batch < 0 || batch > h->max_batch) return DBF_ERR_INVALID_ARG;
    if (batch == 0) return DBF_OK;
    if (!x || !dy || !aligned16(x) || !aligned16(dy) || (dx && !aligned16(dx))) return DBF_ERR_INVALID_ARG;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return DBF_ERR_HIP;
    if (cur != h->device) return DBF_ERR_INVALID_ARG;
    dbf_layer *t = h->bwd;
    dbf_status_t st = DBF_OK;
    auto finish = [&](int ld, int cols, float *out) {
        return timed_launch(h, "grad_sum_finish", stream,
                            [&] { return dbf::launch_colsum_finish(h->red, ld, batch, cols, out, stream); });
    };
    if (da || dmid) {
        // t = (X ⊙ b) Bᵀ in fp32 (for dmid) and T = rne16(t ⊙ mid) (for s), one product
        st = timed_launch(h, "grad_t", stream, [&] {
            return dbf::launch_sign_gemm(x, h->m, batch, h->m, h->B_dev, h->Wm, h->k_pad, h->b_dev, h->mid_dev, h->T,
                                         h->k_pad, h->k_pad, dmid ? h->t32 : nullptr, h->k_pad, nullptr, 0, 0,
                                         nullptr, stream);
        });
        if (st != DBF_OK) return st;
    }
    if (da) {
        // s = T Aᵀ (before a), summed against dY over the batch in the epilogue: da = Σ_r dY ⊙ s
        st = timed_launch(h, "grad_s", stream, [&] {
            return dbf::launch_sign_gemm(h->T, h->k_pad, batch, h->k_pad, h->A_dev, h->Wk, h->n_pad, nullptr, nullptr,
                                         nullptr, 0, h->n, nullptr, 0, dy, 0, h->n, h->red, stream);
        });
        if (st == DBF_OK) st = finish(h->n, h->n, da);
        if (st != DBF_OK) return st;
    }
    if (dmid || db || dx) {
        // g = (dY ⊙ a) A (the transposed layer holds Aᵀ packed along n and a as its input scale),
        // G = rne16(g ⊙ mid); dmid = Σ_r g ⊙ t in the epilogue
        st = timed_launch(h, "grad_g", stream, [&] {
            return dbf::launch_sign_gemm(dy, h->n, batch, h->n, t->B_dev, t->Wm, t->k_pad, t->b_dev, t->mid_dev, t->T,
                                         t->k_pad, t->k_pad, nullptr, 0, h->t32, 1, h->k_pad,
                                         dmid ? h->red : nullptr, stream);
        });
        if (st == DBF_OK && dmid) st = finish(t->k_pad, h->k, dmid);  // the first k of the k_pad columns
        if (st != DBF_OK) return st;
    }
    if (db || dx) {
        // h = G B (Bᵀ packed along k in the transposed layer), dX = rne16(h ⊙ b), db = Σ_r h ⊙ X in the epilogue
        st = timed_launch(h, "grad_h", stream, [&] {
            return dbf::launch_sign_gemm(t->T, t->k_pad, batch, t->k_pad, t->A_dev, t->Wk, t->n_pad, nullptr,
                                         t->a_dev, dx, h->m, h->m, nullptr, 0, x, 0, h->m, db ? h->red : nullptr,
                                         stream);
        });
        if (st == DBF_OK && db) st = finish(h->m, h->m, db);
    }
    return st;
}

extern "C" dbf_status_t dbf_linear_forward(dbf_handle_t h, const void *x, void *y, int32_t batch,
                                           hipStream_t stream) {
    return dbf_linear_forward_ex(h, x, y, batch, DBF_PATH_AUTO, stream);
}

extern "C" dbf_status_t dbf_timing_enable(dbf_handle_t h, int32_t enable) {
    if (!h) return DBF_ERR_INVALID_ARG;
    h->timing = enable != 0;
    if (h->bwd) h->bwd->timing = h->timing;
    return DBF_OK;
}

extern "C" dbf_status_t dbf_timing_read(dbf_handle_t h, dbf_kernel_time_t *out, int32_t cap, int32_t *count) {
    if (!h || !count || cap < 0 || (cap > 0 && !out)) return DBF_ERR_INVALID_ARG;
    dbf_status_t st = DBF_OK;
    if (h->bwd) {
        // launches of the transposed layer (dbf_linear_backward_data) count as "bwd_<kernel>"
        for (auto &p : h->bwd->pending) {
            p.name = "bwd_" + p.name;
            h->pending.push_back(p);
        }
        h->bwd->pending.clear();
    }
    for (auto &p : h->pending) {
        float ms = 0.0f;
        if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
            st = DBF_ERR_HIP;
        } else {
            auto &t = h->totals[p.name];
            t.first += 1;
            t.second += ms;
        }
        h->event_pool.push_back(p.start);
        h->event_pool.push_back(p.stop);
    }
    h->pending.clear();
    int32_t i = 0;
    for (auto &kv : h->totals) {
        if (i < cap) {
            std::memset(out[i].name, 0, sizeof(out[i].name));
            std::strncpy(out[i].name, kv.first.c_str(), sizeof(out[i].name) - 1);
            out[i].launches = kv.second.first;
            out[i].total_ms = kv.second.second;
        }
        ++i;
    }
    *count = i;
    h->totals.clear();
    return st;
}

// ---------------------------------------------------------------------------
// Forward without allocation: the kernels' scratch (the intermediate v or T,
// split-K and stage-1 partials, tickets, row sums of 0/1 layers) comes from
// one static device array instead of the handle's workspace.  Each device
// that runs it holds its own copy of the array until the process ends.

namespace {

constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};  // the array's device address on each device

// The address of this device's copy of the scratch array (resolved once per
// device, with that device current; the array's name is not a device
// address in host code).
dbf_status_t scratch_on_device(int dev, char **out) {
    if (dev < 0 || dev >= kMaxDevices) return DBF_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DBF_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<char *>(g_scratch_ptr[dev]);
    return DBF_OK;
}

__global__ void zero_u32_kernel(unsigned *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Scratch of one forward at this batch on the default path: the pieces the
// chosen kernels use, each 256-byte aligned, with the sizes the handle's own
// workspace would give them for this batch.
struct ScratchPlan {
    size_t v32 = 0, v16 = 0, tpart = 0, tickets = 0, T = 0, split = 0, stats = 0, total = 0;
    size_t tpart_cap = 0, split_cap = 0;
    bool i8 = false, decode = false, parts = false;
};

ScratchPlan plan_scratch(const dbf_layer *h, int32_t batch) {
    ScratchPlan p;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) & ~size_t(255);
        return at;
    };
    p.decode = batch <= dbf::kDecodeMaxBatch;
    if (p.decode && batch == 1 && h->i8_ok) {
        p.i8 = true;
        p.v32 = take(sizeof(float) * size_t(h->k_pad));
    } else if (p.decode) {
        p.v16 = take(sizeof(uint16_t) * 2 * size_t(dbf::kDecodeMaxBatch) * h->k_pad);
        const int parts = dbf::mfma_stage1_parts(h->m_pad, h->k_pad, dbf::kDecodeMaxBatch);
        if (!h->binary && parts > 1) {
            p.parts = true;
            p.tpart_cap = size_t(parts) * dbf::kDecodeMaxBatch * h->k_pad;
            p.tpart = take(sizeof(float) * p.tpart_cap);
            p.tickets = take(sizeof(unsigned) * size_t(h->ntickets));
        }
    } else {
        p.T = take(sizeof(uint16_t) * size_t(batch) * h->k_pad);
        p.split_cap = std::max<size_t>(64, std::max(dbf::sign_gemm_split_elems(batch, h->m, h->Wm, h->k_pad),
                                                    dbf::sign_gemm_split_elems(batch, h->k_pad, h->Wk, h->n)));
        p.split = take(sizeof(float) * p.split_cap);
    }
    if (h->binary) p.stats = take(sizeof(float) * 2 * size_t(batch));
    p.total = off;
    return p;
}

}  // namespace

extern "C" dbf_status_t dbf_linear_forward_noalloc(dbf_handle_t h, const void *x, void *y, int32_t batch,
                                                   hipStream_t stream) {
    if (!h) return DBF_ERR_INVALID_ARG;
    if (batch < 0 || batch > h->max_batch) return DBF_ERR_INVALID_ARG;
    if (batch == 0) return DBF_OK;
    if (!x || !y || !aligned16(x) || !aligned16(y)) return DBF_ERR_INVALID_ARG;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return DBF_ERR_HIP;
    if (cur != h->device) return DBF_ERR_INVALID_ARG;
    if (h->bqq_groups > 0) return DBF_ERR_UNSUPPORTED;  // (group-wise BQQ scalars: the allocating forward only)
    const ScratchPlan p = plan_scratch(h, batch);
    if (p.total > kNoAllocScratchBytes) return DBF_ERR_SHAPE;  // more scratch than the static array holds
    char *base = nullptr;
    dbf_status_t st = scratch_on_device(cur, &base);
    if (st != DBF_OK) return st;
    // tickets start at zero (the kernels leave them at zero; the array may
    // hold anything from an earlier call)
    if (p.parts) {
        const int n = h->ntickets;
        hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                           reinterpret_cast<unsigned *>(base + p.tickets), n);
        if (hipGetLastError() != hipSuccess) return DBF_ERR_HIP;
    }
    // the handle's workspace pointers, pointed at the scratch for this call
    // (calls on one handle are ordered, so nothing else sees the swap); no
    // timing events either, which would be created on first use
    float *const o_v32 = h->v32, *const o_tpart = h->tpart, *const o_split = h->split, *const o_stats = h->bqq_stats;
    uint16_t *const o_v16 = h->v16, *const o_T = h->T;
    unsigned *const o_tickets = h->tickets;
    const size_t o_tpart_cap = h->tpart_cap, o_split_cap = h->split_cap;
    const bool o_timing = h->timing;
    if (p.i8) h->v32 = reinterpret_cast<float *>(base + p.v32);
    if (p.decode && !p.i8) h->v16 = reinterpret_cast<uint16_t *>(base + p.v16);
    if (p.parts) {
        h->tpart = reinterpret_cast<float *>(base + p.tpart);
        h->tpart_cap = p.tpart_cap;
        h->tickets = reinterpret_cast<unsigned *>(base + p.tickets);
    }
    if (!p.decode) {
        h->T = reinterpret_cast<uint16_t *>(base + p.T);
        h->split = reinterpret_cast<float *>(base + p.split);
        h->split_cap = p.split_cap;
    }
    if (h->binary) h->bqq_stats = reinterpret_cast<float *>(base + p.stats);
    h->timing = false;
    st = dbf_linear_forward_ex(h, x, y, batch, DBF_PATH_AUTO, stream);
    h->v32 = o_v32;
    h->tpart = o_tpart;
    h->split = o_split;
    h->bqq_stats = o_stats;
    h->v16 = o_v16;
    h->T = o_T;
    h->tickets = o_tickets;
    h->tpart_cap = o_tpart_cap;
    h->split_cap = o_split_cap;
    h->timing = o_timing;
    return st;
}
