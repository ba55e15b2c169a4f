// Host-side sign packing for the DBF layer.
//
// The factors A (n x k) and B (k x m) hold only +1 and -1 ("Addition is almost
// all you need", gist.science technical summary, §2.1), so one bit per entry
// suffices.  Signs are packed along each matrix's reduction dimension, 32 per
// uint32, least significant bit first, bit 1 meaning -1.  The device copy is
// re-tiled so that a wavefront reading one row per lane reads contiguous
// memory, and the bits inside a word are reordered so that two neighbouring
// elements land on the two fp16 sign-bit positions after a single shift.

#include <cstdint>
#include <cstring>

#include "dbf.h"
#include "dbf_internal.h"

namespace dbf {

// Device bit position of element e (0..31) of a 32-element block.
static inline uint32_t device_bit(uint32_t e) { return (e & 1u) ? 16u + (e >> 1) : (e >> 1); }

uint32_t reorder_word(uint32_t canonical) {
    uint32_t out = 0;
    for (uint32_t e = 0; e < 32; ++e) {
        out |= ((canonical >> e) & 1u) << device_bit(e);
    }
    return out;
}

}  // namespace dbf

extern "C" dbf_status_t dbf_pack_signs(const int8_t *S, int32_t rows, int32_t cols, uint32_t *out,
                                       int32_t words_per_row) {
    if (!S || !out || rows < 1 || cols < 1) return DBF_ERR_INVALID_ARG;
    const int64_t need = (static_cast<int64_t>(cols) + 31) / 32;
    if (words_per_row < need) return DBF_ERR_INVALID_ARG;
    for (int64_t r = 0; r < rows; ++r) {
        const int8_t *src = S + r * static_cast<int64_t>(cols);
        uint32_t *dst = out + r * static_cast<int64_t>(words_per_row);
        for (int64_t w = 0; w < words_per_row; ++w) {
            uint32_t word = 0;
            const int64_t c0 = w * 32;
            for (int64_t p = 0; p < 32 && c0 + p < cols; ++p) {
                const int8_t s = src[c0 + p];
                if (s == -1) {
                    word |= 1u << p;
                } else if (s != 1) {
                    return DBF_ERR_INVALID_ARG;
                }
            }
            dst[w] = word;
        }
    }
    return DBF_OK;
}

extern "C" size_t dbf_layout_words(int32_t rows, int32_t words) {
    if (rows < 1 || words < 1) return 0;
    const size_t tiles = (static_cast<size_t>(rows) + 63) / 64;
    const size_t wpad = (static_cast<size_t>(words) + 1) & ~static_cast<size_t>(1);
    return tiles * 64 * wpad;
}

extern "C" dbf_status_t dbf_layout_signs(const uint32_t *in, int32_t rows, int32_t words, uint32_t *out) {
    if (!in || !out || rows < 1 || words < 1 || (words & 1)) return DBF_ERR_INVALID_ARG;
    const int64_t tiles = (static_cast<int64_t>(rows) + 63) / 64;
    const int64_t pairs = words / 2;
    for (int64_t t = 0; t < tiles; ++t) {
        for (int64_t p = 0; p < pairs; ++p) {
            for (int64_t r = 0; r < 64; ++r) {
                const int64_t row = t * 64 + r;
                for (int64_t h = 0; h < 2; ++h) {
                    const int64_t o = ((t * pairs + p) * 64 + r) * 2 + h;
                    out[o] = row < rows ? dbf::reorder_word(in[row * words + 2 * p + h]) : 0u;
                }
            }
        }
    }
    return DBF_OK;
}

// Layout of the batch-1 decode kernels (int8 matrix cores).  Rows in tiles
// of 16; the reduction dimension, padded to cols_pad (a multiple of 128), in
// superchunks of 512 columns (the last one may hold 128, 256 or 384).  In
// superchunk s of tile T, lane l = r + 16 g holds W_s words (W_s = 4 except
// in a short last superchunk), word i at
//     T * cols_pad / 2 + 256 s + W_s l + i,
// and bit 8 b + j of that word is the sign bit of column
// 512 s + 128 i + 16 j + 4 g + b of row 16 T + r (j < 8, b < 4).  AND-ing a
// word with 0x01010101 << j then gives the four int8 operand values of
// columns 16 j + 4 g + b, b < 4, of each of its 128-column blocks.
extern "C" size_t dbf_layout_words_dec(int32_t rows_pad, int32_t cols_pad) {
    if (rows_pad < 16 || cols_pad < 128 || (rows_pad % 16) || (cols_pad % 128)) return 0;
    return static_cast<size_t>(rows_pad / 16) * (cols_pad / 2) + 4;  // + 4: room for a full-width read of the tail
}

extern "C" dbf_status_t dbf_layout_signs_dec(const uint32_t *in, int32_t rows, int32_t cols, int32_t words,
                                             int32_t rows_pad, int32_t cols_pad, uint32_t *out) {
    if (!in || !out || rows < 1 || cols < 1 || words < (static_cast<int64_t>(cols) + 31) / 32) return DBF_ERR_INVALID_ARG;
    if (rows_pad < rows || cols_pad < cols || (rows_pad % 16) || (cols_pad % 128)) return DBF_ERR_INVALID_ARG;
    const int64_t tiles = rows_pad / 16;
    const int64_t tile_words = cols_pad / 2;
    const int64_t nsc = (cols_pad + 511) / 512;
    const int64_t wlast = (cols_pad - 512 * (nsc - 1)) / 128;
    std::memset(out, 0, sizeof(uint32_t) * dbf_layout_words_dec(rows_pad, cols_pad));
    for (int64_t t = 0; t < tiles; ++t) {
        for (int64_t s = 0; s < nsc; ++s) {
            const int64_t W = s + 1 < nsc ? 4 : wlast;
            for (int64_t l = 0; l < 64; ++l) {
                const int64_t r = l & 15, g = l >> 4, row = 16 * t + r;
                if (row >= rows) continue;
                const uint32_t *src = in + row * static_cast<int64_t>(words);
                for (int64_t i = 0; i < W; ++i) {
                    uint32_t word = 0;
                    for (int64_t j = 0; j < 8; ++j)
                        for (int64_t b = 0; b < 4; ++b) {
                            const int64_t col = 512 * s + 128 * i + 16 * j + 4 * g + b;
                            if (col < cols && ((src[col >> 5] >> (col & 31)) & 1u)) word |= 1u << (8 * b + j);
                        }
                    out[t * tile_words + 256 * s + W * l + i] = word;
                }
            }
        }
    }
    return DBF_OK;
}
