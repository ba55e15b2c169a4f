"""Host packer and device tiling of the sign matrices (CPU only, no GPU needed).

The pages fix only that A and B hold +1/-1 ("Addition is almost all you
need", gist.science technical summary, §2.1); the bit format is the
library's own, stated in include/dbf.h: 32 signs per uint32 along the
reduction dimension, least significant bit first, bit 1 = -1, zero padding.
The checks here use an unpacker written independently from that statement.
"""

import numpy as np
import pytest

import dbf_linear_fwd_amd as dbf


def unpack_reference(words: np.ndarray, cols: int) -> np.ndarray:
    """Independent unpacker: bit p of word w is column 32w+p; 1 means -1."""
    rows, nw = words.shape
    bits = (words[:, :, None] >> np.arange(32, dtype=np.uint32)[None, None, :]) & 1
    flat = bits.reshape(rows, nw * 32)[:, :cols]
    return np.where(flat == 1, -1, 1).astype(np.int8)


def test_known_words():
    row = np.ones(32, dtype=np.int8)
    row[0] = -1
    assert dbf.dbf_pack_signs(row[None, :])[0, 0] == 0x00000001
    row = np.ones(32, dtype=np.int8)
    row[31] = -1
    assert dbf.dbf_pack_signs(row[None, :])[0, 0] == 0x80000000
    assert dbf.dbf_pack_signs(-np.ones((1, 32), np.int8))[0, 0] == 0xFFFFFFFF
    assert dbf.dbf_pack_signs(np.ones((1, 32), np.int8))[0, 0] == 0
    alt = np.array([1, -1] * 16, dtype=np.int8)
    assert dbf.dbf_pack_signs(alt[None, :])[0, 0] == 0xAAAAAAAA
    # a short row: only 3 columns, -1,+1,-1 -> bits 0 and 2; pad bits stay 0
    assert dbf.dbf_pack_signs(np.array([[-1, 1, -1]], np.int8))[0, 0] == 0x5
    # 33 columns spill into a second word
    r = np.ones((1, 33), np.int8)
    r[0, 32] = -1
    w = dbf.dbf_pack_signs(r)
    assert w.shape == (1, 2) and w[0, 0] == 0 and w[0, 1] == 1


@pytest.mark.parametrize("rows,cols", [(1, 1), (1, 31), (3, 32), (5, 33), (7, 37), (31, 64), (33, 100), (2, 4096)])
def test_round_trip_and_padding(rows, cols):
    rng = np.random.default_rng(rows * 1000 + cols)
    S = (1 - 2 * rng.integers(0, 2, size=(rows, cols))).astype(np.int8)
    words = dbf.dbf_pack_signs(S)
    assert words.shape == (rows, (cols + 31) // 32)
    assert np.array_equal(unpack_reference(words, cols), S)
    # bits past the last column are zero
    tail = cols % 32
    if tail:
        assert np.all(words[:, -1] >> np.uint32(tail) == 0)
    # extra words requested past the data are written as zero
    wide = dbf.dbf_pack_signs(S, words_per_row=words.shape[1] + 3)
    assert np.array_equal(wide[:, :words.shape[1]], words)
    assert np.all(wide[:, words.shape[1]:] == 0)


def test_pack_rejects_bad_input():
    with pytest.raises(dbf.DbfError) as e:
        dbf.dbf_pack_signs(np.array([[1, 0, -1]], np.int8))
    assert e.value.status == dbf.DBF_ERR_INVALID_ARG
    with pytest.raises(dbf.DbfError):
        dbf.dbf_pack_signs(np.array([[1, 2]], np.int8))
    with pytest.raises(dbf.DbfError):
        dbf.dbf_pack_signs(np.ones((1, 40), np.int8), words_per_row=1)


def layout_reference(words: np.ndarray) -> np.ndarray:
    """Independent model of the device tiling stated in include/dbf.h.

    Rows are grouped in tiles of 64 (zero-filled), words in pairs; within a
    word, element 2q goes to bit q and element 2q+1 to bit 16+q.
    """
    rows, nw = words.shape
    assert nw % 2 == 0
    tiles = (rows + 63) // 64
    padded = np.zeros((tiles * 64, nw), dtype=np.uint32)
    padded[:rows] = words
    # bit permutation, element by element
    perm = np.zeros_like(padded)
    for e in range(32):
        dst = e // 2 if e % 2 == 0 else 16 + e // 2
        perm |= ((padded >> np.uint32(e)) & np.uint32(1)) << np.uint32(dst)
    # [tile][pair][row in tile][half]
    t = perm.reshape(tiles, 64, nw // 2, 2).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(t).reshape(-1)


@pytest.mark.parametrize("rows,words", [(1, 2), (64, 2), (65, 4), (130, 6), (200, 128)])
def test_device_layout(rows, words):
    rng = np.random.default_rng(rows + words)
    W = rng.integers(0, 2 ** 32, size=(rows, words), dtype=np.uint64).astype(np.uint32)
    got = dbf.dbf_layout_signs(W)
    assert got.size == dbf.dbf_layout_words(rows, words) == ((rows + 63) // 64) * 64 * words
    assert np.array_equal(got, layout_reference(W))


def test_device_layout_pair_positions():
    """Element 2q sits at bit q and element 2q+1 at bit 16+q: after shifting the
    word left by 15-q both land on the fp16 sign bits (15 and 31)."""
    for e in range(32):
        row = np.ones((1, 64), np.int8)
        row[0, e] = -1
        dev = dbf.dbf_layout_signs(dbf.dbf_pack_signs(row))
        word = int(dev[0])
        q = e // 2
        assert word == (1 << (q if e % 2 == 0 else 16 + q))
        shifted = (word << (15 - q)) & 0xFFFFFFFF
        assert shifted & 0x80008000 == (0x8000 if e % 2 == 0 else 0x80000000)


def test_layout_rejects_odd_words():
    with pytest.raises(dbf.DbfError):
        dbf.dbf_layout_signs(np.zeros((2, 3), np.uint32))


# --------------------------------------------------------------------------- batch-1 decode layout

def layout_dec_reference(S: np.ndarray, rows_pad: int, cols_pad: int) -> np.ndarray:
    """Independent construction from the statement in include/dbf.h: word i of
    lane l = r + 16 g in superchunk s of tile T sits at
    T * cols_pad / 2 + 256 s + W l + i, and its bit 8 b + j is the sign bit
    (1 for -1) of column 512 s + 128 i + 16 j + 4 g + b of row 16 T + r."""
    rows, cols = S.shape
    neg = np.zeros((rows_pad, cols_pad), dtype=np.uint32)
    neg[:rows, :cols] = (S == -1)
    out = np.zeros(rows_pad // 16 * cols_pad // 2 + 4, dtype=np.uint32)
    nsc = -(-cols_pad // 512)
    for T in range(rows_pad // 16):
        for s in range(nsc):
            W = 4 if s + 1 < nsc else (cols_pad - 512 * s) // 128
            for l in range(64):
                r, g = l % 16, l // 16
                for i in range(W):
                    word = 0
                    for j in range(8):
                        for b in range(4):
                            word |= int(neg[16 * T + r, 512 * s + 128 * i + 16 * j + 4 * g + b]) << (8 * b + j)
                    out[T * cols_pad // 2 + 256 * s + W * l + i] = word
    return out


@pytest.mark.parametrize("rows,cols,rows_pad,cols_pad", [
    (1, 1, 16, 128), (16, 128, 16, 128), (17, 300, 32, 384), (5, 512, 16, 512), (33, 640, 48, 640),
    (20, 1408, 32, 1408), (16, 1000, 16, 1024), (3, 700, 64, 896)])
def test_decode_layout_matches_statement(rows, cols, rows_pad, cols_pad):
    rng = np.random.default_rng(rows * 7 + cols)
    S = (1 - 2 * rng.integers(0, 2, size=(rows, cols))).astype(np.int8)
    got = dbf.dbf_layout_signs_dec(dbf.dbf_pack_signs(S), cols, rows_pad, cols_pad)
    assert got.size == dbf.dbf_layout_words_dec(rows_pad, cols_pad) == rows_pad // 16 * cols_pad // 2 + 4
    assert np.array_equal(got, layout_dec_reference(S, rows_pad, cols_pad))


def test_decode_layout_bad_arguments():
    P = dbf.dbf_pack_signs(np.ones((4, 40), np.int8))
    for cols, rp, cp in ((40, 8, 128), (40, 16, 100), (200, 16, 128), (40, 2, 128)):
        with pytest.raises(dbf.DbfError):
            dbf.dbf_layout_signs_dec(P, cols, rp, cp)
    assert dbf.dbf_layout_words_dec(8, 128) == 0 and dbf.dbf_layout_words_dec(16, 64) == 0
