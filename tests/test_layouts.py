"""The fragment-layout reader against the index formula include/awq.h states
for the reference output (checked element by element on a ragged matrix)."""

import numpy as np

from layouts import frag_rows


def header_index(t, n, tiles_n):
    tm, tn, a, b = t // 256, n // 256, t % 256, n % 256
    w = (a // 128) * 4 + b // 64
    i, j = (a % 128) // 16, (b % 64) // 16
    l, r = ((a % 16) // 4) * 16 + b % 16, a % 4
    return ((((tm * tiles_n + tn) * 8 + w) * 32 + i * 4 + j) * 64 + l) * 4 + r


def test_frag_rows_follows_the_header_formula():
    T, N = 300, 530                      # 2 x 3 tiles, both ragged
    flat = np.arange(512 * 768, dtype=np.int64)
    M = frag_rows(flat, T, N)
    assert M.shape == (T, N)
    tt, nn = np.meshgrid(np.arange(T), np.arange(N), indexing="ij")
    np.testing.assert_array_equal(M, header_index(tt, nn, 3))
    # every entry of the used tiles appears once
    assert len(np.unique(frag_rows(flat, 512, 768))) == 512 * 768
