"""Readers for the library's internal output layouts (test infrastructure)."""

import numpy as np


def frag_rows(flat, T: int, N: int) -> np.ndarray:
    """The [T, N] matrix held in the fragment layout of include/awq.h: whole
    256 x 256 tiles; in tile (tm, tn), wave w = 4 wm + wn, block (i, j), lane
    l = 16 l16 + lc and component r hold output (256 tm + 128 wm + 16 i +
    4 l16 + r, 256 tn + 64 wn + 16 j + lc)."""
    tm_n, tn_n = -(-T // 256), -(-N // 256)
    a = np.asarray(flat)[:tm_n * tn_n * 65536]
    a = a.reshape(tm_n, tn_n, 2, 4, 8, 4, 4, 16, 4)
    #             tm    tn  wm wn  i  j l16 lc  r
    a = a.transpose(0, 2, 4, 6, 8, 1, 3, 5, 7)
    return a.reshape(tm_n * 256, tn_n * 256)[:T, :N]
