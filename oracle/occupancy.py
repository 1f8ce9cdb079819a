"""Integer tile classification of an additive mask (test infrastructure only).

The method never materialises the Lq x Lk score matrix (NeMo AutoModel
"dflash.draft_kimi_k3" page, KimiK3DFlashAttention.forward), and the DFlash
mask is mostly -inf, so the attention skips tiles that contribute nothing.
This module defines, plainly, which tiles those are:

  class 0: every entry of the tile is exactly -inf  (contributes exp(-inf) = 0)
  class 1: every entry is +0 or -0                  (adding it changes no score)
  class 2: every entry is +-0 or -inf, both present (the mask only hides keys, so
           a visibility bit per entry carries all of it)
  class 3: anything else (some finite non-zero value, NaN, +inf)

A tile is rows [qt*BM, min((qt+1)*BM, Lq)) x cols [kt*BN, min((kt+1)*BN, Lk));
only entries inside the mask count.  The list of a (batch, q-tile) is its
non-class-0 k-tiles in increasing k order.  For a class-2 tile, the visibility
word of tile row r has bit k set iff entry (qt*BM + r, kt*BN + k) is +-0.
"""
from __future__ import annotations

import numpy as np

from ._arrays import f64


def tile_classes(mask, BM: int, BN: int) -> np.ndarray:
    """mask [B, 1, Lq, Lk] -> uint8 [B, ceil(Lq/BM), ceil(Lk/BN)]."""
    m = f64(mask)
    B, _, Lq, Lk = m.shape
    nq = -(-Lq // BM)
    nk = -(-Lk // BN)
    out = np.empty((B, nq, nk), dtype=np.uint8)
    for b in range(B):
        for qt in range(nq):
            rows = m[b, 0, qt * BM:(qt + 1) * BM]
            for kt in range(nk):
                t = rows[:, kt * BN:(kt + 1) * BN]
                hidden = t == -np.inf
                zero = t == 0.0
                if np.all(hidden):
                    out[b, qt, kt] = 0
                elif np.all(zero):
                    out[b, qt, kt] = 1
                elif np.all(hidden | zero):
                    out[b, qt, kt] = 2
                else:
                    out[b, qt, kt] = 3
    return out


def tile_bits(mask, BM: int, BN: int, classes: np.ndarray) -> np.ndarray:
    """uint64 [B, nqt, nkt, BM]: visibility words of the class-2 tiles (0 elsewhere)."""
    m = f64(mask)
    B, _, Lq, Lk = m.shape
    nq, nk = classes.shape[1], classes.shape[2]
    out = np.zeros((B, nq, nk, BM), dtype=np.uint64)
    for b, qt, kt in zip(*np.nonzero(classes == 2)):
        t = m[b, 0, qt * BM:(qt + 1) * BM, kt * BN:(kt + 1) * BN]
        for r in range(t.shape[0]):
            word = 0
            for k in range(t.shape[1]):
                if t[r, k] == 0.0:
                    word |= 1 << k
            out[b, qt, kt, r] = word
    return out


def tile_lists(classes: np.ndarray):
    """For each (b, qt): (k-tile indices, their classes) of the non-empty tiles."""
    B, nq, _ = classes.shape
    res = []
    for b in range(B):
        row = []
        for qt in range(nq):
            idx = np.nonzero(classes[b, qt])[0]
            row.append((idx.astype(np.int64), classes[b, qt, idx].astype(np.uint8)))
        res.append(row)
    return res
