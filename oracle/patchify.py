"""Plain CPU oracle for the stage-5 space-to-depth (patchify) and its inverse.

TEST INFRASTRUCTURE ONLY (like oracle.rope).

What it computes (sglang PR #34471 page, "Key source snippets", the decoder's
_patchify; _unpatchify is named in "Key files" as its counterpart):

    patchify:   (B, C, F, H, W) -> (B, C*p*p, F, H/p, W/p)
    out[b, (c*p + pw)*p + ph, f, hh, ww] = x[b, c, f, hh*p + ph, ww*p + pw]

i.e. the height and width are cut into p x p patches and each patch moves into
the channel dimension with the packing order (channel, width offset, height
offset), the order the page states must match the checkpoints.  Written as the
page's steps: reshape to (B, C, F, H/p, p, W/p, p), permute to
(b, c, w-offset, h-offset, f, h-patch, w-patch), reshape.  unpatchify is the
exact inverse.  Both are pure data movement: the result is bit-exact for any
element type, so arrays of any numpy dtype are accepted.
"""
from __future__ import annotations

import numpy as np


def patchify(x: np.ndarray, p: int) -> np.ndarray:
    B, C, F, H, W = x.shape
    if p < 1 or H % p or W % p:
        raise ValueError("H and W must be multiples of the patch size")
    y = x.reshape(B, C, F, H // p, p, W // p, p)
    y = y.transpose(0, 1, 6, 4, 2, 3, 5)  # b, c, w-offset, h-offset, f, h-patch, w-patch
    return np.ascontiguousarray(y).reshape(B, C * p * p, F, H // p, W // p)


def unpatchify(y: np.ndarray, p: int) -> np.ndarray:
    B, Cpp, F, Hp, Wp = y.shape
    if p < 1 or Cpp % (p * p):
        raise ValueError("the channel count must be a multiple of p*p")
    C = Cpp // (p * p)
    x = y.reshape(B, C, p, p, F, Hp, Wp)  # b, c, w-offset, h-offset, f, h-patch, w-patch
    x = x.transpose(0, 1, 4, 5, 3, 6, 2)  # b, c, f, h-patch, h-offset, w-patch, w-offset
    return np.ascontiguousarray(x).reshape(B, C, F, Hp * p, Wp * p)
