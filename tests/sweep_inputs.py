"""Input tensors that put every bf16 bit pattern through the quantizer's
rounding (test infrastructure, not a test module; no quantization arithmetic:
bit patterns are only placed).

Each 32-element block holds sweep values beside an *anchor*, a value whose
exponent fixes the block's scale code, so that every pattern is rounded at a
chosen scale.  The anchors sit on both sides of the scale codes where the
kernels switch arithmetic order (code 40 for the folded H16 normalisation),
at the ends of the scale range and at typical codes, each as the smallest and
the largest value of its binade.  Layouts:

  hn0:   31 sweep values + 1 anchor per block (anchor at position 31 or 0,
         alternating, sign alternating); every finite pattern at every anchor.
  hn16:  one sweep value in the first 16-element half, the anchor in the
         second; the size-16 rotation spreads each over its half, so the block
         holds the sweep value (divided by 4) 16 times beside the anchor.
         Patterns from the anchor's binade down 24 binades, at every anchor;
         plus every finite pattern paired with its neighbour (one per half).
  hn32:  one sweep value and the anchor 16 positions apart (they meet in the
         last butterfly stage, across the two halves); plus every finite
         pattern alone in a block.
Non-finite patterns (exponent field 0xFF) fill blocks of their own.
"""
from __future__ import annotations

import numpy as np

ALL = np.arange(1 << 16, dtype=np.uint32)
FINITE = ALL[((ALL >> 7) & 0xFF) != 0xFF].astype(np.uint16)       # 65280 patterns
NONFINITE = ALL[((ALL >> 7) & 0xFF) == 0xFF].astype(np.uint16)    # 256 patterns

# scale codes the anchors aim at (each as 1.0 and 1.9921875 times its binade)
ANCHOR_CODES = {"hn0": [1, 2, 38, 39, 40, 41, 42, 64, 100, 126, 127, 128, 200, 250],
                "hn16": [38, 39, 40, 41, 127, 200],
                "hn32": [40, 127, 200]}
NBK = 16          # blocks per line: lines of 512 elements


def _bits(sign, expf, mant):
    return ((np.asarray(sign, np.uint32) << 15) | (np.asarray(expf, np.uint32) << 7)
            | np.asarray(mant, np.uint32)).astype(np.uint16)


def anchors(layout: str, emax: int) -> list[int]:
    """bf16 patterns of the anchors: the block maximum 2^(S - 127 + emax) (times
    1 or 1.9921875) gives scale code S; under a size-16 rotation the anchor is
    divided by 4 first, so it is 4 times larger.  Plus two subnormal anchors
    (scale code 0) and a zero anchor (the block's scale set by the sweep)."""
    extra = 2 if layout == "hn16" else 0
    out = []
    for s in ANCHOR_CODES[layout]:
        expf = s + emax + extra
        if 1 <= expf <= 254:
            out += [int(_bits(0, expf, 0)), int(_bits(0, expf, 0x7F))]
    if layout == "hn0":
        out += [0x0001, 0x0040, 0x0000]
    return out


def _place(vals, width):
    """vals -> [ceil(len / width), width] padded with +0."""
    n = (len(vals) + width - 1) // width
    out = np.zeros(n * width, np.uint16)
    out[:len(vals)] = vals
    return out.reshape(n, width)


def _nonfinite_blocks():
    # each non-finite pattern at position (i % 32) of an otherwise small block
    blk = np.zeros((NONFINITE.size, 32), np.uint16)
    blk[:, :] = 0x3F00                         # 0.5
    blk[np.arange(NONFINITE.size), np.arange(NONFINITE.size) % 32] = NONFINITE
    return blk


def blocks(layout: str, emax: int) -> np.ndarray:
    """[nblocks, 32] bf16 patterns of the sweep for one layout and grid emax."""
    parts = []
    if layout == "hn0":
        for ai, a in enumerate(anchors("hn0", emax)):
            sw = _place(FINITE, 31)
            n = sw.shape[0]
            blk = np.zeros((n, 32), np.uint16)
            odd = (np.arange(n) % 2 == 1)
            sign = ((np.arange(n) // 2 + ai) % 2).astype(np.uint16) << 15
            blk[~odd, :31] = sw[~odd]
            blk[~odd, 31] = a | sign[~odd]
            blk[odd, 1:] = sw[odd]
            blk[odd, 0] = a | sign[odd]
            parts.append(blk)
    elif layout == "hn16":
        for ai, a in enumerate(anchors("hn16", emax)):
            ea = (a >> 7) & 0xFF
            lo = max(ea - 24, 0)
            mags = FINITE[(((FINITE >> 7) & 0xFF) >= lo) & (((FINITE >> 7) & 0xFF) <= ea)]
            n = mags.size
            blk = np.zeros((n, 32), np.uint16)
            p = np.arange(n) % 16
            blk[np.arange(n), p] = mags
            blk[np.arange(n), 16 + (p * 7 + ai) % 16] = a | (((np.arange(n) // 16) % 2) << 15).astype(np.uint16)
            parts.append(blk)
        pairs = _place(FINITE, 2)
        n = pairs.shape[0]
        blk = np.zeros((n, 32), np.uint16)
        p = np.arange(n) % 16
        blk[np.arange(n), p] = pairs[:, 0]
        blk[np.arange(n), 16 + (15 - p)] = pairs[:, 1]
        parts.append(blk)
    elif layout == "hn32":
        for ai, a in enumerate(anchors("hn32", emax)):
            ea = (a >> 7) & 0xFF
            lo = max(ea - 24, 0)
            mags = FINITE[(((FINITE >> 7) & 0xFF) >= lo) & (((FINITE >> 7) & 0xFF) <= ea)]
            n = mags.size
            blk = np.zeros((n, 32), np.uint16)
            p = np.arange(n) % 32
            blk[np.arange(n), p] = mags
            blk[np.arange(n), (p + 16) % 32] = a | (((np.arange(n) // 32 + ai) % 2) << 15).astype(np.uint16)
            parts.append(blk)
        n = FINITE.size
        blk = np.zeros((n, 32), np.uint16)
        blk[np.arange(n), np.arange(n) % 32] = FINITE
        parts.append(blk)
    else:
        raise ValueError(layout)
    parts.append(_nonfinite_blocks())
    return np.concatenate(parts)


def tensor(layout: str, emax: int) -> np.ndarray:
    """The sweep as a row-wise tensor [lines x 512]: block b is line b // 16,
    block b % 16.  Lines are padded with zero blocks to a multiple of 32 that
    is not a multiple of 128, so the column-wise kernels (which read the
    transpose) see full and ragged tiles."""
    blk = blocks(layout, emax)
    lines = (blk.shape[0] + NBK - 1) // NBK
    lines = (lines + 31) // 32 * 32
    if lines % 128 == 0:
        lines += 32
    out = np.zeros((lines * NBK, 32), np.uint16)
    out[:blk.shape[0]] = blk
    return out.reshape(lines, NBK * 32)
