"""The tiling rule of the align stage, written out for the tests.

Every expert's rows are cut into floor(count / BIG) tiles of BIG rows and the
remainder is padded to whole tiles of SMALL rows; with SMALL == BIG there is
one tile class: ceil(count / BIG) tiles, all in the BIG list.
"""
import numpy as np


def tiles_per_expert(counts, BIG, SMALL):
    counts = np.asarray(counts, dtype=np.int64)
    if SMALL == BIG:
        return (counts + BIG - 1) // BIG, np.zeros_like(counts)
    nbig = counts // BIG
    return nbig, (counts - nbig * BIG + SMALL - 1) // SMALL


def padded_rows(counts, BIG, SMALL):
    nbig, nsmall = tiles_per_expert(counts, BIG, SMALL)
    return nbig * BIG + nsmall * SMALL
