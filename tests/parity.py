"""Comparison rules shared by the GPU parity tests.

* Codes: equal, except where the oracle's rotated coordinate lies within
  1e-6 (absolute, unit-sphere units) of a threshold; there a difference of
  one code is allowed.
* Norms: within 1e-6 relative.
* Scores and outputs: per row (one score vector over the context, one output
  head vector), ||x - ref||_inf <= 2e-3 * ||ref||_inf.
"""
import numpy as np

import oracle

BAND = 1e-6
REL = 2e-3


def codes_agree(got, want, y, thresholds, band=BAND):
    got = np.asarray(got, np.int64)
    want = np.asarray(want, np.int64)
    near = np.min(np.abs(np.asarray(y)[..., None] - np.asarray(thresholds)), axis=-1) < band
    ok = (got == want) | (near & (np.abs(got - want) <= 1))
    return bool(np.all(ok)), int(np.sum(got != want)), int(np.sum(near))


def words_to_codes(words_i32, bits, d):
    return oracle.unpack_codes(np.asarray(words_i32).view(np.uint32), bits, d)


def rows_close(got, ref, rel=REL, floor=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.max(np.abs(got - ref), axis=-1)
    scale = np.max(np.abs(ref), axis=-1)
    if floor is not None:
        # a row whose values all cancel to near zero (a one-position decode
        # holds a single score) is judged against the scale of the terms
        # summed instead of its own magnitude
        scale = np.maximum(scale, np.asarray(floor, np.float64))
    worst = float(np.max(err / np.where(scale > 0, scale, 1.0)))
    return bool(np.all(err <= rel * scale + 1e-30)), worst
