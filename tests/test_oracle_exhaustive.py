"""Exhaustive sweeps of the oracle's element encoders over float32 (CPU).

* E2M1: every float32 bit pattern except the NaNs goes through
  oracle.formats.e2m1_encode and through an independent rounding written from
  the format's definition: the value is rounded to the grid of its E2M1 binade
  (quantum 0.5 below 2, 1 below 4, 2 above; ties to the even multiple, which is
  the even code), anything above 6 saturates to 6, and the sign bit is copied.
* E4M3: every float32 in [-464, 464] goes through oracle.formats.e4m3_encode
  and through torch's float8_e4m3fn cast (a library routine: round to nearest
  even with subnormals; it agrees with satfinite on this range); every float32
  of larger magnitude, up to infinity, saturates to +-448 (0x7E / 0xFE).

The sweeps run in chunks of 2^21 patterns over a small process pool.
"""

import multiprocessing as mp

import numpy as np
import pytest
import torch

from oracle import formats as F

CHUNK = 1 << 21
WORKERS = 6


def _patterns(lo, hi):
    return np.arange(lo, hi, dtype=np.int64).astype(np.uint32)


def _ref_e2m1(u):
    a = np.abs(u.astype(np.float64))
    q = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    v = np.minimum(np.rint(a / q) * q, 6.0)
    mag = np.where(v < 2.0, 2.0 * v, np.where(v < 4.0, v + 2.0, v / 2.0 + 4.0)).astype(np.uint8)
    return mag | ((u.view(np.uint32) >> np.uint32(31)).astype(np.uint8) << np.uint8(3))


def _e2m1_chunk(lo):
    u = _patterns(lo, min(lo + CHUNK, 1 << 32)).view(np.float32)
    u = u[~np.isnan(u)]
    got, ref = F.e2m1_encode(u), _ref_e2m1(u)
    bad = np.flatnonzero(got != ref)
    return int(u.size), [int(u.view(np.uint32)[i]) for i in bad[:4]]


def _e4m3_chunk(args):
    lo, hi, sign = args
    p = _patterns(lo, hi) | np.uint32(sign << 31)
    x = p.view(np.float32)
    got = F.e4m3_encode(x)
    if hi <= 0x43E80001:  # |x| <= 464: the library cast
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    else:                 # beyond: saturation to the largest finite value
        ref = np.full(x.shape, 0xFE if sign else 0x7E, np.uint8)
    bad = np.flatnonzero(got != ref)
    return int(x.size), [int(p[i]) for i in bad[:4]]


def _run(fn, items):
    with mp.get_context("fork").Pool(WORKERS) as pool:
        return pool.map(fn, items, chunksize=1)


@pytest.mark.slow
def test_e2m1_exhaustive_over_float32():
    res = _run(_e2m1_chunk, range(0, 1 << 32, CHUNK))
    bad = [b for _, bs in res for b in bs]
    assert sum(n for n, _ in res) == (1 << 32) - 2 * ((1 << 23) - 1)  # all but the NaNs
    assert not bad, [hex(b) for b in bad[:8]]


@pytest.mark.slow
def test_e4m3_exhaustive_over_float32():
    top = 0x43E80001        # one past 464.0
    inf = 0x7F800001        # one past +inf
    items = [(lo, min(lo + CHUNK, top), s) for s in (0, 1) for lo in range(0, top, CHUNK)]
    items += [(lo, min(lo + CHUNK, inf), s) for s in (0, 1) for lo in range(top, inf, CHUNK)]
    res = _run(_e4m3_chunk, items)
    bad = [b for _, bs in res for b in bs]
    assert sum(n for n, _ in res) == 2 * 0x7F800001
    assert not bad, [hex(b) for b in bad[:8]]
