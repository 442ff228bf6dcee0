"""The forward quantiser's division-free scale (host check, no GPU).

For a bf16 group maximum amax = (1 + i/128) * 2^(e-127) with e >= 8, the
kernel takes scale = RN(amax / 127) and inv = RN(1 / scale) as a 128-entry
table of RN((1 + i/128) / 127) and its rounded reciprocal, scaled by 2^(e-127)
and 2^(127-e).  That rests on rounding commuting with scaling by a power of
two while the results stay normal.  This test checks the claim for every
positive finite bf16 value with e >= 8 against IEEE single-precision division
(numpy's float32 division rounds correctly), and that e = 7 is where it first
fails, so the kernel's threshold is the tight one.
"""

import numpy as np


def _table():
    i = np.arange(128, dtype=np.float32)
    s = (np.float32(1) + i / np.float32(128)) / np.float32(127)
    return s, np.float32(1) / s


def _direct(amax):
    scale = amax / np.float32(127)
    return scale, np.float32(1) / scale


def _shortcut(e, i):
    ts, ti = _table()
    return (np.ldexp(ts[i], e - 127).astype(np.float32), np.ldexp(ti[i], 127 - e).astype(np.float32))


def _values(e):
    e = np.repeat(np.asarray(e, dtype=np.int64), 128)
    i = np.tile(np.arange(128), len(e) // 128)
    bits = (e.astype(np.uint32) << np.uint32(23)) | (i.astype(np.uint32) << np.uint32(16))
    return e, i, bits.view(np.float32)


def test_shortcut_equals_division_for_every_bf16_from_2_to_minus_119():
    e, i, amax = _values(np.arange(8, 255))
    ds, di = _direct(amax)
    fs, fi = _shortcut(e, i)
    assert np.all(np.isfinite(ds)) and np.all(np.isfinite(di))
    assert np.array_equal(ds.view(np.uint32), fs.view(np.uint32))
    assert np.array_equal(di.view(np.uint32), fi.view(np.uint32))


def test_below_the_threshold_the_shortcut_would_be_wrong():
    # at e = 7 the scale is subnormal for part of the mantissas: the kernel
    # must (and does) take the division there
    e, i, amax = _values([7])
    ds, _ = _direct(amax)
    fs, _ = _shortcut(e, i)
    assert not np.array_equal(ds.view(np.uint32), fs.view(np.uint32))
