"""Pins of the oracle's weight packing and Q8_0 activation quantisation (CPU only)."""
import numpy as np
import pytest

from goldens import load
import refmath

RANGES = {8: (-128, 127), 4: (-8, 7), 2: (-2, 1)}


@pytest.mark.parametrize("case", sorted(load("pack_layout.txt")))
def test_pack_golden(oracle_lib, case):
    c = load("pack_layout.txt")[case]
    wbits = int(c["wbits"][0])
    vals = np.array([int(v) for v in c["values"]], np.int8)
    want = np.array([int(b, 16) for b in c["bytes"]], np.uint8)
    assert np.array_equal(oracle_lib.pack(vals, wbits), want)
    assert np.array_equal(oracle_lib.unpack(want, wbits, 32), vals)
    assert np.array_equal(refmath.unpack_np(want, wbits, 32), vals.astype(np.int64))


@pytest.mark.parametrize("wbits", [8, 4, 2])
def test_pack_roundtrip_exhaustive(oracle_lib, wbits):
    """Every representable value at every position of a block survives pack -> unpack,
    and every byte value at every byte position survives unpack -> pack."""
    lo, hi = RANGES[wbits]
    vals = np.arange(lo, hi + 1)
    nv = vals.size
    blocks = np.array([[vals[(s + pos) % nv] for pos in range(32)] for s in range(nv)], np.int8)
    for pos in range(32):  # each position sees every value
        assert set(blocks[:, pos].tolist()) == set(vals.tolist())
    q = blocks.reshape(-1)
    assert np.array_equal(oracle_lib.unpack(oracle_lib.pack(q, wbits), wbits, q.size), q)
    rb = 32 * wbits // 8
    allbytes = np.array([[(s + pos) % 256 for pos in range(rb)] for s in range(256)], np.uint8).ravel()
    n = allbytes.size * 8 // wbits
    back = oracle_lib.pack(oracle_lib.unpack(allbytes, wbits, n), wbits)
    assert np.array_equal(back, allbytes)
    assert np.array_equal(oracle_lib.unpack(allbytes, wbits, n).astype(np.int64),
                          refmath.unpack_np(allbytes, wbits, n))


def test_pack_rejects_out_of_range(oracle_lib):
    with pytest.raises(ValueError):
        oracle_lib.pack(np.full(32, 8, np.int8), 4)
    with pytest.raises(ValueError):
        oracle_lib.pack(np.full(32, -3, np.int8), 2)


@pytest.mark.parametrize("case", sorted(load("q8_0_blocks.txt")))
def test_q8_0_golden(oracle_lib, case):
    c = load("q8_0_blocks.txt")[case]
    x = np.array([float(v) for v in c["x"]], np.float32)[None, :]
    q, d = oracle_lib.quantize_q8_0(x)
    assert d[0, 0] == np.float32(float(c["d"][0]))
    assert np.array_equal(q[0], np.array([int(v) for v in c["q"]], np.int8))


def test_q8_0_properties(oracle_lib):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 256)) * rng.uniform(1e-3, 1e3, (64, 1))).astype(np.float32)
    x[3, 32:64] = 0.0
    q, d = oracle_lib.quantize_q8_0(x)
    xb = x.reshape(64, 8, 32).astype(np.float64)
    qb = q.reshape(64, 8, 32).astype(np.float64)
    amax = np.abs(xb).max(axis=2)
    # d is the fp32 quotient max|x| / 127
    assert np.array_equal(d, (amax.astype(np.float32) / np.float32(127.0)))
    dd = d.astype(np.float64)[..., None]
    # reconstruction error at most half a step, plus the rounding of the fp32
    # quotient x / d (half an ulp of a value below 128: 2^-18)
    err = np.abs(xb - dd * qb)
    assert np.all(err <= dd * (0.5 + 2.0 ** -18))
    # the largest magnitude maps to +-127, signs agree, codes in range
    nz = amax > 0
    arg = np.abs(xb).argmax(axis=2)
    top = np.take_along_axis(qb, arg[..., None], axis=2)[..., 0]
    assert np.all(np.abs(top[nz]) == 127)
    assert np.all(np.sign(qb) * np.sign(xb) >= 0)
    assert np.all(np.abs(qb) <= 127)
    # the zero block
    assert d[3, 1] == 0 and np.all(q[3, 32:64] == 0)


def test_q8_0_exact_multiples_roundtrip(oracle_lib):
    """Blocks whose values are integer multiples of a power-of-two step with a +-127
    extreme reproduce exactly: d is the step and q the multiples."""
    rng = np.random.default_rng(11)
    for e in range(-6, 7):
        step = 2.0 ** e
        m = rng.integers(-127, 128, (4, 32))
        m[:, 5] = 127 * np.where(rng.random(4) < 0.5, -1, 1)
        x = (m * step).astype(np.float32)
        q, d = oracle_lib.quantize_q8_0(x)
        assert np.all(d == np.float32(step))
        assert np.array_equal(q.astype(np.int64), m)
