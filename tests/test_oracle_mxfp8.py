"""Pins for the oracle's MXFP8 Step 5 (the FP8 fused projection).

E4M3 rounding is checked against brute force over the decoded code table
(which is a separate bit-field decoder), the block scale against its
defining property, and the MXFP8 product against exact arithmetic on the
dequantised operands."""
import numpy as np

from oracle import engram_oracle as orc


def _table():
    codes = np.array([c for c in range(256) if (c & 0x7f) != 0x7f], dtype=np.uint8)   # no NaN
    vals = orc.e4m3_decode(codes)
    return codes, vals


def test_e4m3_decode_fixed_points_and_range():
    codes, vals = _table()
    pos = np.unique(vals[vals >= 0])
    assert pos.shape[0] == 127 and pos.max() == 448.0 and pos[1] == 2.0 ** -9   # 0, 7 subnormals, 119 normals
    assert np.array_equal(orc.round_to_e4m3(vals), vals)
    assert np.array_equal(orc.e4m3_decode(orc.e4m3_encode(vals)), vals)


def test_round_to_e4m3_is_nearest_even_by_brute_force():
    codes, vals = _table()
    pos_codes = codes[vals >= 0]
    pos_vals = vals[vals >= 0]
    keep = np.unique(pos_vals, return_index=True)[1]
    grid, gcodes = pos_vals[keep], pos_codes[keep]
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.uniform(0, 448, 20000), rng.uniform(0, 2.0 ** -5, 5000),
                        (grid[1:] + grid[:-1]) / 2])                      # every midpoint: a tie
    i = np.clip(np.searchsorted(grid, x), 1, grid.shape[0] - 1)
    lo, hi = grid[i - 1], grid[i]
    tie = (x - lo) == (hi - x)
    even_hi = (gcodes[i] & 1) == 0
    want = np.where(tie, np.where(even_hi, hi, lo), np.where(x - lo < hi - x, lo, hi))
    assert np.array_equal(orc.round_to_e4m3(x), want)
    assert np.array_equal(orc.round_to_e4m3(-x), -want)


def test_block_scale_is_the_smallest_power_of_two_that_fits():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((300, 64)) * np.exp2(rng.integers(-20, 20, (300, 1)))
    x[7, :32] = 0.0                                   # an all-zero block
    x[8, :32] = 0.0
    x[8, 5] = 448.0                                   # amax exactly 448: scale 2^0
    x[9, :32] = 0.0
    x[9, 3] = -449.0                                  # just above: scale 2^1
    q, s = orc.quantize_mxfp8(x)
    assert s[7, 0] == 0 and np.all(q[7, :32] == 0)
    assert s[8, 0] == 127 and s[9, 0] == 128
    blocks = x.reshape(300, 2, 32)
    amax = np.abs(blocks).max(axis=-1)
    nz = amax > 0
    scale = np.ldexp(1.0, s.astype(np.int64) - 127)
    assert np.all(amax[nz] <= 448 * scale[nz])          # fits
    assert np.all(amax[nz] > 224 * scale[nz])           # and half the scale would not
    deq = orc.dequantize_mxfp8(q, s)
    # nearest-even E4M3 of v / scale: within half a quantum, never saturated
    err = np.abs(deq - x).reshape(300, 2, 32)
    v = np.abs(x).reshape(300, 2, 32) / scale[..., None]
    quantum = np.ldexp(1.0, np.maximum(np.floor(np.log2(np.where(v > 0, v, 1.0))), -6).astype(np.int64) - 3)
    assert np.all(err <= quantum / 2 * scale[..., None] * (1 + 1e-12))


def test_mxfp8_product_is_exact_on_the_dequantised_operands():
    rng = np.random.default_rng(14)
    e = rng.standard_normal((5, 128)) * 0.02
    w = rng.standard_normal((7, 128)) / 32
    kv = orc.project_kv_mxfp8(e, w)
    eq, es = orc.quantize_mxfp8(e)
    wq, ws = orc.quantize_mxfp8(w)
    a, b = orc.dequantize_mxfp8(eq, es), orc.dequantize_mxfp8(wq, ws)
    # a brute-force sum of exact products (all operands are small dyadic rationals)
    from fractions import Fraction
    for i in range(5):
        for j in range(7):
            exact = sum(Fraction(float(a[i, k])) * Fraction(float(b[j, k])) for k in range(128))
            assert abs(float(exact) - kv[i, j]) <= 1e-15 * max(1.0, abs(float(exact)))
    # and close to the unquantised product (4 significant bits per operand)
    ref = e @ w.T
    assert np.max(np.abs(kv - ref)) < 0.08 * np.max(np.abs(ref))
