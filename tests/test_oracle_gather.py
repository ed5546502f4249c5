"""Pins for the oracle's Steps 3-4 (table lookup, concatenation, dequantise).

The tables are filled with values that encode their own address, so the
gathered vector can be decoded back to (table, row, column) independently of
the gather code; dequantisation is checked on hand-worked IEEE cases.
"""
import numpy as np

from hashed_gram_embedding_amd import inputs
from oracle import engram_oracle as orc


def _coded_tables(dim=16):
    w = inputs.make_config(0, table_dim=dim)
    tab = w.layers[0].tables
    g = np.arange(tab.total_rows, dtype=np.float32)[:, None] * dim + np.arange(dim, dtype=np.float32)
    return w, tab, g      # value = global_row * dim + column, exact in float32


def test_concat_order_and_offsets_decode():
    """Segment j of e_t is row z_{t,j} of table j = (n-2)K + k, n outer, k
    inner (Step 4), with table j starting at row_offset[j]."""
    for dim in (16, 8):
        w, tab, coded = _coded_tables(dim)
        hp = w.layers[0].hash
        z = orc.hash_indices(w.tokens, hp.proj, hp.mult, hp.prime, 3, hp.heads)
        e = orc.gather(z, coded, "f32", tab.row_offset, dim, out_dtype="f32")
        assert e.shape == (1, 64, 4 * dim)
        for t in range(64):
            for n in (2, 3):
                for k in range(hp.heads):
                    j = (n - 2) * hp.heads + k
                    seg = e[0, t, j * dim:(j + 1) * dim]
                    row = seg[0] // dim
                    assert np.array_equal(seg % dim, np.arange(dim))
                    # decoded global row lies in table j and equals its offset + z
                    assert tab.row_offset[j] <= row < tab.row_offset[j] + tab.n_rows[j]
                    assert row == tab.row_offset[j] + z[0, t, j]


def test_bf16_rows_copy_bit_exact():
    rows = np.array([[0x3F80, 0xBF80, 0x0001, 0x7F7F], [0x4049, 0x0000, 0x8000, 0x3C00]], dtype=np.uint16)
    e = orc.gather(np.array([[1, 0]]), rows, "bf16", np.array([0, 0]), 4, out_dtype="bf16")
    want = [3.140625, 0.0, -0.0, 2.0 ** -7, 1.0, -1.0, 2.0 ** -133, 3.3895313892515355e38]
    assert e.shape == (1, 8)
    assert np.array_equal(e[0], np.array(want))
    assert np.signbit(e[0, 2])


def test_int8_dequant_hand_cases():
    """float32(q) * float32(scale), one IEEE multiply, then nearest-even bf16."""
    q = np.array([[127, -127, 3, 0], [1, 1, 1, 1], [3, 3, 3, 3]], dtype=np.int8)
    scale = np.array([0.5,
                      1.0 + 2.0 ** -8,          # exact tie between 1 and 1+2^-7: even is 1
                      np.float32(1.0 / 3.0)],   # 3 * fl(1/3) = 1 + 2^-25 -> float32 rounds to 1
                     dtype=np.float32)
    off = np.zeros(2, dtype=np.int64)
    e32 = orc.gather(np.array([[0, 0]]), q, "i8", off, 4, scale, out_dtype="f32")
    assert np.array_equal(e32[0, :4], [63.5, -63.5, 1.5, 0.0])
    rows1 = orc.table_rows_f64(q, "i8", np.array([1]), scale, "f32")
    assert rows1[0, 0] == 1.0 + 2.0 ** -8
    assert orc.table_rows_f64(q, "i8", np.array([1]), scale, "bf16")[0, 0] == 1.0
    assert orc.table_rows_f64(q, "i8", np.array([2]), scale, "f32")[0, 0] == 1.0
    # ties of the bf16 rounding: 1 + 3*2^-8 lies halfway between 1+2^-7 (odd) and 1+2^-6 (even)
    s2 = np.array([1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -(1.0 + 3 * 2.0 ** -8)], dtype=np.float32)
    got = orc.table_rows_f64(np.ones((3, 1), np.int8), "i8", np.arange(3), s2, "bf16")[:, 0]
    assert np.array_equal(got, [1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -6)])


def test_round_f32_to_bf16_against_nextafter_bracketing():
    """Nearest-even rounding: the result is one of the two bf16 neighbours and
    is the nearer one; exact ties go to the even mantissa."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * rng.choice([1e-3, 1.0, 1e4], 20000)).astype(np.float32)
    r = orc.round_f32_to_bf16(x)
    u = x.view(np.uint32)
    lo = (u & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)      # truncation toward 0
    hi_bits = (u & np.uint32(0xFFFF0000)) + np.uint32(0x10000)
    hi = hi_bits.view(np.float32).astype(np.float64)                          # next bf16 away from 0
    xd = x.astype(np.float64)
    d_lo, d_hi = np.abs(xd - lo), np.abs(hi - xd)
    nearer = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    even = np.where(((u >> np.uint32(16)) & np.uint32(1)) == 0, lo, hi)
    want = np.where(tie, even, nearer)
    assert np.array_equal(r, want)


def test_int8_quantisation_input_roundtrip_bound():
    """Input preparation check: |q*scale - x| <= scale/2 per element."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((500, 64)) * 0.02).astype(np.float32)
    q, s = inputs.quantize_rows_int8(x)
    back = q.astype(np.float64) * s[:, None]
    assert np.all(np.abs(back - x) <= s[:, None] / 2 * (1 + 1e-6))
    assert np.all(np.abs(q).max(axis=1) == 127)


def test_lfu_admission_hand_example():
    """Counts per row [5, 3, 3, 3, 1, 0, 3]: the 4 most frequent are row 0 and
    the three lowest rows of count 3 (1, 2, 3); row 6 (also 3) loses the tie.
    Slots follow ascending row order."""
    rows = [0] * 5 + [1] * 3 + [2] * 3 + [3] * 3 + [4] + [6] * 3
    slot = orc.lfu_admission(np.array(rows), 7, 4)
    assert list(slot) == [0, 1, 2, 3, -1, -1, -1]
    assert list(orc.lfu_admission(np.array(rows), 7, 0)) == [-1] * 7
    assert list(orc.lfu_admission(np.array(rows), 7, 7)) == [0, 1, 2, 3, 4, 5, 6]
    # zero-count rows fill the cache last, lowest first
    assert list(orc.lfu_admission(np.array([6, 6]), 7, 3)) == [0, 1, -1, -1, -1, -1, 2]


def test_lfu_update_hand_example():
    """counts [5, 3, 3, 3, 1, 0, 3]; rows 0, 4, 6 cached in slots 2, 0, 1 of a
    4-slot cache.  Admitted: row 0 and the three lowest rows of count 3 (1, 2,
    3).  Row 0 keeps slot 2; rows 4 and 6 leave; the free slots 0, 1, 3 go to
    rows 1, 2, 3 in that order.  Aging by one bit halves the counts."""
    counts = np.array([5, 3, 3, 3, 1, 0, 3])
    prev = np.array([2, -1, -1, -1, 0, -1, 1])
    slot, aged = orc.lfu_update(counts, prev, 4, decay_shift=1)
    assert list(slot) == [2, 0, 1, 3, -1, -1, -1]
    assert list(aged) == [2, 1, 1, 1, 0, 0, 1]
    slot0, same = orc.lfu_update(counts, prev, 4)
    assert list(slot0) == list(slot) and list(same) == list(counts)


def test_lfu_update_from_empty_equals_static_admission():
    rng = np.random.default_rng(8)
    rows = rng.zipf(1.3, 5000) % 400
    counts = np.bincount(rows, minlength=400)
    for n in (0, 1, 37, 400):
        slot, _ = orc.lfu_update(counts, np.full(400, -1), n)
        assert np.array_equal(slot, orc.lfu_admission(rows, 400, n))


def test_lfu_update_invariants_under_drift():
    """Random drift: the admitted set is the top cache_n by (count, -row);
    slots form a permutation of 0..n-1; stayers never move."""
    rng = np.random.default_rng(9)
    total, n = 300, 40
    slot = np.full(total, -1)
    counts = np.zeros(total, dtype=np.int64)
    for step in range(6):
        counts = counts + np.bincount(rng.integers(0, total, 500) ** 2 % total, minlength=total)
        new, counts_after = orc.lfu_update(counts, slot, n, decay_shift=1)
        order = np.lexsort((np.arange(total), -counts))
        assert set(np.nonzero(new >= 0)[0]) == set(order[:n])
        assert sorted(new[new >= 0]) == list(range(n))
        stay = (slot >= 0) & (new >= 0)
        assert np.array_equal(new[stay], slot[stay])
        slot, counts = new, counts_after
