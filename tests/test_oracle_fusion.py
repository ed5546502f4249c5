"""Pins for the oracle's Steps 5-7 (projections, gate, short conv).

Closed forms, Cauchy-Schwarz bounds, basis-vector probes and a second route
for the dilated conv (numpy.convolve with a zero-stuffed kernel).
"""
import numpy as np

from oracle import engram_oracle as orc


def test_projection_basis_vectors_return_weight_columns():
    """e = unit vector i gives [v|k] = column i of the stacked W (Step 5);
    catches a transposed operand for any non-square W."""
    rng = np.random.default_rng(1)
    W = rng.standard_normal((3 * 5, 7))
    kv = orc.project_kv(np.eye(7), W)
    assert kv.shape == (7, 15)
    for i in range(7):
        assert np.array_equal(kv[i], W[:, i])


def test_rmsnorm_closed_form():
    x = np.array([3.0, 4.0])
    assert np.allclose(orc.rmsnorm(x, 0.0), x / np.sqrt(12.5), rtol=0, atol=1e-15)
    assert np.array_equal(orc.rmsnorm(np.zeros(5), 1e-6), np.zeros(5))
    y = orc.rmsnorm(np.array([2.0, -2.0, 2.0, -2.0]), 1e-6)
    assert np.allclose(y, np.array([1, -1, 1, -1]) * 2 / np.sqrt(4 + 1e-6), rtol=0, atol=1e-15)


def test_gate_closed_forms():
    """h = k = ones: RMSNorm gives ones/sqrt(1+eps), the dot is d/(1+eps), the
    logit sqrt(d)/(1+eps) (Step 6); h = -k flips the sign; k = 0 gives 1/2."""
    for d in (4, 64, 1024):
        eps = 1e-6
        one = np.ones(d)
        want = 1 / (1 + np.exp(-np.sqrt(d) / (1 + eps)))
        assert abs(orc.gate(one, one, eps) - want) < 1e-15
        assert abs(orc.gate(-one, one, eps) - (1 - want)) < 1e-15
        assert orc.gate(np.arange(d, dtype=float), np.zeros(d), eps) == 0.5


def test_gate_range_bound_and_scale_invariance():
    rng = np.random.default_rng(2)
    d = 256
    h = rng.standard_normal((1000, d))
    k = rng.standard_normal((1000, d))
    a = orc.gate(h, k, 1e-6)
    assert np.all((a > 0) & (a < 1))
    logit = np.log(a / (1 - a))
    assert np.all(np.abs(logit) <= np.sqrt(d) * (1 + 1e-9))       # Cauchy-Schwarz
    # positive rescaling of h or k leaves alpha unchanged up to eps
    assert np.allclose(orc.gate(7.0 * h, k, 1e-6), a, rtol=0, atol=1e-6)
    assert np.allclose(orc.gate(h, 0.1 * k, 1e-6), a, rtol=0, atol=1e-4)
    assert np.allclose(orc.gate(h, 0.1 * k, 0.0), orc.gate(h, k, 0.0), rtol=0, atol=1e-14)
    # fully aligned h and k reach the bound
    assert abs(orc.gate(k[0], 3 * k[0], 0.0) - 1 / (1 + np.exp(-np.sqrt(d)))) < 1e-12


def test_silu_closed_form():
    assert orc.silu(0.0) == 0.0
    assert abs(orc.silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16
    assert abs(orc.silu(-1.0) + 1.0 / (1.0 + np.e)) < 1e-16


def test_short_conv_equals_numpy_convolve_zero_stuffed():
    """c_t = sum_j w[j] u_{t-(3-j)*3}: numpy.convolve with the kernel
    [w3, 0, 0, w2, 0, 0, w1, 0, 0, w0] gives the same causal result."""
    rng = np.random.default_rng(3)
    T, d, dil = 50, 6, 3
    u = rng.standard_normal((T, d))
    w = rng.standard_normal((d, 4))
    c = orc.short_conv(u, w, dil)
    for ch in range(d):
        stuffed = np.zeros(3 * dil + 1)
        for j in range(4):
            stuffed[(3 - j) * dil] = w[ch, j]
        ref = np.convolve(u[:, ch], stuffed)[:T]
        assert np.allclose(c[:, ch], ref, rtol=0, atol=1e-13)


def test_short_conv_impulse_and_causality():
    """An impulse at s lands at s, s+3, s+6, s+9 only, weighted w3, w2, w1, w0
    (receptive field 1 + (w-1)N = 10, Step 7)."""
    T, d = 30, 2
    w = np.array([[0.1, 0.2, 0.3, 0.4], [-1.0, 2.0, -3.0, 4.0]])
    for s in (0, 7, 25):
        u = np.zeros((T, d))
        u[s] = 1.0
        c = orc.short_conv(u, w, 3)
        nz = sorted(set(np.nonzero(c)[0]))
        assert nz == [t for t in (s, s + 3, s + 6, s + 9) if t < T]
        for j, t in enumerate((s + 9, s + 6, s + 3, s)):
            if t < T:
                assert np.array_equal(c[t], w[:, j])


def test_short_conv_state_continues_sequence():
    rng = np.random.default_rng(4)
    u = rng.standard_normal((40, 3))
    w = rng.standard_normal((3, 4))
    full = orc.short_conv(u, w, 3)
    part = orc.short_conv(u[25:], w, 3, prev=u[16:25])
    assert np.allclose(part, full[25:], rtol=0, atol=1e-14)
