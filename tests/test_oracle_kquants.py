"""Pins for the oracle's K-quant decoding (Q4_K and Q6_K: the GGUF super-block
formats the imp engine loads -- imp README, "Features" table, Quantization
row; imp release notes v0.7.0, Q4_K_M -- named but not defined on the pages;
their public definitions are restated in oracle.c).

Each pin reaches the expected weights by another route than the K-quant
decoder: super-blocks whose scales make them equal to Q4_0 or Q8_0 blocks
(formats pinned on their own in tests/test_oracle.py) are decoded both ways;
zeros and extreme codes have closed forms; sums are checked exactly with
rationals.  The tests build the super-block bytes field by field from the
layout (which bytes and bits hold which weight); the values they expect come
from the other formats' decoders or from closed forms."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl


from kq_blocks import q4_0_block, q4k_block, q6k_block, q6k_scale_index, q8_0_block


# --------------------------------------------------------------- Q4_K
@pytest.mark.parametrize("low,high,dmin_over_d,q40_scales", [
    # sub-blocks 0..3 (sc, m) and 4..7 (sc, m); every sub-block is d_j * (q - 8)
    ((1, 2), (16, 32), 4, (1, 16)),     # the high two bits of scale and min (sub-blocks 4..7)
    ((1, 2), (3, 6), 4, (1, 3)),        # the low nibbles of scale and min (sub-blocks 4..7)
    ((5, 40), (2, 16), 1, (5, 2)),      # six-bit mins for sub-blocks 0..3
])
def test_q4k_reduces_to_q4_0(low, high, dmin_over_d, q40_scales):
    """With dmin * m_j = 8 * d * sc_j every weight is d sc_j (q - 8): a Q4_0
    block of scale d sc_j with the same codes."""
    rng = np.random.default_rng(31)
    d = 2.0 ** -8
    n, k = 2, 512
    rows_k, rows_0 = [], []
    for r in range(n):
        sbs_k, sbs_0 = [], []
        for s in range(k // 256):
            codes = rng.integers(0, 16, size=256)
            scmin = [low] * 4 + [high] * 4
            sbs_k.append(q4k_block(d, d * dmin_over_d, scmin, codes))
            for j in range(8):
                sbs_0.append(q4_0_block(d * q40_scales[j // 4], codes[32 * j:32 * j + 32]))
        rows_k.append(np.concatenate(sbs_k))
        rows_0.append(np.concatenate(sbs_0))
    wk = oracle.decode(oracle.Q4_K, np.concatenate(rows_k), n, k)
    w0 = oracle.decode(oracle.Q4_0, np.concatenate(rows_0), n, k)
    assert np.array_equal(wk, w0)


def test_q4k_single_codes_land_in_place():
    """One nonzero code at a time (scale 1, min 0, d 1): exactly that weight is
    nonzero and equals the code."""
    for i in [0, 1, 31, 32, 33, 63, 64, 100, 127, 128, 191, 192, 255]:
        codes = np.zeros(256, dtype=np.int64)
        codes[i] = 13
        w = oracle.decode(oracle.Q4_K, q4k_block(1.0, 0.0, [(1, 0)] * 8, codes), 1, 256)[0]
        assert w[i] == 13.0 and np.count_nonzero(w) == 1, i


def test_q4k_closed_forms():
    codes = np.random.default_rng(32).integers(0, 16, size=256)
    # zero scales and mins: all weights zero
    w = oracle.decode(oracle.Q4_K, q4k_block(0.5, 0.25, [(0, 0)] * 8, codes), 1, 256)[0]
    assert np.array_equal(w, np.zeros(256))
    # scales zero, mins set: w = -dmin * m_j, independent of the codes
    scmin = [(0, m) for m in (1, 2, 3, 63, 4, 5, 6, 7)]
    w = oracle.decode(oracle.Q4_K, q4k_block(0.5, 0.25, scmin, codes), 1, 256)[0]
    assert np.array_equal(w, np.repeat([-0.25 * m for _, m in scmin], 32))
    # largest fields: sc = m = 63, q = 15 and q = 0
    w = oracle.decode(oracle.Q4_K, q4k_block(1.0, 1.0, [(63, 63)] * 8, np.full(256, 15)), 1, 256)[0]
    assert np.all(w == 63 * 15 - 63)
    w = oracle.decode(oracle.Q4_K, q4k_block(1.0, 1.0, [(63, 63)] * 8, np.zeros(256)), 1, 256)[0]
    assert np.all(w == -63)
    # d * sc * q == dmin * m: exact zeros for that code only
    w = oracle.decode(oracle.Q4_K, q4k_block(2.0 ** -6, 2.0 ** -6, [(3, 27)] * 8, codes), 1, 256)[0]
    assert np.array_equal(w == 0, codes == 9)


# --------------------------------------------------------------- Q6_K
@pytest.mark.parametrize("seed", [33, 34])
def test_q6k_reduces_to_q8_0(seed):
    """With scales 1..3 every weight d * s * (q - 32) is an int8 times d: a
    Q8_0 block of scale d whose codes are s * (q - 32)."""
    rng = np.random.default_rng(seed)
    d = -(2.0 ** -10) if seed == 34 else 2.0 ** -9
    n, k = 2, 512
    rows_6, rows_8 = [], []
    for r in range(n):
        sb6, sb8 = [], []
        for s in range(k // 256):
            q = rng.integers(0, 64, size=256)
            q[:4] = [0, 63, 32, 31]
            sc = rng.integers(1, 4, size=16) * rng.choice([-1, 1], size=16)
            sb6.append(q6k_block(d, sc, q))
            c = np.array([sc[q6k_scale_index(i)] * (int(q[i]) - 32) for i in range(256)])
            for j in range(8):
                sb8.append(q8_0_block(d, c[32 * j:32 * j + 32]))
        rows_6.append(np.concatenate(sb6))
        rows_8.append(np.concatenate(sb8))
    w6 = oracle.decode(oracle.Q6_K, np.concatenate(rows_6), n, k)
    w8 = oracle.decode(oracle.Q8_0, np.concatenate(rows_8), n, k)
    assert np.array_equal(w6, w8)


def test_q6k_closed_forms():
    rng = np.random.default_rng(35)
    sc = rng.integers(-128, 128, size=16)
    # code 32 is zero whatever the scale
    w = oracle.decode(oracle.Q6_K, q6k_block(0.75, sc, np.full(256, 32)), 1, 256)[0]
    assert np.array_equal(w, np.zeros(256))
    # extreme codes and scales: -32 * -128 and 31 * 127
    w = oracle.decode(oracle.Q6_K, q6k_block(1.0, np.full(16, -128), np.zeros(256)), 1, 256)[0]
    assert np.all(w == 4096)
    w = oracle.decode(oracle.Q6_K, q6k_block(-1.0, np.full(16, 127), np.full(256, 63)), 1, 256)[0]
    assert np.all(w == -31 * 127)
    # one nonzero code (q = 33) at a time, unit scales: exactly that weight is d
    for i in [0, 15, 16, 31, 32, 64, 96, 127, 128, 160, 200, 255]:
        q = np.full(256, 32)
        q[i] = 33
        w = oracle.decode(oracle.Q6_K, q6k_block(0.5, np.ones(16), q), 1, 256)[0]
        assert w[i] == 0.5 and np.count_nonzero(w) == 1, i


def test_sizes():
    """4.5 and 6.5625 bits per weight."""
    assert oracle.tensor_bytes(oracle.Q4_K, 3, 512) * 8 == 3 * 512 * 4.5
    assert oracle.tensor_bytes(oracle.Q6_K, 3, 512) * 8 == 3 * 512 * 6.5625
    with pytest.raises(ValueError):
        oracle.tensor_bytes(oracle.Q4_K, 3, 96)          # not a whole super-block
    assert wl.canon_bytes(wl.FMT_Q4_K, 3, 512) == oracle.tensor_bytes(oracle.Q4_K, 3, 512)
    assert wl.canon_bytes(wl.FMT_Q6_K, 3, 512) == oracle.tensor_bytes(oracle.Q6_K, 3, 512)


# --------------------------------------------------------------- products
@pytest.mark.parametrize("fmt", [oracle.Q4_K, oracle.Q6_K])
@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
def test_brute_force_exact_sums(fmt, xt):
    """y and l1 against exact rational sums of the decoded weights."""
    n, k, m = 2, 256, 2
    blocks = wl.blocks_for(fmt, n, k, config=94, matrix=fmt)
    rng = wl.rng_for(94, 1, "x")
    x = wl.x_f32((m, k), rng) if xt == oracle.X_F32 else wl.x_bf16_bits((m, k), rng)
    y, l1 = oracle.gemv(fmt, blocks, n, k, x, xt)
    w = oracle.decode(fmt, blocks, n, k)
    xs = x.astype(np.float64) if xt == oracle.X_F32 else (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for t in range(m):
        for r in range(n):
            prods = [Fraction(float(w[r, c])) * Fraction(float(xs[t, c])) for c in range(k)]
            exact = sum(prods, Fraction(0))
            a = sum((abs(p) for p in prods), Fraction(0))
            assert abs(Fraction(y[t, r]) - exact) <= Fraction(1, 2 ** 50) * a
            assert abs(Fraction(l1[t, r]) - a) <= Fraction(1, 2 ** 50) * a


@pytest.mark.parametrize("fmt", [oracle.Q4_K, oracle.Q6_K])
def test_all_equal_rows_closed_form(fmt):
    """Rows whose weights are all equal give w * sum(x)."""
    n, k = 3, 768
    if fmt == oracle.Q4_K:
        sb = q4k_block(2.0 ** -7, 2.0 ** -9, [(5, 3)] * 8, np.full(256, 11))
        wv = 2.0 ** -7 * 5 * 11 - 2.0 ** -9 * 3
    else:
        sb = q6k_block(2.0 ** -8, np.full(16, -7), np.full(256, 45))
        wv = 2.0 ** -8 * -7 * (45 - 32)
    blocks = np.tile(sb, n * k // 256)
    x = wl.x_f32((1, k), np.random.default_rng(36))
    y, _ = oracle.gemv(fmt, blocks, n, k, x, oracle.X_F32)
    ref = float(sum(Fraction(float(v)) for v in x[0]) * Fraction(wv))
    assert np.allclose(y, ref, rtol=1e-14, atol=0)
