"""Pins for the oracle's NVFP4 functions (the format of imp's decode cache and
sm_120a GEMV: imp README, "Why this exists" and the "Features" table; the
pages name it, its definition is the public one).  Each check reaches the
expected value by another route: torch's own float8_e4m3fn type, literal
values, exact rational sums, nearest-value searches written here over the
format's value list, and round trips of tensors that are exactly
representable."""
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")

E2M1_MAG = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _torch_e4m3(codes):
    """fp64 values of E4M3 bytes through torch's float8_e4m3fn."""
    t = torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_round_e4m3(v):
    """fp32 -> E4M3 byte through torch's conversion (round to nearest even)."""
    t = torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_all_patterns_match_torch():
    ref = _torch_e4m3(np.arange(256))
    got = np.array([oracle.e4m3(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2                     # 0x7F and 0xFF only: no infinities
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.e4m3(0x7E) == 448.0 and oracle.e4m3(0x01) == 2.0 ** -9 and oracle.e4m3(0x38) == 1.0


def test_e4m3_rounding_matches_torch_in_range():
    rng = np.random.default_rng(5)
    vals = np.concatenate([rng.uniform(0, 448, 4000), 2.0 ** rng.uniform(-12, 8.8, 4000)]).astype(np.float32)
    grid = np.array([oracle.e4m3(c) for c in range(0x7F)])
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)      # exact ties (all exact in fp32)
    vals = np.concatenate([vals, mids, grid.astype(np.float32)])
    vals = vals[vals <= 448]
    want = _torch_round_e4m3(vals)
    got = np.array([oracle.e4m3_round(v) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_rounding_saturates():
    for v in (448.0, 449.0, 463.9, 464.0, 500.0, 1e30):
        assert oracle.e4m3_round(v) == 0x7E


def test_e2m1_rounding_literals():
    cases = {0.0: 0, 0.2: 0, 0.25: 0, 0.26: 1, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 2.6: 5, 3.5: 6, 5.0: 6,
             5.01: 7, 6.0: 7, 100.0: 7, -0.1: 0, -0.25: 0, -0.3: 9, -3.0: 13, -7.0: 15}
    for r, c in cases.items():
        assert oracle.e2m1_round(r) == c, r


def test_e2m1_rounding_is_nearest():
    rng = np.random.default_rng(6)
    for r in rng.uniform(-8, 8, 3000).astype(np.float32):
        c = oracle.e2m1_round(r)
        got = oracle.e2m1(c)
        best = min(abs(m - abs(r)) for m in E2M1_MAG)
        assert abs(abs(got) - abs(r)) == pytest.approx(best, abs=0)
        assert (got < 0) == (r < 0 and got != 0)


def _hand_tensor():
    """Two rows x 32: row 0 block 0 scale 1.0 (0x38) codes 0..15, block 1
    scale 0.5 (0x30) all code 7 (6.0); row 1 block 0 scale 2^-9 (0x01) code 1
    (0.5), block 1 scale 448 (0x7E) code 15 (-6); tensor scale 0.25."""
    def blk(s, codes):
        return bytes([s]) + bytes(codes[j] | (codes[j + 8] << 4) for j in range(8))
    data = (blk(0x38, list(range(16))) + blk(0x30, [7] * 16) + blk(0x01, [1] * 16) + blk(0x7E, [15] * 16)
            + struct.pack("<f", 0.25))
    return np.frombuffer(data, dtype=np.uint8)


def test_hand_built_tensor_decodes():
    w = oracle.decode(oracle.NVFP4, _hand_tensor(), 2, 32)
    e2m1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    row0 = [(-1 if c >= 8 else 1) * e2m1[c & 7] * 0.25 for c in range(16)] + [6.0 * 0.5 * 0.25] * 16
    row1 = [0.5 * 2.0 ** -9 * 0.25] * 16 + [-6.0 * 448 * 0.25] * 16
    assert np.array_equal(w[0], np.array(row0))
    assert np.array_equal(w[1], np.array(row1))


@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
def test_brute_force_exact_sums(xt):
    n, k, m = 3, 64, 2
    t = wl.nvfp4_tensor(n, k, wl.rng_for(92, 0, "codes"), wl.rng_for(92, 0, "scales"))
    rng = wl.rng_for(92, 1, "x")
    x = wl.x_f32((m, k), rng) if xt == oracle.X_F32 else wl.x_bf16_bits((m, k), rng)
    y, l1 = oracle.gemv(oracle.NVFP4, t, n, k, x, xt)
    ts = Fraction(float(np.frombuffer(t[-4:].tobytes(), dtype=np.float32)[0]))
    body = t[:-4].reshape(n, k // 16, 9)
    if xt == oracle.X_F32:
        X = [Fraction(float(v)) for v in x.reshape(-1)]
    else:
        X = [Fraction(struct.unpack("<f", struct.pack("<I", int(v) << 16))[0]) for v in x.reshape(-1)]
    for r in range(n):
        W = []
        for b in range(k // 16):
            sc = Fraction(float(_torch_e4m3([body[r, b, 0]])[0]))
            for i in range(16):
                byte = int(body[r, b, 1 + (i & 7)])
                c = byte & 15 if i < 8 else byte >> 4
                W.append((-1 if c >= 8 else 1) * Fraction(E2M1_MAG[c & 7]) * sc * ts)
        for tok in range(m):
            prods = [W[c] * X[tok * k + c] for c in range(k)]
            exact = sum(prods, Fraction(0))
            a = sum((abs(p) for p in prods), Fraction(0))
            assert abs(Fraction(y[tok, r]) - exact) <= Fraction(1, 2 ** 50) * a
            assert abs(Fraction(l1[tok, r]) - a) <= Fraction(1, 2 ** 50) * a


def test_moe_accepts_nvfp4_experts():
    E, n, k = 3, 16, 64
    ex = np.concatenate([wl.nvfp4_tensor(n, k, wl.rng_for(93, e, "codes"), wl.rng_for(93, e, "scales"))
                         for e in range(E)])
    ids = np.array([[2, 0]], dtype=np.int32)
    g = np.array([[0.75, 0.25]], dtype=np.float32)
    h = wl.x_f32((1, 2, k), wl.rng_for(93, 9, "h"))
    y, _ = oracle.moe(oracle.NVFP4, ex, E, n, k, ids, g, h, oracle.X_F32, oracle.MOE_DOWN)
    per = oracle.tensor_bytes(oracle.NVFP4, n, k)
    want = 0.75 * oracle.gemv(oracle.NVFP4, ex[2 * per:3 * per], n, k, h[0, 0], oracle.X_F32)[0] + \
        0.25 * oracle.gemv(oracle.NVFP4, ex[0:per], n, k, h[0, 1], oracle.X_F32)[0]
    assert np.allclose(y, want, rtol=1e-14, atol=0)


# ------------------------------------------------------------------ quantizer
def _representable(n, k, rng):
    """A tensor every value of which is exactly E2M1(c) * E4M3(s) * ts with a
    power-of-two ts, each block holding +-6 * its scale and one block with the
    largest scale 448: quantizing it must give back exactly these codes."""
    ts = 2.0 ** -10
    nb = k // 16
    codes = rng.integers(0, 16, size=(n, nb, 16), dtype=np.uint8)
    codes[codes == 8] = 0                     # the quantizer writes +0 for zero
    codes[:, :, 3] = np.where(rng.random((n, nb)) < 0.5, 7, 15)     # +-6 in every block
    sc = rng.integers(0x20, 0x70, size=(n, nb), dtype=np.uint8)
    sc[0, 0] = 0x7E
    w = np.empty((n, k), dtype=np.float64)
    for r in range(n):
        for b in range(nb):
            s = oracle.e4m3(sc[r, b])
            for i in range(16):
                c = int(codes[r, b, i])
                w[r, 16 * b + i] = (-1 if c >= 8 else 1) * E2M1_MAG[c & 7] * s * ts
    return w.astype(np.float32), codes, sc, ts


def test_quantizer_round_trips_representable_tensors():
    n, k = 5, 96
    w, codes, sc, ts = _representable(n, k, np.random.default_rng(7))
    t = oracle.nvfp4_quantize(w)
    assert np.frombuffer(t[-4:].tobytes(), dtype=np.float32)[0] == np.float32(ts)
    body = t[:-4].reshape(n, k // 16, 9)
    assert np.array_equal(body[:, :, 0], sc)
    got = np.concatenate([body[:, :, 1:] & 15, body[:, :, 1:] >> 4], axis=2)
    assert np.array_equal(got, codes)
    assert np.array_equal(oracle.decode(oracle.NVFP4, t, n, k), w.astype(np.float64))


def test_quantizer_block_scales_match_torch_rounding():
    """Each block scale is torch's E4M3 rounding of (max|w| / 6) / s_t, taken in fp32."""
    n, k = 7, 128
    w = (np.random.default_rng(8).standard_normal((n, k)) * 10.0 ** np.random.default_rng(9).uniform(
        -3, 1, size=(n, 1))).astype(np.float32)
    t = oracle.nvfp4_quantize(w)
    st = np.float32(np.abs(w).max() / np.float32(2688.0))
    assert np.frombuffer(t[-4:].tobytes(), dtype=np.float32)[0] == st
    amax = np.abs(w.reshape(n, k // 16, 16)).max(axis=2).astype(np.float32)
    v = (amax / np.float32(6.0)).astype(np.float32) / st
    want = _torch_round_e4m3(np.minimum(v, np.float32(448.0)))
    assert np.array_equal(t[:-4].reshape(n, k // 16, 9)[:, :, 0], want)


def test_quantizer_error_bound():
    """Every decoded value is the nearest point of the block's grid
    E2M1 * S (or its end, +-6 S): |w - w'| <= half the local grid spacing."""
    n, k = 6, 160
    rng = np.random.default_rng(10)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    t = oracle.nvfp4_quantize(w)
    wq = oracle.decode(oracle.NVFP4, t, n, k)
    st = float(np.frombuffer(t[-4:].tobytes(), dtype=np.float32)[0])
    body = t[:-4].reshape(n, k // 16, 9)
    for r in range(n):
        for b in range(k // 16):
            S = oracle.e4m3(body[r, b, 0]) * st
            for i in range(16):
                a = abs(float(w[r, 16 * b + i]))
                pts = [m * S for m in E2M1_MAG]
                best = min(abs(p - a) for p in pts)
                assert abs(abs(wq[r, 16 * b + i]) - a) <= best * (1 + 1e-6) + 1e-30
