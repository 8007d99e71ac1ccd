"""Pins for the fp64 oracle: each check reaches the expected value by a route
other than the oracle's own code (library routines, literal values, exact
rational arithmetic, closed forms, page facts)."""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _page_facts():
    facts = {}
    with open(os.path.join(GOLD, "page_facts.txt")) as f:
        for line in f:
            line = line.split("|")[0].strip()
            if line and not line.startswith("#"):
                k, v = [s.strip() for s in line.split("=")]
                facts[k] = v
    return facts


def _e2m1_table():
    t = {}
    with open(os.path.join(GOLD, "e2m1_values.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                t[int(c)] = float(v)
    return t


# ------------------------------------------------------------- scalar decoders
def test_fp16_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zeros as well
    assert math.copysign(1.0, oracle.fp16(0x8000)) == -1.0


def test_bf16_all_patterns_match_ieee_single_top_half():
    for b in range(0, 65536, 1):
        ref = struct.unpack("<f", struct.pack("<I", b << 16))[0]
        got = oracle.bf16(b)
        if math.isnan(ref):
            assert math.isnan(got)
        else:
            assert got == ref, hex(b)


def test_bf16_literals():
    assert oracle.bf16(0x3F80) == 1.0
    assert oracle.bf16(0xC000) == -2.0
    assert oracle.bf16(0x4049) == 3.140625
    assert oracle.bf16(0x0001) == 2.0 ** -133


def test_e8m0_literals():
    assert oracle.e8m0(127) == 1.0
    assert oracle.e8m0(128) == 2.0
    assert oracle.e8m0(126) == 0.5
    assert oracle.e8m0(119) == 0.00390625        # 2^-8, lower end of the MoE workload draw
    assert oracle.e8m0(125) == 0.25              # 2^-2, upper end
    assert oracle.e8m0(0) == 5.877471754111438e-39
    assert oracle.e8m0(254) == 1.7014118346046923e38
    assert math.isnan(oracle.e8m0(255))


def test_e2m1_table_and_structure():
    table = _e2m1_table()
    for c in range(16):
        assert oracle.e2m1(c) == table[c]
    # sign bit is bit 3; magnitudes are increasing in the 3 low bits
    mags = [oracle.e2m1(c) for c in range(8)]
    assert mags == sorted(mags) and len(set(mags)) == 8
    for c in range(8):
        assert oracle.e2m1(c | 8) == -oracle.e2m1(c)


def test_mxfp4_block_size_matches_pages():
    facts = _page_facts()
    bits = 8 * oracle.BLOCK_BYTES[oracle.MXFP4] / 32.0
    assert bits == float(facts["mxfp4_bits_per_weight"])
    assert 2 * 32 == int(facts["gpt_oss_20b_experts"]) * 2
    assert wl.CONFIGS[4]["n_experts"] == int(facts["gpt_oss_20b_experts"])
    assert wl.CONFIGS[4]["top_k"] == int(facts["gpt_oss_20b_top_k"])


# ------------------------------------------------------------ hand-built blocks
def _hand_q8_block():
    codes = [0, 1, -1, 2, -2, 127, -127, -128] + list(range(-4, 20))
    blk = bytes([0x00, 0x38]) + bytes([(c + 256) % 256 for c in codes])   # d = 0x3800 = 0.5
    return np.frombuffer(blk, dtype=np.uint8), [0.5 * c for c in codes]


def _hand_q4_block():
    body = bytes([(j & 15) | (((15 - j) & 15) << 4) for j in range(16)])
    blk = bytes([0x00, 0x40]) + body                                       # d = 0x4000 = 2.0
    want = [2.0 * (j - 8) for j in range(16)] + [2.0 * ((15 - j) - 8) for j in range(16)]
    return np.frombuffer(blk, dtype=np.uint8), want


def _hand_mxfp4_block():
    table = _e2m1_table()
    body = bytes([(j & 15) | (((15 - j) & 15) << 4) for j in range(16)])
    blk = bytes([126]) + body                                              # scale 2^-1
    want = [0.5 * table[j] for j in range(16)] + [0.5 * table[15 - j] for j in range(16)]
    return np.frombuffer(blk, dtype=np.uint8), want


@pytest.mark.parametrize("fmt,maker", [(oracle.Q8_0, _hand_q8_block), (oracle.Q4_0, _hand_q4_block),
                                       (oracle.MXFP4, _hand_mxfp4_block)])
def test_hand_built_block_decodes(fmt, maker):
    blk, want = maker()
    w = oracle.decode(fmt, blk, 1, 32)
    assert w.shape == (1, 32)
    assert list(w[0]) == want


def test_q8_subnormal_and_negative_scale():
    blk = np.frombuffer(bytes([0x01, 0x80]) + bytes([3] * 32), dtype=np.uint8)   # d = -2^-24
    w = oracle.decode(oracle.Q8_0, blk, 1, 32)
    assert np.all(w == -3.0 * 2.0 ** -24)


def test_rows_and_blocks_are_row_major():
    # two rows x two blocks, each block all-equal with a distinct scale
    blks = []
    for d in (0x3C00, 0x4000, 0x4200, 0x4400):        # 1, 2, 3, 4
        blks.append(bytes([d & 0xFF, d >> 8]) + bytes([1] * 32))
    arr = np.frombuffer(b"".join(blks), dtype=np.uint8)
    w = oracle.decode(oracle.Q8_0, arr, 2, 64)
    assert np.all(w[0, :32] == 1) and np.all(w[0, 32:] == 2)
    assert np.all(w[1, :32] == 3) and np.all(w[1, 32:] == 4)


# --------------------------------------------------------- exact rational sums
def _frac_weights(fmt, blocks, n, k):
    """Exact weights as Fractions, decoded by numpy / struct / the E2M1 table."""
    table = _e2m1_table()
    bb = oracle.BLOCK_BYTES[fmt]
    b = blocks.reshape(n, k // 32, bb)
    W = [[None] * k for _ in range(n)]
    for r in range(n):
        for blk in range(k // 32):
            row = b[r, blk]
            if fmt == oracle.MXFP4:
                sc = Fraction(2) ** (int(row[0]) - 127)
                body = row[1:]
            else:
                sc = Fraction(float(np.array([int(row[0]) | (int(row[1]) << 8)], dtype=np.uint16).view(np.float16)[0]))
                body = row[2:]
            for i in range(32):
                if fmt == oracle.Q8_0:
                    v = int(np.int8(body[i]))
                elif fmt == oracle.Q4_0:
                    v = (int(body[i]) & 15) - 8 if i < 16 else (int(body[i - 16]) >> 4) - 8
                else:
                    c = (int(body[i]) & 15) if i < 16 else (int(body[i - 16]) >> 4)
                    v = Fraction(table[c])
                W[r][32 * blk + i] = sc * v
    return W


def _frac_x(x, xt):
    if xt == oracle.X_F32:
        return [Fraction(float(v)) for v in x.reshape(-1)]
    return [Fraction(struct.unpack("<f", struct.pack("<I", int(v) << 16))[0]) for v in x.reshape(-1)]


@pytest.mark.parametrize("fmt", [oracle.Q8_0, oracle.Q4_0, oracle.MXFP4])
@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
def test_brute_force_4x64_exact(fmt, xt):
    n, k, m = 4, 64, 2
    blocks = wl.blocks_for(fmt, n, k, config=90 + fmt, matrix=xt)
    rng = wl.rng_for(91, fmt, "x")
    x = wl.x_f32((m, k), rng) if xt == oracle.X_F32 else wl.x_bf16_bits((m, k), rng)
    y, l1 = oracle.gemv(fmt, blocks, n, k, x, xt)
    W = _frac_weights(fmt, blocks, n, k)
    X = _frac_x(x, xt)
    for t in range(m):
        for r in range(n):
            prods = [W[r][c] * X[t * k + c] for c in range(k)]
            exact = sum(prods, Fraction(0))
            a = sum((abs(p) for p in prods), Fraction(0))
            assert abs(Fraction(y[t, r]) - exact) <= Fraction(1, 2 ** 50) * a
            assert abs(Fraction(l1[t, r]) - a) <= Fraction(1, 2 ** 50) * a


def test_numpy_blas_cross_check_c0_size():
    n = k = 2048
    blocks = wl.blocks_for(oracle.Q8_0, n, k, config=0, matrix=0)
    x = wl.x_f32((1, k), wl.rng_for(0, 0, "x"))
    W = oracle.decode(oracle.Q8_0, blocks, n, k)
    y, l1 = oracle.gemv(oracle.Q8_0, blocks, n, k, x, oracle.X_F32)
    ref = W @ x.astype(np.float64)[0]
    assert np.max(np.abs(ref - y[0]) / l1[0]) < 1e-13
    assert np.allclose(l1[0], np.abs(W) @ np.abs(x.astype(np.float64)[0]), rtol=1e-13)


def test_numpy_blas_cross_check_many_tokens():
    # the product for a prefill-sized token count (128) against numpy's matmul
    fmt, n, k, m = oracle.Q4_0, 96, 512, 128
    blocks = wl.blocks_for(fmt, n, k, config=93, matrix=1)
    x = wl.x_bf16_bits((m, k), wl.rng_for(93, 1, "x"))
    W = oracle.decode(fmt, blocks, n, k)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y, l1 = oracle.gemv(fmt, blocks, n, k, x, oracle.X_BF16)
    assert np.max(np.abs(xv @ W.T - y) / l1) < 1e-13
    assert np.allclose(l1, np.abs(xv) @ np.abs(W).T, rtol=1e-13)


def test_row_subset_matches_full():
    n, k = 64, 256
    blocks = wl.blocks_for(oracle.Q4_0, n, k, config=92, matrix=0)
    x = wl.x_bf16_bits((3, k), wl.rng_for(92, 0, "x"))
    y, l1 = oracle.gemv(oracle.Q4_0, blocks, n, k, x, oracle.X_BF16)
    rows = np.array([63, 0, 17, 17])
    ys, l1s = oracle.gemv(oracle.Q4_0, blocks, n, k, x, oracle.X_BF16, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(l1s, l1[:, rows])


# --------------------------------------------------------------- closed forms
@pytest.mark.parametrize("fmt", [oracle.Q8_0, oracle.Q4_0, oracle.MXFP4])
def test_all_equal_blocks_closed_form(fmt):
    n, k = 3, 96
    x = wl.x_f32((1, k), wl.rng_for(93, fmt, "x"))
    sx = float(np.sum(x.astype(np.float64)))
    if fmt == oracle.Q8_0:
        blk, val = bytes([0x00, 0x3A]) + bytes([256 - 5] * 32), 0.75 * -5          # d = 0.75
    elif fmt == oracle.Q4_0:
        blk, val = bytes([0x00, 0x3A]) + bytes([0x33] * 16), 0.75 * (3 - 8)
    else:
        blk, val = bytes([125]) + bytes([0xDD] * 16), 0.25 * -3.0                  # code 13 = -3
    blocks = np.frombuffer(blk * (n * k // 32), dtype=np.uint8)
    y, _ = oracle.gemv(fmt, blocks, n, k, x, oracle.X_F32)
    assert np.allclose(y[0], val * sx, rtol=0, atol=1e-12 * abs(val) * np.sum(np.abs(x)))


@pytest.mark.parametrize("fmt", [oracle.Q8_0, oracle.Q4_0, oracle.MXFP4])
def test_one_hot_x_selects_a_column(fmt):
    n, k = 5, 128
    blocks = wl.blocks_for(fmt, n, k, config=94, matrix=fmt)
    W = oracle.decode(fmt, blocks, n, k)
    for col in (0, 31, 32, 77, 127):
        x = np.zeros((1, k), dtype=np.float32)
        x[0, col] = 1.0
        y, l1 = oracle.gemv(fmt, blocks, n, k, x, oracle.X_F32)
        assert np.array_equal(y[0], W[:, col])
        assert np.array_equal(l1[0], np.abs(W[:, col]))


def test_error_metric():
    y = np.array([1.0, 0.0, 2.0])
    l1 = np.array([10.0, 0.0, 4.0])
    assert oracle.max_rel_err(np.array([1.1, 0.0, 2.0]), y, l1) == pytest.approx(0.01)
    assert oracle.max_rel_err(np.array([1.0, 1e-30, 2.0]), y, l1) == math.inf
    assert oracle.max_rel_err(np.array([1.0, 0.0, np.nan]), y, l1) == math.inf


# ----------------------------------------------------------------------- MoE
def test_moe_hand_example_exact():
    # 3 experts of a 1 x 32 Q8_0 matrix; expert e has all codes e+1, d = 1.0
    experts = b"".join(bytes([0x00, 0x3C]) + bytes([e + 1] * 32) for e in range(3))
    experts = np.frombuffer(experts, dtype=np.uint8)
    ids = np.array([[2, 0]], dtype=np.int32)
    g = np.array([[0.75, 0.25]], dtype=np.float32)
    x = np.ones((1, 32), dtype=np.float32)
    y, _ = oracle.moe(oracle.Q8_0, experts, 3, 1, 32, ids, g, x, oracle.X_F32, oracle.MOE_GATE_UP)
    assert y[0, 0, 0] == 3 * 32 and y[0, 1, 0] == 1 * 32
    h = np.stack([np.full(32, 2.0), np.full(32, -1.0)]).astype(np.float32).reshape(1, 2, 32)
    y, l1 = oracle.moe(oracle.Q8_0, experts, 3, 1, 32, ids, g, h, oracle.X_F32, oracle.MOE_DOWN)
    # 0.75 * (3*2*32) + 0.25 * (1*-1*32) = 144 - 8
    assert y[0, 0] == 136.0
    assert l1[0, 0] == 0.75 * 192 + 0.25 * 32


def test_moe_matches_dense_per_slot():
    fmt, E, n, k, m, top_k = oracle.MXFP4, 6, 16, 64, 3, 2
    experts = np.concatenate([wl.blocks_for(fmt, n, k, config=95, matrix=e).reshape(-1) for e in range(E)])
    _, ids, g = wl.router_topk(m, E, top_k, wl.rng_for(95, 0, "router"))
    x = wl.x_bf16_bits((m, k), wl.rng_for(95, 0, "x"))
    h = wl.x_bf16_bits((m, top_k, k), wl.rng_for(95, 0, "h"))
    yg, _ = oracle.moe(fmt, experts, E, n, k, ids, g, x, oracle.X_BF16, oracle.MOE_GATE_UP)
    yd, _ = oracle.moe(fmt, experts, E, n, k, ids, g, h, oracle.X_BF16, oracle.MOE_DOWN)
    mat = n * (k // 32) * 17
    for t in range(m):
        acc = np.zeros(n)
        for j in range(top_k):
            e = ids[t, j]
            Wb = experts[e * mat:(e + 1) * mat]
            yj, _ = oracle.gemv(fmt, Wb, n, k, x[t:t + 1], oracle.X_BF16)
            assert np.array_equal(yg[t, j], yj[0])
            hj, _ = oracle.gemv(fmt, Wb, n, k, h[t, j:j + 1], oracle.X_BF16)
            acc += float(g[t, j]) * hj[0]
        assert np.allclose(yd[t], acc, rtol=1e-14, atol=1e-14)


def test_oracle_rejects_bad_arguments():
    blk, _ = _hand_q8_block()
    with pytest.raises(ValueError):
        oracle.gemv(oracle.Q8_0, blk, 1, 32, np.ones((1, 32), np.float32), 7)
    with pytest.raises(ValueError):
        oracle.gemv(oracle.Q8_0, blk, 1, 32, np.ones((1, 32), np.float32), oracle.X_F32, rows=[1])


# ------------------------------------------------------------------ router
def test_router_hand_example_with_tie():
    """logits (0.5, 2, 2, -1, 3), top 3: expert 4 first, then the tie 2.0
    resolved to the lower id (1 before 2); weights e^0, e^-1, e^-1 normalised."""
    ids, w = oracle.router_topk(np.array([[0.5, 2.0, 2.0, -1.0, 3.0]], dtype=np.float32), 3)
    assert ids.tolist() == [[4, 1, 2]]
    den = 1.0 + 2.0 * math.exp(-1.0)
    assert np.allclose(w[0], [1.0 / den, math.exp(-1.0) / den, math.exp(-1.0) / den], rtol=1e-15, atol=0)


def test_router_closed_forms():
    ids, w = oracle.router_topk(np.zeros((2, 6), dtype=np.float32), 4)        # all equal
    assert ids.tolist() == [[0, 1, 2, 3]] * 2 and np.all(w == 0.25)
    ids, w = oracle.router_topk(np.array([[1.0, -np.inf, 7.0]], dtype=np.float32), 1)
    assert ids.tolist() == [[2]] and w.tolist() == [[1.0]]
    ids, w = oracle.router_topk(np.array([[0.0, -np.inf, np.log(3.0)]], dtype=np.float32), 3)
    assert ids.tolist() == [[2, 0, 1]]
    assert abs(w[0, 0] - 0.75) < 1e-7 and abs(w[0, 1] - 0.25) < 1e-7 and w[0, 2] == 0.0
    with pytest.raises(ValueError):
        oracle.router_topk(np.array([[0.0, np.nan]], dtype=np.float32), 1)


def test_router_against_exhaustive_search():
    """Small cases with repeated values: the chosen list is the lexicographic
    maximum of (logit, -id) over all ordered selections."""
    import itertools
    rng = np.random.default_rng(5)
    for trial in range(200):
        n_experts = int(rng.integers(1, 7))
        top_k = int(rng.integers(1, n_experts + 1))
        logits = rng.integers(-2, 3, size=(1, n_experts)).astype(np.float32)
        ids, w = oracle.router_topk(logits, top_k)
        best = max(itertools.permutations(range(n_experts), top_k),
                   key=lambda p: [(float(logits[0, e]), -e) for e in p])
        assert ids[0].tolist() == list(best)
        assert abs(w.sum() - 1.0) < 1e-15
        assert np.all(np.diff(w[0]) <= 0)


# ------------------------------------------------------- fused steps (SwiGLU, RMSNorm, residual)
def test_silu_against_torch_and_identities():
    torch = pytest.importorskip("torch")
    v = np.concatenate([np.linspace(-60, 60, 2401), [0.0, 1e-300, -1e-300, 700.0, -700.0, 1e4, -1e4]])
    ref = torch.nn.functional.silu(torch.from_numpy(v)).numpy()
    got = oracle.silu(v)
    assert np.all(np.abs(got - ref) <= 4e-16 * np.maximum(np.abs(ref), 1e-300))
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1e4) == 1e4 and oracle.silu(-1e4) == 0.0            # the limits
    w = np.linspace(-30, 30, 601)
    assert np.allclose(oracle.silu(-w), oracle.silu(w) - w, rtol=0, atol=1e-13)   # sigma(-v) = 1 - sigma(v)
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    # |SiLU'| < 1.1 (the error scale of the fused oracle rests on it)
    h = 1e-6
    d = (oracle.silu(w + h) - oracle.silu(w - h)) / (2 * h)
    assert np.max(np.abs(d)) < 1.1 and np.max(d) > 1.09


def test_rmsnorm_against_torch_and_closed_forms():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 256)) * np.array([[1.0], [1e-3], [50.0]])
    gamma = rng.uniform(0.5, 1.5, 256).astype(np.float32)
    for eps in (0.0, 1e-6, 1e-2):
        got, r = oracle.rmsnorm(x, gamma, eps)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (256,),
                                           torch.from_numpy(gamma.astype(np.float64)), eps).numpy()
        assert np.allclose(got, ref, rtol=1e-14, atol=0)
        assert np.allclose(r, [1.0 / math.sqrt(math.fsum(row * row) / 256 + eps) for row in x], rtol=1e-15)
    # a constant row c with eps = 0 normalises to sign(c) * gamma exactly; scaling x changes nothing
    c = np.full((2, 64), [[-3.0], [0.5]])
    got, _ = oracle.rmsnorm(c, np.full(64, 2.0, np.float32), 0.0)
    assert np.array_equal(got, np.full((2, 64), [[-2.0], [2.0]]))
    a, _ = oracle.rmsnorm(x, gamma, 0.0)
    b, _ = oracle.rmsnorm(1024.0 * x, gamma, 0.0)
    assert np.allclose(a, b, rtol=1e-14, atol=0)


def test_x_values_decodes_bf16_and_fp32():
    bits = np.array([[0x3F80, 0xC000, 0x0001, 0x7F7F]], dtype=np.uint16)
    want = [1.0, -2.0, struct.unpack("<f", struct.pack("<I", 0x00010000))[0],
            struct.unpack("<f", struct.pack("<I", 0x7F7F0000))[0]]
    assert np.array_equal(oracle.x_values(bits, oracle.X_BF16)[0], want)
    f = np.array([[1.5, -0.1]], dtype=np.float32)
    assert np.array_equal(oracle.x_values(f, oracle.X_F32), f.astype(np.float64))


@pytest.mark.parametrize("fmt", [oracle.Q8_0, oracle.Q4_0, oracle.MXFP4])
def test_dense_fused_reduces_to_the_c_product(fmt):
    n, k, m = 96, 256, 3
    blocks = wl.blocks_for(fmt, n, k, config=94, matrix=fmt)
    x = wl.x_bf16_bits((m, k), wl.rng_for(94, fmt, "x"))
    y, l1 = oracle.gemv(fmt, blocks, n, k, x, oracle.X_BF16)            # the C loop
    o, scale = oracle.dense_fused(fmt, blocks, n, k, x, oracle.X_BF16)   # decode + numpy product
    assert np.max(np.abs(o - y) / l1) < 1e-13 and np.allclose(scale, l1, rtol=1e-13)
    # SwiGLU: gate rows first, up rows second
    torch = pytest.importorskip("torch")
    o, _ = oracle.dense_fused(fmt, blocks, n, k, x, oracle.X_BF16, act=oracle.ACT_SWIGLU)
    g, u = y[:, : n // 2], y[:, n // 2:]
    want = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u
    assert np.allclose(o, want, rtol=1e-12, atol=1e-12 * np.max(l1))
    # residual: added after everything else
    res = wl.x_f32((m, n // 2), wl.rng_for(94, fmt, "res"))
    o2, _ = oracle.dense_fused(fmt, blocks, n, k, x, oracle.X_BF16, act=oracle.ACT_SWIGLU, residual=res)
    assert np.allclose(o2 - res.astype(np.float64), o, rtol=0, atol=1e-12 * np.max(np.abs(o2)))
    # row subsets
    rows = np.array([47, 0, 5])
    o3, s3 = oracle.dense_fused(fmt, blocks, n, k, x, oracle.X_BF16, act=oracle.ACT_SWIGLU, residual=res, rows=rows)
    _, s2 = oracle.dense_fused(fmt, blocks, n, k, x, oracle.X_BF16, act=oracle.ACT_SWIGLU, residual=res)
    assert np.array_equal(o3, o2[:, rows]) and np.array_equal(s3, s2[:, rows])


def test_dense_fused_norm_is_a_scaled_product():
    # with gamma a power of two, x * gamma is exact in fp32, so the C product of
    # x * gamma times r (computed here with math.fsum) must give the same rows
    fmt, n, k, m = oracle.Q8_0, 64, 512, 2
    blocks = wl.blocks_for(fmt, n, k, config=95, matrix=0)
    x = wl.x_f32((m, k), wl.rng_for(95, 0, "x"))
    gamma = np.where(np.arange(k) % 3 == 0, 0.5, 4.0).astype(np.float32)
    eps = 1e-5
    o, scale = oracle.dense_fused(fmt, blocks, n, k, x, oracle.X_F32, norm_weight=gamma, eps=eps)
    y, l1 = oracle.gemv(fmt, blocks, n, k, (x * gamma).astype(np.float32), oracle.X_F32)
    xd = x.astype(np.float64)
    r = np.array([1.0 / math.sqrt(math.fsum(row * row) / k + eps) for row in xd])
    assert np.max(np.abs(o - r[:, None] * y) / (r[:, None] * l1)) < 1e-13
    assert np.allclose(scale, r[:, None] * l1, rtol=1e-13)


def test_fused_verdict_catches_plausible_mistakes():
    fmt, n, k, m = oracle.Q4_0, 128, 512, 2
    blocks = wl.blocks_for(fmt, n, k, config=96, matrix=0)
    # activations with an RMS far from 1, so that the normalisation matters
    x = (5.0 * wl.x_f32((m, k), wl.rng_for(96, 0, "x"))).astype(np.float32)
    gamma = wl.x_f32((1, k), wl.rng_for(96, 0, "gamma"))[0]
    o, scale = oracle.dense_fused(fmt, blocks, n, k, x, oracle.X_F32, norm_weight=gamma, eps=1e-6,
                                  act=oracle.ACT_SWIGLU)
    assert oracle.fused_err(o, o, scale) == 0.0
    # fp32 rounding of the output passes; bf16 rounding passes only under the bf16 allowance
    assert oracle.fused_err(o.astype(np.float32), o, scale) == 0.0
    ob = ((o.astype(np.float32).view(np.uint32) + 0x8000) & 0xFFFF0000).view(np.float32)
    assert oracle.fused_err(ob, o, scale, y_bf16=True) == 0.0
    # gate and up swapped, the normalisation dropped, gamma dropped: each fails by
    # more than ten times the 2e-3 tolerance
    xv = oracle.x_values(x, oracle.X_F32)
    _, r = oracle.rmsnorm(xv, gamma, 1e-6)
    yn, _ = oracle.dense_fused(fmt, blocks, n, k, x, oracle.X_F32, norm_weight=gamma, eps=1e-6)
    swapped = oracle.silu(yn[:, n // 2:]) * yn[:, : n // 2]
    assert oracle.fused_err(swapped, o, scale) > 10 * 2e-3
    no_norm = oracle.silu(yn[:, : n // 2] / r[:, None]) * (yn[:, n // 2:] / r[:, None])
    assert oracle.fused_err(no_norm, o, scale) > 10 * 2e-3
    ones = np.ones(k, dtype=np.float32)
    no_gamma, _ = oracle.dense_fused(fmt, blocks, n, k, x, oracle.X_F32, norm_weight=ones, eps=1e-6,
                                     act=oracle.ACT_SWIGLU)
    assert oracle.fused_err(no_gamma, o, scale) > 10 * 2e-3


def _moe_case(fmt=oracle.Q4_0, E=6, n=64, k=128, m=3, top_k=2, config=97):
    experts = np.concatenate([wl.blocks_for(fmt, n, k, config=config, matrix=e).reshape(-1) for e in range(E)])
    _, ids, g = wl.router_topk(m, E, top_k, wl.rng_for(config, 0, "router"))
    return fmt, E, n, k, m, top_k, experts, ids, g


def test_moe_fused_reduces_to_the_c_expert_product():
    torch = pytest.importorskip("torch")
    fmt, E, n, k, m, top_k, experts, ids, g = _moe_case()
    x = wl.x_bf16_bits((m, k), wl.rng_for(97, 0, "x"))
    h = wl.x_bf16_bits((m, top_k, k), wl.rng_for(97, 0, "h"))
    yg, l1g = oracle.moe(fmt, experts, E, n, k, ids, g, x, oracle.X_BF16, oracle.MOE_GATE_UP)   # the C loop
    o, s = oracle.moe_fused(fmt, experts, E, n, k, ids, g, x, oracle.X_BF16, oracle.MOE_GATE_UP)
    assert np.max(np.abs(o - yg) / l1g) < 1e-13 and np.allclose(s, l1g, rtol=1e-13)
    o, _ = oracle.moe_fused(fmt, experts, E, n, k, ids, g, x, oracle.X_BF16, oracle.MOE_GATE_UP, act=oracle.ACT_SWIGLU)
    want = torch.nn.functional.silu(torch.from_numpy(yg[..., : n // 2])).numpy() * yg[..., n // 2:]
    assert np.allclose(o, want, rtol=1e-12, atol=1e-12 * np.max(l1g))
    yd, l1d = oracle.moe(fmt, experts, E, n, k, ids, g, h, oracle.X_BF16, oracle.MOE_DOWN)
    res = wl.x_f32((m, n), wl.rng_for(97, 0, "res"))
    o, s = oracle.moe_fused(fmt, experts, E, n, k, ids, g, h, oracle.X_BF16, oracle.MOE_DOWN, residual=res)
    assert np.max(np.abs(o - res - yd) / l1d) < 1e-13 and np.allclose(s, l1d, rtol=1e-13)
    rows = np.array([5, 0, 63])
    o2, s2 = oracle.moe_fused(fmt, experts, E, n, k, ids, g, h, oracle.X_BF16, oracle.MOE_DOWN, residual=res, rows=rows)
    assert np.array_equal(o2, o[:, rows]) and np.array_equal(s2, s[:, rows])


def test_moe_fused_norm_is_a_scaled_expert_product():
    # gamma a power of two: x * gamma is exact in fp32, so the C expert product
    # of x * gamma, times r (math.fsum), gives the normalised rows
    fmt, E, n, k, m, top_k, experts, ids, g = _moe_case(fmt=oracle.MXFP4, config=98)
    x = (4.0 * wl.x_f32((m, k), wl.rng_for(98, 0, "x"))).astype(np.float32)
    gamma = np.where(np.arange(k) % 5 == 0, 2.0, 0.25).astype(np.float32)
    eps = 1e-4
    o, s = oracle.moe_fused(fmt, experts, E, n, k, ids, g, x, oracle.X_F32, oracle.MOE_GATE_UP,
                            norm_weight=gamma, eps=eps)
    y, l1 = oracle.moe(fmt, experts, E, n, k, ids, g, (x * gamma).astype(np.float32), oracle.X_F32,
                       oracle.MOE_GATE_UP)
    r = np.array([1.0 / math.sqrt(math.fsum(row * row) / k + eps) for row in x.astype(np.float64)])
    assert np.max(np.abs(o - r[:, None, None] * y) / (r[:, None, None] * l1)) < 1e-13
    assert np.allclose(s, r[:, None, None] * l1, rtol=1e-13)


def test_moe_fused_invalid_ids():
    fmt, E, n, k, m, top_k, experts, ids, g = _moe_case(config=99)
    ids = ids.copy()
    ids[0, 1] = -1
    ids[1, 0] = E
    x = wl.x_bf16_bits((m, k), wl.rng_for(99, 0, "x"))
    o, _ = oracle.moe_fused(fmt, experts, E, n, k, ids, g, x, oracle.X_BF16, oracle.MOE_GATE_UP, act=oracle.ACT_SWIGLU)
    assert np.all(np.isnan(o[0, 1])) and np.all(np.isnan(o[1, 0])) and np.all(np.isfinite(o[2]))
    # down: every id invalid leaves the residual exactly
    h = wl.x_bf16_bits((m, top_k, k), wl.rng_for(99, 0, "h"))
    res = wl.x_f32((m, n), wl.rng_for(99, 0, "res"))
    o, s = oracle.moe_fused(fmt, experts, E, n, k, np.full_like(ids, -1), g, h, oracle.X_BF16, oracle.MOE_DOWN,
                            residual=res)
    assert np.array_equal(o, res.astype(np.float64)) and not s.any()
    with pytest.raises(ValueError):
        oracle.moe_fused(fmt, experts, E, n, k, ids, g, h, oracle.X_BF16, oracle.MOE_DOWN, act=oracle.ACT_SWIGLU)
