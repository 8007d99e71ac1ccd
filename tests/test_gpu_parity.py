"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bars: bit-exact for packing, unpacking and decoded weights; bit-exact where
every partial sum is exact (one-hot and small-integer activations); elsewhere
max |y - y_oracle| / L1(row) <= 2e-3 (fp32 accumulation; the fp32 summation
bound gamma_{K+2} stays below 7.4e-4 for every K used here).
"""
import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
q = pytest.importorskip("block_quantized_weight_amd")

pytestmark = pytest.mark.gpu
TOL = 2e-3
FMTS = [q.Q8_0, q.Q4_0, q.MXFP4]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_dev(bits, dev):
    return to_dev(np.ascontiguousarray(bits).view(np.int16), dev).view(torch.bfloat16)


def x_dev(x, xt, dev):
    return bf16_dev(x, dev) if xt == oracle.X_BF16 else to_dev(x, dev)


def draw_x(shape, xt, config, matrix, role="x"):
    rng = wl.rng_for(config, matrix, role)
    return wl.x_bf16_bits(shape, rng) if xt == oracle.X_BF16 else wl.x_f32(shape, rng)


def packed_dev(fmt, canon, n, k, dev):
    return q.pack(fmt, to_dev(canon.reshape(-1), dev), n, k)


def run_dense(fmt, canon, n, k, x, xt, dev):
    w = packed_dev(fmt, canon, n, k, dev)
    xd = x_dev(x.reshape(-1, k), xt, dev)
    y = q.qgemv(fmt, w, n, k, xd)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# ------------------------------------------------------------------ packing
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(1, 32), (65, 96), (300, 2048), (19, 608), (2560, 9728)])
def test_device_pack_matches_host_and_round_trips(dev, fmt, n, k):
    say(f"pack fmt={fmt} n={n} k={k}")
    canon = wl.blocks_for(fmt, n, k, config=60, matrix=n).reshape(-1)
    host = q.pack_host(fmt, canon, n, k)
    pd = packed_dev(fmt, canon, n, k, dev)
    assert np.array_equal(pd.cpu().numpy(), host)
    # into a buffer full of junk: every byte of the packed form is written
    junk = torch.full((q.packed_bytes(fmt, n, k),), 0xAB, dtype=torch.uint8, device=dev)
    q.pack(fmt, torch.from_numpy(canon).to(dev), n, k, out=junk)
    assert np.array_equal(junk.cpu().numpy(), host)
    back = q.unpack(fmt, pd, n, k)
    assert np.array_equal(back.cpu().numpy(), canon)


# ------------------------------------------------------------------ decoding
def _finite_fp16_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[np.isfinite(b.view(np.float16))]


def _exhaustive_blocks(fmt, n, k):
    """Blocks in which every code value occurs at every position, and every finite
    fp16 scale (Q8_0, Q4_0) or every UE8M0 exponent 1..252 (MXFP4) occurs."""
    nb = k // 32
    total = n * nb
    r = np.arange(n)[:, None, None]
    b = np.arange(nb)[None, :, None]
    i = np.arange(32)[None, None, :]
    if fmt == q.Q8_0:
        codes = ((r + 7 * b + 11 * i) % 256).astype(np.uint8).view(np.int8)
        pats = _finite_fp16_patterns()
        d = np.resize(pats, total).reshape(n, nb)
        return wl.encode_q8_0(codes, d)
    if fmt == q.Q4_0:
        codes = ((r + 3 * b + 5 * i) % 16).astype(np.uint8)
        pats = _finite_fp16_patterns()
        d = np.resize(pats, total).reshape(n, nb)
        return wl.encode_q4_0(codes, d)
    codes = ((r + 3 * b + 5 * i) % 16).astype(np.uint8)
    e = (1 + (np.arange(total) % 252)).astype(np.uint8).reshape(n, nb)
    return wl.encode_mxfp4(codes, e)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_bit_exact_random(dev, fmt):
    n, k = 333, 1824
    say(f"dequant random fmt={fmt}")
    canon = wl.blocks_for(fmt, n, k, config=61, matrix=fmt)
    w = q.dequant_f32(fmt, packed_dev(fmt, canon, n, k, dev), n, k).cpu().numpy()
    ref = oracle.decode(fmt, canon, n, k)
    assert np.array_equal(w.astype(np.float64), ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_bit_exact_exhaustive(dev, fmt):
    n, k = 2048, 992            # 63,488 blocks: every finite fp16 scale once
    say(f"dequant exhaustive fmt={fmt}")
    canon = _exhaustive_blocks(fmt, n, k)
    w = q.dequant_f32(fmt, packed_dev(fmt, canon, n, k, dev), n, k).cpu().numpy()
    ref = oracle.decode(fmt, canon, n, k)
    assert np.array_equal(w.astype(np.float64), ref)


# --------------------------------------------------------- exact products
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
def test_one_hot_activations_select_columns_exactly(dev, fmt, xt):
    n, k = 200, 1600
    say(f"one-hot fmt={fmt} xt={xt}")
    canon = wl.blocks_for(fmt, n, k, config=62, matrix=fmt)
    cols = [0, 31, 32, 777, 1599, 800, 5, 1000]
    x = np.zeros((len(cols), k), dtype=np.float32)
    for t, c in enumerate(cols):
        x[t, c] = 1.0
    xb = wl.f32_to_bf16_bits_rne(x) if xt == oracle.X_BF16 else x
    y = run_dense(fmt, canon, n, k, xb, xt, dev)
    W = oracle.decode(fmt, canon, n, k)
    for t, c in enumerate(cols):
        assert np.array_equal(y[t].astype(np.float64), W[:, c]), (t, c)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
def test_integer_case_is_exact(dev, fmt, xt):
    """Unit scale and small-integer activations: every partial sum is an exact
    fp32 value, so any summation order gives the oracle's result bit for bit."""
    n, k, m = 130, 4096, 3
    say(f"integer fmt={fmt} xt={xt}")
    rng = np.random.default_rng(63)
    nb = k // 32
    if fmt == q.Q8_0:
        canon = wl.encode_q8_0(rng.integers(-127, 128, size=(n, nb, 32)).astype(np.int8),
                               np.full((n, nb), 0x3C00, dtype=np.uint16))
    elif fmt == q.Q4_0:
        canon = wl.encode_q4_0(rng.integers(0, 16, size=(n, nb, 32)).astype(np.uint8),
                               np.full((n, nb), 0x3C00, dtype=np.uint16))
    else:
        canon = wl.encode_mxfp4(rng.integers(0, 16, size=(n, nb, 32)).astype(np.uint8),
                                np.full((n, nb), 127, dtype=np.uint8))
    x = rng.integers(-3, 4, size=(m, k)).astype(np.float32)
    xb = wl.f32_to_bf16_bits_rne(x) if xt == oracle.X_BF16 else x
    y = run_dense(fmt, canon, n, k, xb, xt, dev)
    ref, _ = oracle.gemv(fmt, canon, n, k, xb, xt)
    assert np.array_equal(y.astype(np.float64), ref)


# ------------------------------------------------------- tolerance parity
SHAPES = [(1, 32), (5, 96), (63, 64), (65, 608), (300, 2048), (129, 1024), (1000, 4096), (64, 9728), (7, 12288)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
@pytest.mark.parametrize("m", [1, 3, 8])
def test_dense_shapes(dev, fmt, xt, m):
    for n, k in SHAPES:
        say(f"dense fmt={fmt} xt={xt} m={m} n={n} k={k}")
        canon = wl.blocks_for(fmt, n, k, config=64, matrix=n + k)
        x = draw_x((m, k), xt, 64, n + k)
        y = run_dense(fmt, canon, n, k, x, xt, dev)
        ref, l1 = oracle.gemv(fmt, canon, n, k, x, xt)
        err = oracle.max_rel_err(y, ref, l1)
        assert err <= TOL, (n, k, err)


def _config_dense(dev, config, fmt, xt, n, k, m, matrix, rows=None):
    canon = wl.blocks_for(fmt, n, k, config=config, matrix=matrix)
    x = draw_x((m, k), xt, config, matrix)
    y = run_dense(fmt, canon, n, k, x, xt, dev)
    ref, l1 = oracle.gemv(fmt, canon, n, k, x, xt, rows=rows)
    yy = y if rows is None else y[:, rows]
    return oracle.max_rel_err(yy, ref, l1)


def test_config0_q8_0_2048(dev):
    say("C0")
    err = _config_dense(dev, 0, q.Q8_0, oracle.X_F32, 2048, 2048, 1, 0)
    assert err <= TOL, err


@pytest.mark.parametrize("name,n,k", [("gate_up", 19456, 2560), ("down", 2560, 9728)])
def test_config1_q4_0_layer(dev, name, n, k):
    say(f"C1 {name}")
    err = _config_dense(dev, 1, q.Q4_0, oracle.X_BF16, n, k, 1, 0 if name == "gate_up" else 1)
    assert err <= TOL, err


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 144])
def test_config2_sweep_shapes(dev, idx):
    j, name, n, k = wl.c2_sweep_shapes()[idx]
    say(f"C2 {name} {n}x{k}")
    rows = None
    if n > 50000:
        rows = np.unique(np.random.default_rng(65).integers(0, n, size=4096))
        rows = np.concatenate([rows, [0, n - 1]])
    err = _config_dense(dev, 2, q.Q8_0, oracle.X_BF16, n, k, 1, j, rows=rows)
    assert err <= TOL, err


# one token over short rows: each wave's whole weight stream requested at once.
# k = 4096 / 2560 / 9728 / 1056 give 8 / 10 / 19 / 33 steps per lane at 16 / 8 /
# 16 / 1 lanes per row (the last split over 4 waves: 9 per wave); rows ragged past
# the last tile
ONE_SHAPES = [(2060, 4096), (4100, 2560), (2000, 9728), (1000, 1056)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
def test_one_batch_path(dev, fmt, xt):
    O, V = q.PATH_VALU_ONE, q.PATH_VALU
    want = [O, O, V, O] if fmt == q.Q8_0 else [O, O, O, O]    # Q8_0 only up to 10 steps per wave
    for (n, k), path in zip(ONE_SHAPES, want):
        assert q.dense_path(fmt, n, k, xt, 1) == path, (n, k)
        say(f"one-batch fmt={fmt} xt={xt} n={n} k={k} path={path}")
        err = _config_dense(dev, 68, fmt, xt, n, k, 1, n % 89)
        assert err <= TOL, (n, k, err)


@pytest.mark.parametrize("fmt", [q.Q4_0, q.MXFP4])
@pytest.mark.parametrize("m", [2, 3])
def test_one_batch_cobatch(dev, fmt, m):
    # the 4-bit formats' vector co-batches: one batch while the call's activation
    # blocks fit three per thread (m x k / 32 <= 768) in one window
    for n, k in ONE_SHAPES[:3]:
        for xt in (oracle.X_BF16, oracle.X_F32):
            path = q.dense_path(fmt, n, k, xt, m)
            if xt == oracle.X_BF16:
                assert path == (q.PATH_VALU_ONE if m * (k // 32) <= 768 else q.PATH_VALU), (n, k)
            say(f"one-batch co-batch fmt={fmt} m={m} xt={xt} n={n} k={k} path={path}")
            err = _config_dense(dev, 69, fmt, xt, n, k, m, n % 83)
            assert err <= TOL, (n, k, xt, err)


@pytest.mark.parametrize("fmt", [q.Q4_0, q.MXFP4])
@pytest.mark.parametrize("n,k", [(1100, 2560), (1000, 1056)])
def test_one_batch_matches_batched_bitwise(dev, fmt, n, k):
    # fp32 activations: two tokens take the one-batch kernel, four the batched one.
    # These shapes (16 and 1 lanes per row, >= 4 steps per lane, windows of >= 4
    # steps at four tokens, < 2048 tiles) get the same split-K (4 waves per tile)
    # at both token counts; each token's arithmetic is then the same, so are its bits
    assert q.dense_path(fmt, n, k, q.X_F32, 2) == q.PATH_VALU_ONE
    assert q.dense_path(fmt, n, k, q.X_F32, 4) == q.PATH_VALU
    say(f"one-batch vs batched fmt={fmt} n={n} k={k}")
    canon = wl.blocks_for(fmt, n, k, config=70, matrix=n % 79)
    x = draw_x((4, k), oracle.X_F32, 70, n % 79)
    w = packed_dev(fmt, canon, n, k, dev)
    xd = to_dev(x, dev)
    y4 = q.qgemv(fmt, w, n, k, xd)
    y2 = q.qgemv(fmt, w, n, k, xd[:2])
    torch.cuda.synchronize()
    assert torch.equal(y2, y4[:2])


@pytest.mark.parametrize("m", [2, 4, 8])
@pytest.mark.parametrize("name,n,k,j", [("qkv", 6144, 4096, 0), ("gate_up", 24576, 4096, 1),
                                        ("down", 4096, 12288, 2)])
def test_config3_cobatch(dev, m, name, n, k, j):
    say(f"C3 {name} m={m}")
    rows = np.arange(0, n, 3) if n > 8192 else None
    err = _config_dense(dev, 3, q.Q4_0, oracle.X_BF16, n, k, m, j, rows=rows)
    assert err <= TOL, err


# ---------------------------------------------------- activation range
def _range_case(dev, fmt, x32, xt, n, k, config=68):
    canon = wl.blocks_for(fmt, n, k, config=config, matrix=fmt)
    x = wl.f32_to_bf16_bits_rne(x32) if xt == oracle.X_BF16 else x32
    y = run_dense(fmt, canon, n, k, x, xt, dev)
    ref, l1 = oracle.gemv(fmt, canon, n, k, x, xt)
    return oracle.max_rel_err(y, ref, l1)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
@pytest.mark.parametrize("scale", [1e-30, 1e30])
def test_activation_magnitudes(dev, fmt, xt, scale):
    """Tiny and huge activations (every product stays a normal fp32 number)."""
    say(f"x magnitude fmt={fmt} xt={xt} scale={scale}")
    x32 = (wl.x_f32((3, 2048), wl.rng_for(68, 1, "x")) * np.float32(scale)).astype(np.float32)
    err = _range_case(dev, fmt, x32, xt, 257, 2048)
    assert err <= TOL, err


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
def test_mixed_range_activations(dev, fmt, xt):
    """Twelve decades of magnitude inside every block."""
    say(f"x mixed range fmt={fmt} xt={xt}")
    rng = wl.rng_for(68, 2, "x")
    x32 = (wl.x_f32((4, 4096), rng) * 10.0 ** rng.uniform(-6, 6, size=(4, 4096))).astype(np.float32)
    err = _range_case(dev, fmt, x32, xt, 129, 4096)
    assert err <= TOL, err


# ------------------------------------------------ matrix-core co-batches
# bf16 co-batches of 4..8 tokens on layouts of 1..8 lanes per row run on the
# matrix cores.  (n, k) pick each layout class: 33001 rows -> 1 lane per row,
# 20000 -> 2, 9001 -> 4, 5000 and 4100 -> 8 (odd tile counts leave a half
# unit); K = 12288 at 8 tokens needs several activation windows.  4090 and
# 4089 rows make 256 units, one workgroup per compute unit, whose plan takes
# the whole LDS: K = 12256 (383 blocks, a ragged last step and tile) in one
# window at 4 and 5 tokens, two at 8; K = 18400 at 4 tokens fills one window.
MFMA_SHAPES = [(33001, 256, 1), (20000, 2048, 2), (9001, 2048, 4), (5000, 2048, 8), (4100, 12288, 8),
               (4090, 12256, 8), (4089, 18400, 8)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k,L", MFMA_SHAPES)
@pytest.mark.parametrize("m", [4, 5, 8])
def test_mfma_cobatch(dev, fmt, n, k, L, m):
    say(f"mfma fmt={fmt} n={n} k={k} m={m}")
    assert q.layout(fmt, n, k)["lanes_per_row"] == L
    assert q.dense_path(fmt, n, k, q.X_BF16, m) == q.PATH_MFMA
    canon = wl.blocks_for(fmt, n, k, config=69, matrix=n)
    x = draw_x((m, k), oracle.X_BF16, 69, n)
    y = run_dense(fmt, canon, n, k, x, oracle.X_BF16, dev)
    ref, l1 = oracle.gemv(fmt, canon, n, k, x, oracle.X_BF16)
    err = oracle.max_rel_err(y, ref, l1)
    assert err <= TOL, err


# Eight-wave workgroups on 8 lanes per row (4+ tokens): the token counts the
# matrix-core test above does not draw, with a ragged last unit and two windows.
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(5000, 2048), (4090, 12256)])
@pytest.mark.parametrize("m", [6, 7])
def test_mfma_cobatch_wide_token_counts(dev, fmt, n, k, m):
    say(f"mfma wide fmt={fmt} n={n} k={k} m={m}")
    assert q.layout(fmt, n, k)["lanes_per_row"] == 8
    assert q.dense_path(fmt, n, k, q.X_BF16, m) == q.PATH_MFMA
    canon = wl.blocks_for(fmt, n, k, config=72, matrix=n + m)
    x = draw_x((m, k), oracle.X_BF16, 72, n + m)
    y = run_dense(fmt, canon, n, k, x, oracle.X_BF16, dev)
    ref, l1 = oracle.gemv(fmt, canon, n, k, x, oracle.X_BF16)
    err = oracle.max_rel_err(y, ref, l1)
    assert err <= TOL, err


# Two and three tokens run on the matrix cores wherever the one-batch vector
# kernel does not apply (long rows, or grids too large to be resident at once).
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k,m", [(4100, 12288, 3), (4089, 18400, 2), (4090, 12256, 3), (24576, 4096, 2)])
def test_mfma_cobatch_few_tokens(dev, fmt, n, k, m):
    say(f"mfma few tokens fmt={fmt} n={n} k={k} m={m}")
    assert q.dense_path(fmt, n, k, q.X_BF16, m) == q.PATH_MFMA
    canon = wl.blocks_for(fmt, n, k, config=69, matrix=n + m)
    x = draw_x((m, k), oracle.X_BF16, 69, n + m)
    y = run_dense(fmt, canon, n, k, x, oracle.X_BF16, dev)
    ref, l1 = oracle.gemv(fmt, canon, n, k, x, oracle.X_BF16)
    err = oracle.max_rel_err(y, ref, l1)
    assert err <= TOL, err


@pytest.mark.parametrize("fmt", FMTS)
def test_mfma_deterministic_and_token_consistent(dev, fmt):
    n, k = 9001, 2048
    say(f"mfma determinism fmt={fmt}")
    canon = wl.blocks_for(fmt, n, k, config=70, matrix=fmt)
    w = packed_dev(fmt, canon, n, k, dev)
    xb = draw_x((8, k), oracle.X_BF16, 70, fmt)
    x = bf16_dev(xb, dev)
    y8a = q.qgemv(fmt, w, n, k, x)
    y8b = q.qgemv(fmt, w, n, k, x)
    xr = x[:1].repeat(6, 1).contiguous()
    yr = q.qgemv(fmt, w, n, k, xr)
    y1 = q.qgemv(fmt, w, n, k, x[:1].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y8a, y8b)
    for t in range(1, 6):
        assert torch.equal(yr[0], yr[t]), t
    # a token's row from the matrix cores agrees with the single-token product
    ref, l1 = oracle.gemv(fmt, canon, n, k, xb[:1], oracle.X_BF16)
    assert oracle.max_rel_err(y8a[:1].cpu().numpy(), ref, l1) <= TOL
    assert oracle.max_rel_err(y1.cpu().numpy(), ref, l1) <= TOL


# ------------------------------------------------------------ properties
def test_deterministic_and_cobatch_invariant(dev):
    """Same call, same bits.  Co-batches of 2..8 tokens share one plan, so a
    token's row does not depend on its companions (bitwise).  A single token
    over these short rows runs without split-K (a different fp32 summation
    order), so it agrees with the co-batch within the bound, not bitwise."""
    fmt, n, k = q.Q4_0, 2560, 9728
    say("determinism")
    assert q.dense_path(fmt, n, k, q.X_BF16, 8) == q.PATH_VALU
    canon = wl.blocks_for(fmt, n, k, config=66, matrix=0)
    w = packed_dev(fmt, canon, n, k, dev)
    xb = draw_x((8, k), oracle.X_BF16, 66, 0)
    x = bf16_dev(xb, dev)
    y8a = q.qgemv(fmt, w, n, k, x)
    y8b = q.qgemv(fmt, w, n, k, x)
    pairs = [q.qgemv(fmt, w, n, k, x[t:t + 2].contiguous()) for t in range(0, 8, 2)]
    ys = [q.qgemv(fmt, w, n, k, x[t:t + 1].contiguous()) for t in range(8)]
    torch.cuda.synchronize()
    assert torch.equal(y8a, y8b)
    for t in range(8):
        assert torch.equal(y8a[t], pairs[t // 2][t % 2]), t
    ref, l1 = oracle.gemv(fmt, canon, n, k, xb, oracle.X_BF16)
    y1 = torch.cat(ys).cpu().numpy()
    assert oracle.max_rel_err(y1, ref, l1) <= TOL
    assert oracle.max_rel_err(y8a.cpu().numpy(), ref, l1) <= TOL
    # identical tokens give identical rows
    xr = x[:1].repeat(4, 1).contiguous()
    yr = q.qgemv(fmt, w, n, k, xr)
    torch.cuda.synchronize()
    for t in range(1, 4):
        assert torch.equal(yr[0], yr[t])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 5])
def test_every_output_written_and_nothing_else(dev, fmt, m):
    n, k = 333, 2048
    say(f"canary fmt={fmt} m={m}")
    canon = wl.blocks_for(fmt, n, k, config=67, matrix=fmt)
    w = packed_dev(fmt, canon, n, k, dev)
    x = bf16_dev(draw_x((m, k), oracle.X_BF16, 67, fmt), dev)
    guard = 256
    buf = torch.full((m * n + 2 * guard,), float("nan"), device=dev)
    buf[:guard] = 12345.0
    buf[-guard:] = -54321.0
    y = buf[guard:guard + m * n].view(m, n)
    q.qgemv(fmt, w, n, k, x, y=y)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    assert torch.all(buf[:guard] == 12345.0) and torch.all(buf[-guard:] == -54321.0)


def test_linearity(dev):
    fmt, n, k = q.MXFP4, 512, 2048
    say("linearity")
    canon = wl.blocks_for(fmt, n, k, config=68, matrix=0)
    w = packed_dev(fmt, canon, n, k, dev)
    x = to_dev(draw_x((2, k), oracle.X_F32, 68, 0), dev)
    y = q.qgemv(fmt, w, n, k, x)
    yc = q.qgemv(fmt, w, n, k, (0.5 * x[0] - 2.0 * x[1]).reshape(1, k).contiguous())
    torch.cuda.synchronize()
    _, l1 = oracle.gemv(fmt, canon, n, k, x.cpu().numpy(), oracle.X_F32)
    lhs = yc[0].double().cpu().numpy()
    rhs = 0.5 * y[0].double().cpu().numpy() - 2.0 * y[1].double().cpu().numpy()
    assert np.max(np.abs(lhs - rhs) / (0.5 * l1[0] + 2.0 * l1[1])) <= 2 * TOL


# -------------------------------------------------------------------- MoE
def _experts(fmt, E, n, k, config, poison=None):
    mats = []
    for e in range(E):
        b = wl.blocks_for(fmt, n, k, config=config, matrix=1000 + e).reshape(n, k // 32, -1).copy()
        if poison is not None and e in poison:
            if fmt == q.MXFP4:
                b[:, :, 0] = 255                        # NaN scale
            else:
                b[:, :, 0], b[:, :, 1] = 0x00, 0x7E     # fp16 NaN
        mats.append(b.reshape(-1))
    return np.concatenate(mats)


def _experts_dev(fmt, experts, E, n, k, dev):
    pb = q.packed_bytes(fmt, n, k)
    out = torch.empty(E * pb, dtype=torch.uint8, device=dev)
    per = n * (k // 32) * q.BLOCK_BYTES[fmt]
    for e in range(E):
        q.pack(fmt, to_dev(experts[e * per:(e + 1) * per], dev), n, k, out=out[e * pb:(e + 1) * pb])
    return out


def _moe_case(dev, fmt, E, n, k, ids, g, xt, mode, config, poison=None):
    m, top_k = ids.shape
    experts = _experts(fmt, E, n, k, config, poison)
    wexp = _experts_dev(fmt, experts, E, n, k, dev)
    shape = (m, k) if mode == q.MOE_GATE_UP else (m, top_k, k)
    x = draw_x(shape, xt, config, 0, "x" if mode == q.MOE_GATE_UP else "h")
    y = q.moe_qgemv_topk(fmt, wexp, E, n, k, to_dev(ids, dev), to_dev(g, dev), x_dev(x, xt, dev), mode)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    ref, l1 = oracle.moe(fmt, experts, E, n, k, ids, g, x, xt, mode)
    return y, ref, l1


@pytest.mark.parametrize("m", [1, 4])
@pytest.mark.parametrize("mode", [q.MOE_GATE_UP, q.MOE_DOWN_COMBINE])
def test_config4_moe(dev, m, mode):
    c = wl.CONFIGS[4]
    E, top_k = c["n_experts"], c["top_k"]
    n, k = (3584, 2048) if mode == q.MOE_GATE_UP else (2048, 1792)
    say(f"C4 m={m} mode={mode}")
    _, ids, g = wl.router_topk(m, E, top_k, wl.rng_for(4, m, "router"))
    y, ref, l1 = _moe_case(dev, q.MXFP4, E, n, k, ids, g, oracle.X_BF16, mode, 4)
    assert oracle.max_rel_err(y, ref, l1) <= TOL


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
@pytest.mark.parametrize("mode", [q.MOE_GATE_UP, q.MOE_DOWN_COMBINE])
def test_moe_formats_and_shapes(dev, fmt, xt, mode):
    E, n, k, m, top_k = 6, 130, 608, 8, 3
    say(f"moe fmt={fmt} xt={xt} mode={mode}")
    _, ids, g = wl.router_topk(m, E, top_k, wl.rng_for(69, fmt, "router"))
    y, ref, l1 = _moe_case(dev, fmt, E, n, k, ids, g, xt, mode, 69)
    assert oracle.max_rel_err(y, ref, l1) <= TOL


# Few tiles: down-combine of several tokens in eight-wave workgroups (all of
# them splitting one tile's items), gate_up of several tokens over short items
# in four-wave splits with batches of 4 steps, and one token with fewer items
# than waves (top-1 / 2 / 4); token counts and top-k around those paths.
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(200, 4096), (2048, 1792), (136, 608)])
@pytest.mark.parametrize("m,top_k", [(1, 1), (1, 2), (1, 4), (2, 1), (3, 8), (5, 4), (8, 8)])
@pytest.mark.parametrize("mode", [q.MOE_GATE_UP, q.MOE_DOWN_COMBINE])
def test_moe_several_tokens_few_tiles(dev, fmt, n, k, m, top_k, mode):
    E = 12
    say(f"moe few tiles fmt={fmt} n={n} k={k} m={m} top_k={top_k} mode={mode}")
    _, ids, g = wl.router_topk(m, E, top_k, wl.rng_for(71, m * 16 + top_k, "router"))
    y, ref, l1 = _moe_case(dev, fmt, E, n, k, ids, g, oracle.X_BF16, mode, 71)
    assert oracle.max_rel_err(y, ref, l1) <= TOL


def test_moe_reads_only_selected_experts(dev):
    """Unselected experts carry NaN scales; the outputs must stay finite."""
    fmt, E, n, k = q.MXFP4, 32, 256, 512
    say("moe poison")
    ids = np.array([[3, 17, 5, 30], [17, 3, 9, 0]], dtype=np.int32)
    g = np.array([[0.4, 0.3, 0.2, 0.1], [0.25, 0.25, 0.25, 0.25]], dtype=np.float32)
    poison = set(range(E)) - set(ids.reshape(-1).tolist())
    for mode in (q.MOE_GATE_UP, q.MOE_DOWN_COMBINE):
        y, ref, l1 = _moe_case(dev, fmt, E, n, k, ids, g, oracle.X_BF16, mode, 70, poison=poison)
        assert np.isfinite(y).all()
        assert oracle.max_rel_err(y, ref, l1) <= TOL


def test_moe_all_tokens_same_experts(dev):
    fmt, E, n, k, m = q.Q4_0, 8, 192, 1024, 8
    say("moe shared experts")
    ids = np.tile(np.array([[6, 1]], dtype=np.int32), (m, 1))
    g = np.tile(np.array([[0.7, 0.3]], dtype=np.float32), (m, 1))
    for mode in (q.MOE_GATE_UP, q.MOE_DOWN_COMBINE):
        y, ref, l1 = _moe_case(dev, fmt, E, n, k, ids, g, oracle.X_BF16, mode, 71)
        assert oracle.max_rel_err(y, ref, l1) <= TOL


@pytest.mark.parametrize("fmt", FMTS)
def test_moe_repeated_expert_in_a_token(dev, fmt):
    """Ids repeated inside a token (outside the documented precondition) still
    follow the definition: expert 5 takes 6 of 8 slots, more than one work
    item's worth for two tokens."""
    E, n, k = 8, 200, 512
    say(f"moe repeated ids fmt={fmt}")
    ids = np.array([[5, 5, 5, 5], [5, 2, 5, 2]], dtype=np.int32)
    g = np.array([[0.1, 0.2, 0.3, 0.4], [0.4, 0.3, 0.2, 0.1]], dtype=np.float32)
    for mode in (q.MOE_GATE_UP, q.MOE_DOWN_COMBINE):
        y, ref, l1 = _moe_case(dev, fmt, E, n, k, ids, g, oracle.X_BF16, mode, 73)
        assert oracle.max_rel_err(y, ref, l1) <= TOL, mode


def test_moe_invalid_ids_contribute_nothing(dev):
    """An id outside [0, n_experts) adds nothing to down-combine and leaves its
    gate_up rows untouched."""
    fmt, E, n, k = q.MXFP4, 8, 256, 1024
    say("moe invalid ids")
    ids = np.array([[3, -1, 7, 40], [1, 3, 99, 2]], dtype=np.int32)
    g = np.array([[0.4, 0.3, 0.2, 0.1], [0.25, 0.25, 0.25, 0.25]], dtype=np.float32)
    valid = (ids >= 0) & (ids < E)
    experts = _experts(fmt, E, n, k, 74)
    wexp = _experts_dev(fmt, experts, E, n, k, dev)
    ids_ref = np.where(valid, ids, 0).astype(np.int32)
    g_ref = np.where(valid, g, 0).astype(np.float32)
    h = draw_x((2, 4, k), oracle.X_BF16, 74, 0, "h")
    y = q.moe_qgemv_topk(fmt, wexp, E, n, k, to_dev(ids, dev), to_dev(g, dev), x_dev(h, oracle.X_BF16, dev),
                         q.MOE_DOWN_COMBINE)
    ref, l1 = oracle.moe(fmt, experts, E, n, k, ids_ref, g_ref, h, oracle.X_BF16, q.MOE_DOWN_COMBINE)
    assert oracle.max_rel_err(y.cpu().numpy(), ref, l1) <= TOL
    x = draw_x((2, k), oracle.X_BF16, 74, 0, "x")
    yg = torch.full((2, 4, n), float("nan"), device=dev)
    q.moe_qgemv_topk(fmt, wexp, E, n, k, to_dev(ids, dev), None, x_dev(x, oracle.X_BF16, dev), q.MOE_GATE_UP, y=yg)
    yg = yg.cpu().numpy()
    ref, l1 = oracle.moe(fmt, experts, E, n, k, ids_ref, g_ref, x, oracle.X_BF16, q.MOE_GATE_UP)
    assert np.isnan(yg[~valid]).all()
    assert oracle.max_rel_err(yg[valid], ref[valid], l1[valid]) <= TOL


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mode", [q.MOE_GATE_UP, q.MOE_DOWN_COMBINE])
def test_moe_general_kernels(dev, fmt, mode):
    """Activation rows too large to stage at once (fp32, 8 tokens x 8 slots or
    K = 8192) take the kernels that stage per expert in windows."""
    E, n, m, top_k = 16, 130, 8, 8
    k = 8192 if mode == q.MOE_GATE_UP else 4096
    say(f"moe general fmt={fmt} mode={mode}")
    _, ids, g = wl.router_topk(m, E, top_k, wl.rng_for(75, fmt, "router"))
    y, ref, l1 = _moe_case(dev, fmt, E, n, k, ids, g, oracle.X_F32, mode, 75)
    assert oracle.max_rel_err(y, ref, l1) <= TOL


def test_moe_deterministic(dev):
    fmt, E, n, k, m, top_k = q.MXFP4, 32, 2048, 1792, 4, 4
    say("moe determinism")
    _, ids, g = wl.router_topk(m, E, top_k, wl.rng_for(72, 0, "router"))
    experts = _experts(fmt, E, n, k, 72)
    wexp = _experts_dev(fmt, experts, E, n, k, dev)
    h = bf16_dev(draw_x((m, top_k, k), oracle.X_BF16, 72, 0, "h"), dev)
    tid, tw = to_dev(ids, dev), to_dev(g, dev)
    a = q.moe_qgemv_topk(fmt, wexp, E, n, k, tid, tw, h, q.MOE_DOWN_COMBINE)
    b = q.moe_qgemv_topk(fmt, wexp, E, n, k, tid, tw, h, q.MOE_DOWN_COMBINE)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------------ router
def _router_check(dev, logits_np, top_k):
    lg = to_dev(logits_np.astype(np.float32), dev)
    ids, w = q.moe_router_topk(lg, top_k)
    torch.cuda.synchronize()
    ref_in = np.where(np.isnan(logits_np), -np.inf, logits_np).astype(np.float32)
    rid, rw = oracle.router_topk(ref_in, top_k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    got = w.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - rw) <= 1e-6 * rw + 1e-7), np.max(np.abs(got - rw))


@pytest.mark.parametrize("m,E,k", [(1, 32, 4), (4, 32, 4), (8, 128, 8), (1000, 64, 2), (3, 1024, 64),
                                   (5, 7, 7), (2, 1, 1), (6, 100, 1)])
def test_router_matches_oracle(dev, m, E, k):
    say(f"router m={m} E={E} k={k}")
    _router_check(dev, wl.x_f32((m, E), wl.rng_for(76, E, "router")), k)


def test_router_ties_and_special_values(dev):
    """Many equal logits (lower id first), -inf entries and NaN (ranked as -inf)."""
    say("router ties")
    rng = np.random.default_rng(77)
    lg = rng.integers(-2, 3, size=(64, 40)).astype(np.float32)
    lg[3, :] = 0.0
    lg[5, ::3] = -np.inf
    lg[7, 1::4] = np.nan
    for k in (1, 4, 13, 40):
        _router_check(dev, lg, k)


def test_router_feeds_expert_product(dev):
    """Device routing straight into the expert product (C4 shapes): ids and
    weights never leave the device; the result matches the oracle routed on
    the same logits."""
    c = wl.CONFIGS[4]
    E, top_k, m = c["n_experts"], c["top_k"], 4
    fmt, n, k = q.MXFP4, 2048, 1792
    say("router -> moe down")
    logits = wl.x_f32((m, E), wl.rng_for(78, 0, "router"))
    ids, w = q.moe_router_topk(to_dev(logits, dev), top_k)
    experts = _experts(fmt, E, n, k, 78)
    wexp = _experts_dev(fmt, experts, E, n, k, dev)
    h = draw_x((m, top_k, k), oracle.X_BF16, 78, 0, "h")
    y = q.moe_qgemv_topk(fmt, wexp, E, n, k, ids, w, x_dev(h, oracle.X_BF16, dev), q.MOE_DOWN_COMBINE)
    torch.cuda.synchronize()
    rid, rw = oracle.router_topk(logits, top_k)
    ref, l1 = oracle.moe(fmt, experts, E, n, k, rid.astype(np.int32), rw.astype(np.float32), h, oracle.X_BF16,
                         q.MOE_DOWN_COMBINE)
    assert oracle.max_rel_err(y.cpu().numpy(), ref, l1) <= TOL
