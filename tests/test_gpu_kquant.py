"""GPU parity of the K-quant path (Q4_K and Q6_K super-blocks: the GGUF
formats of the imp engine's models, imp README "Features" table,
Quantization row; imp release notes v0.7.0, Q4_K_M) against the fp64 oracle:
packing, decoding, the dense product at small and decode shapes, zero
weights, closed forms, and the entry points that refuse these formats."""
import numpy as np
import pytest

import oracle
import workloads as wl
from kq_blocks import q4k_block, q6k_block

torch = pytest.importorskip("torch")
q = pytest.importorskip("block_quantized_weight_amd")

pytestmark = pytest.mark.gpu
TOL = 2e-3
CFG = 88
FMTS = [q.Q4_K, q.Q6_K]


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


def x_of(shape, xt, seed, dev, mixed=False):
    rng = wl.rng_for(CFG, seed, "x")
    xf = wl.x_mixed_f32(shape, rng) if mixed else wl.x_f32(shape, rng)
    if xt == oracle.X_BF16:
        xb = wl.f32_to_bf16_bits_rne(xf)
        return xb, to_dev(xb, dev).view(torch.int16).view(torch.bfloat16)
    return xf, to_dev(xf, dev)


def packed_of(fmt, canon, n, k, dev):
    return q.pack(fmt, to_dev(canon.reshape(-1), dev), n, k)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(1, 256), (65, 768), (300, 2560), (19, 9728)])
def test_pack_matches_host_and_round_trips(dev, fmt, n, k):
    say(f"kq pack fmt={fmt} n={n} k={k}")
    canon = wl.blocks_for(fmt, n, k, config=CFG, matrix=n).reshape(-1)
    host = q.pack_host(fmt, canon, n, k)
    junk = torch.full((q.packed_bytes(fmt, n, k),), 0xAB, dtype=torch.uint8, device=dev)
    q.pack(fmt, to_dev(canon, dev), n, k, out=junk)
    assert np.array_equal(junk.cpu().numpy(), host)
    back = q.unpack(fmt, junk, n, k)
    assert np.array_equal(back.cpu().numpy(), canon)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_is_the_rounded_exact_weight(dev, fmt):
    n, k = 131, 1024
    say(f"kq dequant fmt={fmt}")
    canon = wl.blocks_for(fmt, n, k, config=CFG, matrix=3)
    w = q.dequant_f32(fmt, packed_of(fmt, canon, n, k, dev), n, k).cpu().numpy()
    ref = oracle.decode(fmt, canon, n, k).astype(np.float32)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


SHAPES = [(1, 256), (5, 512), (65, 768), (300, 2560), (1000, 4096), (64, 9728), (7, 12288)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
@pytest.mark.parametrize("m", [1, 3, 8])
def test_dense_shapes(dev, fmt, xt, m):
    for n, k in SHAPES:
        say(f"kq dense fmt={fmt} n={n} k={k} m={m} xt={xt}")
        canon = wl.blocks_for(fmt, n, k, config=CFG, matrix=n + k)
        w = packed_of(fmt, canon, n, k, dev)
        x, xd = x_of((m, k), xt, n + k, dev)
        y = q.qgemv(fmt, w, n, k, xd)
        torch.cuda.synchronize()
        ref, l1 = oracle.gemv(fmt, canon, n, k, x, xt)
        err = oracle.max_rel_err(y.cpu().numpy(), ref, l1)
        assert err <= TOL, (n, k, err)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k,m", [(6144, 2560, 1), (2560, 9728, 1), (19456, 2560, 1), (2560, 4096, 4),
                                   (151936, 2560, 1)])
def test_decode_shapes(dev, fmt, n, k, m):
    say(f"kq decode fmt={fmt} n={n} k={k} m={m} path={q.dense_path(fmt, n, k, q.X_BF16, m)}")
    canon = wl.blocks_for(fmt, n, k, config=2, matrix=7)
    w = packed_of(fmt, canon, n, k, dev)
    x, xd = x_of((m, k), oracle.X_BF16, 7, dev)
    y = q.qgemv(fmt, w, n, k, xd).cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, n, 97 if n < 100000 else 997), [n - 1]]))
    ref, l1 = oracle.gemv(fmt, canon, n, k, x, oracle.X_BF16, rows=rows)
    assert oracle.max_rel_err(y[:, rows], ref, l1) <= TOL


def _rows_of(blocks_per_row, n):
    return np.concatenate([np.concatenate(blocks_per_row(r)) for r in range(n)])


@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
def test_zero_weights_exactly_zero(dev, xt):
    """Rows whose every weight is zero give exactly 0 and mixed rows stay
    within the bar: Q4_K with d sc q == dmin m for the only code present
    (nonzero scales and mins), Q4_K with zero scales and mins, Q6_K with every
    code 32; against activations spread over six decades."""
    n, k = 12, 1024
    rng = np.random.default_rng(41)
    cases = {
        q.Q4_K: lambda r: [q4k_block(2.0 ** -6, 2.0 ** -6, [(3, 27)] * 8,
                                     np.full(256, 9) if r % 3 == 0 else rng.integers(0, 16, 256))
                           if r % 3 != 1 else q4k_block(0.5, 0.25, [(0, 0)] * 8, rng.integers(0, 16, 256))
                           for _ in range(k // 256)],
        q.Q6_K: lambda r: [q6k_block(0.75, rng.integers(-128, 128, 16),
                                     np.full(256, 32) if r % 2 == 0 else rng.integers(0, 64, 256))
                           for _ in range(k // 256)],
    }
    for fmt, make in cases.items():
        say(f"kq zero rows fmt={fmt} xt={xt}")
        canon = _rows_of(make, n)
        w = packed_of(fmt, canon, n, k, dev)
        x, xd = x_of((2, k), xt, 41, dev, mixed=True)
        y = q.qgemv(fmt, w, n, k, xd).cpu().numpy()
        ref, l1 = oracle.gemv(fmt, canon, n, k, x, xt)
        zero = l1 == 0
        assert zero.any()
        assert np.all(y[zero] == 0.0)
        assert oracle.max_rel_err(y, ref, l1) <= TOL


@pytest.mark.parametrize("fmt", FMTS)
def test_all_equal_rows(dev, fmt):
    """Every weight equal: each output is that weight times the sum of x."""
    n, k = 70, 2560
    if fmt == q.Q4_K:
        sb = q4k_block(2.0 ** -7, 2.0 ** -9, [(5, 3)] * 8, np.full(256, 11))
    else:
        sb = q6k_block(2.0 ** -8, np.full(16, -7), np.full(256, 45))
    canon = np.tile(sb, n * k // 256)
    w = packed_of(fmt, canon, n, k, dev)
    x, xd = x_of((1, k), oracle.X_F32, 42, dev)
    y = q.qgemv(fmt, w, n, k, xd).cpu().numpy()
    ref, l1 = oracle.gemv(fmt, canon, n, k, x, oracle.X_F32)
    assert oracle.max_rel_err(y, ref, l1) <= TOL
    assert np.all(y == y[0, 0])                 # every row the same bits


@pytest.mark.parametrize("fmt", FMTS)
def test_deterministic(dev, fmt):
    n, k = 2560, 9728
    canon = wl.blocks_for(fmt, n, k, config=CFG, matrix=5)
    w = packed_of(fmt, canon, n, k, dev)
    _, xd = x_of((1, k), oracle.X_BF16, 5, dev)
    a = q.qgemv(fmt, w, n, k, xd)
    b = q.qgemv(fmt, w, n, k, xd)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("fmt", FMTS)
def test_other_entry_points_refuse(dev, fmt):
    n, k = 64, 256
    w = torch.zeros(q.packed_bytes(fmt, n, k), dtype=torch.uint8, device=dev)
    x = torch.zeros((1, k), dtype=torch.bfloat16, device=dev)
    for call in (lambda: q.qgemv_fused(fmt, w, n, k, x, residual=torch.zeros((1, n), device=dev)),
                 lambda: q.qgemm(fmt, w, n, k, torch.zeros((16, k), dtype=torch.bfloat16, device=dev)),
                 lambda: q.moe_qgemv_topk(fmt, w, 1, n, k, torch.zeros((1, 1), dtype=torch.int32, device=dev),
                                          torch.ones((1, 1), device=dev), x, q.MOE_GATE_UP)):
        with pytest.raises(q.QGError) as e:
            call()
        assert e.value.status == q.QG_EUNSUPPORTED
    with pytest.raises(q.QGError) as e:
        q.gemm_path(fmt, n, k, q.X_BF16, 16)
    assert e.value.status == q.QG_EUNSUPPORTED
