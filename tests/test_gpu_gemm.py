"""GPU parity of qgemm (1..128 tokens, through the C ABI) against the fp64
oracle: every layout class the matrix cores serve (1, 2, 4, 8 and 16 lanes
per row), partial token groups, several activation windows, the dense-pass
fallback (fp32 activations, 32+ lanes per row), and the workload shapes at
full size on sampled rows.  Bar: max |y - y_oracle| / L1(row) <= 2e-3."""
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


def x_dev(x, xt, dev):
    if xt == oracle.X_BF16:
        return to_dev(np.ascontiguousarray(x).view(np.int16), dev).view(torch.bfloat16)
    return to_dev(x, dev)


def draw_x(shape, xt, config, matrix):
    rng = wl.rng_for(config, matrix, "x")
    return wl.x_bf16_bits(shape, rng) if xt == oracle.X_BF16 else wl.x_f32(shape, rng)


def run(fmt, n, k, m, xt, dev, config, rows=None):
    canon = wl.blocks_for(fmt, n, k, config=config, matrix=n % 97)
    x = draw_x((m, k), xt, config, n % 97)
    w = q.pack(fmt, to_dev(canon.reshape(-1), dev), n, k)
    y = q.qgemm(fmt, w, n, k, x_dev(x, xt, dev))
    torch.cuda.synchronize()
    ref, l1 = oracle.gemv(fmt, canon, n, k, x, xt, rows=rows)
    yh = y.cpu().numpy()
    if rows is not None:
        yh = yh[:, rows]
    return oracle.max_rel_err(yh, ref, l1), w, x


# (n, k) per layout class, ragged where the layout allows it
SHAPES = {1: (32768, 256), 2: (16384, 512), 4: (8192, 1280), 8: (4096, 1536), 16: (2048, 6144)}


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("lanes", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("m", [9, 16, 17, 40, 128])
def test_gemm_layout_classes(dev, fmt, lanes, m):
    n, k = SHAPES[lanes]
    assert q.layout(fmt, n, k)["lanes_per_row"] == lanes
    assert q.gemm_path(fmt, n, k, q.X_BF16, m) == q.PATH_MFMA
    say(f"gemm fmt={fmt} n={n} k={k} L={lanes} m={m}")
    rows = None if n * m <= 4096 * 40 else np.unique(np.concatenate([[0, n - 1], np.arange(3, n, 37)]))
    err, _, _ = run(fmt, n, k, m, oracle.X_BF16, dev, 170, rows)
    assert err <= TOL, err


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 5, 8, 12, 33, 100])
def test_gemm_ragged_rows_and_small_m(dev, fmt, m):
    # ragged row counts (tiles past the end, partial 16-row units)
    for n, k in [(1000, 256), (4100, 512), (2060, 4096)]:
        say(f"gemm ragged fmt={fmt} n={n} k={k} m={m}")
        err, _, _ = run(fmt, n, k, m, oracle.X_BF16, dev, 171)
        assert err <= TOL, (n, k, err)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_fallback_paths(dev, fmt):
    # fp32 activations, and a layout of 64 lanes per row: the dense product in passes of 8 tokens
    for n, k, xt in [(512, 1024, oracle.X_F32), (300, 4096, oracle.X_BF16)]:
        m = 20
        assert q.gemm_path(fmt, n, k, xt, m) == q.PATH_VALU
        say(f"gemm fallback fmt={fmt} n={n} k={k} xt={xt}")
        err, _, _ = run(fmt, n, k, m, xt, dev, 172)
        assert err <= TOL, err


def test_gemm_matches_token_by_token_and_is_deterministic(dev):
    # every token group gives each token's row as a co-batch call of that token alone
    # would, within the bound; repeated calls are bitwise equal
    fmt, n, k, m = q.Q4_0, 4096, 1024, 37
    err, w, x = run(fmt, n, k, m, oracle.X_BF16, dev, 173)
    assert err <= TOL
    xd = x_dev(x, oracle.X_BF16, dev)
    y1 = q.qgemm(fmt, w, n, k, xd)
    y2 = q.qgemm(fmt, w, n, k, xd)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    for t in (0, 16, 36):
        yt = q.qgemv(fmt, w, n, k, xd[t:t + 1])
        torch.cuda.synchronize()
        ref, l1 = oracle.gemv(fmt, wl.blocks_for(fmt, n, k, config=173, matrix=n % 97), n, k, x[t:t + 1],
                              oracle.X_BF16)
        assert oracle.max_rel_err(y1[t:t + 1].cpu().numpy(), ref, l1) <= TOL
        assert oracle.max_rel_err(yt.cpu().numpy(), ref, l1) <= TOL


FULL = [("c3 qkv", q.Q4_0, 6144, 4096), ("c3 gate_up", q.Q4_0, 24576, 4096), ("c3 down", q.Q4_0, 4096, 12288),
        ("c1 down", q.Q4_0, 2560, 9728), ("c2 gate_up", q.Q8_0, 19456, 2560), ("c4 gate_up", q.MXFP4, 3584, 2048)]


@pytest.mark.parametrize("case", FULL, ids=[f[0] for f in FULL])
def test_gemm_workload_shapes_sampled(dev, case):
    name, fmt, n, k = case
    m = 128
    say(f"gemm full {name} m={m}")
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(3).integers(0, n, 250)]))
    err, _, _ = run(fmt, n, k, m, oracle.X_BF16, dev, 174, rows)
    assert err <= TOL, err
