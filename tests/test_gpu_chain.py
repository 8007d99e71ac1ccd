"""GPU parity of the persistent chain kernel (qgemv_chain) against the fp64
oracle, plus ordering, determinism and barrier-health checks."""
import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
q = pytest.importorskip("block_quantized_weight_amd")

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def _bf16(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _make(dev, fmt, shapes, m, xt, config):
    mats = []
    for j, (n, k) in enumerate(shapes):
        canon = wl.blocks_for(fmt, n, k, config=config, matrix=j)
        rng = wl.rng_for(config, j, "x")
        xnp = wl.x_bf16_bits((m, k), rng) if xt == oracle.X_BF16 else wl.x_f32((m, k), rng)
        x = _bf16(xnp, dev) if xt == oracle.X_BF16 else torch.from_numpy(xnp).to(dev)
        w = q.pack(fmt, torch.from_numpy(canon.reshape(-1)).to(dev), n, k)
        y = torch.full((m, n), float("nan"), device=dev)
        mats.append((canon, xnp, w, x, y, n, k))
    return mats


def _check(fmt, mats, xt):
    worst = 0.0
    for canon, xnp, w, x, y, n, k in mats:
        ref, l1 = oracle.gemv(fmt, canon, n, k, xnp, xt)
        err = oracle.max_rel_err(y.cpu().numpy(), ref, l1)
        worst = max(worst, err)
        assert err <= TOL, (n, k, err)
    return worst


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0, q.MXFP4])
@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
@pytest.mark.parametrize("m", [1, 3])
def test_chain_mixed_shapes(dev, fmt, xt, m):
    shapes = [(640, 256), (1, 32), (300, 2048), (129, 608), (2560, 1024), (64, 4096), (1000, 96)]
    say(f"chain fmt={fmt} xt={xt} m={m}")
    mats = _make(dev, fmt, shapes, m, xt, 80 + fmt)
    ch = q.Chain(fmt, [(w, n, k, x, y) for _, _, w, x, y, n, k in mats])
    ch.run()
    torch.cuda.synchronize()
    assert q.chain_error() == 0
    _check(fmt, mats, xt)


def test_chain_decode_layer_shapes_repeated(dev):
    """Two layers of the Q8_0 decode sweep shapes, run several times: every run
    matches the oracle, runs are bitwise identical, and no barrier timed out."""
    fmt = q.Q8_0
    shapes = [(n, k) for _, _, n, k in wl.c2_sweep_shapes()[:8]]
    say("chain decode layers")
    mats = _make(dev, fmt, shapes, 1, oracle.X_BF16, 2)
    ch = q.Chain(fmt, [(w, n, k, x, y) for _, _, w, x, y, n, k in mats])
    outs = []
    for r in range(5):
        for _, _, _, _, y, _, _ in mats:
            y.fill_(float("nan"))
        ch.run()
        torch.cuda.synchronize()
        outs.append([y.clone() for _, _, _, _, y, _, _ in mats])
    assert q.chain_error() == 0
    _check(fmt, mats, oracle.X_BF16)
    for r in range(1, 5):
        for a, b in zip(outs[0], outs[r]):
            assert torch.equal(a, b)


def test_chain_many_links_and_relaunch(dev):
    """150 small links in one launch, then the same plan launched back to back."""
    fmt = q.Q4_0
    shapes = [((37 * j) % 700 + 1, 32 * ((j % 5) + 1)) for j in range(150)]
    say("chain 150 links")
    mats = _make(dev, fmt, shapes, 2, oracle.X_BF16, 81)
    ch = q.Chain(fmt, [(w, n, k, x, y) for _, _, w, x, y, n, k in mats])
    for _ in range(4):
        ch.run()
    torch.cuda.synchronize()
    assert q.chain_error() == 0
    _check(fmt, mats, oracle.X_BF16)


def test_chain_matches_single_launch_results(dev):
    fmt = q.MXFP4
    shapes = [(3584, 2048), (2048, 1792)]
    say("chain vs single")
    mats = _make(dev, fmt, shapes, 1, oracle.X_BF16, 82)
    ch = q.Chain(fmt, [(w, n, k, x, y) for _, _, w, x, y, n, k in mats])
    ch.run()
    torch.cuda.synchronize()
    for canon, xnp, w, x, y, n, k in mats:
        ys = q.qgemv(fmt, w, n, k, x)
        torch.cuda.synchronize()
        _, l1 = oracle.gemv(fmt, canon, n, k, xnp, oracle.X_BF16)
        d = (ys.double() - y.double()).abs().cpu().numpy()
        assert np.max(d / l1) <= 2 * TOL
    assert q.chain_error() == 0


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0])
def test_chain_dependent_links(dev, fmt):
    """Link i+1 reads link i's output as its activations (fp32), as consecutive
    projections of a decode step do.  Each link is checked against the oracle
    applied to the activations it was given (the previous link's output, read
    back), so a workgroup that read a stale activation vector fails.  The chain
    runs twice with different inputs, so stale values would differ."""
    shapes = [(2048, 1024), (1536, 2048), (4096, 1536), (1024, 4096), (3072, 1024), (640, 3072)]
    say(f"chain dependent links fmt={fmt}")
    canons, ws, ys = [], [], []
    for j, (n, k) in enumerate(shapes):
        canon = wl.blocks_for(fmt, n, k, config=83, matrix=j)
        canons.append(canon)
        ws.append(q.pack(fmt, torch.from_numpy(canon.reshape(-1)).to(dev), n, k))
        ys.append(torch.full((1, n), float("nan"), device=dev))
    x0 = torch.empty((1, shapes[0][1]), dtype=torch.float32, device=dev)
    xs = [x0] + ys[:-1]
    ch = q.Chain(fmt, [(w, n, k, x, y) for w, (n, k), x, y in zip(ws, shapes, xs, ys)])
    for run in range(2):
        x0.copy_(torch.from_numpy(wl.x_f32((1, shapes[0][1]), wl.rng_for(83, 100 + run, "x"))))
        ch.run()
        torch.cuda.synchronize()
        assert q.chain_error() == 0
        for j, (n, k) in enumerate(shapes):
            xin = xs[j].cpu().numpy()
            ref, l1 = oracle.gemv(fmt, canons[j], n, k, xin, oracle.X_F32)
            err = oracle.max_rel_err(ys[j].cpu().numpy(), ref, l1)
            assert err <= TOL, (run, j, err)
