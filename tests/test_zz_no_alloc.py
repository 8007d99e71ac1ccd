"""qgemv_chain_noalloc, the chain entry point that allocates nothing, against
qgemv_chain with the same plan, both called through the C ABI: identical
output bits on two calls in a row (the second a smaller chain, so a longer
plan is left behind in the static buffer), each also within the oracle's
bar; and its plan-size limit, at the largest accepted plan and one link
beyond it."""
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


def _make(dev, fmt, shapes, config):
    mats = []
    for j, (n, k) in enumerate(shapes):
        canon = wl.blocks_for(fmt, n, k, config=config, matrix=j)
        xb = wl.x_bf16_bits((1, k), wl.rng_for(config, j, "x"))
        x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        w = q.pack(fmt, torch.from_numpy(canon.reshape(-1)).to(dev), n, k)
        y = torch.full((1, n), float("nan"), device=dev)
        mats.append((canon, xb, w, x, y, n, k))
    return mats


def _bits(t):
    return t.view(torch.int32).cpu().numpy().copy()


def _both_ways(fmt, mats):
    """Runs the chain through qgemv_chain, then through qgemv_chain_noalloc
    into NaN-filled outputs; returns the outputs of each, as bits."""
    ch = q.Chain(fmt, [(w, n, k, x, y) for (_, _, w, x, y, n, k) in mats])
    ch.run()
    torch.cuda.synchronize()
    assert q.chain_error() == 0
    ref = [_bits(y) for (*_, y, _n, _k) in mats]
    for (*_, y, _n, _k) in mats:
        y.fill_(float("nan"))
    ch.run_noalloc()
    torch.cuda.synchronize()
    assert q.chain_error() == 0
    got = [_bits(y) for (*_, y, _n, _k) in mats]
    return ch, ref, got


def _oracle_check(fmt, mats):
    for canon, xb, _, _, y, n, k in mats:
        ref, l1 = oracle.gemv(fmt, canon, n, k, xb, oracle.X_BF16)
        assert oracle.max_rel_err(y.cpu().numpy(), ref, l1) <= TOL, (n, k)


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0, q.MXFP4])
def test_noalloc_matches_chain_on_two_calls(dev, fmt):
    big = [(640, 256), (300, 2048), (129, 608), (2560, 1024), (1000, 96), (64, 4096), (6144, 2560)]
    small = [(96, 512), (33, 64)]
    say(f"noalloc fmt={fmt}: first call, {len(big)} links")
    mats = _make(dev, fmt, big, config=95)
    ch1, ref, got = _both_ways(fmt, mats)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    _oracle_check(fmt, mats)
    say(f"noalloc fmt={fmt}: second call, {len(small)} links")
    mats2 = _make(dev, fmt, small, config=96)
    _, ref2, got2 = _both_ways(fmt, mats2)
    for a, b in zip(ref2, got2):
        assert np.array_equal(a, b)
    _oracle_check(fmt, mats2)
    # and the longer chain again after the shorter one overwrote the buffer's start
    for (*_, y, _n, _k) in mats:
        y.fill_(float("nan"))
    ch1.run_noalloc()
    torch.cuda.synchronize()
    assert q.chain_error() == 0
    for a, (*_, y, _n, _k) in zip(ref, mats):
        assert np.array_equal(a, _bits(y))


def test_noalloc_plan_size_limit(dev):
    n, k = 64, 64
    fmt = q.Q8_0
    canon = wl.blocks_for(fmt, n, k, config=97, matrix=0)
    w = q.pack(fmt, torch.from_numpy(canon.reshape(-1)).to(dev), n, k)
    xb = wl.x_bf16_bits((1, k), wl.rng_for(97, 0, "x"))
    x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    most = (q.CHAIN_STATIC_BYTES - q.lib().qg_chain_plan_bytes(1)) // (
        q.lib().qg_chain_plan_bytes(2) - q.lib().qg_chain_plan_bytes(1)) + 1
    assert q.lib().qg_chain_plan_bytes(most) <= q.CHAIN_STATIC_BYTES < q.lib().qg_chain_plan_bytes(most + 1)
    say(f"noalloc limit: {most} links accepted")
    ys = torch.full((most + 1, n), float("nan"), device=dev)
    ch = q.Chain(fmt, [(w, n, k, x, ys[i]) for i in range(most)])
    ch.run_noalloc()
    torch.cuda.synchronize()
    assert q.chain_error() == 0
    ref, l1 = oracle.gemv(fmt, canon, n, k, xb, oracle.X_BF16)
    out = ys[:most].cpu().numpy()
    assert oracle.max_rel_err(out, np.repeat(ref, most, axis=0), np.repeat(l1, most, axis=0)) <= TOL
    assert np.array_equal(out.view(np.int32), np.repeat(out[:1], most, axis=0).view(np.int32))
    say(f"noalloc limit: {most + 1} links refused")
    over = q.Chain(fmt, [(w, n, k, x, ys[i]) for i in range(most + 1)])
    with pytest.raises(q.QGError) as e:
        over.run_noalloc()
    assert e.value.status == q.QG_EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(ys[most]).all()
