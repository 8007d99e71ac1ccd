"""Q4_0 rows dominated by zero weights (code 8), on every kernel family.

Each Q4_0 weight enters the dot product as its exact value (q - 8) times a
power of two, so a row's rounding error is bounded by its own sum of
|w * x| (the fp32 summation bound gamma_{K+2} * L1).  Rows whose codes are
all 8 must therefore give exactly 0 (the verdict fails any non-zero output
where L1 = 0), and rows with a single non-zero code must be exact to a few
ulp of that one product, even with activations spread over six decades.
The Q4_0 weight definition w = d * (q - 8) is the workload's (the pages name
the format only).  Also here: the all-equal-block closed form of every
format, y = d * v * sum(x), checked against that formula directly.
"""
import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
q = pytest.importorskip("block_quantized_weight_amd")

pytestmark = pytest.mark.gpu
TOL = 2e-3
CFG = 80
XKINDS = ["f32", "f32_mixed", "bf16", "bf16_mixed"]


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


def draw(shape, kind, matrix):
    """Activations of one kind: (array, xt) with bf16 as bit patterns."""
    rng = wl.rng_for(CFG, matrix, "x")
    x = wl.x_mixed_f32(shape, rng) if kind.endswith("mixed") else wl.x_f32(shape, rng)
    if kind.startswith("bf16"):
        return wl.f32_to_bf16_bits_rne(x), oracle.X_BF16
    return x, oracle.X_F32


def x_dev(x, xt, dev):
    t = to_dev(x, dev)
    return t.view(torch.int16).view(torch.bfloat16) if xt == oracle.X_BF16 else t


def zero_heavy(n, k, matrix):
    return wl.q4_0_zero_heavy_blocks(n, k, wl.rng_for(CFG, matrix, "codes"), wl.rng_for(CFG, matrix, "scales"))


def packed(canon, n, k, dev):
    return q.pack(q.Q4_0, to_dev(canon.reshape(-1), dev), n, k)


def check_rows(y, ref, l1):
    """The verdict, plus exact zeros on the all-8 rows (L1 = 0)."""
    zero = l1 == 0
    assert zero.any()
    assert np.all(y[zero] == 0.0)
    err = oracle.max_rel_err(y, ref, l1)
    assert err <= TOL, err
    return err


# (n, k, m, xt kinds, family): shapes picked so that each kernel family of the
# dense product serves them (qg_dense_path is asserted)
DENSE = [
    (2560, 9728, 1, ["f32", "f32_mixed", "bf16", "bf16_mixed"], q.PATH_VALU_ONE),
    (19456, 2560, 1, ["bf16", "bf16_mixed"], q.PATH_VALU_ONE),
    (2560, 9728, 2, ["bf16_mixed"], q.PATH_VALU_ONE),
    (24576, 4096, 1, ["bf16", "bf16_mixed"], q.PATH_VALU),
    (6144, 4096, 4, ["f32", "f32_mixed"], q.PATH_VALU),
    (1000, 12288, 8, ["f32_mixed", "bf16_mixed"], q.PATH_VALU),
    (6144, 4096, 4, ["bf16", "bf16_mixed"], q.PATH_MFMA),
    (5000, 2048, 8, ["bf16_mixed"], q.PATH_MFMA),
    (20000, 2048, 5, ["bf16_mixed"], q.PATH_MFMA),
]


@pytest.mark.parametrize("case", range(len(DENSE)))
def test_dense_zero_heavy(dev, case):
    n, k, m, kinds, family = DENSE[case]
    canon = zero_heavy(n, k, case)
    w = packed(canon, n, k, dev)
    for kind in kinds:
        x, xt = draw((m, k), kind, 100 * case + XKINDS.index(kind))
        assert q.dense_path(q.Q4_0, n, k, xt, m) == family, (kind, q.dense_path(q.Q4_0, n, k, xt, m))
        say(f"q4 zero-heavy dense n={n} k={k} m={m} x={kind} path={family}")
        y = q.qgemv(q.Q4_0, w, n, k, x_dev(x, xt, dev))
        torch.cuda.synchronize()
        ref, l1 = oracle.gemv(q.Q4_0, canon, n, k, x, xt)
        check_rows(y.cpu().numpy(), ref, l1)


@pytest.mark.parametrize("kind", ["f32_mixed", "bf16_mixed"])
@pytest.mark.parametrize("m", [1, 3])
def test_fused_rmsnorm_zero_heavy(dev, kind, m):
    """RMSNorm staging keeps x * gamma in fp32 and runs the fp32 inner product."""
    n, k = 2560, 9728
    say(f"q4 zero-heavy fused norm x={kind} m={m}")
    canon = zero_heavy(n, k, 20)
    w = packed(canon, n, k, dev)
    x, xt = draw((m, k), kind, 200 + m)
    gamma = wl.norm_weight_f32(k, wl.rng_for(CFG, 20, "gamma"))
    y = q.qgemv_fused(q.Q4_0, w, n, k, x_dev(x, xt, dev), norm_weight=to_dev(gamma, dev), eps=1e-6)
    torch.cuda.synchronize()
    o, scale = oracle.dense_fused(q.Q4_0, canon, n, k, x, xt, norm_weight=gamma, eps=1e-6)
    yy = y.cpu().numpy()
    assert np.all(yy[scale == 0] == 0.0)
    assert oracle.fused_err(yy, o, scale) <= TOL


def _moe(dev, E, n, k, ids, g, kind, mode, matrix):
    m, top_k = ids.shape
    mats = [zero_heavy(n, k, 1000 * matrix + e).reshape(-1) for e in range(E)]
    experts = np.concatenate(mats)
    pb = q.packed_bytes(q.Q4_0, n, k)
    wexp = torch.empty(E * pb, dtype=torch.uint8, device=dev)
    for e in range(E):
        q.pack(q.Q4_0, to_dev(mats[e], dev), n, k, out=wexp[e * pb:(e + 1) * pb])
    shape = (m, k) if mode == q.MOE_GATE_UP else (m, top_k, k)
    x, xt = draw(shape, kind, 300 + matrix)
    y = q.moe_qgemv_topk(q.Q4_0, wexp, E, n, k, to_dev(ids, dev), to_dev(g, dev), x_dev(x, xt, dev), mode)
    torch.cuda.synchronize()
    ref, l1 = oracle.moe(q.Q4_0, experts, E, n, k, ids, g, x, xt, mode)
    return y.cpu().numpy(), ref, l1


@pytest.mark.parametrize("mode", [q.MOE_GATE_UP, q.MOE_DOWN_COMBINE])
@pytest.mark.parametrize("kind", ["f32_mixed", "bf16", "bf16_mixed"])
@pytest.mark.parametrize("m", [1, 4])
def test_moe_zero_heavy(dev, mode, kind, m):
    """The streaming expert kernel.  For down-combine every slot of a token
    picks the same expert so that all-8 rows stay at L1 = 0 after combining."""
    E, top_k = 8, 2
    n, k = (512, 2048) if mode == q.MOE_GATE_UP else (256, 1792)
    say(f"q4 zero-heavy moe mode={mode} x={kind} m={m}")
    _, ids, g = wl.router_topk(m, E, top_k, wl.rng_for(CFG, 40 + m, "router"))
    y, ref, l1 = _moe(dev, E, n, k, ids, g, kind, mode, 40 + m)
    check_rows(y, ref, l1)


@pytest.mark.parametrize("mode", [q.MOE_GATE_UP, q.MOE_DOWN_COMBINE])
def test_moe_general_zero_heavy(dev, mode):
    """Activation rows too large to stage at once take the per-expert kernels."""
    E, n, m, top_k = 8, 130, 8, 8
    k = 8192 if mode == q.MOE_GATE_UP else 4096
    say(f"q4 zero-heavy moe general mode={mode}")
    _, ids, g = wl.router_topk(m, E, top_k, wl.rng_for(CFG, 50, "router"))
    y, ref, l1 = _moe(dev, E, n, k, ids, g, "f32_mixed", mode, 50)
    check_rows(y, ref, l1)


@pytest.mark.parametrize("kind", ["f32_mixed", "bf16_mixed"])
def test_qgemm_zero_heavy(dev, kind):
    n, k, m = 6144, 4096, 20
    say(f"q4 zero-heavy qgemm x={kind}")
    canon = zero_heavy(n, k, 60)
    w = packed(canon, n, k, dev)
    x, xt = draw((m, k), kind, 600)
    y = q.qgemm(q.Q4_0, w, n, k, x_dev(x, xt, dev))
    torch.cuda.synchronize()
    ref, l1 = oracle.gemv(q.Q4_0, canon, n, k, x, xt)
    check_rows(y.cpu().numpy(), ref, l1)


@pytest.mark.parametrize("kind", ["f32_mixed", "bf16_mixed"])
def test_chain_zero_heavy(dev, kind):
    shapes = [(2560, 4096), (640, 9728), (300, 2048)]
    say(f"q4 zero-heavy chain x={kind}")
    links, cases = [], []
    for j, (n, k) in enumerate(shapes):
        canon = zero_heavy(n, k, 70 + j)
        x, xt = draw((1, k), kind, 700 + j)
        w = packed(canon, n, k, dev)
        xd = x_dev(x, xt, dev)
        y = torch.full((1, n), float("nan"), device=dev)
        links.append((w, n, k, xd, y))
        cases.append((canon, x, xt, y, n, k))
    ch = q.Chain(q.Q4_0, links)
    ch.run()
    assert q.chain_error() == 0
    for canon, x, xt, y, n, k in cases:
        ref, l1 = oracle.gemv(q.Q4_0, canon, n, k, x, xt)
        check_rows(y.cpu().numpy(), ref, l1)


# ------------------------------------------- all-equal blocks, closed form
def _equal_blocks(fmt, n, k, code, scale):
    nb = k // 32
    if fmt == q.Q8_0:
        return wl.encode_q8_0(np.full((n, nb, 32), code, dtype=np.int8), np.full((n, nb), scale, dtype=np.uint16))
    if fmt == q.Q4_0:
        return wl.encode_q4_0(np.full((n, nb, 32), code, dtype=np.uint8), np.full((n, nb), scale, dtype=np.uint16))
    return wl.encode_mxfp4(np.full((n, nb, 32), code, dtype=np.uint8), np.full((n, nb), scale, dtype=np.uint8))


# (fmt, code, scale bits, value of one weight): fp16 0x1C00 = 2^-8; UE8M0 120 = 2^-7;
# E2M1 code 0xB = -1.5
EQUAL = [(q.Q8_0, -77, 0x1C00, -77 * 2.0 ** -8), (q.Q8_0, 0, 0x1C00, 0.0),
         (q.Q4_0, 13, 0x1C00, 5 * 2.0 ** -8), (q.Q4_0, 8, 0x1C00, 0.0), (q.Q4_0, 0, 0x2E66, -8 * 0.0999755859375),
         (q.MXFP4, 0xB, 120, -1.5 * 2.0 ** -7), (q.MXFP4, 0x8, 120, 0.0)]


@pytest.mark.parametrize("case", range(len(EQUAL)))
@pytest.mark.parametrize("kind", ["f32", "bf16_mixed"])
@pytest.mark.parametrize("m", [1, 4])
def test_all_equal_blocks_closed_form(dev, case, kind, m):
    """Every weight equal to v: y[t][r] = v * sum(x[t]) for every row, within
    2e-3 of |v| * sum|x| (exactly 0 when v = 0)."""
    fmt, code, scale, v = EQUAL[case]
    n, k = 384, 4096
    say(f"all-equal fmt={fmt} code={code} x={kind} m={m}")
    canon = _equal_blocks(fmt, n, k, code, scale)
    w = q.pack(fmt, to_dev(canon.reshape(-1), dev), n, k)
    x, xt = draw((m, k), kind, 800 + case)
    y = q.qgemv(fmt, w, n, k, x_dev(x, xt, dev)).cpu().numpy()
    xv = oracle.x_values(x, xt)
    want = v * xv.sum(axis=1)
    bound = abs(v) * np.abs(xv).sum(axis=1)
    for t in range(m):
        if v == 0.0:
            assert np.all(y[t] == 0.0)
        else:
            assert np.max(np.abs(y[t] - want[t])) <= TOL * bound[t]
