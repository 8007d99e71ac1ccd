"""GPU parity of the fused dense product (qgemv_fused, through the C ABI)
against the fp64 oracle's definition (oracle.dense_fused): RMSNorm in the
staging, SwiGLU or a residual add in the epilogue, fp32 or bf16 outputs.

Bar: oracle.fused_err <= 2e-3 -- the product error measured against its
rounding scale (row L1 of |w x'|, and for SwiGLU the first-order propagation
through the gate) once the output's own rounding is allowed for.
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
NONE, SWIGLU = q.ACT_NONE, q.ACT_SWIGLU


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


def draw_x(shape, xt, config, matrix, scale):
    """Activations of RMS about `scale` (so that the normalisation matters)."""
    xf = (scale * wl.x_f32(shape, wl.rng_for(config, matrix, "x"))).astype(np.float32)
    return wl.f32_to_bf16_bits_rne(xf) if xt == oracle.X_BF16 else xf


def x_dev(x, xt, dev):
    if xt == oracle.X_BF16:
        return to_dev(np.ascontiguousarray(x).view(np.int16), dev).view(torch.bfloat16)
    return to_dev(x, dev)


def y_host(y):
    return y.float().cpu().numpy().astype(np.float64)


class Case:
    def __init__(self, fmt, n, k, m, xt, norm, act, res, ybf16, config=110, matrix=0, xscale=3.0):
        self.fmt, self.n, self.k, self.m, self.xt = fmt, n, k, m, xt
        self.norm, self.act, self.res, self.ybf16 = norm, act, res, ybf16
        self.n_out = n // 2 if act == SWIGLU else n
        self.canon = wl.blocks_for(fmt, n, k, config=config, matrix=matrix)
        self.x = draw_x((m, k), xt, config, matrix, xscale)
        self.gamma = wl.norm_weight_f32(k, wl.rng_for(config, matrix, "gamma")) if norm else None
        self.eps = 1e-5
        self.resid = wl.x_f32((m, self.n_out), wl.rng_for(config, matrix, "res")) if res else None

    def label(self):
        return (f"fused fmt={self.fmt} n={self.n} k={self.k} m={self.m} xt={self.xt} norm={self.norm} "
                f"act={self.act} res={self.res} ybf16={self.ybf16}")

    def run(self, dev, w=None, y=None):
        w = q.pack(self.fmt, to_dev(self.canon.reshape(-1), dev), self.n, self.k) if w is None else w
        y = q.qgemv_fused(self.fmt, w, self.n, self.k, x_dev(self.x, self.xt, dev),
                          norm_weight=None if self.gamma is None else to_dev(self.gamma, dev), eps=self.eps,
                          act=self.act, residual=None if self.resid is None else to_dev(self.resid, dev),
                          y=y, out_dtype=torch.bfloat16 if self.ybf16 else torch.float32)
        torch.cuda.synchronize()
        return w, y

    def oracle(self, rows=None):
        return oracle.dense_fused(self.fmt, self.canon, self.n, self.k, self.x, self.xt, norm_weight=self.gamma,
                                  eps=self.eps, act=self.act, residual=self.resid, rows=rows)


COMBOS = [  # norm, act, residual, bf16 out
    (False, NONE, False, False),
    (True, NONE, False, False),
    (False, SWIGLU, False, False),
    (True, SWIGLU, False, True),
    (False, NONE, True, False),
    (True, NONE, True, True),
    (True, SWIGLU, True, False),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xt", [oracle.X_BF16, oracle.X_F32])
@pytest.mark.parametrize("combo", COMBOS)
@pytest.mark.parametrize("m", [1, 3, 8])
def test_fused_parity_small(dev, fmt, xt, combo, m):
    norm, act, res, ybf16 = combo
    # several tiles and a ragged tail; SwiGLU halves of 576 rows (a multiple of 64)
    n, k = (1152, 1056) if act == SWIGLU else (1000, 1056)
    c = Case(fmt, n, k, m, xt, norm, act, res, ybf16, matrix=fmt * 10 + m)
    say(c.label())
    _, y = c.run(dev)
    o, scale = c.oracle()
    err = oracle.fused_err(y_host(y), o, scale, y_bf16=ybf16)
    assert err <= TOL, err


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_fused_plain_matches_qgemv_bitwise_on_the_vector_path(dev, fmt, m):
    # with nothing fused the kernel does the plain product's arithmetic
    n, k = 2304, 2048
    if q.dense_path(fmt, n, k, q.X_BF16, m) == q.PATH_MFMA:
        pytest.skip("plain product runs on the matrix cores at this m")
    c = Case(fmt, n, k, m, oracle.X_BF16, False, NONE, False, False, matrix=40 + m, xscale=1.0)
    say(c.label(), "vs qgemv")
    w, y = c.run(dev)
    yp = q.qgemv(fmt, w, n, k, x_dev(c.x, c.xt, dev))
    torch.cuda.synchronize()
    assert torch.equal(y, yp)


@pytest.mark.parametrize("fmt", [q.Q4_0, q.MXFP4])
@pytest.mark.parametrize("n,k", [(4100, 2560), (2000, 9728), (1000, 1056)])
@pytest.mark.parametrize("m", [1, 2])
def test_fused_plain_matches_one_batch_bitwise(dev, fmt, n, k, m):
    # one batch (one token: 10, 19 and 33/4 steps per wave): the fused call with
    # nothing fused runs the same pass as qgemv, then its own epilogue; same bits
    assert q.dense_path(fmt, n, k, q.X_BF16, m) == q.PATH_VALU_ONE
    c = Case(fmt, n, k, m, oracle.X_BF16, False, NONE, False, False, matrix=60 + n % 7, xscale=1.0)
    say(c.label(), "vs one-batch qgemv")
    w, y = c.run(dev)
    yp = q.qgemv(fmt, w, n, k, x_dev(c.x, c.xt, dev))
    torch.cuda.synchronize()
    assert torch.equal(y, yp)


@pytest.mark.parametrize("n,k", [(4100, 2560), (2060, 4096)])
def test_fused_plain_matches_one_batch_bitwise_q8_0(dev, n, k):
    # Q8_0 one token: 10 and 8 steps per wave, the one-batch kernel's two Q8_0
    # variants; nothing fused, so the same bits as qgemv
    assert q.dense_path(q.Q8_0, n, k, q.X_BF16, 1) == q.PATH_VALU_ONE
    c = Case(q.Q8_0, n, k, 1, oracle.X_BF16, False, NONE, False, False, matrix=61 + n % 7, xscale=1.0)
    say(c.label(), "vs one-batch qgemv")
    w, y = c.run(dev)
    yp = q.qgemv(q.Q8_0, w, n, k, x_dev(c.x, c.xt, dev))
    torch.cuda.synchronize()
    assert torch.equal(y, yp)


def test_fused_residual_in_place_and_deterministic(dev):
    c = Case(q.Q4_0, 2048, 2560, 4, oracle.X_BF16, True, SWIGLU, True, False, matrix=50)
    say(c.label(), "in place")
    w, y1 = c.run(dev)
    _, y2 = c.run(dev, w=w)
    assert torch.equal(y1, y2)                        # same inputs, same bits
    yy = to_dev(c.resid, dev)                         # residual and output in one buffer
    q.qgemv_fused(c.fmt, w, c.n, c.k, x_dev(c.x, c.xt, dev), norm_weight=to_dev(c.gamma, dev), eps=c.eps,
                  act=c.act, residual=yy, y=yy)
    torch.cuda.synchronize()
    assert torch.equal(yy, y1)


@pytest.mark.parametrize("act", [NONE, SWIGLU])
@pytest.mark.parametrize("ybf16", [False, True])
def test_fused_zero_activations(dev, act, ybf16):
    # x = 0 with eps > 0: r = 1/sqrt(eps), the product is 0 and y is the residual (rounded)
    c = Case(q.MXFP4, 1024, 1024, 2, oracle.X_BF16, True, act, True, ybf16, matrix=51)
    c.x = np.zeros_like(c.x)
    say(c.label(), "zero x")
    _, y = c.run(dev)
    want = torch.from_numpy(c.resid)
    if ybf16:
        want = want.to(torch.bfloat16)
    assert torch.equal(y.cpu(), want)


@pytest.mark.parametrize("fmt", [q.Q4_0, q.Q8_0])
def test_fused_several_windows(dev, fmt):
    # K = 12288 with 8 fp32-staged tokens needs several activation windows:
    # the normalisation is computed once and the staging repeated per window
    c = Case(fmt, 1024, 12288, 8, oracle.X_BF16, True, SWIGLU, True, True, matrix=52)
    say(c.label(), "windows")
    _, y = c.run(dev)
    o, scale = c.oracle()
    err = oracle.fused_err(y_host(y), o, scale, y_bf16=True)
    assert err <= TOL, err


# decode-step shapes at full size (sampled rows for the oracle): the Q8_0
# sweep's layer (qkv and gate_up normalised, gate_up through SwiGLU to bf16,
# o and down with the residual) and the Q4_0 gate_up matrices
FULL = [
    ("qkv", q.Q8_0, 6144, 2560, 1, True, NONE, False, False),
    ("o", q.Q8_0, 2560, 4096, 1, False, NONE, True, False),
    ("gate_up", q.Q8_0, 19456, 2560, 1, True, SWIGLU, False, True),
    ("down", q.Q8_0, 2560, 9728, 1, False, NONE, True, False),
    ("gate_up_q4", q.Q4_0, 19456, 2560, 1, True, SWIGLU, False, True),
    ("gate_up_q4_m8", q.Q4_0, 24576, 4096, 8, True, SWIGLU, False, True),
    ("o_norm_res_bf16", q.Q8_0, 2560, 4096, 1, True, NONE, True, True),
]


@pytest.mark.parametrize("case", FULL, ids=[f[0] for f in FULL])
def test_fused_decode_shapes_sampled(dev, case):
    name, fmt, n, k, m, norm, act, res, ybf16 = case
    c = Case(fmt, n, k, m, oracle.X_BF16, norm, act, res, ybf16, config=111, matrix=len(name))
    say(c.label(), name)
    _, y = c.run(dev)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, c.n_out - 1], rng.integers(0, c.n_out, 509)]))
    o, scale = c.oracle(rows=rows)
    err = oracle.fused_err(y_host(y)[:, rows], o, scale, y_bf16=ybf16)
    assert err <= TOL, err


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 4])
def test_fused_gate_on_one_row_tiles(dev, fmt, m):
    # 64 lanes per row (one-row tiles): the gate runs on eight-wave workgroups
    n, k = 600, 4096
    assert q.layout(fmt, n, k)["lanes_per_row"] == 64
    c = Case(fmt, n, k, m, oracle.X_BF16, True, SWIGLU, True, True, matrix=53)
    say(c.label(), "one-row tiles")
    _, y = c.run(dev)
    o, scale = c.oracle()
    err = oracle.fused_err(y_host(y), o, scale, y_bf16=True)
    assert err <= TOL, err
