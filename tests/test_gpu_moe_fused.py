"""GPU parity of the fused top-k expert product (moe_qgemv_topk_fused,
through the C ABI) against the fp64 oracle's definition (oracle.moe_fused):
gate_up with RMSNorm and/or SwiGLU, down-combine with a residual, fp32 or
bf16 outputs.  Bar: oracle.fused_err <= 2e-3 (as for the fused dense
product)."""
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
GATE, DOWN = q.MOE_GATE_UP, q.MOE_DOWN_COMBINE


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


def draw(shape, xt, config, matrix, role, scale):
    xf = (scale * wl.x_f32(shape, wl.rng_for(config, matrix, role))).astype(np.float32)
    return wl.f32_to_bf16_bits_rne(xf) if xt == oracle.X_BF16 else xf


class Experts:
    def __init__(self, fmt, E, n, k, config, dev):
        self.fmt, self.E, self.n, self.k = fmt, E, n, k
        self.canon = np.concatenate([wl.blocks_for(fmt, n, k, config=config, matrix=e).reshape(-1)
                                     for e in range(E)])
        pb = q.packed_bytes(fmt, n, k)
        per = n * (k // 32) * wl.BLOCK_BYTES[fmt]
        self.w = torch.empty(E * pb, dtype=torch.uint8, device=dev)
        for e in range(E):
            q.pack(fmt, to_dev(self.canon[e * per:(e + 1) * per], dev), n, k, out=self.w[e * pb:(e + 1) * pb])


def routing(m, E, top_k, config):
    _, ids, g = wl.router_topk(m, E, top_k, wl.rng_for(config, 0, "router"))
    return ids.astype(np.int32), g.astype(np.float32)


def run(ex, ids, g, x, xt, mode, dev, gamma=None, act=NONE, res=None, ybf16=False, eps=1e-5, y=None):
    out = q.moe_qgemv_topk_fused(ex.fmt, ex.w, ex.E, ex.n, ex.k, to_dev(ids, dev), to_dev(g, dev), x_dev(x, xt, dev),
                                 mode, norm_weight=None if gamma is None else to_dev(gamma, dev), eps=eps, act=act,
                                 residual=None if res is None else to_dev(res, dev), y=y,
                                 out_dtype=torch.bfloat16 if ybf16 else torch.float32)
    torch.cuda.synchronize()
    return out


def check(yhat, o, scale, ybf16):
    valid = np.isfinite(o)
    err = oracle.fused_err(yhat[valid], o[valid], scale[valid], y_bf16=ybf16)
    assert err <= TOL, err


GATE_COMBOS = [(False, NONE, True), (True, NONE, False), (False, SWIGLU, False), (True, SWIGLU, True)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xt", [oracle.X_BF16, oracle.X_F32])
@pytest.mark.parametrize("combo", GATE_COMBOS)
@pytest.mark.parametrize("m", [1, 4, 8])
def test_moe_fused_gate_up(dev, fmt, xt, combo, m):
    norm, act, ybf16 = combo
    E, top_k, n, k = 16, 4, 512, 512
    say(f"moe fused gate_up fmt={fmt} xt={xt} norm={norm} act={act} bf16={ybf16} m={m}")
    ex = Experts(fmt, E, n, k, 120 + fmt, dev)
    ids, g = routing(m, E, top_k, 120 + m)
    x = draw((m, k), xt, 120, m, "x", 3.0)
    gamma = wl.norm_weight_f32(k, wl.rng_for(120, m, "gamma")) if norm else None
    y = run(ex, ids, g, x, xt, GATE, dev, gamma=gamma, act=act, ybf16=ybf16)
    o, s = oracle.moe_fused(fmt, ex.canon, E, n, k, ids, g, x, xt, GATE, norm_weight=gamma, eps=1e-5, act=act)
    check(y.float().cpu().numpy().astype(np.float64), o, s, ybf16)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xt", [oracle.X_BF16, oracle.X_F32])
@pytest.mark.parametrize("ybf16", [False, True])
@pytest.mark.parametrize("m", [1, 4, 8])
def test_moe_fused_down_residual(dev, fmt, xt, ybf16, m):
    E, top_k, n, k = 16, 4, 512, 256
    say(f"moe fused down fmt={fmt} xt={xt} bf16={ybf16} m={m}")
    ex = Experts(fmt, E, n, k, 130 + fmt, dev)
    ids, g = routing(m, E, top_k, 130 + m)
    h = draw((m, top_k, k), xt, 130, m, "h", 1.0)
    res = wl.x_f32((m, n), wl.rng_for(130, m, "res"))
    y = run(ex, ids, g, h, xt, DOWN, dev, res=res, ybf16=ybf16)
    o, s = oracle.moe_fused(fmt, ex.canon, E, n, k, ids, g, h, xt, DOWN, residual=res)
    check(y.float().cpu().numpy().astype(np.float64), o, s, ybf16)


def test_moe_fused_residual_in_place_and_plain_agreement(dev):
    fmt, E, top_k, n, k, m = q.MXFP4, 16, 4, 512, 256, 4
    ex = Experts(fmt, E, n, k, 140, dev)
    ids, g = routing(m, E, top_k, 140)
    h = draw((m, top_k, k), oracle.X_BF16, 140, 0, "h", 1.0)
    res = wl.x_f32((m, n), wl.rng_for(140, 0, "res"))
    say("moe fused down in place")
    y1 = run(ex, ids, g, h, oracle.X_BF16, DOWN, dev, res=res)
    yy = to_dev(res, dev)
    run(ex, ids, g, h, oracle.X_BF16, DOWN, dev, res=res, y=yy)      # residual copy in, sum out (separate)
    assert torch.equal(yy, y1)
    zz = to_dev(res, dev)
    q.moe_qgemv_topk_fused(fmt, ex.w, E, n, k, to_dev(ids, dev), to_dev(g, dev), x_dev(h, oracle.X_BF16, dev), DOWN,
                           residual=zz, y=zz)
    torch.cuda.synchronize()
    assert torch.equal(zz, y1)
    # with nothing fused but the residual, the fused call is the plain product plus the residual, bit for bit
    yp = q.moe_qgemv_topk(fmt, ex.w, E, n, k, to_dev(ids, dev), to_dev(g, dev), x_dev(h, oracle.X_BF16, dev), DOWN)
    torch.cuda.synchronize()
    assert torch.equal(y1, yp + to_dev(res, dev))
    # gate_up with a bf16 output only: the plain product rounded to bf16
    x = draw((m, k), oracle.X_BF16, 140, 1, "x", 1.0)
    yb = run(ex, ids, g, x, oracle.X_BF16, GATE, dev, ybf16=True)
    yf = q.moe_qgemv_topk(fmt, ex.w, E, n, k, to_dev(ids, dev), to_dev(g, dev), x_dev(x, oracle.X_BF16, dev), GATE)
    torch.cuda.synchronize()
    assert torch.equal(yb, yf.to(torch.bfloat16))


def test_moe_fused_repeated_and_invalid_ids(dev):
    fmt, E, top_k, n, k, m = q.Q4_0, 8, 4, 512, 512, 3
    ex = Experts(fmt, E, n, k, 150, dev)
    ids = np.array([[3, 3, 1, 7], [-1, 2, 8, 2], [5, 5, 5, 5]], dtype=np.int32)     # repeats, -1 and E invalid
    g = np.full((m, top_k), 0.25, dtype=np.float32)
    x = draw((m, k), oracle.X_BF16, 150, 0, "x", 3.0)
    gamma = wl.norm_weight_f32(k, wl.rng_for(150, 0, "gamma"))
    say("moe fused ids")
    y = torch.full((m, top_k, n // 2), float("nan"), dtype=torch.float32, device=dev)
    run(ex, ids, g, x, oracle.X_BF16, GATE, dev, gamma=gamma, act=SWIGLU, y=y)
    o, s = oracle.moe_fused(fmt, ex.canon, E, n, k, ids, g, x, oracle.X_BF16, GATE, norm_weight=gamma, eps=1e-5,
                            act=SWIGLU)
    yh = y.cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(yh[1, 0])) and np.all(np.isnan(yh[1, 2]))           # invalid slots untouched
    check(yh, o, s, False)
    h = draw((m, top_k, k), oracle.X_BF16, 150, 0, "h", 1.0)
    res = wl.x_f32((m, n), wl.rng_for(150, 0, "res"))
    yd = run(ex, ids, g, h, oracle.X_BF16, DOWN, dev, res=res)
    o, s = oracle.moe_fused(fmt, ex.canon, E, n, k, ids, g, h, oracle.X_BF16, DOWN, residual=res)
    check(yd.cpu().numpy().astype(np.float64), o, s, False)


@pytest.mark.parametrize("m", [1, 4])
def test_moe_ffn_on_device_at_full_size(dev, m):
    """The whole expert FFN of the MXFP4 workload on the device: router ->
    gate_up with RMSNorm + SwiGLU to bf16 -> down-combine + residual, each
    product checked against the oracle on the inputs it was given."""
    fmt, E, top_k = q.MXFP4, 32, 4
    gn, gk, dn, dk = 3584, 2048, 2048, 1792
    say(f"moe ffn m={m}")
    gate = Experts(fmt, E, gn, gk, 160, dev)
    down = Experts(fmt, E, dn, dk, 161, dev)
    logits = wl.x_f32((m, E), wl.rng_for(160, m, "router"))
    tid, tw = q.moe_router_topk(to_dev(logits, dev), top_k)
    hidden = wl.x_f32((m, gk), wl.rng_for(160, m, "x"))
    gamma = wl.norm_weight_f32(gk, wl.rng_for(160, m, "gamma"))
    hd = to_dev(hidden, dev)
    a = q.moe_qgemv_topk_fused(fmt, gate.w, E, gn, gk, tid, tw, hd, GATE, norm_weight=to_dev(gamma, dev), eps=1e-6,
                               act=SWIGLU, out_dtype=torch.bfloat16)
    out = hd.clone()
    q.moe_qgemv_topk_fused(fmt, down.w, E, dn, dk, tid, tw, a, DOWN, residual=out, y=out)
    torch.cuda.synchronize()
    ids, g = tid.cpu().numpy(), tw.cpu().numpy()
    o, s = oracle.moe_fused(fmt, gate.canon, E, gn, gk, ids, g, hidden, oracle.X_F32, GATE, norm_weight=gamma,
                            eps=1e-6, act=SWIGLU)
    check(a.float().cpu().numpy().astype(np.float64), o, s, True)
    a_bits = a.cpu().view(torch.int16).numpy().view(np.uint16)
    o, s = oracle.moe_fused(fmt, down.canon, E, dn, dk, ids, g, a_bits, oracle.X_BF16, DOWN, residual=hidden)
    check(out.cpu().numpy().astype(np.float64), o, s, False)


@pytest.mark.parametrize("fmt", [q.MXFP4, q.Q4_0])
def test_moe_fused_largest_call(dev, fmt):
    # 8 tokens x top-8 of 16 experts = 64 slots, the most one call takes
    E, top_k, m, n, k = 16, 8, 8, 512, 256
    ex = Experts(fmt, E, n, k, 180 + fmt, dev)
    ids, g = routing(m, E, top_k, 180)
    x = draw((m, k), oracle.X_BF16, 180, 0, "x", 3.0)
    gamma = wl.norm_weight_f32(k, wl.rng_for(180, 0, "gamma"))
    say(f"moe fused largest fmt={fmt}")
    y = run(ex, ids, g, x, oracle.X_BF16, GATE, dev, gamma=gamma, act=SWIGLU, ybf16=True)
    o, s = oracle.moe_fused(fmt, ex.canon, E, n, k, ids, g, x, oracle.X_BF16, GATE, norm_weight=gamma, eps=1e-5,
                            act=SWIGLU)
    check(y.float().cpu().numpy().astype(np.float64), o, s, True)
    exd = Experts(fmt, E, k, n // 2, 181 + fmt, dev)            # down: K = F
    h = draw((m, top_k, n // 2), oracle.X_BF16, 181, 0, "h", 1.0)
    res = wl.x_f32((m, k), wl.rng_for(181, 0, "res"))
    yd = run(exd, ids, g, h, oracle.X_BF16, DOWN, dev, res=res)
    o, s = oracle.moe_fused(fmt, exd.canon, E, k, n // 2, ids, g, h, oracle.X_BF16, DOWN, residual=res)
    check(yd.cpu().numpy().astype(np.float64), o, s, False)
