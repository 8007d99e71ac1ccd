"""Graph capture: every kernel family recorded in one HIP graph (through
torch.cuda.CUDAGraph), replayed several times with the program's own eager
work and synchronisations in between; each replay must reproduce the eager
results bit for bit (all kernels are deterministic), and replays must read
inputs rewritten in place between them."""
import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
q = pytest.importorskip("block_quantized_weight_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()
    return torch.device("cuda:0")


def _bf16(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _packed(fmt, n, k, config, matrix, dev):
    canon = wl.blocks_for(fmt, n, k, config=config, matrix=matrix)
    return q.pack(fmt, torch.from_numpy(canon.reshape(-1)).to(dev), n, k)


def test_graph_replays_match_eager(dev):
    print("graph capture", flush=True)
    # dense, vector path: Q8_0, one token (batched)
    n1, k1 = 6144, 2560
    w1 = _packed(q.Q8_0, n1, k1, 90, 0, dev)
    x1 = _bf16(wl.x_bf16_bits((1, k1), wl.rng_for(90, 0, "x")), dev)
    y1 = torch.empty((1, n1), device=dev)
    # dense, matrix cores: Q4_0, four tokens
    n2, k2 = 5000, 2048
    w2 = _packed(q.Q4_0, n2, k2, 90, 1, dev)
    x2 = _bf16(wl.x_bf16_bits((4, k2), wl.rng_for(90, 1, "x")), dev)
    y2 = torch.empty((4, n2), device=dev)
    assert q.dense_path(q.Q4_0, n2, k2, q.X_BF16, 4) == q.PATH_MFMA
    # experts: router -> gate_up and down-combine (MXFP4, 16 experts, top-4, 2 tokens)
    fmt, E, top_k, m = q.MXFP4, 16, 4, 2
    gn, gk, dn, dk = 512, 1024, 1024, 512
    gpb, dpb = q.packed_bytes(fmt, gn, gk), q.packed_bytes(fmt, dn, dk)
    ge = torch.empty(E * gpb, dtype=torch.uint8, device=dev)
    de = torch.empty(E * dpb, dtype=torch.uint8, device=dev)
    for e in range(E):
        q.pack(fmt, torch.from_numpy(wl.blocks_for(fmt, gn, gk, config=91, matrix=2 * e).reshape(-1)).to(dev),
               gn, gk, out=ge[e * gpb:(e + 1) * gpb])
        q.pack(fmt, torch.from_numpy(wl.blocks_for(fmt, dn, dk, config=91, matrix=2 * e + 1).reshape(-1)).to(dev),
               dn, dk, out=de[e * dpb:(e + 1) * dpb])
    logits = torch.from_numpy(wl.x_f32((m, E), wl.rng_for(91, 0, "router"))).to(dev)
    xg = _bf16(wl.x_bf16_bits((m, gk), wl.rng_for(91, 0, "x")), dev)
    hd = _bf16(wl.x_bf16_bits((m, top_k, dk), wl.rng_for(91, 0, "h")), dev)
    ids = torch.empty((m, top_k), dtype=torch.int32, device=dev)
    gw = torch.empty((m, top_k), device=dev)
    yg = torch.empty((m, top_k, gn), device=dev)
    yd = torch.empty((m, dn), device=dev)
    # fused: dense RMSNorm + SwiGLU -> bf16 (Q4_0 gate_up 2 x 1024 rows, K 2048), expert gate_up
    # with RMSNorm + SwiGLU -> bf16, expert down-combine with the residual added in place
    w3 = _packed(q.Q4_0, 2048, 2048, 90, 2, dev)
    gam3 = torch.from_numpy(wl.norm_weight_f32(2048, wl.rng_for(90, 2, "gamma"))).to(dev)
    y3 = torch.empty((4, 1024), dtype=torch.bfloat16, device=dev)
    hid = torch.from_numpy(wl.x_f32((m, gk), wl.rng_for(91, 1, "x"))).to(dev)
    gam4 = torch.from_numpy(wl.norm_weight_f32(gk, wl.rng_for(91, 1, "gamma"))).to(dev)
    ya = torch.empty((m, top_k, gn // 2), dtype=torch.bfloat16, device=dev)
    res = torch.from_numpy(wl.x_f32((m, dn), wl.rng_for(91, 1, "res"))).to(dev)
    yr = torch.empty((m, dn), device=dev)
    # many-token product: 40 tokens on the matrix cores
    x5 = _bf16(wl.x_bf16_bits((40, k2), wl.rng_for(90, 6, "x")), dev)
    y5 = torch.empty((40, n2), device=dev)
    # one-batch kernels: Q4_0 down-like 2560 x 9728 (19 steps per wave), and the o-like Q8_0
    # 2560 x 4096 with a residual added in place (the fused call's one-batch form)
    n6, k6 = 2560, 9728
    w6 = _packed(q.Q4_0, n6, k6, 90, 7, dev)
    x6 = _bf16(wl.x_bf16_bits((1, k6), wl.rng_for(90, 7, "x")), dev)
    y6 = torch.empty((1, n6), device=dev)
    assert q.dense_path(q.Q4_0, n6, k6, q.X_BF16, 1) == q.PATH_VALU_ONE
    n7, k7 = 2560, 4096
    w7 = _packed(q.Q8_0, n7, k7, 90, 8, dev)
    x7 = _bf16(wl.x_bf16_bits((1, k7), wl.rng_for(90, 8, "x")), dev)
    res7 = torch.from_numpy(wl.x_f32((1, n7), wl.rng_for(90, 8, "res"))).to(dev)
    y7 = torch.empty((1, n7), device=dev)
    assert q.dense_path(q.Q8_0, n7, k7, q.X_BF16, 1) == q.PATH_VALU_ONE

    def step():
        q.qgemv(q.Q8_0, w1, n1, k1, x1, y=y1)
        q.qgemv(q.Q4_0, w2, n2, k2, x2, y=y2)
        q.moe_router_topk(logits, top_k, ids=ids, weights=gw)
        q.moe_qgemv_topk(fmt, ge, E, gn, gk, ids, gw, xg, q.MOE_GATE_UP, y=yg)
        q.moe_qgemv_topk(fmt, de, E, dn, dk, ids, gw, hd, q.MOE_DOWN_COMBINE, y=yd)
        q.qgemv_fused(q.Q4_0, w3, 2048, 2048, x2, norm_weight=gam3, act=q.ACT_SWIGLU, y=y3)
        q.moe_qgemv_topk_fused(fmt, ge, E, gn, gk, ids, gw, hid, q.MOE_GATE_UP, norm_weight=gam4,
                               act=q.ACT_SWIGLU, y=ya)
        yr.copy_(res)
        q.moe_qgemv_topk_fused(fmt, de, E, dn, dk, ids, gw, hd, q.MOE_DOWN_COMBINE, residual=yr, y=yr)
        q.qgemm(q.Q4_0, w2, n2, k2, x5, y=y5)
        q.qgemv(q.Q4_0, w6, n6, k6, x6, y=y6)
        y7.copy_(res7)
        q.qgemv_fused(q.Q8_0, w7, n7, k7, x7, residual=y7, y=y7)

    outs = (y1, y2, ids, gw, yg, yd, y3, ya, yr, y5, y6, y7)

    def eager():
        step()
        torch.cuda.synchronize()
        return [o.clone() for o in outs]

    ref = eager()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    other_w = _packed(q.Q8_0, 256, 512, 92, 0, dev)
    other_x = _bf16(wl.x_bf16_bits((1, 512), wl.rng_for(92, 0, "x")), dev)
    for rep in range(5):
        for o in outs:
            o.fill_(-1 if o.dtype == torch.int32 else float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), rep
        q.qgemv(q.Q8_0, other_w, 256, 512, other_x)      # eager work between replays
        torch.cuda.synchronize()

    # new inputs, written in place: replays see them
    x1.copy_(_bf16(wl.x_bf16_bits((1, k1), wl.rng_for(90, 5, "x")), dev))
    logits.copy_(torch.from_numpy(wl.x_f32((m, E), wl.rng_for(91, 5, "router"))).to(dev))
    torch.cuda.synchronize()
    ref2 = eager()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref2):
            assert torch.equal(a, b), rep
    assert not torch.equal(ref2[0], ref[0])
    rid, _ = oracle.router_topk(logits.cpu().numpy(), top_k)
    assert np.array_equal(ids.cpu().numpy(), rid)
