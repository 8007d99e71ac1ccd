"""GPU parity of the NVFP4 path (imp's decode-cache format: imp README, "Why
this exists" and the "Features" table) against the fp64 oracle: packing,
decoding, the dense and fused products, and the load-time Q8_0 -> NVFP4
re-quantizer, which must produce the oracle's bytes exactly."""
import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
q = pytest.importorskip("block_quantized_weight_amd")

pytestmark = pytest.mark.gpu
TOL = 2e-3
CFG = 85


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


def tensor(n, k, matrix):
    return wl.nvfp4_tensor(n, k, wl.rng_for(CFG, matrix, "codes"), wl.rng_for(CFG, matrix, "scales"))


def x_of(shape, xt, matrix, dev):
    rng = wl.rng_for(CFG, matrix, "x")
    x = wl.x_bf16_bits(shape, rng) if xt == oracle.X_BF16 else wl.x_f32(shape, rng)
    t = to_dev(x, dev)
    return x, (t.view(torch.int16).view(torch.bfloat16) if xt == oracle.X_BF16 else t)


@pytest.mark.parametrize("n,k", [(1, 32), (65, 96), (300, 2048), (2560, 9728)])
def test_pack_matches_host_and_round_trips(dev, n, k):
    say(f"nvfp4 pack n={n} k={k}")
    c = tensor(n, k, n)
    host = q.pack_host(q.NVFP4, c, n, k)
    # into a buffer full of junk: every byte of the packed form must be written
    junk = torch.full((q.packed_bytes(q.NVFP4, n, k),), 0xAB, dtype=torch.uint8, device=dev)
    devp = q.pack(q.NVFP4, to_dev(c, dev), n, k, out=junk)
    assert np.array_equal(devp.cpu().numpy(), host)
    back = q.unpack(q.NVFP4, devp, n, k)
    assert np.array_equal(back.cpu().numpy(), c)
    lo = q.layout(q.NVFP4, n, k)
    assert bytes(host[lo["tensor_scale_offset"]:lo["tensor_scale_offset"] + 4]) == bytes(c[-4:])


def test_dequant_is_the_rounded_exact_weight(dev):
    n, k = 257, 1024
    say("nvfp4 dequant")
    c = tensor(n, k, 1)
    # every scale byte and code, so all 128 non-negative E4M3 codes and 16 E2M1 codes occur
    body = c[:-4].reshape(n, k // 16, 9).copy()
    body[:128, 0, 0] = np.arange(128, dtype=np.uint8)
    body[:128, 0, 0][body[:128, 0, 0] == 0x7F] = 0x7E        # keep the scales finite
    c = np.concatenate([body.reshape(-1), c[-4:]])
    w = q.dequant_f32(q.NVFP4, q.pack(q.NVFP4, to_dev(c, dev), n, k), n, k).cpu().numpy()
    ref = oracle.decode(oracle.NVFP4, c, n, k).astype(np.float32)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


SHAPES = [(1, 32), (5, 96), (65, 608), (300, 2048), (1000, 4096), (64, 9728), (7, 12288)]


@pytest.mark.parametrize("xt", [oracle.X_F32, oracle.X_BF16])
@pytest.mark.parametrize("m", [1, 3, 8])
def test_dense_shapes(dev, xt, m):
    for n, k in SHAPES:
        say(f"nvfp4 dense n={n} k={k} m={m} xt={xt}")
        c = tensor(n, k, n + k)
        w = q.pack(q.NVFP4, to_dev(c, dev), n, k)
        x, xd = x_of((m, k), xt, n + k, dev)
        y = q.qgemv(q.NVFP4, w, n, k, xd)
        torch.cuda.synchronize()
        ref, l1 = oracle.gemv(oracle.NVFP4, c, n, k, x, xt)
        err = oracle.max_rel_err(y.cpu().numpy(), ref, l1)
        assert err <= TOL, (n, k, err)


@pytest.mark.parametrize("n,k,m,path", [(2560, 9728, 1, q.PATH_VALU_ONE), (19456, 2560, 1, q.PATH_VALU_ONE),
                                        (24576, 4096, 1, q.PATH_VALU), (6144, 4096, 4, q.PATH_VALU),
                                        (151936, 2560, 1, q.PATH_VALU)])
def test_decode_shapes_each_family(dev, n, k, m, path):
    assert q.dense_path(q.NVFP4, n, k, q.X_BF16, m) == path
    say(f"nvfp4 family n={n} k={k} m={m}")
    c = tensor(n, k, 7)
    w = q.pack(q.NVFP4, to_dev(c, dev), n, k)
    x, xd = x_of((m, k), oracle.X_BF16, 7, dev)
    y = q.qgemv(q.NVFP4, w, n, k, xd).cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, n, 97 if n < 100000 else 997), [n - 1]]))
    ref, l1 = oracle.gemv(oracle.NVFP4, c, n, k, x, oracle.X_BF16, rows=rows)
    assert oracle.max_rel_err(y[:, rows], ref, l1) <= TOL


def test_fused_norm_swiglu_residual(dev):
    n, k, m = 1152, 1024, 2
    say("nvfp4 fused")
    c = tensor(n, k, 11)
    w = q.pack(q.NVFP4, to_dev(c, dev), n, k)
    x, xd = x_of((m, k), oracle.X_BF16, 11, dev)
    gamma = wl.norm_weight_f32(k, wl.rng_for(CFG, 11, "gamma"))
    y = q.qgemv_fused(q.NVFP4, w, n, k, xd, norm_weight=to_dev(gamma, dev), eps=1e-5, act=q.ACT_SWIGLU)
    torch.cuda.synchronize()
    o, scale = oracle.dense_fused(oracle.NVFP4, c, n, k, x, oracle.X_BF16, norm_weight=gamma, eps=1e-5,
                                  act=oracle.ACT_SWIGLU)
    assert oracle.fused_err(y.cpu().numpy(), o, scale) <= TOL
    res = wl.x_f32((m, n), wl.rng_for(CFG, 12, "res"))
    y2 = q.qgemv_fused(q.NVFP4, w, n, k, xd, residual=to_dev(res, dev))
    o2, s2 = oracle.dense_fused(oracle.NVFP4, c, n, k, x, oracle.X_BF16, residual=res)
    assert oracle.fused_err(y2.cpu().numpy(), o2, s2) <= TOL


def test_qgemm_many_tokens(dev):
    n, k, m = 512, 2048, 20
    say("nvfp4 qgemm")
    assert q.gemm_path(q.NVFP4, n, k, q.X_BF16, m) == q.PATH_VALU
    c = tensor(n, k, 13)
    w = q.pack(q.NVFP4, to_dev(c, dev), n, k)
    x, xd = x_of((m, k), oracle.X_BF16, 13, dev)
    y = q.qgemm(q.NVFP4, w, n, k, xd)
    ref, l1 = oracle.gemv(oracle.NVFP4, c, n, k, x, oracle.X_BF16)
    assert oracle.max_rel_err(y.cpu().numpy(), ref, l1) <= TOL


def test_expert_call_refused(dev):
    n, k, E = 64, 64, 2
    pb = q.packed_bytes(q.NVFP4, n, k)
    wexp = torch.zeros(E * pb, dtype=torch.uint8, device=dev)
    ids = torch.zeros((1, 1), dtype=torch.int32, device=dev)
    g = torch.ones((1, 1), dtype=torch.float32, device=dev)
    x = torch.zeros((1, k), dtype=torch.bfloat16, device=dev)
    with pytest.raises(q.QGError) as e:
        q.moe_qgemv_topk(q.NVFP4, wexp, E, n, k, ids, g, x, q.MOE_GATE_UP)
    assert e.value.status == q.QG_EUNSUPPORTED


# ------------------------------------------------------ decode cache (re-quantizer)
@pytest.mark.parametrize("n,k,config,matrix", [(65, 96, 86, 0), (2048, 2048, 0, 0), (6144, 2560, 2, 0),
                                               (2560, 9728, 2, 3)])
def test_requant_matches_oracle_bytes(dev, n, k, config, matrix):
    """The GPU re-quantizer writes exactly the oracle's NVFP4 tensor (codes,
    block scales and tensor scale) for the workloads' Q8_0 matrices."""
    say(f"requant n={n} k={k}")
    canon = wl.blocks_for(q.Q8_0, n, k, config=config, matrix=matrix)
    junk = torch.full((q.packed_bytes(q.NVFP4, n, k),), 0xAB, dtype=torch.uint8, device=dev)
    packed = q.requant_q8_0_nvfp4(to_dev(canon.reshape(-1), dev), n, k, out=junk)
    got = q.unpack(q.NVFP4, packed, n, k).cpu().numpy()
    # the padding is zero and the trailer word after the tensor scale holds max |w|
    lo = q.layout(q.NVFP4, n, k)
    host = q.pack_host(q.NVFP4, got, n, k)
    pk = packed.cpu().numpy()
    ts = lo["tensor_scale_offset"]
    assert np.array_equal(np.delete(pk, np.arange(ts + 4, ts + 8)), np.delete(host, np.arange(ts + 4, ts + 8)))
    amax = np.float32(np.abs(oracle.decode(oracle.Q8_0, canon, n, k)).max())
    assert pk[ts + 4:ts + 8].view(np.float32)[0] == amax
    w32 = oracle.decode(oracle.Q8_0, canon, n, k).astype(np.float32)     # exact products d * q
    want = oracle.nvfp4_quantize(w32)
    assert np.array_equal(got, want)


def test_requant_deterministic_and_zero_tensor(dev):
    n, k = 300, 640
    canon = wl.blocks_for(q.Q8_0, n, k, config=87, matrix=0)
    cd = to_dev(canon.reshape(-1), dev)
    a = q.requant_q8_0_nvfp4(cd, n, k)
    b = q.requant_q8_0_nvfp4(cd, n, k)
    assert torch.equal(a, b)
    zero = np.zeros_like(canon.reshape(-1))
    z = q.unpack(q.NVFP4, q.requant_q8_0_nvfp4(to_dev(zero, dev), n, k), n, k).cpu().numpy()
    assert np.array_equal(z, oracle.nvfp4_quantize(np.zeros((n, k), dtype=np.float32)))


def test_decode_cache_product_and_its_deviation(dev):
    """The product over the cache matches the oracle of the NVFP4 tensor it
    holds (the parity bar), and its deviation from the Q8_0 product it stands
    for is reported: 4-bit values cannot meet the 2e-3 bar against Q8_0 (imp
    release notes v0.4.1), the deviation is measured, not bounded."""
    n, k = 2560, 4096
    canon = wl.blocks_for(q.Q8_0, n, k, config=2, matrix=1)
    cache = q.requant_q8_0_nvfp4(to_dev(canon.reshape(-1), dev), n, k)
    x, xd = x_of((1, k), oracle.X_BF16, 21, dev)
    y = q.qgemv(q.NVFP4, cache, n, k, xd).cpu().numpy()
    nv = q.unpack(q.NVFP4, cache, n, k).cpu().numpy()
    ref, l1 = oracle.gemv(oracle.NVFP4, nv, n, k, x, oracle.X_BF16)
    assert oracle.max_rel_err(y, ref, l1) <= TOL
    ref8, l18 = oracle.gemv(oracle.Q8_0, canon, n, k, x, oracle.X_BF16)
    dev_err = oracle.max_rel_err(y, ref8, l18)
    say(f"decode cache deviation from the Q8_0 product: {dev_err:.4f} (max |y - y_q8| / L1)")
    assert 0 < dev_err < 0.2


def test_nan_scale_poisons_only_its_rows(dev):
    """An E4M3 NaN scale (S.1111.111) makes its row's output NaN, as the
    definition does; every other row still matches the oracle."""
    n, k = 40, 512
    c = tensor(n, k, 31)
    body = c[:-4].reshape(n, k // 16, 9).copy()
    bad = [3, 17, 39]
    for r in bad:
        body[r, (5 * r) % (k // 16), 0] = 0x7F if r != 17 else 0xFF
    c = np.concatenate([body.reshape(-1), c[-4:]])
    w = q.pack(q.NVFP4, to_dev(c, dev), n, k)
    x, xd = x_of((2, k), oracle.X_BF16, 31, dev)
    y = q.qgemv(q.NVFP4, w, n, k, xd).cpu().numpy()
    good = np.setdiff1d(np.arange(n), bad)
    assert np.all(np.isnan(y[:, bad]))
    ref, l1 = oracle.gemv(oracle.NVFP4, c, n, k, x, oracle.X_BF16, rows=good)
    assert oracle.max_rel_err(y[:, good], ref, l1) <= TOL
