"""Generator checks: determinism, distributions and encodings of the workloads."""
import numpy as np

import workloads as wl


def test_seeded_generators_are_deterministic():
    a = wl.blocks_for(wl.FMT_Q4_0, 8, 64, config=1, matrix=0)
    b = wl.blocks_for(wl.FMT_Q4_0, 8, 64, config=1, matrix=0)
    c = wl.blocks_for(wl.FMT_Q4_0, 8, 64, config=1, matrix=1)
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_q8_0_draws():
    b = wl.blocks_for(wl.FMT_Q8_0, 64, 2048, config=0, matrix=0).reshape(64, 64, 34)
    codes = b[:, :, 2:].view(np.int8)
    assert codes.min() >= -127 and codes.max() <= 127
    d = (b[:, :, 0].astype(np.uint16) | (b[:, :, 1].astype(np.uint16) << 8)).view(np.float16).astype(np.float64)
    assert d.min() >= 1e-3 * (1 - 2 ** -10) and d.max() <= 1e-2 * (1 + 2 ** -10)


def test_mxfp4_scale_draws():
    b = wl.blocks_for(wl.FMT_MXFP4, 64, 2048, config=4, matrix=0).reshape(64, 64, 17)
    e = b[:, :, 0].astype(int) - 127
    assert e.min() == -8 and e.max() == -2


def test_nibble_split_encoding():
    q = np.arange(32, dtype=np.uint8).reshape(1, 1, 32) % 16
    blk = wl.encode_q4_0(q, np.array([[0x3C00]], dtype=np.uint16))
    assert blk[0, 0, 2] == (0 | (0 << 4)) and blk[0, 0, 3] == (1 | (1 << 4))
    q2 = np.array([list(range(16)) + [15 - i for i in range(16)]], dtype=np.uint8).reshape(1, 1, 32)
    blk2 = wl.encode_mxfp4(q2, np.array([[127]], dtype=np.uint8))
    assert blk2[0, 0, 0] == 127 and blk2[0, 0, 1] == 0xF0 and blk2[0, 0, 16] == 0x0F


def test_bf16_rne():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], dtype=np.float32)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 ties to 1+2^-6... (rounds up to even mantissa)
    got = wl.f32_to_bf16_bits_rne(f)
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0xC020]


def test_router_topk():
    logits, ids, w = wl.router_topk(4, 32, 4, wl.rng_for(4, 0, "router"))
    for t in range(4):
        order = np.argsort(-logits[t], kind="stable")[:4]
        assert list(ids[t]) == list(order)
        assert len(set(ids[t])) == 4
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) < 1e-6
        assert np.all(np.diff(w[t]) <= 0)


def test_c2_sweep_shapes():
    s = wl.c2_sweep_shapes()
    assert len(s) == 145
    assert s[-1][2:] == (151936, 2560)
    wbytes = sum(n * k // 32 * 34 for _, _, n, k in s)
    assert wbytes == 4_273_664_000
