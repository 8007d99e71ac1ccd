"""Host-side checks of libqgemv.so: symbols, layout, host packer, argument
validation.  No call here reaches a kernel launch: every device-side call is
made with arguments the host validation rejects."""
import ctypes
import os
import re
import struct

import numpy as np
import pytest

import block_quantized_weight_amd as q
import workloads as wl

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qgemv.h")


def _declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                                 text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"qgemv_q8_0", "qgemv_q4_0", "qgemv_mxfp4", "moe_qgemv_topk"} <= set(names)
    L = ctypes.CDLL(q.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(q.SIGNATURES)


def test_status_strings():
    assert q.status_str(q.QG_OK) == "ok"
    assert q.status_str(q.QG_EALIGN) == "misaligned device pointer"


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0, q.MXFP4])
@pytest.mark.parametrize("n,k", [(1, 32), (65, 96), (300, 2048), (19, 608), (2560, 9728)])
def test_layout_is_consistent(fmt, n, k):
    lo = q.layout(fmt, n, k)
    L, R, S = lo["lanes_per_row"], lo["rows_per_tile"], lo["steps"]
    assert L * R == 64 and L in (1, 2, 4, 8, 16, 32, 64)
    assert S == -(-(k // 32) // L) and lo["tiles"] == -(-n // R)
    assert lo["code_tile_bytes"] == S * lo["parts_per_step"] * 1024
    assert lo["scale_tile_bytes"] == S * 64 * lo["scale_bytes"]
    raw = lo["tiles"] * (lo["code_tile_bytes"] + lo["scale_tile_bytes"])
    assert lo["packed_bytes"] == -(-raw // 256) * 256
    assert lo["packed_bytes"] == q.packed_bytes(fmt, n, k)
    assert lo["code_tile_bytes"] % 1024 == 0
    assert lo["packed_bytes"] >= n * (k // 32) * q.BLOCK_BYTES[fmt]


def test_workload_shapes_pack_without_padding():
    shapes = [(q.Q8_0, n, k) for _, _, n, k in wl.c2_sweep_shapes()[:4]] + [(q.Q8_0, 151936, 2560)]
    shapes += [(q.Q4_0, 19456, 2560), (q.Q4_0, 2560, 9728), (q.Q4_0, 6144, 4096), (q.Q4_0, 24576, 4096),
               (q.Q4_0, 4096, 12288), (q.MXFP4, 3584, 2048), (q.MXFP4, 2048, 1792)]
    for fmt, n, k in shapes:
        assert q.packed_bytes(fmt, n, k) == n * (k // 32) * q.BLOCK_BYTES[fmt], (fmt, n, k)


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0, q.MXFP4])
@pytest.mark.parametrize("n,k", [(1, 32), (3, 64), (65, 96), (300, 2048), (19, 608), (130, 1792)])
def test_host_pack_round_trip(fmt, n, k):
    c = wl.blocks_for(fmt, n, k, config=50, matrix=n).reshape(-1)
    p = q.pack_host(fmt, c, n, k)
    assert np.array_equal(q.unpack_host(fmt, p, n, k), c)


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0, q.MXFP4])
def test_host_pack_round_trip_all_byte_values(fmt):
    n, k = 64, 256
    nbytes = n * (k // 32) * q.BLOCK_BYTES[fmt]
    c = (np.arange(nbytes, dtype=np.int64) * 37 % 256).astype(np.uint8)
    p = q.pack_host(fmt, c, n, k)
    assert np.array_equal(q.unpack_host(fmt, p, n, k), c)


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0, q.MXFP4])
def test_packed_record_placement(fmt):
    """Every block's bytes land in the (tile, step, lane) record the layout names:
    lane l of step j in tile t holds block j*L + l%L of row t*R + l/L."""
    n, k = 70, 320
    lo = q.layout(fmt, n, k)
    L, R, S, P, sb = lo["lanes_per_row"], lo["rows_per_tile"], lo["steps"], lo["parts_per_step"], lo["scale_bytes"]
    nb, bb = k // 32, q.BLOCK_BYTES[fmt]
    c = np.zeros((n, nb, bb), dtype=np.uint8)
    rng = np.random.default_rng(3)
    c[:] = rng.integers(0, 256, size=c.shape, dtype=np.uint8)
    p = q.pack_host(fmt, c.reshape(-1), n, k)
    for (row, blk) in [(0, 0), (n - 1, nb - 1), (R, 1), (5, nb // 2)]:
        t, r = divmod(row, R)
        j, s = divmod(blk, L)
        lane = r * L + s
        # the scale travels unchanged
        so = lo["scale_offset"] + t * lo["scale_tile_bytes"] + j * 64 * sb + lane * sb
        assert bytes(p[so:so + sb]) == bytes(c[row, blk, :sb])
        # the code bytes: Q8_0 as stored; the 4-bit formats with byte B holding
        # elements 2B (low nibble) and 2B+1 (high nibble), Q4_0 nibbles as q ^ 8
        co = t * lo["code_tile_bytes"] + j * P * 1024 + lane * 16
        got = np.concatenate([p[co + h * 1024: co + h * 1024 + 16] for h in range(P)])
        body = c[row, blk, sb:]
        if fmt == q.Q8_0:
            assert np.array_equal(got, body)
        else:
            codes = np.concatenate([body & 15, body >> 4])          # element order
            if fmt == q.Q4_0:
                codes = codes ^ 8
            want = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
            assert np.array_equal(got, want)


def test_padding_bytes_are_zero():
    fmt, n, k = q.Q4_0, 5, 96        # 5 rows -> padded rows in the last tile
    c = np.full(n * 3 * 18, 0xFF, dtype=np.uint8)
    p = q.pack_host(fmt, c, n, k)
    lo = q.layout(fmt, n, k)
    used = n * 3 * (16 + 2)
    assert int(np.count_nonzero(p)) == used
    assert p.size == lo["packed_bytes"]


# ------------------------------------------------ validation (nothing launched)
BAD = ctypes.c_void_p(0)
ODD = ctypes.c_void_p(0x1001)


def test_shape_validation():
    L = q.lib()
    assert L.qg_packed_bytes(q.Q8_0, 4, 33) == -1
    assert L.qg_packed_bytes(q.Q8_0, 0, 32) == -1
    assert L.qg_packed_bytes(7, 4, 32) == -1
    assert L.qg_layout(q.Q4_0, 4, 32, None) == q.QG_EINVAL
    assert L.qg_layout(q.Q4_0, 1 << 32, 32, None) == q.QG_EUNSUPPORTED


def test_gemv_argument_validation():
    L = q.lib()
    st = L.qgemv_q8_0(BAD, 64, 64, BAD, q.X_F32, 1, BAD, None)
    assert st == q.QG_EINVAL                              # null pointers
    a = ctypes.c_void_p(0x100000)
    assert L.qgemv_q8_0(a, 64, 48, a, q.X_F32, 1, a, None) == q.QG_EINVAL      # k % 32
    assert L.qgemv_q4_0(a, 64, 64, a, q.X_F32, 0, a, None) == q.QG_EINVAL      # m = 0
    assert L.qgemv_q4_0(a, 64, 64, a, q.X_F32, 9, a, None) == q.QG_EINVAL      # m = 9
    assert L.qgemv_mxfp4(a, 64, 64, a, 5, 1, a, None) == q.QG_EINVAL           # bad xt
    assert L.qgemv_mxfp4(a, -1, 64, a, q.X_BF16, 1, a, None) == q.QG_EINVAL    # n <= 0
    assert L.qgemv_q8_0(ODD, 64, 64, a, q.X_F32, 1, a, None) == q.QG_EALIGN    # w not 16-aligned
    # packed weights must start on a 256-byte boundary (whole cache lines per 1 KiB wave load)
    W16 = ctypes.c_void_p(0x100000 + 16)
    for f in (L.qgemv_q8_0, L.qgemv_q4_0, L.qgemv_mxfp4):
        assert f(W16, 64, 64, a, q.X_F32, 1, a, None) == q.QG_EALIGN
        assert f(ctypes.c_void_p(0x100000 + 128), 64, 64, a, q.X_F32, 1, a, None) == q.QG_EALIGN
    assert L.qgemm(q.Q4_0, W16, 256, 512, a, q.X_BF16, 16, a, None) == q.QG_EALIGN
    assert L.qgemv_fused(q.Q8_0, W16, 64, 64, a, q.X_F32, 1, None, ctypes.c_float(0.0), 0, None, a, q.X_F32,
                         None) == q.QG_EALIGN
    assert L.qgemv_q8_0(a, 64, 64, ODD, q.X_F32, 1, a, None) == q.QG_EALIGN    # x not 16-aligned
    assert L.qgemv_q8_0(a, 64, 64, a, q.X_F32, 1, ODD, None) == q.QG_EALIGN    # y not 4-aligned


def test_moe_argument_validation():
    L = q.lib()
    a = ctypes.c_void_p(0x100000)
    f = L.moe_qgemv_topk
    assert f(q.MXFP4, a, 32, 64, 64, a, a, 1, 4, a, q.X_BF16, 2, a, None) == q.QG_EINVAL      # mode
    assert f(q.MXFP4, a, 32, 64, 64, a, None, 1, 4, a, q.X_BF16, 1, a, None) == q.QG_EINVAL   # no weights
    assert f(q.MXFP4, a, 32, 64, 64, a, a, 1, 33, a, q.X_BF16, 0, a, None) == q.QG_EINVAL     # top_k > E
    assert f(q.MXFP4, a, 32, 64, 64, a, a, 9, 4, a, q.X_BF16, 0, a, None) == q.QG_EINVAL      # m > 8
    assert f(q.MXFP4, a, 100, 64, 64, a, a, 8, 9, a, q.X_BF16, 0, a, None) == q.QG_EUNSUPPORTED  # m*top_k
    assert f(q.MXFP4, ODD, 32, 64, 64, a, a, 1, 4, a, q.X_BF16, 0, a, None) == q.QG_EALIGN
    assert f(q.MXFP4, ctypes.c_void_p(0x100000 + 64), 32, 64, 64, a, a, 1, 4, a, q.X_BF16, 0, a,
             None) == q.QG_EALIGN                     # experts 16- but not 256-aligned
    assert f(q.MXFP4, a, 32, 64, 64, ODD, a, 1, 4, a, q.X_BF16, 0, a, None) == q.QG_EALIGN


def test_pack_and_dequant_validation():
    L = q.lib()
    a = ctypes.c_void_p(0x100000)
    assert L.qg_pack(q.Q8_0, a, 4, 40, a, None) == q.QG_EINVAL
    assert L.qg_pack(q.Q8_0, a, 4, 64, ODD, None) == q.QG_EALIGN
    assert L.qg_pack(q.Q8_0, a, 4, 64, ctypes.c_void_p(0x100000 + 32), None) == q.QG_EALIGN
    assert L.qg_unpack(q.Q8_0, ctypes.c_void_p(0x100000 + 32), 4, 64, a, None) == q.QG_EALIGN
    assert L.qg_unpack(q.Q8_0, BAD, 4, 64, a, None) == q.QG_EINVAL
    assert L.qg_dequant_f32(q.Q8_0, a, 4, 64, ODD, None) == q.QG_EALIGN
    assert L.qg_pack_host(q.Q8_0, None, 4, 64, None) == q.QG_EINVAL


def test_dense_path_rule():
    """bf16 co-batches of 2..8 tokens on layouts of <= 8 lanes per row take the
    matrix cores unless the one-batch vector kernel applies (4-bit formats, up to
    3 tokens, short rows); everything else the vector path, one token over short
    rows its one-batch form."""
    V, M = q.PATH_VALU, q.PATH_MFMA
    assert q.layout(q.Q4_0, 6144, 4096)["lanes_per_row"] == 8
    assert q.dense_path(q.Q8_0, 6144, 4096, q.X_BF16, 1) == V
    assert q.dense_path(q.Q8_0, 6144, 4096, q.X_BF16, 2) == M
    assert q.dense_path(q.Q4_0, 6144, 4096, q.X_BF16, 3) == q.PATH_VALU_ONE
    assert q.dense_path(q.Q4_0, 6144, 4096, q.X_BF16, 4) == M
    assert q.dense_path(q.MXFP4, 6144, 4096, q.X_BF16, 8) == M
    assert q.dense_path(q.Q4_0, 6144, 4096, q.X_F32, 8) == V          # fp32 activations
    assert q.layout(q.Q4_0, 2560, 9728)["lanes_per_row"] == 16
    assert q.dense_path(q.Q4_0, 2560, 9728, q.X_BF16, 8) == V         # 16 lanes per row
    # one token (4-bit formats: up to 3) over short rows: the one-batch vector
    # kernel (4-bit formats up to 20 steps per wave, Q8_0 up to 10)
    O = q.PATH_VALU_ONE
    assert q.dense_path(q.Q8_0, 2560, 4096, q.X_BF16, 1) == O         # 8 steps per lane
    assert q.dense_path(q.Q8_0, 6144, 2560, q.X_BF16, 1) == O         # 10
    assert q.dense_path(q.Q8_0, 2560, 9728, q.X_BF16, 1) == V         # 38
    assert q.dense_path(q.Q8_0, 2048, 2048, q.X_F32, 1) == O
    assert q.dense_path(q.Q4_0, 2560, 9728, q.X_BF16, 1) == O         # 19
    assert q.dense_path(q.Q4_0, 19456, 2560, q.X_BF16, 1) == O        # 40 over 4 waves
    assert q.dense_path(q.Q4_0, 2560, 9728, q.X_BF16, 2) == O         # two tokens (4-bit: up to 3)
    assert q.dense_path(q.Q4_0, 2560, 9728, q.X_BF16, 3) == V         # 3 x 304 blocks > 3 per thread
    assert q.dense_path(q.Q8_0, 2560, 4096, q.X_F32, 2) == V          # Q8_0: one token only
    assert q.dense_path(q.Q8_0, 151936, 2560, q.X_BF16, 1) == V       # 40 per wave
    assert q.dense_path(q.MXFP4, 6144, 4096, q.X_F32, 1) == O
    # only when every workgroup is resident at once: 768 workgroups of 16 steps per
    # wave need 3 per compute unit, the 20-step variant holds 2 (two tokens then
    # go to the matrix cores)
    assert q.dense_path(q.Q4_0, 24576, 4096, q.X_BF16, 2) == M
    assert q.dense_path(q.Q4_0, 24576, 4096, q.X_BF16, 3) == M
    assert q.dense_path(q.Q4_0, 24576, 4096, q.X_F32, 2) == V
    assert q.dense_path(q.Q4_0, 24576, 4096, q.X_BF16, 1) == V
    # Q8_0 with bf16 activations at one token allows a short second round: 608
    # workgroups of 10 steps per wave against 512 resident
    assert q.dense_path(q.Q8_0, 19456, 2560, q.X_BF16, 1) == O
    assert q.dense_path(q.Q8_0, 19456, 2560, q.X_F32, 1) == V
    assert q.dense_path(q.Q4_0, 6144, 4096, q.X_BF16, 2) == O          # 768 of 4 steps: 4 per unit
    for bad in [(q.Q8_0, 64, 33, q.X_BF16, 1), (q.Q8_0, 64, 64, q.X_BF16, 0), (q.Q8_0, 64, 64, q.X_BF16, 9),
                (q.Q8_0, 64, 64, 5, 1), (9, 64, 64, q.X_BF16, 1), (q.Q8_0, 0, 64, q.X_BF16, 1)]:
        with pytest.raises(q.QGError):
            q.dense_path(*bad)
    assert q.lib().qg_dense_path(q.Q8_0, 1 << 32, 64, q.X_BF16, 1) == -q.QG_EUNSUPPORTED


def test_router_argument_validation():
    """Rejected before any device work (no GPU needed)."""
    L = q.lib()
    a = ctypes.c_void_p(1 << 20)
    ODD = ctypes.c_void_p((1 << 20) + 2)
    assert L.moe_router_topk(None, 1, 32, 4, a, a, None) == q.QG_EINVAL
    assert L.moe_router_topk(a, 0, 32, 4, a, a, None) == q.QG_EINVAL
    assert L.moe_router_topk(a, 1, 32, 0, a, a, None) == q.QG_EINVAL
    assert L.moe_router_topk(a, 1, 4, 5, a, a, None) == q.QG_EINVAL
    assert L.moe_router_topk(a, 1, 2048, 4, a, a, None) == q.QG_EUNSUPPORTED
    assert L.moe_router_topk(a, 1, 128, 65, a, a, None) == q.QG_EUNSUPPORTED
    assert L.moe_router_topk(ODD, 1, 32, 4, a, a, None) == q.QG_EALIGN


def test_fused_argument_validation():
    """qgemv_fused rejects bad arguments before any device work (no GPU needed)."""
    L = q.lib()
    a = ctypes.c_void_p(1 << 20)
    b = ctypes.c_void_p(1 << 24)
    ODD = ctypes.c_void_p((1 << 20) + 2)
    f = ctypes.c_float

    def call(fmt=q.Q8_0, w=a, n=256, k=512, x=a, xt=q.X_BF16, m=1, g=None, eps=1e-6, act=q.ACT_NONE, res=None,
             y=b, yt=q.X_F32):
        return L.qgemv_fused(fmt, w, n, k, x, xt, m, g, f(eps), act, res, y, yt, None)

    assert call(w=None) == q.QG_EINVAL and call(x=None) == q.QG_EINVAL and call(y=None) == q.QG_EINVAL
    assert call(fmt=7) == q.QG_EINVAL and call(k=100) == q.QG_EINVAL and call(n=0) == q.QG_EINVAL
    assert call(xt=2) == q.QG_EINVAL and call(yt=2) == q.QG_EINVAL and call(act=2) == q.QG_EINVAL
    assert call(m=0) == q.QG_EINVAL and call(m=9) == q.QG_EINVAL
    assert call(g=a, eps=-1.0) == q.QG_EINVAL and call(g=a, eps=float("nan")) == q.QG_EINVAL
    assert call(g=a, eps=float("inf")) == q.QG_EINVAL
    assert call(act=q.ACT_SWIGLU, n=255) == q.QG_EINVAL
    assert call(x=ODD) == q.QG_EALIGN and call(g=ODD) == q.QG_EALIGN
    assert call(y=ctypes.c_void_p((1 << 24) + 2)) == q.QG_EALIGN
    assert call(res=ctypes.c_void_p((1 << 24) + 2), y=ctypes.c_void_p(1 << 26)) == q.QG_EALIGN
    # residual overlapping y: only the exact alias with an fp32 output is allowed
    assert call(res=ctypes.c_void_p((1 << 24) + 4)) == q.QG_EINVAL
    assert call(res=b, yt=q.X_BF16) == q.QG_EINVAL
    # SwiGLU needs F to be a multiple of the layout's rows per tile
    lo = q.layout(q.Q8_0, 2 * 4100, 2560)
    assert 4100 % lo["rows_per_tile"] != 0
    assert call(act=q.ACT_SWIGLU, n=2 * 4100, k=2560) == q.QG_EUNSUPPORTED


def test_moe_fused_argument_validation():
    """moe_qgemv_topk_fused rejects bad arguments before any device work."""
    L = q.lib()
    a = ctypes.c_void_p(1 << 20)
    b = ctypes.c_void_p(1 << 24)
    ODD = ctypes.c_void_p((1 << 20) + 2)
    f = ctypes.c_float

    def call(fmt=q.MXFP4, n=1024, k=512, m=2, top_k=4, mode=q.MOE_GATE_UP, g=None, eps=1e-6, act=q.ACT_NONE,
             res=None, y=b, yt=q.X_F32, w=a, x=a):
        return L.moe_qgemv_topk_fused(fmt, w, 16, n, k, a, a, m, top_k, x, q.X_BF16, mode, g, f(eps), act, res, y,
                                      yt, None)

    assert call(res=a) == q.QG_EINVAL                                  # gate_up takes no residual
    assert call(mode=q.MOE_DOWN_COMBINE, g=a) == q.QG_EINVAL           # down takes no normalisation
    assert call(mode=q.MOE_DOWN_COMBINE, act=q.ACT_SWIGLU) == q.QG_EINVAL
    assert call(act=3) == q.QG_EINVAL and call(yt=5) == q.QG_EINVAL
    assert call(g=a, eps=-1.0) == q.QG_EINVAL and call(g=a, eps=float("nan")) == q.QG_EINVAL
    assert call(act=q.ACT_SWIGLU, n=1023) == q.QG_EINVAL
    assert call(g=ODD) == q.QG_EALIGN and call(y=ctypes.c_void_p((1 << 24) + 2)) == q.QG_EALIGN
    assert call(mode=q.MOE_DOWN_COMBINE, res=ctypes.c_void_p((1 << 24) + 8)) == q.QG_EINVAL   # overlaps y
    assert call(mode=q.MOE_DOWN_COMBINE, res=b, yt=q.X_BF16) == q.QG_EINVAL
    lo = q.layout(q.Q8_0, 2 * 4100, 2560)
    assert 4100 % lo["rows_per_tile"] != 0
    assert call(fmt=q.Q8_0, n=2 * 4100, k=2560, act=q.ACT_SWIGLU) == q.QG_EUNSUPPORTED
    # eight normalised (fp32-staged) rows of K = 4096 need 128 KiB of LDS: refused, not run elsewhere
    assert call(k=4096, m=8, top_k=2, g=a) == q.QG_EUNSUPPORTED
    # more than 64 slots per call
    assert call(m=8, top_k=9) == q.QG_EUNSUPPORTED
    assert call(m=0) == q.QG_EINVAL and call(top_k=17) == q.QG_EINVAL


def test_gemm_argument_validation_and_path():
    """qgemm rejects bad arguments before any device work; qg_gemm_path's rule."""
    L = q.lib()
    a = ctypes.c_void_p(1 << 20)
    ODD = ctypes.c_void_p((1 << 20) + 2)
    assert L.qgemm(q.Q4_0, a, 256, 512, a, q.X_BF16, 0, a, None) == q.QG_EINVAL
    assert L.qgemm(q.Q4_0, a, 256, 512, a, q.X_BF16, q.MAX_GEMM_M + 1, a, None) == q.QG_EINVAL
    assert L.qgemm(q.Q4_0, a, 256, 500, a, q.X_BF16, 16, a, None) == q.QG_EINVAL
    assert L.qgemm(q.Q4_0, None, 256, 512, a, q.X_BF16, 16, a, None) == q.QG_EINVAL
    assert L.qgemm(q.Q4_0, a, 256, 512, a, 7, 16, a, None) == q.QG_EINVAL
    assert L.qgemm(q.Q4_0, a, 256, 512, ODD, q.X_BF16, 16, a, None) == q.QG_EALIGN
    # matrix cores for bf16 on layouts of <= 16 lanes per row, else the dense product in passes
    for fmt in (q.Q8_0, q.Q4_0, q.MXFP4):
        for n, k in [(32768, 256), (16384, 512), (8192, 256), (4096, 4096), (2048, 4096), (1024, 4096), (300, 4096)]:
            lanes = q.layout(fmt, n, k)["lanes_per_row"]
            want = q.PATH_MFMA if lanes <= 16 else q.PATH_VALU
            assert q.gemm_path(fmt, n, k, q.X_BF16, 64) == want, (fmt, n, k, lanes)
            assert q.gemm_path(fmt, n, k, q.X_F32, 64) == q.PATH_VALU


def test_nvfp4_host_pack_round_trip_and_placement():
    """NVFP4: two 16-weight blocks per 32-weight record; codes in adjacent-pair
    order, the two E4M3 scales as the record's 16-bit scale entry (first block
    low), and the fp32 tensor scale in the 256-byte trailer."""
    import workloads as wl
    for n, k in [(1, 32), (70, 320), (129, 608)]:
        c = wl.nvfp4_tensor(n, k, np.random.default_rng(n), np.random.default_rng(k))
        p = q.pack_host(q.NVFP4, c, n, k)
        assert np.array_equal(q.unpack_host(q.NVFP4, p, n, k), c)
        lo = q.layout(q.NVFP4, n, k)
        assert lo["packed_bytes"] == p.size and lo["packed_bytes"] % 256 == 0
        assert lo["tensor_scale_offset"] == lo["packed_bytes"] - 256
        assert bytes(p[lo["tensor_scale_offset"]:lo["tensor_scale_offset"] + 4]) == bytes(c[-4:])
        L, R, S = lo["lanes_per_row"], lo["rows_per_tile"], lo["steps"]
        body = c[:-4].reshape(n, k // 16, 9)
        for row, blk in [(0, 0), (n - 1, k // 32 - 1), (n // 2, (k // 32) // 2)]:
            t, r = divmod(row, R)
            j, s = divmod(blk, L)
            lane = r * L + s
            so = lo["scale_offset"] + t * lo["scale_tile_bytes"] + j * 64 * 2 + lane * 2
            assert p[so] == body[row, 2 * blk, 0] and p[so + 1] == body[row, 2 * blk + 1, 0]
            co = t * lo["code_tile_bytes"] + j * 1024 + lane * 16
            codes = []
            for h in range(2):
                b = body[row, 2 * blk + h, 1:]
                codes += list(b & 15) + list(b >> 4)          # elements j and j+8 of each block
            codes = np.array(codes, dtype=np.uint8)
            assert np.array_equal(p[co:co + 16], (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8))


def test_nvfp4_argument_validation():
    L = q.lib()
    a = ctypes.c_void_p(0x100000)
    assert L.qgemv_nvfp4(a, 64, 48, a, q.X_F32, 1, a, None) == q.QG_EINVAL
    assert L.qgemv_nvfp4(ctypes.c_void_p(0x100000 + 16), 64, 64, a, q.X_F32, 1, a, None) == q.QG_EALIGN
    assert L.qg_requant_q8_0_nvfp4(a, 64, 64, ctypes.c_void_p(0x100000 + 64), None) == q.QG_EALIGN
    assert L.qg_requant_q8_0_nvfp4(None, 64, 64, a, None) == q.QG_EINVAL
    assert L.qg_requant_q8_0_nvfp4(a, 64, 40, a, None) == q.QG_EINVAL
    assert q.dense_path(q.NVFP4, 6144, 4096, q.X_BF16, 8) == q.PATH_VALU       # no matrix-core route


def test_chain_noalloc_refuses_on_the_host():
    """qgemv_chain_noalloc's argument and size checks come before any device
    work: no plan, a buffer that is not a plan, and a plan one link over the
    static buffer's capacity."""
    L = q.lib()
    most = 430                  # the header's stated capacity
    assert L.qg_chain_plan_bytes(most) <= q.CHAIN_STATIC_BYTES < L.qg_chain_plan_bytes(most + 1)
    assert L.qgemv_chain_noalloc(None, None) == q.QG_EINVAL
    junk = (ctypes.c_uint8 * 256)()
    assert L.qgemv_chain_noalloc(junk, None) == q.QG_EINVAL
    # a header (magic, fmt, xt, m, count, grid, lds, part_off, out_off) of one link too many
    hdr = struct.pack("<Iiiiiiqqq", 0x51474333, q.Q8_0, q.X_BF16, 1, most + 1, 256, 0, 0, 0)
    buf = (ctypes.c_uint8 * L.qg_chain_plan_bytes(most + 1)).from_buffer_copy(
        hdr + bytes(L.qg_chain_plan_bytes(most + 1) - len(hdr)))
    assert L.qgemv_chain_noalloc(buf, None) == q.QG_EUNSUPPORTED


# ------------------------------------------------------------------ K-quants
@pytest.mark.parametrize("fmt", [q.Q4_K, q.Q6_K])
@pytest.mark.parametrize("n,k", [(1, 256), (3, 256), (65, 768), (300, 2560), (19, 9728)])
def test_kquant_host_pack_round_trip(fmt, n, k):
    canon = wl.blocks_for(fmt, n, k, config=71, matrix=n).reshape(-1)
    packed = q.pack_host(fmt, canon, n, k)
    assert packed.size % 256 == 0
    assert np.array_equal(q.unpack_host(fmt, packed, n, k), canon)


def test_kquant_shape_validation():
    L = q.lib()
    for fmt in (q.Q4_K, q.Q6_K):
        assert L.qg_packed_bytes(fmt, 4, 96) == -1          # not whole super-blocks
        assert L.qg_packed_bytes(fmt, 4, 288) == -1
        assert L.qg_packed_bytes(fmt, 4, 512) > 0
    lo4, lo6 = q.layout(q.Q4_K, 65, 768), q.layout(q.Q6_K, 65, 768)
    assert lo4["high_offset"] == 0 and lo4["superblock_offset"] > lo4["scale_offset"]
    assert lo6["high_offset"] > lo6["scale_offset"] and lo6["superblock_offset"] > lo6["high_offset"]


def _record(lo, row, blk):
    """(code offset, scale offset, record index) of (row, 32-weight block blk)."""
    L, R, S = lo["lanes_per_row"], lo["rows_per_tile"], lo["steps"]
    tile, lane = row // R, (row % R) * L + blk % L
    step = blk // L
    co = tile * lo["code_tile_bytes"] + step * 1024 + lane * 16
    so = lo["scale_offset"] + tile * lo["scale_tile_bytes"] + step * 128 + lane * 2
    return co, so, (tile * S + step) * 64 + lane


def test_kquant_packed_record_placement():
    """Each 32-weight sub-block's codes, scales and super-block words sit
    where the layout says, in the stated encoding (Q4_K codes as q ^ 8
    nibble pairs; Q6_K codes t = q ^ 32 split into low nibbles and high bit
    pairs), read back here from the canonical bytes by position."""
    n, k = 9, 768
    rng = np.random.default_rng(72)
    for fmt in (q.Q4_K, q.Q6_K):
        canon = wl.blocks_for(fmt, n, k, config=72, matrix=fmt)
        packed = q.pack_host(fmt, canon, n, k)
        lo = q.layout(fmt, n, k)
        sbb = 144 if fmt == q.Q4_K else 210
        cb = canon.reshape(n, k // 256, sbb)
        for row, blk in [(0, 0), (n - 1, k // 32 - 1)] + [(int(rng.integers(n)), int(rng.integers(k // 32))) for _ in range(6)]:
            s, j = blk // 8, blk % 8
            sb = cb[row, s]
            co, so, rec = _record(lo, row, blk)
            code = packed[co:co + 16]
            word = packed[lo["superblock_offset"] + (row * (k // 256) + s) * 4:][:4]
            if fmt == q.Q4_K:
                qs = [(sb[16 + 32 * (j // 2) + l] >> (4 * (j % 2))) & 15 for l in range(32)]
                got = [((code[i // 2] >> (4 * (i % 2))) & 15) ^ 8 for i in range(32)]
                assert got == qs
                assert bytes(word) == bytes(sb[0:4])
            else:
                h, r = j // 4, j % 4
                qv = [((sb[64 * h + l + 32 * (r & 1)] >> (4 * (r // 2))) & 15) | (((sb[128 + 32 * h + l] >> (2 * r)) & 3) << 4)
                      for l in range(32)]
                hb = packed[lo["high_offset"] + rec * 8:][:8]
                t = []
                for i in range(32):
                    a4, rem = i // 8, i % 8
                    e, b = rem // 4, rem % 4
                    lo4 = (code[4 * a4 + b] >> (4 * e)) & 15
                    f = 2 * (a4 % 2) + e
                    hi2 = (hb[4 * (a4 // 2) + b] >> (2 * f)) & 3
                    t.append(lo4 | (hi2 << 4))
                assert [v ^ 32 for v in t] == qv
                assert list(packed[so:so + 2]) == [sb[192 + 8 * h + 2 * r], sb[192 + 8 * h + 2 * r + 1]]
                assert bytes(word[:2]) == bytes(sb[208:210]) and bytes(word[2:]) == b"\0\0"
