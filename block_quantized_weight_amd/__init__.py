"""Python binding of libqgemv.so, the block-quantized weight GEMV library for MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/qgemv.h.  PyTorch supplies device
memory and the current stream.  There is no fallback path: if the library is
missing or a call fails, an exception is raised.
"""
import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqgemv.so")

# enums of include/qgemv.h
QG_OK, QG_EINVAL, QG_EUNSUPPORTED, QG_EALIGN, QG_EHIP = 0, 1, 2, 3, 4
Q8_0, Q4_0, MXFP4, NVFP4, Q4_K, Q6_K = 0, 1, 2, 3, 4, 5
X_F32, X_BF16 = 0, 1
MOE_GATE_UP, MOE_DOWN_COMBINE = 0, 1
MAX_M = 8
MAX_GEMM_M = 128
PATH_VALU, PATH_MFMA, PATH_VALU_ONE = 0, 1, 2
ACT_NONE, ACT_SWIGLU = 0, 1
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, MXFP4: 17, NVFP4: 18}     # canonical bytes per 32 weights
SUPERBLOCK_BYTES = {Q4_K: 144, Q6_K: 210}                     # K-quants: canonical bytes per 256 weights


def canon_bytes(fmt, n, k):
    """Bytes of one canonical n x k tensor (NVFP4: its blocks, then the 4-byte
    tensor scale; K-quants: super-blocks of 256 weights)."""
    if fmt in SUPERBLOCK_BYTES:
        return n * (k // 256) * SUPERBLOCK_BYTES[fmt]
    return n * (k // 32) * BLOCK_BYTES[fmt] + (4 if fmt == NVFP4 else 0)

# exported functions: name -> (restype, argtypes)
_i, _i64, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
SIGNATURES = {
    "qg_status_str": (ctypes.c_char_p, [_i]),
    "qg_packed_bytes": (_i64, [_i, _i64, _i64]),
    "qg_layout": (_i, [_i, _i64, _i64, _vp]),
    "qg_pack_host": (_i, [_i, _vp, _i64, _i64, _vp]),
    "qg_unpack_host": (_i, [_i, _vp, _i64, _i64, _vp]),
    "qg_pack": (_i, [_i, _vp, _i64, _i64, _vp, _vp]),
    "qg_unpack": (_i, [_i, _vp, _i64, _i64, _vp, _vp]),
    "qg_dequant_f32": (_i, [_i, _vp, _i64, _i64, _vp, _vp]),
    "qg_dense_path": (_i, [_i, _i64, _i64, _i, _i64]),
    "qg_read_stream": (_i, [_vp, _i64, _vp, _vp]),
    "qgemv_q8_0": (_i, [_vp, _i64, _i64, _vp, _i, _i64, _vp, _vp]),
    "qgemv_q4_0": (_i, [_vp, _i64, _i64, _vp, _i, _i64, _vp, _vp]),
    "qgemv_mxfp4": (_i, [_vp, _i64, _i64, _vp, _i, _i64, _vp, _vp]),
    "qgemv_nvfp4": (_i, [_vp, _i64, _i64, _vp, _i, _i64, _vp, _vp]),
    "qgemv_q4_k": (_i, [_vp, _i64, _i64, _vp, _i, _i64, _vp, _vp]),
    "qgemv_q6_k": (_i, [_vp, _i64, _i64, _vp, _i, _i64, _vp, _vp]),
    "qg_requant_q8_0_nvfp4": (_i, [_vp, _i64, _i64, _vp, _vp]),
    "qgemm": (_i, [_i, _vp, _i64, _i64, _vp, _i, _i64, _vp, _vp]),
    "qg_gemm_path": (_i, [_i, _i64, _i64, _i, _i64]),
    "qgemv_fused": (_i, [_i, _vp, _i64, _i64, _vp, _i, _i64, _vp, ctypes.c_float, _i, _vp, _vp, _i, _vp]),
    "moe_qgemv_topk": (_i, [_i, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _i, _i, _vp, _vp]),
    "moe_qgemv_topk_fused": (_i, [_i, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _i, _i, _vp, ctypes.c_float,
                                  _i, _vp, _vp, _i, _vp]),
    "moe_router_topk": (_i, [_vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "qg_chain_plan_bytes": (_i64, [_i64]),
    "qg_chain_plan": (_i, [_i, _i, _i64, _vp, _i64, _vp]),
    "qgemv_chain": (_i, [_vp, _vp, _vp]),
    "qgemv_chain_noalloc": (_i, [_vp, _vp]),
    "qg_chain_error": (_i, []),
}


class ChainLinkC(ctypes.Structure):
    _fields_ = [("w_packed", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64)]


class QGError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")


class Layout(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("lanes_per_row", ctypes.c_int32),
                ("rows_per_tile", ctypes.c_int32), ("parts_per_step", ctypes.c_int32),
                ("scale_bytes", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("steps", ctypes.c_int64),
                ("tiles", ctypes.c_int64), ("code_tile_bytes", ctypes.c_int64),
                ("scale_tile_bytes", ctypes.c_int64), ("scale_offset", ctypes.c_int64),
                ("packed_bytes", ctypes.c_int64), ("tensor_scale_offset", ctypes.c_int64),
                ("high_offset", ctypes.c_int64), ("superblock_offset", ctypes.c_int64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_ if f != "reserved"}


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with block_quantized_weight_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (rt, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype, f.argtypes = rt, args
        _lib = L
    return _lib


def status_str(status):
    return lib().qg_status_str(int(status)).decode()


def _check(fn, status):
    if status != QG_OK:
        raise QGError(fn, status)


# ------------------------------------------------------------------ layout
def dense_path(fmt, n, k, xt, m):
    """PATH_VALU, PATH_MFMA or PATH_VALU_ONE: the kernel family a dense call would run."""
    v = lib().qg_dense_path(fmt, n, k, xt, m)
    if v < 0:
        raise QGError("qg_dense_path", -v)
    return v


def packed_bytes(fmt, n, k):
    v = lib().qg_packed_bytes(fmt, n, k)
    if v < 0:
        raise QGError("qg_packed_bytes", QG_EINVAL)
    return v


def layout(fmt, n, k):
    out = Layout()
    _check("qg_layout", lib().qg_layout(fmt, n, k, ctypes.byref(out)))
    return out.as_dict()


def _np_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def pack_host(fmt, canon, n, k):
    """Canonical blocks (numpy uint8) -> packed bytes (numpy uint8), on the CPU."""
    c = np.ascontiguousarray(canon, dtype=np.uint8).reshape(-1)
    if (fmt not in BLOCK_BYTES and fmt not in SUPERBLOCK_BYTES) or c.size != canon_bytes(fmt, n, k):
        raise ValueError("canonical array size does not match (fmt, n, k)")
    out = np.empty(packed_bytes(fmt, n, k), dtype=np.uint8)
    _check("qg_pack_host", lib().qg_pack_host(fmt, _np_ptr(c), n, k, _np_ptr(out)))
    return out


def unpack_host(fmt, packed, n, k):
    p = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
    if p.size != packed_bytes(fmt, n, k):
        raise ValueError("packed array size does not match (fmt, n, k)")
    out = np.zeros(canon_bytes(fmt, n, k), dtype=np.uint8)
    _check("qg_unpack_host", lib().qg_unpack_host(fmt, _np_ptr(p), n, k, _np_ptr(out)))
    return out


# ------------------------------------------------------------ device calls
def _torch():
    import torch
    return torch


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev_ptr(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _xt(x):
    torch = _torch()
    if x.dtype == torch.float32:
        return X_F32
    if x.dtype == torch.bfloat16:
        return X_BF16
    raise ValueError("activations must be float32 or bfloat16")


def pack(fmt, canon, n, k, out=None, stream=None):
    """Canonical blocks (device uint8 tensor) -> packed weights (device uint8 tensor)."""
    torch = _torch()
    if out is None:
        out = torch.empty(packed_bytes(fmt, n, k), dtype=torch.uint8, device=canon.device)
    _check("qg_pack", lib().qg_pack(fmt, _dev_ptr(canon, "canon"), n, k, _dev_ptr(out, "out"), _stream(stream)))
    return out


def unpack(fmt, packed, n, k, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.zeros(canon_bytes(fmt, n, k), dtype=torch.uint8, device=packed.device)
    _check("qg_unpack", lib().qg_unpack(fmt, _dev_ptr(packed, "packed"), n, k, _dev_ptr(out, "out"),
                                        _stream(stream)))
    return out


def dequant_f32(fmt, packed, n, k, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=packed.device)
    _check("qg_dequant_f32", lib().qg_dequant_f32(fmt, _dev_ptr(packed, "packed"), n, k, _dev_ptr(out, "out"),
                                                  _stream(stream)))
    return out


STREAM_SINK = 16384
CHAIN_STATIC_BYTES = 65536     # QG_CHAIN_STATIC_BYTES: largest plan of qgemv_chain_noalloc


def read_stream(buf, sink=None, stream=None):
    """Reads every byte of the device tensor buf once (measurement aid: the
    achievable HBM read rate); returns the sink (uint32 [STREAM_SINK])."""
    torch = _torch()
    if sink is None:
        sink = torch.empty(STREAM_SINK, dtype=torch.int32, device=buf.device)
    _check("qg_read_stream", lib().qg_read_stream(_dev_ptr(buf, "buf"), buf.numel() * buf.element_size(),
                                                  _dev_ptr(sink, "sink"), _stream(stream)))
    return sink


_GEMV = {Q8_0: "qgemv_q8_0", Q4_0: "qgemv_q4_0", MXFP4: "qgemv_mxfp4", NVFP4: "qgemv_nvfp4", Q4_K: "qgemv_q4_k",
         Q6_K: "qgemv_q6_k"}


def qgemv(fmt, w_packed, n, k, x, y=None, stream=None):
    """y[m, n] = W x[m, k]^T for packed W; x float32 or bfloat16 [m, k] (or [k])."""
    torch = _torch()
    x2 = x.reshape(-1, k)
    m = x2.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    fn = _GEMV[fmt]
    st = getattr(lib(), fn)(_dev_ptr(w_packed, "w_packed"), n, k, _dev_ptr(x2, "x"), _xt(x2), m,
                            _dev_ptr(y, "y"), _stream(stream))
    _check(fn, st)
    return y


def qgemv_q8_0(w_packed, n, k, x, y=None, stream=None):
    return qgemv(Q8_0, w_packed, n, k, x, y, stream)


def qgemv_q4_0(w_packed, n, k, x, y=None, stream=None):
    return qgemv(Q4_0, w_packed, n, k, x, y, stream)


def qgemv_mxfp4(w_packed, n, k, x, y=None, stream=None):
    return qgemv(MXFP4, w_packed, n, k, x, y, stream)


def qgemv_nvfp4(w_packed, n, k, x, y=None, stream=None):
    return qgemv(NVFP4, w_packed, n, k, x, y, stream)


def requant_q8_0_nvfp4(canon_q8_0, n, k, out=None, stream=None):
    """Load-time decode cache: canonical Q8_0 blocks (device uint8) -> packed
    NVFP4 weights (device uint8) for qgemv_nvfp4."""
    torch = _torch()
    if out is None:
        out = torch.empty(packed_bytes(NVFP4, n, k), dtype=torch.uint8, device=canon_q8_0.device)
    _check("qg_requant_q8_0_nvfp4", lib().qg_requant_q8_0_nvfp4(_dev_ptr(canon_q8_0, "canon_q8_0"), n, k,
                                                               _dev_ptr(out, "out"), _stream(stream)))
    return out


def gemm_path(fmt, n, k, xt, m):
    """PATH_VALU or PATH_MFMA: the kernel family a qgemm call would run."""
    v = lib().qg_gemm_path(fmt, n, k, xt, m)
    if v < 0:
        raise QGError("qg_gemm_path", -v)
    return v


def qgemm(fmt, w_packed, n, k, x, y=None, stream=None):
    """y[m, n] = W x[m, k]^T for 1 <= m <= MAX_GEMM_M tokens (float32 or bfloat16 x)."""
    torch = _torch()
    x2 = x.reshape(-1, k)
    m = x2.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    st = lib().qgemm(fmt, _dev_ptr(w_packed, "w_packed"), n, k, _dev_ptr(x2, "x"), _xt(x2), m, _dev_ptr(y, "y"),
                     _stream(stream))
    _check("qgemm", st)
    return y


def qgemv_fused(fmt, w_packed, n, k, x, norm_weight=None, eps=1e-6, act=ACT_NONE, residual=None, y=None,
                out_dtype=None, stream=None):
    """Dense product with the decode step's neighbours fused in:
    y = [SwiGLU](W RMSNorm(x)) [+ residual], each part optional.
    x float32 or bfloat16 [m, k]; norm_weight float32 [k] or None; act
    ACT_NONE or ACT_SWIGLU (gate rows first, y has n / 2 columns); residual
    float32 [m, n_out] or None (may be y itself when y is float32); y float32
    or bfloat16 [m, n_out] (out_dtype when y is None, default float32)."""
    torch = _torch()
    x2 = x.reshape(-1, k)
    m = x2.shape[0]
    n_out = n // 2 if act == ACT_SWIGLU else n
    if y is None:
        y = torch.empty((m, n_out), dtype=out_dtype or torch.float32, device=x.device)
    if y.dtype == torch.float32:
        yt = X_F32
    elif y.dtype == torch.bfloat16:
        yt = X_BF16
    else:
        raise ValueError("y must be float32 or bfloat16")
    gp = None
    if norm_weight is not None:
        if norm_weight.dtype != torch.float32:
            raise ValueError("norm_weight must be float32")
        gp = _dev_ptr(norm_weight, "norm_weight")
    rp = None
    if residual is not None:
        if residual.dtype != torch.float32:
            raise ValueError("residual must be float32")
        rp = _dev_ptr(residual, "residual")
    st = lib().qgemv_fused(fmt, _dev_ptr(w_packed, "w_packed"), n, k, _dev_ptr(x2, "x"), _xt(x2), m, gp,
                           float(eps), act, rp, _dev_ptr(y, "y"), yt, _stream(stream))
    _check("qgemv_fused", st)
    return y


def moe_qgemv_topk(fmt, w_experts, n_experts, n, k, topk_ids, topk_w, x, mode, y=None, stream=None):
    """Top-k expert GEMV.  GATE_UP: x [m, k] -> y [m, top_k, n];
    DOWN_COMBINE: x [m, top_k, k] -> y [m, n] (router-weighted sum, fixed order)."""
    torch = _torch()
    m, top_k = topk_ids.shape
    if topk_ids.dtype != torch.int32:
        raise ValueError("topk_ids must be int32")
    if topk_w is not None and topk_w.dtype != torch.float32:
        raise ValueError("topk_w must be float32")
    if y is None:
        shape = (m, top_k, n) if mode == MOE_GATE_UP else (m, n)
        y = torch.empty(shape, dtype=torch.float32, device=x.device)
    wp = None if topk_w is None else _dev_ptr(topk_w, "topk_w")
    st = lib().moe_qgemv_topk(fmt, _dev_ptr(w_experts, "w_experts"), n_experts, n, k,
                              _dev_ptr(topk_ids, "topk_ids"), wp, m, top_k, _dev_ptr(x, "x"), _xt(x), mode,
                              _dev_ptr(y, "y"), _stream(stream))
    _check("moe_qgemv_topk", st)
    return y


def moe_qgemv_topk_fused(fmt, w_experts, n_experts, n, k, topk_ids, topk_w, x, mode, norm_weight=None, eps=1e-6,
                         act=ACT_NONE, residual=None, y=None, out_dtype=None, stream=None):
    """Top-k expert product with the neighbours fused in.  GATE_UP: x [m, k]
    -> y [m, top_k, n_out], optionally RMSNorm(x) and SwiGLU (n_out = n / 2);
    DOWN_COMBINE: x [m, top_k, k] -> y [m, n], optionally + residual float32
    [m, n] (may be y).  y float32 or bfloat16 (out_dtype when y is None)."""
    torch = _torch()
    m, top_k = topk_ids.shape
    if topk_ids.dtype != torch.int32:
        raise ValueError("topk_ids must be int32")
    if topk_w is not None and topk_w.dtype != torch.float32:
        raise ValueError("topk_w must be float32")
    n_out = n // 2 if act == ACT_SWIGLU else n
    if y is None:
        shape = (m, top_k, n_out) if mode == MOE_GATE_UP else (m, n)
        y = torch.empty(shape, dtype=out_dtype or torch.float32, device=x.device)
    if y.dtype == torch.float32:
        yt = X_F32
    elif y.dtype == torch.bfloat16:
        yt = X_BF16
    else:
        raise ValueError("y must be float32 or bfloat16")
    gp = None
    if norm_weight is not None:
        if norm_weight.dtype != torch.float32:
            raise ValueError("norm_weight must be float32")
        gp = _dev_ptr(norm_weight, "norm_weight")
    rp = None
    if residual is not None:
        if residual.dtype != torch.float32:
            raise ValueError("residual must be float32")
        rp = _dev_ptr(residual, "residual")
    wp = None if topk_w is None else _dev_ptr(topk_w, "topk_w")
    st = lib().moe_qgemv_topk_fused(fmt, _dev_ptr(w_experts, "w_experts"), n_experts, n, k,
                                    _dev_ptr(topk_ids, "topk_ids"), wp, m, top_k, _dev_ptr(x, "x"), _xt(x), mode,
                                    gp, float(eps), act, rp, _dev_ptr(y, "y"), yt, _stream(stream))
    _check("moe_qgemv_topk_fused", st)
    return y


def moe_router_topk(logits, top_k, ids=None, weights=None, stream=None):
    """Device top-k routing: logits fp32 [m, n_experts] -> (ids int32 [m, top_k],
    weights fp32 [m, top_k]), ready for moe_qgemv_topk."""
    torch = _torch()
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be float32 [m, n_experts]")
    m, n_experts = logits.shape
    if ids is None:
        ids = torch.empty((m, top_k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((m, top_k), dtype=torch.float32, device=logits.device)
    st = lib().moe_router_topk(_dev_ptr(logits, "logits"), m, n_experts, top_k, _dev_ptr(ids, "ids"),
                               _dev_ptr(weights, "weights"), _stream(stream))
    _check("moe_router_topk", st)
    return ids, weights


class Chain:
    """A chain of dense products run in order by one persistent kernel.

    links: list of (w_packed, n, k, x, y) with device tensors; all share the
    format, the activation dtype and the token count m.  The plan (built once)
    holds the tensors' addresses, so they must stay alive and in place.
    """

    def __init__(self, fmt, links):
        torch = _torch()
        if not links:
            raise ValueError("empty chain")
        xt = _xt(links[0][3])
        m = links[0][3].reshape(-1, links[0][2]).shape[0]
        arr = (ChainLinkC * len(links))()
        self._keep = []
        for i, (w, n, k, x, y) in enumerate(links):
            x2 = x.reshape(-1, k)
            if _xt(x2) != xt or x2.shape[0] != m or y.numel() != m * n:
                raise ValueError("chain links must share activation dtype and token count")
            arr[i] = ChainLinkC(_dev_ptr(w, "w_packed").value, _dev_ptr(x2, "x").value, _dev_ptr(y, "y").value,
                                n, k)
            self._keep += [w, x, y]
        nbytes = lib().qg_chain_plan_bytes(len(links))
        if nbytes < 0:
            raise QGError("qg_chain_plan_bytes", QG_EINVAL)
        self.plan_host = (ctypes.c_uint8 * nbytes)()
        _check("qg_chain_plan", lib().qg_chain_plan(fmt, xt, m, arr, len(links), self.plan_host))
        host = torch.frombuffer(bytearray(self.plan_host), dtype=torch.uint8)
        self.plan_device = host.to(links[0][0].device)
        torch.cuda.synchronize()
        self.count = len(links)

    def run(self, stream=None):
        _check("qgemv_chain", lib().qgemv_chain(self.plan_host, _dev_ptr(self.plan_device, "plan"), _stream(stream)))

    def run_noalloc(self, stream=None):
        """The same chain through qgemv_chain_noalloc: the plan travels in the
        library's static device buffer, no device copy of the caller's is read."""
        _check("qgemv_chain_noalloc", lib().qgemv_chain_noalloc(self.plan_host, _stream(stream)))


def chain_error():
    """1 if a chain barrier timed out since the last call (synchronises), else 0."""
    v = lib().qg_chain_error()
    if v < 0:
        raise QGError("qg_chain_error", QG_EHIP)
    return v
