"""fp64 CPU oracle for block-quantized weight GEMV (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product package.  It shares no
code with the HIP library and imports nothing from it.

Functions follow oracle.c; see the header there for the definitions and the
passages of the pages each format rests on.  The verdict metric is
``max_rel_err``: max over outputs of |yhat - y| / L1, where L1 is the sum of
|w * x| over the row (zero L1 requires yhat == 0 exactly).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

Q8_0, Q4_0, MXFP4, NVFP4, Q4_K, Q6_K = 0, 1, 2, 3, 4, 5
X_F32, X_BF16 = 0, 1
MOE_GATE_UP, MOE_DOWN = 0, 1
ACT_NONE, ACT_SWIGLU = 0, 1
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, MXFP4: 17, NVFP4: 9,      # NVFP4: per 16 weights
               Q4_K: 144, Q6_K: 210}                          # K-quants: per 256 weights
BLOCK_LEN = {Q8_0: 32, Q4_0: 32, MXFP4: 32, NVFP4: 16, Q4_K: 256, Q6_K: 256}


def build(force=False):
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        for name, rt, args in [
            ("orc_threads", ctypes.c_int, []),
            ("orc_set_threads", None, [ctypes.c_int]),
            ("orc_fp16", ctypes.c_double, [ctypes.c_uint16]),
            ("orc_bf16", ctypes.c_double, [ctypes.c_uint16]),
            ("orc_e8m0", ctypes.c_double, [ctypes.c_uint8]),
            ("orc_e2m1", ctypes.c_double, [ctypes.c_uint8]),
            ("orc_e4m3", ctypes.c_double, [ctypes.c_uint8]),
            ("orc_e4m3_round", ctypes.c_uint8, [ctypes.c_float]),
            ("orc_e2m1_round", ctypes.c_uint8, [ctypes.c_float]),
            ("orc_tensor_bytes", i64, [ctypes.c_int, i64, i64]),
            ("orc_nvfp4_quantize", ctypes.c_int, [vp, i64, i64, vp]),
            ("orc_decode", ctypes.c_int, [ctypes.c_int, vp, i64, i64, dp]),
            ("orc_gemv", ctypes.c_int, [ctypes.c_int, vp, i64, i64, vp, ctypes.c_int, i64,
                                        vp, i64, dp, dp]),
            ("orc_moe", ctypes.c_int, [ctypes.c_int, vp, i64, i64, i64, vp, vp, i64, i64,
                                       vp, ctypes.c_int, ctypes.c_int, vp, i64, dp, dp]),
        ]:
            f = getattr(L, name)
            f.restype, f.argtypes = rt, args
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def threads():
    """OpenMP threads the oracle's parallel loops use."""
    return lib().orc_threads()


def set_threads(n):
    """Threads for the oracle's parallel loops (for timing; results do not
    depend on it: each row is summed by one thread, in index order)."""
    lib().orc_set_threads(int(n))


def fp16(h):
    return lib().orc_fp16(int(h))


def bf16(b):
    return lib().orc_bf16(int(b))


def e8m0(e):
    return lib().orc_e8m0(int(e))


def e2m1(c):
    return lib().orc_e2m1(int(c))


def e4m3(b):
    """OCP FP8 E4M3 byte -> value (fp64)."""
    return lib().orc_e4m3(int(b))


def e4m3_round(v):
    """Non-negative fp32 v -> the nearest E4M3 code (ties to even, saturating at 448)."""
    return int(lib().orc_e4m3_round(float(np.float32(v))))


def e2m1_round(r):
    """fp32 r -> the nearest E2M1 code (ties to even, saturating at +-6; +0 for zero)."""
    return int(lib().orc_e2m1_round(float(np.float32(r))))


def nvfp4_quantize(w):
    """fp32 weights [n, k] -> one canonical NVFP4 tensor (uint8), by the
    quantizer of oracle.c (fp32 arithmetic in the order written there)."""
    wa = np.ascontiguousarray(w, dtype=np.float32)
    n, k = wa.shape
    out = np.empty(tensor_bytes(NVFP4, n, k), dtype=np.uint8)
    if lib().orc_nvfp4_quantize(_ptr(wa), n, k, _ptr(out)) != 0:
        raise ValueError("orc_nvfp4_quantize rejected its arguments")
    return out


def tensor_bytes(fmt, n, k):
    """Bytes of one canonical n x k tensor (NVFP4: its blocks of 16 weights,
    then the fp32 tensor scale)."""
    v = lib().orc_tensor_bytes(fmt, n, k)
    if v < 0:
        raise ValueError("bad format or shape")
    return v


def _blocks(fmt, blocks, n, k):
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1)
    if b.size != tensor_bytes(fmt, n, k):
        raise ValueError("block array size does not match n, k")
    return b


def _x(x, xt):
    if xt == X_F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    return np.ascontiguousarray(x, dtype=np.uint16)


def decode(fmt, blocks, n, k):
    """All weights as float64 [n, k]."""
    b = _blocks(fmt, blocks, n, k)
    w = np.empty((n, k), dtype=np.float64)
    if lib().orc_decode(fmt, _ptr(b), n, k, _ptr(w)) != 0:
        raise ValueError("orc_decode rejected its arguments")
    return w


def gemv(fmt, blocks, n, k, x, xt, rows=None):
    """y, l1 as float64 [m, nrows]; x is [m, k] (float32 or bf16 bit patterns)."""
    b = _blocks(fmt, blocks, n, k)
    xa = _x(x, xt).reshape(-1, k)
    m = xa.shape[0]
    if rows is None:
        nrows, rp = n, None
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, rp = r.size, _ptr(r)
    y = np.empty((m, nrows), dtype=np.float64)
    l1 = np.empty((m, nrows), dtype=np.float64)
    if lib().orc_gemv(fmt, _ptr(b), n, k, _ptr(xa), xt, m, rp, nrows, _ptr(y), _ptr(l1)) != 0:
        raise ValueError("orc_gemv rejected its arguments")
    return y, l1


def moe(fmt, experts, n_experts, n, k, ids, g, x, xt, mode, rows=None):
    """GATE_UP: y, l1 [m, top_k, nrows]; DOWN: y, l1 [m, nrows]."""
    e = np.ascontiguousarray(experts, dtype=np.uint8).reshape(-1)
    if e.size != n_experts * tensor_bytes(fmt, n, k):
        raise ValueError("expert array size does not match")
    ida = np.ascontiguousarray(ids, dtype=np.int32)
    m, top_k = ida.shape
    ga = None if g is None else np.ascontiguousarray(g, dtype=np.float32).reshape(m, top_k)
    xa = _x(x, xt)
    if rows is None:
        nrows, rp = n, None
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, rp = r.size, _ptr(r)
    shape = (m, top_k, nrows) if mode == MOE_GATE_UP else (m, nrows)
    y = np.empty(shape, dtype=np.float64)
    l1 = np.empty(shape, dtype=np.float64)
    rc = lib().orc_moe(fmt, _ptr(e), n_experts, n, k, _ptr(ida),
                       None if ga is None else _ptr(ga), m, top_k, _ptr(xa), xt, mode,
                       rp, nrows, _ptr(y), _ptr(l1))
    if rc != 0:
        raise ValueError("orc_moe rejected its arguments")
    return y, l1


def router_topk(logits, top_k):
    """Top-k routing by definition, in fp64.

    For each token: the top_k experts by descending logit, the lower expert id
    first among equal logits; weights = softmax over the selected logits
    (exp(l - l_max) / sum).  The pages route each token to 4 of 32 experts
    (tests/golden/page_facts.txt); the softmax domain (the selected logits) is
    a reading.  logits: float32 [m, n_experts], no NaN.  Returns ids int64
    [m, top_k] and weights float64 [m, top_k].
    """
    la = np.asarray(logits, dtype=np.float32)
    if la.ndim != 2 or not 1 <= top_k <= la.shape[1]:
        raise ValueError("router_topk: logits [m, n_experts] and 1 <= top_k <= n_experts")
    if np.isnan(la).any():
        raise ValueError("router_topk: NaN logit")
    m, n_experts = la.shape
    ids = np.empty((m, top_k), dtype=np.int64)
    w = np.empty((m, top_k), dtype=np.float64)
    for t in range(m):
        ranked = sorted(range(n_experts), key=lambda e: (-float(la[t, e]), e))
        chosen = ranked[:top_k]
        vals = [float(la[t, e]) for e in chosen]
        top = vals[0]
        ex = [np.exp(v - top) for v in vals]
        total = sum(ex)
        ids[t] = chosen
        w[t] = [v / total for v in ex]
    return ids, w


def max_rel_err(yhat, y, l1):
    """max |yhat - y| / l1; where l1 == 0 the output must be exactly 0 (else inf)."""
    yhat = np.asarray(yhat, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    l1 = np.asarray(l1, dtype=np.float64)
    diff = np.abs(yhat - y)
    zero = l1 == 0
    err = np.zeros_like(diff)
    nz = ~zero
    err[nz] = diff[nz] / l1[nz]
    err[zero & (yhat != 0)] = np.inf
    err[~np.isfinite(yhat)] = np.inf
    return float(err.max()) if err.size else 0.0


# ------------------------------------------------------------ fused steps
# The decode step around a quantized product: RMS normalisation of the
# activations before it, and a gated activation (SwiGLU) or a residual add
# after it.  The pages report such fusions (imp release notes v0.4: a fused
# RMSNorm-gated + SiLU kernel; Imparo README, "Bonsai CUDA Validation": an
# RMS/Add tail fusion reviewed and deferred; "Design Rules": fusion by hand
# where a measurement justifies it) but define neither operation; the
# definitions below are the published ones (RMSNorm: Zhang and Sennrich,
# "Root Mean Square Layer Normalization", 2019; SwiGLU: Shazeer, "GLU
# Variants Improve Transformer", 2020, with SiLU v * sigmoid(v)).  The
# pages' fused matrices pair a gate_up product of N = 2F rows with a down
# product of K = F columns; the reading taken is gate rows [0, F), up rows
# [F, 2F).  Everything is fp64 and follows the definitions in order.


def x_values(x, xt):
    """Activations as float64 [m, k]: fp32 as is, bf16 bit patterns as the
    upper half of an fp32 (exact)."""
    if xt == X_F32:
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def silu(v):
    """SiLU(v) = v / (1 + exp(-v)), fp64 (exp overflow gives the limit 0)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def rmsnorm(x, gamma, eps):
    """RMSNorm of each row of x (float64 [m, k]): x * r * gamma with
    r = 1 / sqrt(mean(x^2) + eps).  Returns (normalised x, r [m])."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float32).astype(np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + float(eps))
    return x * r[:, None] * g[None, :], r


def _row_weights(fmt, blocks, n, k, rows):
    """Decoded weights of the given rows, float64 [len(rows), k]."""
    b = _blocks(fmt, blocks, n, k)
    tail = b[n * (k // 16) * 9:] if fmt == NVFP4 else b[:0]      # the NVFP4 tensor scale
    body = b[:b.size - tail.size].reshape(n, -1)
    sub = np.ascontiguousarray(body[np.asarray(rows, dtype=np.int64)])
    return decode(fmt, np.concatenate([sub.reshape(-1), tail]), len(rows), k)


def dense_fused(fmt, blocks, n, k, x, xt, norm_weight=None, eps=0.0, act=ACT_NONE, residual=None, rows=None):
    """Fused dense step, by definition in fp64:
        x' = RMSNorm(x) if norm_weight is given, else x
        z  = W x'                          (all n rows)
        o  = SiLU(z[:F]) * z[F:]           if act == ACT_SWIGLU (F = n / 2)
             z                             otherwise
        o += residual                      if given ([m, n_out], fp32)
    Returns (o, scale) as float64 [m, nrows] over the output rows `rows`
    (default all n_out).  scale bounds the output's sensitivity to fp32
    rounding of the products: L1 = sum |w x'| of the row without the gate.
    With it, products off by |dg| <= e * L1_gate and |du| <= e * L1_up
    (e <= 2e-3) move o by at most e * scale with
        scale = 1.1 * L1_gate * (|u| + 2e-3 * L1_up) + |SiLU(g)| * L1_up,
    since |SiLU'| < 1.1 everywhere (the last term of the first product is
    the cross term dg * du)."""
    xv = x_values(x, xt).reshape(-1, k)
    if norm_weight is not None:
        xv, _ = rmsnorm(xv, norm_weight, eps)
    if act == ACT_SWIGLU:
        if n % 2:
            raise ValueError("SwiGLU needs an even row count")
        n_out = n // 2
    else:
        n_out = n
    o, scale = _fused_rows(fmt, blocks, n, k, xv, act, rows)
    r = np.arange(n_out) if rows is None else np.asarray(rows, dtype=np.int64)
    if residual is not None:
        o = o + np.asarray(residual, dtype=np.float32).astype(np.float64).reshape(-1, n_out)[:, r]
    return o, scale


def fused_err(yhat, o, scale, y_bf16=False):
    """max over outputs of (|yhat - o| - out_rel * |o|) / scale: the product
    error against its rounding scale once the output's own rounding is
    allowed for (out_rel = 2^-8 for bf16 outputs, 2^-20 for fp32, which also
    covers the few ulp of exp and the division in SiLU), the remainder
    clamped at 0.  Where scale == 0 the remainder must be 0; non-finite
    outputs give inf."""
    yhat = np.asarray(yhat, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    out_rel = 2.0 ** -8 if y_bf16 else 2.0 ** -20
    rest = np.maximum(np.abs(yhat - o) - out_rel * np.abs(o), 0.0)
    err = np.where(scale > 0, rest / np.where(scale > 0, scale, 1.0), np.where(rest > 0, np.inf, 0.0))
    err[~np.isfinite(yhat)] = np.inf
    return float(err.max()) if err.size else 0.0


def moe_fused(fmt, experts, n_experts, n, k, ids, g, x, xt, mode, norm_weight=None, eps=0.0, act=ACT_NONE,
              residual=None, rows=None):
    """Fused top-k expert step, by definition in fp64 (the definitions of
    dense_fused, per slot):
      MOE_GATE_UP:  x [m, k];  for each token t and slot j with a valid id
                    e = ids[t, j]:  z = W_e RMSNorm(x_t) (RMSNorm optional),
                    o[t, j] = SiLU(z[:F]) * z[F:] with ACT_SWIGLU, else z.
                    Slots with an invalid id get NaN (they have no output).
      MOE_DOWN:     x [m, top_k, k];  o[t] = sum over j ascending of
                    g[t, j] * W_{ids[t, j]} x[t, j]  (+ residual[t]).
    Returns (o, scale): gate_up [m, top_k, nrows], down [m, nrows]; scale as
    in dense_fused, for down the sum over slots of |g| * row L1."""
    ida = np.asarray(ids, dtype=np.int64)
    m, top_k = ida.shape
    per = tensor_bytes(fmt, n, k)
    e_all = np.ascontiguousarray(experts, dtype=np.uint8)
    if e_all.size != n_experts * per:
        raise ValueError("expert array size does not match")

    def expert(e):
        return e_all[e * per:(e + 1) * per]

    xv = x_values(x, xt)
    if mode == MOE_GATE_UP:
        xv = xv.reshape(m, k)
        if residual is not None:
            raise ValueError("gate_up takes no residual")
        n_out = n // 2 if act == ACT_SWIGLU else n
        nr = n_out if rows is None else len(rows)
        o = np.full((m, top_k, nr), np.nan)
        scale = np.zeros((m, top_k, nr))
        for t in range(m):
            for j in range(top_k):
                e = int(ida[t, j])
                if not 0 <= e < n_experts:
                    continue
                xt_row = xv[t:t + 1]
                if norm_weight is not None:
                    xt_row, _ = rmsnorm(xt_row, norm_weight, eps)
                # the product of the (normalised) fp64 row, as dense_fused does
                oo, ss = _fused_rows(fmt, expert(e), n, k, xt_row, act, rows)
                o[t, j], scale[t, j] = oo[0], ss[0]
        return o, scale
    if norm_weight is not None or act != ACT_NONE:
        raise ValueError("down-combine takes neither a normalisation nor a gate")
    xv = xv.reshape(m, top_k, k)
    ga = np.asarray(g, dtype=np.float32).astype(np.float64).reshape(m, top_k)
    nr = n if rows is None else len(rows)
    r = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((m, nr))
    scale = np.zeros((m, nr))
    for t in range(m):
        for j in range(top_k):
            e = int(ida[t, j])
            if not 0 <= e < n_experts:
                continue
            w = _row_weights(fmt, expert(e), n, k, r)
            o[t] += ga[t, j] * (w @ xv[t, j])
            scale[t] += abs(ga[t, j]) * (np.abs(w) @ np.abs(xv[t, j]))
    if residual is not None:
        o += np.asarray(residual, dtype=np.float32).astype(np.float64).reshape(m, n)[:, r]
    return o, scale


def _fused_rows(fmt, blocks, n, k, xv, act, rows):
    """dense_fused's product and gate for activations already in fp64."""
    if act == ACT_SWIGLU:
        if n % 2:
            raise ValueError("SwiGLU needs an even row count")
        n_out = n // 2
    else:
        n_out = n
    r = np.arange(n_out) if rows is None else np.asarray(rows, dtype=np.int64)
    if act == ACT_SWIGLU:
        wg = _row_weights(fmt, blocks, n, k, r)
        wu = _row_weights(fmt, blocks, n, k, r + n_out)
        g, l1g = xv @ wg.T, np.abs(xv) @ np.abs(wg).T
        u, l1u = xv @ wu.T, np.abs(xv) @ np.abs(wu).T
        return silu(g) * u, 1.1 * l1g * (np.abs(u) + 2e-3 * l1u) + np.abs(silu(g)) * l1u
    w = _row_weights(fmt, blocks, n, k, r)
    return xv @ w.T, np.abs(xv) @ np.abs(w).T
