"""Seeded generators for canonical block bytes, activations and router outputs.

Canonical block layouts (the interchange format every entry point and the
oracle consume; little-endian, scale first, one block = 32 weights along K):

* Q8_0  (34 B): fp16 scale d, then 32 int8 codes in element order.
* Q4_0  (18 B): fp16 scale d, then 16 bytes; byte j holds element j in its low
  nibble and element j+16 in its high nibble.
* MXFP4 (17 B): one E8M0 exponent byte, then 16 bytes with the same nibble
  split as Q4_0; each nibble is an FP4 E2M1 code (sign in bit 3).

A matrix of N rows by K columns is N*(K/32) blocks, row-major.

Seeds follow numpy.random.SeedSequence([2026, config, matrix, role]) so every
input of every workload is reproducible on any host.
"""
import numpy as np

QK = 32
FMT_Q8_0, FMT_Q4_0, FMT_MXFP4 = 0, 1, 2
FMT_NAMES = {FMT_Q8_0: "q8_0", FMT_Q4_0: "q4_0", FMT_MXFP4: "mxfp4"}
BLOCK_BYTES = {FMT_Q8_0: 34, FMT_Q4_0: 18, FMT_MXFP4: 17}

ROLES = {"codes": 0, "scales": 1, "x": 2, "router": 3, "h": 4, "gamma": 5, "res": 6}


def rng_for(config, matrix, role):
    """Independent generator per (config, matrix, role)."""
    return np.random.default_rng(np.random.SeedSequence([2026, int(config), int(matrix), ROLES[role]]))


# ---------------------------------------------------------------- encoders
def encode_q8_0(codes, d_bits):
    """codes int8 [n, nb, 32], d_bits uint16 [n, nb] -> uint8 [n, nb, 34]."""
    n, nb, _ = codes.shape
    out = np.empty((n, nb, 34), dtype=np.uint8)
    out[:, :, 0] = (d_bits & 0xFF).astype(np.uint8)
    out[:, :, 1] = (d_bits >> 8).astype(np.uint8)
    out[:, :, 2:] = codes.view(np.uint8)
    return out


def _nibble_pack(q):
    """q uint8 [..., 32] in 0..15 -> [..., 16] with byte j = q[j] | q[j+16] << 4."""
    return (q[..., :16] | (q[..., 16:] << 4)).astype(np.uint8)


def encode_q4_0(q, d_bits):
    """q uint8 [n, nb, 32] in 0..15, d_bits uint16 [n, nb] -> uint8 [n, nb, 18]."""
    n, nb, _ = q.shape
    out = np.empty((n, nb, 18), dtype=np.uint8)
    out[:, :, 0] = (d_bits & 0xFF).astype(np.uint8)
    out[:, :, 1] = (d_bits >> 8).astype(np.uint8)
    out[:, :, 2:] = _nibble_pack(q)
    return out


def encode_mxfp4(c, e):
    """c uint8 [n, nb, 32] E2M1 codes 0..15, e uint8 [n, nb] -> uint8 [n, nb, 17]."""
    n, nb, _ = c.shape
    out = np.empty((n, nb, 17), dtype=np.uint8)
    out[:, :, 0] = e
    out[:, :, 1:] = _nibble_pack(c)
    return out


# ---------------------------------------------------------------- draws
def _fp16_bits_uniform(rng, shape, lo, hi):
    # numpy's float64 -> float16 cast rounds to nearest even
    return rng.uniform(lo, hi, size=shape).astype(np.float16).view(np.uint16)


def q8_0_blocks(n, k, rng_codes, rng_scales, code_lo=-127, code_hi=127, d_lo=1e-3, d_hi=1e-2):
    nb = k // QK
    codes = rng_codes.integers(code_lo, code_hi + 1, size=(n, nb, QK), dtype=np.int8)
    return encode_q8_0(codes, _fp16_bits_uniform(rng_scales, (n, nb), d_lo, d_hi))


def q4_0_blocks(n, k, rng_codes, rng_scales, d_lo=1e-3, d_hi=1e-2):
    nb = k // QK
    q = rng_codes.integers(0, 16, size=(n, nb, QK), dtype=np.uint8)
    return encode_q4_0(q, _fp16_bits_uniform(rng_scales, (n, nb), d_lo, d_hi))


def mxfp4_blocks(n, k, rng_codes, rng_scales, e_lo=-8, e_hi=-2):
    nb = k // QK
    c = rng_codes.integers(0, 16, size=(n, nb, QK), dtype=np.uint8)
    e = (127 + rng_scales.integers(e_lo, e_hi + 1, size=(n, nb))).astype(np.uint8)
    return encode_mxfp4(c, e)


def blocks_for(fmt, n, k, config, matrix):
    """Canonical blocks of one matrix of a workload, drawn with the workload seeds."""
    rc, rs = rng_for(config, matrix, "codes"), rng_for(config, matrix, "scales")
    if fmt == FMT_Q8_0:
        return q8_0_blocks(n, k, rc, rs)
    if fmt == FMT_Q4_0:
        return q4_0_blocks(n, k, rc, rs)
    if fmt == FMT_MXFP4:
        return mxfp4_blocks(n, k, rc, rs)
    raise ValueError(fmt)


def f32_to_bf16_bits_rne(a):
    """float32 array -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def x_f32(shape, rng):
    return rng.standard_normal(size=shape, dtype=np.float64).astype(np.float32)


def x_bf16_bits(shape, rng):
    return f32_to_bf16_bits_rne(x_f32(shape, rng))


def norm_weight_f32(k, rng, lo=0.25, hi=2.0):
    """RMSNorm weights: fp32 uniform in [lo, hi] (positive, around 1, as a
    trained norm's are)."""
    return rng.uniform(lo, hi, size=k).astype(np.float32)


def router_topk(m, n_experts, top_k, rng):
    """Router stand-in for the expert GEMV inputs.

    Logits ~ N(0,1) fp32 [m, n_experts]; the top_k experts by descending logit
    (lower index wins a tie) in that slot order; weights = softmax over the
    selected logits, evaluated in float64 and stored as float32.
    Returns (logits, ids int32 [m, top_k], weights float32 [m, top_k]).
    """
    logits = x_f32((m, n_experts), rng)
    ids = np.empty((m, top_k), dtype=np.int32)
    w = np.empty((m, top_k), dtype=np.float32)
    for t in range(m):
        order = sorted(range(n_experts), key=lambda e: (-float(logits[t, e]), e))[:top_k]
        ids[t] = order
        sel = logits[t, order].astype(np.float64)
        ex = np.exp(sel - sel.max())
        w[t] = (ex / ex.sum()).astype(np.float32)
    return logits, ids, w
