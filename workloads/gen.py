"""Seeded generators for canonical block bytes, activations and router outputs.

Canonical block layouts (the interchange format every entry point and the
oracle consume; little-endian, scale first, one block = 32 weights along K):

* Q8_0  (34 B): fp16 scale d, then 32 int8 codes in element order.
* Q4_0  (18 B): fp16 scale d, then 16 bytes; byte j holds element j in its low
  nibble and element j+16 in its high nibble.
* MXFP4 (17 B): one E8M0 exponent byte, then 16 bytes with the same nibble
  split as Q4_0; each nibble is an FP4 E2M1 code (sign in bit 3).
* NVFP4 (9 B per 16 weights): one FP8 E4M3 scale byte, then 8 bytes; byte j
  holds element j in its low nibble and element j+8 in its high nibble (E2M1
  codes).  A tensor ends with its fp32 scale (4 bytes, little-endian).
* Q4_K (144 B per 256 weights): fp16 d, fp16 dmin, 12 bytes of packed 6-bit
  sub-block scales and mins, 128 bytes of 4-bit codes (the GGUF super-block).
* Q6_K (210 B per 256 weights): 128 bytes of low code bits, 64 bytes of high
  code bits, 16 int8 scales, fp16 d (the GGUF super-block).

A matrix of N rows by K columns is N*(K/32) blocks (N*(K/256) super-blocks
for the K-quants), row-major.

Seeds follow numpy.random.SeedSequence([2026, config, matrix, role]) so every
input of every workload is reproducible on any host.
"""
import numpy as np

QK = 32
FMT_Q8_0, FMT_Q4_0, FMT_MXFP4, FMT_NVFP4, FMT_Q4_K, FMT_Q6_K = 0, 1, 2, 3, 4, 5
FMT_NAMES = {FMT_Q8_0: "q8_0", FMT_Q4_0: "q4_0", FMT_MXFP4: "mxfp4", FMT_NVFP4: "nvfp4", FMT_Q4_K: "q4_k",
             FMT_Q6_K: "q6_k"}
BLOCK_BYTES = {FMT_Q8_0: 34, FMT_Q4_0: 18, FMT_MXFP4: 17, FMT_NVFP4: 9,   # NVFP4 per 16 weights
               FMT_Q4_K: 144, FMT_Q6_K: 210}                              # K-quants per 256 weights
BLOCK_LEN = {FMT_Q8_0: 32, FMT_Q4_0: 32, FMT_MXFP4: 32, FMT_NVFP4: 16, FMT_Q4_K: 256, FMT_Q6_K: 256}


def canon_bytes(fmt, n, k):
    """Bytes of one canonical n x k tensor (NVFP4: blocks of 16 weights, then
    the 4-byte fp32 tensor scale)."""
    if fmt == FMT_NVFP4:
        return n * (k // 16) * 9 + 4
    return n * (k // BLOCK_LEN[fmt]) * BLOCK_BYTES[fmt]


def bytes_per_weight(fmt):
    """Canonical bytes per weight (the NVFP4 tensor scale left out)."""
    return BLOCK_BYTES[fmt] / BLOCK_LEN[fmt]

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


def q4_0_zero_heavy_blocks(n, k, rng_codes, rng_scales, d_lo=1e-3, d_hi=1e-2):
    """Q4_0 rows dominated by code 8 (weight zero), with non-zero scales:
    row r % 4 == 0 all code 8; 1 one code other than 8, anywhere in the row;
    2 mostly 8 (each code drawn from 0..15 with probability 1/16); 3 uniform."""
    nb = k // QK
    q = np.full((n, nb, QK), 8, dtype=np.uint8)
    kind = np.arange(n) % 4
    others = np.array([c for c in range(16) if c != 8], dtype=np.uint8)
    for r in np.nonzero(kind == 1)[0]:
        pos = rng_codes.integers(0, nb * QK)
        q[r].reshape(-1)[pos] = others[rng_codes.integers(0, len(others))]
    few = (kind == 2)[:, None, None] & (rng_codes.random((n, nb, QK)) < 1.0 / 16)
    q[few] = rng_codes.integers(0, 16, size=int(few.sum()), dtype=np.uint8)
    full = kind == 3
    q[full] = rng_codes.integers(0, 16, size=(int(full.sum()), nb, QK), dtype=np.uint8)
    return encode_q4_0(q, _fp16_bits_uniform(rng_scales, (n, nb), d_lo, d_hi))


def mxfp4_blocks(n, k, rng_codes, rng_scales, e_lo=-8, e_hi=-2):
    nb = k // QK
    c = rng_codes.integers(0, 16, size=(n, nb, QK), dtype=np.uint8)
    e = (127 + rng_scales.integers(e_lo, e_hi + 1, size=(n, nb))).astype(np.uint8)
    return encode_mxfp4(c, e)


def nvfp4_tensor(n, k, rng_codes, rng_scales, ts=None):
    """Canonical NVFP4 tensor: per 16 weights one E4M3 scale byte (uniform
    over the normal codes 0x20..0x57, values 2^-3 .. 15) then 8 code bytes
    (byte j = element j | element j+8 << 4, codes uniform 0..15); then the fp32
    tensor scale (drawn log-uniform in [1e-4, 1e-3] unless given)."""
    nb = k // 16
    codes = rng_codes.integers(0, 16, size=(n, nb, 16), dtype=np.uint8)
    sc = rng_scales.integers(0x20, 0x58, size=(n, nb), dtype=np.uint8)
    body = np.empty((n, nb, 9), dtype=np.uint8)
    body[:, :, 0] = sc
    body[:, :, 1:] = codes[..., :8] | (codes[..., 8:] << 4)
    if ts is None:
        ts = float(np.float32(10.0 ** rng_scales.uniform(-4, -3)))
    tail = np.array([ts], dtype=np.float32).view(np.uint8)
    return np.concatenate([body.reshape(-1), tail])


def _f16_bits(v):
    return np.asarray(v, dtype=np.float16).view(np.uint16)


def q4_k_blocks(n, k, rng_codes, rng_scales):
    """Canonical Q4_K super-blocks [n, k/256, 144]: d and dmin fp16 drawn
    uniform in [1e-4, 1e-3], the 12 scale/min bytes and the 128 code bytes
    uniform over all byte values (so every 6-bit scale and min and every
    4-bit code occurs)."""
    ns = k // 256
    out = np.empty((n, ns, 144), dtype=np.uint8)
    d = _f16_bits(rng_scales.uniform(1e-4, 1e-3, size=(n, ns)))
    dm = _f16_bits(rng_scales.uniform(1e-4, 1e-3, size=(n, ns)))
    out[:, :, 0], out[:, :, 1] = d & 0xFF, d >> 8
    out[:, :, 2], out[:, :, 3] = dm & 0xFF, dm >> 8
    out[:, :, 4:16] = rng_scales.integers(0, 256, size=(n, ns, 12), dtype=np.uint8)
    out[:, :, 16:] = rng_codes.integers(0, 256, size=(n, ns, 128), dtype=np.uint8)
    return out


def q6_k_blocks(n, k, rng_codes, rng_scales):
    """Canonical Q6_K super-blocks [n, k/256, 210]: code bytes (low and high
    bits) uniform over all byte values, int8 scales uniform in [-128, 127], d
    fp16 drawn uniform in [1e-6, 1e-5] with a random sign."""
    ns = k // 256
    out = np.empty((n, ns, 210), dtype=np.uint8)
    out[:, :, :192] = rng_codes.integers(0, 256, size=(n, ns, 192), dtype=np.uint8)
    out[:, :, 192:208] = rng_scales.integers(0, 256, size=(n, ns, 16), dtype=np.uint8)
    d = _f16_bits(rng_scales.uniform(1e-6, 1e-5, size=(n, ns)) * rng_scales.choice([-1.0, 1.0], size=(n, ns)))
    out[:, :, 208], out[:, :, 209] = d & 0xFF, d >> 8
    return out


def blocks_for(fmt, n, k, config, matrix):
    """Canonical blocks of one matrix of a workload, drawn with the workload seeds."""
    rc, rs = rng_for(config, matrix, "codes"), rng_for(config, matrix, "scales")
    if fmt == FMT_Q8_0:
        return q8_0_blocks(n, k, rc, rs)
    if fmt == FMT_Q4_0:
        return q4_0_blocks(n, k, rc, rs)
    if fmt == FMT_MXFP4:
        return mxfp4_blocks(n, k, rc, rs)
    if fmt == FMT_NVFP4:
        return nvfp4_tensor(n, k, rc, rs)
    if fmt == FMT_Q4_K:
        return q4_k_blocks(n, k, rc, rs)
    if fmt == FMT_Q6_K:
        return q6_k_blocks(n, k, rc, rs)
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


def x_mixed_f32(shape, rng, decades=3.0):
    """N(0,1) times 10^U(-decades, decades): magnitudes spread over
    2 * decades decades inside every block."""
    x = rng.standard_normal(size=shape) * 10.0 ** rng.uniform(-decades, decades, size=shape)
    return x.astype(np.float32)


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
