"""Byte builders for K-quant super-blocks (and the Q4_0 / Q8_0 blocks they
reduce to), shared by the K-quant tests: each writes the fields of one block
where the format puts them (which bytes and bits hold which weight), from
the values given."""
import numpy as np


def _f16(v):
    return int(np.array(v, dtype=np.float16).view(np.uint16))


def q4k_block(d, dmin, scmin, codes):
    """Q4_K super-block bytes from d, dmin, eight (sc, m) 6-bit pairs and 256
    codes (0..15) in weight order."""
    b = np.zeros(144, dtype=np.uint8)
    b[0:2] = np.frombuffer(np.array(_f16(d), dtype=np.uint16).tobytes(), dtype=np.uint8)
    b[2:4] = np.frombuffer(np.array(_f16(dmin), dtype=np.uint16).tobytes(), dtype=np.uint8)
    s = np.zeros(12, dtype=np.int64)
    for j, (sc, m) in enumerate(scmin):
        assert 0 <= sc < 64 and 0 <= m < 64
        if j < 4:
            s[j] |= sc
            s[j + 4] |= m
        else:
            s[j + 4] |= (sc & 15) | ((m & 15) << 4)
            s[j - 4] |= (sc >> 4) << 6
            s[j] |= (m >> 4) << 6
    b[4:16] = s.astype(np.uint8)
    codes = np.asarray(codes).astype(np.int64)
    for c in range(4):
        for l in range(32):
            b[16 + 32 * c + l] = codes[64 * c + l] | (codes[64 * c + 32 + l] << 4)
    return b


def q6k_block(d, scales, q):
    """Q6_K super-block bytes from d, sixteen int8 scales and 256 six-bit codes
    (0..63) in weight order."""
    b = np.zeros(210, dtype=np.uint8)
    q = np.asarray(q)
    for i in range(256):
        h, r, l = i // 128, (i % 128) // 32, i % 32
        lo, hi = int(q[i]) & 15, int(q[i]) >> 4
        li = 64 * h + l + 32 * (r & 1)
        b[li] |= lo if r < 2 else lo << 4
        b[128 + 32 * h + l] |= hi << (2 * r)
    b[192:208] = np.asarray(scales, dtype=np.int8).view(np.uint8)
    b[208:210] = np.frombuffer(np.array(_f16(d), dtype=np.uint16).tobytes(), dtype=np.uint8)
    return b


def q6k_scale_index(i):
    """Scale slot of weight i of a Q6_K super-block."""
    h, r, l = i // 128, (i % 128) // 32, i % 32
    return 8 * h + 2 * r + l // 16


def q4_0_block(d, q32):
    """Q4_0 block (32 weights) from d and codes 0..15 in element order."""
    q32 = np.asarray(q32)
    b = np.zeros(18, dtype=np.uint8)
    b[0:2] = np.frombuffer(np.array(_f16(d), dtype=np.uint16).tobytes(), dtype=np.uint8)
    b[2:] = q32[:16] | (q32[16:] << 4)
    return b


def q8_0_block(d, c32):
    b = np.zeros(34, dtype=np.uint8)
    b[0:2] = np.frombuffer(np.array(_f16(d), dtype=np.uint16).tobytes(), dtype=np.uint8)
    b[2:] = np.asarray(c32, dtype=np.int8).view(np.uint8)
    return b


