"""Test-side encoders and decoders for the two weight formats.

Written independently of the oracle's C decoder (Python integers for the 96-bit
scale string, numpy views for fp16 and int8) so that a special-case input built
here pins the oracle's decoding: if the oracle read a field, a nibble or a scale
from the wrong place, the closed-form expectations in the tests would not hold.

Layouts (the library's own; the pages name the formats but give no bytes):
  Q8_0 block: fp16 d, then 32 int8 quants (34 bytes).
  Q4_K superblock: fp16 d, fp16 dmin, 12 bytes holding sixteen 6-bit fields as
  a little-endian 96-bit string (fields 0..7 scales, 8..15 mins), then 128 bytes
  of nibbles: sub-block 2p in the low nibbles of bytes 16+32p..16+32p+31,
  sub-block 2p+1 in the high nibbles of the same bytes (144 bytes).
"""
import numpy as np


def fp16_bits(v: float) -> int:
    return int(np.array([v], np.float16).view(np.uint16)[0])


def pack_q4k_superblock(d: float, dmin: float, sc, m, q) -> bytes:
    """sc, m: 8 ints in 0..63; q: [8][32] ints in 0..15."""
    fields = list(sc) + list(m)
    assert len(fields) == 16 and all(0 <= f < 64 for f in fields)
    bits = 0
    for f, val in enumerate(fields):
        bits |= int(val) << (6 * f)
    out = bytearray()
    out += fp16_bits(d).to_bytes(2, "little")
    out += fp16_bits(dmin).to_bytes(2, "little")
    out += bits.to_bytes(12, "little")
    for p in range(4):
        for i in range(32):
            lo, hi = int(q[2 * p][i]), int(q[2 * p + 1][i])
            assert 0 <= lo < 16 and 0 <= hi < 16
            out.append(lo | (hi << 4))
    assert len(out) == 144
    return bytes(out)


def pack_q4k_matrix(d, dmin, sc, m, q) -> np.ndarray:
    """d, dmin: [N, S]; sc, m: [N, S, 8]; q: [N, S, 8, 32]  ->  uint8 [N, S*144]."""
    d = np.asarray(d, np.float64)
    N, S = d.shape
    rows = []
    for n in range(N):
        row = b"".join(pack_q4k_superblock(d[n, s], dmin[n, s], sc[n, s], m[n, s], q[n, s]) for s in range(S))
        rows.append(np.frombuffer(row, np.uint8))
    return np.stack(rows)


def unpack_q4k_fields(W: np.ndarray, N: int, K: int):
    """numpy decode: d, dmin [N,S] float64; sc, m [N,S,8] int; q [N,S,8,32] int."""
    S = K // 256
    sb = np.asarray(W, np.uint8).reshape(N, S, 144)
    d = sb[:, :, 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    dmin = sb[:, :, 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    sc = np.empty((N, S, 8), np.int64)
    m = np.empty((N, S, 8), np.int64)
    for n in range(N):
        for s in range(S):
            bits = int.from_bytes(bytes(sb[n, s, 4:16]), "little")
            for f in range(16):
                val = (bits >> (6 * f)) & 63
                if f < 8:
                    sc[n, s, f] = val
                else:
                    m[n, s, f - 8] = val
    qs = sb[:, :, 16:].reshape(N, S, 4, 32).astype(np.int64)
    q = np.empty((N, S, 8, 32), np.int64)
    q[:, :, 0::2, :] = qs & 15
    q[:, :, 1::2, :] = qs >> 4
    return d, dmin, sc, m, q


def numpy_dequant_q4k(W: np.ndarray, N: int, K: int) -> np.ndarray:
    d, dmin, sc, m, q = unpack_q4k_fields(W, N, K)
    w = d[:, :, None, None] * sc[:, :, :, None] * q - dmin[:, :, None, None] * m[:, :, :, None]
    return w.reshape(N, K)


def unpack_q8_0(W: np.ndarray, N: int, K: int):
    nb = K // 32
    blk = np.asarray(W, np.uint8).reshape(N, nb, 34)
    d = blk[:, :, 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    q = blk[:, :, 2:].copy().view(np.int8).astype(np.int64)
    return d, q


def numpy_dequant_q8_0(W: np.ndarray, N: int, K: int) -> np.ndarray:
    d, q = unpack_q8_0(W, N, K)
    return (d[:, :, None] * q).reshape(N, K)


def integer_activation(g: np.random.Generator, M: int, K: int) -> np.ndarray:
    """fp32 integer-valued activations with |x| <= 127 and every 32-block holding a +-127,
    so the Q8 quantizer must return scale 1 and quants equal to x."""
    x = g.integers(-127, 128, size=(M, K // 32, 32)).astype(np.float32)
    pos = g.integers(0, 32, size=(M, K // 32))
    sign = np.where(g.integers(0, 2, size=(M, K // 32)) == 0, -1.0, 1.0).astype(np.float32)
    np.put_along_axis(x, pos[..., None], (127.0 * sign)[..., None], axis=2)
    return x.reshape(M, K)
