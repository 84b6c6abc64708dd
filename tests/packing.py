"""The packed weight layout written by wq_prepack_weight, restated in NumPy for the tests.

A (k, n) weight is cut into 64 k x 32 column blocks, k blocks outer, n blocks inner.  A block
holds, for each 16-k step s (0..3), the codes of 64 lanes in lane order: lane l is column
l % 32 and k 16 s + 8 (l // 32) + e for e = 0..7.  One-byte codes (int8, FLOAT8_E4M3FN) take
8 bytes per lane (e ascending).  int4 blocks go in pairs (2p, 2p + 1), stored as one 2048-byte
unit of the same lane order: byte e of a lane holds the codes of both blocks at that lane's
column and k, block 2p in bits 0-3.  Codes at k past the end are zero.  This layout is the library's own
(include/wqgemm.h describes it); these helpers are test infrastructure.
"""
import numpy as np


def logical_codes(x2, weight, transposed=False):
    """Storage (as the workloads module draws it) -> (k, n) integer codes: int8 values, the
    FLOAT8_E4M3FN bit patterns as 0..255, or int4 values -8..7."""
    if weight == "int4":
        b = np.asarray(x2, dtype=np.uint8)
        lo = (b & 0xF).astype(np.int16)
        hi = (b >> 4).astype(np.int16)
        lo[lo >= 8] -= 16
        hi[hi >= 8] -= 16
        v = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int16)
        v[:, 0::2] = lo
        v[:, 1::2] = hi
        return v.T if transposed else v   # transposed storage is (n, k/2), nibbles along k
    v = np.asarray(x2).view(np.uint8 if weight == "fp8e4m3" else np.int8).astype(np.int16)
    return v.T if transposed else v


def pack_reference(codes, int4):
    """(k, n) codes -> the packed bytes (uint8, flat)."""
    codes = np.asarray(codes, dtype=np.int64)
    k, n = codes.shape
    kb, nb = -(-k // 64), n // 32
    c = np.zeros((kb * 64, n), dtype=np.int64)
    c[:k] = codes
    # k = 64 kb + 16 s + 8 h + e, column = 32 nb + col  ->  [kb][nb][s][h][col][e]
    t = c.reshape(kb, 4, 2, 8, nb, 32).transpose(0, 4, 1, 2, 5, 3)
    if not int4:
        return (t & 0xFF).astype(np.uint8).reshape(-1)
    # column blocks 2p and 2p + 1 share the bytes of pair p: [kb][p][s][h][col][e]
    nib = (t & 0xF).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8).reshape(-1)


def unpack_reference(packed, k, n, int4):
    """The inverse, element by element (a loop over the layout's definition, for small
    shapes)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.zeros((k, n), dtype=np.int64)
    for kk in range(k):
        for col in range(n):
            kb, kr = divmod(kk, 64)
            s, r = divmod(kr, 16)
            h, e = divmod(r, 8)
            lane = 32 * h + col % 32
            if int4:   # 2048-byte units of two column blocks, n // 64 per k block
                base = (kb * (n // 64) + col // 64) * 2048 + (s * 64 + lane) * 8
                v = (int(packed[base + e]) >> (4 * ((col // 32) % 2))) & 0xF
                out[kk, col] = v - 16 if v >= 8 else v
            else:
                base = (kb * (n // 32) + col // 32) * 2048 + (s * 64 + lane) * 8
                out[kk, col] = int(packed[base + e])
    return out
