"""Host-side (numpy) reference of the packed int8 layout of include/int8mm.h:
16-row x 64-byte blocks ordered row-block major, chunk-major inside, rows
padded to 16 and K to 64 with zeros.  Used to prepare and to read back
packed buffers in tests; independent of the HIP code."""
import numpy as np


def kpad(K):
    return (K + 63) // 64 * 64


def rpad(R):
    return (R + 15) // 16 * 16


def pack(a):
    """row-major int8 [R,K] -> packed bytes, shape [rpad(R), kpad(K)]"""
    a = np.asarray(a, dtype=np.int8)
    R, K = a.shape
    Rp, Kp = rpad(R), kpad(K)
    full = np.zeros((Rp, Kp), np.int8)
    full[:R, :K] = a
    # [rb, r, kb, c, b] -> [rb, kb, c, r, b]
    blk = full.reshape(Rp // 16, 16, Kp // 64, 4, 16).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(blk).reshape(Rp, Kp)


def unpack(p, R, K):
    """packed bytes (any shape, rpad(R)*kpad(K) bytes) -> [rpad(R), kpad(K)] row-major;
    slice [:R, :K] for the matrix, the rest is padding."""
    Rp, Kp = rpad(R), kpad(K)
    p = np.asarray(p, dtype=np.int8).reshape(Rp // 16, Kp // 64, 4, 16, 16)
    return np.ascontiguousarray(p.transpose(0, 3, 1, 2, 4)).reshape(Rp, Kp)
