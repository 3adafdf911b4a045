"""Host-side reference of the tiled MXFP4 payload layout, written from its definition
in include/sharq.h (used by the tests to check device payloads independently of the
library's own re-layout kernel).

codes: fragment (rt, kc) = rows 32rt..32rt+31, elements 64kc..64kc+63, at byte
((rt * Kp/64) + kc) * 1024; row r's block b = 2kc + c occupies slot (r % 32) + 32c
(16 bytes).  scales: byte (b % 4) of the 32-bit word (ks * Rp + r), ks = b // 4.
Rp = rows rounded up to 32, Kp = K rounded up to 128; padding is zero.
"""
import numpy as np


def padded(rows, K):
    return (rows + 31) // 32 * 32, (K + 127) // 128 * 128


def tile(codes, scales):
    """Row-major codes [rows, K/2] and scales [rows, K/32] -> flat tiled arrays."""
    rows, kb = codes.shape
    K = kb * 2
    Rp, Kp = padded(rows, K)
    c = np.zeros((Rp, Kp // 2), np.uint8)
    c[:rows, :K // 2] = codes
    s = np.zeros((Rp, Kp // 32), np.uint8)
    s[:rows, :K // 32] = scales
    # [Rp/32, 32 rows, Kp/64 kc, 2 c, 16 bytes] -> [Rp/32, kc, c, 32 rows, 16 bytes]
    ct = c.reshape(Rp // 32, 32, Kp // 64, 2, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
    # scales [Rp, Kp/128, 4] -> [Kp/128, Rp, 4]
    st = s.reshape(Rp, Kp // 128, 4).transpose(1, 0, 2).reshape(-1)
    return ct.copy(), st.copy()


def untile(ct, st, rows, K):
    """Flat tiled arrays -> row-major codes [rows, K/2], scales [rows, K/32]."""
    Rp, Kp = padded(rows, K)
    c = np.asarray(ct, np.uint8).reshape(Rp // 32, Kp // 64, 2, 32, 16).transpose(0, 3, 1, 2, 4).reshape(Rp, Kp // 2)
    s = np.asarray(st, np.uint8).reshape(Kp // 128, Rp, 4).transpose(1, 0, 2).reshape(Rp, Kp // 32)
    return c[:rows, :K // 2].copy(), s[:rows, :K // 32].copy()


def padding_is_zero(ct, st, rows, K):
    Rp, Kp = padded(rows, K)
    c = np.asarray(ct, np.uint8).reshape(Rp // 32, Kp // 64, 2, 32, 16).transpose(0, 3, 1, 2, 4).reshape(Rp, Kp // 2)
    s = np.asarray(st, np.uint8).reshape(Kp // 128, Rp, 4).transpose(1, 0, 2).reshape(Rp, Kp // 32)
    return (not c[rows:].any() and not c[:, K // 2:].any() and not s[rows:].any() and not s[:, K // 32:].any())
