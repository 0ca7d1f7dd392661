"""numpy implementation of the MFMA-tiled code layout, written from its
definition in include/rudder.h (used by the tests to compare the library's
packed bytes with the oracle's codes).

Block (rb, kb) covers rows 32rb..32rb+31 and k 32kb..32kb+31 and sits at
block index rb*(K/32)+kb; slot l = (r%32) + 32*((k%32)//16) holds the 16 codes
k = 32kb + 16*(l//32) + j.  8-bit: 16 bytes, byte j = code j.  4-bit: 8 bytes =
two split-nibble words (codes 8w..8w+7; byte i holds code 8w+i low, 8w+4+i high).
Rows R..ceil(R/32)*32-1 are zero padding.
"""
import numpy as np


def _pad_rows(codes: np.ndarray) -> np.ndarray:
    R, K = codes.shape
    Rp = (R + 31) // 32 * 32
    if Rp == R:
        return codes
    out = np.zeros((Rp, K), codes.dtype)
    out[:R] = codes
    return out


def _nibble_bytes(codes16: np.ndarray) -> np.ndarray:
    """[..., 16] int codes -> [..., 8] bytes in split-nibble words."""
    c = (codes16.astype(np.int16) & 0xF).astype(np.uint8)
    c = c.reshape(codes16.shape[:-1] + (2, 8))               # word, code-in-word
    lo = c[..., 0:4]
    hi = c[..., 4:8]
    return (lo | (hi << 4)).reshape(codes16.shape[:-1] + (8,))


def tile_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """int8 codes [R, K] -> flat uint8 buffer in the tiled layout."""
    codes = _pad_rows(np.asarray(codes, np.int8))
    Rp, K = codes.shape
    assert K % 32 == 0
    # [rb, r32, kb, half, j]
    t = codes.reshape(Rp // 32, 32, K // 32, 2, 16)
    # -> [rb, kb, half, r32, j]  (slot = r32 + 32*half)
    t = t.transpose(0, 2, 3, 1, 4)
    if bits == 8:
        return np.ascontiguousarray(t).view(np.uint8).reshape(-1)
    return np.ascontiguousarray(_nibble_bytes(t)).reshape(-1)


def untile_codes(buf: np.ndarray, R: int, K: int, bits: int) -> np.ndarray:
    """Flat tiled buffer -> int8 codes [ceil(R/32)*32, K] (padding rows kept)."""
    Rp = (R + 31) // 32 * 32
    buf = np.asarray(buf, np.uint8).reshape(-1)
    if bits == 8:
        t = buf[: Rp * K].view(np.int8).reshape(Rp // 32, K // 32, 2, 32, 16)
    else:
        b = buf[: Rp * K // 2].reshape(Rp // 32, K // 32, 2, 32, 2, 4)
        lo = (b & 0xF).astype(np.int8)
        hi = (b >> 4).astype(np.int8)
        lo = np.where(lo >= 8, lo - 16, lo)
        hi = np.where(hi >= 8, hi - 16, hi)
        t = np.concatenate([lo, hi], axis=-1).reshape(Rp // 32, K // 32, 2, 32, 16)
        t = t.astype(np.int8)
    return np.ascontiguousarray(t.transpose(0, 3, 1, 2, 4)).reshape(Rp, K)
