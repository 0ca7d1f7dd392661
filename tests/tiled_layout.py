"""numpy implementation of the MFMA-tiled code layout, written from its
definition in include/rudder.h (used by the tests to compare the library's
packed bytes with the oracle's codes).

Block (rb, kb) covers rows 32rb..32rb+31 and k 32kb..32kb+31 and sits at
block index rb*(K/32)+kb; slot l = (r%32) + 32*((k%32)//16) holds the 16 codes
k = 32kb + 16*(l//32) + j.  8-bit: 16 bytes, byte j = code j.  4-bit: 8 bytes =
two split-nibble words (codes 8w..8w+7; byte i holds code 8w+i low, 8w+4+i high).
Rows R..ceil(R/32)*32-1 are zero padding.  The E2M3 container (4-bit codes,
and 8-bit codes as two digit planes) follows below.
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


# ---------------------------------------------------------------------------
# E2M3 container (definition in include/rudder.h): each code c in [-7, 7] is
# the 6-bit FP6 E2M3 encoding of the integer c; 32 x 64 blocks of 1536 bytes;
# slot l = (r%32) + 32*((k%64)//32) holds 32 codes as a 192-bit little-endian
# string (code t at bits 6t..6t+5): bits 0..127 at byte 16*l (plane 0), bits
# 128..191 at byte 1024 + 8*l (plane 1).
# ---------------------------------------------------------------------------
E2M3_OF = {0: 0x00, 1: 0x08, 2: 0x10, 3: 0x14, 4: 0x18, 5: 0x1A, 6: 0x1C, 7: 0x1E}


def e2m3_value(code6: np.ndarray) -> np.ndarray:
    """Decode 6-bit E2M3 fields to floats straight from the format (sign,
    2-bit exponent with bias 1, 3-bit mantissa, subnormals at exponent 0)."""
    c = np.asarray(code6, np.int64)
    sign = np.where(c & 0x20, -1.0, 1.0)
    e = (c >> 3) & 0x3
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0, (1.0 + m / 8.0) * 2.0 ** (e - 1))
    return sign * mag


def e2m3_field(v: np.ndarray) -> np.ndarray:
    """Encode values exactly representable in E2M3 as 6-bit fields, from the
    format's definition: |v| = m/8 (exponent field 0) or (1 + m/8) 2^(e-1)
    (exponent field e = 1..3), sign in bit 5, zero as 0x00."""
    v = np.asarray(v, np.float64)
    mag = np.abs(v)
    e = np.where(mag < 1.0, 0, np.floor(np.log2(np.maximum(mag, 1.0))) + 1).astype(np.int64)
    m = np.where(e == 0, mag * 8.0, (mag / 2.0 ** (np.maximum(e, 1) - 1) - 1.0) * 8.0)
    assert np.all(e <= 3) and np.all(m == np.round(m)) and np.all(m < 8), "not exact in E2M3"
    sign = np.where((v < 0) & (mag > 0), 0x20, 0)
    return (sign | (e << 3) | m.astype(np.int64)).astype(np.uint8)


def digits_a8(codes: np.ndarray):
    """8-bit codes q -> the digits (h, l) of q = 16 h + l, l = ((q + 8) mod 16) - 8."""
    q = np.asarray(codes, np.int64)
    lo = np.mod(q + 8, 16) - 8
    hi = (q - lo) // 16
    return hi, lo


def tile_codes_e2m3(codes: np.ndarray) -> np.ndarray:
    codes = _pad_rows(np.asarray(codes, np.int8))
    enc = np.vectorize(lambda v: E2M3_OF[abs(int(v))] | (0x20 if v < 0 else 0))(codes)
    return _tile_fields_e2m3(enc).reshape(-1)


def tile_codes_e2m3_a8(codes: np.ndarray) -> np.ndarray:
    """8-bit codes -> 3072-byte blocks: the h/2 block, then the l/2 block."""
    codes = _pad_rows(np.asarray(codes, np.int8))
    hi, lo = digits_a8(codes)
    th = _tile_fields_e2m3(e2m3_field(hi / 2.0))
    tl = _tile_fields_e2m3(e2m3_field(lo / 2.0))
    return np.ascontiguousarray(np.concatenate([th, tl], axis=-1)).reshape(-1)


def _tile_fields_e2m3(enc: np.ndarray) -> np.ndarray:
    """6-bit fields [Rp, K] -> blocks [Rp/32, K/64, 1536]."""
    Rp, K = enc.shape
    assert K % 64 == 0 and Rp % 32 == 0
    enc = enc.astype(np.uint64)
    # [rb, r32, kb, half, t] -> [rb, kb, half, r32, t]
    t = enc.reshape(Rp // 32, 32, K // 64, 2, 32).transpose(0, 2, 3, 1, 4)
    # assemble 192-bit strings as three 64-bit words
    words = np.zeros(t.shape[:-1] + (3,), np.uint64)
    for ti in range(32):
        bit = 6 * ti
        w, off = bit // 64, bit % 64
        words[..., w] |= t[..., ti] << np.uint64(off)
        if off > 58:
            words[..., w + 1] |= t[..., ti] >> np.uint64(64 - off)
    b = words.view(np.uint8).reshape(t.shape[:-1] + (24,))      # [rb, kb, half, r32, 24]
    b = b.reshape(Rp // 32, K // 64, 64, 24)                      # slot = r32 + 32*half
    out = np.concatenate([b[..., :16].reshape(Rp // 32, K // 64, 1024),
                          b[..., 16:].reshape(Rp // 32, K // 64, 512)], axis=-1)
    return np.ascontiguousarray(out)


def untile_values_e2m3(blk: np.ndarray, Rp: int, K: int) -> np.ndarray:
    """Blocks [Rp/32, K/64, 1536] -> decoded E2M3 values [Rp, K]."""
    p0 = blk[..., :1024].reshape(Rp // 32, K // 64, 64, 16)
    p1 = blk[..., 1024:].reshape(Rp // 32, K // 64, 64, 8)
    b = np.concatenate([p0, p1], axis=-1)                          # [rb, kb, slot, 24]
    words = np.ascontiguousarray(b).view(np.uint64)                # [rb, kb, slot, 3]
    vals = np.zeros(b.shape[:-1] + (32,), np.int64)
    for ti in range(32):
        bit = 6 * ti
        w, off = bit // 64, bit % 64
        v = words[..., w] >> np.uint64(off)
        if off > 58:
            v |= words[..., w + 1] << np.uint64(64 - off)
        vals[..., ti] = (v & np.uint64(0x3F)).astype(np.int64)
    dec = e2m3_value(vals).reshape(Rp // 32, K // 64, 2, 32, 32)      # [rb, kb, half, r32, t]
    return np.ascontiguousarray(dec.transpose(0, 3, 1, 2, 4)).reshape(Rp, K)


def untile_codes_e2m3(buf: np.ndarray, R: int, K: int) -> np.ndarray:
    Rp = (R + 31) // 32 * 32
    blk = np.asarray(buf, np.uint8).reshape(-1)[: Rp * K * 3 // 4].reshape(Rp // 32, K // 64,
                                                                             1536)
    dec = untile_values_e2m3(blk, Rp, K)
    assert np.all(dec == np.round(dec)) and np.all(np.abs(dec) <= 7.5)
    return dec.astype(np.int8)


def untile_codes_e2m3_a8(buf: np.ndarray, R: int, K: int) -> np.ndarray:
    """3072-byte digit blocks -> 8-bit codes 32 * (h/2) + 2 * (l/2)."""
    Rp = (R + 31) // 32 * 32
    blk = np.asarray(buf, np.uint8).reshape(-1)[: Rp * K * 3 // 2].reshape(Rp // 32, K // 64,
                                                                             3072)
    h2 = untile_values_e2m3(np.ascontiguousarray(blk[..., :1536]), Rp, K)
    l2 = untile_values_e2m3(np.ascontiguousarray(blk[..., 1536:]), Rp, K)
    q = 32.0 * h2 + 2.0 * l2
    assert np.all(q == np.round(q)) and np.all(np.abs(q) <= 127)
    return q.astype(np.int8)
