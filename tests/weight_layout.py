"""Fragment-packed orders of FP8 and 4-bit weight codes: a test helper.

These orders are the library's storage formats (moe_pack_weight_fp8 /
moe_pack_weight_int4), not part of the method the oracle computes: the oracle
always takes row-major weights.  The tests use this module to check the
library's packers byte for byte and to feed the GEMMs packed weights in small
cases; it is written from the layout definition in include/moe.h and imports
nothing from the library.

Weights are quantised once, offline, and may be stored in whatever order the
kernel reads fastest: ONNX Runtime's MatMulNBits page describes prepacked
weight layouts for its fpA_intB path (the ``weight_prepacked`` attribute), and
the DeepGEMM article ("补偿机制三") transforms weight scales once and reuses
them.  The packed order here is a permutation of the row-major codes
[E, N, K]; it carries exactly the same values.

Definition (per expert, N and K multiples of 128): the 16 x 128 block of
columns 16cb .. 16cb+15 and K values 128kb .. 128kb+127 is stored as 2048
contiguous bytes at ((kb * (N/16) + cb) * 2048); inside it, byte j of the
16-byte piece for column 16cb + c and K offset 64h + 16g + j sits at
h*1024 + (c + 16g)*16 + j.

4-bit weights (MatMulNBits order [E, N, K/2], two weights per byte, low
nibble first) are packed at the level of single weights.  For expert e, K group
g (128 weights), 16-column block cb, lane L = c + 16h (c < 16, h < 4), dword
d < 4 and nibble position p < 8 (bits 4p..4p+3 of the little-endian dword):
    column 16cb + c, k = 128g + 8(4d + h) + sigma(p),  sigma = (0 2 4 6 1 3 5 7)
sits at byte (g*(N/16) + cb)*1024 + 16L + 4d + p//2, nibble p % 2.  Each
dword then holds 8 consecutive k of one column with k and k+1 at nibbles i and
i+4, so shifting by 4i and masking both 16-bit halves yields the pair
(k + 2i, k + 2i + 1) in natural order.
The group scales [E, N, K/128] are packed to [E, K/128, N/64, 16, 4]: scale
(n, g) sits at ((g*(N/64) + n//64)*16 + n%16)*4 + (n%64)//16.
"""

from __future__ import annotations

import numpy as np


def packed_offset(n: int, k: int, N: int) -> int:
    """Byte offset (within one expert) of row-major element (n, k) in the packed order.

    Pinned by: bijection over every (n, k) of small shapes (tests)."""
    kb, kk = divmod(k, 128)
    h, rest = divmod(kk, 64)
    g, j = divmod(rest, 16)
    cb, c = divmod(n, 16)
    return ((kb * (N // 16) + cb) * 2 + h) * 1024 + (c + 16 * g) * 16 + j


def pack_weight_fp8(codes: np.ndarray) -> np.ndarray:
    """uint8 [E, N, K] row-major -> uint8 [E, N*K] in the packed order (a pure permutation).

    Pinned by: equality with packed_offset element by element (tests)."""
    codes = np.asarray(codes, dtype=np.uint8)
    E, N, K = codes.shape
    if N % 128 or K % 128:
        raise ValueError("N and K must be multiples of 128")
    # axes: e, cb, c, kb, h, g, j  ->  e, kb, cb, h, g, c, j
    x = codes.reshape(E, N // 16, 16, K // 128, 2, 4, 16)
    return np.ascontiguousarray(x.transpose(0, 3, 1, 4, 5, 2, 6)).reshape(E, N * K)


def unpack_weight_fp8(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Inverse of pack_weight_fp8: uint8 [E, N*K] -> [E, N, K]."""
    packed = np.asarray(packed, dtype=np.uint8)
    E = packed.shape[0]
    x = packed.reshape(E, K // 128, N // 16, 2, 4, 16, 16)  # e, kb, cb, h, g, c, j
    return np.ascontiguousarray(x.transpose(0, 2, 5, 1, 3, 4, 6)).reshape(E, N, K)


def pack_weight_bf16(w_bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns uint16 [E, N, K] -> uint16 [E, N*K]: the weight bytes, viewed as uint8 [E, N, 2K]
    (little-endian), in pack_weight_fp8's order with 2K bytes per row (moe_pack_weight_bf16).

    Pinned by: the inverse round trip and one-hot positions (tests)."""
    w_bits = np.ascontiguousarray(np.asarray(w_bits, dtype="<u2"))
    E, N, K = w_bits.shape
    if N % 128 or K % 64:
        raise ValueError("N must be a multiple of 128 and 2K of 128")
    return pack_weight_fp8(w_bits.view(np.uint8).reshape(E, N, 2 * K)).view("<u2").reshape(E, N * K)


def unpack_weight_bf16(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Inverse of pack_weight_bf16: uint16 [E, N*K] -> [E, N, K]."""
    packed = np.ascontiguousarray(np.asarray(packed, dtype="<u2"))
    E = packed.shape[0]
    return unpack_weight_fp8(packed.view(np.uint8).reshape(E, 2 * N * K), N, 2 * K).view("<u2").reshape(E, N, K)


SIGMA = (0, 2, 4, 6, 1, 3, 5, 7)


def packed_nibble_int4(n: int, k: int, N: int) -> tuple[int, int]:
    """(byte offset within one expert, nibble 0 = low / 1 = high) of weight (n, k) in the packed order.

    Pinned by: bijection over every (n, k) of small shapes and hand-decoded dwords (tests)."""
    g, kk = divmod(k, 128)
    chunk, j = divmod(kk, 8)
    d, h = divmod(chunk, 4)
    p = SIGMA.index(j)
    cb, c = divmod(n, 16)
    L = c + 16 * h
    return (g * (N // 16) + cb) * 1024 + 16 * L + 4 * d + p // 2, p % 2


def packed_scale_offset_int4(n: int, g: int, N: int) -> int:
    """Element offset (within one expert) of the scale of column n, group g, in the packed scale order."""
    return ((g * (N // 64) + n // 64) * 16 + n % 16) * 4 + (n % 64) // 16


def _nibbles(q4: np.ndarray) -> np.ndarray:
    """uint8 [..., B] -> the 2B 4-bit values, low nibble first."""
    out = np.empty(q4.shape[:-1] + (2 * q4.shape[-1],), np.uint8)
    out[..., 0::2] = q4 & 15
    out[..., 1::2] = q4 >> 4
    return out


def pack_weight_int4(q4: np.ndarray, s16: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """MatMulNBits codes uint8 [E, N, K/2] and scales uint16 [E, N, K/128] -> the packed orders
    (uint8 [E, N*K/2], uint16 [E, N*K/128]); a permutation of weights and of scales."""
    q4 = np.asarray(q4, dtype=np.uint8)
    s16 = np.asarray(s16, dtype=np.uint16)
    E, N, K2 = q4.shape
    K = 2 * K2
    if N % 128 or K % 128:
        raise ValueError("N and K must be multiples of 128")
    w = _nibbles(q4)  # [E, N, K]
    # k = 128g + 8(4d + h) + sigma(p); n = 16cb + c
    x = w.reshape(E, N // 16, 16, K // 128, 4, 4, 8)       # e, cb, c, g, d, h, j
    x = x[..., list(SIGMA)]                               # j -> nibble position p
    x = x.transpose(0, 3, 1, 5, 2, 4, 6)                  # e, g, cb, h, c, d, p  (L = c + 16h)
    x = np.ascontiguousarray(x).reshape(E, N * K // 8, 8)  # dwords of 8 nibbles
    packed = np.zeros((E, N * K // 8, 4), np.uint8)
    for b in range(4):
        packed[..., b] = x[..., 2 * b] | (x[..., 2 * b + 1] << 4)
    sp = s16.reshape(E, N // 64, 4, 16, K // 128)         # e, n64, cb, c, g
    sp = np.ascontiguousarray(sp.transpose(0, 4, 1, 3, 2)).reshape(E, N * K // 128)
    return packed.reshape(E, N * K // 2), sp


def unpack_weight_int4(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Inverse of the weight half of pack_weight_int4: uint8 [E, N*K/2] -> [E, N, K/2]."""
    packed = np.asarray(packed, dtype=np.uint8)
    E = packed.shape[0]
    by = packed.reshape(E, N * K // 8, 4)
    x = np.empty((E, N * K // 8, 8), np.uint8)
    for b in range(4):
        x[..., 2 * b] = by[..., b] & 15
        x[..., 2 * b + 1] = by[..., b] >> 4
    x = x.reshape(E, K // 128, N // 16, 4, 16, 4, 8)      # e, g, cb, h, c, d, p
    inv = [SIGMA.index(j) for j in range(8)]
    x = x[..., inv]                                       # p -> j
    w = x.transpose(0, 2, 4, 1, 5, 3, 6).reshape(E, N, K)  # e, cb, c, g, d, h, j
    return (w[..., 0::2] | (w[..., 1::2] << 4)).astype(np.uint8)


# ------------------------------------------------------------------------------------------------ MXFP4 --
# moe_pack_weight_fp4 (include/moe.h): codes [E, N, K/2] and E8M0 scales [E, N, K/32] are permuted so that, per
# step ks of 128 K values and 16-column block cb, lane L = c + 16g (c < 16, g < 4) finds its 16 bytes of codes
# (column 16cb + c, K 128ks + 32g .. +31) at ((ks*(N/16) + cb)*64 + L)*16, and per step and 64-column group n64
# one dword at ((ks*(N/64) + n64)*64 + L)*4 whose byte j is the scale of column 64 n64 + 16 j + c, block 4 ks + g.


def pack_weight_fp4(w4: np.ndarray, sw: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """uint8 codes [E, N, K/2] and scales [E, N, K/32] -> packed orders (uint8 [E, N*K/2], uint8 [E, N*K/32])."""
    w4 = np.asarray(w4, dtype=np.uint8)
    sw = np.asarray(sw, dtype=np.uint8)
    E, N, K2 = w4.shape
    K = 2 * K2
    if N % 128 or K % 128:
        raise ValueError("N and K must be multiples of 128")
    # codes: axes e, cb, c, ks, g, bytes(16) -> e, ks, cb, g, c, bytes
    x = w4.reshape(E, N // 16, 16, K // 128, 4, 16)
    codes = np.ascontiguousarray(x.transpose(0, 3, 1, 4, 2, 5)).reshape(E, N * K2)
    # scales: n = 64 n64 + 16 j + c, block b = 4 ks + g: axes e, n64, j, c, ks, g -> e, ks, n64, g, c, j
    y = sw.reshape(E, N // 64, 4, 16, K // 128, 4)
    scales = np.ascontiguousarray(y.transpose(0, 4, 1, 5, 3, 2)).reshape(E, N * K // 32)
    return codes, scales


def packed_code_offset_fp4(n: int, k: int, N: int) -> tuple[int, int]:
    """(byte offset within one expert, nibble 0 = low) of the code of weight (n, k) in the packed order."""
    ks, kk = divmod(k, 128)
    g, j = divmod(kk, 32)
    cb, c = divmod(n, 16)
    return ((ks * (N // 16) + cb) * 64 + c + 16 * g) * 16 + j // 2, j % 2


def packed_scale_offset_fp4(n: int, b: int, N: int) -> int:
    """Byte offset (within one expert) of the scale of column n, 32-value block b, in the packed order."""
    ks, g = divmod(b, 4)
    n64, r = divmod(n, 64)
    j, c = divmod(r, 16)
    return ((ks * (N // 64) + n64) * 64 + c + 16 * g) * 4 + j
