"""Fragment-packed orders of FP8 and 4-bit weight codes.  TEST INFRASTRUCTURE ONLY.

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

4-bit weights (MatMulNBits order [E, N, K/2], two weights per byte): the 64
bytes of column 16cb + c in K group g (one quantisation group of 128 weights)
are four 16-byte pieces h = 0..3; the 16 columns' pieces of group g form 1024
contiguous bytes at (g * (N/16) + cb) * 1024, piece h of column c at
(c + 16h) * 16.
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


def packed_offset_int4(n: int, b: int, N: int) -> int:
    """Byte offset (within one expert) of byte b of column n (MatMulNBits order) in the packed order.

    Pinned by: bijection over every (n, b) of small shapes (tests)."""
    g, rest = divmod(b, 64)
    h, j = divmod(rest, 16)
    cb, c = divmod(n, 16)
    return (g * (N // 16) + cb) * 1024 + (c + 16 * h) * 16 + j


def pack_weight_int4(q4: np.ndarray) -> np.ndarray:
    """uint8 [E, N, K/2] MatMulNBits bytes -> uint8 [E, N*K/2] in the packed order (a pure permutation)."""
    q4 = np.asarray(q4, dtype=np.uint8)
    E, N, K2 = q4.shape
    if N % 128 or (2 * K2) % 128:
        raise ValueError("N and K must be multiples of 128")
    # axes: e, cb, c, g, h, j  ->  e, g, cb, h, c, j
    x = q4.reshape(E, N // 16, 16, K2 // 64, 4, 16)
    return np.ascontiguousarray(x.transpose(0, 3, 1, 4, 2, 5)).reshape(E, N * K2)


def unpack_weight_int4(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Inverse of pack_weight_int4: uint8 [E, N*K/2] -> [E, N, K/2]."""
    packed = np.asarray(packed, dtype=np.uint8)
    E = packed.shape[0]
    x = packed.reshape(E, K // 128, N // 16, 4, 16, 16)  # e, g, cb, h, c, j
    return np.ascontiguousarray(x.transpose(0, 2, 4, 1, 3, 5)).reshape(E, N, K // 2)
