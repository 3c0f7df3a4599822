"""Pins of the test helper's fragment-packed weight orders (permutations of bytes)."""

import numpy as np
import pytest

import weight_layout as wl


@pytest.mark.parametrize("E,N,K", [(1, 128, 128), (2, 256, 384)])
def test_pack_matches_scalar_offsets_everywhere(E, N, K):
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 256, size=(E, N, K), dtype=np.uint8)
    packed = wl.pack_weight_fp8(codes)
    offs = np.array([[wl.packed_offset(n, k, N) for k in range(K)] for n in range(N)])
    # bijection onto [0, N*K)
    assert np.array_equal(np.sort(offs.reshape(-1)), np.arange(N * K))
    for e in range(E):
        assert np.array_equal(packed[e][offs], codes[e])


def test_unpack_inverts_pack_and_blocks_are_2kb_fragments():
    rng = np.random.default_rng(7)
    E, N, K = 1, 256, 256
    codes = rng.integers(0, 256, size=(E, N, K), dtype=np.uint8)
    packed = wl.pack_weight_fp8(codes)
    assert np.array_equal(wl.unpack_weight_fp8(packed, N, K), codes)
    # block (kb=1, cb=2): first 16 bytes are column 32, K 128..143; lane 17 is column 33, K 144..159
    base = (1 * (N // 16) + 2) * 2048
    assert np.array_equal(packed[0, base:base + 16], codes[0, 32, 128:144])
    assert np.array_equal(packed[0, base + 17 * 16:base + 18 * 16], codes[0, 33, 144:160])
    # second half: K 192..207 of column 32 at +1024
    assert np.array_equal(packed[0, base + 1024:base + 1040], codes[0, 32, 192:208])


def test_bf16_pack_round_trip_and_hand_placed_values():
    """bf16 weights: the 16-bit values of each 16-column x 64-value block form one 2 KB fragment."""
    rng = np.random.default_rng(8)
    E, N, K = 2, 256, 192
    w = rng.integers(0, 1 << 16, size=(E, N, K), dtype=np.uint16)
    packed = wl.pack_weight_bf16(w)
    assert packed.shape == (E, N * K) and packed.dtype == np.uint16
    assert np.array_equal(wl.unpack_weight_bf16(packed, N, K), w)
    assert np.array_equal(np.sort(packed[1]), np.sort(w[1].reshape(-1)))
    # block (K values 64..127, columns 32..47) starts at value (1 * 16 + 2) * 1024: column 32, K 64..71 first;
    # the 18th 8-value piece is column 33, K 72..79; the second half (+512 values) starts with column 32, K 96..103
    base = (1 * (N // 16) + 2) * 1024
    assert np.array_equal(packed[1, base:base + 8], w[1, 32, 64:72])
    assert np.array_equal(packed[1, base + 17 * 8:base + 18 * 8], w[1, 33, 72:80])
    assert np.array_equal(packed[1, base + 512:base + 520], w[1, 32, 96:104])


def _nib(q4, n, k):
    b = q4[n, k // 2]
    return (b >> 4) & 15 if k % 2 else b & 15


@pytest.mark.parametrize("E,N,K", [(1, 128, 128), (2, 256, 384)])
def test_int4_pack_matches_scalar_positions_everywhere(E, N, K):
    rng = np.random.default_rng(N * K)
    q4 = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    s16 = rng.integers(0, 65536, size=(E, N, K // 128), dtype=np.uint16)
    packed, sp = wl.pack_weight_int4(q4, s16)
    pos = np.array([[2 * o + h for o, h in (wl.packed_nibble_int4(n, k, N),)] for n in range(N) for k in range(K)])
    assert np.array_equal(np.sort(pos.reshape(-1)), np.arange(N * K))  # a bijection onto the nibbles
    for e in range(E):
        flat = np.empty(N * K, np.uint8)
        flat[0::2] = packed[e] & 15
        flat[1::2] = packed[e] >> 4
        want = np.array([_nib(q4[e], n, k) for n in range(N) for k in range(K)], np.uint8)
        assert np.array_equal(flat[pos.reshape(-1)], want)
        soff = np.array([[wl.packed_scale_offset_int4(n, g, N) for g in range(K // 128)] for n in range(N)])
        assert np.array_equal(np.sort(soff.reshape(-1)), np.arange(N * K // 128))
        assert np.array_equal(sp[e][soff], s16[e])
    assert np.array_equal(wl.unpack_weight_int4(packed, N, K), q4)


def test_int4_dword_holds_natural_pairs_after_shift_and_mask():
    """Column 37 of group 1 holds k = 128 + j with value j % 16; the packed dwords decode to natural pairs."""
    N, K = 128, 256
    q = np.zeros((N, K), np.uint8)
    q[37, :] = np.arange(K) % 16
    q4 = (q[:, 0::2] | (q[:, 1::2] << 4))[None]
    packed, _ = wl.pack_weight_int4(q4, np.zeros((1, N, 2), np.uint16))
    cb, c = divmod(37, 16)
    for h in range(4):
        for d in range(4):
            off = (1 * (N // 16) + cb) * 1024 + 16 * (c + 16 * h) + 4 * d
            w = int.from_bytes(packed[0, off:off + 4].tobytes(), "little")
            k0 = 128 + 8 * (4 * d + h)
            for i in range(4):
                lo, hi = (w >> (4 * i)) & 15, (w >> (4 * i + 16)) & 15
                assert (lo, hi) == ((k0 + 2 * i) % 16, (k0 + 2 * i + 1) % 16)
    # scales: column 37 is in 64-column slice 0, c = 5, cb = 2
    assert wl.packed_scale_offset_int4(37, 1, N) == ((1 * 2 + 0) * 16 + 5) * 4 + 2


@pytest.mark.parametrize("E,N,K", [(1, 128, 384), (2, 256, 1024)])
def test_fp4_pack_matches_scalar_offsets_everywhere(E, N, K):
    rng = np.random.default_rng(N + K + 1)
    w4 = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    sw = rng.integers(0, 255, size=(E, N, K // 32), dtype=np.uint8)
    codes, scales = wl.pack_weight_fp4(w4, sw)
    pos = np.array([[2 * o + h for o, h in (wl.packed_code_offset_fp4(n, k, N),)] for n in range(N) for k in range(K)])
    assert np.array_equal(np.sort(pos.reshape(-1)), np.arange(N * K))
    soff = np.array([[wl.packed_scale_offset_fp4(n, b, N) for b in range(K // 32)] for n in range(N)])
    assert np.array_equal(np.sort(soff.reshape(-1)), np.arange(N * K // 32))
    for e in range(E):
        flat = np.empty(N * K, np.uint8)
        flat[0::2] = codes[e] & 15
        flat[1::2] = codes[e] >> 4
        want = np.empty((N, K), np.uint8)
        want[:, 0::2] = w4[e] & 15
        want[:, 1::2] = w4[e] >> 4
        assert np.array_equal(flat[pos.reshape(-1)], want.reshape(-1))
        assert np.array_equal(scales[e][soff], sw[e])


def test_fp4_pack_hand_decoded_lane():
    """Lane L = 5 + 16*2 of block cb = 3 in step 1: column 53, K 128 + 64 .. 128 + 95; its scale dword in step 1,
    64-column group 0, holds block 4*1 + 2 of columns 5, 21, 37, 53."""
    N, K = 128, 512
    w4 = np.arange(N * K // 2, dtype=np.int64).reshape(1, N, K // 2).astype(np.uint8)
    sw = (np.arange(N * K // 32, dtype=np.int64).reshape(1, N, K // 32) % 251).astype(np.uint8)
    codes, scales = wl.pack_weight_fp4(w4, sw)
    L = 5 + 16 * 2
    off = ((1 * (N // 16) + 3) * 64 + L) * 16
    assert np.array_equal(codes[0, off:off + 16], w4[0, 53, 64 + 32:64 + 48])
    soff = ((1 * (N // 64) + 0) * 64 + L) * 4
    assert list(scales[0, soff:soff + 4]) == [int(sw[0, 5 + 16 * j, 4 * 1 + 2]) for j in range(4)]
