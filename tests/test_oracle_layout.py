"""Pins of the oracle's fragment-packed weight order (a permutation of bytes)."""

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("E,N,K", [(1, 128, 128), (2, 256, 384)])
def test_pack_matches_scalar_offsets_everywhere(E, N, K):
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 256, size=(E, N, K), dtype=np.uint8)
    packed = oracle.pack_weight_fp8(codes)
    offs = np.array([[oracle.packed_offset(n, k, N) for k in range(K)] for n in range(N)])
    # bijection onto [0, N*K)
    assert np.array_equal(np.sort(offs.reshape(-1)), np.arange(N * K))
    for e in range(E):
        assert np.array_equal(packed[e][offs], codes[e])


def test_unpack_inverts_pack_and_blocks_are_2kb_fragments():
    rng = np.random.default_rng(7)
    E, N, K = 1, 256, 256
    codes = rng.integers(0, 256, size=(E, N, K), dtype=np.uint8)
    packed = oracle.pack_weight_fp8(codes)
    assert np.array_equal(oracle.unpack_weight_fp8(packed, N, K), codes)
    # block (kb=1, cb=2): first 16 bytes are column 32, K 128..143; lane 17 is column 33, K 144..159
    base = (1 * (N // 16) + 2) * 2048
    assert np.array_equal(packed[0, base:base + 16], codes[0, 32, 128:144])
    assert np.array_equal(packed[0, base + 17 * 16:base + 18 * 16], codes[0, 33, 144:160])
    # second half: K 192..207 of column 32 at +1024
    assert np.array_equal(packed[0, base + 1024:base + 1040], codes[0, 32, 192:208])


@pytest.mark.parametrize("E,N,K", [(1, 128, 128), (2, 256, 384)])
def test_int4_pack_matches_scalar_offsets_everywhere(E, N, K):
    rng = np.random.default_rng(N * K)
    q4 = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    packed = oracle.pack_weight_int4(q4)
    offs = np.array([[oracle.packed_offset_int4(n, b, N) for b in range(K // 2)] for n in range(N)])
    assert np.array_equal(np.sort(offs.reshape(-1)), np.arange(N * K // 2))
    for e in range(E):
        assert np.array_equal(packed[e][offs], q4[e])
    assert np.array_equal(oracle.unpack_weight_int4(packed, N, K), q4)


def test_int4_blocks_are_1kb_group_fragments():
    rng = np.random.default_rng(11)
    E, N, K = 1, 256, 384
    q4 = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    packed = oracle.pack_weight_int4(q4)
    # group 2 (bytes 128..191 of each column), columns 48..63 (cb = 3)
    base = (2 * (N // 16) + 3) * 1024
    assert np.array_equal(packed[0, base:base + 16], q4[0, 48, 128:144])            # lane 0
    assert np.array_equal(packed[0, base + 5 * 16:base + 6 * 16], q4[0, 53, 128:144])  # lane 5
    assert np.array_equal(packed[0, base + 21 * 16:base + 22 * 16], q4[0, 53, 144:160])  # lane 21: piece 1
    assert np.array_equal(packed[0, base + 63 * 16:base + 64 * 16], q4[0, 63, 176:192])  # lane 63: piece 3
