"""GPU quantisers vs the oracle, bit-exact (codes and scales)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (DEV, bf16_from_u16, fp8_quant_gpu, fp8_quant_weight_gpu, int4_quant_weight_gpu,
                         require_gpu, u16)

pytestmark = pytest.mark.gpu


def _exhaustive_rows():
    """Every finite bf16 with |x| <= 448, 127 per row next to 448 (so the scale is 1)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_bits_to_f64(bits)
    keep = bits[np.isfinite(v) & (np.abs(v) <= 448.0)]
    n = -(-keep.size // 127) * 127
    keep = np.concatenate([keep, np.zeros(n - keep.size, np.uint16)]).reshape(-1, 127)
    top = np.full((keep.shape[0], 1), 0x43E0, np.uint16)  # 448.0
    return np.concatenate([top, keep], axis=1)


def _edge_rows(rng):
    rows = []
    K = 384
    rows.append(np.zeros(K, np.uint16))                                # all zero -> scale 1
    r = np.zeros(K, np.uint16); r[5] = 0x8000; rows.append(r)         # -0
    r = np.full(K, 0x0001, np.uint16); rows.append(r)                  # bf16 subnormals only
    r = rng.integers(0, 0x0080, K).astype(np.uint16) | 0x8000; rows.append(r)  # negative subnormals
    r = np.full(K, 0x7F7F, np.uint16); rows.append(r)                  # bf16 max
    r = np.full(K, 0x43E0, np.uint16); r[7] = 0x43E1; rows.append(r)   # 448 and just above
    x = (rng.standard_normal((12, K)) * np.exp(rng.uniform(-30, 30, (12, 1)))).astype(np.float32)
    for row in x:
        rows.append(u16(torch.from_numpy(row).to(torch.bfloat16)))
    return np.stack(rows)


def test_quant_act_bit_exact_exhaustive_and_edges():
    require_gpu()
    rng = np.random.default_rng(11)
    for bits in (_exhaustive_rows(), _edge_rows(rng)):
        x = bf16_from_u16(bits)
        q, sf = fp8_quant_gpu(x)
        rq, rsf = oracle.quant_act(bits)
        assert np.array_equal(q.cpu().numpy(), rq)
        assert np.array_equal(sf.cpu().numpy().view(np.uint32), rsf.view(np.uint32))


def test_quant_act_random_ragged_rows_and_determinism():
    require_gpu()
    torch.manual_seed(3)
    x = (torch.randn(77, 1152) * torch.exp(torch.randn(77, 1) * 4)).to(torch.bfloat16)
    bits = u16(x)
    xg = x.to(DEV)
    q, sf = fp8_quant_gpu(xg)
    rq, rsf = oracle.quant_act(bits)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(sf.cpu().numpy(), rsf)
    for _ in range(20):
        q2, sf2 = fp8_quant_gpu(xg)
        assert torch.equal(q, q2) and torch.equal(sf, sf2)


def test_quant_weight_fp8_bit_exact():
    require_gpu()
    torch.manual_seed(4)
    w = (torch.randn(3, 384, 512) * 0.02).to(torch.bfloat16)
    w[1, 128:256, 128:256] *= 1000
    w[2, :128, :128] = 0
    q, sfw = fp8_quant_weight_gpu(w.to(DEV))
    rq, rsfw = oracle.quant_weight_fp8(u16(w))
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(sfw.cpu().numpy(), rsfw)


def test_quant_weight_int4_bit_exact():
    require_gpu()
    torch.manual_seed(5)
    w = (torch.randn(3, 136, 512) * 0.02).to(torch.bfloat16)
    w[0, 7, :128] = 0
    w[1, 3, 128:256] *= 1e-30          # fp16 scale underflow path
    w[2, 9, 256:384] = 3e38            # fp16 scale overflow path
    q4, s16 = int4_quant_weight_gpu(w.to(DEV))
    rq4, rs16 = oracle.quant_weight_int4(u16(w))
    assert np.array_equal(q4.cpu().numpy(), rq4)
    assert np.array_equal(u16(s16), rs16)
