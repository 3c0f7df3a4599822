"""GPU weighted combine vs the oracle, bit for bit.

The path defines the combine's precision (reading A13): an fp32 fused
multiply-add per slot in slot order r = 0..k-1 from +0, then round to nearest
even to bf16.  oracle.combine_fp32 evaluates exactly that, so the GPU result
must equal it in every bit.  The float64 oracle.combine is checked as well,
with the bound the fp32 chain implies:
  |z - z_exact| <= ulp_bf16/2 + (k+1) * 2^-24 * sum_r |p_r y_r|.
"""

import json
import os

import numpy as np
import pytest
import torch

import int4_weights_amd as moe
import oracle
from gpu_helpers import DEV, bf16_from_u16, require_gpu, u16

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _bf16_ulp(x):
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _run(y_bits, oi, w):
    Y = bf16_from_u16(y_bits)
    T, k = oi.shape
    Z = torch.empty(T, y_bits.shape[1], dtype=torch.bfloat16, device=DEV)
    moe.moe_unpermute_combine(Y, torch.from_numpy(oi.astype(np.int32)).to(DEV),
                              torch.from_numpy(w.astype(np.float32)).to(DEV), Z)
    torch.cuda.synchronize()
    return u16(Z)


def _check(y_bits, oi, w, z_bits):
    assert np.array_equal(z_bits, oracle.combine_fp32(y_bits, oi, w.astype(np.float32)))
    z = oracle.bf16_bits_to_f64(z_bits)
    y = oracle.bf16_bits_to_f64(y_bits)
    ref = oracle.combine(y, oi, w.astype(np.float32).astype(np.float64))
    mag = oracle.combine(np.abs(y), oi, np.abs(w.astype(np.float32).astype(np.float64)))
    k = oi.shape[1]
    bound = 0.5 * _bf16_ulp(np.maximum(np.abs(ref), np.abs(z))) + (k + 1) * 2.0 ** -24 * mag
    assert (np.abs(z - ref) <= bound).all(), float(np.max(np.abs(z - ref) - bound))


def test_combine_worked_example():
    require_gpu()
    g = json.load(open(GOLDEN, encoding="utf-8"))
    ids = np.array(g["topk_ids"], np.int32)
    w = np.array(g["topk_weights"], np.float32)
    r = oracle.route(ids, 4, "contiguous", align=128)
    rng = np.random.default_rng(0)
    y = u16(torch.from_numpy(rng.standard_normal((r["rows_cap"], 64)).astype(np.float32)).to(torch.bfloat16))
    z = _run(y, r["output_index"], w)
    _check(y, r["output_index"], w, z)
    # the page's z_0 = 0.70 * y_packed[0] + 0.30 * y_packed[256]
    yf = oracle.bf16_bits_to_f64(y)
    z0 = np.float32(0.70) * yf[0] + np.float32(0.30) * yf[256]
    assert np.allclose(oracle.bf16_bits_to_f64(z[0]), z0, rtol=2 ** -7, atol=1e-6)


@pytest.mark.parametrize("T,k,N,rows", [(1, 1, 8, 1), (333, 8, 4096, 3000), (64, 2, 256, 512), (9, 5, 1032, 40),
                                        (50, 12, 136, 64), (7, 64, 16, 100)])
def test_combine_random_with_dropped_slots(T, k, N, rows):
    require_gpu()
    rng = np.random.default_rng(T + k + N)
    y = u16(torch.from_numpy(rng.standard_normal((rows, N)).astype(np.float32)).to(torch.bfloat16))
    oi = rng.integers(0, rows, size=(T, k)).astype(np.int32)
    oi[rng.random((T, k)) < 0.1] = -1
    oi[rng.random((T, k)) < 0.02] = rows + 5  # past the rows of Y: skipped like -1
    w = rng.random((T, k)).astype(np.float32)
    w[rng.random((T, k)) < 0.1] *= -1
    z = _run(y, oi, w)
    _check(y, oi, w, z)


def test_combine_halfway_accumulator():
    """Sums whose float64 value is an fp32 halfway point while the exact value is not."""
    require_gpu()
    import test_oracle_combine as pins

    cases = pins._halfway_cases()
    yb = oracle.f32_to_bf16_bits(np.array([[c[0]] * 8 for c in cases] + [[c[2]] * 8 for c in cases], np.float32))
    n = len(cases)
    oi = np.array([[i, n + i] for i in range(n)], np.int32)
    w = np.array([[1.0, c[1]] for c in cases], np.float32)
    _check(yb, oi, w, _run(yb, oi, w))


def test_combine_determinism_20_runs():
    require_gpu()
    rng = np.random.default_rng(5)
    y = u16(torch.from_numpy(rng.standard_normal((500, 512)).astype(np.float32)).to(torch.bfloat16))
    oi = rng.integers(0, 500, size=(100, 8)).astype(np.int32)
    w = rng.random((100, 8)).astype(np.float32)
    z = _run(y, oi, w)
    for _ in range(20):
        assert np.array_equal(_run(y, oi, w), z)


def test_combine_full_size_qwen3_routing_bit_exact():
    """The Qwen3-shaped combine (65536 routes into 8192 x 4096) on seeded rows, every bit of sampled tokens."""
    require_gpu()
    import synth

    cfg = synth.config_by_name("qwen3_skewed")
    ids, tw = synth.route_inputs(cfg)
    r = oracle.route(ids.numpy(), cfg.E, "contiguous", align=cfg.align)
    rows, N = r["rows_cap"], cfg.N_down
    Y = synth.activations(cfg, rows, N, stream=synth.STREAM_ACT_DOWN, device=DEV)
    T, k = r["output_index"].shape
    Z = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
    moe.moe_unpermute_combine(Y, torch.from_numpy(r["output_index"].astype(np.int32)).to(DEV), tw.to(DEV), Z)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([np.arange(0, T, 97), [T - 1]]))
    oi = r["output_index"][toks]
    used = np.unique(oi[oi >= 0])
    local = np.searchsorted(used, oi).astype(np.int32)
    local[oi < 0] = -1
    yb = u16(Y[torch.from_numpy(used).to(DEV)])
    want = oracle.combine_fp32(yb, local, tw.numpy()[toks])
    assert np.array_equal(u16(Z[torch.from_numpy(toks).to(DEV)]), want)
