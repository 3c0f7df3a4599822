"""Determinism and shape checks for the seeded input generator (CPU only)."""

import torch

import synth


def test_route_inputs_deterministic_and_valid():
    for cfg in synth.CONFIGS:
        ids, w = synth.route_inputs(cfg, T=min(cfg.T, 256))
        ids2, w2 = synth.route_inputs(cfg, T=min(cfg.T, 256))
        assert torch.equal(ids, ids2) and torch.equal(w, w2)
        assert ids.dtype == torch.int32 and w.dtype == torch.float32
        assert int(ids.min()) >= 0 and int(ids.max()) < cfg.E
        # k distinct experts per token
        s = torch.sort(ids, dim=1).values
        assert bool((s[:, 1:] != s[:, :-1]).all())
        assert torch.allclose(w.sum(1), torch.ones(w.shape[0]), atol=1e-6)


def test_zipf_is_skewed():
    cfg = synth.config_by_name("qwen3_skewed")
    ids, _ = synth.route_inputs(cfg, T=2048)
    c = torch.bincount(ids.flatten().long(), minlength=cfg.E)
    assert int(c[0]) > 20 * int(c[-1])


def test_weights_per_expert_seed():
    cfg = synth.config_by_name("tiny")
    w_all = synth.expert_weights(cfg, 128, 128)
    w_one = synth.expert_weights(cfg, 128, 128, experts=[2])
    assert torch.equal(w_all[2], w_one[0])
    assert w_all.dtype == torch.bfloat16
    assert 0.015 < float(w_all.float().std()) < 0.025
    a = synth.activations(cfg, 16, 256)
    assert torch.equal(a, synth.activations(cfg, 16, 256))
    assert not torch.equal(a, synth.activations(cfg, 16, 256, stream=synth.STREAM_ACT_DOWN))
