"""The seeded generators are deterministic and produce the stated shapes."""
import numpy as np

import synth


def test_copy_process_deterministic_in_range_and_repetitive():
    a = synth.copy_process(synth.rng_for(5, 0), 5000, 151936, 0.6, 8.0)
    b = synth.copy_process(synth.rng_for(5, 0), 5000, 151936, 0.6, 8.0)
    assert (a == b).all() and a.dtype == np.int32
    assert a.min() >= 0 and a.max() < 151936
    # copied spans make bigram repeats far more common than under Zipf alone
    bigrams = set(zip(a[:-1].tolist(), a[1:].tolist()))
    assert len(bigrams) < 0.75 * (len(a) - 1)


def test_streams_uniforms_and_positions():
    cfg = synth.config(1, steps=3)
    gt = synth.token_streams(cfg)
    assert gt.shape == (1, cfg.hist_len + 4 * 4)
    u = synth.uniforms(cfg, 0)
    assert u.shape == (1, 4) and u.dtype == np.float32
    assert ((u >= 0) & (u < 1)).all()
    n = np.array([cfg.hist_len])
    pos = synth.boost_positions(cfg, gt, n)
    assert pos.tolist() == [gt[0, cfg.hist_len:cfg.hist_len + 4].tolist()]
    m = synth.boost_mask(cfg, 0)
    assert m.shape == (1, 4) and m.dtype == bool


def test_target_logits_boost_and_bf16():
    import torch
    cfg = synth.config(4, B=2, V=1000, hist_len=50, steps=1)
    gt = synth.token_streams(cfg)
    n = np.array([50, 50])
    x = synth.target_logits(cfg, 0, gt, n)
    assert x.dtype == torch.bfloat16 and tuple(x.shape) == (2, 6, 1000)
    z = synth.noise(cfg, 0)
    pos = synth.boost_positions(cfg, gt, n)
    for b in range(2):
        for j in range(6):
            want = (z[b, j, pos[b, j]] + cfg.boost).to(torch.bfloat16)
            assert x[b, j, pos[b, j]] == want
