"""The seeded generators are deterministic and have the stated distributions."""
import numpy as np
import torch

import synth


def test_codes_and_scales_deterministic_and_uniform():
    c1 = synth.codes(synth.stream_key(1, 2, 3), 64, 4096)
    c2 = synth.codes(synth.stream_key(1, 2, 3), 64, 4096)
    assert torch.equal(c1, c2) and c1.shape == (64, 2048) and c1.dtype == torch.uint8
    nib = torch.cat([c1 & 0xF, c1 >> 4]).flatten().numpy()
    hist = np.bincount(nib, minlength=16)
    assert hist.min() > 0.9 * nib.size / 16 and hist.max() < 1.1 * nib.size / 16
    s = synth.scales(synth.stream_key(1, 2, 4), 256, 4096).numpy()
    assert s.min() == 119 and s.max() == 127
    assert not torch.equal(c1, synth.codes(synth.stream_key(1, 2, 4), 64, 4096))


def test_slices_regenerate():
    a = synth.hash_words(12345, 1000)
    b = synth.hash_words(12345, 100, start=900)
    assert torch.equal(a[900:], b)


def test_normal_and_hot_experts():
    x = synth.activations(4, 0, 512, 256)
    assert x.dtype == np.float32 and abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    hot = synth.hot_experts(3, 256, 16)
    assert len(set(hot.tolist())) == 16
    lg = synth.router_logits(3, 0, 4, 256, hot_bias=2.0)
    base = synth.router_logits(3, 0, 4, 256)
    assert np.allclose(lg[:, hot] - base[:, hot], 2.0)
