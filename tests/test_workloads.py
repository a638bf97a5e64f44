"""The seeded input generators are deterministic and have the stated shapes."""
import numpy as np
import torch

import workloads as wl


def test_generators_are_seeded_and_shaped():
    w1 = wl.base_weight(wl.C1, 0)
    w2 = wl.base_weight(wl.C1, 0)
    assert w1.shape == (1024, 1024) and w1.dtype == torch.float32 and torch.equal(w1, w2)
    l1, l2 = wl.lora_factors(wl.C1, 0)
    assert l1.shape == (1024, 8) and l2.shape == (8, 1024) and l1.dtype == torch.bfloat16
    x = wl.activations(wl.C1, 0)
    assert x.shape == (16, 1024) and x.dtype == torch.bfloat16
    assert 0.9 < float(x.float().std()) < 1.1
    assert abs(float(w1.std()) - 0.02) < 1e-3


def test_outliers_and_heavy_blocks():
    w = wl.base_weight(wl.C2, 0).numpy()
    frac = np.mean(np.abs(w) > 0.02 * 6)
    assert 2e-4 < frac < 2e-3                     # ~0.1% entries scaled x10
    c = wl.codec_chunk_f32(64 * 4096, seed=3)
    assert c.dtype == np.float32 and c.size == 64 * 4096
    assert np.array_equal(c, wl.codec_chunk_f32(64 * 4096, seed=3))
