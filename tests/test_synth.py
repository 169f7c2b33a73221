"""The shared seeded input generator: Philox known answers and the weight/token laws."""
import numpy as np
import pytest
import torch

import synth
from golden_util import philox_kat


def test_philox_known_answers():
    for ctr, key, out in philox_kat():
        assert synth.philox4x32_10(ctr, key) == out


def test_weight_law_and_determinism():
    w = synth.weight_host((512, 1024), 7, "f64")
    assert abs(w.mean()) < 3 * 0.02 / np.sqrt(w.size)
    assert abs(w.std() - 0.02) < 0.02 * 5e-3
    # Irwin-Hall(12): support is +-6 sigma, kurtosis 3 - 1.2/12 = 2.9
    assert np.abs(w).max() <= 6 * 0.02
    kurt = np.mean((w / w.std()) ** 4)
    assert abs(kurt - 2.9) < 0.05
    w2 = synth.weight_host((512, 1024), 7, "f64")
    assert np.array_equal(w, w2)
    w3 = synth.weight_host((512, 1024), 8, "f64")
    assert not np.array_equal(w, w3)
    # an element range drawn on its own equals the same slice of the whole tensor
    part = synth.weight_host((1000,), 7, "f64", e0=12345)
    assert np.array_equal(part, w.reshape(-1)[12345:13345])


def test_weight_element_definition():
    """Element e is the documented Irwin-Hall sum of twelve 16-bit Philox halves."""
    seed, tid = 0x1234567890AB, 0xFFFF0001
    w = synth.weight_host((64,), tid, "f32", seed=seed)
    for e in (0, 1, 17, 63):
        a = synth.philox4x32_10([e, 0, tid, 0], [seed & 0xFFFFFFFF, seed >> 32])
        b = synth.philox4x32_10([e, 0, tid, 1], [seed & 0xFFFFFFFF, seed >> 32])
        s = sum((x & 0xFFFF) + (x >> 16) for x in a) + sum((x & 0xFFFF) + (x >> 16) for x in b[:2])
        expect = np.float32(s - 393210) * np.float32(np.float32(0.02) * np.float32(2.0 ** -16))
        assert w[e] == expect


def test_bf16_form_is_rne_of_f32():
    f = synth.weight_host((4096,), 3, "f32")
    b = synth.weight_host((4096,), 3, "bf16")
    t = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, t)
    d = synth.weight_host((4096,), 3, "f64", bf16=True)
    assert np.array_equal(d, (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64))


def test_tokens_uniform():
    V = 50
    t = synth.tokens_host(50000, 9, V)
    assert t.min() >= 0 and t.max() < V
    counts = np.bincount(t, minlength=V)
    chi2 = ((counts - 1000.0) ** 2 / 1000.0).sum()
    assert chi2 < 120      # 49 dof: p ~ 1e-7 at 120


def test_random_skip_layers():
    a = synth.random_skip_layers(40, 20, 2, 0)
    assert len(a) == 20 and len(set(a)) == 20 and all(0 <= x < 40 for x in a)
    assert a == synth.random_skip_layers(40, 20, 2, 0)
    assert a != synth.random_skip_layers(40, 20, 2, 1)


def test_norm_gain_law():
    """RMSNorm gains: float32 1 + w with w of the weight law at GAIN_STD; distinct per tensor id."""
    g = synth.norm_gain_host(4096, synth.layer_tid(3, synth.KIND_ATTN_NORM))
    assert g.dtype == np.float32
    w = synth.weight_host((4096,), synth.layer_tid(3, synth.KIND_ATTN_NORM), "f32", std=synth.GAIN_STD)
    assert np.array_equal(g, np.float32(1.0) + w)
    assert abs(float(g.mean()) - 1.0) < 4 * synth.GAIN_STD / 64
    assert abs(float(g.std()) - synth.GAIN_STD) < 0.01
    g2 = synth.norm_gain_host(4096, synth.layer_tid(3, synth.KIND_MLP_NORM))
    assert not np.array_equal(g, g2)


def test_scoring_masks_law():
    """Scoring candidates: k_c skipped layers with k_c in [lo, hi], both
    sub-layer bits of a skipped layer set, distinct seeded subsets, reproducible."""
    m = synth.scoring_masks(40, 16, 16, 24)
    assert m.shape == (16, 80) and m.dtype == np.uint8
    assert np.array_equal(m[:, 0::2], m[:, 1::2])
    k = m[:, 0::2].sum(axis=1)
    assert k.min() >= 16 and k.max() <= 24 and len(set(k.tolist())) > 1
    assert len({row.tobytes() for row in m}) == 16
    assert np.array_equal(m, synth.scoring_masks(40, 16, 16, 24))
