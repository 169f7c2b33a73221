"""Pins of the oracle's elementary numerics against closed forms and library routines."""
import numpy as np
import torch

from golden_util import philox_kat
from oracle import philox
from oracle.numerics import bf16_round, rmsnorm, rope, rope_angles, silu, softmax


def test_oracle_philox_known_answers():
    for ctr, key, out in philox_kat():
        got = philox.philox4x32_10(*[np.uint32(c) for c in ctr], key[0], key[1])
        assert [int(x) for x in got] == out


def test_philox_addressing():
    """words(seed, it, row, purpose, n): block v//4, word v%4 of counter (it, row, purpose, v//4)."""
    seed = (7 << 32) | 11
    w = philox.words(seed, 5, 2, 1, 10)
    for v in range(10):
        blk = philox.philox4x32_10(np.uint32(5), np.uint32(2), np.uint32(1), np.uint32(v // 4), 11, 7)
        assert int(w[v]) == int(blk[v % 4])


def test_uniform_grid():
    u = philox.uniforms(3, 1, 0, 2, 100000)
    assert u.dtype == np.float32
    assert u.min() > 0 and u.max() < 1
    k = u.astype(np.float64) * 2 ** 24
    assert np.all(k == np.round(k)) and np.all(k.astype(np.int64) % 2 == 1)
    assert abs(u.mean() - 0.5) < 0.005


def _torch_bf16(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    assert np.array_equal(bf16_round(x.astype(np.float64)), _torch_bf16(x))


def test_bf16_round_ties_and_edges():
    # exact halfway points between consecutive bf16 values: ties go to the even mantissa
    base = np.array([1.0, 1.5, -3.0, 1e-3, 7e30], np.float32)
    bits = base.view(np.uint32)
    ties = ((bits & 0xFFFF0000) | 0x8000).view(np.float32)
    ties_odd = (((bits & 0xFFFF0000) + 0x10000) | 0x8000).view(np.float32)
    for t in (ties, ties_odd):
        assert np.array_equal(bf16_round(t.astype(np.float64)), _torch_bf16(t))
    sub = np.array([1e-40, -3e-39, 5e-45], np.float32)       # float32 subnormals
    assert np.array_equal(bf16_round(sub.astype(np.float64)), _torch_bf16(sub))
    big = np.array([3.3e38, 3.39e38, -3.4e38], np.float32)
    assert np.array_equal(bf16_round(big.astype(np.float64)), _torch_bf16(big))


def test_rope_relative_position_and_norm():
    """<R(p)q, R(p')k> depends only on p - p'; rotations keep norms."""
    rng = np.random.default_rng(1)
    hd = 64
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))
    def dot(pq, pk):
        return float(np.sum(rope(q, [pq], 1e4) * rope(k, [pk], 1e4)))
    assert abs(dot(10, 3) - dot(107, 100)) < 1e-10
    assert abs(dot(0, 0) - float(np.sum(q * k))) < 1e-12
    assert abs(np.linalg.norm(rope(q, [12345], 1e4)) - np.linalg.norm(q)) < 1e-10


def test_rope_is_complex_rotation():
    """Rotate-half pairing == multiplying (x_i + i x_{i+hd/2}) by exp(i * pos * theta^(-2i/hd))."""
    rng = np.random.default_rng(2)
    hd = 32
    x = rng.standard_normal((3, 2, hd))
    pos = [0, 5, 77]
    z = x[..., : hd // 2] + 1j * x[..., hd // 2:]
    ang = np.array([[p * 10000.0 ** (-2.0 * i / hd) for i in range(hd // 2)] for p in pos])
    zr = z * np.exp(1j * ang)[:, None, :]
    ref = np.concatenate([zr.real, zr.imag], axis=-1)
    assert np.allclose(rope(x, pos, 10000.0), ref, atol=1e-12)
    assert rope_angles([3], 8, 10000.0).shape == (1, 4)


def test_softmax_rmsnorm_silu():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((5, 1000)) * 10
    p = softmax(z)
    assert np.allclose(p.sum(-1), 1, atol=1e-12) and np.all(p >= 0)
    assert np.allclose(p, torch.softmax(torch.from_numpy(z), -1).numpy(), atol=1e-14)
    h = rng.standard_normal((4, 256)) * 3
    y = rmsnorm(h, np.ones(256), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, -1)), 1, atol=1e-12)
    assert np.allclose(rmsnorm(5 * h, np.ones(256), 0.0), y, atol=1e-12)
    assert np.allclose(silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(), atol=1e-12)
