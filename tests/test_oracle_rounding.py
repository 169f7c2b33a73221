"""Pins of the oracle's bf16 rounding points, one by one.

The bf16 workloads store bf16 values at six kinds of points: the normalised
input of every projection (after the RMSNorm gain), the rotated q and k, v, the
attention output entering Wo and the SwiGLU product entering Wdown.  Each test
below takes the oracle's traced tensors and rebuilds every rounding point from
its traced inputs with torch routines (``rms_norm``, ``silu``,
``scaled_dot_product_attention``, complex rotation, the float32 -> bfloat16
conversion), sharing no code with ``oracle/``.  A dropped, moved or extra
rounding makes one of these comparisons fail; the planted-mistake tests show
that they do.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import model as mdl
from oracle import numerics
from oracle import ssd

# GQA (4 query heads over 2 KV heads), head_dim 32, three layers, a ragged vocabulary
SHAPE = synth.ModelShape("bf16-round", 3, 128, 4, 2, 32, 160, 300, "bf16")
N_TOK = 9


def tbf16(a):
    """torch's RNE conversion to bfloat16 (through float32, exact for these magnitudes), back to float64."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def T(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def rope_complex(x, positions, theta):
    """Rotate-half RoPE as a complex product: (x_i + i x_{i+hd/2}) * exp(i pos theta^(-2i/hd))."""
    x = T(x)
    hd = x.shape[-1]
    inv = theta ** (-2.0 * torch.arange(hd // 2, dtype=torch.float64) / hd)
    ang = torch.tensor(positions, dtype=torch.float64)[:, None] * inv[None, :]
    z = torch.complex(x[..., : hd // 2], x[..., hd // 2:]) * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.cat([z.real, z.imag], dim=-1).numpy()


def traced_forward(m, toks):
    rec = {}

    def trace(name, l, v):
        rec[(name, l)] = np.array(v, copy=True)

    kv = mdl.KVCache(m.shape, N_TOK + 1)
    z = mdl.forward(m, toks, range(len(toks)), kv, trace=trace)
    return z, rec, kv


def check_rounding_points(m, toks):
    """Rebuild every traced rounding point from its traced inputs; raise AssertionError on a mismatch."""
    s = m.shape
    z, rec, kv = traced_forward(m, toks)
    pos = list(range(len(toks)))
    eps = s.rms_eps
    H, KVH, hd = s.n_heads, s.n_kv_heads, s.head_dim
    M = len(toks)
    h = m.embed[np.asarray(toks)].astype(np.float64)
    for l, lw in enumerate(m.layers):
        # attention sub-layer
        assert np.array_equal(rec[("h_attn", l)], h), f"layer {l}: residual entering attention"
        x = tbf16(F.rms_norm(T(h), (s.d_model,), T(lw.attn_norm), eps).numpy())
        assert np.array_equal(rec[("x_attn", l)], x), f"layer {l}: attention input"
        xt = T(x)
        q = tbf16(rope_complex((xt @ T(lw.wq).T).numpy().reshape(M, H, hd), pos, s.rope_theta))
        k = tbf16(rope_complex((xt @ T(lw.wk).T).numpy().reshape(M, KVH, hd), pos, s.rope_theta))
        v = tbf16((xt @ T(lw.wv).T).numpy().reshape(M, KVH, hd))
        assert np.array_equal(rec[("q", l)], q), f"layer {l}: rotated q"
        assert np.array_equal(rec[("k", l)], k), f"layer {l}: rotated k"
        assert np.array_equal(rec[("v", l)], v), f"layer {l}: v"
        assert np.array_equal(kv.K[l, :M], k) and np.array_equal(kv.V[l, :M], v), f"layer {l}: cache"
        # causal attention, query head j on KV head j // (H / KVH)
        qt = T(q).permute(1, 0, 2)[None]                      # [1, H, M, hd]
        kt = T(k).permute(1, 0, 2)[None].repeat_interleave(H // KVH, dim=1)
        vt = T(v).permute(1, 0, 2)[None].repeat_interleave(H // KVH, dim=1)
        o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)[0].permute(1, 0, 2).reshape(M, H * hd)
        o = tbf16(o.numpy())
        assert np.array_equal(rec[("o", l)], o), f"layer {l}: attention output"
        h = (T(h) + T(o) @ T(lw.wo).T).numpy()
        # MLP sub-layer
        assert np.allclose(rec[("h_mlp", l)], h, rtol=0, atol=1e-12), f"layer {l}: residual entering the MLP"
        h = rec[("h_mlp", l)]
        x = tbf16(F.rms_norm(T(h), (s.d_model,), T(lw.mlp_norm), eps).numpy())
        assert np.array_equal(rec[("x_mlp", l)], x), f"layer {l}: MLP input"
        xt = T(x)
        a = tbf16((F.silu(xt @ T(lw.wgate).T) * (xt @ T(lw.wup).T)).numpy())
        assert np.array_equal(rec[("a", l)], a), f"layer {l}: SwiGLU product"
        h = (T(h) + T(a) @ T(lw.wdown).T).numpy()
        nxt = ("h_attn", l + 1) if l + 1 < m.L else ("h_final", m.L)
        assert np.allclose(rec[nxt], h, rtol=0, atol=1e-12), f"layer {l}: residual leaving the layer"
        h = rec[nxt]
    x = tbf16(F.rms_norm(T(h), (s.d_model,), T(m.final_norm), eps).numpy())
    assert np.array_equal(rec[("x_final", m.L)], x), "final norm input of the LM head"
    assert np.allclose(z, (T(x) @ T(m.lm_head).T).numpy(), rtol=0, atol=1e-12), "LM head"
    return rec


@pytest.fixture(scope="module")
def model():
    return mdl.Model.synthetic(SHAPE)


@pytest.fixture(scope="module")
def toks():
    return synth.prompt_tokens(N_TOK, SHAPE.vocab)


def test_every_rounding_point_matches_torch(model, toks):
    rec = check_rounding_points(model, toks)
    # every rounding point holds bf16 values, and the rounding is not vacuous: the unrounded values are not
    for name in ("x_attn", "q", "k", "v", "o", "x_mlp", "a", "x_final"):
        for (nm, l), v in rec.items():
            if nm == name:
                assert np.array_equal(numerics.bf16_round(v), v)
    assert not np.array_equal(rec[("h_mlp", 0)], numerics.bf16_round(rec[("h_mlp", 0)]))


# ----------------------------------------------------------------- planted mistakes in the oracle
# Each variant drops or moves one rounding point; the pin above must reject every one.


def _drop_nth_rounding(monkeypatch, n):
    """Model.rnd becomes the identity on its n-th call of each forward (calls counted from 0)."""
    real = mdl.Model.rnd
    count = {"i": 0}

    def rnd(self, x):
        i = count["i"]
        count["i"] += 1
        return x if i == n else real(self, x)

    monkeypatch.setattr(mdl.Model, "rnd", rnd)
    return count


# the rounding calls of one forward in order: layer 0 x_attn, q, k, v, o, x_mlp, a, layer 1 ..., x_final
CALLS_PER_LAYER = 7


@pytest.mark.parametrize("which", ["x_attn", "q", "k", "v", "o", "x_mlp", "a", "x_final"])
def test_dropped_rounding_point_fails_the_pin(model, toks, monkeypatch, which):
    order = ["x_attn", "q", "k", "v", "o", "x_mlp", "a"]
    n = SHAPE.n_layers * CALLS_PER_LAYER if which == "x_final" else CALLS_PER_LAYER + order.index(which)
    _drop_nth_rounding(monkeypatch, n)
    with pytest.raises(AssertionError):
        check_rounding_points(model, toks)


def test_gain_rounded_before_the_norm_fails_the_pin(model, toks, monkeypatch):
    """The rounding placed on h * gain with 1/rms applied after the projection (the form of a kernel that
    scales its products) is a different function: the pin rejects it."""

    def norm_input(m, h, gain):
        return m.rnd(h * gain) / numerics.rms(h, m.shape.rms_eps)

    monkeypatch.setattr(mdl, "norm_input", norm_input)
    with pytest.raises(AssertionError):
        check_rounding_points(model, toks)


# ----------------------------------------------------------------- confidence at T > 0


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_confidence_uses_the_temperature(T):
    """conf = max softmax(z / T): logits (c, c + T ln 3) give (1/4, 3/4) at any c; a row with logit
    gaps g gives 1 / (1 + sum exp(-g / T))."""
    c = 1.7
    z = np.array([c, c + T * np.log(3.0)])
    assert abs(ssd.confidence(z, T) - 0.75) < 1e-12
    z3 = np.array([0.0, -1.0, -2.5, 3.0])
    gaps = 3.0 - z3[[0, 1, 2]]
    assert abs(ssd.confidence(z3, T) - 1.0 / (1.0 + np.exp(-gaps / T).sum())) < 1e-12


def test_confidence_greedy_uses_unit_temperature():
    z = np.array([0.0, np.log(3.0)])
    assert abs(ssd.confidence(z, 0.0) - 0.75) < 1e-12
    assert abs(ssd.confidence(z, 0.5) - 0.9) < 1e-12      # softmax(2z) = (1, 9) / 10
