"""Elementary numerics of the Llama-style decoder (float64), oracle side.

The pages fix the model family only as a Llama-2 decoder with a shared LM head
(LayerSkip blog §2 "Shared Early Exit Loss" and §3; SWIFT digest §5.1 names
LLaMA-2).  The layer definitions below are the standard Llama-2 ones, pinned
against an independent implementation (Hugging Face ``LlamaForCausalLM`` in
float64, tests/test_oracle_model.py).
"""
import numpy as np


def bf16_round(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 has an 8-bit significand and float32's exponent range.  For a
    finite x with |x| = m * 2^e (m in [0.5, 1)), the spacing of bf16 values is
    2^(e-8) in the normal range and 2^-133 below 2^-126.  Pinned against
    torch's float32 -> bfloat16 conversion (tests/test_oracle_numerics.py).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)
    e = np.maximum(e, -125)                     # below 2^-126: fixed subnormal spacing 2^-133
    ulp = np.ldexp(1.0, e - 8)
    r = np.round(xf / ulp) * ulp                # np.round rounds half to even; /ulp is exact
    big = np.abs(r) >= 2.0 ** 128               # past the largest finite bf16 (0x7F7F): overflow to inf
    r[big] = np.copysign(np.inf, r[big])
    out[fin] = r
    return out


def rms(h, eps):
    """Per-row root mean square with the RMSNorm epsilon: sqrt(mean(h^2) + eps), shape [M, 1]."""
    return np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def rmsnorm(h, gain, eps):
    """RMSNorm: h / sqrt(mean(h^2) + eps) * gain, per row."""
    return h / rms(h, eps) * gain


def rope_angles(positions, head_dim, theta):
    """Rotation angles pos * theta^(-2i/hd), i = 0..hd/2-1 (rotate-half pairing)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(x, positions, theta):
    """Rotary embedding on x [M, heads, hd]: pairs (i, i + hd/2) rotated by the angle of i."""
    hd = x.shape[-1]
    a = rope_angles(positions, hd, theta)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : hd // 2], x[..., hd // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


def softmax(z):
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def argmax_lowest(z):
    """Index of the maximum; the lowest index among equal maxima (np.argmax's rule)."""
    return int(np.argmax(z))
