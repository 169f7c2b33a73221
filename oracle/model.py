"""Llama-style decoder with a KV cache and sub-layer skipping (float64 oracle).

Model (SWIFT digest §5.1: LLaMA-2 backbones; LayerSkip blog §2 "Shared Early
Exit Loss": one LM head shared by every exit; SpecEE notes, AdaInfer §1: the
LM head maps a d-dim hidden state to V logits):
  h = Emb[token]
  per layer l:  attention sub-layer  h += Wo . attn(RoPE(Wq x), RoPE(Wk x), Wv x),  x = RMSNorm(h)
                MLP sub-layer        h += Wdown . (silu(Wgate x) * (Wup x)),        x = RMSNorm(h)
  logits = LMhead . RMSNorm_final(h)
Readings where the pages are silent: no biases, RMSNorm eps 1e-5, RoPE base
10000 with rotate-half pairing, attention scale hd^-1/2, grouped-query
attention maps query head j to KV head j // (H / KVH), untied embedding, the
shared final RMSNorm applied before the shared LM head at every exit.

Skip plan (SWIFT digest §3.1 and Appendix A Fig. 10: skipped attention and MLP
layers are marked separately): uint8[2L], entry 2l = skip the attention
sub-layer of layer l, entry 2l+1 = skip its MLP sub-layer.  A LayerSkip exit at
E (LayerSkip blog §3.1) is the plan that skips every sub-layer of layers E..L-1.

RMSNorm before a projection is the plain definition: the projection input is
x = rnd(h / rms(h) * gain) with rms(h) = sqrt(mean(h^2) + eps), and the
projection is x . W^T.

Precision (bf16 models): the model stores bf16 tensors at these points and
rounds to nearest-even there; everything else is float64 here —
the normalised residual entering a projection (after the gain), RoPE'd q, the
cached k and v, the attention output entering Wo, the SwiGLU product entering
Wdown.  fp32 models are computed in float64 with no rounding.

Tracing: a callable ``trace(name, layer, value)`` passed to the functions below
receives each rounding point's tensor and the residual it was formed from
(names "h_attn", "x_attn", "q", "k", "v", "o", "h_mlp", "x_mlp", "a", "h_final",
"x_final"), so that tests can check every rounding point on its own.
"""
import dataclasses

import numpy as np

import synth
from .numerics import bf16_round, rmsnorm, rope, silu, softmax


@dataclasses.dataclass
class LayerWeights:
    attn_norm: np.ndarray      # [D]
    wq: np.ndarray             # [H*hd, D]
    wk: np.ndarray             # [KVH*hd, D]
    wv: np.ndarray             # [KVH*hd, D]
    wo: np.ndarray             # [D, H*hd]
    mlp_norm: np.ndarray       # [D]
    wgate: np.ndarray          # [F, D]
    wup: np.ndarray            # [F, D]
    wdown: np.ndarray          # [D, F]


@dataclasses.dataclass
class Model:
    shape: synth.ModelShape
    embed: np.ndarray          # [V, D]
    layers: list
    final_norm: np.ndarray     # [D]
    lm_head: np.ndarray        # [V, D]

    @property
    def L(self):
        return self.shape.n_layers

    def rnd(self, x):
        """bf16 storage rounding for bf16 models; identity for fp32 models."""
        return bf16_round(x) if self.shape.dtype == "bf16" else x

    @staticmethod
    def synthetic(shape, seed=synth.SEED_WEIGHTS, n_layers=None):
        """Weights from the shared seeded generator (norm gains 1 + w, float32)."""
        s = shape
        bf = s.dtype == "bf16"
        W = lambda rows, cols, tid: synth.weight_host((rows, cols), tid, "f64", bf16=bf, seed=seed)
        G = lambda tid: synth.norm_gain_host(s.d_model, tid, seed=seed).astype(np.float64)
        layers = []
        for l in range(s.n_layers if n_layers is None else n_layers):
            layers.append(LayerWeights(
                attn_norm=G(synth.layer_tid(l, synth.KIND_ATTN_NORM)),
                wq=W(s.q_dim, s.d_model, synth.layer_tid(l, synth.KIND_WQ)),
                wk=W(s.kv_dim, s.d_model, synth.layer_tid(l, synth.KIND_WK)),
                wv=W(s.kv_dim, s.d_model, synth.layer_tid(l, synth.KIND_WV)),
                wo=W(s.d_model, s.q_dim, synth.layer_tid(l, synth.KIND_WO)),
                mlp_norm=G(synth.layer_tid(l, synth.KIND_MLP_NORM)),
                wgate=W(s.ffn_dim, s.d_model, synth.layer_tid(l, synth.KIND_WGATE)),
                wup=W(s.ffn_dim, s.d_model, synth.layer_tid(l, synth.KIND_WUP)),
                wdown=W(s.d_model, s.ffn_dim, synth.layer_tid(l, synth.KIND_WDOWN)),
            ))
        return Model(shape=s, embed=W(s.vocab, s.d_model, synth.TID_EMBED), layers=layers,
                     final_norm=G(synth.TID_FINAL_NORM), lm_head=W(s.vocab, s.d_model, synth.TID_LM_HEAD))


class KVCache:
    """Per-layer key/value store indexed by absolute position: K[l, pos, kv_head, hd]."""

    def __init__(self, shape, capacity):
        self.K = np.zeros((shape.n_layers, capacity, shape.n_kv_heads, shape.head_dim))
        self.V = np.zeros_like(self.K)

    def copy(self):
        c = KVCache.__new__(KVCache)
        c.K = self.K.copy()
        c.V = self.V.copy()
        return c


def skip_attn(mask, l):
    return mask is not None and bool(mask[2 * l])


def skip_mlp(mask, l):
    return mask is not None and bool(mask[2 * l + 1])


def first_skipped_layer(mask, n_layers):
    """Reuse boundary b: the first layer with a skipped sub-layer (n_layers if none).
    Every sub-layer below b runs in the draft exactly as in the full model."""
    if mask is None:
        return n_layers
    for l in range(n_layers):
        if mask[2 * l] or mask[2 * l + 1]:
            return l
    return n_layers


def norm_input(model, h, gain):
    """Projection input of an RMSNorm sub-layer: rnd(RMSNorm(h) * gain), per row."""
    return model.rnd(rmsnorm(h, gain, model.shape.rms_eps))


def _tr(trace, name, l, v):
    if trace is not None:
        trace(name, l, v)


def attention_sublayer(model, l, h, positions, kv, trace=None):
    """One attention sub-layer over rows h[M, D] at absolute positions (increasing).

    Writes the rows' keys and values at their positions, then each row attends
    causally to every cached position <= its own.
    """
    s = model.shape
    lw = model.layers[l]
    M = h.shape[0]
    H, KVH, hd = s.n_heads, s.n_kv_heads, s.head_dim
    x = norm_input(model, h, lw.attn_norm)
    _tr(trace, "h_attn", l, h)
    _tr(trace, "x_attn", l, x)
    q = (x @ lw.wq.T).reshape(M, H, hd)
    k = (x @ lw.wk.T).reshape(M, KVH, hd)
    v = (x @ lw.wv.T).reshape(M, KVH, hd)
    q = model.rnd(rope(q, positions, s.rope_theta))
    k = model.rnd(rope(k, positions, s.rope_theta))
    v = model.rnd(v)
    _tr(trace, "q", l, q)
    _tr(trace, "k", l, k)
    _tr(trace, "v", l, v)
    for i, p in enumerate(positions):
        kv.K[l, p] = k[i]
        kv.V[l, p] = v[i]
    G = H // KVH
    o = np.empty((M, H, hd))
    scale = 1.0 / np.sqrt(hd)
    for i, p in enumerate(positions):
        Kc = kv.K[l, : p + 1]                    # [p+1, KVH, hd]
        Vc = kv.V[l, : p + 1]
        qg = q[i].reshape(KVH, G, hd)
        sc = np.einsum("gjd,kgd->gjk", qg, Kc) * scale
        pr = softmax(sc)
        o[i] = np.einsum("gjk,kgd->gjd", pr, Vc).reshape(H, hd)
    o = model.rnd(o.reshape(M, H * hd))
    _tr(trace, "o", l, o)
    return h + o @ lw.wo.T


def mlp_sublayer(model, l, h, trace=None):
    lw = model.layers[l]
    x = norm_input(model, h, lw.mlp_norm)
    _tr(trace, "h_mlp", l, h)
    _tr(trace, "x_mlp", l, x)
    a = model.rnd(silu(x @ lw.wgate.T) * (x @ lw.wup.T))
    _tr(trace, "a", l, a)
    return h + a @ lw.wdown.T


def run_layers(model, h, positions, kv, mask=None, l_begin=0, l_end=None, trace=None):
    """Layers l_begin..l_end-1 over rows h, skipping the sub-layers the plan marks."""
    l_end = model.L if l_end is None else l_end
    for l in range(l_begin, l_end):
        if not skip_attn(mask, l):
            h = attention_sublayer(model, l, h, positions, kv, trace)
        if not skip_mlp(mask, l):
            h = mlp_sublayer(model, l, h, trace)
    return h


def embed(model, tokens):
    return model.embed[np.asarray(tokens, dtype=np.int64)].astype(np.float64)


def final_logits(model, h, trace=None):
    """Shared final RMSNorm and shared LM head: logits [M, V] (LayerSkip blog §2)."""
    x = norm_input(model, h, model.final_norm)
    _tr(trace, "h_final", model.L, h)
    _tr(trace, "x_final", model.L, x)
    return x @ model.lm_head.T


def forward(model, tokens, positions, kv, mask=None, trace=None):
    """Embed + every (non-skipped) layer + final norm + LM head for a block of rows."""
    h = embed(model, tokens)
    h = run_layers(model, h, list(positions), kv, mask, trace=trace)
    return final_logits(model, h, trace)
