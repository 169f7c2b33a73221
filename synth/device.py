"""Device copies of the synthetic model, in the layout the C ABI takes.

Layout only (no arithmetic of the method): w_qkv stacks Wq, Wk, Wv row blocks;
w_gate_up stacks Wgate then Wup; bf16 projection weights (and the LM head) are
packed in the C ABI's tile layout; norm gains are float32 1 + w (the same single
fp32 addition as norm_gain_host).
"""
import torch

from . import KIND_WDOWN, KIND_WGATE, KIND_WK, KIND_WO, KIND_WQ, KIND_WUP, KIND_WV, TID_EMBED, TID_LM_HEAD
from . import GAIN_STD, KIND_ATTN_NORM, KIND_MLP_NORM, SEED_WEIGHTS, TID_FINAL_NORM, layer_tid, weight_dev


def pack_bf16(w):
    """Row-major [N, K] bf16 -> the packed tile layout of the C ABI (1-D): 16-row groups of
    32-column steps, each 16 x 32 block contiguous; N padded to a multiple of 16 with zeros."""
    N, K = w.shape
    Np = (N + 15) // 16 * 16
    if Np != N:
        w = torch.cat([w, w.new_zeros(Np - N, K)])
    return w.view(Np // 16, 16, K // 32, 32).permute(0, 2, 1, 3).contiguous().view(-1)


def unpack_bf16(t, N, K):
    """Inverse of pack_bf16: the [N, K] row-major matrix."""
    Np = (N + 15) // 16 * 16
    return t.view(Np // 16, K // 32, 16, 32).permute(0, 2, 1, 3).reshape(Np, K)[:N]


def norm_gain_dev(n, tensor_id, seed=SEED_WEIGHTS, device="cuda"):
    w = weight_dev(torch.empty(n, dtype=torch.float32, device=device), tensor_id, seed=seed, std=GAIN_STD)
    return w + 1.0


def build_weights(shape, seed=SEED_WEIGHTS, device="cuda", n_layers=None):
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    D, F = shape.d_model, shape.ffn_dim
    qd, kd = shape.q_dim, shape.kv_dim

    def fill_rows(t, row0, rows, tid):
        weight_dev(t.view(-1)[row0 * t.shape[1]:(row0 + rows) * t.shape[1]], tid, seed=seed)

    layers = []
    for l in range(shape.n_layers if n_layers is None else n_layers):
        wqkv = torch.empty(qd + 2 * kd, D, dtype=dt, device=device)
        fill_rows(wqkv, 0, qd, layer_tid(l, KIND_WQ))
        fill_rows(wqkv, qd, kd, layer_tid(l, KIND_WK))
        fill_rows(wqkv, qd + kd, kd, layer_tid(l, KIND_WV))
        wo = weight_dev(torch.empty(D, qd, dtype=dt, device=device), layer_tid(l, KIND_WO), seed=seed)
        wgu = torch.empty(2 * F, D, dtype=dt, device=device)
        fill_rows(wgu, 0, F, layer_tid(l, KIND_WGATE))
        fill_rows(wgu, F, F, layer_tid(l, KIND_WUP))
        wd = weight_dev(torch.empty(D, F, dtype=dt, device=device), layer_tid(l, KIND_WDOWN), seed=seed)
        if dt == torch.bfloat16:
            wqkv, wo, wgu, wd = pack_bf16(wqkv), pack_bf16(wo), pack_bf16(wgu), pack_bf16(wd)
        layers.append({"attn_norm": norm_gain_dev(D, layer_tid(l, KIND_ATTN_NORM), seed, device), "w_qkv": wqkv,
                       "w_o": wo, "mlp_norm": norm_gain_dev(D, layer_tid(l, KIND_MLP_NORM), seed, device),
                       "w_gate_up": wgu, "w_down": wd})
    lm_head = weight_dev(torch.empty(shape.vocab, D, dtype=dt, device=device), TID_LM_HEAD, seed=seed)
    if dt == torch.bfloat16:
        lm_head = pack_bf16(lm_head)
    return {
        "embed": weight_dev(torch.empty(shape.vocab, D, dtype=dt, device=device), TID_EMBED, seed=seed),
        "lm_head": lm_head,
        "final_norm": norm_gain_dev(D, TID_FINAL_NORM, seed, device),
        "layers": layers,
    }
