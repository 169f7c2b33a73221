"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Holds no arithmetic of the decoding method: it only maps (seed, tensor id,
element index) to weights and token ids, with a counter-based generator
(Philox4x32-10) whose host and device implementations produce identical bits
(definitions in synth.h).  Also holds the workload shapes and the tensor-id
scheme, which both sides need to build the same model.
"""
import ctypes
import dataclasses
import os

import numpy as np

from . import build as _build

_HOST = None
_DEV = None

F32, BF16, F64 = 0, 1, 2

# Seeds of the synthetic workloads (weights, prompt, masks, sampling, window).
SEED_WEIGHTS, SEED_PROMPT, SEED_MASKS, SEED_SAMPLING = 0, 1, 2, 3
WEIGHT_STD = 0.02


def host_lib():
    global _HOST
    if _HOST is None:
        if not os.path.exists(_build.HOST_LIB):
            _build.build_host()
        lib = ctypes.CDLL(_build.HOST_LIB)
        lib.synth_philox4x32_10.argtypes = [ctypes.POINTER(ctypes.c_uint32)] * 3
        lib.synth_philox4x32_10.restype = None
        lib.synth_fill_weight_host.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                               ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float]
        lib.synth_fill_weight_host.restype = ctypes.c_int
        lib.synth_fill_tokens_host.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                               ctypes.c_uint32, ctypes.c_int32]
        lib.synth_fill_tokens_host.restype = ctypes.c_int
        _HOST = lib
    return _HOST


def dev_lib():
    global _DEV
    if _DEV is None:
        if not os.path.exists(_build.DEV_LIB):
            raise RuntimeError("device generator library missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(_build.DEV_LIB)
        lib.synth_fill_weight_dev.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                              ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p]
        lib.synth_fill_weight_dev.restype = ctypes.c_int
        lib.synth_fill_tokens_dev.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                              ctypes.c_uint32, ctypes.c_int32, ctypes.c_void_p]
        lib.synth_fill_tokens_dev.restype = ctypes.c_int
        _DEV = lib
    return _DEV


def philox4x32_10(ctr, key):
    """One Philox4x32-10 block: 4 counter words, 2 key words -> 4 output words."""
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (ctypes.c_uint32 * 4)()
    host_lib().synth_philox4x32_10(c, k, o)
    return [int(x) for x in o]


def weight_host(shape, tensor_id, dtype="f64", bf16=False, seed=SEED_WEIGHTS, std=WEIGHT_STD, e0=0):
    """Host copy of a weight tensor.  dtype 'f64' gives float64 holding the fp32
    value (or its bf16 rounding when bf16=True); 'f32' gives float32; 'bf16'
    gives uint16 bit patterns."""
    n = int(np.prod(shape))
    if dtype == "f64":
        out = np.empty(n, np.float64); code = F64
    elif dtype == "f32":
        out = np.empty(n, np.float32); code = F32
    elif dtype == "bf16":
        out = np.empty(n, np.uint16); code = BF16
    else:
        raise ValueError(dtype)
    rc = host_lib().synth_fill_weight_host(out.ctypes.data, code, 1 if bf16 else 0, e0, n, seed,
                                           tensor_id & 0xFFFFFFFF, std)
    if rc != 0:
        raise RuntimeError("synth_fill_weight_host failed")
    return out.reshape(shape)


def tokens_host(n, stream_id, vocab, seed=SEED_PROMPT):
    out = np.empty(n, np.int32)
    if host_lib().synth_fill_tokens_host(out.ctypes.data, n, seed, stream_id & 0xFFFFFFFF, vocab) != 0:
        raise RuntimeError("synth_fill_tokens_host failed")
    return out


def weight_dev(tensor, tensor_id, seed=SEED_WEIGHTS, std=WEIGHT_STD, e0=0, stream=0):
    """Fill a contiguous torch device tensor (float32 or bfloat16) in place."""
    import torch
    assert tensor.is_contiguous() and tensor.is_cuda
    code = {torch.float32: F32, torch.bfloat16: BF16}[tensor.dtype]
    rc = dev_lib().synth_fill_weight_dev(tensor.data_ptr(), code, e0, tensor.numel(), seed,
                                         tensor_id & 0xFFFFFFFF, std, stream)
    if rc != 0:
        raise RuntimeError("synth_fill_weight_dev failed: %d" % rc)
    return tensor


def tokens_dev(tensor, stream_id, vocab, seed=SEED_PROMPT, stream=0):
    import torch
    assert tensor.is_contiguous() and tensor.is_cuda and tensor.dtype == torch.int32
    rc = dev_lib().synth_fill_tokens_dev(tensor.data_ptr(), tensor.numel(), seed, stream_id & 0xFFFFFFFF,
                                         vocab, stream)
    if rc != 0:
        raise RuntimeError("synth_fill_tokens_dev failed: %d" % rc)
    return tensor


# ---------------------------------------------------------------------------
# Tensor ids.  Logical layouts are row-major [out, in] ("N x K").
KIND_WQ, KIND_WK, KIND_WV, KIND_WO, KIND_WGATE, KIND_WUP, KIND_WDOWN = 1, 2, 3, 4, 6, 7, 8
KIND_ATTN_NORM, KIND_MLP_NORM = 9, 10
TID_EMBED = 0xFFFF0001
TID_LM_HEAD = 0xFFFF0002
TID_FINAL_NORM = 0xFFFF0003
GAIN_STD = 0.1        # RMSNorm gains: 1 + w, w of the weight law with this deviation (fp32 add)


def norm_gain_host(n, tensor_id, seed=SEED_WEIGHTS):
    """float32 RMSNorm gain vector 1 + w (one fp32 addition per element)."""
    w = weight_host((n,), tensor_id, "f32", seed=seed, std=GAIN_STD)
    return (np.float32(1.0) + w).astype(np.float32)
STREAM_PROMPT = 0x50000001


def layer_tid(layer, kind):
    return (layer << 4) | kind


@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    dtype: str            # "f32" or "bf16": storage type of weights and activations
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def q_dim(self):
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_dim(self):
        return self.q_dim + 2 * self.kv_dim

    def layer_param_count(self):
        D = self.d_model
        return D * self.qkv_dim + self.q_dim * D + 2 * self.ffn_dim * D + self.ffn_dim * D

    def param_count(self):
        return self.n_layers * self.layer_param_count() + 2 * self.vocab * self.d_model


# The five workloads' model shapes.
TINY = ModelShape("tiny-f32", 4, 256, 4, 4, 64, 688, 1024, "f32")
LLAMA7B = ModelShape("llama2-7b-shape", 32, 4096, 32, 32, 128, 11008, 32000, "bf16")
LLAMA13B = ModelShape("llama2-13b-shape", 40, 5120, 40, 40, 128, 13824, 32000, "bf16")
LLAMA70B = ModelShape("llama2-70b-shape", 80, 8192, 64, 8, 128, 28672, 32000, "bf16")

SHAPES = {s.name: s for s in (TINY, LLAMA7B, LLAMA13B, LLAMA70B)}


def prompt_tokens(n, vocab, seed=SEED_PROMPT):
    return tokens_host(n, STREAM_PROMPT, vocab, seed=seed)


def random_skip_layers(n_layers, n_skip, seed, index=0):
    """Layer indices (sorted) of a seeded uniform n_skip-of-n_layers subset."""
    # Fisher-Yates driven by the token stream (uniform draws over shrinking ranges).
    idx = list(range(n_layers))
    draws = []
    for i in range(n_skip):
        draws.append(int(tokens_host(1, 0x4D000000 + (index << 8) + i, n_layers - i, seed=seed)[0]))
    chosen = []
    for i, r in enumerate(draws):
        j = i + r
        idx[i], idx[j] = idx[j], idx[i]
        chosen.append(idx[i])
    return sorted(chosen)


def scoring_masks(n_layers, n_masks, lo, hi, seed=SEED_MASKS):
    """Candidate skip masks for mask scoring: candidate c skips a seeded uniform
    subset of k_c layers, k_c uniform over [lo, hi]."""
    ks = tokens_host(n_masks, 0x4E000000, hi - lo + 1, seed=seed) + lo
    return np.stack([mask_from_layers(n_layers, random_skip_layers(n_layers, int(k), seed, index=c + 1))
                     for c, k in enumerate(ks)])


def mask_from_layers(n_layers, layers):
    """uint8[2L] skip mask: bit pair (2l, 2l+1) = (attention, MLP) of layer l skipped."""
    m = np.zeros(2 * n_layers, np.uint8)
    for l in layers:
        m[2 * l] = 1
        m[2 * l + 1] = 1
    return m


def mask_exit(n_layers, exit_layer):
    """Early-exit plan at E: every sub-layer of layers E..L-1 skipped."""
    return mask_from_layers(n_layers, range(exit_layer, n_layers))
