"""ctypes binding of include/ssd.h (same names; argument marshalling only)."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssd.so")

SSD_OK = 0
SSD_ERR_ARG, SSD_ERR_SHAPE, SSD_ERR_CAPACITY, SSD_ERR_HIP, SSD_ERR_UNSUPPORTED, SSD_ERR_NUMERIC = -1, -2, -3, -4, -5, -6
SSD_DTYPE_F32, SSD_DTYPE_BF16 = 0, 1

ERROR_NAMES = {-1: "SSD_ERR_ARG", -2: "SSD_ERR_SHAPE", -3: "SSD_ERR_CAPACITY", -4: "SSD_ERR_HIP",
               -5: "SSD_ERR_UNSUPPORTED", -6: "SSD_ERR_NUMERIC"}

# Every symbol include/ssd.h declares.
EXPORTS = ["ssd_model_create", "ssd_model_destroy", "ssd_packed_bf16_bytes", "ssd_pack_bf16", "ssd_kv_pool_bytes",
           "ssd_workspace_bytes", "ssd_seq_create",
           "ssd_seq_destroy", "ssd_prefill", "ssd_decode_ar", "ssd_decode_exit", "ssd_draft", "ssd_verify",
           "ssd_accept", "ssd_accept_noalloc", "ssd_commit", "ssd_tree_candidates", "ssd_verify_tree", "ssd_accept_tree",
           "ssd_score_masks", "ssd_uniform_mask", "ssd_swift_propose", "ssd_swift_search", "ssd_swift_begin",
           "ssd_swift_generate", "ssd_specee_features",
           "ssd_row_stats",
           "ssd_read_state", "ssd_read_output", "ssd_last_error",
           "ssd_profile_enable", "ssd_profile_disable", "ssd_profile_read", "ssd_probe_read"]


class SSDError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%d): %s" % (ERROR_NAMES.get(code, "?"), code, msg))
        self.code = code


class ssd_layer_weights(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p),
                ("mlp_norm", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p)]


class ssd_model_desc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("d_model", ctypes.c_int), ("n_heads", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("ffn_dim", ctypes.c_int),
                ("vocab", ctypes.c_int), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("dtype", ctypes.c_int), ("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("lm_head", ctypes.c_void_p), ("layers", ctypes.POINTER(ssd_layer_weights))]


class ssd_row_stat(ctypes.Structure):
    _fields_ = [("max", ctypes.c_float), ("argmax", ctypes.c_int32), ("max2", ctypes.c_float),
                ("lse", ctypes.c_float), ("conf", ctypes.c_float), ("sample", ctypes.c_int32)]


class ssd_swift_config(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_int32), ("accumulate", ctypes.c_int32), ("n_skip", ctypes.c_int32),
                ("sublayers", ctypes.c_int32), ("n_cand", ctypes.c_int32), ("steps_per_phase", ctypes.c_int32),
                ("max_steps", ctypes.c_int32), ("patience", ctypes.c_int32), ("target", ctypes.c_float),
                ("bo_every", ctypes.c_int32), ("d", ctypes.c_int32), ("conf_thresh", ctypes.c_float),
                ("temperature", ctypes.c_float), ("seed", ctypes.c_uint64)]


class ssd_swift_state(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int32), ("unimproved", ctypes.c_int32), ("done", ctypes.c_int32),
                ("last_phase_n_out", ctypes.c_int32), ("phases", ctypes.c_int32), ("switches", ctypes.c_int32),
                ("score", ctypes.c_float), ("iterations", ctypes.c_int32)]


class ssd_state(ctypes.Structure):
    _fields_ = [("kvlen", ctypes.c_int32), ("last_token", ctypes.c_int32), ("iteration", ctypes.c_int32),
                ("n_out", ctypes.c_int32), ("error_flags", ctypes.c_int32), ("last_n_drafted", ctypes.c_int32),
                ("last_n_emitted", ctypes.c_int32)]


_LIB = None
P = ctypes.c_void_p
I = ctypes.c_int
F = ctypes.c_float
U64 = ctypes.c_uint64
SZ = ctypes.POINTER(ctypes.c_size_t)


def lib():
    """Load libssd.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libssd.so is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "ssd_model_create": [ctypes.POINTER(ssd_model_desc), ctypes.POINTER(P)],
            "ssd_model_destroy": [P],
            "ssd_packed_bf16_bytes": [I, I, ctypes.POINTER(ctypes.c_size_t)],
            "ssd_pack_bf16": [P, P, I, I, P],
            "ssd_kv_pool_bytes": [P, I, I, SZ],
            "ssd_workspace_bytes": [P, I, I, I, SZ],
            "ssd_seq_create": [P, P, I, I, P, I, P, ctypes.c_size_t, I, I, P, ctypes.POINTER(P)],
            "ssd_seq_destroy": [P],
            "ssd_prefill": [P, P, I, F, U64, P, P],
            "ssd_decode_ar": [P, F, U64, P, P],
            "ssd_decode_exit": [P, P, I, F, U64, P, P],
            "ssd_draft": [P, P, I, I, F, F, U64, P, P, P, P],
            "ssd_verify": [P, P, I, I, P, P, I, P, P],
            "ssd_accept": [P, P, P, P, P, I, F, U64, P, P, P],
            "ssd_accept_noalloc": [P, P, P, P, I, I, F, U64, ctypes.c_int32, P, P, P],
            "ssd_commit": [P, P, P, P],
            "ssd_tree_candidates": [P, P, P, I, F, U64, F, I, I, P, P, P, P],
            "ssd_verify_tree": [P, P, I, I, P, P, P, P, P, I, I, P, P],
            "ssd_accept_tree": [P, P, P, P, P, I, P, P, P, I, F, U64, P, P, P],
            "ssd_score_masks": [P, P, I, P, I, I, P, P, P, P],
            "ssd_uniform_mask": [I, I, P],
            "ssd_specee_features": [P, P, I, P, I, P, P, P],
            "ssd_swift_propose": [I, I, I, U64, I, I, P],
            "ssd_swift_search": [P, P, I, I, P, I, I, I, I, I, F, U64, I, P, ctypes.POINTER(F), ctypes.POINTER(I), P],
            "ssd_swift_begin": [P, ctypes.POINTER(ssd_swift_config), ctypes.POINTER(ssd_swift_state), P],
            "ssd_swift_generate": [P, ctypes.POINTER(ssd_swift_config), ctypes.POINTER(ssd_swift_state), P, I, P, P, P,
                                   P, P, P, P],
            "ssd_row_stats": [P, I, I, F, U64, ctypes.c_int32, P, P],
            "ssd_read_state": [P, ctypes.POINTER(ssd_state), P],
            "ssd_read_output": [P, P, I, ctypes.POINTER(I), P],
            "ssd_profile_enable": [I, I],
            "ssd_profile_disable": [],
            "ssd_profile_read": [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I), ctypes.POINTER(ctypes.c_double)],
            "ssd_probe_read": [P, U64, P, P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.ssd_last_error.argtypes = []
        L.ssd_last_error.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def check(rc):
    if rc != SSD_OK:
        raise SSDError(rc, lib().ssd_last_error().decode())
    return rc


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _mask_arg(mask):
    if mask is None:
        return None, None
    import numpy as np
    m = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8))
    return m, m.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# thin wrappers, same names as the C ABI

def ssd_model_create(desc):
    h = ctypes.c_void_p()
    check(lib().ssd_model_create(ctypes.byref(desc), ctypes.byref(h)))
    return h


def ssd_model_destroy(model):
    check(lib().ssd_model_destroy(model))


def ssd_packed_bf16_bytes(N, K):
    b = ctypes.c_size_t()
    check(lib().ssd_packed_bf16_bytes(N, K, ctypes.byref(b)))
    return b.value


def ssd_pack_bf16(src, dst, N, K, stream=None):
    check(lib().ssd_pack_bf16(_ptr(src), _ptr(dst), N, K, _stream(stream)))


def ssd_kv_pool_bytes(model, n_pages, page_size):
    n = ctypes.c_size_t()
    check(lib().ssd_kv_pool_bytes(model, n_pages, page_size, ctypes.byref(n)))
    return n.value


def ssd_workspace_bytes(model, max_rows, max_draft, max_ctx):
    n = ctypes.c_size_t()
    check(lib().ssd_workspace_bytes(model, max_rows, max_draft, max_ctx, ctypes.byref(n)))
    return n.value


def ssd_seq_create(model, kv_pool, n_pages, page_size, page_table, workspace, max_rows, max_draft, stream=None):
    import numpy as np
    pt = np.ascontiguousarray(np.asarray(page_table, dtype=np.int32))
    h = ctypes.c_void_p()
    check(lib().ssd_seq_create(model, _ptr(kv_pool), n_pages, page_size, pt.ctypes.data_as(ctypes.c_void_p), len(pt),
                               _ptr(workspace), workspace.numel() * workspace.element_size(), max_rows, max_draft,
                               _stream(stream), ctypes.byref(h)))
    return h


def ssd_seq_destroy(seq):
    check(lib().ssd_seq_destroy(seq))




def ssd_prefill(seq, tokens, temperature=0.0, seed=0, last_logits=None, stream=None):
    check(lib().ssd_prefill(seq, _ptr(tokens), tokens.numel(), temperature, seed, _ptr(last_logits), _stream(stream)))


def ssd_decode_ar(seq, temperature=0.0, seed=0, logits=None, stream=None):
    check(lib().ssd_decode_ar(seq, temperature, seed, _ptr(logits), _stream(stream)))


def ssd_decode_exit(seq, skip_mask, exit_layer, temperature=0.0, seed=0, logits=None, stream=None):
    keep, mp = _mask_arg(skip_mask)
    check(lib().ssd_decode_exit(seq, mp, -1 if exit_layer is None else exit_layer, temperature, seed, _ptr(logits),
                                _stream(stream)))


def ssd_draft(seq, skip_mask, exit_layer, d, conf_thresh, temperature, seed, draft_tokens, draft_logits, n_drafted,
              stream=None):
    keep, mp = _mask_arg(skip_mask)
    check(lib().ssd_draft(seq, mp, -1 if exit_layer is None else exit_layer, d, conf_thresh, temperature, seed,
                          _ptr(draft_tokens), _ptr(draft_logits), _ptr(n_drafted), _stream(stream)))


def ssd_verify(seq, skip_mask, exit_layer, d, draft_tokens, n_drafted, reuse, logits, stream=None):
    keep, mp = _mask_arg(skip_mask)
    check(lib().ssd_verify(seq, mp, -1 if exit_layer is None else exit_layer, d, _ptr(draft_tokens), _ptr(n_drafted),
                           1 if reuse else 0, _ptr(logits), _stream(stream)))


def ssd_accept(seq, p_logits, q_logits, draft_tokens, n_drafted, d, temperature, seed, out_tokens, n_out,
               stream=None):
    check(lib().ssd_accept(seq, _ptr(p_logits), _ptr(q_logits), _ptr(draft_tokens), _ptr(n_drafted), d, temperature,
                           seed, _ptr(out_tokens), _ptr(n_out), _stream(stream)))


def ssd_accept_noalloc(p_logits, q_logits, draft_tokens, n_drafted, d, vocab, temperature, seed, iteration,
                       out_tokens, n_out, stream=None):
    check(lib().ssd_accept_noalloc(_ptr(p_logits), _ptr(q_logits), _ptr(draft_tokens), _ptr(n_drafted), d, vocab,
                                   temperature, seed, iteration, _ptr(out_tokens), _ptr(n_out), _stream(stream)))


def ssd_commit(seq, out_tokens, n_out, stream=None):
    check(lib().ssd_commit(seq, _ptr(out_tokens), _ptr(n_out), _stream(stream)))


def ssd_tree_candidates(seq, draft_logits, n_drafted, d, rho, k_max, max_leaves, leaf_tokens, leaf_depth, n_leaves,
                        temperature=0.0, seed=0, stream=None):
    check(lib().ssd_tree_candidates(seq, _ptr(draft_logits), _ptr(n_drafted), d, temperature, seed, rho, k_max,
                                    max_leaves, _ptr(leaf_tokens), _ptr(leaf_depth), _ptr(n_leaves),
                                    _stream(stream)))


def ssd_verify_tree(seq, skip_mask, exit_layer, d, draft_tokens, n_drafted, leaf_tokens, leaf_depth, n_leaves,
                    max_leaves, reuse, logits, stream=None):
    keep, mp = _mask_arg(skip_mask)
    check(lib().ssd_verify_tree(seq, mp, -1 if exit_layer is None else exit_layer, d, _ptr(draft_tokens),
                                _ptr(n_drafted), _ptr(leaf_tokens), _ptr(leaf_depth), _ptr(n_leaves), max_leaves,
                                1 if reuse else 0, _ptr(logits), _stream(stream)))


def ssd_accept_tree(seq, logits, draft_tokens, n_drafted, d, leaf_tokens, leaf_depth, n_leaves, max_leaves,
                    out_tokens, n_out, q_logits=None, temperature=0.0, seed=0, stream=None):
    check(lib().ssd_accept_tree(seq, _ptr(logits), _ptr(q_logits), _ptr(draft_tokens), _ptr(n_drafted), d,
                                _ptr(leaf_tokens), _ptr(leaf_depth), _ptr(n_leaves), max_leaves, temperature, seed,
                                _ptr(out_tokens), _ptr(n_out), _stream(stream)))


def ssd_score_masks(seq, masks, window, pos0, gamma, scores, best, row_pred=None, stream=None):
    import numpy as np
    m = np.ascontiguousarray(np.asarray(masks, dtype=np.uint8))
    check(lib().ssd_score_masks(seq, m.ctypes.data_as(ctypes.c_void_p), m.shape[0], _ptr(window), pos0, gamma,
                                _ptr(scores), _ptr(best), _ptr(row_pred), _stream(stream)))


def ssd_uniform_mask(n_layers, n_skip):
    import numpy as np
    m = np.zeros(2 * n_layers, np.uint8)
    check(lib().ssd_uniform_mask(n_layers, n_skip, m.ctypes.data_as(ctypes.c_void_p)))
    return m


def ssd_swift_propose(n_layers, n_skip, seed, step, cand, sublayers=False):
    import numpy as np
    m = np.zeros(2 * n_layers, np.uint8)
    check(lib().ssd_swift_propose(n_layers, n_skip, 1 if sublayers else 0, seed, step, cand,
                                  m.ctypes.data_as(ctypes.c_void_p)))
    return m


def ssd_swift_search(seq, window, pos0, gamma, init_mask, n_skip, n_cand, max_steps, patience, target, seed,
                     n_layers, sublayers=False, bo_every=0, stream=None):
    """Returns (best mask, best score, steps run)."""
    import numpy as np
    im = np.ascontiguousarray(np.asarray(init_mask, dtype=np.uint8))
    out = np.zeros(2 * n_layers, np.uint8)
    sc, ns = F(0.0), I(0)
    check(lib().ssd_swift_search(seq, _ptr(window), pos0, gamma, im.ctypes.data_as(ctypes.c_void_p), n_skip,
                                 1 if sublayers else 0, n_cand, max_steps, patience, target, seed, bo_every,
                                 out.ctypes.data_as(ctypes.c_void_p),
                                 ctypes.byref(sc), ctypes.byref(ns), _stream(stream)))
    return out, float(sc.value), int(ns.value)


def swift_config(gamma, n_skip, n_cand, steps_per_phase, max_steps, patience, target, d, seed, accumulate=0,
                 sublayers=False, bo_every=0, conf_thresh=0.0, temperature=0.0):
    return ssd_swift_config(gamma, accumulate, n_skip, 1 if sublayers else 0, n_cand, steps_per_phase, max_steps,
                            patience, target, bo_every, d, conf_thresh, temperature, seed)


def ssd_swift_begin(seq, cfg, stream=None):
    st = ssd_swift_state()
    check(lib().ssd_swift_begin(seq, ctypes.byref(cfg), ctypes.byref(st), _stream(stream)))
    return st


def ssd_swift_generate(seq, cfg, state, plan, n_tokens, draft_tokens, draft_logits, n_drafted, verify_logits,
                       out_tokens, n_out, stream=None):
    """plan: a C-contiguous uint8 numpy array [2L], updated in place; state: updated in place."""
    import numpy as np
    assert isinstance(plan, np.ndarray) and plan.dtype == np.uint8 and plan.flags["C_CONTIGUOUS"]
    check(lib().ssd_swift_generate(seq, ctypes.byref(cfg), ctypes.byref(state), plan.ctypes.data_as(ctypes.c_void_p),
                                   n_tokens, _ptr(draft_tokens), _ptr(draft_logits), _ptr(n_drafted),
                                   _ptr(verify_logits), _ptr(out_tokens), _ptr(n_out), _stream(stream)))


def ssd_specee_features(model, h, rows, tokens, k, prev_probs, features, stream=None):
    check(lib().ssd_specee_features(model, _ptr(h), rows, _ptr(tokens), k, _ptr(prev_probs), _ptr(features),
                                    _stream(stream)))


def ssd_row_stats(logits, rows, V, temperature, seed, iteration, stats, stream=None):
    check(lib().ssd_row_stats(_ptr(logits), rows, V, temperature, seed, iteration, _ptr(stats), _stream(stream)))


def ssd_read_state(seq, stream=None, raise_flags=True):
    st = ssd_state()
    rc = lib().ssd_read_state(seq, ctypes.byref(st), _stream(stream))
    if rc != SSD_OK and (raise_flags or rc not in (SSD_ERR_CAPACITY, SSD_ERR_NUMERIC)):
        check(rc)
    return st


def ssd_read_output(seq, max_tokens, stream=None, raise_flags=True):
    import numpy as np
    out = np.zeros(max(1, max_tokens), np.int32)
    n = ctypes.c_int()
    rc = lib().ssd_read_output(seq, out.ctypes.data_as(ctypes.c_void_p), max_tokens, ctypes.byref(n),
                               _stream(stream))
    if rc != SSD_OK and (raise_flags or rc not in (SSD_ERR_CAPACITY, SSD_ERR_NUMERIC)):
        check(rc)
    return out[: n.value]


SSD_PROF_GEMM_STORE, SSD_PROF_GEMM_RESID, SSD_PROF_GEMM_SWIGLU = 0, 1, 2


def ssd_profile_enable(kernel_class, max_launches):
    check(lib().ssd_profile_enable(kernel_class, max_launches))


def ssd_profile_disable():
    check(lib().ssd_profile_disable())


def ssd_profile_read():
    ms, by = ctypes.c_double(), ctypes.c_double()
    n = ctypes.c_int()
    check(lib().ssd_profile_read(ctypes.byref(ms), ctypes.byref(n), ctypes.byref(by)))
    return ms.value, n.value, by.value


def ssd_probe_read(src, nbytes, sink, stream=None):
    check(lib().ssd_probe_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)))



# ---------------------------------------------------------------------------
# convenience owners of device memory

ROW_STAT_BYTES = ctypes.sizeof(ssd_row_stat)


class Model:
    """Owns an ssd_model handle over caller-provided weight tensors (kept alive here)."""

    def __init__(self, n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab, dtype, tensors,
                 rms_eps=1e-5, rope_theta=10000.0):
        self.tensors = tensors
        self.vocab = vocab
        self.n_layers = n_layers
        self.dtype = dtype
        lays = (ssd_layer_weights * n_layers)()
        for l, t in enumerate(tensors["layers"]):
            lays[l] = ssd_layer_weights(t["attn_norm"].data_ptr(), t["w_qkv"].data_ptr(), t["w_o"].data_ptr(),
                                        t["mlp_norm"].data_ptr(), t["w_gate_up"].data_ptr(), t["w_down"].data_ptr())
        self._lays = lays
        desc = ssd_model_desc(n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab, rms_eps, rope_theta,
                              SSD_DTYPE_BF16 if dtype == "bf16" else SSD_DTYPE_F32, tensors["embed"].data_ptr(),
                              tensors["final_norm"].data_ptr(), tensors["lm_head"].data_ptr(), lays)
        self.desc = desc
        self.handle = ssd_model_create(desc)

    def close(self):
        if self.handle is not None:
            ssd_model_destroy(self.handle)
            self.handle = None


class Sequence:
    """A sequence with its own KV pool and workspace (torch device tensors)."""

    def __init__(self, model, max_ctx, max_rows=64, max_draft=16, page_size=64, page_table=None, device="cuda",
                 stream=None):
        import numpy as np
        import torch
        self.model = model
        n_lpages = (max_ctx + page_size - 1) // page_size
        if page_table is None:
            page_table = np.arange(n_lpages, dtype=np.int32)
        page_table = np.asarray(page_table, dtype=np.int32)
        n_pages = int(page_table.max()) + 1
        self.kv = torch.empty(ssd_kv_pool_bytes(model.handle, n_pages, page_size), dtype=torch.uint8, device=device)
        self.max_ctx = n_lpages * page_size
        ws = ssd_workspace_bytes(model.handle, max_rows, max_draft, self.max_ctx)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=device)
        self.max_draft = max_draft
        self.stream = stream
        self.handle = ssd_seq_create(model.handle, self.kv, n_pages, page_size, page_table, self.ws, max_rows,
                                     max_draft, stream)
        V = model.vocab
        self.draft_tokens = torch.zeros(max_draft, dtype=torch.int32, device=device)
        self.draft_logits = torch.zeros(max_draft * V, dtype=torch.float32, device=device)
        self.verify_logits = torch.zeros((max_draft + 1) * V, dtype=torch.float32, device=device)
        self.n_drafted = torch.zeros(1, dtype=torch.int32, device=device)
        self.out_tokens = torch.zeros(max_draft + 1, dtype=torch.int32, device=device)
        self.n_out = torch.zeros(1, dtype=torch.int32, device=device)
        # draft trees: at most 15 leaves, 16 verify rows
        self.leaf_tokens = torch.zeros(16, dtype=torch.int32, device=device)
        self.leaf_depth = torch.zeros(16, dtype=torch.int32, device=device)
        self.n_leaves = torch.zeros(1, dtype=torch.int32, device=device)
        self.tree_logits = torch.zeros(16 * V, dtype=torch.float32, device=device)

    def close(self):
        if self.handle is not None:
            ssd_seq_destroy(self.handle)
            self.handle = None

    def ssd_iteration(self, skip_mask, exit_layer, d, conf_thresh=0.0, temperature=0.0, seed=0, reuse=True):
        """Enqueues draft -> verify -> accept -> commit (no host round trip)."""
        s = self.stream
        ssd_draft(self.handle, skip_mask, exit_layer, d, conf_thresh, temperature, seed, self.draft_tokens,
                  self.draft_logits, self.n_drafted, s)
        ssd_verify(self.handle, skip_mask, exit_layer, d, self.draft_tokens, self.n_drafted, reuse,
                   self.verify_logits, s)
        ssd_accept(self.handle, self.verify_logits, self.draft_logits, self.draft_tokens, self.n_drafted, d,
                   temperature, seed, self.out_tokens, self.n_out, s)
        ssd_commit(self.handle, self.out_tokens, self.n_out, s)

    def tree_iteration(self, skip_mask, exit_layer, d, rho, k_max, max_leaves, conf_thresh=0.0, reuse=True,
                       temperature=0.0, seed=0):
        """Enqueues draft -> leaves -> tree verify -> tree accept -> commit."""
        s = self.stream
        ssd_draft(self.handle, skip_mask, exit_layer, d, conf_thresh, temperature, seed, self.draft_tokens,
                  self.draft_logits, self.n_drafted, s)
        ssd_tree_candidates(self.handle, self.draft_logits, self.n_drafted, d, rho, k_max, max_leaves,
                            self.leaf_tokens, self.leaf_depth, self.n_leaves, temperature, seed, s)
        ssd_verify_tree(self.handle, skip_mask, exit_layer, d, self.draft_tokens, self.n_drafted, self.leaf_tokens,
                        self.leaf_depth, self.n_leaves, max_leaves, reuse, self.tree_logits, s)
        ssd_accept_tree(self.handle, self.tree_logits, self.draft_tokens, self.n_drafted, d, self.leaf_tokens,
                        self.leaf_depth, self.n_leaves, max_leaves, self.out_tokens, self.n_out, self.draft_logits,
                        temperature, seed, s)
        ssd_commit(self.handle, self.out_tokens, self.n_out, s)

    def generate_tree(self, prompt, n_gen, skip_mask=None, exit_layer=None, d=4, rho=0.9, k_max=4, max_leaves=3,
                      conf_thresh=0.0, reuse=True, temperature=0.0, seed=0):
        """Decoding with draft trees; returns (tokens[:n_gen], per-iteration (d', emitted) list)."""
        ssd_prefill(self.handle, prompt, temperature, seed, None, self.stream)
        stats = []
        st = ssd_read_state(self.handle, self.stream)
        while st.n_out < n_gen:
            self.tree_iteration(skip_mask, exit_layer, d, rho, k_max, max_leaves, conf_thresh, reuse, temperature,
                                seed)
            st = ssd_read_state(self.handle, self.stream)
            stats.append((st.last_n_drafted, st.last_n_emitted))
        return ssd_read_output(self.handle, n_gen, self.stream)[:n_gen], stats

    def generate_ssd(self, prompt, n_gen, skip_mask=None, exit_layer=None, d=4, conf_thresh=0.0, temperature=0.0,
                     seed=0, reuse=True, on_iteration=None):
        """Prefill, then SSD iterations until n_gen tokens are committed; returns
        (tokens[:n_gen], per-iteration (d', emitted) list)."""
        ssd_prefill(self.handle, prompt, temperature, seed, None, self.stream)
        stats = []
        st = ssd_read_state(self.handle, self.stream)
        while st.n_out < n_gen:
            self.ssd_iteration(skip_mask, exit_layer, d, conf_thresh, temperature, seed, reuse)
            st = ssd_read_state(self.handle, self.stream)
            stats.append((st.last_n_drafted, st.last_n_emitted))
            if on_iteration is not None:
                on_iteration(self, st)
        return ssd_read_output(self.handle, n_gen, self.stream)[:n_gen], stats

    def generate_ar(self, prompt, n_gen, temperature=0.0, seed=0):
        ssd_prefill(self.handle, prompt, temperature, seed, None, self.stream)
        for _ in range(n_gen - 1):
            ssd_decode_ar(self.handle, temperature, seed, None, self.stream)
        return ssd_read_output(self.handle, n_gen, self.stream)
