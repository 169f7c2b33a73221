"""The C-ABI library loads and exports every symbol include/*.h declares; host-side
argument checks (no GPU needed: these calls touch no device)."""
import ctypes
import os
import re

import pytest

from self_speculative_layer_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"^\s*(?:int|const char\*)\s+(ssd_\w+)\s*\(", text, flags=re.M))
    return names


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    decl = declared_symbols()
    assert len(decl) >= 17
    for name in sorted(decl):
        assert hasattr(lib, name), name
    assert decl == set(B.EXPORTS)


def test_synth_device_library_exports():
    import synth
    lib = synth.dev_lib()
    for name in ("synth_fill_weight_dev", "synth_fill_tokens_dev"):
        assert hasattr(lib, name)


def _desc(**kw):
    base = dict(n_layers=2, d_model=128, n_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=256, vocab=100,
                rms_eps=1e-5, rope_theta=1e4, dtype=B.SSD_DTYPE_BF16)
    base.update(kw)
    lays = (B.ssd_layer_weights * base["n_layers"])()
    for l in range(base["n_layers"]):
        lays[l] = B.ssd_layer_weights(*([0x1000] * 6))
    d = B.ssd_model_desc(base["n_layers"], base["d_model"], base["n_heads"], base["n_kv_heads"], base["head_dim"],
                         base["ffn_dim"], base["vocab"], base["rms_eps"], base["rope_theta"], base["dtype"],
                         0x1000, 0x1000, 0x1000, lays)
    return d, lays


def test_model_create_validates_shapes():
    d, keep = _desc()
    m = B.ssd_model_create(d)
    assert B.ssd_kv_pool_bytes(m, 3, 64) == 3 * 2 * 2 * 2 * 64 * 64 * 2
    assert B.ssd_workspace_bytes(m, 64, 8, 512) > 0
    B.ssd_model_destroy(m)
    for kw, code in [(dict(head_dim=96), B.SSD_ERR_SHAPE), (dict(n_kv_heads=3), B.SSD_ERR_SHAPE),
                     (dict(d_model=100), B.SSD_ERR_SHAPE), (dict(vocab=0), B.SSD_ERR_ARG),
                     (dict(dtype=7), B.SSD_ERR_ARG)]:
        d, keep = _desc(**kw)
        with pytest.raises(B.SSDError) as e:
            B.ssd_model_create(d)
        assert e.value.code == code
    d, keep = _desc(dtype=B.SSD_DTYPE_F32, d_model=100)       # fp32 path takes any width
    B.ssd_model_destroy(B.ssd_model_create(d))


def test_workspace_limits():
    d, keep = _desc()
    m = B.ssd_model_create(d)
    with pytest.raises(B.SSDError):
        B.ssd_workspace_bytes(m, 0, 8, 512)
    with pytest.raises(B.SSDError):
        B.ssd_workspace_bytes(m, 64, 33, 512)
    # up to 4096 rows (scoring passes); the split-key attention's partial buffer stays at 1024 rows
    assert B.ssd_workspace_bytes(m, 4096, 8, 512) > B.ssd_workspace_bytes(m, 1024, 8, 512)
    with pytest.raises(B.SSDError):
        B.ssd_workspace_bytes(m, 4097, 8, 512)
    B.ssd_model_destroy(m)


def test_null_arguments_are_errors():
    lib = B.lib()
    assert lib.ssd_model_create(None, None) == B.SSD_ERR_ARG
    assert b"null" in lib.ssd_last_error()
    assert lib.ssd_draft(None, None, 1, 4, 0.0, 0.0, 0, None, None, None, None) == B.SSD_ERR_ARG
    assert lib.ssd_accept(None, None, None, None, None, 4, 0.0, 0, None, None, None) == B.SSD_ERR_ARG


def test_accept_noalloc_rejects_bad_arguments_on_the_host():
    """The allocation-free acceptance checks its arguments before touching the device: null pointers,
    non-positive sizes and a bad temperature are SSD_ERR_ARG, a chain longer than its scratch array
    SSD_ERR_CAPACITY."""
    L = B.lib()
    p = ctypes.c_void_p(0x1000)
    args = lambda d=4, vocab=100, T=1.0, ptr=p: (ptr, p, p, p, d, vocab, T, 3, 1, p, p, None)
    assert L.ssd_accept_noalloc(*args(ptr=None)) == B.SSD_ERR_ARG
    assert L.ssd_accept_noalloc(*args(d=0)) == B.SSD_ERR_ARG
    assert L.ssd_accept_noalloc(*args(vocab=0)) == B.SSD_ERR_ARG
    assert L.ssd_accept_noalloc(*args(T=-1.0)) == B.SSD_ERR_ARG
    assert L.ssd_accept_noalloc(*args(T=float("nan"))) == B.SSD_ERR_ARG
    assert L.ssd_accept_noalloc(*args(d=33)) == B.SSD_ERR_CAPACITY
    assert b"SSD_ACCEPT_NOALLOC_MAX_DRAFT" in L.ssd_last_error()


def test_unknown_handles_are_rejected_on_the_host():
    """Handles the library did not create (or has destroyed) are refused before any device work."""
    L = B.lib()
    bogus = ctypes.c_void_p(0x12345678)
    st = B.ssd_state()
    assert L.ssd_read_state(bogus, ctypes.byref(st), None) == B.SSD_ERR_ARG
    assert b"live sequence" in L.ssd_last_error()
    assert L.ssd_seq_destroy(bogus) == B.SSD_ERR_ARG
    assert L.ssd_commit(bogus, bogus, bogus, None) == B.SSD_ERR_ARG
    assert L.ssd_model_destroy(bogus) == B.SSD_ERR_ARG
    assert b"live model" in L.ssd_last_error()
    size = ctypes.c_size_t()
    assert L.ssd_workspace_bytes(bogus, 16, 4, 64, ctypes.byref(size)) == B.SSD_ERR_ARG
