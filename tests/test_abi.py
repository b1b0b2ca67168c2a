"""The C-ABI library loads and exports every symbol the headers declare, and
host-checkable argument errors are rejected without touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("lmstep.h", "lmstep_kernels.h")]


def declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M):
            name = m.group(1)
            if name not in ("if", "while", "for", "sizeof"):
                names.append(name)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    so = os.path.join(ROOT, "scratch_decoder_only_amd", "liblmstep.so")
    if not os.path.exists(so):
        import importlib.util
        spec = importlib.util.spec_from_file_location("lm_build", os.path.join(ROOT, "scratch_decoder_only_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build(verbose=False)
    return ctypes.CDLL(so)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 25, names
    for n in ("model_create", "train_step", "forward_logits", "lmk_gemm", "lmk_attn_bwd"):
        assert n in names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_exposes_the_same_names(lib):
    import scratch_decoder_only_amd as sd
    for n in declared_functions():
        assert hasattr(sd.lib, n)


def _cfg(**kw):
    import scratch_decoder_only_amd as sd
    base = dict(vocab=257, d_model=128, n_heads=4, d_mlp=256, n_layers=3, max_seq=80, max_batch=4, precision=0,
                ln_eps=1e-5)
    base.update(kw)
    return sd.LmConfig(**base)


@pytest.mark.parametrize("bad", [dict(d_model=96), dict(n_heads=3), dict(n_heads=1), dict(d_mlp=100),
                                 dict(vocab=0), dict(max_seq=0), dict(precision=3), dict(d_model=2048, n_heads=32),
                                 dict(untied_head=2)])
def test_invalid_configs_are_rejected(lib, bad):
    import scratch_decoder_only_amd as sd
    cfg = _cfg(**bad)
    assert sd.lib.lm_workspace_bytes(ctypes.byref(cfg)) == 0
    h = ctypes.c_void_p()
    rc = sd.lib.model_create(ctypes.byref(cfg), ctypes.c_void_p(256), 1 << 30, None, ctypes.byref(h))
    assert rc in (sd.LM_ERR_SHAPE, sd.LM_ERR_UNSUPPORTED, sd.LM_ERR_ARG)
    assert sd.lib.lm_last_error()


def test_workspace_size_and_arena_checks(lib):
    import scratch_decoder_only_amd as sd
    cfg = _cfg()
    need = sd.lib.lm_workspace_bytes(ctypes.byref(cfg))
    assert need > 4 * 4 * 440832  # params, grads and both moments at least
    h = ctypes.c_void_p()
    assert sd.lib.model_create(ctypes.byref(cfg), None, need, None, ctypes.byref(h)) == sd.LM_ERR_ARG
    assert sd.lib.model_create(ctypes.byref(cfg), ctypes.c_void_p(256), need - 1, None, ctypes.byref(h)) == sd.LM_ERR_WORKSPACE
    assert b"too small" in sd.lib.lm_last_error()
    assert sd.lib.model_create(ctypes.byref(cfg), ctypes.c_void_p(258), need, None, ctypes.byref(h)) == sd.LM_ERR_WORKSPACE
    bf = _cfg(precision=1)
    assert sd.lib.lm_workspace_bytes(ctypes.byref(bf)) > 0
    assert sd.lib.lm_workspace_bytes(ctypes.byref(_cfg(precision=2))) == sd.lib.lm_workspace_bytes(ctypes.byref(bf))
    # a separate head adds head.w [V, C] and head.b [V] to each of the four
    # fp32 buffers
    un = _cfg(untied_head=1)
    assert sd.lib.lm_workspace_bytes(ctypes.byref(un)) >= need + 4 * 4 * (257 * 128 + 257)


def test_kernel_entry_points_reject_bad_shapes(lib):
    import scratch_decoder_only_amd as sd
    P = ctypes.c_void_p(256)
    # bf16 GEMM with a leading dimension that is not a multiple of 8
    assert sd.lib.lmk_gemm(1, 16, 16, 16, P, 12, 1, P, 16, 1, P, 16, 0, 1, None, None, 0, None, 0, 0, 0, None, 0, None) != 0
    # LayerNorm width must be a multiple of 128
    assert sd.lib.lmk_layernorm_fwd(0, P, P, P, 4, 96, 1e-5, P, P, P, None) != 0
    # attention head dim 48 is not supported
    assert sd.lib.lmk_attn_fwd(1, P, P, P, 1, 8, 2, 48, P, P, None) != 0
    # AdamW needs a multiple of 4 elements and step >= 1
    assert sd.lib.lmk_adamw(P, P, P, P, 6, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, P, P, None, 0, None) != 0
    assert sd.lib.lmk_adamw(P, P, P, P, 8, 1e-3, 0.9, 0.999, 1e-8, 0.0, 0, P, P, None, 0, None) != 0
    # the key-count arrays of the counting sort must be 16-byte aligned
    Q = ctypes.c_void_p(260)
    assert sd.lib.lmk_csr(P, 16, 64, Q, P, P, P, P, None) != 0
    assert sd.lib.lmk_csr(P, 16, 64, P, P, Q, P, P, None) != 0
    # 16-bit GEMM outputs are addressed with 32-bit offsets within a tile
    assert sd.lib.lmk_gemm(1, 16, 16, 16, P, 16, 1, P, 16, 1, P, 1 << 22, 0, 0, None, None, 0, None, 0, 0, 0,
                           None, 0, None) != 0
