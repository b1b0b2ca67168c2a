"""Python binding of the gfx950 training-step library (liblmstep.so).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch provides device memory (the arena and the input/output
tensors) and the current stream. Importing fails loudly when the library has
not been built; there is no CPU fallback.

The C ABI is declared in include/lmstep.h (model level) and
include/lmstep_kernels.h (one kernel at a time).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblmstep.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()' or python scratch_decoder_only_amd/build.py)")

# torch first: its HIP runtime and the system's share the soname
# libamdhip64.so.7, so whichever loads first serves both. Loaded first, the
# system runtime leaves torch without devices; loaded after torch, the library
# runs on torch's runtime, as its streams and allocations require.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

c_int, c_int64, c_float, c_void_p, c_size_t = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
c_char_p, c_double = ctypes.c_char_p, ctypes.c_double

LM_OK, LM_ERR_ARG, LM_ERR_WORKSPACE, LM_ERR_SHAPE, LM_ERR_HIP, LM_ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5
LM_PARAMS, LM_GRADS, LM_ADAM_M, LM_ADAM_V = 0, 1, 2, 3
EPI_STORE, EPI_RESID, EPI_GELU, EPI_DGELU = 0, 1, 2, 3
PRECISIONS = {"fp32": 0, "bf16": 1, "fp16": 2}


class LmConfig(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_mlp", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("max_batch", ctypes.c_int32), ("precision", ctypes.c_int32), ("ln_eps", ctypes.c_float),
                ("untied_head", ctypes.c_int32)]


class LmLossScaler(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("growth", ctypes.c_float), ("backoff", ctypes.c_float),
                ("interval", ctypes.c_int32), ("good_steps", ctypes.c_int32)]


class LmOptim(ctypes.Structure):
    _fields_ = [("lr", c_float), ("beta1", c_float), ("beta2", c_float), ("eps", c_float),
                ("weight_decay", c_float), ("clip_norm", c_float), ("step", ctypes.c_int32)]


class LmTensorInfo(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("offset", c_int64), ("rows", c_int64), ("cols", c_int64)]


class LmProfileEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 40), ("launches", c_int64), ("ms", c_double), ("flops", c_double),
                ("bytes", c_double)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_sig("lm_workspace_bytes", c_size_t, [ctypes.POINTER(LmConfig)])
_sig("model_create", c_int, [ctypes.POINTER(LmConfig), c_void_p, c_size_t, c_void_p, ctypes.POINTER(c_void_p)])
_sig("model_destroy", None, [c_void_p])
_sig("model_param_table", c_int, [c_void_p, ctypes.POINTER(LmTensorInfo), ctypes.POINTER(ctypes.c_int32),
                                  ctypes.POINTER(c_int64)])
_sig("model_set", c_int, [c_void_p, c_int, c_void_p, c_int, c_void_p])
_sig("model_get", c_int, [c_void_p, c_int, c_void_p, c_int, c_void_p])
_sig("train_step", c_int, [c_void_p, c_void_p, c_void_p, c_void_p, ctypes.c_int32, ctypes.c_int32,
                           ctypes.POINTER(LmOptim), c_void_p, c_void_p])
_sig("forward_logits", c_int, [c_void_p, c_void_p, c_void_p, ctypes.c_int32, ctypes.c_int32, c_void_p, c_void_p])
_sig("lm_last_error", c_char_p, [])
_sig("model_config", c_int, [c_void_p, ctypes.POINTER(LmConfig)])
_sig("lm_lr_schedule", ctypes.c_float, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float])
_sig("model_save", c_int, [c_void_p, c_char_p, ctypes.c_int32, c_void_p])
_sig("model_load", c_int, [c_void_p, c_char_p, ctypes.POINTER(ctypes.c_int32), c_void_p])
_sig("lm_kv_cache_bytes", c_size_t, [ctypes.POINTER(LmConfig), ctypes.c_int32])
_sig("model_prefill", c_int, [c_void_p, c_void_p, ctypes.c_int32, ctypes.c_int32, c_void_p, c_void_p, c_void_p])
_sig("model_decode", c_int, [c_void_p, c_void_p, ctypes.c_int32, ctypes.c_int32, c_void_p, c_void_p, c_void_p])
_sig("model_decode_at", c_int, [c_void_p, c_void_p, ctypes.c_int32, c_void_p, c_void_p, c_void_p, c_void_p])
_sig("sample_tokens", c_int, [c_void_p, ctypes.c_int32, ctypes.c_int32, c_int64, ctypes.c_float, ctypes.c_int32,
                              c_void_p, c_void_p, c_void_p])
_sig("model_set_loss_scaler", c_int, [c_void_p, ctypes.POINTER(LmLossScaler), c_void_p])
_sig("model_get_loss_scaler", c_int, [c_void_p, ctypes.POINTER(LmLossScaler), c_void_p])
_sig("model_profile_enable", c_int, [c_void_p, c_int])
_sig("model_profile_read", c_int, [c_void_p, ctypes.POINTER(LmProfileEntry), ctypes.c_int32,
                                   ctypes.POINTER(ctypes.c_int32), c_int])

_P = c_void_p
_sig("lmk_gemm", c_int, [c_int, c_int, c_int, c_int, _P, c_int64, c_int, _P, c_int64, c_int, _P, c_int64, c_int, c_int,
                         _P, _P, c_int64, _P, c_int64, c_int, c_int, _P, c_int64, _P])
_sig("lmk_gemm_cfg", c_int, [c_int, c_int, c_int, c_int, c_int, _P, c_int64, c_int, _P, c_int64, c_int, _P, c_int64,
                             c_int, c_int, _P, _P, c_int64, _P, c_int64, c_int, c_int, _P, c_int64, _P])
_sig("lmk_gemm_group_table_bytes", c_int64, [c_int])
_PI, _PV, _PL = ctypes.POINTER(c_int), ctypes.POINTER(c_void_p), ctypes.POINTER(c_int64)
_sig("lmk_gemm_group", c_int, [c_int, c_int, _PI, _PV, _PL, _PV, _PL, _PV, _PL, _P, c_int64, _P])
_sig("lmk_layernorm_fwd", c_int, [c_int, _P, _P, _P, c_int, c_int, c_float, _P, _P, _P, _P])
_sig("lmk_layernorm_bwd", c_int, [c_int, _P, _P, _P, _P, _P, c_int, c_int, _P, _P, _P, _P, _P, _P, _P, _P])
_sig("lmk_layernorm_bwd_ws_floats", c_int64, [c_int, c_int])
_sig("lmk_colsum", c_int, [c_int, _P, c_int64, c_int, c_int, _P, _P, _P])
_sig("lmk_colsum_ws_floats", c_int64, [c_int, c_int])
_sig("lmk_index_layout", c_int, [_P, c_int, c_int, _P, _P, _P, _P, _P])
_sig("lmk_embed_fwd", c_int, [_P, _P, _P, _P, c_int, c_int, c_int, _P, _P, _P])
_sig("lmk_attn_fwd", c_int, [c_int, _P, _P, _P, c_int, c_int, c_int, c_int, _P, _P, _P])
_sig("lmk_attn_bwd", c_int, [c_int, _P, _P, _P, _P, _P, _P, c_int, c_int, c_int, c_int, _P, _P, _P])
_sig("lmk_xent", c_int, [c_int, _P, c_int64, c_int, c_int, _P, _P, _P, _P, _P, _P, _P])
_sig("lmk_xent_noalloc", c_int, [c_int, _P, c_int64, c_int, c_int, _P, _P, _P, _P, _P])
_sig("lmk_csr", c_int, [_P, c_int, c_int, _P, _P, _P, _P, _P, _P])
_sig("lmk_segment_sum", c_int, [_P, c_int, c_int, c_int, _P, _P, _P, _P, _P, _P, c_int, _P])
_sig("lmk_segment_sum_ws_floats", c_int64, [c_int, c_int, c_int])
_sig("lmk_csr_ws_ints", c_int64, [c_int, c_int])
_sig("lmk_grad_norm", c_int, [_P, c_int64, c_float, _P, _P, _P, _P, c_float, c_float, c_int, _P])
_sig("lmk_adamw", c_int, [_P, _P, _P, _P, c_int64, c_float, c_float, c_float, c_float, c_float, c_int, _P, _P, _P, c_int,
                          _P])

lib = _lib


class LmError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != LM_OK:
        msg = _lib.lm_last_error()
        raise LmError(f"{what} failed with status {rc}: {msg.decode() if msg else ''}")


def _kcheck(rc: int, what: str):
    if rc != 0:
        raise LmError(f"{what}: the kernel rejected its arguments (rc {rc})")


def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _need(t, name: str, dtype, device=None, shape=None, min_numel: int = 0, min_bytes: int = 0):
    """Checks a tensor argument before its pointer crosses the C ABI: a
    contiguous CUDA tensor of `dtype` on `device`, of `shape` and at least
    `min_numel` elements / `min_bytes` bytes (the kernels read and write by
    raw pointer, so a wrong dtype, device or size would be read as garbage or
    written out of bounds)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise LmError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise LmError(f"{name} must be a CUDA (HIP) device tensor, got one on {t.device}")
    if device is not None and t.device != device:
        raise LmError(f"{name} is on {t.device} but the model is on {device}")
    if dtype is not None and t.dtype != dtype:
        raise LmError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise LmError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise LmError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.numel() < min_numel:
        raise LmError(f"{name} needs at least {min_numel} elements, got {t.numel()}")
    if t.numel() * t.element_size() < min_bytes:
        raise LmError(f"{name} needs at least {min_bytes} bytes, got {t.numel() * t.element_size()}")
    return t


class Model:
    """One model instance on the current CUDA (HIP) device.

    dims: object with vocab, d_model, n_heads, d_mlp, n_layers, max_seq,
    ln_eps and optionally untied_head (e.g. a synth.ModelShape); precision
    "fp32", "bf16" or "fp16" (fp16 operands with dynamic loss scaling).
    """

    def __init__(self, dims, max_batch: int, precision: Optional[str] = None, device="cuda"):
        torch = _torch()
        prec = precision or getattr(dims, "precision", "bf16")
        self.cfg = LmConfig(dims.vocab, dims.d_model, dims.n_heads, dims.d_mlp, dims.n_layers, dims.max_seq,
                            max_batch, PRECISIONS[prec], float(getattr(dims, "ln_eps", 1e-5)),
                            1 if getattr(dims, "untied_head", False) else 0)
        self.precision = prec
        nbytes = _lib.lm_workspace_bytes(ctypes.byref(self.cfg))
        if nbytes == 0:
            _check(LM_ERR_SHAPE, "lm_workspace_bytes")
        self.arena = torch.empty(int(nbytes), dtype=torch.uint8, device=device)
        # held by the instance: at interpreter exit the module's globals may
        # already be gone when __del__ runs
        self._destroy = _lib.model_destroy
        self._h = c_void_p()
        _check(_lib.model_create(ctypes.byref(self.cfg), _ptr(self.arena), nbytes, _stream(), ctypes.byref(self._h)),
               "model_create")
        n = ctypes.c_int32(0)
        total = c_int64(0)
        _check(_lib.model_param_table(self._h, None, ctypes.byref(n), ctypes.byref(total)), "model_param_table")
        arr = (LmTensorInfo * n.value)()
        _check(_lib.model_param_table(self._h, arr, ctypes.byref(n), ctypes.byref(total)), "model_param_table")
        self.table: List[Tuple[str, int, int, int]] = [(e.name.decode(), e.offset, e.rows, e.cols) for e in arr]
        self.total = total.value
        self.stats = torch.zeros(4, dtype=torch.float32, device=device)

    def __del__(self):
        h, destroy = getattr(self, "_h", None), getattr(self, "_destroy", None)
        if h is not None and h.value and destroy is not None:
            destroy(h)
            self._h = None

    # ---- flat buffers <-> named tensors
    def flatten(self, named: Dict[str, np.ndarray]) -> np.ndarray:
        flat = np.zeros(self.total, np.float32)
        for name, off, rows, cols in self.table:
            a = np.asarray(named[name], dtype=np.float32).reshape(-1)
            assert a.size == rows * cols, (name, a.shape, rows, cols)
            flat[off:off + a.size] = a
        return flat

    def unflatten(self, flat: np.ndarray) -> Dict[str, np.ndarray]:
        out = {}
        for name, off, rows, cols in self.table:
            a = flat[off:off + rows * cols]
            out[name] = a.reshape(rows, cols) if cols > 1 else a.copy()
        return out

    def set(self, which: int, named: Dict[str, np.ndarray]):
        flat = np.ascontiguousarray(self.flatten(named))
        _check(_lib.model_set(self._h, which, flat.ctypes.data, 0, _stream()), "model_set")

    def _tokens(self, t, name="tokens", ndim=2):
        torch = _torch()
        if not isinstance(t, torch.Tensor) or t.dim() != ndim:
            raise LmError(f"{name} must be a {ndim}-D int32 CUDA tensor")
        return _need(t, name, torch.int32, self.stats.device)

    def set_flat_device(self, which: int, t):
        _need(t, "src", _torch().float32, self.stats.device, min_numel=self.total)
        _check(_lib.model_set(self._h, which, _ptr(t), 1, _stream()), "model_set")

    def get(self, which: int) -> Dict[str, np.ndarray]:
        flat = np.zeros(self.total, np.float32)
        _check(_lib.model_get(self._h, which, flat.ctypes.data, 0, _stream()), "model_get")
        return self.unflatten(flat)

    def get_flat(self, which: int) -> np.ndarray:
        flat = np.zeros(self.total, np.float32)
        _check(_lib.model_get(self._h, which, flat.ctypes.data, 0, _stream()), "model_get")
        return flat

    def get_flat_device(self, which: int, out):
        _need(out, "out", _torch().float32, self.stats.device, min_numel=self.total)
        _check(_lib.model_get(self._h, which, _ptr(out), 1, _stream()), "model_get")

    # ---- the step
    def train_step(self, tokens, targets, doc_ids=None, *, lr, step, beta1=0.9, beta2=0.999, eps=1e-8,
                   weight_decay=0.0, clip=1.0, stats=None):
        torch = _torch()
        B, T = self._tokens(tokens).shape
        _need(targets, "targets", torch.int32, self.stats.device, shape=(B, T))
        if doc_ids is not None:
            _need(doc_ids, "doc_ids", torch.int32, self.stats.device, shape=(B, T))
        opt = LmOptim(lr, beta1, beta2, eps, weight_decay, clip, step)
        st = self.stats if stats is None else _need(stats, "stats", torch.float32, self.stats.device, min_numel=4)
        _check(_lib.train_step(self._h, _ptr(tokens), _ptr(targets), _ptr(doc_ids), B, T, ctypes.byref(opt),
                               _ptr(st), _stream()), "train_step")
        return st

    def forward_logits(self, tokens, doc_ids=None, out=None):
        torch = _torch()
        B, T = self._tokens(tokens).shape
        if doc_ids is not None:
            _need(doc_ids, "doc_ids", torch.int32, self.stats.device, shape=(B, T))
        if out is None:
            out = torch.empty((B, T, self.cfg.vocab), dtype=torch.float32, device=tokens.device)
        _need(out, "out", torch.float32, self.stats.device, min_numel=B * T * self.cfg.vocab)
        _check(_lib.forward_logits(self._h, _ptr(tokens), _ptr(doc_ids), B, T, _ptr(out), _stream()),
               "forward_logits")
        return out

    # ---- generation with a key/value cache
    def kv_cache(self, batch: int):
        """Device buffer for the key/value cache of `batch` rows."""
        torch = _torch()
        n = _lib.lm_kv_cache_bytes(ctypes.byref(self.cfg), int(batch))
        if n == 0:
            _check(LM_ERR_SHAPE, "lm_kv_cache_bytes")
        return torch.empty(int(n), dtype=torch.uint8, device=self.stats.device)

    def _cache(self, cache, batch: int):
        n = _lib.lm_kv_cache_bytes(ctypes.byref(self.cfg), int(batch))
        if n == 0:
            _check(LM_ERR_SHAPE, "lm_kv_cache_bytes")
        return _need(cache, "cache", None, self.stats.device, min_bytes=int(n))

    def prefill(self, tokens, cache, out=None):
        """Forward over tokens [B, T] (filling cache positions < T); returns the
        logits [B, vocab] of each row's last position."""
        torch = _torch()
        B, T = self._tokens(tokens).shape
        self._cache(cache, B)
        if out is None:
            out = torch.empty((B, self.cfg.vocab), dtype=torch.float32, device=tokens.device)
        _need(out, "out", torch.float32, self.stats.device, min_numel=B * self.cfg.vocab)
        _check(_lib.model_prefill(self._h, _ptr(tokens), B, T, _ptr(cache), _ptr(out), _stream()), "model_prefill")
        return out

    def decode(self, tokens, pos: int, cache, out=None):
        """One new token per row (tokens [B]) at position pos; returns its logits [B, vocab]."""
        torch = _torch()
        B = self._tokens(tokens, ndim=1).shape[0]
        self._cache(cache, B)
        if out is None:
            out = torch.empty((B, self.cfg.vocab), dtype=torch.float32, device=tokens.device)
        _need(out, "out", torch.float32, self.stats.device, min_numel=B * self.cfg.vocab)
        _check(_lib.model_decode(self._h, _ptr(tokens), B, int(pos), _ptr(cache), _ptr(out), _stream()),
               "model_decode")
        return out

    def decode_at(self, tokens, pos, cache, out=None):
        """decode with the position in device memory (pos: int32 CUDA tensor of
        one element, read when the kernels run; clamped to [1, max_seq))."""
        torch = _torch()
        B = self._tokens(tokens, ndim=1).shape[0]
        self._cache(cache, B)
        _need(pos, "pos", torch.int32, self.stats.device, min_numel=1)
        if out is None:
            out = torch.empty((B, self.cfg.vocab), dtype=torch.float32, device=tokens.device)
        _need(out, "out", torch.float32, self.stats.device, min_numel=B * self.cfg.vocab)
        _check(_lib.model_decode_at(self._h, _ptr(tokens), B, _ptr(pos), _ptr(cache), _ptr(out), _stream()),
               "model_decode_at")
        return out

    # ---- checkpoints
    # ---- dynamic loss scale (precision "fp16")
    def loss_scaler(self) -> Dict[str, float]:
        ls = LmLossScaler()
        _check(_lib.model_get_loss_scaler(self._h, ctypes.byref(ls), _stream()), "model_get_loss_scaler")
        return {"scale": ls.scale, "growth": ls.growth, "backoff": ls.backoff, "interval": ls.interval,
                "good_steps": ls.good_steps}

    def set_loss_scaler(self, scale=65536.0, growth=2.0, backoff=0.5, interval=2000, good_steps=0):
        ls = LmLossScaler(scale, growth, backoff, interval, good_steps)
        _check(_lib.model_set_loss_scaler(self._h, ctypes.byref(ls), _stream()), "model_set_loss_scaler")

    def save(self, path: str, step: int):
        """Parameters and Adam moments to a checkpoint file (safetensors layout)."""
        _check(_lib.model_save(self._h, os.fsencode(path), int(step), _stream()), "model_save")

    def load(self, path: str) -> int:
        """Restores parameters and moments from a checkpoint; returns its step."""
        st = ctypes.c_int32(0)
        _check(_lib.model_load(self._h, os.fsencode(path), ctypes.byref(st), _stream()), "model_load")
        return st.value

    # ---- measurement hooks
    def profile(self, enable: bool):
        _check(_lib.model_profile_enable(self._h, 1 if enable else 0), "model_profile_enable")

    def profile_read(self, reset=True) -> Dict[str, dict]:
        n = ctypes.c_int32(0)
        _check(_lib.model_profile_read(self._h, None, 0, ctypes.byref(n), 0), "model_profile_read")
        arr = (LmProfileEntry * max(1, n.value))()
        _check(_lib.model_profile_read(self._h, arr, n.value, ctypes.byref(n), 1 if reset else 0),
               "model_profile_read")
        return {e.name.decode(): {"launches": e.launches, "ms": e.ms, "flops": e.flops, "bytes": e.bytes}
                for e in arr[:n.value]}


# ------------------------------------------------------------ training driver

def lr_schedule(step: int, warmup_steps: int, total_steps: int, lr_max: float, lr_min: float) -> float:
    """Learning rate of 1-based step: linear warm-up, then a half cosine down
    to lr_min at total_steps (the library's lm_lr_schedule)."""
    return float(_lib.lm_lr_schedule(int(step), int(warmup_steps), int(total_steps), float(lr_max), float(lr_min)))


def train(model: "Model", batch, steps: int, *, lr_max: float, lr_min: float = 0.0, warmup_steps: int = 0,
          total_steps: Optional[int] = None, start_step: int = 1, save_every: int = 0, ckpt_path=None, **opt):
    """Runs `steps` training steps from `start_step` on the model's stream.

    batch: (tokens, targets, doc_ids) device tensors, or a callable step ->
    such a tuple. The learning rate follows lr_schedule(step, warmup_steps,
    total_steps or the last step, lr_max, lr_min); every `save_every` steps the
    model is saved to ckpt_path. opt: beta1, beta2, eps, weight_decay, clip.
    Returns the per-step losses as a device tensor (no host synchronisation).
    """
    torch = _torch()
    last = start_step + steps - 1
    total = last if total_steps is None else total_steps
    losses = torch.zeros(steps, dtype=torch.float32, device=model.stats.device)
    for i in range(steps):
        step = start_step + i
        tok, tgt, doc = batch(step) if callable(batch) else batch
        lr = lr_schedule(step, warmup_steps, total, lr_max, lr_min)
        model.train_step(tok, tgt, doc, lr=lr, step=step, **opt)
        losses[i:i + 1].copy_(model.stats[0:1])
        if save_every and ckpt_path and step % save_every == 0:
            model.save(ckpt_path, step)
    return losses


# ------------------------------------------------------------------ generation

def sample_tokens(logits, temperature: float = 0.0, top_k: int = 0, uniforms=None, out=None):
    """Next token of each row of `logits` (a 2-D fp32 CUDA tensor whose rows
    may be strided): greedy for temperature <= 0, else top-k sampling that
    picks with the given per-row uniforms in [0, 1) (a CUDA fp32 tensor)."""
    torch = _torch()
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2 or not logits.is_cuda:
        raise LmError("logits must be a 2-D CUDA tensor")
    rows, vocab = logits.shape
    if logits.dtype != torch.float32 or logits.stride(1) != 1 or logits.stride(0) < vocab:
        raise LmError("logits must be float32 with contiguous rows")
    if temperature > 0:
        _need(uniforms, "uniforms", torch.float32, logits.device, min_numel=rows)
    if out is None:
        out = torch.empty(rows, dtype=torch.int32, device=logits.device)
    _need(out, "out", torch.int32, logits.device, min_numel=rows)
    _check(_lib.sample_tokens(_ptr(logits), rows, vocab, logits.stride(0), float(temperature), int(top_k),
                              _ptr(uniforms), _ptr(out), _stream()), "sample_tokens")
    return out


class DecodeGraph:
    """One decode step of `model` on `cache` (batch rows), captured once as a
    HIP graph and replayed per token: step(tokens, pos) copies the tokens into
    the graph's input, writes pos to its device position and replays; the
    logits land in the graph's output [batch, vocab] (returned, overwritten
    by the next step). The first step runs eagerly and also warms the path
    up; the graph is captured right after it."""

    def __init__(self, model: "Model", cache, batch: int):
        torch = _torch()
        dev = cache.device
        self.model, self.cache = model, cache
        self.tok = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.pos = torch.ones(1, dtype=torch.int32, device=dev)
        self.out = torch.empty((batch, model.cfg.vocab), dtype=torch.float32, device=dev)
        self.graph = None

    def step(self, tokens, pos: int):
        torch = _torch()
        self.tok.copy_(tokens)
        self.pos.fill_(int(pos))
        if self.graph is None:
            self.model.decode_at(self.tok, self.pos, self.cache, out=self.out)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.model.decode_at(self.tok, self.pos, self.cache, out=self.out)
            self.graph = g
        else:
            self.graph.replay()
        return self.out


def generate(model: "Model", prompt, n_new: int, *, temperature: float = 0.0, top_k: int = 0, seed: int = 0,
             kv_cache: bool = True, graph: bool = False):
    """Extends each row of `prompt` ([B, T0] int32 CUDA tensor) by n_new tokens.

    kv_cache=True: one prefill over the prompt, then one decode step per new
    token against the key/value cache (graph=True: the decode step replayed
    from a captured HIP graph, DecodeGraph). kv_cache=False: forward_logits
    over the whole sequence so far for every new token. Either way sample_tokens picks
    the token from the last position's logits; uniforms for sampling are drawn
    on the host from numpy's PCG64(seed), one per row and step, and passed in.
    Returns the [B, T0 + n_new] token tensor."""
    torch = _torch()
    B, T0 = prompt.shape
    if T0 + n_new > model.cfg.max_seq:
        raise LmError("prompt plus new tokens exceed max_seq")
    toks = torch.zeros((B, T0 + n_new), dtype=torch.int32, device=prompt.device)
    toks[:, :T0] = prompt
    rng = np.random.Generator(np.random.PCG64(seed))
    cache = model.kv_cache(B) if kv_cache and n_new > 0 else None
    dg = DecodeGraph(model, cache, B) if cache is not None and graph else None
    for i in range(n_new):
        T = T0 + i
        if cache is None:
            last = model.forward_logits(toks[:, :T].contiguous())[:, T - 1, :]
        elif i == 0:
            last = model.prefill(toks[:, :T].contiguous(), cache)
        elif dg is not None:
            last = dg.step(toks[:, T - 1], T - 1)
        else:
            last = model.decode(toks[:, T - 1].contiguous(), T - 1, cache)
        u = None
        if temperature > 0:
            u = torch.from_numpy(rng.random(B).astype(np.float32)).to(prompt.device)
        toks[:, T] = sample_tokens(last, temperature, top_k, u)
    return toks


# --------------------------------------------------------------- kernel level
# Thin wrappers of include/lmstep_kernels.h for per-kernel parity tests; all
# tensors are torch CUDA tensors.

def gemm(precision, M, N, K, A, lda, a_kc, B, ldb, b_kc, C, ldc, epi=EPI_STORE, c_f32=False, bias=None, R=None,
         ldr=0, aux=None, ld_aux=0, force_split=0, M_out=0, ws=None, cfg=0):
    rc = _lib.lmk_gemm_cfg(int(cfg), precision, M, N, K, _ptr(A), lda, int(a_kc), _ptr(B), ldb, int(b_kc), _ptr(C), ldc, epi,
                       int(c_f32), _ptr(bias), _ptr(R), ldr, _ptr(aux), ld_aux, force_split, M_out, _ptr(ws),
                       0 if ws is None else ws.numel(), _stream())
    _kcheck(rc, "lmk_gemm")


def gemm_group_table_bytes(n):
    return _lib.lmk_gemm_group_table_bytes(n)


def gemm_group(precision, problems, table):
    """Weight gradients of several layers in one launch: problems is a list of
    (M, N, K, A, lda, B, ldb, C, ldc), C[r, c] = sum_k A[k, r] B[k, c] (fp32 C)."""
    n = len(problems)
    mnk = (ctypes.c_int * (3 * n))(*[int(v) for p in problems for v in p[:3]])
    As = (c_void_p * n)(*[_ptr(p[3]) for p in problems])
    ldas = (c_int64 * n)(*[int(p[4]) for p in problems])
    Bs = (c_void_p * n)(*[_ptr(p[5]) for p in problems])
    ldbs = (c_int64 * n)(*[int(p[6]) for p in problems])
    Cs = (c_void_p * n)(*[_ptr(p[7]) for p in problems])
    ldcs = (c_int64 * n)(*[int(p[8]) for p in problems])
    rc = _lib.lmk_gemm_group(precision, n, mnk, As, ldas, Bs, ldbs, Cs, ldcs, _ptr(table), table.numel() *
                             table.element_size(), _stream())
    _kcheck(rc, "lmk_gemm_group")


def layernorm_fwd(precision, x, g, b, eps, y, mu, rstd):
    M, C = x.shape
    _kcheck(_lib.lmk_layernorm_fwd(precision, _ptr(x), _ptr(g), _ptr(b), M, C, eps, _ptr(y), _ptr(mu), _ptr(rstd),
                                   _stream()), "lmk_layernorm_fwd")


def layernorm_bwd_ws_floats(M, C):
    return _lib.lmk_layernorm_bwd_ws_floats(M, C)


def layernorm_bwd(precision, dy, x, mu, rstd, g, g_in, g_out, g_act, dgamma, dbeta, ws, dsum=None):
    M, C = x.shape
    _kcheck(_lib.lmk_layernorm_bwd(precision, _ptr(dy), _ptr(x), _ptr(mu), _ptr(rstd), _ptr(g), M, C, _ptr(g_in),
                                   _ptr(g_out), _ptr(g_act), _ptr(dgamma), _ptr(dbeta), _ptr(dsum), _ptr(ws),
                                   _stream()),
            "lmk_layernorm_bwd")


def colsum_ws_floats(M, N):
    return _lib.lmk_colsum_ws_floats(M, N)


def colsum(precision_of_a, a, lda, M, N, out, ws):
    _kcheck(_lib.lmk_colsum(precision_of_a, _ptr(a), lda, M, N, _ptr(out), _ptr(ws), _stream()), "lmk_colsum")


def index_layout(doc, B, T, start, end, pos, flags):
    _kcheck(_lib.lmk_index_layout(_ptr(doc), B, T, _ptr(start), _ptr(end), _ptr(pos), _ptr(flags), _stream()),
            "lmk_index_layout")


def embed_fwd(tok, pos, wte, wpe, x, flags):
    M = tok.numel()
    V, C = wte.shape
    _kcheck(_lib.lmk_embed_fwd(_ptr(tok), _ptr(pos), _ptr(wte), _ptr(wpe), M, C, V, _ptr(x), _ptr(flags), _stream()),
            "lmk_embed_fwd")


def attn_fwd(precision, qkv, start, end, B, T, H, D, o, lse):
    _kcheck(_lib.lmk_attn_fwd(precision, _ptr(qkv), _ptr(start), _ptr(end), B, T, H, D, _ptr(o), _ptr(lse),
                              _stream()), "lmk_attn_fwd")


def attn_bwd(precision, qkv, o, lse, dout, start, end, B, T, H, D, delta, dqkv):
    _kcheck(_lib.lmk_attn_bwd(precision, _ptr(qkv), _ptr(o), _ptr(lse), _ptr(dout), _ptr(start), _ptr(end), B, T, H,
                              D, _ptr(delta), _ptr(dqkv), _stream()), "lmk_attn_bwd")


def xent(precision, z, ldz, M, V, tgt, loss, ws_n, ws_rows, flags, loss_scale=None):
    _kcheck(_lib.lmk_xent(precision, _ptr(z), ldz, M, V, _ptr(tgt), _ptr(loss), _ptr(ws_n), _ptr(ws_rows),
                          _ptr(flags), _ptr(loss_scale), _stream()), "lmk_xent")


def xent_noalloc(precision, z, ldz, M, V, tgt, loss, flags, loss_scale=None):
    """lmk_xent with the library's static scratch (no workspace arguments)."""
    _kcheck(_lib.lmk_xent_noalloc(precision, _ptr(z), ldz, M, V, _ptr(tgt), _ptr(loss), _ptr(flags),
                                  _ptr(loss_scale), _stream()), "lmk_xent_noalloc")


def csr(keys, M, nkeys, counts, offsets, chunk_base, perm, rank):
    _kcheck(_lib.lmk_csr(_ptr(keys), M, nkeys, _ptr(counts), _ptr(offsets), _ptr(chunk_base), _ptr(perm),
                         _ptr(rank), _stream()), "lmk_csr")


def csr_ws_ints(M, nkeys):
    return _lib.lmk_csr_ws_ints(M, nkeys)


def segment_sum_ws_floats(M, nkeys, C):
    return _lib.lmk_segment_sum_ws_floats(M, nkeys, C)


def segment_sum(dx, M, C, nkeys, counts, offsets, chunk_base, perm, partial, dst, accumulate):
    _kcheck(_lib.lmk_segment_sum(_ptr(dx), M, C, nkeys, _ptr(counts), _ptr(offsets), _ptr(chunk_base), _ptr(perm),
                                 _ptr(partial), _ptr(dst), int(accumulate), _stream()), "lmk_segment_sum")


def grad_norm(g, clip, part, norm_scale, flags, scale_state=None, growth=2.0, backoff=0.5, interval=2000):
    _kcheck(_lib.lmk_grad_norm(_ptr(g), g.numel(), clip, _ptr(part), _ptr(norm_scale), _ptr(flags), _ptr(scale_state),
                               growth, backoff, interval, _stream()), "lmk_grad_norm")


def adamw(p, g, m, v, lr, beta1, beta2, eps, wd, step, norm_scale, flags, shadow=None, shadow_f16=False):
    _kcheck(_lib.lmk_adamw(_ptr(p), _ptr(g), _ptr(m), _ptr(v), p.numel(), lr, beta1, beta2, eps, wd, step,
                           _ptr(norm_scale), _ptr(flags), _ptr(shadow), int(shadow_f16), _stream()), "lmk_adamw")
