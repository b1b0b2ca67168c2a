"""Seeded synthetic inputs for the decoder-only training step.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark. It holds no arithmetic of the method itself: only the five model
shapes, the optimiser settings, and seeded generators for token ids, packed
document layouts and initial parameters.

Why synthetic: the pages train on corpora that are not available here (byte text
of an educational web crawl on the Smallem page, a Persian SFT set on the
LucilleAI page, Shakespeare on the Feste page). Only the id distribution (which
embedding rows are hot, what cross-entropy sees) and the packing structure (how
much attention work there is) affect cost, so those are reproduced: uniform or
Zipf-distributed ids, and variable-length documents packed greedily into rows.

Generators use numpy's PCG64 with `data_seed = 1000 + k` and `init_seed =
2000 + k` for shape Ck (k = 1..5) unless a caller passes other seeds.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Dimensions of one pre-LayerNorm decoder-only model and its batch."""

    name: str
    vocab: int
    d_model: int
    n_heads: int
    d_mlp: int
    n_layers: int
    max_seq: int
    batch: int
    seq: int
    precision: str  # "fp32", "bf16" or "fp16" (16-bit compute, fp32 master weights; fp16 with loss scaling)
    # token-id distribution: ("uniform", 0.0) or ("zipf", s)
    ids: Tuple[str, float]
    # packing: None, ("uniform", lo, hi) or ("loguniform", lo, hi) document lengths
    docs: Optional[Tuple[str, int, int]]
    # optimiser
    lr: float
    weight_decay: float
    clip: float
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    ln_eps: float = 1e-5
    init_std: float = 0.02
    # scale the std of the residual output projections (w_o, w_proj) by
    # 1/sqrt(2 * n_layers) (GPT-2 style); only the GPT-2-small shape does
    scaled_resid_init: bool = False
    # a separate vocabulary projection with bias (head.w [V, C], head.b [V])
    # instead of the one tied to wte
    untied_head: bool = False

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_heads

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    def with_batch(self, batch: int, seq: Optional[int] = None) -> "ModelShape":
        return dataclasses.replace(self, batch=batch, seq=self.seq if seq is None else seq)

    def replace(self, **kw) -> "ModelShape":
        return dataclasses.replace(self, **kw)


# The five workloads. Dims follow the pages: 128/256/80/3 blocks and lr 5e-4 with
# clip 5.0 (RustGPT page, technical implementation list); V = 257 byte tokens
# (Smallem page, "what a language model is"); a ~1.9M-parameter packed SFT model
# at seq 512 (LucilleAI page, measured numbers); 768 = 12 x 64 with 12 blocks
# (Feste page, model architecture); a ~30M-parameter subword model (Smallem page).
C1 = ModelShape("C1", vocab=257, d_model=128, n_heads=4, d_mlp=256, n_layers=3, max_seq=80,
                batch=4, seq=80, precision="fp32", ids=("uniform", 0.0), docs=None,
                lr=5e-4, weight_decay=0.0, clip=5.0)
C2 = ModelShape("C2", vocab=257, d_model=256, n_heads=8, d_mlp=1024, n_layers=4, max_seq=256,
                batch=16, seq=256, precision="bf16", ids=("zipf", 1.1), docs=None,
                lr=3e-4, weight_decay=0.1, clip=5.0)
C3 = ModelShape("C3", vocab=8000, d_model=128, n_heads=4, d_mlp=512, n_layers=4, max_seq=512,
                batch=32, seq=512, precision="bf16", ids=("zipf", 1.05), docs=("uniform", 20, 200),
                lr=1e-4, weight_decay=0.0, clip=5.0)
C4 = ModelShape("C4", vocab=50257, d_model=768, n_heads=12, d_mlp=3072, n_layers=12, max_seq=1024,
                batch=8, seq=1024, precision="bf16", ids=("zipf", 1.1), docs=None,
                lr=6e-4, weight_decay=0.0, clip=1.0, scaled_resid_init=True)
C5 = ModelShape("C5", vocab=16384, d_model=512, n_heads=8, d_mlp=2048, n_layers=8, max_seq=2048,
                batch=16, seq=2048, precision="bf16", ids=("zipf", 1.1), docs=("loguniform", 64, 2048),
                lr=3e-4, weight_decay=0.1, clip=1.0)

SHAPES: Dict[str, ModelShape] = {c.name: c for c in (C1, C2, C3, C4, C5)}


def seeds(shape: ModelShape) -> Tuple[int, int]:
    """(data_seed, init_seed) for a named shape Ck: 1000 + k and 2000 + k."""
    k = int(shape.name[1:]) if shape.name[1:].isdigit() else 0
    return 1000 + k, 2000 + k


# --------------------------------------------------------------------------- ids

def sample_ids(rng: np.random.Generator, kind: Tuple[str, float], vocab: int, n: int) -> np.ndarray:
    """Draw n token ids in [0, vocab).

    uniform: i.i.d. uniform. zipf(s): P(id = k) proportional to (k + 1)^-s,
    sampled by inverse CDF on float64 uniforms (id = rank, so id 0 is hottest).
    """
    if kind[0] == "uniform":
        return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)
    s = kind[1]
    w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def _doc_lengths(rng: np.random.Generator, docs: Tuple[str, int, int]) -> int:
    kind, lo, hi = docs
    if kind == "uniform":
        return int(rng.integers(lo, hi + 1))
    # log-uniform: round(exp(U(ln lo, ln hi)))
    return int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))


@dataclasses.dataclass
class Batch:
    tokens: np.ndarray            # [B, T] int32
    targets: np.ndarray           # [B, T] int32, -1 = ignored
    doc_ids: Optional[np.ndarray]  # [B, T] int32 non-decreasing per row, or None
    n_docs: int = 0


def make_batch(shape: ModelShape, seed: Optional[int] = None) -> Batch:
    """One seeded batch of the shape's workload.

    Unpacked shapes draw T + 1 ids per row: inputs are the first T, targets the
    last T (every position is a valid target).

    Packed shapes draw document lengths L and L + 1 ids per document (inputs the
    first L, targets the last L), and pack documents greedily in draw order:
    append while the next document fits; when it does not, the row is closed
    with trailing padding (token 0, target -1, its own document id) and the
    next row starts with that document. Document ids count up from 0 within a
    row. A document longer than T is cut to T (never happens for the pages'
    length ranges, which stay <= T).
    """
    data_seed = seeds(shape)[0] if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(data_seed))
    B, T, V = shape.batch, shape.seq, shape.vocab
    if shape.docs is None:
        ids = sample_ids(rng, shape.ids, V, B * (T + 1)).reshape(B, T + 1)
        return Batch(np.ascontiguousarray(ids[:, :T]), np.ascontiguousarray(ids[:, 1:]), None, B)

    tokens = np.zeros((B, T), np.int32)
    targets = np.full((B, T), -1, np.int32)
    doc_ids = np.zeros((B, T), np.int32)
    row, fill, doc, n_docs = 0, 0, 0, 0
    pending = None
    while row < B:
        if pending is None:
            L = min(_doc_lengths(rng, shape.docs), T)
            pending = sample_ids(rng, shape.ids, V, L + 1)
        L = len(pending) - 1
        if fill + L <= T:
            tokens[row, fill:fill + L] = pending[:L]
            targets[row, fill:fill + L] = pending[1:]
            doc_ids[row, fill:fill + L] = doc
            fill += L
            doc += 1
            n_docs += 1
            pending = None
            if fill == T:
                row, fill, doc = row + 1, 0, 0
        else:
            doc_ids[row, fill:] = doc  # the pad run is its own document
            row, fill, doc = row + 1, 0, 0
    return Batch(tokens, targets, doc_ids, n_docs)


def structured_batch(shape: ModelShape, seed: int = 7, period: int = 16, batch: Optional[int] = None) -> Batch:
    """Learnable synthetic text for loss-descent runs (no corpus exists here):
    a seeded cycle of `period` distinct ids; every row starts at a random point
    of the cycle and walks it, so the next id is a function of the current
    one. T + 1 ids per row: inputs the first T, targets the last T."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B = shape.batch if batch is None else batch
    T, V = shape.seq, shape.vocab
    cycle = rng.choice(V, size=min(period, V), replace=False).astype(np.int32)
    starts = rng.integers(0, len(cycle), size=B)
    idx = (starts[:, None] + np.arange(T + 1)[None, :]) % len(cycle)
    ids = cycle[idx]
    return Batch(np.ascontiguousarray(ids[:, :T]), np.ascontiguousarray(ids[:, 1:]), None, B)


# --------------------------------------------------------------------- parameters

def param_specs(shape: ModelShape) -> List[Tuple[str, Tuple[int, ...]]]:
    """Names and shapes of the model's parameters, in storage order.

    Weight matrices are [out, in] row-major. The vocabulary projection is tied
    to wte, so there is no separate head matrix, unless the shape asks for an
    untied head: then head.w [V, C] and head.b [V] come last.
    """
    V, C, F, S = shape.vocab, shape.d_model, shape.d_mlp, shape.max_seq
    out = [("wte", (V, C)), ("wpe", (S, C))]
    for l in range(shape.n_layers):
        p = f"blocks.{l}."
        out += [
            (p + "ln1.g", (C,)), (p + "ln1.b", (C,)),
            (p + "attn.w_qkv", (3 * C, C)), (p + "attn.b_qkv", (3 * C,)),
            (p + "attn.w_o", (C, C)), (p + "attn.b_o", (C,)),
            (p + "ln2.g", (C,)), (p + "ln2.b", (C,)),
            (p + "mlp.w_fc", (F, C)), (p + "mlp.b_fc", (F,)),
            (p + "mlp.w_proj", (C, F)), (p + "mlp.b_proj", (C,)),
        ]
    out += [("lnf.g", (C,)), ("lnf.b", (C,))]
    if shape.untied_head:
        out += [("head.w", (V, C)), ("head.b", (V,))]
    return out


def init_params(shape: ModelShape, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Seeded fp32 initial parameters.

    Every matrix (wte and wpe included) ~ N(0, init_std); with
    scaled_resid_init, w_o and w_proj use init_std / sqrt(2 * n_layers).
    Biases 0, LayerNorm gains 1 and shifts 0. Draws happen in storage order.
    """
    init_seed = seeds(shape)[1] if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(init_seed))
    out: Dict[str, np.ndarray] = {}
    for name, shp in param_specs(shape):
        if len(shp) == 2:
            std = shape.init_std
            if shape.scaled_resid_init and (name.endswith("attn.w_o") or name.endswith("mlp.w_proj")):
                std = shape.init_std / math.sqrt(2 * shape.n_layers)
            out[name] = (rng.standard_normal(shp) * std).astype(np.float32)
        elif name.endswith(".g"):
            out[name] = np.ones(shp, np.float32)
        else:
            out[name] = np.zeros(shp, np.float32)
    return out


def random_tensor(rng: np.random.Generator, shape, scale: float = 1.0, dtype=np.float32) -> np.ndarray:
    """Standard-normal tensor times scale (for per-kernel parity inputs)."""
    return (rng.standard_normal(shape) * scale).astype(dtype)


def n_params(shape: ModelShape) -> int:
    return sum(int(np.prod(s)) for _, s in param_specs(shape))
