"""Float64 reference of the training step (TEST INFRASTRUCTURE ONLY).

Only tests/, the smoke check and the benchmark's CPU-baseline leg use this
module; the HIP product path never does.

Sources (cited by page and section; the pages are five web pages about
building GPT-style language models without a framework):

* Feste page (GPT-2 from scratch in Rust), "Model Architecture": token
  embedding with the positional encoding added directly; a stack of blocks that
  ends in a LayerNorm; multi-head attention by splitting 768 dims into 12 heads
  of 64; causal masking by filling future positions with -infinity before the
  softmax; GELU as the activation.
* Feste page, "Manual Backpropagation": a hand-written chain-rule backward
  through softmax, attention heads and residual connections; AdamW with weight
  decay decoupled from the gradient; gradient clipping.
* RustGPT page, technical-implementation list: cross-entropy loss, Adam with
  gradient clipping to an L2 norm of 5.0; LayerNorm as its own layer.
* Smallem page, "Ce qu'est un modèle de langage": the model returns V positive
  numbers that sum to 1 (the next-token distribution).
* Smallem page, "Deux implémentations de tout": every op written a second time,
  as simply as possible, on the CPU, as the oracle; gradient checks in double
  precision.
* LucilleAI page, "what makes it special" and measured numbers: sequence
  packing (several documents per row).

Readings where the pages are silent (each one is listed with its reason in the
design notes): GELU is the tanh form; LayerNorm uses the biased variance and
eps = 1e-5; the attention scale is 1/sqrt(D); the mask admits key j for query
i iff start(i) <= j <= i (same document, not in the future); positions restart
at 0 in each packed document; the vocabulary projection is tied to wte with no
bias, unless the parameters hold a separate head ("head.w" [V, C] and "head.b"
[V], the RustGPT page's output projection, a linear layer of its own); the loss is the mean over positions whose target is >= 0; the clip is on
the global L2 norm of all gradients, applied only when the norm exceeds it;
AdamW decays every parameter by lr * wd * p (pre-update p).

Layouts: activations are [B, T, ...]; weights are [out, in] (Y = X W^T + b).
The QKV projection's 3C output columns are q | k | v, and head h owns columns
h*D .. h*D + D - 1 of each third.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np

F64 = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


# ----------------------------------------------------------------- index layout

def index_layout(doc_ids: Optional[np.ndarray], B: int, T: int, max_seq: Optional[int] = None):
    """start[b, t] and pos[b, t] for the (optionally packed) rows.

    Packing (LucilleAI page) puts several documents in one row. A document is a
    maximal run of equal doc ids in a row; doc ids must be non-decreasing.
    start[b, t] is the index of the first token of t's run, and the position
    used for the positional embedding is pos = t - start (positions restart
    in every document). Without doc ids the whole row is one document:
    start = 0, pos = t.
    """
    if doc_ids is None:
        start = np.zeros((B, T), np.int64)
    else:
        doc = np.asarray(doc_ids).reshape(B, T)
        if np.any(np.diff(doc.astype(np.int64), axis=1) < 0):
            raise ValueError("doc_ids must be non-decreasing along each row")
        start = np.zeros((B, T), np.int64)
        for b in range(B):
            s = 0
            for t in range(T):
                if t > 0 and doc[b, t] != doc[b, t - 1]:
                    s = t
                start[b, t] = s
    pos = np.arange(T, dtype=np.int64)[None, :] - start
    if max_seq is not None and pos.size and pos.max() >= max_seq:
        raise ValueError("a document is longer than max_seq")
    return start, pos


def csr_by_key(keys: np.ndarray, n_keys: int):
    """Stable counting sort of flat keys: (offsets[n_keys + 1], perm[n]).

    perm lists the flat indices grouped by key, ascending key, and in ascending
    index order within a key. This is the gather order the embedding backward
    sums in.
    """
    keys = np.asarray(keys).reshape(-1).astype(np.int64)
    counts = np.zeros(n_keys, np.int64)
    for k in keys:
        counts[k] += 1
    offsets = np.zeros(n_keys + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    perm = np.zeros(len(keys), np.int64)
    for i, k in enumerate(keys):
        perm[fill[k]] = i
        fill[k] += 1
    return offsets, perm


# -------------------------------------------------------------------- embedding

def embedding_fwd(wte, wpe, tok, pos) -> np.ndarray:
    """x = wte[tok] + wpe[pos] (Feste page, "Model Architecture": the
    positional encoding is added straight onto the token embedding)."""
    return _f64(wte)[np.asarray(tok)] + _f64(wpe)[np.asarray(pos)]


def embedding_bwd(dx, tok, pos, V: int, S: int):
    """Scatter-add of dx into the rows it was gathered from: dwte[v] = sum of
    dx over positions whose token is v; dwpe[p] = sum over positions p."""
    dx = _f64(dx)
    C = dx.shape[-1]
    dwte = np.zeros((V, C))
    dwpe = np.zeros((S, C))
    np.add.at(dwte, np.asarray(tok).reshape(-1), dx.reshape(-1, C))
    np.add.at(dwpe, np.asarray(pos).reshape(-1), dx.reshape(-1, C))
    return dwte, dwpe


# -------------------------------------------------------------------- LayerNorm

def layernorm_fwd(x, g, b, eps: float):
    """LayerNorm over the last axis: mu = mean(x), var = mean((x - mu)^2)
    (biased), rstd = (var + eps)^-1/2, y = g * (x - mu) * rstd + b.
    (A LayerNorm layer of its own on the RustGPT page; the final one before the
    vocabulary projection on the Feste page.)"""
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu) * rstd
    y = xhat * _f64(g) + _f64(b)
    return y, mu[..., 0], rstd[..., 0]


def layernorm_bwd(dy, x, mu, rstd, g):
    """Chain rule through LayerNorm (Feste page, "Manual Backpropagation").

    With xhat = (x - mu) * rstd and dxhat = dy * g:
    dx = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat));
    dg = sum over rows of dy * xhat; db = sum over rows of dy.
    """
    dy, x = _f64(dy), _f64(x)
    mu, rstd = _f64(mu)[..., None], _f64(rstd)[..., None]
    xhat = (x - mu) * rstd
    dxhat = dy * _f64(g)
    dx = rstd * (dxhat - dxhat.mean(axis=-1, keepdims=True)
                 - xhat * (dxhat * xhat).mean(axis=-1, keepdims=True))
    C = x.shape[-1]
    dg = (dy * xhat).reshape(-1, C).sum(axis=0)
    db = dy.reshape(-1, C).sum(axis=0)
    return dx, dg, db


# ----------------------------------------------------------------------- linear

def linear_fwd(x, W, b=None):
    """Y = X W^T (+ b), W stored [out, in]."""
    y = _f64(x) @ _f64(W).T
    if b is not None:
        y = y + _f64(b)
    return y


def linear_bwd(dy, x, W):
    """For Y = X W^T + b: dX = dY W, dW = dY^T X, db = column sums of dY."""
    dy, x = _f64(dy), _f64(x)
    N, K = np.shape(W)
    dy2, x2 = dy.reshape(-1, N), x.reshape(-1, K)
    dx = (dy2 @ _f64(W)).reshape(x.shape)
    dW = dy2.T @ x2
    db = dy2.sum(axis=0)
    return dx, dW, db


# ------------------------------------------------------------------------- GELU

_GELU_C = math.sqrt(2.0 / math.pi)
_GELU_A = 0.044715


def gelu(u):
    """GELU (Feste page, "Model Architecture" uses GELU instead of ReLU), in the
    tanh form of the GPT-2 lineage: 0.5 u (1 + tanh(c (u + a u^3))),
    c = sqrt(2/pi), a = 0.044715."""
    u = _f64(u)
    return 0.5 * u * (1.0 + np.tanh(_GELU_C * (u + _GELU_A * u ** 3)))


def gelu_grad(u):
    """d GELU / du of the tanh form: with t = tanh(c (u + a u^3)),
    0.5 (1 + t) + 0.5 u (1 - t^2) c (1 + 3 a u^2)."""
    u = _f64(u)
    t = np.tanh(_GELU_C * (u + _GELU_A * u ** 3))
    return 0.5 * (1.0 + t) + 0.5 * u * (1.0 - t * t) * _GELU_C * (1.0 + 3.0 * _GELU_A * u * u)


# -------------------------------------------------------------------- attention

def _mask(start_row: np.ndarray) -> np.ndarray:
    """allowed[i, j] = start(i) <= j <= i: causal (Feste page, future positions
    filled with -inf before the softmax), and, for packed rows, within the
    query's own document."""
    T = len(start_row)
    j = np.arange(T)[None, :]
    i = np.arange(T)[:, None]
    return (j <= i) & (j >= start_row[:, None])


def attention_probs(q, k, start_row):
    """P = softmax(S) per row, S_ij = q_i . k_j / sqrt(D) on allowed pairs and
    -inf elsewhere; also returns the row log-sum-exp of S. q, k: [T, D]."""
    q, k = _f64(q), _f64(k)
    D = q.shape[-1]
    s = (q @ k.T) / math.sqrt(D)
    s = np.where(_mask(np.asarray(start_row)), s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[:, 0]


def attention_fwd(q, k, v, start):
    """Multi-head causal self-attention (Feste page, "Model Architecture").

    q, k, v: [B, H, T, D]; start: [B, T]. Returns o [B, H, T, D] with
    o_i = sum_j P_ij v_j, and lse [B, H, T] (natural-log log-sum-exp of the
    scaled, masked scores of each query row).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, D = q.shape
    o = np.zeros_like(q)
    lse = np.zeros((B, H, T))
    for b in range(B):
        for h in range(H):
            p, l = attention_probs(q[b, h], k[b, h], start[b])
            o[b, h] = p @ v[b, h]
            lse[b, h] = l
    return o, lse


def attention_bwd(do, q, k, v, start):
    """Chain rule through attention (Feste page, "Manual Backpropagation":
    gradients flow back through the softmax and the heads).

    With P recomputed from q, k: dv = P^T do; dP = do v^T;
    dS = P * (dP - rowsum(dP * P)); dq = dS k / sqrt(D); dk = dS^T q / sqrt(D).
    """
    do, q, k, v = _f64(do), _f64(q), _f64(k), _f64(v)
    B, H, T, D = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    sc = 1.0 / math.sqrt(D)
    for b in range(B):
        for h in range(H):
            p, _ = attention_probs(q[b, h], k[b, h], start[b])
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
            dq[b, h] = ds @ k[b, h] * sc
            dk[b, h] = ds.T @ q[b, h] * sc
    return dq, dk, dv


def _split_heads(t, H):
    B, T, C = t.shape
    return t.reshape(B, T, H, C // H).transpose(0, 2, 1, 3)


def _merge_heads(t):
    B, H, T, D = t.shape
    return t.transpose(0, 2, 1, 3).reshape(B, T, H * D)


# ---------------------------------------------------------------- cross-entropy

def xent_fwd_bwd(z, tgt):
    """Softmax cross-entropy (RustGPT page: cross-entropy loss; Smallem page:
    the V outputs are positive and sum to 1).

    Over the valid set {tgt >= 0} of size N: loss = (1/N) sum (logsumexp(z) -
    z[tgt]); dz = (softmax(z) - onehot(tgt)) / N on valid rows and 0 on ignored
    rows. N = 0 gives loss 0 and dz 0. Returns (loss, dz, N).
    """
    z = _f64(z)
    V = z.shape[-1]
    z2 = z.reshape(-1, V)
    t = np.asarray(tgt).reshape(-1)
    valid = t >= 0
    n = int(valid.sum())
    dz = np.zeros_like(z2)
    if n == 0:
        return 0.0, dz.reshape(z.shape), 0
    m = z2.max(axis=-1, keepdims=True)
    e = np.exp(z2 - m)
    s = e.sum(axis=-1, keepdims=True)
    lse = (m + np.log(s))[:, 0]
    rows = np.nonzero(valid)[0]
    loss = float((lse[rows] - z2[rows, t[rows]]).sum() / n)
    p = e / s
    dz[rows] = p[rows]
    dz[rows, t[rows]] -= 1.0
    dz[rows] /= n
    return loss, dz.reshape(z.shape), n


# --------------------------------------------------------------------- the model

def _p(params, name):
    return _f64(params[name])


def forward(params: Dict[str, np.ndarray], cfg, tok, doc_ids=None, keep=True):
    """Forward pass of the pre-LN decoder (Feste page, "Model Architecture").

    cfg needs: vocab, d_model, n_heads, d_mlp, n_layers, max_seq, ln_eps.
    x0 = wte[tok] + wpe[pos]; per block l:
      y1 = LN1(x); qkv = y1 W_qkv^T + b_qkv; o = MHSA(q, k, v); x += o W_o^T + b_o
      y2 = LN2(x); u = y2 W_fc^T + b_fc; a = GELU(u); x += a W_proj^T + b_proj
    h_f = LN_f(x); z = h_f wte^T (tied head, no bias), or, with a separate
    head in params (RustGPT page, file list: output_projection),
    z = h_f head.w^T + head.b.
    Returns (z [B, T, V], cache) where cache holds what the backward reads.
    """
    tok = np.asarray(tok)
    B, T = tok.shape
    H = cfg.n_heads
    eps = cfg.ln_eps
    start, pos = index_layout(doc_ids, B, T, cfg.max_seq)
    x = embedding_fwd(params["wte"], params["wpe"], tok, pos)
    cache = {"start": start, "pos": pos, "tok": tok, "layers": []}
    for l in range(cfg.n_layers):
        p = f"blocks.{l}."
        c = {"x_in": x}
        y1, mu1, r1 = layernorm_fwd(x, params[p + "ln1.g"], params[p + "ln1.b"], eps)
        qkv = linear_fwd(y1, params[p + "attn.w_qkv"], params[p + "attn.b_qkv"])
        C = x.shape[-1]
        q, k, v = (_split_heads(qkv[..., i * C:(i + 1) * C], H) for i in range(3))
        o, lse = attention_fwd(q, k, v, start)
        o = _merge_heads(o)
        x_mid = x + linear_fwd(o, params[p + "attn.w_o"], params[p + "attn.b_o"])
        y2, mu2, r2 = layernorm_fwd(x_mid, params[p + "ln2.g"], params[p + "ln2.b"], eps)
        u = linear_fwd(y2, params[p + "mlp.w_fc"], params[p + "mlp.b_fc"])
        a = gelu(u)
        x = x_mid + linear_fwd(a, params[p + "mlp.w_proj"], params[p + "mlp.b_proj"])
        if keep:
            c.update(y1=y1, mu1=mu1, r1=r1, qkv=qkv, o=o, lse=lse, x_mid=x_mid,
                     y2=y2, mu2=mu2, r2=r2, u=u, a=a)
            cache["layers"].append(c)
    hf, muf, rf = layernorm_fwd(x, params["lnf.g"], params["lnf.b"], eps)
    if "head.w" in params:
        z = linear_fwd(hf, params["head.w"], params["head.b"])
    else:
        z = hf @ _p(params, "wte").T
    cache.update(x_f=x, hf=hf, muf=muf, rf=rf)
    return z, cache


def loss_and_grads(params: Dict[str, np.ndarray], cfg, tok, tgt, doc_ids=None):
    """Loss and the gradients of the mean loss for every parameter, by the
    hand-derived chain rule (Feste page, "Manual Backpropagation").

    Returns (loss, grads dict, logits z, n_valid).
    """
    z, cache = forward(params, cfg, tok, doc_ids)
    loss, dz, n = xent_fwd_bwd(z, tgt)
    H = cfg.n_heads
    V, C = np.shape(params["wte"])
    S = np.shape(params["wpe"])[0]
    g: Dict[str, np.ndarray] = {}
    if "head.w" in params:
        # separate head z = h_f head.w^T + head.b
        dhf, g["head.w"], g["head.b"] = linear_bwd(dz, cache["hf"], params["head.w"])
        dwte_head = 0.0
    else:
        # tied head z = h_f wte^T
        dz2 = dz.reshape(-1, V)
        hf2 = cache["hf"].reshape(-1, C)
        dwte_head = dz2.T @ hf2
        dhf = (dz2 @ _p(params, "wte")).reshape(cache["hf"].shape)
    dx, g["lnf.g"], g["lnf.b"] = layernorm_bwd(dhf, cache["x_f"], cache["muf"], cache["rf"], params["lnf.g"])
    for l in reversed(range(cfg.n_layers)):
        p = f"blocks.{l}."
        c = cache["layers"][l]
        # MLP: x = x_mid + a W_proj^T + b_proj
        da, g[p + "mlp.w_proj"], g[p + "mlp.b_proj"] = linear_bwd(dx, c["a"], params[p + "mlp.w_proj"])
        du = da * gelu_grad(c["u"])
        dy2, g[p + "mlp.w_fc"], g[p + "mlp.b_fc"] = linear_bwd(du, c["y2"], params[p + "mlp.w_fc"])
        dxm, g[p + "ln2.g"], g[p + "ln2.b"] = layernorm_bwd(dy2, c["x_mid"], c["mu2"], c["r2"], params[p + "ln2.g"])
        dx = dx + dxm
        # attention: x_mid = x_in + o W_o^T + b_o
        do, g[p + "attn.w_o"], g[p + "attn.b_o"] = linear_bwd(dx, c["o"], params[p + "attn.w_o"])
        qkv = c["qkv"]
        q, k, v = (_split_heads(qkv[..., i * C:(i + 1) * C], H) for i in range(3))
        dq, dk, dv = attention_bwd(_split_heads(do, H), q, k, v, cache["start"])
        dqkv = np.concatenate([_merge_heads(dq), _merge_heads(dk), _merge_heads(dv)], axis=-1)
        dy1, g[p + "attn.w_qkv"], g[p + "attn.b_qkv"] = linear_bwd(dqkv, c["y1"], params[p + "attn.w_qkv"])
        dxi, g[p + "ln1.g"], g[p + "ln1.b"] = layernorm_bwd(dy1, c["x_in"], c["mu1"], c["r1"], params[p + "ln1.g"])
        dx = dx + dxi
    dwte_emb, g["wpe"] = embedding_bwd(dx, cache["tok"], cache["pos"], V, S)
    g["wte"] = dwte_head + dwte_emb
    return loss, g, z, n


# -------------------------------------------------------------- clip and AdamW

def grad_norm_and_scale(grads: Dict[str, np.ndarray], clip: float):
    """Global L2 norm n of all gradients and the clip factor s = clip / n when
    n > clip, else 1 (RustGPT page: clipping to an L2 norm of 5.0; Feste page:
    clipping against exploding gradients)."""
    n = math.sqrt(sum(float((_f64(v) ** 2).sum()) for v in grads.values()))
    s = clip / n if (math.isfinite(n) and n > clip) else 1.0
    return n, s


def adamw(p, g, m, v, step: int, lr, beta1, beta2, eps, weight_decay, scale=1.0):
    """One AdamW update (Feste page, "Manual Backpropagation": weight decay kept
    out of the gradient). With gh = scale * g and a 1-based step t:
    m = b1 m + (1 - b1) gh; v = b2 v + (1 - b2) gh^2;
    mhat = m / (1 - b1^t); vhat = v / (1 - b2^t);
    p = p - lr (mhat / (sqrt(vhat) + eps) + wd p), wd acting on the old p."""
    p, g, m, v = _f64(p), _f64(g), _f64(m), _f64(v)
    gh = scale * g
    m2 = beta1 * m + (1.0 - beta1) * gh
    v2 = beta2 * v + (1.0 - beta2) * gh * gh
    mhat = m2 / (1.0 - beta1 ** step)
    vhat = v2 / (1.0 - beta2 ** step)
    p2 = p - lr * (mhat / (np.sqrt(vhat) + eps) + weight_decay * p)
    return p2, m2, v2


def train_step(params, m, v, cfg, tok, tgt, doc_ids, *, step: int, lr, beta1=0.9, beta2=0.999,
               eps=1e-8, weight_decay=0.0, clip=1.0):
    """Forward, loss, hand-derived backward, global-norm clip and AdamW.

    A non-finite gradient norm skips the update (parameters and moments stay
    as they were) and reports it in the result.
    Returns a dict with loss, n_valid, grad_norm (pre-clip), scale, grads,
    params, m, v (updated), logits and finite.
    """
    loss, grads, z, n = loss_and_grads(params, cfg, tok, tgt, doc_ids)
    norm, s = grad_norm_and_scale(grads, clip)
    finite = math.isfinite(norm)
    newp, newm, newv = {}, {}, {}
    for name in params:
        if finite:
            newp[name], newm[name], newv[name] = adamw(
                params[name], grads[name], m[name], v[name], step, lr, beta1, beta2, eps, weight_decay, s)
        else:
            newp[name], newm[name], newv[name] = _f64(params[name]), _f64(m[name]), _f64(v[name])
    return {"loss": loss, "n_valid": n, "grad_norm": norm, "scale": s, "grads": grads,
            "params": newp, "m": newm, "v": newv, "logits": z, "finite": finite}
