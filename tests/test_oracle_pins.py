"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what it pins. None of them re-types the oracle's formula:
they use finite differences, an independent autograd derivation, closed forms
and invariants the pages fix (causal -inf mask, rows of probabilities summing
to 1, clip to an L2 norm, decoupled weight decay), library routines for special
cases, and hand-derived fixtures under tests/golden/.
"""
import math
import os
import types

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_cfg(**kw):
    base = dict(vocab=11, d_model=8, n_heads=2, d_mlp=16, n_layers=2, max_seq=6, ln_eps=1e-5)
    base.update(kw)
    return types.SimpleNamespace(**base)


def random_params(cfg, seed, std=0.3):
    """Parameters with non-trivial gains and biases, so no gradient is zero by
    accident of the init."""
    rng = np.random.default_rng(seed)
    V, C, F, S = cfg.vocab, cfg.d_model, cfg.d_mlp, cfg.max_seq
    p = {"wte": rng.standard_normal((V, C)) * std, "wpe": rng.standard_normal((S, C)) * std}
    for l in range(cfg.n_layers):
        q = f"blocks.{l}."
        p[q + "ln1.g"] = 1 + 0.2 * rng.standard_normal(C)
        p[q + "ln1.b"] = 0.2 * rng.standard_normal(C)
        p[q + "attn.w_qkv"] = rng.standard_normal((3 * C, C)) * std
        p[q + "attn.b_qkv"] = rng.standard_normal(3 * C) * 0.1
        p[q + "attn.w_o"] = rng.standard_normal((C, C)) * std
        p[q + "attn.b_o"] = rng.standard_normal(C) * 0.1
        p[q + "ln2.g"] = 1 + 0.2 * rng.standard_normal(C)
        p[q + "ln2.b"] = 0.2 * rng.standard_normal(C)
        p[q + "mlp.w_fc"] = rng.standard_normal((F, C)) * std
        p[q + "mlp.b_fc"] = rng.standard_normal(F) * 0.1
        p[q + "mlp.w_proj"] = rng.standard_normal((C, F)) * std
        p[q + "mlp.b_proj"] = rng.standard_normal(C) * 0.1
    p["lnf.g"] = 1 + 0.2 * rng.standard_normal(C)
    p["lnf.b"] = 0.2 * rng.standard_normal(C)
    if getattr(cfg, "untied_head", False):
        p["head.w"] = rng.standard_normal((V, C)) * std
        p["head.b"] = rng.standard_normal(V) * 0.1
    return p


def tiny_batch(cfg, seed=3):
    """Row 0 packs documents of length 2 and 3 followed by one pad position;
    row 1 is one document with one ignored target."""
    rng = np.random.default_rng(seed)
    B, T = 2, 6
    tok = rng.integers(0, cfg.vocab, (B, T)).astype(np.int32)
    tgt = rng.integers(0, cfg.vocab, (B, T)).astype(np.int32)
    doc = np.array([[0, 0, 1, 1, 1, 2], [0, 0, 0, 0, 0, 0]], np.int32)
    tok[0, 5] = 0
    tgt[0, 5] = -1
    tgt[1, 3] = -1
    return tok, tgt, doc


# ------------------------------------------------------------- P8: finite diffs

@pytest.mark.parametrize("untied", [False, True])
def test_finite_difference_gradients_every_parameter(untied):
    """P8: the whole hand-derived backward against central differences in
    float64 (Smallem page: gradient checks need double precision), with the
    tied head and with a separate head and bias."""
    cfg = tiny_cfg(untied_head=untied)
    params = random_params(cfg, 7)
    tok, tgt, doc = tiny_batch(cfg)
    loss, grads, _, n = oracle.loss_and_grads(params, cfg, tok, tgt, doc)
    assert n == 10
    h = 1e-6

    def f(p):
        return oracle.xent_fwd_bwd(oracle.forward(p, cfg, tok, doc, keep=False)[0], tgt)[0]

    worst = 0.0
    for name, val in params.items():
        flat = val.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + h
            fp = f(params)
            flat[i] = old - h
            fm = f(params)
            flat[i] = old
            g_fd = (fp - fm) / (2 * h)
            g = grads[name].reshape(-1)[i]
            err = abs(g_fd - g) / max(1.0, abs(g))
            worst = max(worst, err)
            assert err <= 1e-6, (name, i, g_fd, g)
    # 10 random directions through all parameters at once
    rng = np.random.default_rng(11)
    for _ in range(10):
        d = {k: rng.standard_normal(v.shape) for k, v in params.items()}
        pp = {k: params[k] + h * d[k] for k in params}
        pm = {k: params[k] - h * d[k] for k in params}
        g_fd = (f(pp) - f(pm)) / (2 * h)
        g = sum(float((grads[k] * d[k]).sum()) for k in params)
        assert abs(g_fd - g) <= 1e-6 * max(1.0, abs(g))


# ------------------------------------------------ P15: independent autograd pin

def _torch_loss(tp, cfg, tok, tgt, doc):
    """The same network written directly in torch float64 with autograd; only
    the forward definition is restated, the backward is torch's own."""
    import torch
    B, T = tok.shape
    H, C = cfg.n_heads, cfg.d_model
    D = C // H
    start, pos = oracle.index_layout(doc, B, T, cfg.max_seq)
    tok_t = torch.as_tensor(tok.astype(np.int64))
    pos_t = torch.as_tensor(pos)
    x = tp["wte"][tok_t] + tp["wpe"][pos_t]
    ii = torch.arange(T)[:, None]
    jj = torch.arange(T)[None, :]
    st = torch.as_tensor(start)
    allowed = (jj <= ii)[None] & (jj[None] >= st[:, :, None])  # [B, T, T]

    def ln(x, g, b):
        return torch.nn.functional.layer_norm(x, (C,), g, b, cfg.ln_eps)

    for l in range(cfg.n_layers):
        p = f"blocks.{l}."
        y = ln(x, tp[p + "ln1.g"], tp[p + "ln1.b"])
        qkv = torch.nn.functional.linear(y, tp[p + "attn.w_qkv"], tp[p + "attn.b_qkv"])
        q, k, v = qkv.split(C, dim=-1)
        q = q.reshape(B, T, H, D).transpose(1, 2)
        k = k.reshape(B, T, H, D).transpose(1, 2)
        v = v.reshape(B, T, H, D).transpose(1, 2)
        s = (q @ k.transpose(-1, -2)) / math.sqrt(D)
        s = s.masked_fill(~allowed[:, None], float("-inf"))
        o = torch.softmax(s, dim=-1) @ v
        o = o.transpose(1, 2).reshape(B, T, C)
        x = x + torch.nn.functional.linear(o, tp[p + "attn.w_o"], tp[p + "attn.b_o"])
        y = ln(x, tp[p + "ln2.g"], tp[p + "ln2.b"])
        u = torch.nn.functional.linear(y, tp[p + "mlp.w_fc"], tp[p + "mlp.b_fc"])
        a = torch.nn.functional.gelu(u, approximate="tanh")
        x = x + torch.nn.functional.linear(a, tp[p + "mlp.w_proj"], tp[p + "mlp.b_proj"])
    hf = ln(x, tp["lnf.g"], tp["lnf.b"])
    if "head.w" in tp:
        z = torch.nn.functional.linear(hf, tp["head.w"], tp["head.b"])
    else:
        z = hf @ tp["wte"].T
    tgt_t = torch.as_tensor(tgt.astype(np.int64)).reshape(-1)
    return torch.nn.functional.cross_entropy(z.reshape(-1, cfg.vocab), tgt_t, ignore_index=-1), z


@pytest.mark.parametrize("which", ["tiny", "tiny_untied", "c1_like"])
def test_torch_autograd_cross_check(which):
    """P15: gradients of the hand-derived backward equal torch's autograd of
    the same network to 1e-10 relative per tensor; logits and loss too."""
    torch = pytest.importorskip("torch")
    if which.startswith("tiny"):
        cfg = tiny_cfg(untied_head=which == "tiny_untied")
        params = random_params(cfg, 5)
        tok, tgt, doc = tiny_batch(cfg, 9)
    else:
        shape = synth.C1.with_batch(2, 40)
        cfg = shape
        params = {k: v.astype(np.float64) for k, v in synth.init_params(shape).items()}
        rng = np.random.default_rng(4)
        for k in params:  # move gains/biases off their init so their grads are generic
            if params[k].ndim == 1:
                params[k] = params[k] + 0.1 * rng.standard_normal(params[k].shape)
        b = synth.make_batch(shape)
        tok, tgt = b.tokens, b.targets
        doc = np.repeat(np.array([[0] * 15 + [1] * 25]), 2, axis=0).astype(np.int32)
        tgt = tgt.copy()
        tgt[1, 7] = -1
    loss, grads, z, _ = oracle.loss_and_grads(params, cfg, tok, tgt, doc)
    tp = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in params.items()}
    tl, tz = _torch_loss(tp, cfg, tok, tgt, doc)
    tl.backward()
    assert abs(tl.item() - loss) <= 1e-12 * abs(loss)
    np.testing.assert_allclose(z, tz.detach().numpy(), rtol=1e-11, atol=1e-12)
    for k in params:
        ref = tp[k].grad.numpy()
        rel = np.linalg.norm(grads[k] - ref) / max(np.linalg.norm(ref), 1e-300)
        assert rel <= 1e-10 or np.linalg.norm(grads[k] - ref) <= 1e-14, (k, rel)


# --------------------------------------------------------- P1, P2: loss values

@pytest.mark.parametrize("name,batch,seq", [("C1", 4, 80), ("C2", 2, 256), ("C3", 2, 512),
                                            ("C4", 1, 128), ("C5", 1, 256)])
def test_init_loss_near_log_vocab(name, batch, seq):
    """P1: at init (tiny weights, N(0, 0.02)) logits are nearly independent
    zero-mean with variance C * 0.02^2, so the loss is ln V + C * 0.02^2 / 2
    within 0.1 nats (ln 257 = 5.549 for the byte vocabulary)."""
    shape = synth.SHAPES[name].with_batch(batch, seq).replace(docs=None)
    params = synth.init_params(shape)
    b = synth.make_batch(shape)
    z, _ = oracle.forward(params, shape, b.tokens, None, keep=False)
    loss, _, _ = oracle.xent_fwd_bwd(z, b.targets)
    expect = math.log(shape.vocab) + 0.5 * shape.d_model * 0.02 ** 2
    assert abs(loss - expect) < 0.1, (loss, expect)


def test_zero_final_gain_gives_exact_log_vocab():
    """P2: with the final LayerNorm's gain and shift at 0, every logit is 0, so
    the loss is ln V exactly, dz = (1/V - onehot)/N, nothing below the final
    LayerNorm gets a gradient, and d(lnf.b) has the closed form
    sum over valid positions of (mean_v wte[v] - wte[tgt]) / N."""
    cfg = tiny_cfg()
    params = random_params(cfg, 2)
    params["lnf.g"] = np.zeros(cfg.d_model)
    params["lnf.b"] = np.zeros(cfg.d_model)
    tok, tgt, doc = tiny_batch(cfg)
    loss, grads, z, n = oracle.loss_and_grads(params, cfg, tok, tgt, doc)
    assert np.all(z == 0)
    assert abs(loss - math.log(cfg.vocab)) <= 1e-15 * math.log(cfg.vocab)
    t = tgt.reshape(-1)
    valid = t[t >= 0]
    wte = params["wte"]
    expect_db = (wte.mean(axis=0)[None, :] - wte[valid]).sum(axis=0) / n
    np.testing.assert_allclose(grads["lnf.b"], expect_db, rtol=1e-12, atol=1e-15)
    for k, g in grads.items():
        if k in ("lnf.g", "lnf.b"):
            continue
        if k == "wte":
            # only the head part, dz^T h_f with h_f = 0, which is 0
            assert np.all(g == 0), k
        else:
            assert np.all(g == 0), k


# ------------------------------------------------------ P3: probabilities sum 1

def test_softmax_rows_sum_to_one():
    """P3 (Smallem page: V positive numbers that sum to 1): attention rows and
    the next-token distribution are positive and sum to 1; dz rows sum to 0."""
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((2, 9, 4)) * 3
    start = np.array([0, 0, 0, 3, 3, 3, 3, 7, 7])
    p, _ = oracle.attention_probs(q, k, start)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, atol=1e-12)
    assert np.all(p >= 0)
    z = rng.standard_normal((5, 13)) * 4
    tgt = np.array([1, 2, -1, 12, 0])
    _, dz, n = oracle.xent_fwd_bwd(z, tgt)
    probs = dz * n
    probs[np.arange(5), np.maximum(tgt, 0)] += (tgt >= 0)
    np.testing.assert_allclose(probs[tgt >= 0].sum(axis=-1), 1.0, atol=1e-12)
    np.testing.assert_allclose(dz.sum(axis=-1), 0.0, atol=1e-15)
    assert np.all(dz[2] == 0)


def test_cross_entropy_special_cases():
    """Uniform logits give ln V for any target; a target logit far above the
    rest gives loss -> 0; all targets ignored gives 0 and a zero gradient."""
    z = np.full((3, 7), 2.5)
    loss, _, _ = oracle.xent_fwd_bwd(z, np.array([0, 3, 6]))
    assert abs(loss - math.log(7)) < 1e-14
    z = np.zeros((1, 7))
    z[0, 4] = 60.0
    loss, _, _ = oracle.xent_fwd_bwd(z, np.array([4]))
    assert 0 <= loss < 1e-20
    loss, dz, n = oracle.xent_fwd_bwd(np.ones((2, 3)), np.array([-1, -1]))
    assert loss == 0 and n == 0 and np.all(dz == 0)


# --------------------------------------------------------------- P4: causality

def test_causality_bit_exact():
    """P4 (Feste page: future positions masked with -inf before the softmax):
    changing tokens after t leaves every logit at positions <= t bit-identical."""
    shape = synth.C1.with_batch(2, 40)
    params = synth.init_params(shape)
    b = synth.make_batch(shape)
    z0, _ = oracle.forward(params, shape, b.tokens, None, keep=False)
    rng = np.random.default_rng(0)
    for t in (0, 13, 38):
        tok = b.tokens.copy()
        tok[:, t + 1:] = rng.integers(0, shape.vocab, tok[:, t + 1:].shape)
        z1, _ = oracle.forward(params, shape, tok, None, keep=False)
        assert np.array_equal(z0[:, :t + 1], z1[:, :t + 1])
        if t < 38:
            assert not np.array_equal(z0[:, t + 1:], z1[:, t + 1:])


# ------------------------------------------------------- P5, P6: packed rows

def test_packed_row_equals_documents_run_separately():
    """P5: a packed row (block-diagonal mask, positions restarting per
    document) gives each document the logits it gets alone in its own row, and
    the loss sums agree."""
    cfg = tiny_cfg(vocab=13, max_seq=12)
    params = random_params(cfg, 8)
    rng = np.random.default_rng(2)
    lens = [4, 5, 3]
    T = sum(lens)
    tok = rng.integers(0, cfg.vocab, (1, T)).astype(np.int32)
    tgt = rng.integers(0, cfg.vocab, (1, T)).astype(np.int32)
    doc = np.repeat(np.arange(3), lens)[None].astype(np.int32)
    zp, _ = oracle.forward(params, cfg, tok, doc, keep=False)
    lp, _, npk = oracle.xent_fwd_bwd(zp, tgt)
    total, off = 0.0, 0
    for L in lens:
        zs, _ = oracle.forward(params, cfg, tok[:, off:off + L], None, keep=False)
        np.testing.assert_allclose(zp[:, off:off + L], zs, rtol=1e-12, atol=1e-13)
        ls, _, ns = oracle.xent_fwd_bwd(zs, tgt[:, off:off + L])
        total += ls * ns
        off += L
    assert abs(lp * npk - total) <= 1e-12 * abs(total)


def test_single_document_row_equals_causal_path():
    """P6: doc ids that are all equal select exactly the plain causal path."""
    cfg = tiny_cfg()
    params = random_params(cfg, 1)
    tok, tgt, _ = tiny_batch(cfg)
    za, _ = oracle.forward(params, cfg, tok, np.full(tok.shape, 4, np.int32), keep=False)
    zb, _ = oracle.forward(params, cfg, tok, None, keep=False)
    assert np.array_equal(za, zb)


# ----------------------------------------------------------- P7: special cases

def test_attention_single_position_returns_value():
    """P7: with one key the softmax is [1], so o = v exactly and lse = s_00."""
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((3, 1, 2, 1, 8))
    o, lse = oracle.attention_fwd(q, k, v, np.zeros((1, 1), np.int64))
    assert np.array_equal(o, v)
    np.testing.assert_allclose(lse[0, :, 0], (q[0, :, 0] * k[0, :, 0]).sum(-1) / math.sqrt(8), rtol=1e-14)


def test_attention_closed_forms():
    """With q = 0 every allowed score is 0, so P is uniform over the allowed
    keys: o_i is the mean of v over start(i)..i and lse_i = ln(i - start(i) + 1).
    With all keys equal the output is the same mean for any q."""
    rng = np.random.default_rng(4)
    T, D = 9, 4
    start = np.array([[0, 0, 0, 3, 3, 3, 3, 7, 7]])
    v = rng.standard_normal((1, 1, T, D))
    k = rng.standard_normal((1, 1, T, D))
    q = np.zeros((1, 1, T, D))
    o, lse = oracle.attention_fwd(q, k, v, start)
    for i in range(T):
        s = start[0, i]
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, s:i + 1].mean(axis=0), rtol=1e-13, atol=1e-15)
        assert abs(lse[0, 0, i] - math.log(i - s + 1)) < 1e-13
    k_same = np.repeat(k[:, :, :1], T, axis=2)
    q2 = rng.standard_normal((1, 1, T, D)) * 5
    o2, _ = oracle.attention_fwd(q2, k_same, v, start)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)


def test_attention_picks_the_dominant_key():
    """A query aligned with one allowed key and scaled up attends only to it
    (the softmax tends to the argmax), so o_i -> v_j."""
    T, D = 6, 6
    k = np.eye(T, D)[None, None] * 1.0
    v = np.arange(T * D, dtype=float).reshape(1, 1, T, D)
    q = np.zeros((1, 1, T, D))
    q[0, 0, 5, 2] = 400.0  # query 5 points at key 2
    o, _ = oracle.attention_fwd(q, k, v, np.zeros((1, T), np.int64))
    np.testing.assert_allclose(o[0, 0, 5], v[0, 0, 2], rtol=0, atol=1e-9)


def test_zero_layer_model_is_a_bigram_lookup():
    """P7, L = 0: the network reduces to z = LN_f(wte[tok] + wpe[pos]) wte^T,
    a lookup of the current token and position, the bigram-shaped model the
    Smallem series starts from. Checked with torch's layer_norm as the library
    routine for the normalisation."""
    torch = pytest.importorskip("torch")
    cfg = tiny_cfg(n_layers=0)
    params = random_params(cfg, 6)
    tok, tgt, _ = tiny_batch(cfg)
    z, _ = oracle.forward(params, cfg, tok, None, keep=False)
    x = torch.tensor(params["wte"][tok] + params["wpe"][np.arange(6)][None])
    h = torch.nn.functional.layer_norm(x, (cfg.d_model,), torch.tensor(params["lnf.g"]),
                                       torch.tensor(params["lnf.b"]), cfg.ln_eps)
    np.testing.assert_allclose(z, (h @ torch.tensor(params["wte"]).T).numpy(), rtol=1e-12, atol=1e-13)


# -------------------------------------------------------------- LayerNorm pins

def test_layernorm_closed_form_and_library():
    """An alternating row a, -a, a, ... has mean 0 and biased variance a^2, so
    LN gives g * (+-a) / sqrt(a^2 + eps) + b; generic rows match torch's
    layer_norm."""
    torch = pytest.importorskip("torch")
    C, a, eps = 8, 3.0, 1e-5
    x = np.array([a, -a] * (C // 2))[None]
    g = np.linspace(0.5, 2.0, C)
    b = np.linspace(-1, 1, C)
    y, mu, rstd = oracle.layernorm_fwd(x, g, b, eps)
    np.testing.assert_allclose(y[0], g * x[0] / math.sqrt(a * a + eps) + b, rtol=1e-14)
    assert abs(mu[0]) < 1e-15 and abs(rstd[0] - 1 / math.sqrt(a * a + eps)) < 1e-15
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 37)) * 3 + 1
    g, b = rng.standard_normal(37), rng.standard_normal(37)
    y, _, _ = oracle.layernorm_fwd(x, g, b, eps)
    ref = torch.nn.functional.layer_norm(torch.tensor(x), (37,), torch.tensor(g), torch.tensor(b), eps)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_layernorm_backward_sum_rules():
    """P9: per row, sum_c dx = 0, and at eps = 0 also sum_c dx * xhat = 0."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 24)) * 2 + 0.5
    g = rng.standard_normal(24)
    dy = rng.standard_normal((5, 24))
    for eps in (1e-5, 0.0):
        _, mu, rstd = oracle.layernorm_fwd(x, g, np.zeros(24), eps)
        dx, _, _ = oracle.layernorm_bwd(dy, x, mu, rstd, g)
        np.testing.assert_allclose(dx.sum(axis=-1), 0.0, atol=1e-12)
        if eps == 0.0:
            xhat = (x - mu[:, None]) * rstd[:, None]
            np.testing.assert_allclose((dx * xhat).sum(axis=-1), 0.0, atol=1e-12)


# ------------------------------------------------------------- P10, P11 rules

def test_attention_backward_sum_rules():
    """P10: dS rows sum to 0, so sum_j dk_j = 0 over each document (hence the
    k-part of the QKV bias gradient is 0), and sum_j dv_j = sum_i do_i over
    each document."""
    rng = np.random.default_rng(7)
    B, H, T, D = 1, 2, 9, 4
    q, k, v, do = rng.standard_normal((4, B, H, T, D))
    start = np.array([[0, 0, 0, 3, 3, 3, 3, 7, 7]])
    dq, dk, dv = oracle.attention_bwd(do, q, k, v, start)
    for s, e in ((0, 3), (3, 7), (7, 9)):
        np.testing.assert_allclose(dk[..., s:e, :].sum(axis=-2), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv[..., s:e, :].sum(axis=-2), do[..., s:e, :].sum(axis=-2), atol=1e-12)
    cfg = tiny_cfg()
    params = random_params(cfg, 3)
    tok, tgt, doc = tiny_batch(cfg)
    _, grads, _, _ = oracle.loss_and_grads(params, cfg, tok, tgt, doc)
    C = cfg.d_model
    for l in range(cfg.n_layers):
        db = grads[f"blocks.{l}.attn.b_qkv"]
        assert np.abs(db[C:2 * C]).max() <= 1e-12 * np.abs(db).max()


def test_head_and_tied_embedding_sum_rules():
    """P11: dz rows sum to 0, so the head part of dwte sums to 0 over the
    vocabulary; with the tied head, sum_v dwte = sum_p dwpe (both equal the sum
    of the embedding-output gradient)."""
    cfg = tiny_cfg()
    params = random_params(cfg, 4)
    tok, tgt, doc = tiny_batch(cfg)
    _, grads, _, _ = oracle.loss_and_grads(params, cfg, tok, tgt, doc)
    np.testing.assert_allclose(grads["wte"].sum(axis=0), grads["wpe"].sum(axis=0), atol=1e-12)


def test_untied_head_reduces_to_tied_and_bias_rule():
    """A separate head equal to wte with a zero bias computes the tied model:
    the same logits and loss, and the tied wte gradient splits into the
    embedding part (untied wte) plus the head part (head.w). The head bias
    gradient is the column sum of dz, and dz rows sum to 0, so it sums to 0
    over the vocabulary."""
    cfg = tiny_cfg()
    ucfg = tiny_cfg(untied_head=True)
    params = random_params(cfg, 12)
    tok, tgt, doc = tiny_batch(cfg)
    loss_t, g_t, z_t, _ = oracle.loss_and_grads(params, cfg, tok, tgt, doc)
    up = dict(params, **{"head.w": params["wte"].copy(), "head.b": np.zeros(cfg.vocab)})
    loss_u, g_u, z_u, _ = oracle.loss_and_grads(up, ucfg, tok, tgt, doc)
    assert loss_u == pytest.approx(loss_t, rel=1e-14)
    np.testing.assert_allclose(z_u, z_t, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(g_u["wte"] + g_u["head.w"], g_t["wte"], rtol=1e-12, atol=1e-14)
    for k in params:
        if k != "wte":
            np.testing.assert_allclose(g_u[k], g_t[k], rtol=1e-12, atol=1e-14)
    assert abs(g_u["head.b"].sum()) < 1e-14
    # a bias that is constant over the vocabulary shifts every logit of a row
    # equally: softmax, loss and every other gradient are unchanged
    up2 = dict(up, **{"head.b": np.full(cfg.vocab, 0.75)})
    loss_c, g_c, z_c, _ = oracle.loss_and_grads(up2, ucfg, tok, tgt, doc)
    assert loss_c == pytest.approx(loss_u, rel=1e-13)
    np.testing.assert_allclose(z_c - 0.75, z_u, rtol=1e-13, atol=1e-13)
    for k in g_u:
        np.testing.assert_allclose(g_c[k], g_u[k], rtol=1e-11, atol=1e-14)


# ----------------------------------------------------------- P12, P13: AdamW

def test_adam_closed_form_first_two_steps():
    """P12: from m = v = 0, step 1 gives m = (1-b1) g, v = (1-b2) g^2 and, after
    bias correction, p1 = p0 - lr (g / (|g| + eps) + wd p0); step 2 with
    gradient g2 follows from the recurrence with corrections 1-b1^2, 1-b2^2."""
    rng = np.random.default_rng(8)
    p0, g1, g2 = rng.standard_normal((3, 50))
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.1
    z = np.zeros(50)
    p1, m1, v1 = oracle.adamw(p0, g1, z, z, 1, lr, b1, b2, eps, wd)
    np.testing.assert_allclose(m1, 0.1 * g1, rtol=1e-15)
    np.testing.assert_allclose(v1, 0.001 * g1 * g1, rtol=1e-13)
    np.testing.assert_allclose(p1, p0 - lr * (g1 / (np.abs(g1) + eps) + wd * p0), rtol=1e-13)
    p2, m2, v2 = oracle.adamw(p1, g2, m1, v1, 2, lr, b1, b2, eps, wd)
    mh = (0.09 * g1 + 0.1 * g2) / (1 - 0.81)
    vh = (0.999 * 0.001 * g1 ** 2 + 0.001 * g2 ** 2) / (1 - 0.999 ** 2)
    np.testing.assert_allclose(p2, p1 - lr * (mh / (np.sqrt(vh) + eps) + wd * p1), rtol=1e-12)


def test_adamw_matches_torch_optimizer():
    """P12: the update equals torch.optim.AdamW (an independent implementation
    with decoupled decay) over three steps."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    p = rng.standard_normal(40)
    grads = rng.standard_normal((3, 40))
    lr, b1, b2, eps, wd = 3e-4, 0.9, 0.999, 1e-8, 0.1
    tp = torch.tensor(p.copy(), requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    m = v = np.zeros(40)
    for t in range(3):
        p, m, v = oracle.adamw(p, grads[t], m, v, t + 1, lr, b1, b2, eps, wd)
        tp.grad = torch.tensor(grads[t])
        opt.step()
    np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15)


def test_clip_to_global_norm():
    """P13 (RustGPT page: L2 norm capped at 5.0): when the global norm n
    exceeds the clip, the scaled gradients have norm exactly the clip; below
    it they are unchanged; a non-finite norm skips the update."""
    rng = np.random.default_rng(10)
    grads = {"a": rng.standard_normal((3, 4)) * 4, "b": rng.standard_normal(7) * 4}
    n, s = oracle.grad_norm_and_scale(grads, 5.0)
    assert n > 5.0
    assert abs(math.sqrt(sum(((s * g) ** 2).sum() for g in grads.values())) - 5.0) <= 1e-12 * 5
    n2, s2 = oracle.grad_norm_and_scale(grads, 1e9)
    assert s2 == 1.0 and abs(n2 - n) < 1e-12
    cfg = tiny_cfg()
    params = random_params(cfg, 12)
    params["blocks.0.mlp.w_fc"][0, 0] = np.nan
    tok, tgt, doc = tiny_batch(cfg)
    zeros = {k: np.zeros_like(v) for k, v in params.items()}
    out = oracle.train_step(params, zeros, zeros, cfg, tok, tgt, doc, step=1, lr=1e-3, clip=1.0)
    assert not out["finite"]
    for k in params:
        assert np.array_equal(out["params"][k], params[k], equal_nan=True)
        assert np.all(out["m"][k] == 0) and np.all(out["v"][k] == 0)


def test_gelu_tanh_form_close_to_exact_gelu():
    """The tanh form of GELU stays within 5e-4 of the exact u * Phi(u)
    (math.erf), the known accuracy of that approximation; without the cubic
    term or with a wrong constant it would miss by far more."""
    u = np.linspace(-8, 8, 4001)
    exact = np.array([0.5 * x * (1 + math.erf(x / math.sqrt(2))) for x in u])
    assert np.abs(oracle.gelu(u) - exact).max() < 5e-4
    # derivative against central differences of the exact function's form
    h = 1e-6
    fd = (oracle.gelu(u + h) - oracle.gelu(u - h)) / (2 * h)
    np.testing.assert_allclose(oracle.gelu_grad(u), fd, atol=1e-8)
    assert oracle.gelu(np.array([0.0]))[0] == 0.0


# ----------------------------------------------------------- index and CSR

def test_index_layout_golden():
    """Bit-exact start/pos on hand-derived packed rows (tests/golden)."""
    rows = []
    with open(os.path.join(GOLDEN, "index_layout.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = [np.array(p.split(), np.int64) for p in line.split("|")]
            rows.append(parts)
    doc = np.stack([r[0] for r in rows]).astype(np.int32)
    start, pos = oracle.index_layout(doc, doc.shape[0], doc.shape[1])
    assert np.array_equal(start, np.stack([r[1] for r in rows]))
    assert np.array_equal(pos, np.stack([r[2] for r in rows]))
    with pytest.raises(ValueError):
        oracle.index_layout(np.array([[0, 1, 0]]), 1, 3)
    with pytest.raises(ValueError):
        oracle.index_layout(np.zeros((1, 5), np.int32), 1, 5, max_seq=4)


def test_csr_is_a_stable_sort():
    """The CSR gather order equals a library stable argsort of the keys."""
    rng = np.random.default_rng(12)
    keys = rng.integers(0, 9, 200)
    off, perm = oracle.csr_by_key(keys, 12)
    assert np.array_equal(perm, np.argsort(keys, kind="stable"))
    assert np.array_equal(np.diff(off), np.bincount(keys, minlength=12))


def test_embedding_backward_against_dense_one_hot():
    """Scatter-add equals the dense one-hot product onehot(tok)^T dx."""
    rng = np.random.default_rng(13)
    tok = rng.integers(0, 7, (3, 5))
    pos = np.tile(np.arange(5), (3, 1))
    dx = rng.standard_normal((3, 5, 4))
    dwte, dwpe = oracle.embedding_bwd(dx, tok, pos, 7, 6)
    oh = np.eye(7)[tok.reshape(-1)]
    np.testing.assert_allclose(dwte, oh.T @ dx.reshape(-1, 4), rtol=1e-14)
    np.testing.assert_allclose(dwpe[:5], dx.sum(axis=0), rtol=1e-14)
    assert np.all(dwpe[5] == 0)
