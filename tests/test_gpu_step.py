"""Full-step parity of train_step / forward_logits (include/lmstep.h) against
the CPU oracle on the seeded workloads, plus invariants that hold at any size.

Tolerances (relative Frobenius error rel, cosine cos, per tensor):
  fp32 path: loss, logits, every gradient and the grad norm rel <= 1e-4; the
    update p' - p rel <= 1e-3 on elements whose oracle gradient is not
    negligible (|g| >= 1e-3 rms of its tensor);
  bf16 path: loss rel <= 2e-2; logits and every gradient cos >= 0.999; the
    update cos >= 0.99 on the same mask.
The k-part of the QKV bias gradient is 0 analytically (dS rows sum to 0), so
it is compared with an absolute bound against the tensor's scale instead.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from helpers import cos, dev, host, rel, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sd():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    import scratch_decoder_only_amd as m
    return m


def _inputs(shape, batch):
    b = synth.make_batch(shape)
    tok, tgt = b.tokens[:batch], b.targets[:batch]
    doc = None if b.doc_ids is None else b.doc_ids[:batch]
    return tok, tgt, doc


def run_gpu(sd, shape, tok, tgt, doc, params, step=1, m=None, v=None):
    t = torch()
    B = tok.shape[0]
    model = sd.Model(shape, max_batch=B)
    model.set(sd.LM_PARAMS, params)
    if m is not None:
        model.set(sd.LM_ADAM_M, m)
        model.set(sd.LM_ADAM_V, v)
    tok_d, tgt_d = dev(tok), dev(tgt)
    doc_d = None if doc is None else dev(doc)
    logits = model.forward_logits(tok_d, doc_d)
    # fp16: the gradient buffer holds S g for the loss scale S of the step
    S = model.loss_scaler()["scale"] if shape.precision == "fp16" else 1.0
    stats = model.train_step(tok_d, tgt_d, doc_d, lr=shape.lr, step=step, beta1=shape.beta1, beta2=shape.beta2,
                             eps=shape.eps, weight_decay=shape.weight_decay, clip=shape.clip)
    t.cuda.synchronize()
    return {"model": model, "logits": host(logits), "stats": stats.cpu().numpy().astype(np.float64),
            "grads": {k: g / S for k, g in model.get(sd.LM_GRADS).items()}, "params": model.get(sd.LM_PARAMS),
            "m": model.get(sd.LM_ADAM_M), "v": model.get(sd.LM_ADAM_V)}


def run_oracle(shape, tok, tgt, doc, params, step=1, m=None, v=None):
    zeros = {k: np.zeros_like(a, dtype=np.float64) for k, a in params.items()}
    return oracle.train_step(params, m or zeros, v or zeros, shape, tok, tgt, doc, step=step, lr=shape.lr,
                             beta1=shape.beta1, beta2=shape.beta2, eps=shape.eps,
                             weight_decay=shape.weight_decay, clip=shape.clip)


def _ulp_close(got, ref, base, rtol):
    """|got - ref| <= 4 ulp(fp32 of base) + rtol |ref - base|: p' is stored in
    fp32, so the update p' - p is only known to the ulp of p."""
    ulp = np.abs(base.astype(np.float64)) * 2.0 ** -23 + 1e-38
    return np.all(np.abs(got - ref) <= 4 * ulp + rtol * np.abs(ref - base))


def compare(shape, got, ref, params, step=1, m0=None, v0=None):
    fp32 = shape.precision == "fp32"
    C = shape.d_model
    loss, ref_loss = got["stats"][0], ref["loss"]
    assert abs(loss - ref_loss) <= (1e-4 if fp32 else 2e-2) * abs(ref_loss), (loss, ref_loss)
    assert int(got["stats"][3]) == ref["n_valid"]
    assert int(got["stats"][2]) == 0
    assert abs(got["stats"][1] - ref["grad_norm"]) <= (1e-4 if fp32 else 2e-2) * ref["grad_norm"]
    z = ref["logits"]
    if fp32:
        assert rel(got["logits"], z) <= 1e-4
    else:
        assert cos(got["logits"], z) >= 0.999
    for k, g_ref in ref["grads"].items():
        g = got["grads"][k]
        if k.endswith("attn.b_qkv"):
            scale = max(np.abs(g_ref).max(), 1e-30)
            assert np.abs(g[C:2 * C]).max() <= (1e-4 if fp32 else 2e-2) * scale, k
            g, g_ref = np.concatenate([g[:C], g[2 * C:]]), np.concatenate([g_ref[:C], g_ref[2 * C:]])
        if fp32:
            assert rel(g, g_ref) <= 1e-4, (k, rel(g, g_ref))
        else:
            assert cos(g, g_ref) >= 0.999, (k, cos(g, g_ref))
    if fp32:
        # the update against the oracle's, where the oracle gradient is not negligible
        for k in ref["grads"]:
            gr = ref["grads"][k]
            mask = np.abs(gr) >= 1e-3 * math.sqrt(np.mean(gr ** 2) + 1e-300)
            if k.endswith("attn.b_qkv"):
                mask[C:2 * C] = False
            dp, dp_ref = (got["params"][k] - params[k])[mask], (ref["params"][k] - params[k])[mask]
            if dp_ref.size:
                assert rel(dp, dp_ref) <= 1e-3, (k, rel(dp, dp_ref))
                assert rel(got["m"][k][mask], ref["m"][k][mask]) <= 1e-3, k
    else:
        # bf16: the first Adam steps are ~lr sign(g), which turns gradient noise
        # at bf16 level into sign flips; the optimiser stage is checked as the
        # oracle's clip + AdamW applied to the GPU's own gradients
        # the hyper-parameters cross the C ABI as fp32 (lm_optim), so the oracle
        # takes the same fp32-rounded values here (1 - 0.999f is 1.3e-5 off 1e-3)
        f32 = lambda x: float(np.float32(x))
        gg = {k: got["grads"][k].astype(np.float64) for k in got["grads"]}
        n, s = oracle.grad_norm_and_scale(gg, f32(shape.clip))
        assert abs(got["stats"][1] - n) <= 1e-5 * n
        for k in gg:
            mm = np.zeros_like(gg[k]) if m0 is None else m0[k]
            vv = np.zeros_like(gg[k]) if v0 is None else v0[k]
            pe, me, ve = oracle.adamw(params[k], gg[k], mm, vv, step, f32(shape.lr), f32(shape.beta1),
                                      f32(shape.beta2), f32(shape.eps), f32(shape.weight_decay), s)
            assert _ulp_close(got["params"][k], pe, params[k], 1e-4), k
            assert rel(got["m"][k], me) <= 1e-5 and rel(got["v"][k], ve) <= 1e-5, k


@pytest.mark.parametrize("name,batch", [("C1", 4), ("C2", 16), ("C3", 32), ("C4", 1), ("C5", 1)])
def test_train_step_matches_oracle(sd, name, batch):
    shape = synth.SHAPES[name].with_batch(batch)
    print(f"train_step parity {name} B={batch} T={shape.seq}", flush=True)
    tok, tgt, doc = _inputs(shape, batch)
    params = synth.init_params(shape)
    got = run_gpu(sd, shape, tok, tgt, doc, params)
    ref = run_oracle(shape, tok, tgt, doc, params)
    compare(shape, got, ref, params)


@pytest.mark.parametrize("name,batch", [("C1", 4), ("C2", 16), ("C3", 8)])
def test_untied_head_step_matches_oracle(sd, name, batch):
    """A separate vocabulary projection with bias (head.w, head.b) instead of
    the tied one, checked like the tied step; the bias starts off zero so its
    forward term is exercised too."""
    shape = synth.SHAPES[name].with_batch(batch).replace(untied_head=True)
    print(f"untied-head train_step parity {name} B={batch} T={shape.seq}", flush=True)
    tok, tgt, doc = _inputs(shape, batch)
    params = synth.init_params(shape)
    params["head.b"] = synth.random_tensor(np.random.default_rng(3), params["head.b"].shape, 0.5)
    got = run_gpu(sd, shape, tok, tgt, doc, params)
    ref = run_oracle(shape, tok, tgt, doc, params)
    assert set(got["grads"]) == set(ref["grads"]) and "head.w" in got["grads"]
    compare(shape, got, ref, params)


@pytest.mark.parametrize("untied", [False, True])
def test_vocab_padding_rows_stay_zero(sd, untied):
    """bf16 reserves round_up(V, 128) rows for wte (and head.w, head.b): after
    parameters with garbage in those gaps are set and a step runs, every
    buffer's padding is zero and the logits equal those of a clean upload."""
    t = torch()
    shape = synth.C2.with_batch(2).replace(untied_head=untied)
    tok, tgt, doc = _inputs(shape, 2)
    params = synth.init_params(shape)
    clean = sd.Model(shape, max_batch=2)
    clean.set(sd.LM_PARAMS, params)
    model = sd.Model(shape, max_batch=2)
    table = model.table
    flat = np.zeros(model.total, np.float32)
    for name, off, rows, cols in table:
        flat[off:off + rows * cols] = params[name].reshape(-1)
    ends = sorted((off, off + rows * cols) for _, off, rows, cols in table)
    gaps = [(e, nxt[0]) for (o, e), nxt in zip(ends, ends[1:] + [(model.total, 0)]) if nxt[0] > e]
    for a, b in gaps:
        flat[a:b] = 7.0
    model.set_flat_device(sd.LM_PARAMS, dev(flat))
    za = clean.forward_logits(dev(tok)).cpu().numpy()
    zb = model.forward_logits(dev(tok)).cpu().numpy()
    assert np.array_equal(za, zb)
    model.train_step(dev(tok), dev(tgt), None, lr=shape.lr, step=1, clip=shape.clip)
    t.cuda.synchronize()
    for which in (sd.LM_PARAMS, sd.LM_GRADS, sd.LM_ADAM_M, sd.LM_ADAM_V):
        f = model.get_flat(which)
        for name, off, rows, cols in table:
            if name in ("wte", "head.w", "head.b"):
                nxt = min([o for o, _ in ends if o > off] + [model.total])
                assert not np.any(f[off + rows * cols:nxt]), (which, name)


@pytest.mark.parametrize("name,batch", [("C2", 16), ("C3", 8), ("C4", 1)])
def test_fp16_step_matches_oracle(sd, name, batch):
    """fp16 operands with the default loss scale (2^16): the same bounds as
    the bf16 path, on gradients divided by the step's scale."""
    shape = synth.SHAPES[name].with_batch(batch).replace(precision="fp16")
    print(f"fp16 train_step parity {name} B={batch} T={shape.seq}", flush=True)
    tok, tgt, doc = _inputs(shape, batch)
    params = synth.init_params(shape)
    got = run_gpu(sd, shape, tok, tgt, doc, params)
    assert got["model"].loss_scaler()["scale"] == 65536.0  # one finite step: no change yet
    ref = run_oracle(shape, tok, tgt, doc, params)
    compare(shape, got, ref, params)


def test_fp16_loss_scale_backoff_and_growth(sd):
    """An overflowing scale (2^60: the scaled loss gradient exceeds fp16)
    skips the step bit-exactly and halves S until the gradients are finite;
    then S doubles after every `interval` finite steps. The scale sequence
    follows the oracle's rule fed with the steps' finite flags."""
    t = torch()
    shape = synth.C2.with_batch(4).replace(precision="fp16")
    tok, tgt, doc = _inputs(shape, 4)
    model = sd.Model(shape, max_batch=4)
    model.set(sd.LM_PARAMS, synth.init_params(shape))
    model.set_loss_scaler(scale=2.0 ** 60, growth=2.0, backoff=0.25, interval=3)
    p0 = model.get_flat(sd.LM_PARAMS)
    flags, scales = [], []
    for step in range(1, 31):
        before = [model.get_flat(b) for b in (sd.LM_PARAMS, sd.LM_ADAM_M, sd.LM_ADAM_V)]
        st = model.train_step(dev(tok), dev(tgt), None, lr=shape.lr, step=step, clip=shape.clip)
        finite = (int(st.cpu().numpy()[2]) & 1) == 0
        flags.append(finite)
        sc = model.loss_scaler()
        scales.append((sc["scale"], sc["good_steps"]))
        if not finite:  # skipped: parameters and moments untouched
            after = [model.get_flat(b) for b in (sd.LM_PARAMS, sd.LM_ADAM_M, sd.LM_ADAM_V)]
            assert all(np.array_equal(x, y) for x, y in zip(before, after)), step
    t.cuda.synchronize()
    assert not flags[0] and any(flags), flags
    assert scales == oracle.loss_scale_trace(2.0 ** 60, flags, 2.0, 0.25, 3)
    assert not np.array_equal(model.get_flat(sd.LM_PARAMS), p0)


def test_fp16_scaler_is_fp16_only(sd):
    shape = synth.C1
    model = sd.Model(shape, max_batch=1)
    with pytest.raises(RuntimeError):
        model.loss_scaler()
    m16 = sd.Model(shape.replace(precision="fp16"), max_batch=1)
    with pytest.raises(RuntimeError):
        m16.set_loss_scaler(scale=0.0)
    with pytest.raises(RuntimeError):
        m16.set_loss_scaler(interval=0)


def test_fp32_path_on_a_packed_workload(sd):
    """The fp32 path with a block-diagonal mask (C3's packing at C1-like size)."""
    shape = synth.C3.replace(precision="fp32", batch=4, seq=256, max_seq=256, vocab=300, n_layers=2)
    tok, tgt, doc = _inputs(shape, 4)
    params = synth.init_params(shape)
    got = run_gpu(sd, shape, tok, tgt, doc, params)
    ref = run_oracle(shape, tok, tgt, doc, params)
    compare(shape, got, ref, params)


def test_second_step_and_resume_bit_exact(sd):
    """Step 2 from step 1's state matches the oracle's two steps, and resuming
    through model_get/model_set is bit-identical to running on."""
    t = torch()
    shape = synth.C2.with_batch(4, 64)
    tok, tgt, doc = _inputs(shape, 4)
    params = synth.init_params(shape)
    got1 = run_gpu(sd, shape, tok, tgt, doc, params)
    model = got1["model"]
    tok_d, tgt_d = dev(tok), dev(tgt)
    st = model.train_step(tok_d, tgt_d, None, lr=shape.lr, step=2, weight_decay=shape.weight_decay, clip=shape.clip)
    t.cuda.synchronize()
    cont = model.get(sd.LM_PARAMS)
    got2 = run_gpu(sd, shape, tok, tgt, doc, got1["params"], step=2, m=got1["m"], v=got1["v"])
    for k in cont:
        assert np.array_equal(cont[k], got2["params"][k]), k
    # step 2 from the GPU's step-1 state against the oracle from the same state
    ref2 = run_oracle(shape, tok, tgt, doc, got1["params"], step=2, m=got1["m"], v=got1["v"])
    compare(shape, got2, ref2, got1["params"], step=2, m0=got1["m"], v0=got1["v"])


def test_run_to_run_bit_identical(sd):
    shape = synth.C3.with_batch(8)
    tok, tgt, doc = _inputs(shape, 8)
    params = synth.init_params(shape)
    a = run_gpu(sd, shape, tok, tgt, doc, params)
    b = run_gpu(sd, shape, tok, tgt, doc, params)
    assert np.array_equal(a["stats"], b["stats"])
    for k in a["grads"]:
        assert np.array_equal(a["grads"][k], b["grads"][k]), k
        assert np.array_equal(a["params"][k], b["params"][k]), k


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_causality_bit_exact(sd, name):
    """Changing tokens after t leaves the logits at positions <= t bit-identical."""
    t = torch()
    shape = synth.SHAPES[name].with_batch(2, 128 if name == "C2" else 80)
    tok, _, _ = _inputs(shape, 2)
    model = sd.Model(shape, max_batch=2)
    model.set(sd.LM_PARAMS, synth.init_params(shape))
    z0 = model.forward_logits(dev(tok)).cpu().numpy()
    rng = np.random.default_rng(1)
    for cut in (0, 31, shape.seq - 2):
        tok2 = tok.copy()
        tok2[:, cut + 1:] = rng.integers(0, shape.vocab, tok2[:, cut + 1:].shape)
        z1 = model.forward_logits(dev(tok2)).cpu().numpy()
        t.cuda.synchronize()
        assert np.array_equal(z0[:, :cut + 1], z1[:, :cut + 1]), cut
        assert not np.array_equal(z0[:, cut + 1:], z1[:, cut + 1:])


@pytest.mark.parametrize("batch", [8, 70])
def test_unpacked_position_gradient_equals_sorted_path_bit_exact(sd, batch):
    """Without document ids the position gradient is a column sum over the
    batch; with one document per row it goes through the counting sort. Both
    take the same summation order (chunks of 64 rows, chunk sums in order:
    batch 70 gives two chunks per position), so the whole step is
    bit-identical, the rows of positions past T included."""
    shape = synth.C2.with_batch(batch, 32).replace(n_layers=1)
    tok, tgt, _ = _inputs(shape, batch)
    params = synth.init_params(shape)
    a = run_gpu(sd, shape, tok, tgt, None, params)
    b = run_gpu(sd, shape, tok, tgt, np.zeros(tok.shape, np.int32), params)
    assert np.array_equal(a["stats"], b["stats"])
    for k in a["grads"]:
        assert np.array_equal(a["grads"][k], b["grads"][k]), k
    assert not a["grads"]["wpe"][shape.seq:].any()


def test_single_document_equals_causal_bit_exact(sd):
    shape = synth.C2.with_batch(2, 96)
    tok, _, _ = _inputs(shape, 2)
    model = sd.Model(shape, max_batch=2)
    model.set(sd.LM_PARAMS, synth.init_params(shape))
    za = model.forward_logits(dev(tok)).cpu().numpy()
    zb = model.forward_logits(dev(tok), dev(np.full(tok.shape, 3, np.int32))).cpu().numpy()
    assert np.array_equal(za, zb)


def test_packed_row_equals_separate_documents(sd):
    """Each packed document gets the logits it gets alone in its own row
    (within the bf16 tolerance: tiles align differently)."""
    shape = synth.C3.with_batch(1, 256).replace(max_seq=256)
    rng = np.random.default_rng(2)
    lens = [100, 37, 119]
    tok = rng.integers(0, shape.vocab, (1, 256)).astype(np.int32)
    doc = np.repeat(np.arange(3), lens)[None].astype(np.int32)
    model = sd.Model(shape, max_batch=1)
    model.set(sd.LM_PARAMS, synth.init_params(shape))
    zp = model.forward_logits(dev(tok), dev(doc)).cpu().numpy()
    off = 0
    for L in lens:
        zs = model.forward_logits(dev(np.ascontiguousarray(tok[:, off:off + L]))).cpu().numpy()
        assert cos(zp[:, off:off + L], zs) >= 0.9999
        off += L


@pytest.mark.parametrize("name", ["C4", "C5"])
def test_full_size_sampled_rows(sd, name):
    """At the full benchmark shape: rows 0 and B-1 of the logits against the
    oracle run on those rows alone, the init-loss band, and the gradient sum
    rules (sum_v dwte = sum_p dwpe; the k-part of the QKV bias gradient ~ 0)."""
    t = torch()
    shape = synth.SHAPES[name]
    print(f"full-size sampled check {name}", flush=True)
    b = synth.make_batch(shape)
    params = synth.init_params(shape)
    model = sd.Model(shape, max_batch=shape.batch)
    model.set(sd.LM_PARAMS, params)
    tok_d, tgt_d = dev(b.tokens), dev(b.targets)
    doc_d = None if b.doc_ids is None else dev(b.doc_ids)
    z = model.forward_logits(tok_d, doc_d)
    st = model.train_step(tok_d, tgt_d, doc_d, lr=shape.lr, step=1, weight_decay=shape.weight_decay, clip=shape.clip)
    t.cuda.synchronize()
    for r in (0, shape.batch - 1):
        doc = None if b.doc_ids is None else b.doc_ids[r:r + 1]
        zr, _ = oracle.forward(params, shape, b.tokens[r:r + 1], doc, keep=False)
        assert cos(host(z[r:r + 1]), zr) >= 0.999, r
        del zr
    loss = float(st[0])
    assert abs(loss - (math.log(shape.vocab) + 0.5 * shape.d_model * 0.02 ** 2)) < 0.15
    grads = model.get(sd.LM_GRADS)
    sv, sp = grads["wte"].sum(axis=0), grads["wpe"].sum(axis=0)
    assert rel(sv, sp) <= 2e-2
    C = shape.d_model
    for l in range(shape.n_layers):
        db = grads[f"blocks.{l}.attn.b_qkv"]
        assert np.abs(db[C:2 * C]).max() <= 2e-2 * np.abs(db).max()


def test_error_paths(sd):
    t = torch()
    shape = synth.C1.with_batch(2, 16)
    model = sd.Model(shape, max_batch=2)
    model.set(sd.LM_PARAMS, synth.init_params(shape))
    tok = dev(np.zeros((3, 16), np.int32))
    with pytest.raises(sd.LmError, match="max_batch"):
        model.train_step(tok, tok, None, lr=1e-3, step=1)
    long_tok = dev(np.zeros((1, 81), np.int32))
    with pytest.raises(sd.LmError, match="max_seq"):
        model.forward_logits(long_tok)
    ok = dev(np.zeros((2, 16), np.int32))
    with pytest.raises(sd.LmError, match="step"):
        model.train_step(ok, ok, None, lr=1e-3, step=0)
    # out-of-range tokens are clamped and flagged (bit 1); the step still completes
    bad = np.zeros((2, 16), np.int32)
    bad[0, 3] = 10_000
    st = model.train_step(dev(bad), ok, None, lr=1e-3, step=1)
    t.cuda.synchronize()
    assert int(st[2]) & 2
    # a NaN parameter: the norm is not finite, the update is skipped
    p = synth.init_params(shape)
    p["blocks.1.mlp.w_fc"][2, 3] = np.nan
    model.set(sd.LM_PARAMS, p)
    before = [model.get_flat(w) for w in (sd.LM_PARAMS, sd.LM_ADAM_M, sd.LM_ADAM_V)]
    st = model.train_step(ok, ok, None, lr=1e-3, step=1)
    t.cuda.synchronize()
    assert int(st[2]) & 1
    after = [model.get_flat(w) for w in (sd.LM_PARAMS, sd.LM_ADAM_M, sd.LM_ADAM_V)]
    for a, b in zip(before, after):
        assert np.array_equal(a, b, equal_nan=True)
