"""Multi-step training driver: the scheduled learning rate and several steps
against the oracle, checkpoint save/resume (bit-exact continuation, the file
read back by an independent safetensors reader, mismatches rejected), and a
loss-descent run on learnable synthetic text.

Tolerances: the fp32 multi-step parity uses the per-tensor bounds of the
single-step parity (rel <= 1e-4 on gradients and loss; the update within a few
fp32 ulps of p plus 1e-3 of |update|), applied after every step. Resume and
run-to-run checks are bit-exact.
"""
import dataclasses
import os

import numpy as np
import pytest

import oracle
import synth
from helpers import dev, rel, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sd():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    import scratch_decoder_only_amd as m
    return m


def _model(sd, shape, B):
    model = sd.Model(shape, max_batch=B)
    model.set(sd.LM_PARAMS, synth.init_params(shape))
    return model


def _opt(shape):
    return dict(beta1=shape.beta1, beta2=shape.beta2, eps=shape.eps, weight_decay=shape.weight_decay,
                clip=shape.clip)


def test_scheduled_steps_match_oracle(sd):
    """Three fp32 steps with warm-up 2 and cosine to lr/10 at step 3, each
    checked like a single step (loss, norm, logits, gradients, update)."""
    from test_gpu_step import compare
    t = torch()
    shape = synth.SHAPES["C1"]
    b = synth.make_batch(shape)
    model = _model(sd, shape, shape.batch)
    lr_max, lr_min, W, S = shape.lr, shape.lr / 10, 2, 3
    f32 = lambda x: float(np.float32(x))
    batch = (dev(b.tokens), dev(b.targets), None)
    params = {k: a.astype(np.float64) for k, a in model.get(sd.LM_PARAMS).items()}
    m0 = v0 = None
    for step in range(1, S + 1):
        logits = model.forward_logits(batch[0])
        sd.train(model, batch, 1, start_step=step, lr_max=lr_max, lr_min=lr_min, warmup_steps=W, total_steps=S,
                 **_opt(shape))
        t.cuda.synchronize()
        got = {"stats": model.stats.cpu().numpy().astype(np.float64), "logits": logits.cpu().numpy(),
               "grads": model.get(sd.LM_GRADS), "params": model.get(sd.LM_PARAMS),
               "m": model.get(sd.LM_ADAM_M), "v": model.get(sd.LM_ADAM_V)}
        zeros = {k: np.zeros_like(a) for k, a in params.items()}
        lr = oracle.lr_schedule(step, W, S, f32(lr_max), f32(lr_min))
        ref = oracle.train_step(params, m0 or zeros, v0 or zeros, shape, b.tokens, b.targets, None, step=step,
                                lr=f32(lr), beta1=f32(shape.beta1), beta2=f32(shape.beta2), eps=f32(shape.eps),
                                weight_decay=shape.weight_decay, clip=f32(shape.clip))
        compare(shape, got, ref, params, step, m0, v0)
        # the next step starts from the GPU's fp32 state on both sides
        params = {k: a.astype(np.float64) for k, a in got["params"].items()}
        m0 = {k: a.astype(np.float64) for k, a in got["m"].items()}
        v0 = {k: a.astype(np.float64) for k, a in got["v"].items()}


@pytest.mark.parametrize("name", ["C1", "C2", "C2-fp16"])
def test_checkpoint_resume_is_bit_exact(sd, name, tmp_path):
    """fp16: the checkpoint also carries the loss scale and its run of finite
    steps (interval 2 here, so both change during the run)."""
    t = torch()
    fp16 = name.endswith("fp16")
    shape = synth.SHAPES[name.split("-")[0]]
    if fp16:
        shape = shape.replace(precision="fp16")
    b = synth.make_batch(shape)
    batch = (dev(b.tokens), dev(b.targets), None)
    kw = dict(lr_max=shape.lr, lr_min=shape.lr / 10, warmup_steps=2, total_steps=6, **_opt(shape))
    path = str(tmp_path / "ck.safetensors")

    def fresh():
        mdl = _model(sd, shape, shape.batch)
        if fp16:
            mdl.set_loss_scaler(scale=1024.0, interval=2)
        return mdl

    a = fresh()
    la = sd.train(a, batch, 6, save_every=3, ckpt_path=path, **kw)   # saves after step 3 and step 6
    os.replace(path, path + ".6")
    a3 = fresh()
    sd.train(a3, batch, 3, save_every=3, ckpt_path=path, **kw)       # the step-3 checkpoint
    bmodel = sd.Model(shape, max_batch=shape.batch)
    assert bmodel.load(path) == 3
    for which in (sd.LM_PARAMS, sd.LM_ADAM_M, sd.LM_ADAM_V):
        assert np.array_equal(bmodel.get_flat(which), a3.get_flat(which))
    if fp16:
        assert bmodel.loss_scaler() == a3.loss_scaler()
        assert a3.loss_scaler()["scale"] == 2048.0 and a3.loss_scaler()["good_steps"] == 1
    lb = sd.train(bmodel, batch, 3, start_step=4, **kw)
    t.cuda.synchronize()
    for which in (sd.LM_PARAMS, sd.LM_ADAM_M, sd.LM_ADAM_V):
        assert np.array_equal(bmodel.get_flat(which), a.get_flat(which))
    assert t.equal(lb, la[3:])
    # the step-6 file restores the uninterrupted run's state exactly
    c = sd.Model(shape, max_batch=shape.batch)
    assert c.load(path + ".6") == 6
    assert np.array_equal(c.get_flat(sd.LM_PARAMS), a.get_flat(sd.LM_PARAMS))


def test_checkpoint_file_is_safetensors(sd, tmp_path):
    from safetensors.numpy import load_file
    from safetensors import safe_open
    shape = synth.SHAPES["C1"]
    model = _model(sd, shape, shape.batch)
    b = synth.make_batch(shape)
    sd.train(model, (dev(b.tokens), dev(b.targets), None), 2, lr_max=shape.lr, **_opt(shape))
    path = str(tmp_path / "c1.safetensors")
    model.save(path, 2)
    data = load_file(path)
    p, m, v = model.get(sd.LM_PARAMS), model.get(sd.LM_ADAM_M), model.get(sd.LM_ADAM_V)
    assert len(data) == 3 * len(p)
    for name in p:
        for prefix, ref in (("param.", p), ("adam_m.", m), ("adam_v.", v)):
            got = data[prefix + name]
            assert got.dtype == np.float32
            assert np.array_equal(got.reshape(ref[name].shape), ref[name])
    with safe_open(path, framework="numpy") as f:
        meta = f.metadata()
    assert meta["format"] == "lmstep-checkpoint" and meta["step"] == "2"
    assert int(meta["vocab"]) == shape.vocab and int(meta["n_layers"]) == shape.n_layers


def test_checkpoint_mismatch_and_bad_files_are_rejected(sd, tmp_path):
    shape = synth.SHAPES["C1"]
    model = _model(sd, shape, shape.batch)
    path = str(tmp_path / "c1.safetensors")
    model.save(path, 1)
    other = dataclasses.replace(shape, n_layers=2)
    with pytest.raises(RuntimeError, match="n_layers"):
        sd.Model(other, max_batch=shape.batch).load(path)
    raw = open(path, "rb").read()
    trunc = str(tmp_path / "trunc.safetensors")
    open(trunc, "wb").write(raw[: len(raw) // 2])
    fresh = sd.Model(shape, max_batch=shape.batch)
    with pytest.raises(RuntimeError):
        fresh.load(trunc)
    garbage = str(tmp_path / "garbage.safetensors")
    open(garbage, "wb").write(b"\x10\x00\x00\x00\x00\x00\x00\x00{not json here}")
    with pytest.raises(RuntimeError):
        fresh.load(garbage)
    with pytest.raises(RuntimeError):
        fresh.load(str(tmp_path / "missing.safetensors"))


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_loss_descends_on_learnable_text(sd, name):
    """Warm-up then cosine decay on text whose next id is a function of the
    current one: the loss falls from about ln V to a small fraction of it."""
    t = torch()
    shape = synth.SHAPES[name]
    b = synth.structured_batch(shape, batch=shape.batch)
    model = _model(sd, shape, shape.batch)
    steps = 80
    losses = sd.train(model, (dev(b.tokens), dev(b.targets), None), steps, lr_max=3e-3, lr_min=3e-4,
                      warmup_steps=10, **_opt(shape)).cpu().numpy()
    t.cuda.synchronize()
    assert np.all(np.isfinite(losses))
    assert abs(losses[0] - np.log(shape.vocab)) < 0.5
    assert losses[-10:].mean() < 0.25 * losses[:5].mean(), losses
