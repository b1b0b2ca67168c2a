"""Generation: the next-token kernel (sample_tokens) against the oracle's
choice, and greedy decoding through forward_logits against the oracle's
forward pass.

Where floating point decides the token, several answers can be correct: the
GPU's pick must be a kept id whose oracle interval of the running weight sum
contains u up to a slack of 1e-5 (fp32 sums over up to 50k terms), and must
equal the oracle's pick whenever u is farther than that from every interval
boundary. Greedy on the same fp32 logits is bit-exact. Greedy decoding checks
that every generated id is an argmax of the oracle's logits up to 1e-4 of
their scale, continuing both sides from the GPU's sequence.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import cos, dev, rel, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sd():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    import scratch_decoder_only_amd as m
    return m


def _rows(rng, rows, V, kind):
    if kind == "normal":
        return (rng.standard_normal((rows, V)) * 3).astype(np.float32)
    # coarse values: many ties, including at the k-th value
    return (np.round(rng.standard_normal((rows, V)) * 2) / 2).astype(np.float32)


@pytest.mark.parametrize("V", [257, 8000, 50257])
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_sample_kernel_matches_oracle(sd, V, kind):
    t = torch()
    rng = np.random.Generator(np.random.PCG64(V + len(kind)))
    rows = 24
    z = _rows(rng, rows, V, kind)
    ld = V + 13  # strided rows
    buf = np.zeros((rows, ld), np.float32)
    buf[:, :V] = z
    zd = dev(buf)[:, :V]
    # greedy: bit-exact on the same fp32 values
    got = sd.sample_tokens(zd, 0.0).cpu().numpy()
    for r in range(rows):
        assert got[r] == oracle.next_token(z[r], 0.0, 0, 0.0)
    slack = 1e-5
    for T, k in [(0.7, 0), (1.5, 5), (1.0, 1), (0.9, 50), (2.0, V + 3)]:
        u = rng.random(rows).astype(np.float32)
        got = sd.sample_tokens(zd, T, k, dev(u)).cpu().numpy()
        for r in range(rows):
            ids, lo, hi = oracle.cdf_bounds(z[r], T, k)
            assert got[r] in set(ids.tolist()), (T, k, r)
            j = int(np.flatnonzero(ids == got[r])[0])
            assert lo[j] - slack <= u[r] <= hi[j] + slack, (T, k, r, lo[j], u[r], hi[j])
            near = np.min(np.abs(np.concatenate([lo, hi]) - u[r])) <= slack
            if not near:
                assert got[r] == oracle.next_token(z[r], T, k, float(u[r])), (T, k, r)


def test_sample_kernel_is_deterministic_and_checks_arguments(sd):
    t = torch()
    rng = np.random.Generator(np.random.PCG64(5))
    z = dev(_rows(rng, 8, 3000, "normal"))
    u = dev(rng.random(8).astype(np.float32))
    a = sd.sample_tokens(z, 1.2, 40, u)
    b = sd.sample_tokens(z, 1.2, 40, u)
    assert t.equal(a, b)
    with pytest.raises(RuntimeError):
        sd.sample_tokens(z, 1.0, 0, None)  # sampling without uniforms


def test_greedy_generation_matches_oracle(sd):
    t = torch()
    shape = synth.SHAPES["C1"]
    params = synth.init_params(shape)
    model = sd.Model(shape, max_batch=2)
    model.set(sd.LM_PARAMS, params)
    b = synth.make_batch(shape)
    T0, n_new = 12, 6
    prompt = b.tokens[:2, :T0]
    toks = sd.generate(model, dev(prompt), n_new).cpu().numpy()
    assert np.array_equal(toks[:, :T0], prompt)
    p64 = {k: v.astype(np.float64) for k, v in params.items()}
    for i in range(n_new):
        T = T0 + i
        z, _ = oracle.forward(p64, shape, toks[:, :T], None, keep=False)
        z = z[:, T - 1, :]
        for r in range(2):
            zr = z[r]
            assert zr[toks[r, T]] >= zr.max() - 1e-4 * (abs(zr.max()) + 1.0), (i, r)


def test_sampled_generation_is_reproducible(sd):
    t = torch()
    shape = synth.SHAPES["C2"]
    model = sd.Model(shape, max_batch=4)
    model.set(sd.LM_PARAMS, synth.init_params(shape))
    prompt = dev(synth.make_batch(shape).tokens[:4, :16])
    a = sd.generate(model, prompt, 8, temperature=1.0, top_k=20, seed=3)
    b = sd.generate(model, prompt, 8, temperature=1.0, top_k=20, seed=3)
    c = sd.generate(model, prompt, 8, temperature=1.0, top_k=20, seed=4)
    assert t.equal(a, b)
    assert not t.equal(a, c)
    assert int(a.max()) < shape.vocab and int(a.min()) >= 0


# ------------------------------------------------------- key/value cache

@pytest.mark.parametrize("name,untied,prec", [("C1", False, None), ("C2", False, None), ("C1", True, None),
                                              ("C2", True, None), ("C2", False, "fp16")])
def test_cached_decode_matches_oracle(sd, name, untied, prec):
    """prefill over a prompt, then decode steps fed known tokens: the logits of
    every step against the oracle's forward pass over the sequence so far
    (fp32: rel <= 1e-4; bf16 and fp16: cos >= 0.999), with the tied head and
    with a separate head and bias."""
    t = torch()
    shape = synth.SHAPES[name].replace(untied_head=untied)
    if prec:
        shape = shape.replace(precision=prec)
    params = synth.init_params(shape)
    if untied:
        params["head.b"] = synth.random_tensor(np.random.default_rng(5), params["head.b"].shape, 0.5)
    model = sd.Model(shape, max_batch=2)
    model.set(sd.LM_PARAMS, params)
    toks = synth.make_batch(shape).tokens[:2]
    T0, steps = 10, 6
    cache = model.kv_cache(2)
    got = [model.prefill(dev(toks[:, :T0]), cache).cpu().numpy()]
    for i in range(steps):
        pos = T0 + i
        got.append(model.decode(dev(np.ascontiguousarray(toks[:, pos])), pos, cache).cpu().numpy())
    t.cuda.synchronize()
    p64 = {k: v.astype(np.float64) for k, v in params.items()}
    for i, g in enumerate(got):
        T = T0 + i
        z, _ = oracle.forward(p64, shape, toks[:, :T], None, keep=False)
        ref = z[:, T - 1, :]
        if shape.precision == "fp32":
            assert rel(g, ref) <= 1e-4, (i, rel(g, ref))
        else:
            assert cos(g, ref) >= 0.999, (i, cos(g, ref))


def test_cached_greedy_generation_equals_recomputed(sd):
    t = torch()
    shape = synth.SHAPES["C1"]
    model = sd.Model(shape, max_batch=4)
    model.set(sd.LM_PARAMS, synth.init_params(shape))
    prompt = dev(synth.make_batch(shape).tokens[:4, :16])
    a = sd.generate(model, prompt, 12, kv_cache=True)
    b = sd.generate(model, prompt, 12, kv_cache=False)
    assert t.equal(a, b)


def test_decode_rejects_bad_positions(sd):
    shape = synth.SHAPES["C1"]
    model = sd.Model(shape, max_batch=2)
    cache = model.kv_cache(2)
    tok = dev(np.zeros(2, np.int32))
    with pytest.raises(RuntimeError):
        model.decode(tok, 0, cache)
    with pytest.raises(RuntimeError):
        model.decode(tok, shape.max_seq, cache)


# ------------------------------------------------- device position and graphs

def _prefilled(sd, name, B, T0):
    shape = synth.SHAPES[name]
    model = sd.Model(shape, max_batch=B)
    model.set(sd.LM_PARAMS, synth.init_params(shape))
    toks = dev(np.ascontiguousarray(synth.make_batch(shape).tokens[:B]))
    cache = model.kv_cache(B)
    cache.zero_()
    model.prefill(toks[:, :T0].contiguous(), cache)
    return shape, model, toks, cache


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_decode_at_equals_decode(sd, name):
    """The device-position variant runs the same kernels: bit-identical logits
    and cache contents."""
    t = torch()
    B, T0 = 2, 9
    shape, model, toks, cache = _prefilled(sd, name, B, T0)
    cache2 = cache.clone()
    pos_d = t.zeros(1, dtype=t.int32, device="cuda")
    for p in range(T0, T0 + 4):
        a = model.decode(toks[:, p].contiguous(), p, cache)
        pos_d.fill_(p)
        b = model.decode_at(toks[:, p].contiguous(), pos_d, cache2)
        t.cuda.synchronize()
        assert t.equal(a, b), p
    assert t.equal(cache, cache2)


def test_decode_graph_replays_match_eager(sd):
    """A captured decode step replayed at successive positions, with eager
    work on the stream between replays, gives the eager logits bit for bit at
    every replay."""
    t = torch()
    B, T0 = 4, 12
    shape, model, toks, cache = _prefilled(sd, "C2", B, T0)
    cache_g = cache.clone()
    dg = sd.DecodeGraph(model, cache_g, B)
    for p in range(T0, T0 + 6):
        ref = model.decode(toks[:, p].contiguous(), p, cache).clone()
        _ = (t.arange(1000, device="cuda", dtype=t.float32) * 2).sum()  # unrelated eager work
        got = dg.step(toks[:, p], p).clone()
        t.cuda.synchronize()
        assert t.equal(ref, got), p
    assert dg.graph is not None


@pytest.mark.parametrize("temperature,top_k", [(0.0, 0), (1.0, 20)])
def test_generate_with_graph_equals_eager(sd, temperature, top_k):
    t = torch()
    shape = synth.SHAPES["C1"]
    model = sd.Model(shape, max_batch=4)
    model.set(sd.LM_PARAMS, synth.init_params(shape))
    prompt = dev(synth.make_batch(shape).tokens[:4, :16])
    a = sd.generate(model, prompt, 10, temperature=temperature, top_k=top_k, seed=7)
    b = sd.generate(model, prompt, 10, temperature=temperature, top_k=top_k, seed=7, graph=True)
    assert t.equal(a, b)


def test_decode_at_clamps_the_position(sd):
    """A device position past the cache is clamped to max_seq - 1: the same
    result as decoding there, and nothing outside the cache is touched."""
    t = torch()
    B, T0 = 2, 8
    shape, model, toks, cache = _prefilled(sd, "C1", B, T0)
    cache2 = cache.clone()
    S = shape.max_seq
    tok = toks[:, T0].contiguous()
    a = model.decode(tok, S - 1, cache)
    b = model.decode_at(tok, t.tensor([S + 7], dtype=t.int32, device="cuda"), cache2)
    t.cuda.synchronize()
    assert t.equal(a, b)
    assert t.equal(cache, cache2)
    with pytest.raises(RuntimeError):
        model.decode_at(tok, None, cache2)
