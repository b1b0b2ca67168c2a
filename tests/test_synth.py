"""Host logic of the seeded input generators (no GPU)."""
import math

import numpy as np
import pytest

import synth


def test_parameter_counts_match_the_pages():
    """Tied head: C3 comes to ~1.9M parameters (the LucilleAI SFT model) and C5
    to ~30M (the Smallem series' larger network); C4 is GPT-2 small."""
    counts = {k: synth.n_params(s) for k, s in synth.SHAPES.items()}
    assert counts == {"C1": 440832, "C2": 3290880, "C3": 1882880, "C4": 124439808, "C5": 34657280}


def test_unpacked_batch_shifts_targets():
    b = synth.make_batch(synth.C1)
    assert b.tokens.shape == (4, 80) and b.doc_ids is None
    assert np.array_equal(b.tokens[:, 1:], b.targets[:, :-1])
    assert b.tokens.min() >= 0 and b.tokens.max() < 257


@pytest.mark.parametrize("name,pad_lo,pad_hi", [("C3", 0.08, 0.20), ("C5", 0.12, 0.32)])
def test_packed_batch_structure(name, pad_lo, pad_hi):
    shape = synth.SHAPES[name]
    b = synth.make_batch(shape)
    B, T = b.tokens.shape
    assert (B, T) == (shape.batch, shape.seq)
    assert np.all(np.diff(b.doc_ids, axis=1) >= 0)
    pad = 0
    for r in range(B):
        ids = b.doc_ids[r]
        for d in np.unique(ids):
            idx = np.nonzero(ids == d)[0]
            seg_t, seg_g = b.tokens[r, idx], b.targets[r, idx]
            if np.all(seg_g == -1):  # the trailing pad document
                assert idx[-1] == T - 1 and np.all(seg_t == 0)
                pad += len(idx)
            else:
                lo, hi = shape.docs[1], shape.docs[2]
                assert lo - 1 <= len(idx) <= hi + 1
                assert np.array_equal(seg_t[1:], seg_g[:-1])  # next-token targets
                assert np.all(seg_g >= 0)
    frac = pad / (B * T)
    assert pad_lo < frac < pad_hi, frac


def test_zipf_ids_follow_the_power_law():
    rng = np.random.Generator(np.random.PCG64(0))
    ids = synth.sample_ids(rng, ("zipf", 1.1), 50257, 400000)
    h = np.bincount(ids, minlength=50257)
    w = np.arange(1, 50258, dtype=float) ** -1.1
    p0 = w[0] / w.sum()
    assert abs(h[0] / len(ids) - p0) < 0.003  # id 0 carries about 13.9 %
    assert abs(h[0] / h[1] - 2 ** 1.1) < 0.05


def test_generators_are_seeded():
    a, b = synth.make_batch(synth.C3), synth.make_batch(synth.C3)
    assert np.array_equal(a.tokens, b.tokens) and np.array_equal(a.doc_ids, b.doc_ids)
    p, q = synth.init_params(synth.C2), synth.init_params(synth.C2)
    assert all(np.array_equal(p[k], q[k]) for k in p)
    c4 = synth.init_params(synth.C4.replace(n_layers=2))
    assert abs(c4["blocks.0.attn.w_o"].std() - 0.02 / math.sqrt(4)) < 1e-3
