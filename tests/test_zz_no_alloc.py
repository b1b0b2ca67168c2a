"""The allocation-free cross-entropy entry point (lmk_xent_noalloc) against the
workspace one (lmk_xent) on the same inputs: bit-identical loss, valid count
and dz, on two calls in a row, the second with fewer rows (the static scratch
keeps the first call's contents, which must not leak into the second)."""
import numpy as np
import pytest

from helpers import act, dev, exact, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sd():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    import scratch_decoder_only_amd as m
    return m


def _case(prec, M, V, seed):
    rng = np.random.default_rng(seed)
    ldz = (V + 127) // 128 * 128
    z = np.zeros((M, ldz), np.float32)
    z[:, :V] = exact((rng.standard_normal((M, V)) * 3).astype(np.float32), prec)
    tgt = rng.integers(0, V, M).astype(np.int32)
    tgt[::5] = -1
    return z, tgt, ldz


@pytest.mark.parametrize("prec", [0, 1])
def test_noalloc_cross_entropy_matches_workspace_version(sd, prec):
    t = torch()
    V = 8000
    for M, seed in ((4096, 1), (300, 2)):  # the second call is smaller
        print(f"xent no-alloc prec={prec} M={M}", flush=True)
        z, tgt, ldz = _case(prec, M, V, seed)
        za, zb = act(z, prec), act(z, prec)
        tg = dev(tgt)
        la, lb = t.zeros(4, device="cuda"), t.zeros(4, device="cuda")
        fa, fb = t.zeros(4, dtype=t.int32, device="cuda"), t.zeros(4, dtype=t.int32, device="cuda")
        ws_n = t.zeros(4, dtype=t.int32, device="cuda")
        ws_rows = t.zeros(M, device="cuda")
        sd.xent(prec, za, ldz, M, V, tg, la, ws_n, ws_rows, fa)
        sd.xent_noalloc(prec, zb, ldz, M, V, tg, lb, fb)
        t.cuda.synchronize()
        assert t.equal(la, lb), (la, lb)
        assert int(lb[3]) == int((tgt >= 0).sum())
        assert t.equal(za, zb)
        assert t.equal(fa, fb)


def test_noalloc_cross_entropy_rejects_more_rows_than_its_scratch(sd):
    t = torch()
    M, V = (1 << 16) + 8, 16
    P = t.zeros(8, device="cuda")
    with pytest.raises(sd.LmError):
        sd.xent_noalloc(1, P, 16, M, V, P, P, P)
