"""Per-kernel parity of the HIP kernels against the CPU oracle, through the
per-kernel C ABI (include/lmstep_kernels.h).

Inputs are seeded; bf16 operands are rounded to bf16 first so the oracle
works on exactly the values the kernels read. Tolerances: integer and index
outputs bit-exact; fp32 outputs of fp32-accumulated contractions rel 2e-5;
outputs stored in bf16 rel 6e-3 (one bf16 rounding, 2^-9 relative, per
element).
"""
import math

import numpy as np
import pytest

import oracle
from helpers import act, act_dtype, cos, dev, exact, host, rel, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sd():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    import scratch_decoder_only_amd as m
    return m


def tol(prec, out_f32):
    return 2e-5 if (prec == 0 or out_f32) else 6e-3


def _operands(rng, prec, *shapes, scale=1.0):
    out = []
    for s in shapes:
        a = (rng.standard_normal(s) * scale).astype(np.float32)
        out.append(exact(a, prec))
    return out


# ------------------------------------------------------------------- GEMM

@pytest.mark.parametrize("prec", [0, 1, 2])
@pytest.mark.parametrize("layout", ["fwd", "dx", "dw"])
@pytest.mark.parametrize("MNK", [(200, 136, 72), (1000, 648, 576), (8, 8, 8), (136, 264, 1536)])
@pytest.mark.parametrize("split", [0, 3])
def test_gemm_layouts(sd, prec, layout, MNK, split, cfg=0):
    t = torch()
    M, N, K = MNK
    rng = np.random.default_rng(hash((prec, layout, MNK, split)) % 2**32)
    print(f"gemm prec={prec} layout={layout} M,N,K={MNK} split={split} cfg={cfg}", flush=True)
    if layout == "fwd":      # Y = X W^T
        X, W = _operands(rng, prec, (M, K), (N, K))
        A, lda, akc, B, ldb, bkc = X, K, True, W, K, True
        expect = oracle.linear_fwd(X, W)
    elif layout == "dx":     # dX = dY W, W stored [K, N]
        dY, W = _operands(rng, prec, (M, K), (K, N))
        A, lda, akc, B, ldb, bkc = dY, K, True, W, N, False
        expect = dY.astype(np.float64) @ W
    else:                    # dW = dY^T X, dY stored [K, M], X stored [K, N]
        dY, X = _operands(rng, prec, (K, M), (K, N))
        A, lda, akc, B, ldb, bkc = dY, M, False, X, N, False
        expect = oracle.linear_bwd(dY, X, np.zeros((M, N)))[1]
    C = t.zeros((M, N), dtype=t.float32, device="cuda")
    ws = t.zeros(4 * M * N + 16, dtype=t.float32, device="cuda")
    Ad, Bd = act(A, prec), act(B, prec)
    sd.gemm(prec, M, N, K, Ad, lda, akc, Bd, ldb, bkc, C, N, c_f32=True, force_split=split, ws=ws, cfg=cfg)
    t.cuda.synchronize()
    assert rel(host(C), expect) <= tol(prec, True)
    # slices are summed in a fixed order: a second run is bit-identical
    C2 = t.zeros_like(C)
    sd.gemm(prec, M, N, K, Ad, lda, akc, Bd, ldb, bkc, C2, N, c_f32=True, force_split=split, ws=ws, cfg=cfg)
    t.cuda.synchronize()
    assert t.equal(C, C2)


@pytest.mark.parametrize("prec", [0, 1, 2])
@pytest.mark.parametrize("epi", ["store", "resid", "gelu", "dgelu"])
@pytest.mark.parametrize("split", [0, 2])
def test_gemm_epilogues(sd, prec, epi, split, cfg=0, MNK=(264, 200, 320)):
    t = torch()
    M, N, K = MNK
    rng = np.random.default_rng(17 + prec)
    print(f"gemm epilogue prec={prec} epi={epi} split={split} cfg={cfg} M,N,K={MNK}", flush=True)
    X, W = _operands(rng, prec, (M, K), (N, K), scale=0.3)
    bias = rng.standard_normal(N).astype(np.float32)
    ws = t.zeros(4 * M * N, dtype=t.float32, device="cuda")
    adt = act_dtype(prec)
    lin = oracle.linear_fwd(X, W, bias)
    args = dict(bias=dev(bias), force_split=split, ws=ws, cfg=cfg)
    if epi == "store":
        C = t.zeros((M, N), dtype=adt, device="cuda")
        sd.gemm(prec, M, N, K, act(X, prec), K, True, act(W, prec), K, True, C, N, sd.EPI_STORE, **args)
        t.cuda.synchronize()
        assert rel(host(C), lin) <= tol(prec, False)
    elif epi == "resid":
        R = rng.standard_normal((M, N)).astype(np.float32)
        C = t.zeros((M, N), dtype=t.float32, device="cuda")
        sd.gemm(prec, M, N, K, act(X, prec), K, True, act(W, prec), K, True, C, N, sd.EPI_RESID, R=dev(R), ldr=N, **args)
        t.cuda.synchronize()
        assert rel(host(C), R + lin) <= tol(prec, True)
    elif epi == "gelu":
        U = t.zeros((M, N), dtype=adt, device="cuda")
        Aout = t.zeros((M, N), dtype=adt, device="cuda")
        sd.gemm(prec, M, N, K, act(X, prec), K, True, act(W, prec), K, True, U, N, sd.EPI_GELU, aux=Aout, ld_aux=N, **args)
        t.cuda.synchronize()
        assert rel(host(U), oracle.gelu_grad(lin)) <= tol(prec, False)  # the stored GELU'(u)
        assert rel(host(Aout), oracle.gelu(lin)) <= tol(prec, False)
    else:
        # aux: GELU'(u) as the forward's GELU epilogue stores it
        u = rng.standard_normal((M, N)).astype(np.float32) * 2
        d = exact(oracle.gelu_grad(u).astype(np.float32), prec)
        C = t.zeros((M, N), dtype=adt, device="cuda")
        args.pop("bias")
        sd.gemm(prec, M, N, K, act(X, prec), K, True, act(W, prec), K, True, C, N, sd.EPI_DGELU, aux=act(d, prec),
                ld_aux=N, **args)
        t.cuda.synchronize()
        assert rel(host(C), oracle.linear_fwd(X, W) * d) <= tol(prec, False)


# The persistent K-split kernel (configurations 15: 128 x 192 tiles, 16:
# 128 x 128), forced: every layout and epilogue, ragged in every dimension,
# with K splits, and with more tiles than its one-block-per-CU grid holds
# (8200 x 776: 325 tiles of 128 x 192 for 256 blocks).
@pytest.mark.parametrize("cfg", [15, 16])
@pytest.mark.parametrize("prec", [1, 2])
@pytest.mark.parametrize("layout", ["fwd", "dx", "dw"])
@pytest.mark.parametrize("MNK,split", [((1000, 648, 576), 0), ((8200, 776, 200), 0), ((136, 264, 1536), 3),
                                       ((8, 8, 8), 0)])
def test_gemm_ksplit_layouts(sd, cfg, prec, layout, MNK, split):
    test_gemm_layouts(sd, prec, layout, MNK, split, cfg=cfg)


@pytest.mark.parametrize("cfg", [15, 16])
@pytest.mark.parametrize("prec", [1, 2])
@pytest.mark.parametrize("epi", ["store", "resid", "gelu", "dgelu"])
@pytest.mark.parametrize("MNK", [(264, 200, 320), (8200, 776, 136)])
def test_gemm_ksplit_epilogues(sd, cfg, prec, epi, MNK):
    test_gemm_epilogues(sd, prec, epi, 0, cfg=cfg, MNK=MNK)


# Shapes with one dimension of 16384 or more run on the persistent 256 x 256
# kernel (the others on the 128 x 128 one): every layout, ragged tails in all
# three dimensions, with and without a K split.
@pytest.mark.parametrize("prec", [1, 2])
@pytest.mark.parametrize("layout", ["fwd", "dx", "dw"])
@pytest.mark.parametrize("MNK", [(16392, 264, 200), (136, 16520, 96), (264, 136, 16400)])
@pytest.mark.parametrize("split", [0, 3])
def test_gemm_layouts_wide(sd, prec, layout, MNK, split):
    test_gemm_layouts(sd, prec, layout, MNK, split)


@pytest.mark.parametrize("prec", [1, 2])
@pytest.mark.parametrize("epi", ["store", "resid", "gelu", "dgelu"])
def test_gemm_epilogues_wide(sd, prec, epi):
    t = torch()
    M, N, K = 16392, 200, 136
    rng = np.random.default_rng(23 + prec)
    print(f"gemm wide epilogue prec={prec} epi={epi}", flush=True)
    X, W = _operands(rng, prec, (M, K), (N, K), scale=0.3)
    bias = rng.standard_normal(N).astype(np.float32)
    adt = act_dtype(prec)
    lin = oracle.linear_fwd(X, W, bias)
    args = dict(bias=dev(bias))
    if epi == "store":
        C = t.zeros((M, N), dtype=adt, device="cuda")
        sd.gemm(prec, M, N, K, act(X, prec), K, True, act(W, prec), K, True, C, N, sd.EPI_STORE, **args)
        t.cuda.synchronize()
        assert rel(host(C), lin) <= tol(prec, False)
    elif epi == "resid":
        R = rng.standard_normal((M, N)).astype(np.float32)
        C = t.zeros((M, N), dtype=t.float32, device="cuda")
        sd.gemm(prec, M, N, K, act(X, prec), K, True, act(W, prec), K, True, C, N, sd.EPI_RESID, R=dev(R), ldr=N, **args)
        t.cuda.synchronize()
        assert rel(host(C), R + lin) <= tol(prec, True)
    elif epi == "gelu":
        U = t.zeros((M, N), dtype=adt, device="cuda")
        Aout = t.zeros((M, N), dtype=adt, device="cuda")
        sd.gemm(prec, M, N, K, act(X, prec), K, True, act(W, prec), K, True, U, N, sd.EPI_GELU, aux=Aout, ld_aux=N, **args)
        t.cuda.synchronize()
        assert rel(host(U), oracle.gelu_grad(lin)) <= tol(prec, False)  # the stored GELU'(u)
        assert rel(host(Aout), oracle.gelu(lin)) <= tol(prec, False)
    else:
        d = exact(oracle.gelu_grad(rng.standard_normal((M, N)) * 2).astype(np.float32), prec)
        C = t.zeros((M, N), dtype=adt, device="cuda")
        args.pop("bias")
        sd.gemm(prec, M, N, K, act(X, prec), K, True, act(W, prec), K, True, C, N, sd.EPI_DGELU, aux=act(d, prec),
                ld_aux=N, **args)
        t.cuda.synchronize()
        assert rel(host(C), oracle.linear_fwd(X, W) * d) <= tol(prec, False)


@pytest.mark.parametrize("prec", [1, 2])
def test_gemm_store_16bit_tall(sd, prec):
    """The QKV-projection shape class (K-contiguous operands, 16-bit store with
    bias, M >= 4096) runs on the 192 x 128 tiles: ragged in M (8200 = 42 x 192 +
    136), N and K."""
    t = torch()
    M, N, K = 8200, 264, 200
    rng = np.random.default_rng(41 + prec)
    print(f"gemm tall store prec={prec}", flush=True)
    X, W = _operands(rng, prec, (M, K), (N, K), scale=0.3)
    bias = rng.standard_normal(N).astype(np.float32)
    C = t.zeros((M, N), dtype=act_dtype(prec), device="cuda")
    sd.gemm(prec, M, N, K, act(X, prec), K, True, act(W, prec), K, True, C, N, sd.EPI_STORE, bias=dev(bias))
    t.cuda.synchronize()
    assert rel(host(C), oracle.linear_fwd(X, W, bias)) <= tol(prec, False)


@pytest.mark.parametrize("prec", [1, 2])
@pytest.mark.parametrize("epi,b_kc", [("store", True), ("store", False), ("gelu", True), ("gelu", False)])
def test_gemm_persistent_rounds(sd, prec, epi, b_kc):
    """More tiles than the persistent grid holds (731 units of 192 x 128 for
    the K-contiguous store, 1105 of 128 x 128 otherwise, for 512 blocks), so
    blocks run several units and a unit's first loads overlap the previous
    unit's stores; ragged in M (8200), N (2056) and K (200), with bias."""
    t = torch()
    M, N, K = 8200, 2056, 200
    rng = np.random.default_rng(57 + prec + 2 * b_kc)
    print(f"gemm persistent rounds prec={prec} epi={epi} b_kc={b_kc}", flush=True)
    X, W = _operands(rng, prec, (M, K), (N, K), scale=0.3)
    bias = rng.standard_normal(N).astype(np.float32)
    adt = act_dtype(prec)
    Wd = act(W, prec) if b_kc else act(np.ascontiguousarray(W.T), prec)
    ldb = K if b_kc else N
    lin = oracle.linear_fwd(X, W, bias)
    C = t.zeros((M, N), dtype=adt, device="cuda")
    if epi == "store":
        sd.gemm(prec, M, N, K, act(X, prec), K, True, Wd, ldb, b_kc, C, N, sd.EPI_STORE, bias=dev(bias))
        t.cuda.synchronize()
        assert rel(host(C), lin) <= tol(prec, False)
    else:
        Aout = t.zeros((M, N), dtype=adt, device="cuda")
        sd.gemm(prec, M, N, K, act(X, prec), K, True, Wd, ldb, b_kc, C, N, sd.EPI_GELU, aux=Aout, ld_aux=N,
                bias=dev(bias))
        t.cuda.synchronize()
        assert rel(host(C), oracle.gelu_grad(lin)) <= tol(prec, False)  # the stored GELU'(u)
        assert rel(host(Aout), oracle.gelu(lin)) <= tol(prec, False)


@pytest.mark.parametrize("prec", [1, 2])
@pytest.mark.parametrize("case", ["w192", "ragged"])
def test_gemm_group(sd, prec, case):
    """Weight gradients of several layers in one grouped launch (each output
    one unit's fixed-order sum over all of K): every problem against the
    oracle's dW = dY^T X, ragged in M and K; more units than the persistent
    grid holds, so blocks walk several problems; 128 x 192 tiles, with widths
    that are multiples of 192 (w192) or not (ragged: partly empty last tiles,
    down to a single 8 x 8 output); bit-identical reruns."""
    t = torch()
    if case == "w192":
        shapes = [(200, 384, 1000), (1000, 192, 520), (136, 576, 64), (1280, 3840, 136), (2056, 1920, 200)]
    else:
        shapes = [(264, 200, 320), (8, 8, 8), (1000, 648, 576), (2056, 1288, 72), (1024, 1024, 96)]
    rng = np.random.default_rng(71 + prec + 10 * len(case))
    print(f"gemm group prec={prec} case={case}", flush=True)
    probs, expect, outs = [], [], []
    for (M, N, K) in shapes:
        dY, X = _operands(rng, prec, (K, M), (K, N))
        C = t.full((M, N), 3.0, dtype=t.float32, device="cuda")
        probs.append((M, N, K, act(dY, prec), M, act(X, prec), N, C, N))
        expect.append(oracle.linear_bwd(dY, X, np.zeros((M, N)))[1])
        outs.append(C)
    table = t.zeros(sd.gemm_group_table_bytes(len(probs)), dtype=t.uint8, device="cuda")
    sd.gemm_group(prec, probs, table)
    t.cuda.synchronize()
    first = [c.clone() for c in outs]
    for c, e in zip(outs, expect):
        assert rel(host(c), e) <= tol(prec, True)
    sd.gemm_group(prec, probs, table)
    t.cuda.synchronize()
    for c, f in zip(outs, first):
        assert t.equal(c, f)


def test_gemm_output_row_limit(sd):
    """Rows >= M_out are computed but never stored (the padded vocabulary)."""
    t = torch()
    rng = np.random.default_rng(3)
    M, N, K = 136, 64, 96
    A, B = _operands(rng, 1, (K, M), (K, N))
    C = t.full((M, N), 7.0, dtype=t.float32, device="cuda")
    sd.gemm(1, M, N, K, act(A, 1), M, False, act(B, 1), N, False, C, N, c_f32=True, M_out=131)
    t.cuda.synchronize()
    c = host(C)
    assert rel(c[:131], (A.astype(np.float64).T @ B)[:131]) <= 2e-5
    assert np.all(c[131:] == 7.0)


# -------------------------------------------------------------- LayerNorm

@pytest.mark.parametrize("prec", [0, 1, 2])
@pytest.mark.parametrize("C", [128, 768])
def test_layernorm_fwd_bwd(sd, prec, C):
    t = torch()
    M, eps = 300, 1e-5
    rng = np.random.default_rng(C + prec)
    x = (rng.standard_normal((M, C)) * 2 + 0.3).astype(np.float32)
    g = (1 + 0.2 * rng.standard_normal(C)).astype(np.float32)
    b = (0.1 * rng.standard_normal(C)).astype(np.float32)
    adt = act_dtype(prec)
    y = t.zeros((M, C), dtype=adt, device="cuda")
    mu = t.zeros(M, device="cuda")
    rs = t.zeros(M, device="cuda")
    sd.layernorm_fwd(prec, dev(x), dev(g), dev(b), eps, y, mu, rs)
    ey, emu, ers = oracle.layernorm_fwd(x, g, b, eps)
    t.cuda.synchronize()
    assert rel(host(y), ey) <= tol(prec, False)
    assert rel(host(mu), emu) <= 1e-5 and rel(host(rs), ers) <= 1e-5
    dy = rng.standard_normal((M, C)).astype(np.float32)
    gin = rng.standard_normal((M, C)).astype(np.float32)
    gout = dev(gin)
    gact = t.zeros((M, C), dtype=adt, device="cuda")
    dg = t.zeros(C, device="cuda")
    db = t.zeros(C, device="cuda")
    ws = t.zeros(sd.layernorm_bwd_ws_floats(M, C), device="cuda")
    dsum = t.zeros(C, device="cuda")
    sd.layernorm_bwd(prec, dev(dy), dev(x), mu, rs, dev(g), gout, gout, gact, dg, db, ws, dsum=dsum)
    edx, edg, edb = oracle.layernorm_bwd(dy, x, host(mu), host(rs), g)
    t.cuda.synchronize()
    assert rel(host(gout), gin + edx) <= 2e-5
    assert rel(host(gact), gin + edx) <= tol(prec, False)
    assert rel(host(dg), edg) <= 2e-5 and rel(host(db), edb) <= 2e-5
    # column sums of the output gradient (the bias gradient fused into this pass)
    assert rel(host(dsum), (gin.astype(np.float64) + edx).sum(axis=0)) <= 2e-5


# ------------------------------------------------- index layout, embedding

def _doc_ids(rng, B, T, lens=(1, 40)):
    doc = np.zeros((B, T), np.int32)
    for b in range(B):
        t0, d = 0, 0
        while t0 < T:
            L = int(rng.integers(lens[0], lens[1] + 1))
            doc[b, t0:t0 + L] = d
            t0 += L
            d += 1
    return doc


def test_index_layout_bit_exact(sd):
    t = torch()
    rng = np.random.default_rng(5)
    B, T = 3, 300
    doc = _doc_ids(rng, B, T)
    doc[2] = 7  # one document
    start, pos, end = (t.zeros((B, T), dtype=t.int32, device="cuda") for _ in range(3))
    flags = t.zeros(4, dtype=t.int32, device="cuda")
    sd.index_layout(dev(doc), B, T, start, end, pos, flags)
    es, ep = oracle.index_layout(doc, B, T)
    ee = np.zeros((B, T), np.int64)
    for b in range(B):
        for i in range(T):
            j = i
            while j < T and doc[b, j] == doc[b, i]:
                j += 1
            ee[b, i] = j
    t.cuda.synchronize()
    assert np.array_equal(start.cpu().numpy(), es) and np.array_equal(pos.cpu().numpy(), ep)
    assert np.array_equal(end.cpu().numpy(), ee)
    assert int(flags[0]) == 0
    # no doc ids: start 0, pos t, end T
    sd.index_layout(None, B, T, start, end, pos, flags)
    t.cuda.synchronize()
    assert np.all(start.cpu().numpy() == 0) and np.all(end.cpu().numpy() == T)
    assert np.array_equal(pos.cpu().numpy(), np.tile(np.arange(T), (B, 1)))
    # decreasing doc ids set flags bit 1
    bad = doc.copy()
    bad[0, 100] = -5
    sd.index_layout(dev(bad), B, T, start, end, pos, flags)
    t.cuda.synchronize()
    assert int(flags[0]) & 2


def test_embedding_forward(sd):
    t = torch()
    rng = np.random.default_rng(6)
    V, S, C, M = 1000, 64, 256, 777
    wte = rng.standard_normal((V, C)).astype(np.float32)
    wpe = rng.standard_normal((S, C)).astype(np.float32)
    tok = rng.integers(0, V, M).astype(np.int32)
    pos = rng.integers(0, S, M).astype(np.int32)
    x = t.zeros((M, C), device="cuda")
    flags = t.zeros(4, dtype=t.int32, device="cuda")
    sd.embed_fwd(dev(tok), dev(pos), dev(wte), dev(wpe), x, flags)
    t.cuda.synchronize()
    assert np.array_equal(host(x).astype(np.float32), wte[tok] + wpe[pos])
    assert rel(host(x), oracle.embedding_fwd(wte, wpe, tok, pos)) <= 1e-7


# -------------------------------------------------------------- attention

@pytest.mark.parametrize("prec", [0, 1, 2])
@pytest.mark.parametrize("D", [32, 64])
@pytest.mark.parametrize("packed", [False, True])
def test_attention_fwd_bwd(sd, prec, D, packed):
    t = torch()
    B, T, H = 2, 200, 3
    C = H * D
    rng = np.random.default_rng(D + 2 * prec + 4 * packed)
    print(f"attention prec={prec} D={D} packed={packed}", flush=True)
    qkv = (rng.standard_normal((B, T, 3 * C)) * 1.5).astype(np.float32)
    qkv = exact(qkv, prec)
    doc = _doc_ids(rng, B, T, (1, 90)) if packed else None
    start_np, _ = oracle.index_layout(doc, B, T)
    start, end, pos = (t.zeros((B, T), dtype=t.int32, device="cuda") for _ in range(3))
    flags = t.zeros(4, dtype=t.int32, device="cuda")
    sd.index_layout(None if doc is None else dev(doc), B, T, start, end, pos, flags)
    adt = act_dtype(prec)
    o = t.zeros((B, T, C), dtype=adt, device="cuda")
    lse = t.zeros((B, H, T), device="cuda")
    qkv_d = act(qkv, prec)
    sd.attn_fwd(prec, qkv_d, start, end, B, T, H, D, o, lse)

    def heads(a):
        return a.reshape(B, T, H, D).transpose(0, 2, 1, 3)

    q, k, v = heads(qkv[..., :C]), heads(qkv[..., C:2 * C]), heads(qkv[..., 2 * C:])
    eo, else_ = oracle.attention_fwd(q, k, v, start_np)
    eo = eo.transpose(0, 2, 1, 3).reshape(B, T, C)
    t.cuda.synchronize()
    assert rel(host(o), eo) <= (2e-5 if prec == 0 else 8e-3)
    assert np.abs(host(lse) - else_).max() <= (2e-5 if prec == 0 else 2e-3)
    do = rng.standard_normal((B, T, C)).astype(np.float32)
    do = exact(do, prec)
    dqkv = t.zeros((B, T, 3 * C), dtype=adt, device="cuda")
    delta = t.zeros((B, H, T), device="cuda")
    sd.attn_bwd(prec, qkv_d, o, lse, act(do, prec), start, end, B, T, H, D, delta, dqkv)
    dq, dk, dv = oracle.attention_bwd(heads(do), q, k, v, start_np)
    got = host(dqkv)
    t.cuda.synchronize()
    for i, e in enumerate((dq, dk, dv)):
        e = e.transpose(0, 2, 1, 3).reshape(B, T, C)
        g = got[..., i * C:(i + 1) * C]
        if prec == 0:
            assert rel(g, e) <= 5e-5, i
        else:
            assert rel(g, e) <= 2e-2 and cos(g, e) >= 0.9995, i


# ------------------------------------------------------------ column sums

@pytest.mark.parametrize("prec", [0, 1, 2])
@pytest.mark.parametrize("M,N", [(300, 768), (1000, 2304), (129, 3076)])
def test_column_sums(sd, prec, M, N):
    """Bias gradients: out[c] = sum over rows of a[:, c] (fixed order, 8 or 4
    columns per thread depending on the alignment of N)."""
    t = torch()
    rng = np.random.default_rng(M + N + prec)
    a = rng.standard_normal((M, N)).astype(np.float32)
    a = exact(a, prec)
    out = t.zeros(N, device="cuda")
    ws = t.zeros(sd.colsum_ws_floats(M, N), device="cuda")
    sd.colsum(prec, act(a, prec), N, M, N, out, ws)
    t.cuda.synchronize()
    assert rel(host(out), a.astype(np.float64).sum(axis=0)) <= 2e-6


# ----------------------------------------------------------- cross-entropy

# V = 50257 and 70000 also cover the row-in-memory kernel (rows too long to
# stay in registers) next to the register-resident one
@pytest.mark.parametrize("prec", [0, 1, 2])
@pytest.mark.parametrize("V", [257, 8000, 50257, 70000])
def test_cross_entropy(sd, prec, V):
    t = torch()
    M = 300 if V < 50000 else 64
    ldz = (V + 127) // 128 * 128
    rng = np.random.default_rng(V + prec)
    z = (rng.standard_normal((M, V)) * 3).astype(np.float32)
    z = exact(z, prec)
    tgt = rng.integers(0, V, M).astype(np.int32)
    tgt[::7] = -1
    zp = np.zeros((M, ldz), np.float32)
    zp[:, :V] = z
    zp[:, V:] = 5.0  # padding columns must be ignored and zeroed
    zd = act(zp, prec)
    loss = t.zeros(4, device="cuda")
    ws_n = t.zeros(4, dtype=t.int32, device="cuda")
    ws_rows = t.zeros(M, device="cuda")
    flags = t.zeros(4, dtype=t.int32, device="cuda")
    sd.xent(prec, zd, ldz, M, V, dev(tgt), loss, ws_n, ws_rows, flags)
    el, edz, n = oracle.xent_fwd_bwd(z, tgt)
    t.cuda.synchronize()
    got = host(zd)
    assert abs(float(loss[0]) - el) <= 2e-5 * abs(el)
    assert int(loss[3]) == n
    assert rel(got[:, :V], edz) <= (2e-5 if prec == 0 else 6e-3)
    assert np.all(got[:, V:] == 0)
    assert np.all(got[tgt < 0] == 0)
    # with a loss scale S = 1024 dz is S times as large and the loss unchanged
    zd2 = act(zp, prec)
    S = dev(np.array([1024.0], np.float32))
    sd.xent(prec, zd2, ldz, M, V, dev(tgt), loss, ws_n, ws_rows, flags, loss_scale=S)
    t.cuda.synchronize()
    assert abs(float(loss[0]) - el) <= 2e-5 * abs(el)
    assert rel(host(zd2)[:, :V] / 1024.0, edz) <= (2e-5 if prec == 0 else 6e-3)
    if prec == 0:
        assert np.array_equal(host(zd2), got * 1024.0)  # a power of two scales exactly


# ------------------------------------------------ embedding backward (CSR)

@pytest.mark.parametrize("nkeys,M", [(1000, 5000), (64, 3000), (50257, 8192), (4095, 3000), (4096, 3000),
                                     (70000, 20000), (50257, 33000), (16384, 32768), (2048, 32768)])
def test_csr_bit_exact_and_segment_sums(sd, nkeys, M):
    """Key counts scanned in one round of 4096 (up to 4095 keys: nkeys + 1
    entries), in one batch of rounds, and over several batches (70000); ranks
    counted pairwise (fewer than 128 blocks of 256 rows) and from per-block
    key counts (128 blocks and more, a ragged last block at 33000 rows)."""
    t = torch()
    import synth
    rng = np.random.Generator(np.random.PCG64(nkeys))
    keys = synth.sample_ids(rng, ("zipf", 1.1), nkeys, M)
    C = 128
    counts, offsets, chunk = (t.zeros(nkeys + 1, dtype=t.int32, device="cuda") for _ in range(3))
    perm = t.zeros(M, dtype=t.int32, device="cuda")
    assert sd.csr_ws_ints(M, nkeys) == (M if M <= 127 * 256 else ((M + 255) // 256) * nkeys)
    rank = t.full((sd.csr_ws_ints(M, nkeys),), 7, dtype=t.int32, device="cuda")  # stale scratch must not matter
    sd.csr(dev(keys), M, nkeys, counts, offsets, chunk, perm, rank)
    eoff, eperm = oracle.csr_by_key(keys, nkeys)
    t.cuda.synchronize()
    assert np.array_equal(offsets.cpu().numpy(), eoff)
    assert np.array_equal(perm.cpu().numpy(), eperm)
    dx = rng.standard_normal((M, C)).astype(np.float32)
    base = rng.standard_normal((nkeys, C)).astype(np.float32)
    dst = dev(base)
    part = t.zeros(sd.segment_sum_ws_floats(M, nkeys, C), device="cuda")
    sd.segment_sum(dev(dx), M, C, nkeys, counts, offsets, chunk, perm, part, dst, True)
    ew, _ = oracle.embedding_bwd(dx, keys, np.zeros(M, np.int64), nkeys, 1)
    t.cuda.synchronize()
    assert rel(host(dst), base + ew) <= 1e-6
    # bit-reproducible
    dst2 = dev(base)
    sd.segment_sum(dev(dx), M, C, nkeys, counts, offsets, chunk, perm, part, dst2, True)
    t.cuda.synchronize()
    assert t.equal(dst, dst2)


# ---------------------------------------------------------- norm and AdamW

@pytest.mark.parametrize("clip", [1.0, 1e9])
def test_grad_norm_and_adamw(sd, clip):
    t = torch()
    rng = np.random.default_rng(9)
    n = 1_000_004
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    p = rng.standard_normal(n).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.random(n) * 1e-7).astype(np.float32)
    part = t.zeros(1024, dtype=t.float64, device="cuda")
    ns = t.zeros(2, device="cuda")
    flags = t.zeros(4, dtype=t.int32, device="cuda")
    gd = dev(g)
    sd.grad_norm(gd, clip, part, ns, flags)
    en, es = oracle.grad_norm_and_scale({"g": g}, clip)
    t.cuda.synchronize()
    assert abs(float(ns[0]) - en) <= 1e-6 * en and abs(float(ns[1]) - es) <= 1e-6 * es
    pd, md, vd = dev(p), dev(m), dev(v)
    shadow = t.zeros(n, dtype=t.bfloat16, device="cuda")
    sd.adamw(pd, gd, md, vd, 3e-4, 0.9, 0.999, 1e-8, 0.1, 3, ns, flags, shadow)
    ep, em, ev = oracle.adamw(p, g, m, v, 3, 3e-4, 0.9, 0.999, 1e-8, 0.1, es)
    t.cuda.synchronize()
    # p' is fp32, so p' - p is known to the ulp of p: compare p' within 4 ulp
    # plus 1e-5 of the update
    ulp = np.abs(p.astype(np.float64)) * 2.0 ** -23
    assert np.all(np.abs(host(pd) - ep) <= 4 * ulp + 1e-5 * np.abs(ep - p))
    assert rel(host(md), em) <= 1e-6 and rel(host(vd), ev) <= 1e-6
    assert t.equal(shadow, pd.to(t.bfloat16))
    # the fp16 operand copy
    pd2, md2, vd2 = dev(p), dev(m), dev(v)
    sh16 = t.zeros(n, dtype=t.float16, device="cuda")
    sd.adamw(pd2, gd, md2, vd2, 3e-4, 0.9, 0.999, 1e-8, 0.1, 3, ns, flags, sh16, shadow_f16=True)
    t.cuda.synchronize()
    assert t.equal(pd2, pd) and t.equal(sh16, pd2.to(t.float16))


def test_grad_norm_with_loss_scale(sd):
    """The buffer holds S g: the norm and clip factor are those of g, the
    update factor is (clip factor) / S, and the scale state follows the
    oracle's rule (finite steps, growth at the interval, backoff on inf)."""
    t = torch()
    rng = np.random.default_rng(4)
    n = 100_000
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    S0 = 4096.0
    gs = dev(g * np.float32(S0))
    part = t.zeros(1024, dtype=t.float64, device="cuda")
    ns = t.zeros(2, device="cuda")
    flags = t.zeros(4, dtype=t.int32, device="cuda")
    state = dev(np.array([S0, 0.0], np.float32))
    en, es = oracle.grad_norm_and_scale({"g": g}, 1.0)
    trace = []
    for i in range(4):
        sd.grad_norm(gs, 1.0, part, ns, flags, scale_state=state, growth=2.0, backoff=0.5, interval=3)
        t.cuda.synchronize()
        if i == 0:
            assert abs(float(ns[0]) - en) <= 1e-6 * en
            assert abs(float(ns[1]) * S0 - es) <= 1e-6 * es
        trace.append((float(state[0]), int(state[1])))
    assert int(flags[0]) & 1 == 0
    g_inf = g.copy()
    g_inf[7] = np.inf
    sd.grad_norm(dev(g_inf), 1.0, part, ns, flags, scale_state=state, growth=2.0, backoff=0.5, interval=3)
    t.cuda.synchronize()
    trace.append((float(state[0]), int(state[1])))
    assert int(flags[0]) & 1
    assert trace == oracle.loss_scale_trace(S0, [True] * 4 + [False], 2.0, 0.5, 3)


def test_adamw_skips_on_nonfinite_norm(sd):
    t = torch()
    n = 4096
    g = np.ones(n, np.float32)
    g[5] = np.inf
    p = np.arange(n, dtype=np.float32)
    part = t.zeros(1024, dtype=t.float64, device="cuda")
    ns = t.zeros(2, device="cuda")
    flags = t.zeros(4, dtype=t.int32, device="cuda")
    gd, pd, md, vd = dev(g), dev(p), t.zeros(n, device="cuda"), t.zeros(n, device="cuda")
    sd.grad_norm(gd, 1.0, part, ns, flags)
    sd.adamw(pd, gd, md, vd, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, ns, flags)
    t.cuda.synchronize()
    assert int(flags[0]) & 1
    assert np.array_equal(pd.cpu().numpy(), p) and float(md.abs().sum()) == 0
