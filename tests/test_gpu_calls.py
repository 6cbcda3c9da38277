"""Per-call parity of the HIP library against the float64 oracle on seeded
inputs, at sizes that span several tiles and a ragged tail, through the C ABI.
Both kernel paths of each call are exercised: the MFMA path (bf16, the
configuration shapes) and the generic fp32-math path (fp32 or odd shapes)."""
import math

import numpy as np
import pytest

from oracle import codecs as K
import oracle as O
from synth import gen as G
from tests.dsv4_testlib import (ROW_BF16, ROW_F32, ROW_FP8, ROW_MXFP4, assert_close, assert_quantized, decode_act,
                                dev, empty_rows, host, rows_to_f64, stored_rows_f64, topk_sets_match)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_08_amd as lib
    return lib


def act_arr(seed, stream, shape, std, dtype):
    x = G.normal(seed, stream, shape, std)
    return G.to_bf16(x) if dtype == "bf16" else x


# ====================================================================== compressors

CSA_CASES = [
    # (dtype, n, d, c, m, block0, n_left, comp_layout, raw_layout)
    ("f32", 61, 24, 8, 4, 0, 0, ROW_F32, ROW_F32),                # generic, ragged tail
    ("f32", 40, 16, 6, 2, 3, 2, ROW_F32, ROW_F32),                # generic, chunk with left context
    ("bf16", 200, 128, 64, 4, 0, 0, ROW_F32, ROW_F32),            # MFMA, ragged
    ("bf16", 256, 192, 128, 4, 0, 0, ROW_BF16, ROW_BF16),         # MFMA, bf16 outputs
    ("bf16", 128, 128, 128, 4, 17, 4, ROW_FP8, ROW_FP8),          # MFMA, fp8 rows, chunked
    ("bf16", 96, 64, 64, 4, 5, 4, ROW_MXFP4, ROW_F32),            # MFMA, MXFP4 keys
    ("bf16", 64, 40, 32, 4, 0, 0, ROW_MXFP4, ROW_BF16),           # generic (d % 64 != 0), MXFP4
    ("bf16", 36, 64, 64, 1, 0, 0, ROW_F32, ROW_F32),              # generic, m = 1
    ("bf16", 520, 256, 256, 4, 3, 4, ROW_FP8, ROW_FP8),           # pipelined 256-token tiles, ragged, left context
    ("bf16", 300, 192, 512, 4, 0, 0, ROW_BF16, ROW_F32),          # pipelined, entry 0 without b-window
]


@pytest.mark.parametrize("case", CSA_CASES, ids=[str(i) for i in range(len(CSA_CASES))])
def test_csa_compress(L, case):
    import torch
    dt, n, d, c, m, block0, n_left, cl, rl = case
    seed = 100 + n + d + c
    H = act_arr(seed, "H", (n_left + n, d), 1.0, dt)
    W = act_arr(seed, "W_kv", (4 * c, d), 2.0 / math.sqrt(d), dt)   # larger Z logits exercise the softmax
    B = G.normal(seed, "B_kv", (2, m, c), 0.5)
    S = n // m
    comp = empty_rows(max(S, 1), cl, c)
    sc = torch.zeros((max(S, 1), c // 32), dtype=torch.uint8, device="cuda") if cl == ROW_MXFP4 else None
    raw = empty_rows(n, rl, c)
    L.csa_compress(dev(H), dev(W), dev(B), m, c, comp, cl, n_left=n_left, block0=block0, comp_scales=sc,
                   raw_out=raw, raw_layout=rl)
    torch.cuda.synchronize()
    ref, ref_raw = O.csa_compress(decode_act(H), decode_act(W), B, m, block0, n_left)
    got = rows_to_f64(comp[:S], cl, c, sc[:S] if sc is not None else None)
    got_raw = rows_to_f64(raw, rl, c)
    for g_, r_, lay, what in ((got, ref, cl, "comp"), (got_raw, ref_raw, rl, "raw")):
        if lay == ROW_F32:
            assert_close(g_, r_, fp32=True, tol=1e-4 * max(1.0, np.abs(r_).max()), what=what)
        else:
            assert_quantized(g_, r_, lay, what=what)


HCA_CASES = [
    ("f32", 70, 16, 8, 8, ROW_F32, ROW_F32),          # generic, ragged
    ("bf16", 300, 128, 64, 128, ROW_F32, ROW_F32),    # MFMA, ragged tail
    ("bf16", 512, 64, 128, 128, ROW_BF16, ROW_BF16),  # MFMA
    ("bf16", 256, 128, 512, 128, ROW_FP8, ROW_FP8),   # MFMA, fp8 rows at c = 512
    ("bf16", 64, 64, 32, 16, ROW_MXFP4, ROW_F32),     # generic, MXFP4
    ("bf16", 700, 128, 256, 128, ROW_F32, ROW_BF16),  # pipelined 256-token tiles, ragged tail
]


@pytest.mark.parametrize("case", HCA_CASES, ids=[str(i) for i in range(len(HCA_CASES))])
def test_hca_compress(L, case):
    import torch
    dt, n, d, c, mp, cl, rl = case
    seed = 200 + n + c
    H = act_arr(seed, "H", (n, d), 1.0, dt)
    W = act_arr(seed, "W_hca", (2 * c, d), 2.0 / math.sqrt(d), dt)
    B = G.normal(seed, "B_hca", (mp, c), 0.5)
    S = n // mp
    comp = empty_rows(max(S, 1), cl, c)
    sc = torch.zeros((max(S, 1), c // 32), dtype=torch.uint8, device="cuda") if cl == ROW_MXFP4 else None
    raw = empty_rows(n, rl, c)
    L.hca_compress(dev(H), dev(W), dev(B), mp, c, comp, cl, comp_scales=sc, raw_out=raw, raw_layout=rl)
    torch.cuda.synchronize()
    ref, ref_raw = O.hca_compress(decode_act(H), decode_act(W), B, mp)
    got = rows_to_f64(comp[:S], cl, c, sc[:S] if sc is not None else None)
    got_raw = rows_to_f64(raw, rl, c)
    for g_, r_, lay, what in ((got, ref, cl, "comp"), (got_raw, ref_raw, rl, "raw")):
        if lay == ROW_F32:
            assert_close(g_, r_, fp32=True, tol=1e-4 * max(1.0, np.abs(r_).max()), what=what)
        else:
            assert_quantized(g_, r_, lay, what=what)


def test_compress_validation_errors(L):
    import torch
    H = torch.zeros((16, 8), dtype=torch.float32, device="cuda")
    W = torch.zeros((32, 8), dtype=torch.float32, device="cuda")
    B = torch.zeros((2, 4, 8), dtype=torch.float32, device="cuda")
    out = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(L.Dsv4Error) as e:
        L.csa_compress(H, W, B, 4, 8, out, ROW_F32, block0=2)          # no left context
    assert e.value.status == 1
    with pytest.raises(L.Dsv4Error) as e:
        L.csa_compress(H, W, B, 4, 8, out, ROW_MXFP4)                 # c % 32 != 0
    assert e.value.status == 2


CHUNK_CASES = [
    # (H dtype, n, d, n_left, block0, (c, layout, raw layout) of CSA KV / keys / HCA or None)
    ("bf16", 520, 256, 4, 5, (256, ROW_FP8, ROW_FP8), (64, ROW_MXFP4, None), (256, ROW_FP8, ROW_FP8)),  # fused, ragged
    ("bf16", 512, 192, 4, 0, (128, ROW_BF16, None), None, (64, ROW_F32, ROW_BF16)),                    # fused, no keys
    ("bf16", 300, 128, 4, 2, (64, ROW_F32, ROW_F32), (32, ROW_MXFP4, None), None),     # keys c = 32: one by one
    ("f32", 260, 64, 4, 3, (64, ROW_F32, ROW_F32), None, (32, ROW_BF16, ROW_F32)),     # f32 H: HCA rows start n_left in
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=[str(i) for i in range(len(CHUNK_CASES))])
def test_compress_chunk_equals_separate_calls(L, case):
    """The compressors of a chunk in one call give the separate calls' rows
    bit for bit (those calls are checked against the oracle above)."""
    import torch
    dt, n, d, n_left, block0, kv, ki, hc = case
    seed = 900 + n + d
    H = dev(act_arr(seed, "H", (n_left + n, d), 1.0, dt))

    def job(name, spec, mult, ratio):
        if spec is None:
            return None
        c, cl, rl = spec
        W = dev(act_arr(seed, "W_" + name, (mult * c, d), 2.0 / math.sqrt(d), dt))
        B = dev(G.normal(seed, "B_" + name, (2, ratio, c) if mult == 4 else (ratio, c), 0.5))
        S = n // ratio

        def outs():
            comp = empty_rows(max(S, 1), cl, c)
            sc = torch.zeros((max(S, 1), c // 32), dtype=torch.uint8, device="cuda") if cl == ROW_MXFP4 else None
            raw = empty_rows(n, rl, c) if rl is not None else None
            return comp, sc, raw
        return dict(W=W, B=B, c=c, cl=cl, rl=rl if rl is not None else ROW_F32, fused=outs(), sep=outs())

    jobs = {"kv": job("kv", kv, 4, 4), "ki": job("ki", ki, 4, 4), "hca": job("hca", hc, 2, 128)}
    mk = lambda j: None if j is None else L.compressor(j["W"], j["B"], j["c"], j["fused"][0], j["cl"],
                                                      comp_scales=j["fused"][1], raw_out=j["fused"][2],
                                                      raw_layout=j["rl"])
    L.compress_chunk(H, 4, n_left=n_left, block0=block0, csa_kv=mk(jobs["kv"]), csa_keys=mk(jobs["ki"]),
                     m_prime=128, hca=mk(jobs["hca"]))
    for name in ("kv", "ki"):
        j = jobs[name]
        if j is not None:
            comp, sc, raw = j["sep"]
            L.csa_compress(H, j["W"], j["B"], 4, j["c"], comp, j["cl"], n_left=n_left, block0=block0,
                           comp_scales=sc, raw_out=raw, raw_layout=j["rl"])
    j = jobs["hca"]
    if j is not None:
        comp, sc, raw = j["sep"]
        L.hca_compress(H[n_left:], j["W"], j["B"], 128, j["c"], comp, j["cl"], comp_scales=sc, raw_out=raw,
                       raw_layout=j["rl"])
    torch.cuda.synchronize()
    for name, j in jobs.items():
        if j is None:
            continue
        for a, b in zip(j["fused"], j["sep"]):
            if a is not None:
                assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                                   b.view(torch.uint8) if b.dtype != torch.uint8 else b), name


# ====================================================================== indexer

IDX_CASES = [
    # (q dtype, key layout, B, nq, hI, cI, S, m, pos0 list)
    ("f32", ROW_F32, 2, 37, 4, 32, 70, 4, [0, 200]),            # generic
    ("bf16", ROW_BF16, 1, 100, 32, 64, 600, 4, [1700]),         # MFMA prefill, ragged key tiles
    ("bf16", ROW_MXFP4, 2, 40, 32, 64, 1000, 4, [3, 3900]),     # MFMA prefill, MXFP4, causal boundary
    ("bf16", ROW_MXFP4, 3, 1, 32, 64, 5000, 4, [19999, 10000, 3]),   # MFMA decode mode
    ("bf16", ROW_BF16, 1, 20, 32, 128, 300, 4, [1199]),         # MFMA, cI = 128
    ("bf16", ROW_BF16, 1, 9, 16, 64, 50, 1, [30]),              # generic (hI = 16), m = 1
]


@pytest.mark.parametrize("case", IDX_CASES, ids=[str(i) for i in range(len(IDX_CASES))])
def test_indexer_score(L, case):
    import torch
    qd, kl, B, nq, hI, cI, S, m, pos = case
    seed = 300 + S + nq
    qI = act_arr(seed, "qI", (B, nq, hI, cI), 0.5, qd)
    wI = G.normal(seed, "wI", (B, nq, hI))
    kx = G.normal(seed, "cache_ki", (B, S, cI))
    keys, ksc = G.store(kx, kl) if kl != ROW_F32 else (kx, None)
    scores = torch.full((B, nq, S), float("nan"), dtype=torch.float32, device="cuda")
    L.indexer_score(dev(qI), dev(wI), dev(keys), kl, m, pos, scores, k_scales=dev(ksc) if ksc is not None else None)
    got = host(scores)
    for b in range(B):
        kf = stored_rows_f64(keys[b], kl, cI, ksc[b] if ksc is not None else None)
        ref = O.indexer_score(decode_act(qI[b]), wI[b].astype(np.float64), kf, m, pos[b] + np.arange(nq))
        vis = np.isfinite(ref)
        assert np.array_equal(np.isneginf(got[b]), ~vis), "visibility mask"
        if vis.any():
            scale = np.abs(ref[vis]).max()
            err = np.abs(got[b][vis] - ref[vis]).max() / scale
            assert err < 2e-5, "normalised score error %.3g" % err


def test_indexer_small_integers_bit_exact(L):
    """Small-integer queries/keys (E2M1 values) and weights in {+-1, +-2} make
    every partial sum an exactly representable integer, so any accumulation
    order gives the oracle's value bit for bit."""
    import torch
    rng = np.random.default_rng(7)
    B, nq, hI, cI, S, m = 1, 48, 32, 64, 700, 4
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6], dtype=np.float32)
    q = vals[rng.integers(0, len(vals), (B, nq, hI, cI))] * 2
    kx = vals[rng.integers(0, len(vals), (B, S, cI))]
    w = rng.choice(np.array([-2, -1, 1, 2], dtype=np.float32), (B, nq, hI))
    for kl in (ROW_BF16, ROW_MXFP4):
        keys, ksc = G.store(kx, kl)
        kf = stored_rows_f64(keys[0], kl, cI, ksc[0] if ksc is not None else None)
        scores = torch.empty((B, nq, S), dtype=torch.float32, device="cuda")
        L.indexer_score(dev(G.to_bf16(q)), dev(w), dev(keys), kl, m, [2000], scores,
                        k_scales=dev(ksc) if ksc is not None else None)
        ref = O.indexer_score(q[0].astype(np.float64), w[0].astype(np.float64), kf, m, 2000 + np.arange(nq))
        assert np.array_equal(host(scores)[0], ref.astype(np.float32))


IDX4_CASES = [
    # (q dtype, B, nq, hI, cI, S, m, pos0 list)
    ("bf16", 2, 40, 32, 64, 1000, 4, [3, 3900]),      # scaled-MFMA prefill, causal boundary, ragged tile
    ("bf16", 3, 1, 32, 64, 5000, 4, [19999, 10000, 3]),   # scaled-MFMA decode mode
    ("bf16", 1, 20, 32, 128, 300, 4, [1199]),         # scaled-MFMA, cI = 128
    ("f32", 2, 37, 4, 32, 70, 4, [0, 200]),           # generic (f32 query, cI = 32)
    ("bf16", 1, 9, 16, 64, 50, 1, [30]),              # generic (hI = 16), m = 1
]


@pytest.mark.parametrize("fmt", [4, 8])
@pytest.mark.parametrize("case", IDX4_CASES, ids=[str(i) for i in range(len(IDX4_CASES))])
def test_indexer_score_quantised_queries(L, case, fmt):
    """FP4 / FP8 indexer: the library rounds the query to MXFP4 or MXFP8
    itself; the oracle rounds the same stored query; the rounding decisions are
    exact on both sides (power-of-two scaling of the same bf16/f32 values), so
    only the summation order differs."""
    import torch
    qd, B, nq, hI, cI, S, m, pos = case
    call = L.indexer_score_fp8q if fmt == 8 else L.indexer_score_fp4q
    oracle_fn = O.indexer_score_fp8q if fmt == 8 else O.indexer_score_fp4q
    seed = 700 + S + nq
    qI = act_arr(seed, "qI", (B, nq, hI, cI), 0.5, qd)
    wI = G.normal(seed, "wI", (B, nq, hI))
    kx = G.normal(seed, "cache_ki", (B, S, cI))
    codes, ksc = G.store(kx, ROW_MXFP4)
    scores = torch.full((B, nq, S), float("nan"), dtype=torch.float32, device="cuda")
    call(dev(qI), dev(wI), dev(codes), dev(ksc), m, pos, scores)
    got = host(scores)
    for b in range(B):
        kf = stored_rows_f64(codes[b], ROW_MXFP4, cI, ksc[b])
        ref = oracle_fn(decode_act(qI[b]), wI[b].astype(np.float64), kf, m, pos[b] + np.arange(nq))
        vis = np.isfinite(ref)
        assert np.array_equal(np.isneginf(got[b]), ~vis), "visibility mask"
        if vis.any():
            scale = np.abs(ref[vis]).max()
            err = np.abs(got[b][vis] - ref[vis]).max() / scale
            assert err < 2e-5, "normalised score error %.3g" % err


def test_indexer_fp4q_small_integers_bit_exact(L):
    """Queries on the E2M1 grid (times 2) round to themselves, and every product
    and partial sum is a multiple of 1/2 below 2^24: any accumulation order
    gives the oracle's value bit for bit."""
    import torch
    rng = np.random.default_rng(8)
    B, nq, hI, cI, S, m = 1, 48, 32, 128, 700, 4
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6], dtype=np.float32)
    q = vals[rng.integers(0, len(vals), (B, nq, hI, cI))] * 2
    kx = vals[rng.integers(0, len(vals), (B, S, cI))]
    w = rng.choice(np.array([-2, -1, 1, 2], dtype=np.float32), (B, nq, hI))
    codes, ksc = G.store(kx, ROW_MXFP4)
    kf = stored_rows_f64(codes[0], ROW_MXFP4, cI, ksc[0])
    scores = torch.empty((B, nq, S), dtype=torch.float32, device="cuda")
    L.indexer_score_fp4q(dev(G.to_bf16(q)), dev(w), dev(codes), dev(ksc), m, [2000], scores)
    ref = O.indexer_score_fp4q(q[0].astype(np.float64), w[0].astype(np.float64), kf, m, 2000 + np.arange(nq))
    assert np.array_equal(host(scores)[0], ref.astype(np.float32))


def test_indexer_fp8q_small_integers_bit_exact(L):
    """Integer queries with |q| <= 14 and a block maximum of 8 or more (scale
    2^-5) sit on the E4M3 grid, E2M1 keys are multiples of 1/2, so every
    product and partial sum is a multiple of 1/2 below 2^24: any accumulation
    order gives the oracle's value bit for bit."""
    import torch
    rng = np.random.default_rng(9)
    B, nq, hI, cI, S, m = 1, 40, 32, 128, 650, 4
    q = rng.integers(-14, 15, (B, nq, hI, cI)).astype(np.float32)
    q[..., 0::32] = rng.choice(np.array([8, 9, 13, -9, -14], dtype=np.float32), q[..., 0::32].shape)
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6], dtype=np.float32)
    kx = vals[rng.integers(0, len(vals), (B, S, cI))]
    w = rng.choice(np.array([-2, -1, 1, 2], dtype=np.float32), (B, nq, hI))
    codes, ksc = G.store(kx, ROW_MXFP4)
    kf = stored_rows_f64(codes[0], ROW_MXFP4, cI, ksc[0])
    scores = torch.empty((B, nq, S), dtype=torch.float32, device="cuda")
    L.indexer_score_fp8q(dev(G.to_bf16(q)), dev(w), dev(codes), dev(ksc), m, [1900], scores)
    ref = O.indexer_score_fp8q(q[0].astype(np.float64), w[0].astype(np.float64), kf, m, 1900 + np.arange(nq))
    assert np.array_equal(host(scores)[0], ref.astype(np.float32))


# ====================================================================== top-k

TOPK_CASES = [
    # (rows B, nq, S, k, m, pos0 list, value kind)
    (1, 50, 256, 16, 4, [0], "int"),          # prefill causal, ties
    (2, 30, 16384, 512, 4, [40000, 100], "normal"),
    (1, 20, 40000, 1024, 4, [200000], "int"),  # two parts
    (16, 1, 262144, 1024, 4, [1 << 20] * 16, "normal"),   # decode shape: 16 parts + merge
    (1, 8, 300, 64, 1, [290], "zeros"),       # all ties incl. -0.0
    (1, 4, 5000, 4096, 4, [30000], "normal"), # large k
    (1, 3, 65536, 1024, 4, [300000], "asc"),  # every score beats the running threshold
    (1, 3, 65536, 1024, 4, [300000], "desc"), # the first scores are the answer
    (1, 6, 50001, 512, 4, [250000], "normal"), # rows not 16-byte aligned
    (1, 8, 100000, 1024, 1, [200000], "int"),  # long rows, heavy ties at the threshold
    (1, 2, 70000, 512, 4, [300000], "zeros"),  # long rows: the threshold bin holds 10000 equal keys
    (1, 3, 40000, 1024, 4, [1000], "normal"),  # long rows with fewer visible scores than k
    # the layer-pair chunk's routing: 512 or more rows of 264192 scores (2^18 + 2048 entries) at
    # positions 2^20 + 7000 + t, each row read whole by one streaming block (float4 loads)
    (1, 512, 264192, 1024, 4, [(1 << 20) + 7000], "asc"),
    (1, 512, 264192, 1024, 4, [(1 << 20) + 7000], "desc"),
    (1, 512, 264192, 1024, 4, [(1 << 20) + 7000], "int"),
    (1, 512, 264192, 1024, 4, [(1 << 20) + 7000], "zeros"),
    (2, 300, 264192, 1024, 4, [(1 << 20) + 1, (1 << 20) + 8000], "normal"),   # 600 rows over two sequences
    # S % 4 != 0: the same streaming kernel with scalar loads
    (1, 512, 264193, 1024, 4, [(1 << 20) + 7000], "normal"),
    (1, 512, 264193, 1024, 4, [(1 << 20) + 7000], "int"),
]


def topk_scores(B, nq, S, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "int":
        return rng.integers(-20, 20, (B, nq, S)).astype(np.float32)
    if kind == "zeros":
        sc = np.where(rng.random((B, nq, S)) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        sc[..., ::7] = 1.0
        return sc
    if kind in ("asc", "desc"):
        ramp = np.linspace(-3.0, 5.0, S, dtype=np.float32)
        return np.broadcast_to(ramp if kind == "asc" else ramp[::-1], (B, nq, S)).copy()
    return G.normal(S, "extra", (B, nq, S), 10.0)


def topk_check_rows(B, nq, seed):
    """Every row of small cases; 64 seeded rows plus the first and last of each
    sequence when there are many (the oracle sorts whole rows)."""
    if B * nq <= 128:
        return [(b, t) for b in range(B) for t in range(nq)]
    rng = np.random.default_rng(seed)
    rows = {(b, 0) for b in range(B)} | {(b, nq - 1) for b in range(B)}
    for r in rng.choice(B * nq, size=64, replace=False):
        rows.add((int(r) // nq, int(r) % nq))
    return sorted(rows)


@pytest.mark.parametrize("case", TOPK_CASES, ids=[str(i) for i in range(len(TOPK_CASES))])
def test_topk_select_bit_exact(L, case):
    import torch
    B, nq, S, k, m, pos, kind = case
    sc = topk_scores(B, nq, S, kind, S + k)
    scores = dev(sc)
    idx = torch.empty((B, nq, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, L.topk_workspace_size(B, nq, S, k)), dtype=torch.uint8, device="cuda")
    L.topk_select(scores, m, pos, k, idx, ws)
    got = host(idx)
    del scores
    for b, t in topk_check_rows(B, nq, S + nq):
        ref = O.topk_select(sc[b, t:t + 1].astype(np.float64), m, [pos[b] + t], k)
        assert np.array_equal(got[b, t], ref[0]), (b, t)


# ====================================================================== attention cores

def make_rows(seed, stream, shape, layout):
    x = G.normal(seed, stream, shape)
    st, _ = G.store(x, layout)
    return st


SPARSE_CASES = [
    # (q dtype, layout, B, nq, nh, c, S, k, n_win, W, pos0, sink)
    ("f32", ROW_F32, 2, 20, 8, 64, 40, 16, 64, 300, [100, 230], True),       # generic
    ("bf16", ROW_BF16, 1, 40, 64, 128, 300, 64, 128, 1400, [1200], True),    # MFMA no split
    ("bf16", ROW_FP8, 3, 2, 64, 512, 2000, 200, 128, 300, [250, 160, 130], True),   # MFMA split (decode)
    ("bf16", ROW_FP8, 1, 33, 64, 512, 500, 100, 0, 0, [4000], False),        # no window
    ("bf16", ROW_BF16, 1, 5, 64, 128, 50, 0, 16, 40, [20], True),            # k = 0: window only
    ("bf16", ROW_BF16, 1, 6, 16, 128, 50, 8, 16, 40, [20], True),            # generic (nh = 16 sparse)
    ("bf16", ROW_BF16, 2, 3, 32, 128, 900, 300, 128, 300, [800, 450], True), # c = 128, one row group, split
    ("bf16", ROW_BF16, 1, 35, 128, 128, 600, 200, 64, 300, [500], False),    # c = 128, four row groups
]


@pytest.mark.parametrize("case", SPARSE_CASES, ids=[str(i) for i in range(len(SPARSE_CASES))])
def test_sparse_mqa(L, case):
    import torch
    qd, lay, B, nq, nh, c, S, k, nw, W, pos, use_sink = case
    seed = 500 + S + c + nq
    rng = np.random.default_rng(seed)
    q = act_arr(seed, "q", (B, nq, nh, c), 1.0, qd)
    kv = make_rows(seed, "cache_kv", (B, S, c), lay)
    win = make_rows(seed, "win_kv", (B, max(W, 1), c), lay)
    wpos = [max(0, p - nw + 1) for p in pos]
    idx = np.full((B, nq, max(k, 1)), -1, dtype=np.int32)
    for b in range(B):
        for t in range(nq):
            sel = rng.choice(S, size=min(k, S), replace=False)
            keep = rng.random(sel.size) > 0.1                       # some padding slots
            idx[b, t, :sel.size] = np.where(keep, sel, -1)
    if k == 0:
        idx = idx[:, :, :0]
    sink = G.normal(seed, "sink", (nh,), 0.5)
    scale = 1 / math.sqrt(c)
    qt = dev(q)
    out = torch.empty_like(qt)
    ws = torch.empty(max(1, L.attn_workspace_size(False, B, nq, nh, c, k + nw)), dtype=torch.uint8, device="cuda")
    L.sparse_mqa_fwd(qt, dev(kv), lay, dev(idx) if k > 0 else None, dev(win) if nw > 0 else None, wpos, nw, pos,
                     dev(sink) if use_sink else None, scale, out, ws, W=W)
    got = host(out)
    got = decode_act(got)
    for b in range(B):
        kvf = stored_rows_f64(kv[b], lay, c)
        winf = stored_rows_f64(win[b], lay, c)[:W]
        ref = O.sparse_mqa(decode_act(q[b]), kvf, idx[b], winf, wpos[b], nw, pos[b] + np.arange(nq),
                           sink.astype(np.float64) if use_sink else None, scale)
        assert_close(got[b], ref, fp32=(qd == "f32"), what="sparse b=%d" % b)


DENSE_CASES = [
    # (q dtype, layout, B, nq, nh, c, S, mp, n_win, pos0, sink)
    ("f32", ROW_F32, 1, 30, 4, 64, 20, 8, 16, [120], True),                  # generic
    ("bf16", ROW_BF16, 1, 70, 16, 128, 40, 128, 128, [4000], True),          # MFMA, 4 queries per block
    ("bf16", ROW_FP8, 1, 40, 64, 512, 200, 128, 128, [20000], True),         # MFMA, c = 512
    ("bf16", ROW_FP8, 1, 33, 64, 512, 600, 128, 128, [64100], True),         # c = 512, visible count steps mid-chunk
    ("bf16", ROW_FP8, 1, 10, 32, 512, 300, 128, 128, [40000], False),        # c = 512, 2 queries per block, odd tail
    ("bf16", ROW_FP8, 1, 13, 16, 512, 150, 128, 64, [19000], True),          # c = 512, 4 queries per block, ragged
    ("bf16", ROW_FP8, 2, 1, 64, 512, 700, 128, 128, [1 << 16, 30000], True), # decode: split + combine
    ("bf16", ROW_FP8, 1, 8, 64, 512, 10, 128, 128, [50], True),              # no entry visible yet: window only
    ("bf16", ROW_FP8, 2, 1, 64, 512, 700, 128, 0, [1 << 16, 50], True),     # split launch, second sequence keyless
    ("bf16", ROW_BF16, 1, 37, 32, 128, 10, 16, 0, [100], False),             # 2 queries per block, no window
    # HCA decode with 3965 visible entries, in the workspace the call needs exactly (the visible counts where
    # the split plan of the size query, the argument check and the launch once disagreed)
    ("bf16", ROW_FP8, 1, 1, 64, 512, 8192, 128, 128, [3965 * 128 + 5], True),
    # c = 512 prefill over 64 or more queries (ragged last block, visible count stepping mid-chunk, 1 / 2 / 4
    # queries per block, window only, no window, two sequences)
    ("bf16", ROW_FP8, 1, 67, 64, 512, 300, 128, 128, [38000], True),
    ("bf16", ROW_FP8, 1, 130, 32, 512, 500, 128, 64, [64000], False),
    ("bf16", ROW_FP8, 2, 260, 16, 512, 100, 128, 128, [12700, 200], True),
    ("bf16", ROW_FP8, 1, 70, 64, 512, 10, 128, 128, [0], True),
    ("bf16", ROW_FP8, 1, 64, 64, 512, 257, 128, 0, [40000], False),
    # c = 128 bf16 rows: a split key range merged by the combine kernel, one query per block
    ("bf16", ROW_BF16, 1, 3, 64, 128, 2100, 128, 128, [2000 * 128 + 50], True),
    ("bf16", ROW_BF16, 1, 20, 128, 128, 300, 128, 128, [30000], True),
]


@pytest.mark.parametrize("case", DENSE_CASES, ids=[str(i) for i in range(len(DENSE_CASES))])
def test_hca_dense(L, case):
    import torch
    qd, lay, B, nq, nh, c, S, mp, nw, pos, use_sink = case
    seed = 600 + S + c + nq
    q = act_arr(seed, "q", (B, nq, nh, c), 1.0, qd)
    kv = make_rows(seed, "cache_hca", (B, S, c), lay)
    wpos = [max(0, p - nw + 1) for p in pos]
    W = nq + nw
    win = make_rows(seed, "win_hca", (B, W, c), lay)
    sink = G.normal(seed, "sink", (nh,), 0.5)
    scale = 1 / math.sqrt(c)
    qt = dev(q)
    out = torch.empty_like(qt)
    need = L.attn_plan(True, L.BF16 if qd == "bf16" else L.F32, lay, B, nq, nh, c, S, 0, mp, nw, pos).workspace_bytes
    assert need <= L.attn_workspace_size(True, B, nq, nh, c, S + nw)
    ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")
    L.hca_dense_fwd(qt, dev(kv), lay, mp, dev(win), wpos, nw, pos, dev(sink) if use_sink else None, scale, out, ws)
    got = decode_act(host(out))
    for b in range(B):
        ref = O.hca_dense(decode_act(q[b]), stored_rows_f64(kv[b], lay, c), mp, stored_rows_f64(win[b], lay, c),
                          wpos[b], nw, pos[b] + np.arange(nq), sink.astype(np.float64) if use_sink else None, scale)
        assert_close(got[b], ref, fp32=(qd == "f32"), what="dense b=%d" % b)


@pytest.mark.parametrize("dense,late", [(True, True), (True, False), (False, True), (False, False)])
def test_attention_late_key_far_above_first_tiles(L, dense, late):
    """A key whose logits exceed those of the first key tile by far more than
    2^32 (log2 units): the softmax of a row is taken against the maximum of
    its first visible tile, so a key this large in a later tile makes the
    block run its keys a second time against the exact maximum.  The output
    must match the oracle either way (late = False puts the key first)."""
    import torch
    B, nq, nh, c, S, mp, nw = 1, 3, 64, 512, 300, 4, 128
    pos = [1500]
    seed = 700 + int(dense) + 2 * int(late)
    q = np.abs(G.normal(seed, "q", (B, nq, nh, c), 1.0)).astype(np.float32)
    x = G.normal(seed, "cache_hca", (B, S, c), 1.0)
    big = 250 if late else 3                       # a visible entry in a late / the first key tile
    x[0, big, :c - 64] = 400.0
    x[0, big, c - 64:] = 2.0
    kv, _ = G.store(x, ROW_FP8)
    win, _ = G.store(G.normal(seed, "win_hca", (B, nq + nw, c), 1.0), ROW_FP8)
    wpos = [pos[0] - nw + 1]
    sink = G.normal(seed, "sink", (nh,), 0.5)
    scale = 1 / math.sqrt(c)
    qt = dev(G.to_bf16(q))
    out = torch.empty_like(qt)
    qd = decode_act(G.to_bf16(q))
    kvf, winf = stored_rows_f64(kv[0], ROW_FP8, c), stored_rows_f64(win[0], ROW_FP8, c)
    pq = pos[0] + np.arange(nq)
    if dense:
        need = L.attn_plan(True, L.BF16, ROW_FP8, B, nq, nh, c, S, 0, mp, nw, pos).workspace_bytes
        ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")
        L.hca_dense_fwd(qt, dev(kv), ROW_FP8, mp, dev(win), wpos, nw, pos, dev(sink), scale, out, ws)
        ref = O.hca_dense(qd[0], kvf, mp, winf, wpos[0], nw, pq, sink.astype(np.float64), scale)
    else:
        k = 256
        others = np.array([e for e in range(S) if e != big])
        rows = [np.random.default_rng(seed + t).permutation(others)[:k - 1] for t in range(nq)]
        # the big key last (a late tile) or first
        idx = np.stack([np.append(r, big) if late else np.insert(r, 0, big) for r in rows])[None].astype(np.int32)
        need = L.attn_plan(False, L.BF16, ROW_FP8, B, nq, nh, c, S, k, 1, nw, pos).workspace_bytes
        ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")
        L.sparse_mqa_fwd(qt, dev(kv), ROW_FP8, dev(idx), dev(win), wpos, nw, pos, dev(sink), scale, out, ws)
        ref = O.sparse_mqa(qd[0], kvf, idx[0], winf, wpos[0], nw, pq, sink.astype(np.float64), scale)
    assert_close(decode_act(host(out))[0], ref, what="late large key")


def test_attention_decodes_every_fp8_code(L):
    """q = 0 and a single key: the output is that key, so each stored E4M3 code
    (all 254 finite ones) and the bf16 RoPE dims come back exactly."""
    import torch
    c, nh = 512, 64
    codes = np.array([x for x in range(256) if x & 0x7F != 0x7F], dtype=np.uint8)
    row = np.zeros((1, 1, c + 64), np.uint8)
    row[0, 0, :254] = codes
    row[0, 0, 254:448] = codes[:194]
    row[0, 0, 448:] = G.to_bf16(G.normal(1, "extra", (64,))).view(np.uint8)
    q = torch.zeros((1, 1, nh, c), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    idx = torch.zeros((1, 1, 1), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, L.attn_workspace_size(False, 1, 1, nh, c, 1)), dtype=torch.uint8, device="cuda")
    L.sparse_mqa_fwd(q, dev(row), ROW_FP8, idx, None, [0], 0, [10], None, 0.1, out, ws)
    got = decode_act(host(out))[0, 0]
    want = K.decode_rows(row[0, 0], ROW_FP8, c)
    # the output is stored as bf16: every E4M3 value and every bf16 value is exact in bf16
    assert np.array_equal(got, np.broadcast_to(want, (nh, c)))


@pytest.mark.parametrize("use_sink", [False, True])
def test_sparse_all_padding_gives_zero(L, use_sink):
    """Every index slot is padding and there is no window: no key is visible,
    so the output is exactly zero (the sink, if any, carries a zero value)."""
    import torch
    c, nh, nq, S, k = 512, 64, 3, 100, 64
    q = torch.from_numpy(G.to_bf16(G.normal(5, "q", (1, nq, nh, c))).view(np.int16)).cuda().view(torch.bfloat16)
    kv = make_rows(5, "cache_kv", (1, S, c), ROW_FP8)
    idx = torch.full((1, nq, k), -1, dtype=torch.int32, device="cuda")
    sink = torch.from_numpy(G.normal(5, "sink", (nh,), 0.5)).cuda() if use_sink else None
    out = torch.full_like(q, 7.0)
    ws = torch.empty(max(1, L.attn_workspace_size(False, 1, nq, nh, c, k)), dtype=torch.uint8, device="cuda")
    L.sparse_mqa_fwd(q, dev(kv), ROW_FP8, idx, None, [0], 0, [400], sink, 0.05, out, ws)
    ref = O.sparse_mqa(np.zeros((nq, nh, c)), K.decode_rows(kv[0], ROW_FP8, c), np.full((nq, k), -1), np.zeros((0, c)), 0, 0,
                       400 + np.arange(nq), G.normal(5, "sink", (nh,), 0.5).astype(np.float64) if use_sink else None,
                       0.05)
    assert not ref.any()
    assert not host(out.float()).any()


def test_attention_window_must_be_covered(L):
    import torch
    q = torch.zeros((1, 4, 64, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    win = torch.zeros((1, 10, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    idx = torch.zeros((1, 4, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(L.Dsv4Error) as e:   # query 103 needs position 103 but rows cover [90, 100)
        L.sparse_mqa_fwd(q, kv, ROW_BF16, idx, win, [90], 8, [100], None, 1.0, out, None)
    assert e.value.status == 1


# ====================================================================== Q/KV RMSNorm, partial RoPE, output rotation

NRQ_CASES = [
    # (dtype, B, nq, nh, c, rope_dims, pos0 list, gamma)
    ("bf16", 2, 5, 64, 512, 64, [1 << 20, 17], True),    # the configs' shape, positions near 2^20
    ("f32", 1, 3, 4, 128, 64, [5], True),
    ("f32", 1, 2, 3, 1024, 64, [999999], False),         # two passes of 512 per row
    ("bf16", 1, 2, 8, 64, 0, [3], True),                 # no rotated dims
]


def _gamma(seed, c):
    return (1.0 + G.normal(seed, "gamma", (c,), 0.3)).astype(np.float32)


@pytest.mark.parametrize("case", NRQ_CASES, ids=[str(i) for i in range(len(NRQ_CASES))])
def test_q_norm_rope(L, case):
    import torch
    dt, B, nq, nh, c, R, pos, use_g = case
    seed = 800 + c + nh
    q = act_arr(seed, "q", (B, nq, nh, c), 2.0, dt)
    g = _gamma(seed, c) if use_g else None
    qd = dev(q)
    out = torch.empty_like(qd)
    L.q_norm_rope(qd, dev(g) if use_g else None, pos, out=out, rope_dims=R)
    got = host(out)
    for b in range(B):
        ref = O.q_norm_rope(decode_act(q[b]), g if use_g else np.ones(c), pos[b] + np.arange(nq), rope_dims=R)
        if dt == "f32":
            assert_close(got[b], ref, fp32=True, tol=2e-5, what="q_norm_rope")
        else:
            assert_quantized(decode_act(got[b]), ref, ROW_BF16, rel=2e-6, what="q_norm_rope")
    # in place gives the same bytes
    L.q_norm_rope(qd, dev(g) if use_g else None, pos, rope_dims=R)
    assert np.array_equal(host(qd), got)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_out_rope(L, dt):
    B, nq, nh, c, pos = 2, 7, 64, 512, [1 << 20, 3]
    o = act_arr(900, "o", (B, nq, nh, c), 1.0, dt)
    od = dev(o)
    L.out_rope(od, pos)
    got = host(od)
    assert np.array_equal(got[..., :c - 64], o[..., :c - 64]), "dims outside the rotated block changed"
    for b in range(B):
        ref = O.out_rope(decode_act(o[b]), pos[b] + np.arange(nq))
        if dt == "f32":
            assert_close(got[b], ref, fp32=True, tol=2e-6, what="out_rope")
        else:
            assert_quantized(decode_act(got[b]), ref, ROW_BF16, rel=2e-6, what="out_rope")


NRKV_CASES = [
    # (in layout, out layout, B, n, c, rope_dims, pos0 list, stride, gamma)
    (ROW_F32, ROW_FP8, 2, 37, 512, 64, [4 * (262144 + 1) - 1, 7], 4, True),   # compressed entries -> cache rows
    (ROW_BF16, ROW_BF16, 1, 130, 128, 64, [(1 << 20) - 127], 1, True),         # window rows
    (ROW_F32, ROW_F32, 1, 9, 512, 64, [1023], 128, False),                     # in place, HCA entry stride
]


@pytest.mark.parametrize("case", NRKV_CASES, ids=[str(i) for i in range(len(NRKV_CASES))])
def test_kv_norm_rope(L, case):
    il, ol, B, n, c, R, pos0, stride, use_g = case
    seed = 950 + n + c
    x = G.normal(seed, "rows", (B, n, c), 1.5)
    rows, _ = G.store(x, il)
    g = _gamma(seed, c) if use_g else None
    rd = dev(rows)
    inplace = il == ol and il == ROW_F32
    out = rd if inplace else empty_rows(B * n, ol, c).view(B, n, -1)
    L.kv_norm_rope(rd, il, c, dev(g) if use_g else None, pos0, stride, out, ol, rope_dims=R)
    for b in range(B):
        xin = stored_rows_f64(rows[b], il, c)
        ref = O.kv_norm_rope(xin, g if use_g else np.ones(c), pos0[b] + stride * np.arange(n), rope_dims=R)
        got = rows_to_f64(out[b], ol, c)
        if ol == ROW_F32:
            assert_close(got, ref, fp32=True, tol=2e-5, what="kv_norm_rope")
        else:
            assert_quantized(got, ref, ol, rel=2e-6, what="kv_norm_rope")


# ====================================================================== projections (bf16 GEMM)

GEMM_CASES = [
    # (M, N, K, batch, out dtype, rows checked (None: all))
    (300, 200, 128, 1, "bf16", None),          # 128 x 128 tiles, ragged in M and N
    (4096, 4096, 128, 1, "bf16", 96),          # 256 x 256 tiles, XCD tile order
    (130, 96, 192, 3, "f32", None),            # batched, fp32 output
    (8192, 32, 256, 1, "f32", 64),             # a skinny output (the indexer head weights)
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=[str(i) for i in range(len(GEMM_CASES))])
def test_gemm_bf16_nt(L, case):
    import torch
    M, N, Kd, nb, od, nrows = case
    seed = 1000 + M + N
    A = G.to_bf16(G.normal(seed, "extra", (nb, M, Kd)))
    Bm = G.to_bf16(G.normal(seed + 1, "extra", (nb, N, Kd)))
    C = torch.empty((nb, M, N), dtype=torch.float32 if od == "f32" else torch.bfloat16, device="cuda")
    L.gemm_bf16_nt(dev(A), dev(Bm), C, batch=nb, stride_a=M * Kd, stride_b=N * Kd, stride_c=M * N, M=M, N=N, K=Kd)
    got = host(C)
    rows = np.arange(M) if nrows is None else np.unique(np.linspace(0, M - 1, nrows).astype(np.int64))
    for b in range(nb):
        ref = K.bf16_decode(A[b][rows]) @ K.bf16_decode(Bm[b]).T
        g = got[b][rows]
        if od == "f32":
            assert_close(g, ref, fp32=True, tol=2e-6 * np.sqrt(Kd) * np.abs(ref).max(), what="gemm f32")
        else:
            assert_quantized(decode_act(g), ref, ROW_BF16, rel=2e-6, what="gemm bf16")


def test_query_proj(L):
    import torch
    n, d, dc, nh, c, hI, cI = 200, 256, 128, 2, 128, 2, 64
    r = lambda st, sh, sd: G.to_bf16(G.normal(1100 + len(sh), st, sh, sd))
    h = r("H", (n, d), 1.0)
    W_DQ, W_UQ, W_IUQ, W_w = (r("W_kv", (dc, d), d ** -0.5), r("W_ki", (nh * c, dc), dc ** -0.5),
                              r("W_hca", (hI * cI, dc), dc ** -0.5), r("extra", (hI, d), d ** -0.5))
    q = torch.empty((n, nh, c), dtype=torch.bfloat16, device="cuda")
    qI = torch.empty((n, hI, cI), dtype=torch.bfloat16, device="cuda")
    wI = torch.empty((n, hI), dtype=torch.float32, device="cuda")
    ws = torch.empty(L.query_proj_workspace_size(n, dc), dtype=torch.uint8, device="cuda")
    L.query_proj(dev(h), dev(W_DQ), dev(W_UQ), dev(W_IUQ), dev(W_w), nh=nh, c=c, hI=hI, cI=cI, q=q, qI=qI, wI=wI,
                 ws=ws)
    rq, rqI, rwI = O.query_proj(*[K.bf16_decode(x) for x in (h, W_DQ, W_UQ, W_IUQ, W_w)], nh=nh, c=c, hI=hI, cI=cI)
    # the two sides round c^Q to bf16 from fp32 / fp64 sums: a rare one-ulp difference there moves q slightly
    assert_close(decode_act(host(q)), rq, tol=1e-2, what="q")
    assert_close(decode_act(host(qI)), rqI, tol=1e-2, what="qI")
    assert_close(host(wI), rwI, fp32=True, tol=1e-4, what="wI")


def test_output_proj(L):
    import torch
    n, nh, c, g, dg, d = 130, 8, 64, 4, 64, 192
    r = lambda st, sh, sd: G.to_bf16(G.normal(1200 + len(sh), st, sh, sd))
    o = r("o", (n, nh, c), 1.0)
    W1 = r("W_kv", (g, dg, nh // g * c), (nh // g * c) ** -0.5)
    W2 = r("W_ki", (d, g * dg), (g * dg) ** -0.5)
    out = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(L.output_proj_workspace_size(n, g, dg), dtype=torch.uint8, device="cuda")
    L.output_proj(dev(o), dev(W1), dev(W2), out, g=g, ws=ws)
    ref = O.output_proj(K.bf16_decode(o), K.bf16_decode(W1), K.bf16_decode(W2), g)
    assert_close(decode_act(host(out)), ref, tol=1e-2, what="output_proj")
