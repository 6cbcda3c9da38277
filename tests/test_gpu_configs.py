"""End-to-end parity of the five workload configurations at their full sizes,
through the C ABI, against the float64 oracle.  Where the oracle cannot
afford every query, a seeded sample of query rows (first, last, block
boundaries, random) is checked one by one; compressors are checked in full.

Tolerances: fp32 configuration max-abs <= 1e-4; bf16/fp8 configurations
||d||_inf / ||ref||_inf <= 2e-2; stored (quantised) entries must be a correct
rounding of the oracle value; top-k sets compared margin-aware (scores are
computed independently on both sides)."""
import math

import numpy as np
import pytest

import oracle as O
from oracle import codecs as K
from synth import gen as G
from tests.dsv4_testlib import (ROW_F32, ROW_FP8, ROW_MXFP4, assert_close, assert_quantized, decode_act, dev,
                                gpu_csa_layer, gpu_hca_layer, host, oracle_csa_layer, oracle_hca_layer,
                                rows_to_f64, stored_rows_f64, topk_sets_match)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_08_amd as lib
    return lib


def sample_rows(n, m, count, seed, also=()):
    """First and last rows, block boundaries of ratio m, the rows in `also`,
    and seeded random rows up to `count` in all."""
    rng = np.random.default_rng(seed)
    base = sorted(set(int(x) for x in [0, 1, m - 1, m, 2 * m - 1, n // 2, n - 2, n - 1] + list(also) if 0 <= x < n))
    rest = np.setdiff1d(np.arange(n), base)
    extra = list(rng.choice(rest, size=max(0, count - len(base)), replace=False))
    return np.array(sorted(set(base + [int(x) for x in extra])))


def assert_topk_exact_on_gpu_scores(g_idx, g_sc, m, pos, k, what):
    """Top-k index sets bit-exact given identical scores: the oracle's selector
    run on the GPU's own fp32 scores picks exactly the GPU's indices."""
    ref = O.topk_select(g_sc.astype(np.float64), m, pos, k)
    bad = [i for i in range(len(pos)) if not np.array_equal(g_idx[i], ref[i])]
    assert not bad, "%s: top-k differs from the oracle's on identical scores at rows %s" % (what, bad[:8])


def check_attention_rows(got_out, ref, rows, gpu_idx, ref_idx, ref_scores, k, fp32, ref_with_idx=None):
    """Rows whose GPU selection equals the oracle's are compared with the
    oracle output; a row whose selection differs only among near-tied scores
    (allowed: the scores are computed independently on both sides) is
    compared with the oracle run on the GPU's own selection."""
    near = topk_sets_match(gpu_idx, ref_idx, ref_scores, k) if gpu_idx is not None else []
    keep = [i for i in range(len(rows)) if i not in near]
    assert len(near) <= max(1, len(rows) // 20), "too many near-tie rows: %d" % len(near)
    assert_close(got_out[keep], ref[keep], fp32=fp32, what="attention output")
    if near:
        assert ref_with_idx is not None, "near-tie rows %s need a reference on the GPU's selection" % near
        sel = np.asarray(near)
        assert_close(got_out[sel], ref_with_idx(sel, gpu_idx[sel]), fp32=fp32, what="attention output (GPU top-k)")


# ---------------------------------------------------------------------- configuration 1

def test_cfg1_csa_fp32_end_to_end(L):
    inp = G.make(1)
    g = gpu_csa_layer(L, inp)
    r = oracle_csa_layer(inp)
    assert_close(rows_to_f64(g["comp"], ROW_F32, 64), r["comp"], fp32=True, what="compressed KV")
    assert_close(rows_to_f64(g["raw"], ROW_F32, 64), r["raw"], fp32=True, what="window rows")
    assert_close(rows_to_f64(g["ki"], ROW_F32, 32), r["ki"], fp32=True, what="indexer keys")
    sc = host(g["scores"])[0]
    vis = np.isfinite(r["scores"])
    assert np.array_equal(np.isfinite(sc), vis)
    assert_close(sc[vis], r["scores"][vis], fp32=True, what="scores")
    out = decode_act(host(g["out"])[0])
    g_idx = host(g["idx"])[0]
    assert_topk_exact_on_gpu_scores(g_idx, sc, 4, r["rows"], 16, "cfg1")
    ref_fn = lambda sel, ix: O.sparse_mqa(decode_act(inp["q"])[r["rows"][sel]], r["comp_s"], ix, r["raw_s"], 0, 64,
                                          r["rows"][sel], inp["sink"].astype(np.float64), 1 / 8.0)
    check_attention_rows(out, r["out"], r["rows"], g_idx, r["idx"], r["scores"], 16, fp32=True, ref_with_idx=ref_fn)


# ---------------------------------------------------------------------- configuration 2

def test_cfg2_hca_bf16(L):
    inp = G.make(2)
    cfg = inp["cfg"]
    g = gpu_hca_layer(L, inp)
    rows = sample_rows(cfg["n"], cfg["mp"], 48, 1)
    r = oracle_hca_layer(inp, rows)
    assert_quantized(rows_to_f64(g["comp"], cfg["kv_layout"], cfg["c"]), r["comp"], cfg["kv_layout"], what="comp")
    assert_quantized(rows_to_f64(g["raw"], cfg["kv_layout"], cfg["c"]), r["raw"], cfg["kv_layout"], what="raw")
    out = decode_act(host(g["out"])[0])[rows]
    assert_close(out, r["out"], what="hca output")


# ---------------------------------------------------------------------- configuration 3

def test_cfg3_csa_prefill_bf16(L):
    inp = G.make(3)
    cfg = inp["cfg"]
    g = gpu_csa_layer(L, inp)
    rows = sample_rows(cfg["n"], cfg["m"], 40, 2)
    r = oracle_csa_layer(inp, rows)
    c, cI = cfg["c"], cfg["cI"]
    assert_quantized(rows_to_f64(g["comp"], cfg["kv_layout"], c), r["comp"], cfg["kv_layout"], what="comp")
    assert_quantized(rows_to_f64(g["ki"], cfg["key_layout"], cI), r["ki"], cfg["key_layout"], what="keys")
    sc = host(g["scores"][0, rows])
    # scores: the stored keys on both sides may differ by one rounding step at
    # a midpoint, so compare with the bf16-level tolerance
    vis = np.isfinite(r["scores"])
    assert np.array_equal(np.isfinite(sc), vis)
    assert_close(sc[vis], r["scores"][vis], tol=1e-3, what="scores")
    g_idx = host(g["idx"][0, rows])
    assert_topk_exact_on_gpu_scores(g_idx, sc, cfg["m"], rows, cfg["k"], "cfg3")
    out = decode_act(host(g["out"][0, rows]))
    ref_fn = lambda sel, ix: O.sparse_mqa(decode_act(inp["q"])[rows[sel]], r["comp_s"], ix, r["raw_s"], 0,
                                          cfg["n_win"], rows[sel], inp["sink"].astype(np.float64), 1 / math.sqrt(c))
    check_attention_rows(out, r["out"], rows, g_idx, r["idx"], r["scores"], cfg["k"], fp32=False, ref_with_idx=ref_fn)


# ---------------------------------------------------------------------- configuration 4

def run_decode(L, inp, bsel=None):
    import torch
    cfg = inp["cfg"]
    c, nh, hI, cI, k, nw, m, mp = cfg["c"], cfg["nh"], cfg["hI"], cfg["cI"], cfg["k"], cfg["n_win"], cfg["m"], cfg["mp"]
    bs = list(range(cfg["B"])) if bsel is None else list(bsel)
    B = len(bs)
    S = inp["kv_cache"].shape[1]
    Sh = inp["hca_cache"].shape[1]
    sub = lambda key: dev(inp[key][bs])
    qp = [int(inp["q_pos0"][b]) for b in bs]
    wp = [int(inp["win_pos0"][b]) for b in bs]
    scores = torch.empty((B, 1, S), dtype=torch.float32, device="cuda")
    L.indexer_score(sub("qI"), sub("wI"), sub("ki_codes"), ROW_MXFP4, m, qp, scores, k_scales=sub("ki_scales"))
    idx = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, L.topk_workspace_size(B, 1, S, k)), dtype=torch.uint8, device="cuda")
    L.topk_select(scores, m, qp, k, idx, ws)
    q = sub("q")
    out = torch.empty_like(q)
    aws = torch.empty(max(1, L.attn_workspace_size(True, B, 1, nh, c, Sh + nw)), dtype=torch.uint8, device="cuda")
    L.sparse_mqa_fwd(q, sub("kv_cache"), ROW_FP8, idx, sub("kv_win"), wp, nw, qp, dev(inp["sink"]),
                     1 / math.sqrt(c), out, aws)
    qh = sub("q_hca")
    out_h = torch.empty_like(qh)
    L.hca_dense_fwd(qh, sub("hca_cache"), ROW_FP8, mp, sub("hca_win"), wp, nw, qp, dev(inp["sink_hca"]),
                    1 / math.sqrt(c), out_h, aws)
    torch.cuda.synchronize()
    return dict(scores=scores, idx=idx, out=out, out_h=out_h)


@pytest.fixture(scope="module")
def cfg4():
    return G.make(4)


def test_cfg4_decode(L, cfg4):
    inp = cfg4
    cfg = inp["cfg"]
    c, m, mp, k, nw = cfg["c"], cfg["m"], cfg["mp"], cfg["k"], cfg["n_win"]
    g = run_decode(L, inp)
    scores = host(g["scores"])
    idx = host(g["idx"])
    out = decode_act(host(g["out"]))
    out_h = decode_act(host(g["out_h"]))
    scale = 1 / math.sqrt(c)
    for b in range(cfg["B"]):
        p = int(inp["q_pos0"][b])
        keys = K.mxfp4_decode(inp["ki_codes"][b], inp["ki_scales"][b])
        I = O.indexer_score(decode_act(inp["qI"][b]), inp["wI"][b].astype(np.float64), keys, m, [p])
        # identical stored inputs on both sides: fp32 accumulation only
        assert_close(scores[b], I, tol=2e-5, what="decode scores b=%d" % b)
        ref_idx = O.topk_select(I, m, [p], k)
        near = topk_sets_match(idx[b], ref_idx, I, k)
        assert_topk_exact_on_gpu_scores(idx[b], scores[b], m, [p], k, "cfg4 b=%d" % b)
        kv = K.decode_rows(inp["kv_cache"][b], ROW_FP8, c)
        win = K.decode_rows(inp["kv_win"][b], ROW_FP8, c)
        # a sequence whose selection differs from the oracle's only among near-tied
        # scores is checked with the GPU's own (valid) selection
        use_idx = idx[b] if near else ref_idx
        ref = O.sparse_mqa(decode_act(inp["q"][b]), kv, use_idx, win, int(inp["win_pos0"][b]), nw, [p],
                           inp["sink"].astype(np.float64), scale)
        assert_close(out[b], ref, what="csa decode b=%d" % b)
        hc = K.decode_rows(inp["hca_cache"][b], ROW_FP8, c)
        hw = K.decode_rows(inp["hca_win"][b], ROW_FP8, c)
        ref_h = O.hca_dense(decode_act(inp["q_hca"][b]), hc, mp, hw, int(inp["win_pos0"][b]), nw, [p],
                            inp["sink_hca"].astype(np.float64), scale)
        assert_close(out_h[b], ref_h, what="hca decode b=%d" % b)


def test_cfg4_deterministic_and_batch_invariant(L, cfg4):
    """news page (批不變 + 確定性內核): a B = 16 decode equals 16 single-sequence
    decodes bit for bit, and repeated calls are bitwise equal."""
    a = run_decode(L, cfg4)
    b = run_decode(L, cfg4)
    for key in a:
        assert np.array_equal(host(a[key]), host(b[key])), key
    for s in (0, 7, 15):
        one = run_decode(L, cfg4, [s])
        for key in a:
            assert np.array_equal(host(one[key])[0], host(a[key])[s]), (key, s)


def test_cfg4_two_streams(L, cfg4):
    """The decode step with HCA attention on a second stream (its own
    workspace), forked once the index scores are done, beside the top-k and
    sparse attention on the first: every output equals the one-stream run bit
    for bit, on three repetitions (nothing in the library is shared between
    calls on different streams)."""
    import torch
    ref = run_decode(L, cfg4)
    inp, cfg = cfg4, cfg4["cfg"]
    c, nh, k, nw, m, mp = cfg["c"], cfg["nh"], cfg["k"], cfg["n_win"], cfg["m"], cfg["mp"]
    B, S, Sh = cfg["B"], inp["kv_cache"].shape[1], inp["hca_cache"].shape[1]
    d = {key: dev(inp[key]) for key in ("qI", "wI", "ki_codes", "ki_scales", "q", "kv_cache", "kv_win", "sink", "q_hca",
                                       "hca_cache", "hca_win", "sink_hca")}
    qp, wp = [int(x) for x in inp["q_pos0"]], [int(x) for x in inp["win_pos0"]]
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    scores = torch.empty((B, 1, S), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    tws = torch.empty(max(1, L.topk_workspace_size(B, 1, S, k)), dtype=torch.uint8, device="cuda")
    need = max(1, L.attn_workspace_size(True, B, 1, nh, c, Sh + nw))
    aws, aws2 = (torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(2))
    out, out_h = torch.empty_like(d["q"]), torch.empty_like(d["q_hca"])
    fork, join = torch.cuda.Event(), torch.cuda.Event()
    for rep in range(3):
        out.zero_()
        out_h.zero_()
        L.indexer_score(d["qI"], d["wI"], d["ki_codes"], ROW_MXFP4, m, qp, scores, k_scales=d["ki_scales"])
        fork.record(main)
        side.wait_event(fork)
        L.hca_dense_fwd(d["q_hca"], d["hca_cache"], ROW_FP8, mp, d["hca_win"], wp, nw, qp, d["sink_hca"],
                        1 / math.sqrt(c), out_h, aws2, stream=side)
        L.topk_select(scores, m, qp, k, idx, tws)
        L.sparse_mqa_fwd(d["q"], d["kv_cache"], ROW_FP8, idx, d["kv_win"], wp, nw, qp, d["sink"], 1 / math.sqrt(c), out,
                         aws)
        join.record(side)
        main.wait_event(join)
        torch.cuda.synchronize()
        for key, got in (("scores", scores), ("idx", idx), ("out", out), ("out_h", out_h)):
            assert np.array_equal(host(got), host(ref[key])), (rep, key)


# ---------------------------------------------------------------------- configuration 5

def test_cfg5_layer_pair(L):
    import torch
    from long_context_attention_08_amd.layer import pair_from_arrays
    inp = G.make(5)
    cfg = inp["cfg"]
    n, c, cI, m, mp, k, nw, nl = cfg["n"], cfg["c"], cfg["cI"], cfg["m"], cfg["mp"], cfg["k"], cfg["n_win"], cfg["n_left"]
    P, S0, Sh0 = int(inp["q_pos0"][0]), inp["S0"], inp["Sh0"]
    layer = pair_from_arrays(inp)
    layer.step()
    # the step's one-call index scores + top-k against the two calls through the stored scores, on all 8192 rows
    idx_step = layer.idx.clone()
    layer.indexer()
    layer.topk()
    torch.cuda.synchronize()
    assert torch.equal(idx_step, layer.idx), "indexer_topk differs from indexer_score + topk_select"
    H = decode_act(inp["H"])
    # ---- compressors (in full)
    comp, raw = O.csa_compress(H, decode_act(inp["W_kv"]), inp["B_kv"], m, block0=S0, n_left=nl)
    ki, _ = O.csa_compress(H, decode_act(inp["W_ki"]), inp["B_ki"], m, block0=S0, n_left=nl)
    hca, hraw = O.hca_compress(H[nl:], decode_act(inp["W_hca"]), inp["B_hca"], mp)
    # the step normalises and rotates the KV rows at their positions (gamma 1): entries at their newest
    # pooled token, window rows at their own
    kvn = layer.kv_nr
    prep = lambda x, p: O.kv_norm_rope(x, np.ones(c), p, kvn["eps"], kvn["theta"], kvn["rope_dims"])
    comp = prep(comp, O.entry_positions(m, S0, comp.shape[0]))
    raw = prep(raw, P + np.arange(n))
    hca = prep(hca, P + mp * (np.arange(hca.shape[0]) + 1) - 1)
    hraw = prep(hraw, P + np.arange(n))
    g_comp = K.decode_rows(host(layer.kv_new), ROW_FP8, c)
    g_raw = K.decode_rows(host(layer.kv_win_new), ROW_FP8, c)
    g_ki = K.mxfp4_decode(host(layer.ki_new), host(layer.ki_sc_new))
    g_hca = K.decode_rows(host(layer.hca_new), ROW_FP8, c)
    g_hraw = K.decode_rows(host(layer.hca_win_new), ROW_FP8, c)
    assert_quantized(g_comp, comp, ROW_FP8, what="csa comp")
    assert_quantized(g_raw, raw, ROW_FP8, what="csa window rows")
    assert_quantized(g_ki, ki, ROW_MXFP4, what="indexer keys")
    assert_quantized(g_hca, hca, ROW_FP8, what="hca comp")
    assert_quantized(g_hraw, hraw, ROW_FP8, what="hca window rows")
    # ---- oracle caches: prefilled stored rows ++ the oracle's own new entries
    kv_all = np.concatenate([K.decode_rows(inp["kv_cache"][:S0], ROW_FP8, c), K.round_rows(comp, ROW_FP8)])
    ki_all = np.concatenate([K.mxfp4_decode(inp["ki_codes"][:S0], inp["ki_scales"][:S0]), K.round_rows(ki, ROW_MXFP4)])
    hc_all = np.concatenate([K.decode_rows(inp["hca_cache"][:Sh0], ROW_FP8, c), K.round_rows(hca, ROW_FP8)])
    win_kv = np.concatenate([K.decode_rows(inp["kv_win"][:nw], ROW_FP8, c), K.round_rows(raw, ROW_FP8)])
    win_h = np.concatenate([K.decode_rows(inp["hca_win"][:nw], ROW_FP8, c), K.round_rows(hraw, ROW_FP8)])
    # 64 rows, with the rows where a query's visible HCA count steps (t = 127 mod 128) and the rows after them
    rows = sample_rows(n, m, 64, 5, also=[127, 128, 255, 256, 1023, 1024, 4095, 4096, 8063, 8064, 8191])
    pos = P + rows
    I = O.indexer_score(decode_act(inp["qI"])[rows], inp["wI"][rows].astype(np.float64), ki_all, m, pos)
    g_sc = host(layer.scores[0, rows])
    vis = np.isfinite(I)
    assert np.array_equal(np.isfinite(g_sc), vis)
    assert_close(g_sc[:, :S0], I[:, :S0], tol=2e-5, what="scores over the prefilled cache")
    assert_close(g_sc[vis], I[vis], tol=2e-2, what="scores")
    ref_idx = O.topk_select(I, m, pos, k)
    g_idx = host(layer.idx[0, rows])
    assert_topk_exact_on_gpu_scores(g_idx, g_sc, m, pos, k, "cfg5")
    scale = 1 / math.sqrt(c)
    # the step rotates both outputs' RoPE dims back by the query position in the attention store
    theta, R = layer.out_rope
    rot = lambda o, p: O.out_rope(o, p, theta, R)
    ref = rot(O.sparse_mqa(decode_act(inp["q"])[rows], kv_all, ref_idx, win_kv, P - nw, nw, pos,
                           inp["sink"].astype(np.float64), scale), pos)
    out = decode_act(host(layer.out[rows]))
    ref_fn = lambda sel, ix: rot(O.sparse_mqa(decode_act(inp["q"])[rows[sel]], kv_all, ix, win_kv, P - nw, nw,
                                              pos[sel], inp["sink"].astype(np.float64), scale), pos[sel])
    check_attention_rows(out, ref, rows, g_idx, ref_idx, I, k, fp32=False, ref_with_idx=ref_fn)
    ref_h = rot(O.hca_dense(decode_act(inp["q_hca"])[rows], hc_all, mp, win_h, P - nw, nw, pos,
                            inp["sink_hca"].astype(np.float64), scale), pos)
    assert_close(decode_act(host(layer.out_hca[rows])), ref_h, what="hca output")


def test_cfg5_step_is_bitwise_repeatable(L):
    """Every reduction order in the step is fixed (no floating-point atomics,
    split-K merged in split order, exact integer top-k), so two steps over the
    same chunk give the same bytes in every output: caches, indices and both
    attention outputs."""
    import torch
    from long_context_attention_08_amd.layer import pair_from_arrays
    layer = pair_from_arrays(G.make(5))
    outs = lambda: [t.clone() for t in (layer.kv_new, layer.kv_win_new, layer.ki_new, layer.ki_sc_new, layer.hca_new,
                                        layer.hca_win_new, layer.idx, layer.out, layer.out_hca)]
    layer.step()
    torch.cuda.synchronize()
    first = outs()
    layer.step()
    torch.cuda.synchronize()
    for a, b in zip(first, outs()):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                           b.view(torch.uint8) if b.dtype != torch.uint8 else b)
