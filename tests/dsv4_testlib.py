"""Helpers shared by the tests: device upload of stored arrays, oracle-side
decoding, tolerance checks and the two pipelines (HIP library / oracle).

The oracle pipeline takes only seeded inputs and its own intermediate values;
nothing computed by the HIP library is ever fed to it."""
import math

import numpy as np

import oracle as O
from oracle import codecs as K
from synth.configs import BF16, F32

ROW_F32, ROW_BF16, ROW_FP8, ROW_MXFP4 = 0, 1, 2, 3


# ------------------------------------------------------------------ upload / download

def dev(x):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x).cuda()


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def decode_act(x):
    """stored activation (float32 or bf16 bits) -> float64"""
    return K.bf16_decode(x) if x.dtype == np.uint16 else x.astype(np.float64)


def empty_rows(n, layout, c):
    import torch
    if layout == ROW_F32:
        return torch.zeros((n, c), dtype=torch.float32, device="cuda")
    if layout == ROW_BF16:
        return torch.zeros((n, c), dtype=torch.bfloat16, device="cuda")
    if layout == ROW_FP8:
        return torch.zeros((n, c + 64), dtype=torch.uint8, device="cuda")
    return torch.zeros((n, c // 2), dtype=torch.uint8, device="cuda")


def rows_to_f64(t, layout, c, scales=None):
    x = host(t)
    if layout == ROW_F32:
        return x.astype(np.float64)
    if layout == ROW_BF16:
        return K.bf16_decode(x)
    if layout == ROW_MXFP4:
        return K.mxfp4_decode(x, host(scales))
    return K.decode_rows(x, layout, c)


def stored_rows_f64(x, layout, c, scales=None):
    """numpy stored rows -> float64"""
    if layout == ROW_F32:
        return x.astype(np.float64)
    if layout == ROW_BF16:
        return K.bf16_decode(x)
    if layout == ROW_MXFP4:
        return K.mxfp4_decode(x, scales)
    return K.decode_rows(x, layout, c)


# ------------------------------------------------------------------ tolerance checks

def norm_err(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def assert_close(got, ref, *, fp32=False, tol=None, what=""):
    """fp32 paths: max-abs <= 1e-4; bf16/fp8 paths: ||d||_inf / ||ref||_inf <= 2e-2."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), what + ": non-finite output"
    if fp32:
        err = float(np.max(np.abs(got - ref))) if got.size else 0.0
        assert err <= (tol or 1e-4), "%s: max-abs error %.3g" % (what, err)
    else:
        err = norm_err(got, ref) if got.size else 0.0
        assert err <= (tol or 2e-2), "%s: normalised error %.3g" % (what, err)
    return err


def assert_quantized(got_dec, ref, layout, rel=1e-5, what=""):
    """A stored (rounded) output must be a correct rounding of a value within
    rel * (largest magnitude of its row) of the oracle's float64 value: exact
    except where the oracle value sits on a rounding boundary.  (The HIP side
    accumulates in fp32, so its pre-rounding value carries an absolute error
    of that order, also for small values produced by cancellation.)"""
    ref = np.asarray(ref, dtype=np.float64)
    got_dec = np.asarray(got_dec, dtype=np.float64)
    delta = rel * np.max(np.abs(ref), axis=-1, keepdims=True)
    # rounding is monotone: every value in [ref - delta, ref + delta] rounds
    # into [round(ref - delta), round(ref + delta)]
    lo = K.round_rows(ref - delta, layout)
    hi = K.round_rows(ref + delta, layout)
    ok = (got_dec >= lo) & (got_dec <= hi)
    bad = np.argwhere(~ok)
    if len(bad):
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d stored values are not a rounding of the oracle value; first at %s: "
                             "got %r, oracle %r (row max %r)" % (what, len(bad), ok.size, i, got_dec[i], ref[i],
                                                                 float(np.max(np.abs(ref[i[:-1]])))))


def topk_sets_match(gpu_idx, ref_idx, ref_scores, k, slack=1e-5):
    """Margin-aware comparison of selected sets computed from independently
    rounded scores: a difference is allowed only between entries whose oracle
    scores lie within `slack` (relative) of the k-th score."""
    bad_rows = []
    for t in range(gpu_idx.shape[0]):
        a = set(int(x) for x in gpu_idx[t] if x >= 0)
        b = set(int(x) for x in ref_idx[t] if x >= 0)
        if a == b:
            continue
        kth = ref_scores[t, int(ref_idx[t][min(k, len(b)) - 1])]
        tolv = slack * max(1.0, abs(kth)) * 4
        diff = a ^ b
        if all(abs(ref_scores[t, s] - kth) <= tolv for s in diff):
            bad_rows.append(t)
        else:
            raise AssertionError("row %d: top-k differs beyond the score margin: %s" % (t, sorted(diff)[:10]))
    return bad_rows


# ------------------------------------------------------------------ oracle-side chains

def oracle_csa_layer(inp, rows=None):
    """Oracle CSA layer (cfg1/cfg3 style prefill from position 0).  Returns a
    dict of float64 results; `rows` restricts the per-query steps."""
    cfg = inp["cfg"]
    m, c, cI, k, nw = cfg["m"], cfg["c"], cfg["cI"], cfg["k"], cfg["n_win"]
    H = decode_act(inp["H"])
    comp, raw = O.csa_compress(H, decode_act(inp["W_kv"]), inp["B_kv"], m)
    ki, _ = O.csa_compress(H, decode_act(inp["W_ki"]), inp["B_ki"], m)
    comp_s = K.round_rows(comp, cfg["kv_layout"])
    raw_s = K.round_rows(raw, cfg["kv_layout"])
    ki_s = K.round_rows(ki, cfg["key_layout"])
    n = H.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    qI = decode_act(inp["qI"])[rows]
    wI = inp["wI"].astype(np.float64)[rows]
    I = O.indexer_score(qI, wI, ki_s, m, rows)
    idx = O.topk_select(I, m, rows, k)
    q = decode_act(inp["q"])[rows]
    out = O.sparse_mqa(q, comp_s, idx, raw_s, 0, nw, rows, inp["sink"].astype(np.float64), 1 / math.sqrt(c))
    return dict(comp=comp, raw=raw, ki=ki, comp_s=comp_s, raw_s=raw_s, ki_s=ki_s, scores=I, idx=idx, out=out,
                rows=rows)


def oracle_hca_layer(inp, rows=None):
    cfg = inp["cfg"]
    mp, c, nw = cfg["mp"], cfg["c"], cfg["n_win"]
    H = decode_act(inp["H"])
    comp, raw = O.hca_compress(H, decode_act(inp["W_hca"]), inp["B_hca"], mp)
    comp_s = K.round_rows(comp, cfg["kv_layout"])
    raw_s = K.round_rows(raw, cfg["kv_layout"])
    n = H.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    q = decode_act(inp["q"])[rows]
    out = O.hca_dense(q, comp_s, mp, raw_s, 0, nw, rows, inp["sink"].astype(np.float64), 1 / math.sqrt(c))
    return dict(comp=comp, raw=raw, comp_s=comp_s, raw_s=raw_s, out=out, rows=rows)


# ------------------------------------------------------------------ HIP-side chains

def gpu_csa_layer(L, inp):
    """CSA layer through the C ABI (cfg1/cfg3 style).  Returns torch tensors."""
    import torch
    cfg = inp["cfg"]
    m, c, cI, hI, k, nw, nh = cfg["m"], cfg["c"], cfg["cI"], cfg["hI"], cfg["k"], cfg["n_win"], cfg["nh"]
    n = inp["H"].shape[0]
    S = n // m
    H = dev(inp["H"])
    comp = empty_rows(S, cfg["kv_layout"], c)
    raw = empty_rows(n, cfg["kv_layout"], c)
    L.csa_compress(H, dev(inp["W_kv"]), dev(inp["B_kv"]), m, c, comp, cfg["kv_layout"], raw_out=raw,
                   raw_layout=cfg["kv_layout"])
    ki = empty_rows(S, cfg["key_layout"], cI)
    ki_sc = torch.zeros((S, cI // 32), dtype=torch.uint8, device="cuda") if cfg["key_layout"] == ROW_MXFP4 else None
    L.csa_compress(H, dev(inp["W_ki"]), dev(inp["B_ki"]), m, cI, ki, cfg["key_layout"], comp_scales=ki_sc)
    scores = torch.empty((1, n, S), dtype=torch.float32, device="cuda")
    L.indexer_score(dev(inp["qI"]).view(1, n, hI, cI), dev(inp["wI"]).view(1, n, hI), ki.view(1, S, -1),
                    cfg["key_layout"], m, [0], scores, k_scales=ki_sc)
    idx = torch.empty((1, n, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, L.topk_workspace_size(1, n, S, k)), dtype=torch.uint8, device="cuda")
    L.topk_select(scores, m, [0], k, idx, ws)
    q = dev(inp["q"]).view(1, n, nh, c)
    out = torch.empty_like(q)
    aws = torch.empty(max(1, L.attn_workspace_size(False, 1, n, nh, c, k + nw)), dtype=torch.uint8, device="cuda")
    L.sparse_mqa_fwd(q, comp.view(1, S, -1), cfg["kv_layout"], idx, raw.view(1, n, -1), [0], nw, [0],
                     dev(inp["sink"]), 1 / math.sqrt(c), out, aws)
    return dict(comp=comp, raw=raw, ki=ki, ki_sc=ki_sc, scores=scores, idx=idx, out=out)


def gpu_hca_layer(L, inp):
    import torch
    cfg = inp["cfg"]
    mp, c, nw, nh = cfg["mp"], cfg["c"], cfg["n_win"], cfg["nh"]
    n = inp["H"].shape[0]
    S = n // mp
    H = dev(inp["H"])
    comp = empty_rows(S, cfg["kv_layout"], c)
    raw = empty_rows(n, cfg["kv_layout"], c)
    L.hca_compress(H, dev(inp["W_hca"]), dev(inp["B_hca"]), mp, c, comp, cfg["kv_layout"], raw_out=raw,
                   raw_layout=cfg["kv_layout"])
    q = dev(inp["q"]).view(1, n, nh, c)
    out = torch.empty_like(q)
    aws = torch.empty(max(1, L.attn_workspace_size(True, 1, n, nh, c, S + nw)), dtype=torch.uint8, device="cuda")
    L.hca_dense_fwd(q, comp.view(1, S, -1), cfg["kv_layout"], mp, raw.view(1, n, -1), [0], nw, [0],
                    dev(inp["sink"]), 1 / math.sqrt(c), out, aws)
    return dict(comp=comp, raw=raw, out=out)
