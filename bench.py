"""Benchmark: query tokens/s of the interleaved CSA + HCA layer pair at 1M context.

Workload (one step = every call of the hot path once: the chunk's three
compressors with the KV RMSNorm + RoPE in one call, index scores + top-k in
one call, sparse MQA and HCA dense MQA, each with the output rotation in its
store): an 8192-token chunk
at positions [2^20, 2^20 + 8192) against caches prefilled with 2^20 tokens
(262144 CSA entries, 8192 HCA entries, 128-row SWA tails); bf16 activations,
fp8 + bf16-RoPE KV rows, MXFP4 indexer keys, d = 4096, c = 512, 64 heads,
top-k 1024, window 128.  Inputs are seeded synthetic data resident in HBM
before the timed region.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]

Prints one JSON line.  Per-call durations come from HIP events recorded on the
stream the library launches on; the roofline is reported for the call that
takes the most time, from the algorithmic work of one launch.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "query tokens/s for CSA+HCA layer at 1M ctx; % of HBM/MFMA roofline"
PEAK = {"mfma": 2500.0, "hbm": 8000.0}    # MI355X: dense bf16 TFLOP/s, HBM GB/s
CALLS = ["compress", "indexer_topk", "sparse", "hca_dense"]


def algorithmic_work(cfg, P, S0, Sh0):
    """Algorithmic FLOPs / bytes of each call for one step (visible work only)."""
    n, d, c, m, mp, cI, hI, k, nw, nh = (cfg[x] for x in ("n", "d", "c", "m", "mp", "cI", "hI", "k", "n_win", "nh"))
    t = np.arange(n, dtype=np.int64)
    S = S0 + n // m
    Sh = Sh0 + n // mp
    nvis = np.minimum(S, (P + t + 1) // m)
    nvis_h = np.minimum(Sh, (P + t + 1) // mp)
    row = c + 64                                               # fp8 + bf16-RoPE row bytes
    w = {}
    w["csa_compress"] = dict(flop=2.0 * (n + cfg["n_left"]) * d * (4 * c + 4 * cI), bound="mfma")
    w["indexer"] = dict(flop=2.0 * float(nvis.sum()) * hI * cI, bound="mfma",
                        bytes=float(n) * S * 4 + S * (cI // 2 + cI // 32) + n * hI * (2 * cI + 4))
    w["topk"] = dict(bytes=float(nvis.sum()) * 4 + n * k * 4, bound="hbm")
    # index scores + top-k in one call: the index-score contraction (the score
    # rows never reach HBM; the strided sample pass is overhead, not counted)
    w["indexer_topk"] = dict(flop=w["indexer"]["flop"], bound="mfma",
                             bytes=S * (cI // 2 + cI // 32) + n * hI * (2 * cI + 4) + n * k * 4)
    keys_sparse = float(n) * (k + nw)
    w["sparse"] = dict(flop=4.0 * keys_sparse * nh * c, bound="mfma",
                       bytes=2.0 * n * nh * c * 2 + S * row + n * k * 4)
    w["hca_compress"] = dict(flop=2.0 * n * d * 2 * c, bound="mfma")
    # the three compressors in one launch (dsv4_compress_chunk)
    w["compress"] = dict(flop=w["csa_compress"]["flop"] + w["hca_compress"]["flop"], bound="mfma")
    keys_dense = float((nvis_h + nw).sum())
    w["hca_dense"] = dict(flop=4.0 * keys_dense * nh * c, bound="mfma", bytes=2.0 * n * nh * c * 2 + Sh * row)
    return w


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hca_dense_traffic.json")


def source_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_attention_08_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter record, or
    None when there is none or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel") != kernel or rec.get("source_sha256") != source_digest(rec.get("sources", [])):
        return None
    return rec.get("hbm_bytes_per_launch")


def calibrate_copy(gib=1):
    """A plain device-to-device copy of a known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters (each launch moves `gib` GiB each way)."""
    import torch
    n = gib * (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 3}), flush=True)


def cpu_baseline(inp, rows_n=256, seed=4):
    """The float64 oracle on a bounded sample: the three compressors with the
    KV norm + RoPE in full, then the per-query steps (index scores, top-k,
    sparse MQA, dense MQA, each output rotated back) for `rows_n` seeded query
    rows.  Returns query tokens/s with the compress cost amortised over the
    chunk."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle as O
    from oracle import codecs as K
    cfg = inp["cfg"]
    n, c, m, mp, k, nw, nl = (cfg[x] for x in ("n", "c", "m", "mp", "k", "n_win", "n_left"))
    P, S0, Sh0 = int(inp["q_pos0"][0]), inp["S0"], inp["Sh0"]
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        dec = lambda x: K.bf16_decode(x)
        H = dec(inp["H"])
        t0 = time.perf_counter()
        comp, raw = O.csa_compress(H, dec(inp["W_kv"]), inp["B_kv"], m, block0=S0, n_left=nl)
        ki, _ = O.csa_compress(H, dec(inp["W_ki"]), inp["B_ki"], m, block0=S0, n_left=nl)
        hca, hraw = O.hca_compress(H[nl:], dec(inp["W_hca"]), inp["B_hca"], mp)
        prep = lambda x, p: O.kv_norm_rope(x, np.ones(c), p, 1e-6, 10000.0, 64)
        comp, raw = prep(comp, O.entry_positions(m, S0, comp.shape[0])), prep(raw, P + np.arange(n))
        hca, hraw = prep(hca, P + mp * (np.arange(hca.shape[0]) + 1) - 1), prep(hraw, P + np.arange(n))
        t_comp = time.perf_counter() - t0
        kv_all = np.concatenate([K.decode_rows(inp["kv_cache"][:S0], 2, c), K.round_rows(comp, 2)])
        ki_all = np.concatenate([K.mxfp4_decode(inp["ki_codes"][:S0], inp["ki_scales"][:S0]), K.round_rows(ki, 3)])
        hc_all = np.concatenate([K.decode_rows(inp["hca_cache"][:Sh0], 2, c), K.round_rows(hca, 2)])
        wk = np.concatenate([K.decode_rows(inp["kv_win"][:nw], 2, c), K.round_rows(raw, 2)])
        wh = np.concatenate([K.decode_rows(inp["hca_win"][:nw], 2, c), K.round_rows(hraw, 2)])
        rows = np.sort(np.random.default_rng(seed).choice(n, size=rows_n, replace=False))
        pos = P + rows
        qI, wI = dec(inp["qI"])[rows], inp["wI"][rows].astype(np.float64)
        q, qh = dec(inp["q"])[rows], dec(inp["q_hca"])[rows]
        t0 = time.perf_counter()
        I = O.indexer_score(qI, wI, ki_all, m, pos)
        idx = O.topk_select(I, m, pos, k)
        O.out_rope(O.sparse_mqa(q, kv_all, idx, wk, P - nw, nw, pos, inp["sink"].astype(np.float64),
                                1 / math.sqrt(c)), pos)
        O.out_rope(O.hca_dense(qh, hc_all, mp, wh, P - nw, nw, pos, inp["sink_hca"].astype(np.float64),
                               1 / math.sqrt(c)), pos)
        t_rows = time.perf_counter() - t0
    per_token = t_comp / n + t_rows / rows_n
    return {"value": 1.0 / per_token, "unit": "query tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": "float64 numpy oracle: the three compressors over the full 8192-token chunk (%.1f s, "
                      "amortised per token) + index scores, top-k, sparse and dense MQA for %d seeded query "
                      "rows (%.1f s); host cores available %d" % (t_comp, rows_n, t_rows, cores)}


def quantised_indexer_report(layer, fmt, flop, steps, stream, rows_n=256):
    """Time the FP4- (fmt 4) or FP8-query (fmt 8) indexer on the same chunk and
    measure the recall of its top-k against the bf16-query top-k on rows_n
    evenly spaced rows."""
    import torch
    call = layer.indexer_fp8q if fmt == 8 else layer.indexer_fp4q
    layer.indexer()
    layer.topk()
    torch.cuda.synchronize()
    ref = layer.idx[0].cpu().numpy()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    call()
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    layer.topk()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    got = layer.idx[0].cpu().numpy()
    rows = np.linspace(0, ref.shape[0] - 1, rows_n).astype(np.int64)
    rec = []
    for r in rows:
        a, b = set(ref[r][ref[r] >= 0].tolist()), set(got[r][got[r] >= 0].tolist())
        if a:
            rec.append(len(a & b) / len(a))
    layer.indexer()          # leave the bf16 scores in place
    torch.cuda.synchronize()
    return {"ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
            "recall_at_k_vs_bf16_query": round(float(np.mean(rec)), 4), "recall_rows": len(rec)}


def two_call_report(layer, work, steps, stream):
    """The same selection as two calls through the stored [n, S] score rows
    (indexer_score, then topk_select), timed alone, against the one-call
    index scores + top-k of the step; checks that both give the same indices."""
    import torch
    layer.indexer_topk()
    torch.cuda.synchronize()
    one = layer.idx.clone()
    ms = _time_calls([("indexer", layer.indexer), ("topk", layer.topk), ("indexer_topk", layer.indexer_topk)],
                     steps, stream)
    layer.indexer()
    layer.topk()
    torch.cuda.synchronize()
    same = bool(torch.equal(one, layer.idx))
    fi = work["indexer"]["flop"]
    return {"indexer_ms": round(ms["indexer"], 4), "topk_ms": round(ms["topk"], 4),
            "two_calls_ms": round(ms["indexer"] + ms["topk"], 4), "one_call_ms": round(ms["indexer_topk"], 4),
            "saved_ms": round(ms["indexer"] + ms["topk"] - ms["indexer_topk"], 4),
            "indexer_tflops": round(fi / (ms["indexer"] * 1e-3) / 1e12, 2),
            "topk_gbps": round(work["topk"]["bytes"] / (ms["topk"] * 1e-3) / 1e9, 1),
            "identical_indices": same}


def norm_rope_report(layer, steps, stream):
    """Time the Q/KV RMSNorm + partial RoPE and the output rotation at the
    chunk's shapes (outside the step: the six calls take their inputs already
    normalised and rotated): every query head, the chunk's new compressed
    entries and window rows, every output row."""
    import torch
    from long_context_attention_08_amd import _lib as L
    n, nh, c = layer.n, layer.nh, layer.c
    q = layer.q.view(1, n, nh, c)
    qo = torch.empty_like(q)
    o = layer.out.view(1, n, nh, c).clone()
    g = torch.ones(c, dtype=torch.float32, device="cuda")
    ncomp = n // layer.m
    comp_in = torch.randn((1, ncomp, c), dtype=torch.float32, device="cuda")
    comp_out = torch.empty((1, ncomp, c + 64), dtype=torch.uint8, device="cuda")
    win_in = torch.randn((1, n, c), dtype=torch.bfloat16, device="cuda")
    win_out = torch.empty((1, n, c + 64), dtype=torch.uint8, device="cuda")
    p0 = layer.q_pos0
    calls = {
        "q_norm_rope": (lambda: L.q_norm_rope(q, g, p0, out=qo), 2 * q.numel() * 2),
        "out_rope": (lambda: L.out_rope(o, p0), 2 * n * nh * 64 * 2),
        "kv_norm_rope (entries + window rows)": (
            lambda: (L.kv_norm_rope(comp_in, L.ROW_F32, c, g, [layer.m * (layer.S0 + 1) - 1], layer.m, comp_out,
                                    L.ROW_FP8_ROPE_BF16),
                     L.kv_norm_rope(win_in, L.ROW_BF16, c, g, p0, 1, win_out, L.ROW_FP8_ROPE_BF16)),
            ncomp * (4 * c + c + 64) + n * (2 * c + c + 64)),
    }
    rep = {}
    for name, (f, nbytes) in calls.items():
        f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        rep[name] = {"ms": round(ms, 4), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK["hbm"], 4)}
    return rep


def projections_report(steps, stream, n=8192, d=4096, d_c=1024, nh=64, c=512, hI=32, cI=64, g=8, d_g=1024):
    """Time the low-rank query path and the grouped output projection on the
    bf16 GEMM at the chunk's shapes (weights N(0, 1/fan_in), synthetic)."""
    import torch
    from long_context_attention_08_amd import _lib as L
    bf = torch.bfloat16
    r = lambda *sh: (torch.randn(sh, device="cuda") * sh[-1] ** -0.5).to(bf)
    h = torch.randn((n, d), device="cuda").to(bf)
    W_DQ, W_UQ, W_IUQ, W_w = r(d_c, d), r(nh * c, d_c), r(hI * cI, d_c), r(hI, d)
    q = torch.empty((n, nh, c), dtype=bf, device="cuda")
    qI = torch.empty((n, hI, cI), dtype=bf, device="cuda")
    wI = torch.empty((n, hI), dtype=torch.float32, device="cuda")
    wsq = torch.empty(L.query_proj_workspace_size(n, d_c), dtype=torch.uint8, device="cuda")
    o = torch.randn((n, nh, c), device="cuda").to(bf)
    W1, W2 = r(g, d_g, nh // g * c), r(d, g * d_g)
    out = torch.empty((n, d), dtype=bf, device="cuda")
    wso = torch.empty(L.output_proj_workspace_size(n, g, d_g), dtype=torch.uint8, device="cuda")
    fq = 2.0 * n * (d * d_c + d_c * nh * c + d_c * hI * cI + d * hI)
    fo = 2.0 * n * (nh * c * d_g + g * d_g * d)
    calls = {"query_proj": (lambda: L.query_proj(h, W_DQ, W_UQ, W_IUQ, W_w, nh=nh, c=c, hI=hI, cI=cI, q=q, qI=qI,
                                                 wI=wI, ws=wsq), fq),
             "output_proj": (lambda: L.output_proj(o, W1, W2, out, g=g, ws=wso), fo)}
    rep = {}
    for name, (f, flop) in calls.items():
        f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        rep[name] = {"ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
                     "frac_mfma": round(flop / (ms * 1e-3) / 1e12 / PEAK["mfma"], 4)}
    return rep


def decode_cache_report(steps, stream, B=16, d=4096, c=512, cI=64, m=4, mp=128, ring_w=128):
    """Time the decode-time cache maintenance of one token for each of B
    sequences at position 2^20 + 127, which completes a CSA block and an HCA
    block, so every compressor pools: the CSA KV compressor and the HCA
    compressor (RMSNorm + partial RoPE, FP8 + bf16-RoPE rows, window rings of
    2 x 128 rows) and the indexer-key compressor (MXFP4 rows).  The states are
    first fed the earlier tokens of the blocks.  Algorithmic bytes: the weights
    and hidden rows read once, the per-channel softmax accumulators of the
    state read and written, the ring and cache rows written."""
    import torch
    from long_context_attention_08_amd import _lib as L
    bf = torch.bfloat16
    p = (1 << 20) + 127
    r = lambda *sh: (torch.randn(sh, device="cuda") * sh[-1] ** -0.5).to(bf)
    H = torch.randn((B, 1, d), device="cuda").to(bf)
    g = torch.ones(c, dtype=torch.float32, device="cuda")
    rb = c + 64
    comps = {
        # name: (overlap, m, width, layout, norm + rope, ring)
        "csa_kv": (1, m, c, L.ROW_FP8_ROPE_BF16, True, True),
        "indexer_keys": (1, m, cI, L.ROW_MXFP4, False, False),
        "hca": (0, mp, c, L.ROW_FP8_ROPE_BF16, True, True),
    }
    rep = {}
    total_ms, total_bytes = 0.0, 0
    for name, (ov, mm, cw, lay, nr, use_ring) in comps.items():
        nmat = 4 if ov else 2
        W = r(nmat * cw, d)
        bias = torch.randn((2, mm, cw) if ov else (mm, cw), device="cuda") * 0.5
        st = torch.zeros(B * L.stream_state_bytes(ov, mm, cw), dtype=torch.uint8, device="cuda")
        L.stream_state_reset(st, B, ov, mm, cw)
        S = (p + 1) // mm
        row = L.row_bytes(lay, cw)
        cache = torch.empty((B, S, row), dtype=torch.uint8, device="cuda")
        scales = torch.empty((B, S, cw // 32), dtype=torch.uint8, device="cuda") if lay == L.ROW_MXFP4 else None
        ring = torch.empty((B, 2 * ring_w, rb), dtype=torch.uint8, device="cuda") if use_ring else None
        kw = dict(cache=cache, cache_scales=scales, cache_layout=lay, ring=ring, ring_w=ring_w if use_ring else 0,
                  ring_layout=lay if use_ring else L.ROW_F32, norm=nr, gamma=g[:cw] if nr else None,
                  rope_dims=64 if nr else 0)
        first = p - (2 * mm - 1 if ov else mm - 1)      # the rows the entry pools
        Hp = torch.randn((B, p - first, d), device="cuda").to(bf)
        L.stream_compress(Hp, W, bias, ov, mm, cw, [first] * B, st, **kw)
        ws = torch.empty(max(16, L.stream_workspace_size(B, 1, d, ov, cw)), dtype=torch.uint8, device="cuda")
        f = lambda: L.stream_compress(H, W, bias, ov, mm, cw, [p] * B, st, ws=ws, **kw)
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        nbytes = W.numel() * 2 + B * (d * 2 + 2 * L.stream_state_bytes(ov, mm, cw) + row +
                                      (2 * row if use_ring else 0))
        rep[name] = {"us": round(ms * 1e3, 2), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK["hbm"], 4), "bytes": int(nbytes)}
        total_ms += ms
        total_bytes += nbytes
        del cache, scales, ring, st, W, Hp
    rep["all_three"] = {"us": round(total_ms * 1e3, 2),
                        "frac_hbm": round(total_bytes / (total_ms * 1e-3) / 1e9 / PEAK["hbm"], 4)}
    rep["shape"] = {"sequences": B, "position": p, "d": d, "c": c, "c_I": cI, "m": m, "m_prime": mp}
    return rep


def neighbour_overlap(idx, k):
    """How many selected entries consecutive queries of the chunk share (the
    fraction of query t + 1's k entries also selected by query t, averaged):
    what a sparse-attention block serving several neighbouring queries over
    the union of their index lists could save in gathered rows."""
    import torch
    s = idx.sort(dim=-1).values
    a, b = s[:-1].contiguous(), s[1:].contiguous()
    pos = torch.searchsorted(a, b).clamp(max=a.shape[1] - 1)
    shared = ((a.gather(1, pos) == b) & (b >= 0)).sum(dim=1).float() / k
    return {"shared_fraction_mean": round(float(shared.mean()), 4), "shared_fraction_max": round(float(shared.max()), 4),
            "union_of_two_over_k": round(float(2.0 - shared.mean()), 4)}


def _time_calls(calls, steps, stream):
    """Average ms of each callable over `steps` back-to-back launches (HIP
    events on the library's stream), after one untimed call each."""
    import torch
    out = {}
    for name, f in calls:
        f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) / steps
    return out


def _dev(x):
    """numpy array -> device tensor; uint16 arrays hold bf16 bit patterns"""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t.view(torch.bfloat16) if x.dtype == np.uint16 else t


def decode_report(steps, stream):
    """One decode step of configuration 4 (16 sequences, one query each at
    position 2^20, caches of 2^20 tokens): the indexer over 262144 MXFP4 keys,
    top-k 1024, sparse MQA over 1024 FP8 + bf16-RoPE entries plus the 128-row
    window, and HCA dense attention over 8192 entries plus the window, each
    timed alone, and index scores + top-k as one call; then the step back to
    back with the faster of the two selection paths.  Algorithmic bytes:
    inputs read once, outputs written once (the gathered rows of the selected
    entries for sparse MQA; no score rows for the one-call path)."""
    from long_context_attention_08_amd import _lib as L
    from synth import gen as G
    import torch
    inp = G.make(4)
    cfg = inp["cfg"]
    B, c, nh, hI, cI, k, nw, m, mp = (cfg[x] for x in ("B", "c", "nh", "hI", "cI", "k", "n_win", "m", "mp"))
    S, Sh = inp["kv_cache"].shape[1], inp["hca_cache"].shape[1]
    qp, wp = [int(x) for x in inp["q_pos0"]], [int(x) for x in inp["win_pos0"]]
    d = {key: _dev(inp[key]) for key in ("q", "qI", "wI", "q_hca", "sink", "sink_hca", "kv_cache", "ki_codes",
                                         "ki_scales", "hca_cache", "kv_win", "hca_win")}
    del inp
    scores = torch.empty((B, 1, S), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    tws = torch.empty(max(1, L.topk_workspace_size(B, 1, S, k)), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["q"])
    out_h = torch.empty_like(d["q_hca"])
    need_s = L.attn_plan(False, L.BF16, L.ROW_FP8_ROPE_BF16, B, 1, nh, c, S, k, 1, nw, qp)
    need_h = L.attn_plan(True, L.BF16, L.ROW_FP8_ROPE_BF16, B, 1, nh, c, Sh, 0, mp, nw, qp)
    aws = torch.empty(max(1, need_s.workspace_bytes, need_h.workspace_bytes), dtype=torch.uint8, device="cuda")
    scale = 1 / math.sqrt(c)
    f_idx = lambda: L.indexer_score(d["qI"], d["wI"], d["ki_codes"], L.ROW_MXFP4, m, qp, scores, k_scales=d["ki_scales"])
    f_topk = lambda: L.topk_select(scores, m, qp, k, idx, tws)
    itws = torch.empty(max(1, L.indexer_topk_workspace_size(L.BF16, L.ROW_MXFP4, B, 1, hI, cI, S, k)),
                       dtype=torch.uint8, device="cuda")
    f_it = lambda: L.indexer_topk(d["qI"], d["wI"], d["ki_codes"], L.ROW_MXFP4, m, qp, k, idx, itws,
                                  k_scales=d["ki_scales"])
    f_sparse = lambda: L.sparse_mqa_fwd(d["q"], d["kv_cache"], L.ROW_FP8_ROPE_BF16, idx, d["kv_win"], wp, nw, qp,
                                        d["sink"], scale, out, aws)
    f_hca = lambda: L.hca_dense_fwd(d["q_hca"], d["hca_cache"], L.ROW_FP8_ROPE_BF16, mp, d["hca_win"], wp, nw, qp,
                                    d["sink_hca"], scale, out_h, aws)
    f_idx()
    f_topk()
    torch.cuda.synchronize()
    row = c + 64
    qb = B * nh * c * 2
    work = {
        "indexer": B * S * (cI // 2 + cI // 32) + B * hI * (cI * 2 + 4) + B * S * 4,
        "topk": B * S * 4 + B * k * 4,
        "sparse": B * (k + nw) * row + 2 * qb + B * k * 4,
        "hca_dense": B * (Sh + nw) * row + 2 * qb,
    }
    work["indexer_topk"] = work["indexer"] - B * S * 4 + B * k * 4
    ms = _time_calls([("indexer", f_idx), ("topk", f_topk), ("indexer_topk", f_it), ("sparse", f_sparse),
                      ("hca_dense", f_hca)], steps, stream)
    # the step takes whichever selection path makes it faster (the two give the same indices)
    one_stream = {True: lambda: (f_it(), f_sparse(), f_hca()),
                  False: lambda: (f_idx(), f_topk(), f_sparse(), f_hca())}
    # HCA attention needs nothing the selection or the sparse call produce: on a second stream (its own
    # workspace) it runs beside them.  At one query per sequence only the index-score pass fills the GPU
    # (2048 blocks); the top-k and the sparse call are a few blocks per sequence, so the HCA launch goes
    # out when the index scores are done (with the one-call selection, at the start)
    side = torch.cuda.Stream()
    aws2 = torch.empty_like(aws)
    ev_in, ev_out = torch.cuda.Event(), torch.cuda.Event()
    f_hca_side = lambda: L.hca_dense_fwd(d["q_hca"], d["hca_cache"], L.ROW_FP8_ROPE_BF16, mp, d["hca_win"], wp, nw,
                                         qp, d["sink_hca"], scale, out_h, aws2, stream=side)

    def fork():
        ev_in.record(stream)
        side.wait_event(ev_in)
        f_hca_side()

    def two_streams(one_call):
        def step():
            if one_call:
                fork()
                f_it()
            else:
                f_idx()
                fork()
                f_topk()
            f_sparse()
            ev_out.record(side)
            stream.wait_event(ev_out)
        return step
    t2 = _time_calls([("one", two_streams(True)), ("two", two_streams(False))], steps, stream)
    one_call = t2["one"] < t2["two"]
    ms["step"] = t2["one" if one_call else "two"]
    ms["step_serial"] = _time_calls([("step", one_stream[one_call])], steps, stream)["step"]
    # the two-stream step's outputs are those of the one-stream step, bit for bit
    one_stream[one_call]()
    torch.cuda.synchronize()
    ref_o, ref_h = out.clone(), out_h.clone()
    out.zero_()
    out_h.zero_()
    two_streams(one_call)()
    torch.cuda.synchronize()
    same = bool(torch.equal(out.view(torch.int16), ref_o.view(torch.int16)) and
                torch.equal(out_h.view(torch.int16), ref_h.view(torch.int16)))
    rep = {}
    for name in ("indexer", "topk", "indexer_topk", "sparse", "hca_dense"):
        gbps = work[name] / (ms[name] * 1e-3) / 1e9
        rep[name] = {"us": round(ms[name] * 1e3, 2), "gbps": round(gbps, 1), "frac_hbm": round(gbps / PEAK["hbm"], 4),
                     "bytes": int(work[name])}
    rep["sparse"]["plan"] = {"splits": need_s.splits, "split_slots": need_s.split_slots}
    rep["hca_dense"]["plan"] = {"splits": need_h.splits, "split_slots": need_h.split_slots}
    sel = ["indexer_topk"] if one_call else ["indexer", "topk"]
    tot = sum(work[x] for x in sel + ["sparse", "hca_dense"])
    rep["step"] = {"us": round(ms["step"] * 1e3, 2), "query_tokens_per_s": round(B / (ms["step"] * 1e-3), 1),
                   "frac_hbm": round(tot / (ms["step"] * 1e-3) / 1e9 / PEAK["hbm"], 4), "bytes": int(tot),
                   "calls": sel + ["sparse", "hca_dense"], "hca_dense_stream": "second",
                   "one_stream_us": round(ms["step_serial"] * 1e3, 2), "outputs_equal_one_stream": same}
    rep["shape"] = {"sequences": B, "position": qp[0], "csa_entries": S, "hca_entries": Sh, "top_k": k,
                    "window": nw, "heads": nh, "c": c}
    return rep


def prefill_configs_report(steps, stream):
    """Configurations 2 (HCA layer, bf16, n = 32768, c = 128, 16 heads) and 3
    (CSA prefill, bf16, n = 65536, c = 128, 64 heads, top-k 512): each call
    timed alone on the configuration's own seeded inputs, with its binding
    roofline (HBM for configuration 2 and the top-k, MFMA for the indexer,
    the compressors and the sparse core of configuration 3)."""
    from long_context_attention_08_amd import _lib as L
    from synth import gen as G
    import torch
    rep = {}
    # ---- configuration 2
    inp = G.make(2)
    cfg = inp["cfg"]
    n, d, c, nh, mp, nw = (cfg[x] for x in ("n", "d", "c", "nh", "mp", "n_win"))
    S = n // mp
    H, W, Bb, q, sink = (_dev(inp[x]) for x in ("H", "W_hca", "B_hca", "q", "sink"))
    del inp
    rb = c * 2
    comp = torch.empty((S, rb), dtype=torch.uint8, device="cuda")
    raw = torch.empty((n, rb), dtype=torch.uint8, device="cuda")
    qv = q.view(1, n, nh, c)
    out = torch.empty_like(qv)
    need = L.attn_plan(True, L.BF16, L.ROW_BF16, 1, n, nh, c, S, 0, mp, nw, [0]).workspace_bytes
    ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")
    f_c = lambda: L.hca_compress(H, W, Bb, mp, c, comp, L.ROW_BF16, raw_out=raw, raw_layout=L.ROW_BF16)
    f_a = lambda: L.hca_dense_fwd(qv, comp.view(1, S, -1), L.ROW_BF16, mp, raw.view(1, n, -1), [0], nw, [0], sink,
                                  1 / math.sqrt(c), out, ws)
    f_c()
    torch.cuda.synchronize()
    ms = _time_calls([("hca_compress", f_c), ("hca_dense", f_a)], steps, stream)
    t = np.arange(n)
    keys = float((np.minimum(S, (t + 1) // mp) + np.minimum(nw, t + 1)).sum())
    work = {"hca_compress": (n * d * 2 + 2 * c * d * 2 + S * rb + n * rb, 2.0 * n * d * 2 * c),
            "hca_dense": (2 * n * nh * c * 2 + (S + n) * rb, 4.0 * keys * nh * c)}
    r2 = {}
    for name, (nbytes, flop) in work.items():
        t_s = ms[name] * 1e-3
        r2[name] = {"us": round(ms[name] * 1e3, 2), "gbps": round(nbytes / t_s / 1e9, 1),
                    "tflops": round(flop / t_s / 1e12, 2), "frac_hbm": round(nbytes / t_s / 1e9 / PEAK["hbm"], 4)}
    tot_ms = ms["hca_compress"] + ms["hca_dense"]
    r2["layer"] = {"us": round(tot_ms * 1e3, 2), "query_tokens_per_s": round(n / (tot_ms * 1e-3), 1),
                   "frac_hbm": round(sum(v[0] for v in work.values()) / (tot_ms * 1e-3) / 1e9 / PEAK["hbm"], 4)}
    rep["hca_bf16_n32768"] = r2
    del H, W, Bb, q, sink, comp, raw, out, ws
    # ---- configuration 3
    inp = G.make(3)
    cfg = inp["cfg"]
    n, d, c, nh, m, cI, hI, k, nw = (cfg[x] for x in ("n", "d", "c", "nh", "m", "cI", "hI", "k", "n_win"))
    S = n // m
    H, Wkv, Bkv, Wki, Bki, q, qI, wI, sink = (_dev(inp[x]) for x in ("H", "W_kv", "B_kv", "W_ki", "B_ki", "q", "qI",
                                                                    "wI", "sink"))
    del inp
    rb = c * 2
    comp = torch.empty((S, rb), dtype=torch.uint8, device="cuda")
    raw = torch.empty((n, rb), dtype=torch.uint8, device="cuda")
    ki = torch.empty((S, cI * 2), dtype=torch.uint8, device="cuda")
    scores = torch.empty((1, n, S), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, n, k), dtype=torch.int32, device="cuda")
    tws = torch.empty(max(1, L.topk_workspace_size(1, n, S, k)), dtype=torch.uint8, device="cuda")
    qv = q.view(1, n, nh, c)
    out = torch.empty_like(qv)
    need = L.attn_plan(False, L.BF16, L.ROW_BF16, 1, n, nh, c, S, k, 1, nw, [0]).workspace_bytes
    ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")
    kvc = L.compressor(Wkv, Bkv, c, comp, L.ROW_BF16, raw_out=raw, raw_layout=L.ROW_BF16)
    kic = L.compressor(Wki, Bki, cI, ki, L.ROW_BF16)
    f_c = lambda: L.compress_chunk(H, m, csa_kv=kvc, csa_keys=kic)
    f_i = lambda: L.indexer_score(qI.view(1, n, hI, cI), wI.view(1, n, hI), ki.view(1, S, -1), L.ROW_BF16, m, [0],
                                  scores)
    f_t = lambda: L.topk_select(scores, m, [0], k, idx, tws)
    itws = torch.empty(max(1, L.indexer_topk_workspace_size(L.BF16, L.ROW_BF16, 1, n, hI, cI, S, k)),
                       dtype=torch.uint8, device="cuda")
    f_it = lambda: L.indexer_topk(qI.view(1, n, hI, cI), wI.view(1, n, hI), ki.view(1, S, -1), L.ROW_BF16, m, [0], k,
                                  idx, itws)
    f_s = lambda: L.sparse_mqa_fwd(qv, comp.view(1, S, -1), L.ROW_BF16, idx, raw.view(1, n, -1), [0], nw, [0], sink,
                                   1 / math.sqrt(c), out, ws)
    f_c()
    f_i()
    f_t()
    torch.cuda.synchronize()
    ms = _time_calls([("compress", f_c), ("indexer", f_i), ("topk", f_t), ("indexer_topk", f_it), ("sparse", f_s)],
                     steps, stream)
    t = np.arange(n)
    nvis = np.minimum(S, (t + 1) // m)
    work = {"compress": (n * d * 2, 2.0 * n * d * (4 * c + 4 * cI), "mfma"),
            "indexer": (float(n) * S * 4 + S * cI * 2, 2.0 * float(nvis.sum()) * hI * cI, "mfma"),
            "topk": (float(nvis.sum()) * 4 + n * k * 4, 0.0, "hbm"),
            "indexer_topk": (float(S) * cI * 2 + n * k * 4, 2.0 * float(nvis.sum()) * hI * cI, "mfma"),
            "sparse": (2.0 * n * nh * c * 2 + (S + n) * rb + n * k * 4,
                       4.0 * float((np.minimum(k, nvis) + np.minimum(nw, t + 1)).sum()) * nh * c, "mfma")}
    r3 = {}
    for name, (nbytes, flop, bound) in work.items():
        t_s = ms[name] * 1e-3
        e = {"us": round(ms[name] * 1e3, 2), "gbps": round(nbytes / t_s / 1e9, 1)}
        if flop:
            e["tflops"] = round(flop / t_s / 1e12, 2)
        e["frac_" + bound] = round((flop / t_s / 1e12 / PEAK["mfma"]) if bound == "mfma" else
                                   (nbytes / t_s / 1e9 / PEAK["hbm"]), 4)
        r3[name] = e
    # the layer: compress, the faster selection path, sparse
    sel = min(ms["indexer_topk"], ms["indexer"] + ms["topk"])
    tot_ms = ms["compress"] + sel + ms["sparse"]
    r3["layer"] = {"us": round(tot_ms * 1e3, 2), "query_tokens_per_s": round(n / (tot_ms * 1e-3), 1),
                   "selection": "indexer_topk" if ms["indexer_topk"] <= ms["indexer"] + ms["topk"] else
                                "indexer + topk"}
    rep["csa_prefill_bf16_n65536"] = r3
    return rep


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=256)   # about 10 s of oracle work on 16 cores
    ap.add_argument("--step-only", action="store_true",
                    help="time the layer-pair step only (no side reports, no CPU baseline): for profiler runs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode step of configuration 4 (16 sequences at 2^20), as the `decode` field")
    ap.add_argument("--prefill-configs-only", action="store_true",
                    help="only configurations 2 and 3 (c = 128 bf16 layers), as the `prefill_configs` field")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print("bench.py: the library runs on one GPU; --gpus %d is not supported (multi-GPU sharding is a "
              "design note only)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_attention_08_amd.layer import pair_from_arrays
    from synth import gen as G

    if args.decode_only:
        stream = torch.cuda.current_stream()
        print(json.dumps({"decode": decode_report(args.steps, stream)}), flush=True)
        return
    if args.prefill_configs_only:
        stream = torch.cuda.current_stream()
        print(json.dumps({"prefill_configs": prefill_configs_report(args.steps, stream)}), flush=True)
        return

    inp = G.make(5)
    cfg = inp["cfg"]
    layer = pair_from_arrays(inp)
    stream = torch.cuda.current_stream()
    fns = [layer.compress, layer.indexer_topk, layer.sparse, layer.hca_dense]
    for _ in range(args.warmup):
        layer.step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for i, f in enumerate(fns):
            f()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = {name: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]))
                for i, name in enumerate(CALLS)}
    ms_step = wall * 1e3 / args.steps
    value = cfg["n"] * args.steps / wall

    work = algorithmic_work(cfg, int(inp["q_pos0"][0]), inp["S0"], inp["Sh0"])
    calls = {}
    for name in CALLS:
        w, t = work[name], per_call[name] * 1e-3
        ent = {"ms": round(per_call[name], 4)}
        if "flop" in w:
            ent["tflops"] = round(w["flop"] / t / 1e12, 2)
        if "bytes" in w:
            ent["gbps"] = round(w["bytes"] / t / 1e9, 1)
        b = w["bound"]
        ach = w["flop"] / t / 1e12 if b == "mfma" else w["bytes"] / t / 1e9
        ent["frac_" + b] = round(ach / PEAK[b], 4)
        calls[name] = ent
    dom = max(CALLS, key=lambda x: per_call[x])
    w = work[dom]
    b = w["bound"]
    ach = (w["flop"] / (per_call[dom] * 1e-3) / 1e12) if b == "mfma" else (w["bytes"] / (per_call[dom] * 1e-3) / 1e9)
    roof = {"kernel": dom, "bound": b, "achieved": round(ach, 2), "peak": PEAK[b],
            "unit": "TFLOP/s" if b == "mfma" else "GB/s", "frac": round(ach / PEAK[b], 4),
            "traffic": measured_traffic(dom),
            "work_per_launch": w.get("flop") if b == "mfma" else w.get("bytes")}

    line = {"metric": METRIC, "value": round(value, 1), "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": cfg["name"], "chunk_tokens": cfg["n"], "context": cfg["ctx"], "d": cfg["d"],
                       "c": cfg["c"], "heads": cfg["nh"], "m": cfg["m"], "m_prime": cfg["mp"], "top_k": cfg["k"],
                       "window": cfg["n_win"], "kv": "fp8_e4m3+bf16_rope", "indexer_keys": "mxfp4"},
            "roofline": roof, "calls": calls}
    if args.step_only:
        print(json.dumps(line), flush=True)
        return
    line["sparse_neighbours"] = neighbour_overlap(layer.idx[0], cfg["k"])
    line["indexer_then_topk"] = two_call_report(layer, work, args.steps, stream)
    line["fp4_indexer"] = quantised_indexer_report(layer, 4, work["indexer"]["flop"], args.steps, stream)
    line["fp8_indexer"] = quantised_indexer_report(layer, 8, work["indexer"]["flop"], args.steps, stream)
    line["norm_rope"] = norm_rope_report(layer, args.steps, stream)
    line["projections"] = projections_report(args.steps, stream)
    line["decode_cache"] = decode_cache_report(args.steps, stream)
    del layer
    torch.cuda.empty_cache()
    line["decode"] = decode_report(args.steps, stream)
    torch.cuda.empty_cache()
    line["prefill_configs"] = prefill_configs_report(args.steps, stream)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, rows_n=args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
