"""Parity of the streaming cache maintenance (dsv4_stream_compress and the
mirrored window ring) against the float64 oracle, through the C ABI: token
chunks of varying sizes crossing block boundaries, both projection paths
(bf16 MFMA and fp32), every row layout, prefix resume against the batch
compressor, the NaN marker of entries whose rows were never fed, and the ring
read by the attention kernels as a window buffer."""
import math

import numpy as np
import pytest

import oracle as O
from oracle import codecs as K
from oracle import stream as OS
from synth import gen as G
from tests.dsv4_testlib import (ROW_BF16, ROW_F32, ROW_FP8, ROW_MXFP4, assert_close, assert_quantized, decode_act,
                                dev, empty_rows, host, rows_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_08_amd as lib
    return lib


def _arr(seed, stream, shape, std, dtype):
    x = G.normal(seed, stream, shape, std)
    return G.to_bf16(x) if dtype == "bf16" else x


def _check_rows(got, ref, layout, what):
    if layout == ROW_F32:
        assert_close(got, ref, fp32=True, tol=1e-4 * max(1.0, float(np.abs(ref).max())), what=what)
    else:
        assert_quantized(got, ref, layout, what=what)


def _state(L, B, ov, m, c):
    import torch
    st = torch.zeros(B * L.stream_state_bytes(ov, m, c), dtype=torch.uint8, device="cuda")
    L.stream_state_reset(st, B, ov, m, c)
    return st


def _cache(B, S, layout, c):
    import torch
    cache = empty_rows(B * S, layout, c).view(B, S, -1)
    sc = torch.zeros((B, S, max(1, c // 32)), dtype=torch.uint8, device="cuda") if layout == ROW_MXFP4 else None
    return cache, sc


STREAM_CASES = [
    # (overlap, dtype, B, d, c, m, cache layout, ring layout, rope dims (norm when > 0), ring_w, chunks)
    (1, "bf16", 3, 128, 128, 4, ROW_FP8, ROW_FP8, 64, 8, [1, 3, 2, 5, 4, 1, 7]),
    (1, "f32", 2, 40, 32, 4, ROW_F32, ROW_F32, 0, 6, [2, 2, 5, 1, 9, 3]),
    (0, "bf16", 2, 256, 64, 16, ROW_BF16, ROW_BF16, 32, 16, [7, 1, 16, 3, 13, 5]),
    (1, "bf16", 2, 64, 64, 4, ROW_MXFP4, None, 0, 0, [4, 1, 1, 6, 3, 8]),
    (0, "bf16", 2, 256, 512, 128, ROW_FP8, ROW_FP8, 64, 128, [37, 64, 1, 90, 60, 20, 38]),
]


@pytest.mark.parametrize("case", STREAM_CASES, ids=[str(i) for i in range(len(STREAM_CASES))])
def test_stream_compress(L, case):
    import torch
    ov, dt, B, d, c, m, cl, rl, R, ring_w, chunks = case
    N = sum(chunks)
    seed = 1200 + N + c + m
    H = _arr(seed, "H", (B, N, d), 1.0, dt)
    W = _arr(seed, "W_kv" if ov else "W_hca", ((4 if ov else 2) * c, d), 2.0 / math.sqrt(d), dt)
    Bias = G.normal(seed, "B_kv" if ov else "B_hca", (2, m, c) if ov else (m, c), 0.5).astype(np.float32)
    gamma = (1.0 + G.normal(seed, "gamma", (c,), 0.3)).astype(np.float32)
    S = N // m + 1
    st = _state(L, B, ov, m, c)
    cache, sc = _cache(B, S, cl, c)
    ring = empty_rows(B * 2 * ring_w, rl, c).view(B, 2 * ring_w, -1) if rl is not None else None
    Hd, Wd, Bd, gd = dev(H), dev(W), dev(Bias), dev(gamma)
    x = 0
    for n_new in chunks:
        L.stream_compress(Hd[:, x:x + n_new].contiguous(), Wd, Bd, ov, m, c, [x] * B, st, cache=cache,
                          cache_scales=sc, cache_layout=cl, ring=ring, ring_w=ring_w,
                          ring_layout=rl if rl is not None else ROW_F32, norm=R > 0, gamma=gd if R > 0 else None,
                          rope_dims=R)
        x += n_new
    torch.cuda.synchronize()
    ne = N // m
    for b in range(B):
        ents, raw = OS.stream_feed(OS.stream_init(ov, m), decode_act(H[b]), 0, decode_act(W), Bias)
        ref = np.stack([ents[s] for s in range(ne)])
        if R > 0:
            ref = O.kv_norm_rope(ref, gamma, O.entry_positions(m, 0, ne), rope_dims=R)
        got = rows_to_f64(cache[b, :ne], cl, c, sc[b, :ne] if sc is not None else None)
        _check_rows(got, ref, cl, "entries of sequence %d" % b)
        if ring is None:
            continue
        lo = N - ring_w
        ref_w = raw[lo:N]
        if R > 0:
            ref_w = O.kv_norm_rope(ref_w, gamma, np.arange(lo, N), rope_dims=R)
        p0 = L.swa_ring_pos0(N - 1, ring_w)
        assert p0 == OS.ring_pos0(N - 1, ring_w)
        got_w = rows_to_f64(ring[b, lo - p0:N - p0], rl, c)
        _check_rows(got_w, ref_w, rl, "window ring of sequence %d" % b)


@pytest.mark.parametrize("P", [0, 4, 13, 16, 22])
def test_stream_resume_after_batch_prefix(L, P):
    # the prefix's entries come from the batch compressor (persisted), the tail
    # is replayed through the streaming state, and the rest is streamed
    import torch
    B, N, d, c, m, R = 2, 41, 128, 128, 4, 64
    seed = 1300 + P
    H = _arr(seed, "H", (B, N, d), 1.0, "bf16")
    W = _arr(seed, "W_kv", (4 * c, d), 2.0 / math.sqrt(d), "bf16")
    Bias = G.normal(seed, "B_kv", (2, m, c), 0.5).astype(np.float32)
    gamma = (1.0 + G.normal(seed, "gamma", (c,), 0.3)).astype(np.float32)
    S = N // m
    cache, _ = _cache(B, S, ROW_FP8, c)
    Hd, Wd, Bd, gd = dev(H), dev(W), dev(Bias), dev(gamma)
    npref = P // m
    for b in range(B):
        if npref == 0:
            continue
        comp = empty_rows(npref, ROW_F32, c)
        L.csa_compress(Hd[b, :P].contiguous(), Wd, Bd, m, c, comp, ROW_F32)
        L.kv_norm_rope(comp.view(1, npref, c), ROW_F32, c, gd, [m - 1], m, cache[b:b + 1, :npref], ROW_FP8,
                       rope_dims=R)
    st = _state(L, B, 1, m, c)
    t0 = OS.tail_start(P, m, 1)
    if P > t0:
        L.stream_compress(Hd[:, t0:P].contiguous(), Wd, Bd, 1, m, c, [t0] * B, st, emit_from=[npref] * B,
                          cache=cache, cache_layout=ROW_FP8, norm=True, gamma=gd, rope_dims=R)
    x = P
    for n_new in (3, 1, 5, 2, 7, 4, 6, 9, 11):
        n_new = min(n_new, N - x)
        if n_new <= 0:
            break
        L.stream_compress(Hd[:, x:x + n_new].contiguous(), Wd, Bd, 1, m, c, [x] * B, st, cache=cache,
                          cache_layout=ROW_FP8, norm=True, gamma=gd, rope_dims=R)
        x += n_new
    assert x == N
    torch.cuda.synchronize()
    for b in range(B):
        comp, _ = O.csa_compress(decode_act(H[b]), decode_act(W), Bias, m)
        ref = O.kv_norm_rope(comp, gamma, O.entry_positions(m, 0, S), rope_dims=R)
        _check_rows(rows_to_f64(cache[b], ROW_FP8, c), ref, ROW_FP8, "resumed cache of sequence %d" % b)


def test_stream_missing_rows_are_nan(L):
    import torch
    c, d = 32, 64
    for ov, m, first in ((1, 4, 12), (0, 8, 20)):
        H = _arr(7, "H", (1, 4, d), 1.0, "bf16")
        W = _arr(7, "W_kv", ((4 if ov else 2) * c, d), 0.2, "bf16")
        Bias = G.normal(7, "B_kv", (2, m, c) if ov else (m, c), 0.5).astype(np.float32)
        st = _state(L, 1, ov, m, c)
        cache = torch.zeros((1, 4, c), dtype=torch.float32, device="cuda")
        # positions first .. first + 3 complete block (first + 4) / m - 1, whose
        # b-window (CSA) or first half (HCA) was never fed
        L.stream_compress(dev(H), dev(W), dev(Bias), ov, m, c, [first], st, cache=cache, cache_layout=ROW_F32)
        torch.cuda.synchronize()
        got = host(cache)[0]
        s = (first + 4) // m - 1
        assert np.isnan(got[s]).all()
        assert not np.isnan(np.delete(got, s, axis=0)).any()


def test_ring_read_by_attention(L):
    # decode over the ring: the attention reads the mirrored ring as its window
    # buffer and must give bitwise the same output as with the same rows laid
    # out in position order, and match the oracle
    import torch
    B, d, c, mp, ring_w, n_win, nh = 2, 128, 512, 128, 128, 128, 16
    N = 300
    seed = 1400
    H = _arr(seed, "H", (B, N, d), 1.0, "bf16")
    W = _arr(seed, "W_hca", (2 * c, d), 2.0 / math.sqrt(d), "bf16")
    Bias = G.normal(seed, "B_hca", (mp, c), 0.5).astype(np.float32)
    gamma = (1.0 + G.normal(seed, "gamma", (c,), 0.3)).astype(np.float32)
    S = N // mp
    st = _state(L, B, 0, mp, c)
    cache, _ = _cache(B, S, ROW_FP8, c)
    ring = empty_rows(B * 2 * ring_w, ROW_FP8, c).view(B, 2 * ring_w, -1)
    Hd, Wd, Bd, gd = dev(H), dev(W), dev(Bias), dev(gamma)
    for x in range(0, N, 50):
        n_new = min(50, N - x)
        L.stream_compress(Hd[:, x:x + n_new].contiguous(), Wd, Bd, 0, mp, c, [x] * B, st, cache=cache,
                          cache_layout=ROW_FP8, ring=ring, ring_w=ring_w, ring_layout=ROW_FP8, norm=True,
                          gamma=gd, rope_dims=64)
    p = N - 1
    q = G.to_bf16(G.normal(seed, "q", (B, 1, nh, c), 1.0))
    sink = G.normal(seed, "sink", (nh,), 0.02).astype(np.float32)
    qd, sd = dev(q), dev(sink)
    scale = 1.0 / math.sqrt(c)
    ws_n = L.attn_workspace_size(1, B, 1, nh, c, S + n_win)
    ws = torch.empty(max(16, ws_n), dtype=torch.uint8, device="cuda")
    p0 = L.swa_ring_pos0(p, ring_w)
    out_ring = torch.empty((B, 1, nh, c), dtype=torch.bfloat16, device="cuda")
    L.hca_dense_fwd(qd, cache, ROW_FP8, mp, ring, [p0] * B, n_win, [p] * B, sd, scale, out_ring, ws)
    lo = p - n_win + 1
    lin = ring[:, lo - p0:p + 1 - p0].contiguous()
    out_lin = torch.empty_like(out_ring)
    L.hca_dense_fwd(qd, cache, ROW_FP8, mp, lin, [lo] * B, n_win, [p] * B, sd, scale, out_lin, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_ring.view(torch.int16), out_lin.view(torch.int16))
    for b in range(B):
        # the oracle's own cache and window: stream oracle -> norm / rope -> stored rounding
        ents, raw = OS.stream_feed(OS.stream_init(0, mp), decode_act(H[b]), 0, decode_act(W), Bias)
        kv_comp = np.stack([ents[s] for s in range(S)])
        kv_comp = K.round_rows(O.kv_norm_rope(kv_comp, gamma, O.entry_positions(mp, 0, S)), ROW_FP8)
        kv_win = K.round_rows(O.kv_norm_rope(raw[lo:p + 1], gamma, np.arange(lo, p + 1)), ROW_FP8)
        ref = O.hca_dense(decode_act(q[b]), kv_comp, mp, kv_win, lo, n_win, [p], sink, scale)
        assert_close(decode_act(host(out_ring[b])), ref, what="attention over the ring, sequence %d" % b)
