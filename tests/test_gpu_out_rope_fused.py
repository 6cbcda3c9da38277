"""The output rotation fused into the attention store (dsv4_sparse_mqa_fwd_rope,
dsv4_hca_dense_fwd_rope) against the two calls it replaces: the attention
call, then dsv4_out_rope on its output.  Bit for bit, on every attention case
of the per-call suite (generic fp32 kernel, c = 128 MFMA, c = 512 FP8 kernel,
split key ranges merged by the combine kernel), and against the oracle's
attention followed by its output rotation."""
import math

import numpy as np
import pytest

import oracle as O
from synth import gen as G
from tests.dsv4_testlib import assert_close, decode_act, dev, host, stored_rows_f64
from tests.test_gpu_calls import DENSE_CASES, SPARSE_CASES, act_arr, make_rows

pytestmark = pytest.mark.gpu
THETA = 10000.0


@pytest.fixture(scope="module")
def L():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_08_amd as lib
    return lib


def _same_bits(a, b):
    import torch
    va = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
    vb = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
    return torch.equal(va, vb)


def _rope_dims(c, i):
    # 64 (the pages' RoPE width) where it fits; every second case another width
    if c < 64:
        return 8 * (c // 16)
    return 64 if i % 2 == 0 or c == 64 else min(c, 128)


@pytest.mark.parametrize("i", range(len(SPARSE_CASES)))
def test_sparse_rope_fused_equals_two_calls(L, i):
    import torch
    qd, lay, B, nq, nh, c, S, k, nw, W, pos, use_sink = SPARSE_CASES[i]
    R = _rope_dims(c, i)
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
            idx[b, t, :sel.size] = np.where(rng.random(sel.size) > 0.1, sel, -1)
    if k == 0:
        idx = idx[:, :, :0]
    sink = G.normal(seed, "sink", (nh,), 0.5)
    scale = 1 / math.sqrt(c)
    qt, kvt = dev(q), dev(kv)
    it = dev(idx) if k > 0 else None
    wt = dev(win) if nw > 0 else None
    st = dev(sink) if use_sink else None
    ws = torch.empty(max(1, L.attn_workspace_size(False, B, nq, nh, c, k + nw)), dtype=torch.uint8, device="cuda")
    two = torch.empty_like(qt)
    L.sparse_mqa_fwd(qt, kvt, lay, it, wt, wpos, nw, pos, st, scale, two, ws, W=W)
    L.out_rope(two, pos, theta=THETA, rope_dims=R)
    one = torch.full_like(qt, float("nan"))
    L.sparse_mqa_fwd(qt, kvt, lay, it, wt, wpos, nw, pos, st, scale, one, ws, W=W, out_rope=(THETA, R))
    torch.cuda.synchronize()
    assert _same_bits(one, two), "fused rotation differs from attention + out_rope (R=%d)" % R
    got = decode_act(host(one))
    for b in range(B):
        ref = O.sparse_mqa(decode_act(q[b]), stored_rows_f64(kv[b], lay, c), idx[b], stored_rows_f64(win[b], lay, c)[:W],
                           wpos[b], nw, pos[b] + np.arange(nq), sink.astype(np.float64) if use_sink else None, scale)
        ref = O.out_rope(ref, pos[b] + np.arange(nq), THETA, R)
        assert_close(got[b], ref, fp32=(qd == "f32"), what="sparse+rot b=%d" % b)


@pytest.mark.parametrize("i", range(len(DENSE_CASES)))
def test_dense_rope_fused_equals_two_calls(L, i):
    import torch
    qd, lay, B, nq, nh, c, S, mp, nw, pos, use_sink = DENSE_CASES[i]
    R = _rope_dims(c, i)
    seed = 600 + S + c + nq
    q = act_arr(seed, "q", (B, nq, nh, c), 1.0, qd)
    kv = make_rows(seed, "cache_hca", (B, S, c), lay)
    wpos = [max(0, p - nw + 1) for p in pos]
    W = nq + nw
    win = make_rows(seed, "win_hca", (B, W, c), lay)
    sink = G.normal(seed, "sink", (nh,), 0.5)
    scale = 1 / math.sqrt(c)
    qt, kvt, wt = dev(q), dev(kv), dev(win)
    st = dev(sink) if use_sink else None
    need = L.attn_plan(True, L.BF16 if qd == "bf16" else L.F32, lay, B, nq, nh, c, S, 0, mp, nw, pos).workspace_bytes
    ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")
    two = torch.empty_like(qt)
    L.hca_dense_fwd(qt, kvt, lay, mp, wt, wpos, nw, pos, st, scale, two, ws)
    L.out_rope(two, pos, theta=THETA, rope_dims=R)
    one = torch.full_like(qt, float("nan"))
    L.hca_dense_fwd(qt, kvt, lay, mp, wt, wpos, nw, pos, st, scale, one, ws, out_rope=(THETA, R))
    torch.cuda.synchronize()
    assert _same_bits(one, two), "fused rotation differs from attention + out_rope (R=%d)" % R
    got = decode_act(host(one))
    for b in range(B):
        ref = O.hca_dense(decode_act(q[b]), stored_rows_f64(kv[b], lay, c), mp, stored_rows_f64(win[b], lay, c),
                          wpos[b], nw, pos[b] + np.arange(nq), sink.astype(np.float64) if use_sink else None, scale)
        ref = O.out_rope(ref, pos[b] + np.arange(nq), THETA, R)
        assert_close(got[b], ref, fp32=(qd == "f32"), what="dense+rot b=%d" % b)
