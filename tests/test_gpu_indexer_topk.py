"""Index scores + top-k in one call (dsv4_indexer_topk) against the two calls
it replaces, and against the oracle's top-k over the same scores.

The one-call path keeps only scores at or above a per-row threshold taken
from a strided sample of the keys; rows the threshold does not settle are
recomputed in full.  Its result must equal dsv4_indexer_score followed by
dsv4_topk_select bit for bit on every row, whichever way a row went: the
cases cover rows settled by the threshold, rows with fewer visible entries
than k, rows of all-equal scores (every key passes the threshold, the lists
overflow and the full-score path takes the row), a mix of both in one block,
single-query blocks (decode), two launch slices (more than 64 sequences), and
the paths that never sample (fp32 queries)."""
import numpy as np
import pytest

import oracle as O
from synth import gen as G
from tests.dsv4_testlib import ROW_BF16, ROW_F32, ROW_MXFP4, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_08_amd as lib
    return lib


IT_CASES = [
    # (q dtype, key layout, B, nq, hI, cI, S, m, k, pos0 list, query kind)
    ("bf16", ROW_MXFP4, 1, 64, 32, 64, 40000, 4, 1024, [200000], "normal"),      # 16-query blocks, k = 1024
    ("bf16", ROW_MXFP4, 2, 40, 32, 64, 20011, 4, 512, [3000, 80000], "normal"),  # ragged S; rows with < k visible
    ("bf16", ROW_BF16, 1, 20, 32, 128, 30000, 4, 256, [100000], "normal"),       # cI = 128: 8-query blocks
    ("bf16", ROW_BF16, 1, 33, 32, 32, 9000, 4, 64, [36000], "normal"),           # cI = 32, ragged query block
    ("bf16", ROW_MXFP4, 16, 1, 32, 64, 262144, 4, 1024, [1 << 20] * 16, "normal"),   # decode: single-query blocks
    ("bf16", ROW_MXFP4, 3, 5, 32, 64, 30000, 4, 1024, [120000, 50, 4000], "normal"),  # nq < 16; 12 and 1000 visible
    ("bf16", ROW_MXFP4, 1, 64, 32, 64, 40000, 4, 1024, [200000], "zeros"),       # all ties: every row recomputed
    ("bf16", ROW_MXFP4, 1, 64, 32, 64, 40000, 4, 1024, [200000], "mixed"),       # tied and normal rows in one block
    ("bf16", ROW_MXFP4, 4, 3, 32, 64, 50000, 4, 512, [200000] * 4, "mixed"),     # the same with single-query blocks
    ("bf16", ROW_MXFP4, 65, 1, 32, 64, 3000, 4, 64, list(range(11000, 11000 + 65 * 7, 7)), "normal"),  # two slices
    ("f32", ROW_F32, 2, 10, 4, 32, 5000, 4, 64, [20000, 100], "normal"),         # no sampled path (fp32 queries)
    ("bf16", ROW_BF16, 1, 9, 16, 64, 6000, 1, 128, [5990], "normal"),            # no sampled path (hI = 16), m = 1
    ("bf16", ROW_MXFP4, 2, 1, 32, 64, 600000, 4, 1024, [2400000, 1800000], "normal"),   # sample rows > 16384
    ("bf16", ROW_MXFP4, 1, 3, 32, 64, 400000, 4, 1024, [1600000], "normal"),   # 12500-score sample rows (LDS-staged)
    # small-integer scores: many equal scores among a row's candidates (the select's dense-tie path)
    ("bf16", ROW_BF16, 1, 32, 32, 64, 3000, 4, 256, [6000], "int"),
    ("bf16", ROW_MXFP4, 2, 20, 32, 64, 9000, 4, 512, [30000, 8000], "int"),
    # the layer-pair chunk's rows: 512 queries at 2^20 + 7000 + t over 2^18 + 2048 MXFP4 keys
    ("bf16", ROW_MXFP4, 1, 512, 32, 64, 264192, 4, 1024, [(1 << 20) + 7000], "normal"),
]


def _inputs(case, seed):
    qd, kl, B, nq, hI, cI, S, m, k, pos, kind = case
    qx = G.normal(seed, "qI", (B, nq, hI, cI), 0.5)
    if kind == "zeros":
        qx[:] = 0.0
    elif kind == "mixed":
        qx[:, ::2] = 0.0
    wI = G.normal(seed, "wI", (B, nq, hI))
    kx = G.normal(seed, "cache_ki", (B, S, cI))
    if kind == "int":
        # E2M1 values (exact in bf16 and MXFP4) and weights +-1: integer-valued scores, many of them equal
        rng = np.random.default_rng(seed)
        vals = np.array([0, 0.5, 1, -0.5, -1], dtype=np.float32)
        qx = vals[rng.integers(0, len(vals), (B, nq, hI, cI))]
        kx = vals[rng.integers(0, len(vals), (B, S, cI))]
        wI = rng.choice(np.array([-1, 1], dtype=np.float32), (B, nq, hI))
    qI = G.to_bf16(qx) if qd == "bf16" else qx
    keys, ksc = G.store(kx, kl) if kl != ROW_F32 else (kx, None)
    return qI, wI, keys, ksc


def _check_rows(B, nq, seed):
    if B * nq <= 96:
        return [(b, t) for b in range(B) for t in range(nq)]
    rng = np.random.default_rng(seed)
    rows = {(0, 0), (B - 1, nq - 1)}
    for r in rng.choice(B * nq, size=48, replace=False):
        rows.add((int(r) // nq, int(r) % nq))
    return sorted(rows)


@pytest.mark.parametrize("case", IT_CASES, ids=[str(i) for i in range(len(IT_CASES))])
def test_indexer_topk_equals_separate_calls(L, case):
    import torch
    qd, kl, B, nq, hI, cI, S, m, k, pos, kind = case
    seed = 900 + S + nq + k
    qI, wI, keys, ksc = _inputs(case, seed)
    qI_d, wI_d, keys_d = dev(qI), dev(wI), dev(keys)
    ksc_d = dev(ksc) if ksc is not None else None
    # the two separate calls
    scores = torch.empty((B, nq, S), dtype=torch.float32, device="cuda")
    L.indexer_score(qI_d, wI_d, keys_d, kl, m, pos, scores, k_scales=ksc_d)
    ref = torch.empty((B, nq, k), dtype=torch.int32, device="cuda")
    tws = torch.empty(max(1, L.topk_workspace_size(B, nq, S, k)), dtype=torch.uint8, device="cuda")
    L.topk_select(scores, m, pos, k, ref, tws)
    # one call, twice on a workspace that starts as garbage and then holds the first call's state
    qdt = L.BF16 if qd == "bf16" else L.F32
    nbytes = L.indexer_topk_workspace_size(qdt, kl, B, nq, hI, cI, S, k)
    ws = torch.full((max(1, nbytes),), 0xA5, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        idx = torch.full((B, nq, k), -7, dtype=torch.int32, device="cuda")
        L.indexer_topk(qI_d, wI_d, keys_d, kl, m, pos, k, idx, ws, k_scales=ksc_d)
        torch.cuda.synchronize()
        if not torch.equal(idx, ref):
            bad = (idx != ref).any(dim=2).nonzero().tolist()
            raise AssertionError("call %d: %d rows differ, first %s" % (rep, len(bad), bad[:4]))
    # the top-k of the same scores by the oracle, on sampled rows
    sc = host(scores)
    got = host(idx)
    del scores, ws
    for b, t in _check_rows(B, nq, seed):
        want = O.topk_select(sc[b, t:t + 1].astype(np.float64), m, [pos[b] + t], k)
        assert np.array_equal(got[b, t], want[0]), (b, t)

