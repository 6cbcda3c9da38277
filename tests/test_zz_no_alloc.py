"""The allocation-free top-k call (dsv4_topk_select_noalloc) against the
workspace call (dsv4_topk_select) through the C ABI: identical indices, bit
for bit, on two calls in a row whose second input is smaller (the static
workspace keeps the first call's contents), and a shape beyond its workspace
is refused before anything runs."""
import numpy as np
import pytest

from synth import gen as G
from tests.dsv4_testlib import dev, host

pytestmark = pytest.mark.gpu


def run_both(L, B, nq, S, k, m, pos, seed):
    import torch
    sc = G.normal(seed, "extra", (B, nq, S), 10.0)
    sc[..., ::5] = np.round(sc[..., ::5])            # ties
    scores = dev(sc)
    ref = torch.empty((B, nq, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, L.topk_workspace_size(B, nq, S, k)), dtype=torch.uint8, device="cuda")
    L.topk_select(scores, m, pos, k, ref, ws)
    got = torch.full((B, nq, k), -7, dtype=torch.int32, device="cuda")
    L.topk_select_noalloc(scores, m, pos, k, got)
    torch.cuda.synchronize()
    return host(ref), host(got)


def test_noalloc_topk_matches_workspace_call_twice():
    import long_context_attention_08_amd as L
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # decode shape: 16 rows of 2^18 scores (the histogram select: about 5 MB of workspace)
    need1 = L.topk_workspace_size(16, 1, 262144, 1024)
    assert 0 < need1 <= L.lib.dsv4_topk_workspace_size(16, 1, 262144, 1024)
    r1, g1 = run_both(L, 16, 1, 262144, 1024, 4, [1 << 20] * 16, 31)
    assert np.array_equal(r1, g1)
    # a smaller second call on the same array
    r2, g2 = run_both(L, 3, 2, 50000, 512, 4, [190000, 150000, 200000], 32)
    assert L.topk_workspace_size(3, 2, 50000, 512) < need1
    assert np.array_equal(r2, g2)
    # a shape whose workspace exceeds the array is refused (status 2)
    big = torch.zeros((1, 300, 262144), dtype=torch.float32, device="cuda")   # sized in full all the same
    idx = torch.empty((1, 300, 1024), dtype=torch.int32, device="cuda")
    st = L.lib.dsv4_topk_select_noalloc(big.data_ptr(), 1, 300, 262144, 4, L._lib._host_i64([1 << 20]), 1024,
                                       idx.data_ptr(), None)
    assert st == 2 and b"allocation-free" in L.lib.dsv4_last_error()
