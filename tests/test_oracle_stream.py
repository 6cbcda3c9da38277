"""Pins of the streaming cache-maintenance oracle (oracle/stream.py): the
token-by-token compressors against the batch compressors, prefix resume, and
the mirrored window ring against direct slicing."""
import numpy as np
import pytest

import oracle
from oracle import stream as OS


def _problem(seed, overlap, n, d=24, c=8, m=4):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((n, d))
    W = rng.standard_normal(((4 if overlap else 2) * c, d)) / np.sqrt(d)
    B = rng.standard_normal((2, m, c) if overlap else (m, c)) * 0.5
    return H, W, B


def _feed_chunks(st, H, W, B, pos0, seed, emit_from=0):
    rng = np.random.default_rng(seed)
    ents, raws = {}, []
    i = pos0
    while i < H.shape[0]:
        n = int(rng.integers(1, 8))
        e, r = OS.stream_feed(st, H[i:i + n], i, W, B, emit_from)
        assert not set(e) & set(ents)
        ents.update(e)
        raws.append(r)
        i += n
    return ents, (np.concatenate(raws) if raws else np.zeros((0, 0)))


@pytest.mark.parametrize("n", [3, 4, 37, 40])
def test_csa_stream_equals_batch(n):
    H, W, B = _problem(1, 1, n)
    comp, raw = oracle.csa_compress(H, W, B, 4)
    ents, r = _feed_chunks(OS.stream_init(1, 4), H, W, B, 0, seed=n)
    assert sorted(ents) == list(range(n // 4))
    for s in ents:
        np.testing.assert_allclose(ents[s], comp[s], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r, raw, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [7, 8, 33])
def test_hca_stream_equals_batch(n):
    H, W, B = _problem(2, 0, n, m=8)
    comp, raw = oracle.hca_compress(H, W, B, 8)
    ents, r = _feed_chunks(OS.stream_init(0, 8), H, W, B, 0, seed=n)
    assert sorted(ents) == list(range(n // 8))
    for s in ents:
        np.testing.assert_allclose(ents[s], comp[s], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r, raw, rtol=0, atol=1e-12)


def test_stream_entry0_has_no_b_window():
    # entry 0 pools only its own block: changing the b-weights changes nothing in it
    H, W, B = _problem(3, 1, 8)
    e1, _ = OS.stream_feed(OS.stream_init(1, 4), H, 0, W, B)
    W2 = W.copy()
    W2[8:16] *= -3.0          # C^b rows
    W2[24:32] += 1.0          # Z^b rows
    e2, _ = OS.stream_feed(OS.stream_init(1, 4), H, 0, W2, B)
    np.testing.assert_array_equal(e1[0], e2[0])
    assert np.abs(e1[1] - e2[1]).max() > 1e-3


@pytest.mark.parametrize("overlap,m", [(1, 4), (0, 8)])
@pytest.mark.parametrize("P", [0, 3, 4, 5, 8, 12, 13, 16])
def test_resume_after_prefix(overlap, m, P):
    n = 41
    H, W, B = _problem(4 + overlap, overlap, n, m=m)
    comp = (oracle.csa_compress(H, W, B, m) if overlap else oracle.hca_compress(H, W, B, m))[0]
    st = OS.resume(H, P, W, B, m, overlap)
    ents, _ = _feed_chunks(st, H, W, B, P, seed=P)
    assert sorted(ents) == list(range(P // m, n // m))
    for s in ents:
        np.testing.assert_allclose(ents[s], comp[s], rtol=0, atol=1e-12)


def test_tail_start_values():
    assert [OS.tail_start(P, 4, 1) for P in (0, 3, 4, 7, 8, 9)] == [0, 0, 0, 0, 4, 4]
    assert [OS.tail_start(P, 8, 0) for P in (0, 7, 8, 17)] == [0, 0, 8, 16]


def test_resume_without_the_b_window_fails():
    # replaying only the incomplete block is not enough for CSA: the next
    # entry's b-window is the last complete block
    H, W, B = _problem(6, 1, 20)
    st = OS.stream_init(1, 4)
    OS.stream_feed(st, H[12:14], 12, W, B, emit_from=3)
    with pytest.raises(ValueError):
        OS.stream_feed(st, H[14:16], 14, W, B)


@pytest.mark.parametrize("ring_w,n_win", [(8, 1), (8, 5), (8, 8), (5, 3)])
def test_ring_window_equals_slice(ring_w, n_win):
    rng = np.random.default_rng(ring_w * 10 + n_win)
    n = 4 * ring_w + 3
    rows = rng.standard_normal((n, 3))
    ring = np.full((2 * ring_w, 3), np.nan)
    x = 0
    while x < n:
        k = int(rng.integers(1, ring_w + 1))
        k = min(k, n - x)
        OS.ring_append(ring, ring_w, rows[x:x + k], x)
        x += k
        p = x - 1
        got = OS.ring_window(ring, ring_w, p, n_win)
        np.testing.assert_array_equal(got, rows[max(0, p - n_win + 1):p + 1])


def test_ring_pos0_range():
    for ring_w in (1, 4, 7, 128):
        for p in range(0, 5 * ring_w):
            p0 = OS.ring_pos0(p, ring_w)
            assert p0 % ring_w == 0
            assert ring_w - 1 <= p - p0 <= 2 * ring_w - 2
