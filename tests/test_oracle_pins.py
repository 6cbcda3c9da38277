"""Pins of the float64 oracle against what the pages and the mathematics fix:
invariants, closed forms, special cases that reduce to a textbook routine
(torch's scaled_dot_product_attention on the CPU in float64) and pairwise
brute force on tiny inputs.  CPU only.

Each test names the passage it pins: "digest" is the ai-papers-daily page
"DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence",
"blog" the jsqmd page "DeepSeek V4大模型算法解析"."""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O


def rnd(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def csa_weights(c, d, seed, zscale=1.0):
    W = rnd(seed, 4 * c, d) / np.sqrt(d)
    W[2 * c:] *= zscale
    return W


# ======================================================================
# CSA compressor (digest 模块 B eq 9-12; blog 第一阶段)
# ======================================================================

@pytest.mark.parametrize("m", [1, 2, 4])
def test_csa_pool_weights_sum_to_one(m):
    """blog 第一阶段: the softmax normalises the 2m weights to sum 1."""
    d, c, n = 16, 8, 8 * m
    H, W, B = rnd(0, n, d), csa_weights(c, d, 1, zscale=4.0), rnd(2, 2, m, c)
    for i in range(n // m):
        Wt = O.csa_pool_weights(H, W, B, m, i)
        assert Wt.shape == ((2 * m if i else m), c)
        assert np.allclose(Wt.sum(axis=0), 1.0, atol=1e-14)
        assert (Wt > 0).all()


@pytest.mark.parametrize("m,block0", [(1, 0), (2, 0), (4, 0), (4, 3)])
def test_csa_constant_kv_pools_to_constant(m, block0):
    """Constant C^a = C^b = v pools to v for every entry, entry 0 included."""
    d, c, n = 12, 8, 6 * m
    n_left = m if block0 else 0
    H = rnd(3, n_left + n, d)
    H[:, 0] = 1.0
    v = rnd(4, c)
    W = csa_weights(c, d, 5, zscale=3.0)
    W[:2 * c] = 0.0
    W[0:c, 0] = v          # C^a = H W_aKV^T = v for every row
    W[c:2 * c, 0] = v      # C^b = v
    comp, raw = O.csa_compress(H, W, rnd(6, 2, m, c), m, block0, n_left)
    assert np.allclose(comp, v[None, :], atol=1e-13)
    assert np.allclose(raw, v[None, :], atol=1e-13)


@pytest.mark.parametrize("m", [1, 2, 4])
def test_csa_zero_logits_is_mean_of_window_rows(m):
    """Z = 0, B = 0: every softmax weight is 1/(2m) (1/m for entry 0), so entry
    i is the mean of C^a rows [m i, m i + m) and C^b rows [m (i-1), m i)
    (blog 第一阶段 window description)."""
    d, c, n = 10, 6, 7 * m
    H = rnd(7, n, d)
    W = csa_weights(c, d, 8)
    W[2 * c:] = 0.0
    comp, raw = O.csa_compress(H, W, np.zeros((2, m, c)), m)
    Ca, Cb = H @ W[:c].T, H @ W[c:2 * c].T
    assert np.allclose(raw, Ca)
    assert np.allclose(comp[0], Ca[0:m].mean(axis=0))
    for i in range(1, n // m):
        want = (Ca[m * i:m * i + m].sum(axis=0) + Cb[m * (i - 1):m * i].sum(axis=0)) / (2 * m)
        assert np.allclose(comp[i], want)


def test_csa_contraction_orientation():
    """H = I, m = 1, Z = B = 0: entry i = (W_aKV[:, i] + W_bKV[:, i-1]) / 2, which
    fixes C = H W^T with W stored [out, in]."""
    d = c = 6
    W = csa_weights(c, d, 9)
    W[2 * c:] = 0.0
    comp, _ = O.csa_compress(np.eye(d), W, np.zeros((2, 1, c)), 1)
    assert np.allclose(comp[0], W[:c, 0])
    for i in range(1, d):
        assert np.allclose(comp[i], (W[:c, i] + W[c:2 * c, i - 1]) / 2)


@pytest.mark.parametrize("r0", [0, 1, 3])
def test_csa_bias_selects_row(r0):
    """A +60 position bias on row r0 of B^a (Z = 0) picks C^a[m i + r0]; on B^b it
    picks C^b[m (i-1) + r0] for i >= 1 and leaves entry 0 the a-mean."""
    m, d, c, n = 4, 9, 5, 24
    H = rnd(10, n, d)
    W = csa_weights(c, d, 11)
    W[2 * c:] = 0.0
    Ca, Cb = H @ W[:c].T, H @ W[c:2 * c].T
    B = np.zeros((2, m, c))
    B[0, r0] = 60.0
    comp, _ = O.csa_compress(H, W, B, m)
    for i in range(n // m):
        assert np.allclose(comp[i], Ca[m * i + r0], atol=1e-20 + 1e-12)
    B = np.zeros((2, m, c))
    B[1, r0] = 60.0
    comp, _ = O.csa_compress(H, W, B, m)
    assert np.allclose(comp[0], Ca[:m].mean(axis=0))
    for i in range(1, n // m):
        assert np.allclose(comp[i], Cb[m * (i - 1) + r0], atol=1e-12)


def test_csa_logit_shift_invariance():
    """Adding the same constant to every Z logit of a channel changes nothing."""
    m, d, c, n = 4, 8, 6, 32
    H = rnd(12, n, d)
    H[:, 0] = 1.0
    W = csa_weights(c, d, 13, zscale=2.0)
    B = rnd(14, 2, m, c)
    base, _ = O.csa_compress(H, W, B, m)
    W2 = W.copy()
    shift = rnd(15, c) * 5
    W2[2 * c:3 * c, 0] += shift
    W2[3 * c:4 * c, 0] += shift
    comp, _ = O.csa_compress(H, W2, B, m)
    assert np.allclose(comp, base, atol=1e-12)


def test_csa_chunked_equals_whole():
    """Compressing in two chunks (the second with block0 and m rows of left
    context) equals one call over the whole sequence (digest 模块 F: cached
    entries are reused and only incomplete blocks are recomputed)."""
    m, d, c, n = 4, 8, 5, 40
    H, W, B = rnd(16, n, d), csa_weights(c, d, 17, 2.0), rnd(18, 2, m, c)
    whole, raw = O.csa_compress(H, W, B, m)
    n1 = 16
    a, ra = O.csa_compress(H[:n1], W, B, m)
    b, rb = O.csa_compress(H[n1 - m:], W, B, m, block0=n1 // m, n_left=m)
    assert np.allclose(np.concatenate([a, b]), whole, atol=1e-13)
    assert np.allclose(np.concatenate([ra, rb]), raw)


def test_csa_incomplete_tail_emits_nothing_and_stays_in_hull():
    m, d, c = 4, 8, 5
    H, W, B = rnd(19, 22, d), csa_weights(c, d, 20, 3.0), rnd(21, 2, m, c)
    comp, raw = O.csa_compress(H, W, B, m)
    assert comp.shape == (5, c) and raw.shape == (22, c)
    Ca, Cb = H @ W[:c].T, H @ W[c:2 * c].T
    for i in range(1, 5):
        rows = np.concatenate([Ca[m * i:m * i + m], Cb[m * (i - 1):m * i]])
        assert (comp[i] <= rows.max(axis=0) + 1e-12).all()
        assert (comp[i] >= rows.min(axis=0) - 1e-12).all()


def test_csa_b_window_vanishing_reduces_to_non_overlapping_pool():
    """B^b -> -inf removes the b-window: CSA then equals the non-overlapping HCA
    pooling with ratio m on (W_aKV, W_aZ, B^a) (digest 模块 C: HCA is CSA without
    overlap)."""
    m, d, c, n = 4, 8, 5, 32
    H, W, B = rnd(22, n, d), csa_weights(c, d, 23, 2.0), rnd(24, 2, m, c)
    B[1] = -1e4
    comp, _ = O.csa_compress(H, W, B, m)
    Wh = np.concatenate([W[:c], W[2 * c:3 * c]])
    hca, _ = O.hca_compress(H, Wh, B[0], m)
    assert np.allclose(comp, hca, atol=1e-12)


def test_csa_missing_left_context_raises():
    with pytest.raises(ValueError):
        O.csa_compress(rnd(0, 8, 4), rnd(1, 8, 4), np.zeros((2, 4, 2)), 4, block0=2, n_left=0)


# ======================================================================
# HCA compressor (digest 模块 C eq 20-23)
# ======================================================================

def test_hca_closed_forms():
    mp, d, c, n = 8, 10, 6, 40
    H = rnd(25, n, d)
    W = rnd(26, 2 * c, d)
    W[c:] = 0.0
    comp, raw = O.hca_compress(H, W, np.zeros((mp, c)), mp)
    C = H @ W[:c].T
    assert comp.shape == (5, c)
    for i in range(5):
        assert np.allclose(comp[i], C[mp * i:mp * (i + 1)].mean(axis=0))   # mean pooling
    B = np.zeros((mp, c))
    B[5] = 60.0
    comp, _ = O.hca_compress(H, W, B, mp)
    for i in range(5):
        assert np.allclose(comp[i], C[mp * i + 5], atol=1e-12)
    # constant KV pools to the constant
    H[:, 0] = 1.0
    W2 = rnd(27, 2 * c, d)
    W2[:c] = 0
    W2[:c, 0] = np.arange(c)
    comp, _ = O.hca_compress(H, W2, rnd(28, mp, c), mp)
    assert np.allclose(comp, np.arange(c)[None, :])


# ======================================================================
# Lightning indexer (digest 模块 B eq 13-16; blog 第二阶段)
# ======================================================================

def test_indexer_single_head_is_relu_dot():
    qI, KI = rnd(30, 6, 1, 8), rnd(31, 20, 8)
    I = O.indexer_score(qI, np.ones((6, 1)), KI, 1, np.full(6, 100))
    assert np.allclose(I, np.maximum(qI[:, 0] @ KI.T, 0))


def test_indexer_basis_query_picks_key_coordinate():
    """q^I_{t,h} = e_{j_h}: I[t,s] = sum_h w_h ReLU(K[s, j_h]) -- fixes which axis
    is contracted."""
    KI = rnd(32, 12, 5)
    qI = np.zeros((1, 3, 5))
    js = [4, 0, 2]
    for h, j in enumerate(js):
        qI[0, h, j] = 1.0
    w = np.array([[0.5, -2.0, 3.0]])
    I = O.indexer_score(qI, w, KI, 1, [11])
    want = sum(w[0, h] * np.maximum(KI[:, j], 0) for h, j in enumerate(js))
    assert np.allclose(I[0], want)


def test_indexer_integer_closed_form():
    """q_h = (h+1) e_0, K_s = (s-2) e_0, w = 1: I[s] = (s-2) H (H+1) / 2 for s > 2
    and 0 otherwise (ReLU clips every negative dot product)."""
    nh, S = 4, 9
    qI = np.zeros((1, nh, 3))
    qI[0, :, 0] = np.arange(1, nh + 1)
    KI = np.zeros((S, 3))
    KI[:, 0] = np.arange(S) - 2
    I = O.indexer_score(qI, np.ones((1, nh)), KI, 1, [S - 1])
    want = np.where(np.arange(S) > 2, (np.arange(S) - 2) * nh * (nh + 1) / 2, 0)
    assert np.array_equal(I[0], want)


def test_indexer_negative_dots_are_zero_and_weights_linear():
    KI = np.abs(rnd(33, 10, 4))
    qI = -np.abs(rnd(34, 2, 3, 4))
    I = O.indexer_score(qI, rnd(35, 2, 3), KI, 1, [20, 20])
    assert np.array_equal(I, np.zeros_like(I))
    qI, KI = rnd(36, 3, 4, 6), rnd(37, 15, 6)
    w1, w2 = rnd(38, 3, 4), rnd(39, 3, 4)
    pos = [40, 40, 40]
    I1 = O.indexer_score(qI, w1, KI, 1, pos)
    I2 = O.indexer_score(qI, w2, KI, 1, pos)
    I12 = O.indexer_score(qI, w1 + w2, KI, 1, pos)
    assert np.allclose(I12, I1 + I2)
    assert np.allclose(O.indexer_score(qI, -w1, KI, 1, pos), -I1)
    perm = [2, 0, 3, 1]
    assert np.allclose(O.indexer_score(qI[:, perm], w1[:, perm], KI, 1, pos), I1)


@pytest.mark.parametrize("p,nvis", [(0, 0), (2, 0), (3, 1), (6, 1), (7, 2), (8, 2), (11, 3), (1000, 6)])
def test_indexer_visibility_boundary(p, nvis):
    """Entry s (pooling tokens up to m(s+1)-1) is visible at p iff m(s+1) <= p+1
    (digest 模块 D: a query attends only to earlier compressed blocks)."""
    I = O.indexer_score(rnd(40, 1, 2, 3), rnd(41, 1, 2), rnd(42, 6, 3), 4, [p])
    assert np.isfinite(I[0, :nvis]).all()
    assert np.isneginf(I[0, nvis:]).all()


# ----------------------------------------------------------------------
# FP4 lightning indexer (digest 模块 F; reading R19b: q^I rounded to MXFP4
# per head in blocks of 32 along c_I, then eq 16)
# ----------------------------------------------------------------------

def test_indexer_fp4q_hand_example():
    """Scores worked by hand on basis keys.  Head 0, block 0: amax 5.5 gives
    scale 2^0, so 5.5 -> 6 (beyond the 5 boundary), 1.3 -> 1.5, 0.2 -> 0,
    -2.75 -> -3.  Head 0, block 1: amax 0.1 gives scale 2^-6, 0.1 -> 6 * 2^-6
    (saturated), 0.03 -> 2 * 2^-6.  Head 1, block 0: amax 0.75 gives scale 2^-3;
    the ties 0.3125 = 2.5 * 2^-3 and 0.15625 = 1.25 * 2^-3 go to the even codes
    2 and 1."""
    q = np.zeros((1, 2, 64))
    q[0, 0, [0, 1, 2, 3, 32, 33]] = [5.5, 1.3, 0.2, -2.75, 0.1, 0.03]
    q[0, 1, [0, 1, 2]] = [0.75, 0.3125, 0.15625]
    w = np.array([[1.0, 10.0]])
    I = O.indexer_score_fp4q(q, w, np.eye(64), 1, [63])
    want = np.zeros(64)
    want[[0, 1, 2, 32, 33]] = [6 + 10 * 0.75, 1.5 + 10 * 0.25, 10 * 0.125, 6 * 2.0**-6, 2 * 2.0**-6]
    assert np.array_equal(I[0], want)
    # the unrounded query scores differently (13 at key 0), so rounding is applied
    assert O.indexer_score(q, w, np.eye(64), 1, [63])[0, 0] == 13.0


def test_indexer_fp4q_grid_query_equals_plain_scores():
    """A query already on the MXFP4 grid (each 32-block holds a +-6 element, so
    its scale is its own) rounds to itself: the FP4 scores equal eq 16."""
    rng = np.random.default_rng(90)
    nq, hI, cI, S = 3, 4, 64, 40
    codes = rng.integers(0, 256, (nq, hI, cI // 2)).astype(np.uint8)
    codes[..., 0] = (codes[..., 0] & 0xF0) | 0x7          # element 0 of block 0 = +6
    codes[..., 16] = (codes[..., 16] & 0xF0) | 0xF        # element 0 of block 1 = -6
    scales = rng.integers(118, 136, (nq, hI, cI // 32)).astype(np.uint8)
    q = O.codecs.mxfp4_decode(codes, scales)
    K = rnd(91, S, cI)
    w = rnd(92, nq, hI)
    pos = [39, 20, 5]
    assert np.array_equal(O.indexer_score_fp4q(q, w, K, 1, pos), O.indexer_score(q, w, K, 1, pos))


def test_indexer_fp4q_blocks_are_per_head():
    """Scaling one head by 2^20 (and its weight by 2^-20) leaves every score
    unchanged: MXFP4 rounding is equivariant under powers of two and the blocks
    never span heads; a scale shared across heads would flush head 0 to zero."""
    q = rnd(93, 2, 3, 64)
    w = rnd(94, 2, 3)
    K = rnd(95, 30, 64)
    pos = [29, 12]
    base = O.indexer_score_fp4q(q, w, K, 1, pos)
    q2, w2 = q.copy(), w.copy()
    q2[:, 1] *= 2.0**20
    w2[:, 1] *= 2.0**-20
    assert np.array_equal(O.indexer_score_fp4q(q2, w2, K, 1, pos), base)
    assert np.array_equal(O.indexer_score_fp4q(q * 2.0**-7, w, K, 1, pos)[np.isfinite(base)],
                          base[np.isfinite(base)] * 2.0**-7)


def test_indexer_fp8q_hand_example():
    """FP8 queries (R19c) on basis keys.  Head 0, block 0: amax 3 gives scale
    2^-7; 3 -> 384 (exact), 0.1 -> 12.8 -> 13 on the E4M3 grid, so 0.1015625.
    Head 1: amax 0.3 gives scale 2^-10; 0.3 -> 307.2 -> 320, so 0.3125."""
    q = np.zeros((1, 2, 64))
    q[0, 0, [0, 1]] = [3.0, 0.1]
    q[0, 1, 0] = 0.3
    w = np.array([[1.0, 10.0]])
    I = O.indexer_score_fp8q(q, w, np.eye(64), 1, [63])
    want = np.zeros(64)
    want[[0, 1]] = [3.0 + 10 * 0.3125, 0.1015625]
    assert np.array_equal(I[0], want)
    assert O.indexer_score(q, w, np.eye(64), 1, [63])[0, 0] == 6.0


def test_indexer_fp8q_grid_query_equals_plain_scores():
    """A query already on the MXFP8 grid (each block holds a +-448 element, so
    its scale is its own) rounds to itself: the FP8 scores equal eq 16."""
    rng = np.random.default_rng(96)
    nq, hI, cI, S = 3, 4, 64, 40
    codes = rng.integers(0, 0x7F, (nq, hI, cI)).astype(np.uint8)
    codes = codes | (rng.integers(0, 2, codes.shape).astype(np.uint8) << 7)
    codes[..., 0] = 0x7E                                   # +448 in block 0
    codes[..., 32] = 0xFE                                  # -448 in block 1
    scales = rng.integers(110, 130, (nq, hI, cI // 32)).astype(np.uint8)
    q = O.codecs.mxfp8_decode(codes, scales)
    K = rnd(97, S, cI)
    w = rnd(98, nq, hI)
    pos = [39, 20, 5]
    assert np.array_equal(O.indexer_score_fp8q(q, w, K, 1, pos), O.indexer_score(q, w, K, 1, pos))


def test_indexer_fp8q_blocks_are_per_head_and_closer_than_fp4():
    """Power-of-two scaling of one head (and the inverse on its weight) leaves
    the scores unchanged; on random data FP8 queries stay well closer to the
    bf16 scores than FP4 queries (not by the full 4x of the finer grid: block
    maxima between 1.75 and 2 times a power of two saturate at 448)."""
    q = rnd(99, 2, 3, 64)
    w = rnd(100, 2, 3)
    K = rnd(101, 30, 64)
    pos = [29, 12]
    base = O.indexer_score_fp8q(q, w, K, 1, pos)
    q2, w2 = q.copy(), w.copy()
    q2[:, 1] *= 2.0**20
    w2[:, 1] *= 2.0**-20
    assert np.array_equal(O.indexer_score_fp8q(q2, w2, K, 1, pos), base)
    ref = O.indexer_score(q, w, K, 1, pos)
    f = np.isfinite(ref)
    e8 = np.abs(base[f] - ref[f]).max()
    e4 = np.abs(O.indexer_score_fp4q(q, w, K, 1, pos)[f] - ref[f]).max()
    assert e8 < e4 / 2


# ----------------------------------------------------------------------
# Q/KV RMSNorm and partial RoPE (digest 模块 D; readings R32-R35)
# ----------------------------------------------------------------------

def test_rmsnorm_closed_forms():
    """A constant vector a*1 normalises to a / sqrt(a^2 + eps) per channel,
    times gamma; gamma scales channel by channel; the output's mean square is
    ms / (ms + eps) for unit gamma."""
    c, eps = 16, 1e-6
    g = np.linspace(0.5, 2.0, c)
    y = O.rmsnorm(np.full(c, 3.0), g, eps)
    assert np.allclose(y, 3.0 / np.sqrt(9.0 + eps) * g, rtol=1e-15, atol=0)
    x = rnd(60, 5, c)
    ms = np.mean(x * x, axis=-1)
    y1 = O.rmsnorm(x, np.ones(c), eps)
    assert np.allclose(np.mean(y1 * y1, axis=-1), ms / (ms + eps), rtol=1e-13)
    assert np.allclose(O.rmsnorm(x, g, eps), y1 * g, rtol=1e-15)


def test_rope_hand_example_pins_interleaved_pairs():
    """Pair j of the last 64 dims is (c-64+2j, c-64+2j+1), rotated by
    pos * 10000^(-2j/64): at pos 1, (1, 0) in pair 0 becomes (cos 1, sin 1) and
    (1, 0) in pair 1 becomes (cos a, sin a), a = 10000^(-1/32); earlier dims
    are untouched (a half-split pairing would move dim c-32 instead)."""
    c = 72
    x = np.zeros(c)
    x[c - 64] = 1.0
    x[c - 62] = 1.0
    x[3] = 7.0
    y = O.rope_last(x[None], [1.0])[0]
    a = 10000.0 ** (-1.0 / 32)
    want = np.zeros(c)
    want[3] = 7.0
    want[c - 64], want[c - 63] = np.cos(1.0), np.sin(1.0)
    want[c - 62], want[c - 61] = np.cos(a), np.sin(a)
    assert np.allclose(y, want, rtol=0, atol=1e-15)


def test_rope_rotation_identities():
    """R(0) = I, each pair keeps its length, R(a) R(b) = R(a + b)."""
    x = rnd(61, 4, 128)
    assert np.array_equal(O.rope_last(x, np.zeros(4)), x)
    y = O.rope_last(x, [5.0, -3.0, 1e6, 0.25])
    n0 = x[:, 64::2] ** 2 + x[:, 65::2] ** 2
    n1 = y[:, 64::2] ** 2 + y[:, 65::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)
    ab = O.rope_last(O.rope_last(x, [2.0, 7.0, 11.0, 13.0]), [3.0, -7.0, 100.0, 0.5])
    assert np.allclose(ab, O.rope_last(x, [5.0, 0.0, 111.0, 13.5]), rtol=0, atol=1e-12)


def test_rope_chain_depends_only_on_relative_positions():
    """Logits (R(p) q) . (R(s) k) and the rotated-back output R(-p) sum_s P_s
    R(s) v_s are unchanged when every position moves by the same offset: the
    reason the pages rotate the output by the query's position."""
    c = 96
    q = O.rmsnorm(rnd(62, 1, c), np.ones(c))
    ks = O.rmsnorm(rnd(63, 9, c), np.ones(c))
    p, s = 40.0, np.arange(20.0, 29.0)
    def chain(shift):
        qr = O.rope_last(q, [p + shift])
        kr = O.rope_last(ks, s + shift)
        lg = kr @ qr[0] / np.sqrt(c)
        P = np.exp(lg - lg.max())
        P /= P.sum()
        o = (P[:, None] * kr).sum(axis=0)
        return lg, O.out_rope(o[None, None], [p + shift])[0, 0]
    l0, o0 = chain(0.0)
    l1, o1 = chain(12345.0)
    assert np.allclose(l0, l1, rtol=0, atol=1e-9)
    assert np.allclose(o0, o1, rtol=0, atol=1e-9)


def test_q_norm_rope_hand_example_order_and_positions():
    """Query preparation normalises first, then rotates (digest 模块 D: RMSNorm of
    each head before core attention; partial RoPE of the last dims), and every
    head of query t turns by that query's own position.  With c = 8, 4 rotated
    dims and gamma = (1 .. 8): the row (2, 0, 2, 0, 2, 0, 2, 0) has
    rms = sqrt(2), so the normalised row is sqrt(2) * (1, 0, 3, 0, 5, 0, 7, 0);
    its pairs (4, 5) and (6, 7) then turn by p and by p / 100 (theta = 10000,
    angle p * theta^(-2j/4)).  Rotating before normalising would scale the
    rotated components by gamma 6 and 8 instead of 5 and 7, and broadcasting
    the positions over heads instead of queries would turn head h by q_pos[h]."""
    c, R = 8, 4
    g = np.arange(1.0, 9.0)
    row = np.array([2.0, 0, 2.0, 0, 2.0, 0, 2.0, 0])
    q = np.zeros((2, 3, c))
    q[0, 0] = q[0, 1] = q[1, 0] = q[1, 2] = row
    q[0, 2] = q[1, 1] = 3.0 * row            # RMSNorm is scale invariant (eps = 0)
    pos = [1.0, 3.0]
    y = O.q_norm_rope(q, g, pos, eps=0.0, theta=10000.0, rope_dims=R)
    r2 = np.sqrt(2.0)

    def want(p):
        a, b = p, p / 100.0
        return np.array([r2 * 1, 0, r2 * 3, 0, r2 * 5 * np.cos(a), r2 * 5 * np.sin(a),
                         r2 * 7 * np.cos(b), r2 * 7 * np.sin(b)])

    for h in range(3):
        assert np.allclose(y[0, h], want(1.0), rtol=0, atol=1e-14), h
        assert np.allclose(y[1, h], want(3.0), rtol=0, atol=1e-14), h
    # the composition in the other order is a different function on this input
    wrong = O.rmsnorm(O.rope_last(q[0, 0][None], [1.0], 10000.0, R), g, 0.0)[0]
    assert not np.allclose(wrong, want(1.0), atol=1e-3)


def test_kv_norm_rope_hand_example_rows_use_their_own_positions():
    """KV row preparation (R32-R34): each row is normalised with the per-channel
    gamma and then turned by its own position; entries at m(s+1) - 1.  Row 0 =
    (0, 0, 0, 4) has rms 2, so the normalised row is (0, 0, 0, 2 gamma_3) =
    (0, 0, 0, 8); its only rotated pair (2, 3) with R = 2 turns by p: (0, 8)
    becomes (-8 sin p, 8 cos p).  Row 1 = (1, 1, 1, 1) normalises to gamma and
    turns by its own position q: (3 cos q - 4 sin q, 3 sin q + 4 cos q)."""
    g = np.array([1.0, 2.0, 3.0, 4.0])
    rows = np.array([[0.0, 0, 0, 4.0], [1.0, 1, 1, 1]])
    m, s0 = 4, 5
    pos = O.entry_positions(m, s0, 2)              # 23, 27
    assert list(pos) == [23, 27]
    y = O.kv_norm_rope(rows, g, pos, eps=0.0, theta=10000.0, rope_dims=2)
    p, q = 23.0, 27.0
    assert np.allclose(y[0], [0, 0, -8 * np.sin(p), 8 * np.cos(p)], rtol=0, atol=1e-13)
    assert np.allclose(y[1], [1, 2, 3 * np.cos(q) - 4 * np.sin(q), 3 * np.sin(q) + 4 * np.cos(q)], rtol=0,
                       atol=1e-13)
    # eps enters under the root: (0, 0, 0, 4) with eps = 12 has rms sqrt(4 + 12) = 4
    y2 = O.kv_norm_rope(rows[:1], g, [0], eps=12.0, theta=10000.0, rope_dims=2)
    assert np.allclose(y2[0], [0, 0, 0, 4.0], rtol=0, atol=1e-15)


def test_entry_positions_match_visibility():
    """Entry s sits at the newest token it pools, m (s + 1) - 1, so it is visible
    at position p exactly when its position is <= p (R5, R34)."""
    for m in (1, 4, 128):
        pos = O.entry_positions(m, 0, 50)
        assert pos[0] == m - 1 and pos[2] == 3 * m - 1
        for p in (0, m - 2, m - 1, 3 * m, 7 * m + 3):
            assert (pos <= p).sum() == O.visible_count(p, m, 50)
    assert np.array_equal(O.entry_positions(4, 10, 3), [43, 47, 51])


# ----------------------------------------------------------------------
# Low-rank query path and grouped output projection (digest 模块 B eq 13-15,
# 18 and the grouped output projection; readings R36, R37)
# ----------------------------------------------------------------------

def test_query_proj_orientation_and_head_layout():
    """Selector and permutation weights: c^Q = h W^DQ^T picks h's first 4 dims,
    q = c^Q W^UQ^T permutes them, and the result is split head-major
    (q[t, h, :] = columns [h c, (h+1) c)).  Integer values stay exact in bf16."""
    n, d, dc = 3, 8, 4
    h = np.arange(n * d, dtype=np.float64).reshape(n, d) - 7.0
    W_DQ = np.eye(dc, d)
    P = np.eye(4)[[2, 0, 3, 1]]                       # q column i = c^Q column perm[i]
    W_w = np.zeros((2, d))
    W_w[0, 5], W_w[1, 7] = 1.0, -2.0
    q, qI, wI = O.query_proj(h, W_DQ, P, np.eye(4)[::-1], W_w, nh=2, c=2, hI=1, cI=4)
    cq = h[:, :4]
    assert np.array_equal(q, cq[:, [2, 0, 3, 1]].reshape(n, 2, 2))
    assert np.array_equal(qI, cq[:, ::-1].reshape(n, 1, 4))
    assert np.array_equal(wI, np.stack([h[:, 5], -2.0 * h[:, 7]], axis=1))


def test_query_proj_latent_is_stored_bf16():
    """c^Q = 1 + 2^-10 is stored as 1.0 (below half an ulp of bf16), so
    q = c^Q * 1 is exactly 1.0, while w^I, formed from h directly, keeps it."""
    h = np.array([[1.0, 2.0 ** -10]])
    q, qI, wI = O.query_proj(h, np.ones((1, 2)), np.ones((1, 1)), np.ones((1, 1)), np.ones((1, 2)),
                             nh=1, c=1, hI=1, cI=1)
    assert q[0, 0, 0] == 1.0 and qI[0, 0, 0] == 1.0
    assert wI[0, 0] == 1.0 + 2.0 ** -10


def test_output_proj_groups_are_consecutive_heads():
    """With identity weights the grouped projection is the head-major flatten;
    zeroing group 1's weights zeroes exactly columns [d_g, 2 d_g), the heads
    2 and 3."""
    n, nh, c, g = 2, 4, 2, 2
    o = np.arange(n * nh * c, dtype=np.float64).reshape(n, nh, c) + 1.0
    W1 = np.stack([np.eye(4), np.eye(4)])
    out = O.output_proj(o, W1, np.eye(8), g)
    assert np.array_equal(out, o.reshape(n, 8))
    W1[1] = 0.0
    out = O.output_proj(o, W1, np.eye(8), g)
    assert np.array_equal(out[:, :4], o[:, :2].reshape(n, 4)) and not out[:, 4:].any()


def test_projections_scale_by_powers_of_two_exactly():
    """bf16 storage commutes with scaling by 2^k, so both paths are exactly
    2^k-homogeneous."""
    rng = np.random.default_rng(64)
    o = rng.standard_normal((3, 4, 8))
    W1 = rng.standard_normal((2, 5, 16))
    W2 = rng.standard_normal((6, 10))
    a = O.output_proj(o, W1, W2, 2)
    assert np.array_equal(O.output_proj(o * 8.0, W1, W2, 2), a * 8.0)
    h = rng.standard_normal((3, 8))
    ws = [rng.standard_normal(sh) for sh in ((4, 8), (6, 4), (4, 4), (2, 8))]
    q, qI, wI = O.query_proj(h, *ws, nh=2, c=3, hI=2, cI=2)
    q2, qI2, wI2 = O.query_proj(h * 0.25, *ws, nh=2, c=3, hI=2, cI=2)
    assert np.array_equal(q2, q * 0.25) and np.array_equal(qI2, qI * 0.25) and np.array_equal(wI2, wI * 0.25)


# ======================================================================
# Top-k selector (digest 模块 B eq 17)
# ======================================================================

def _beats(a, b, scores):
    return scores[a] > scores[b] or (scores[a] == scores[b] and a < b)


@pytest.mark.parametrize("seed", range(6))
def test_topk_pairwise_brute_force(seed):
    rng = np.random.default_rng(seed)
    S = 12
    scores = rng.integers(-3, 4, (5, S)).astype(np.float64)   # many ties
    scores[0, 3] = -0.0
    scores[0, 5] = 0.0
    pos = rng.integers(0, 4 * S + 4, 5)
    for k in (1, 3, 5, 12, 20):
        idx = O.topk_select(scores, 4, pos, k)
        for t in range(5):
            nv = min(S, (pos[t] + 1) // 4)
            sel = [s for s in idx[t] if s >= 0]
            assert len(sel) == min(k, nv)
            assert all(s == -1 for s in idx[t][len(sel):])
            assert all(0 <= s < nv for s in sel)
            rest = [s for s in range(nv) if s not in sel]
            for a, b in itertools.product(sel, rest):
                assert _beats(a, b, scores[t])
            for a, b in zip(sel, sel[1:]):
                assert _beats(a, b, scores[t])
            want = sorted(range(nv), key=lambda s: (-scores[t, s], s))[:k]
            assert sel == want


def test_topk_all_equal_and_signed_zero():
    I = np.zeros((1, 10))
    I[0, ::2] = -0.0
    assert list(O.topk_select(I, 1, [100], 4)[0]) == [0, 1, 2, 3]
    assert list(O.topk_select(I, 1, [3], 6)[0]) == [0, 1, 2, 3, -1, -1]


# ======================================================================
# Core attention (digest 模块 B eq 18-19, 模块 C eq 24-26, 模块 D)
# ======================================================================

def sdpa(q, k, v, mask, scale):
    """torch's textbook attention in float64 on the CPU; q [nh, T, c]."""
    return F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                          torch.from_numpy(v), attn_mask=torch.from_numpy(mask),
                                          scale=scale).numpy()


def test_sparse_m1_full_topk_no_window_is_causal_mqa():
    """m = 1, k >= n, n_win = 0, no sink: dense causal MQA with K = V = C^Comp."""
    n, nh, c = 14, 3, 8
    q, C = rnd(50, n, nh, c), rnd(51, n, c)
    pos = np.arange(n)
    idx = O.topk_select(rnd(52, n, n), 1, pos, n + 3)
    scale = 1 / np.sqrt(c)
    out = O.sparse_mqa(q, C, idx, C[:0], 0, 0, pos, None, scale)
    causal = np.tril(np.ones((n, n), dtype=bool))
    ref = sdpa(q.transpose(1, 0, 2), np.broadcast_to(C, (nh, n, c)).copy(),
               np.broadcast_to(C, (nh, n, c)).copy(), causal, scale)
    assert np.allclose(out, ref.transpose(1, 0, 2), atol=1e-12)


def test_sparse_no_selection_is_banded_causal_over_window():
    n, nh, c, nw = 20, 2, 6, 5
    q, R = rnd(53, n, nh, c), rnd(54, n, c)
    pos = np.arange(n)
    idx = -np.ones((n, 4), dtype=np.int32)
    out = O.sparse_mqa(q, R[:3], idx, R, 0, nw, pos, None, 0.7)
    u = np.arange(n)
    band = (u[None, :] <= pos[:, None]) & (u[None, :] > pos[:, None] - nw)
    ref = sdpa(q.transpose(1, 0, 2), np.broadcast_to(R, (nh, n, c)).copy(),
               np.broadcast_to(R, (nh, n, c)).copy(), band, 0.7)
    assert np.allclose(out, ref.transpose(1, 0, 2), atol=1e-12)


def test_hca_window_covering_sequence_is_masked_dense():
    """n_win >= n: HCA equals dense attention over [C^Comp ; raw] with the
    visibility mask of the compressed entries and the causal mask of raw rows."""
    n, mp, nh, c = 24, 4, 3, 8
    q, raw = rnd(55, n, nh, c), rnd(56, n, c)
    comp = rnd(57, n // mp, c)
    pos = np.arange(n)
    scale = 0.3
    out = O.hca_dense(q, comp, mp, raw, 0, n, pos, None, scale)
    keys = np.concatenate([comp, raw])
    s = np.arange(n // mp)
    vis = mp * (s[None, :] + 1) <= pos[:, None] + 1
    causal = np.arange(n)[None, :] <= pos[:, None]
    mask = np.concatenate([vis, causal], axis=1)
    K = np.broadcast_to(keys, (nh,) + keys.shape).copy()
    ref = sdpa(q.transpose(1, 0, 2), K, K, mask, scale)
    assert np.allclose(out, ref.transpose(1, 0, 2), atol=1e-12)


def test_hca_short_sequence_sees_no_block():
    n, mp, nh, c = 6, 8, 2, 4
    q, raw = rnd(58, n, nh, c), rnd(59, n, c)
    out = O.hca_dense(q, rnd(60, 3, c), mp, raw, 0, 16, np.arange(n), None, 0.5)
    causal = np.tril(np.ones((n, n), dtype=bool))
    K = np.broadcast_to(raw, (nh, n, c)).copy()
    assert np.allclose(out, sdpa(q.transpose(1, 0, 2), K, K, causal, 0.5).transpose(1, 0, 2))


def test_sink_is_an_extra_zero_value_key():
    """digest 模块 D: exp(z'_h) joins the denominator only -- the same as one
    more key with logit z'_h and a zero value vector."""
    nh, N, c = 4, 7, 5
    q, keys, z = rnd(61, nh, c), rnd(62, N, c), rnd(63, nh) * 2
    scale = 0.4
    out = O.core_attention(q, keys, scale, z)
    qa = np.concatenate([q * scale, np.ones((nh, 1))], axis=1)[:, None, :]     # [nh, 1, c+1]
    Ka = np.zeros((nh, N + 1, c + 1))
    Ka[:, :N, :c] = keys
    Ka[:, N, c] = z
    Va = np.zeros((nh, N + 1, c))
    Va[:, :N] = keys
    ref = sdpa(qa, Ka, Va, np.ones((1, N + 1), dtype=bool), 1.0)[:, 0]
    assert np.allclose(out, ref, atol=1e-12)


def test_attention_closed_forms():
    nh, N, c = 3, 9, 6
    keys, z = rnd(64, N, c), rnd(65, nh)
    mean = keys.mean(axis=0)
    out = O.core_attention(np.zeros((nh, c)), keys, 1.0, None)
    assert np.allclose(out, mean[None])
    out = O.core_attention(np.zeros((nh, c)), keys, 1.0, z)
    assert np.allclose(out, mean[None] * (N / (N + np.exp(z)))[:, None])
    one = keys[:1]
    assert np.allclose(O.core_attention(rnd(66, nh, c), one, 1.0, None), np.broadcast_to(one, (nh, c)))
    assert np.array_equal(O.core_attention(rnd(67, nh, c), keys[:0], 1.0, z), np.zeros((nh, c)))


def test_sparse_index_permutation_and_padding_invariance():
    S, nh, c = 30, 4, 6
    q, C, R = rnd(68, 1, nh, c), rnd(69, S, c), rnd(70, 50, c)
    idx = np.array([[3, 17, 29, 0, 8]], dtype=np.int32)
    a = O.sparse_mqa(q, C, idx, R, 10, 8, [40], rnd(71, nh), 0.3)
    b = O.sparse_mqa(q, C, idx[:, ::-1].copy(), R, 10, 8, [40], rnd(71, nh), 0.3)
    c2 = O.sparse_mqa(q, C, np.array([[3, -1, 17, 29, -1, 0, 8, -1]], np.int32), R, 10, 8, [40],
                      rnd(71, nh), 0.3)
    assert np.allclose(a, b, atol=1e-13) and np.allclose(a, c2, atol=1e-13)


def test_window_must_be_covered():
    with pytest.raises(ValueError):
        O.window_rows(np.zeros((10, 2)), 5, 4, 7)      # needs position 4
    with pytest.raises(ValueError):
        O.window_rows(np.zeros((10, 2)), 0, 4, 10)     # position 10 not stored
    assert O.window_rows(np.zeros((10, 2)), 0, 4, 2).shape == (3, 2)
