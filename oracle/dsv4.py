"""Plain float64 CPU oracle for the DeepSeek-V4 CSA / HCA attention hot path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark use this module.  It shares no code with the HIP
library (no kernels, headers, tables or helpers) and never imports it.

Sources (cited by page title and section; the pages print no code):
  digest = ai-papers-daily page "DeepSeek-V4: Towards Highly Efficient
           Million-Token Context Intelligence", 子模块实现 / 模块 B (CSA,
           eq 9-19), 模块 C (HCA, eq 20-26), 模块 D (sliding window, sink,
           partial RoPE, Q/KV norm), 模块 F (precisions, on-disk cache).
  blog   = jsqmd page "DeepSeek V4大模型算法解析", 二、核心算法, 1.) CSA
           (第一阶段 compression, 第二阶段 lightning indexer, 第三阶段 shared-KV
           MQA) and 2.) HCA.

Readings where the pages are silent or garbled (each is listed, with its
reason, in the design notes of the repository):
  R1  pooling weights are a per-channel softmax over the 2m logits Z+B of an
      entry (Z and B are n x c and m x c, so a softmax per channel is the only
      shape-consistent reading of the digest's row-softmax over 2m elements);
  R2  entry i pools a-rows [m*i, m*i+m) and b-rows [m*(i-1), m*i) (blog,
      第一阶段 window description, reconstructed from its garbled superscripts);
  R3  entry 0 has no b-rows: its softmax runs over its m a-logits only;
  R4  an incomplete final block emits no entry (digest 模块 F: an incomplete
      tail block is recomputed later);
  R5  entry s is visible to the query at absolute position p iff m*(s+1) <= p+1
      (every pooled token is at or before p);
  R6  the indexer keys come from the same compressor at width c_I with their
      own weights and biases;
  R7  the index score has no scale; R8 head weights may be negative;
  R9  top-k ties go to the lower index; fewer than k visible -> all visible,
      padded with -1; order (score desc, index asc);
  R10 compressed entries and window entries are concatenated, no de-dup;
  R11 the window of query p is the uncompressed rows at positions
      [max(0, p-n_win+1), p];
  R13 a selected entry is both key and value (K = V);
  R14 logits are scale * q.k with the scale passed in (1/sqrt(c) by default);
  R15 the sink adds exp(z'_h) to the softmax denominator only;
  R16 an empty key set gives a zero output;
  R19b the FP4 indexer rounds each query head q^I[t, h] to MXFP4 (blocks of
      32 consecutive c_I dims, the key encoder) before eq 16; the keys are the
      stored MXFP4 rows, decoded;
  R19c the FP8-query indexer rounds each query head to MXFP8 instead: blocks
      of 32 consecutive c_I dims share the E8M0 scale 2^(floor(log2 amax) - 8),
      elements rounded to E4M3 (nearest even, saturating at 448);
  R32 RMSNorm (digest 模块 D, Q/KV normalisation) of a vector x of width c is
      x / sqrt(mean(x^2) + eps) * gamma, eps = 1e-6, gamma per channel; it is
      applied to every query head and to every KV row that core attention
      reads (compressed entries and window rows);
  R33 partial RoPE (digest 模块 D) rotates the last 64 dims as interleaved
      pairs (2j, 2j + 1), j < 32, by the angle pos * theta^(-2j/64),
      theta = 10000, after the RMSNorm;
  R34 positions: a query at its own position p; a window row at its token's
      position; a compressed entry at the position of the newest token it
      pools, m (s + 1) - 1 (HCA: m' (s + 1) - 1);
  R35 the attention output's last 64 dims are rotated by -p (the query's
      position), so that they carry relative positions;
  R36 the low-rank latent c^Q and the grouped projection's intermediate z are
      activations: stored in bf16 between their two products (as the
      library's GEMMs do), the products themselves exact;
  R37 output group j (of g) takes the consecutive heads [j nh/g, (j+1) nh/g),
      flattened head-major, and fills columns [j d_g, (j+1) d_g) of z.
"""
import numpy as np

from . import codecs as _codecs


# ---------------------------------------------------------------------------
# compressors
# ---------------------------------------------------------------------------

def softmax_pool(C_rows, Z_rows, B_rows):
    """Per-channel softmax pooling of one entry.

    C_rows, Z_rows, B_rows: [r, c].  Returns (pooled [c], weights [r, c]);
    the weights of each channel are softmax over the r logits Z+B
    (digest 模块 B eq 11, 模块 C eq 22; blog 第一阶段: the Softmax normalises
    the 2m elements so that they sum to 1)."""
    L = Z_rows + B_rows
    L = L - L.max(axis=0, keepdims=True)
    E = np.exp(L)
    Wt = E / E.sum(axis=0, keepdims=True)
    return (Wt * C_rows).sum(axis=0), Wt


def csa_compress(H, W, B_ab, m, block0=0, n_left=0):
    """CSA token-level compressor (digest 模块 B eq 9-12; blog 第一阶段).

    H:     [n_left + n, d] hidden states; row n_left is the token at absolute
           position m*block0; the n_left rows before it are left context
           (needed for the b-window of the first entry when block0 > 0).
    W:     [4c, d] = rows of W^{aKV} | W^{bKV} | W^{aZ} | W^{bZ} (so C = H W^T).
    B_ab:  [2, m, c] = B^a, B^b position biases.
    Returns (comp [n//m, c], raw [n, c]); raw are the uncompressed C^a rows of
    the chunk, the sliding-window KV source for CSA.
    """
    H = np.asarray(H, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    B_ab = np.asarray(B_ab, dtype=np.float64)
    c = W.shape[0] // 4
    n = H.shape[0] - n_left
    Ca = H @ W[0 * c:1 * c].T          # eq 9-10: two KV streams and two weight streams
    Cb = H @ W[1 * c:2 * c].T
    Za = H @ W[2 * c:3 * c].T
    Zb = H @ W[3 * c:4 * c].T
    Ba, Bb = B_ab[0], B_ab[1]
    n_ent = n // m                     # R4
    comp = np.zeros((n_ent, c))
    for i in range(n_ent):
        a0 = n_left + m * i            # local row of token m*(block0+i)
        rows_C = [Ca[a0:a0 + m]]
        rows_Z = [Za[a0:a0 + m]]
        rows_B = [Ba]
        if block0 + i >= 1:            # R3: entry 0 has no b-window
            b0 = a0 - m
            if b0 < 0:
                raise ValueError("b-window of entry %d needs %d rows of left context" % (block0 + i, m))
            rows_C.append(Cb[b0:b0 + m])
            rows_Z.append(Zb[b0:b0 + m])
            rows_B.append(Bb)
        comp[i], _ = softmax_pool(np.concatenate(rows_C), np.concatenate(rows_Z),
                                  np.concatenate(rows_B))
    return comp, Ca[n_left:n_left + n]


def csa_pool_weights(H, W, B_ab, m, i, block0=0, n_left=0):
    """The 2m (or m) pooling weights of local entry i, [r, c] (for invariants)."""
    H = np.asarray(H, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    c = W.shape[0] // 4
    Za = H @ W[2 * c:3 * c].T
    Zb = H @ W[3 * c:4 * c].T
    a0 = n_left + m * i
    Z = [Za[a0:a0 + m]]
    B = [B_ab[0]]
    if block0 + i >= 1:
        Z.append(Zb[a0 - m:a0])
        B.append(B_ab[1])
    _, Wt = softmax_pool(np.zeros((len(Z) * m, c)), np.concatenate(Z), np.concatenate(B))
    return Wt


def hca_compress(H, W, B, m_prime):
    """HCA compressor (digest 模块 C eq 20-23; blog 2.) HCA: same as CSA with a
    larger ratio m' and no overlap).

    H: [n, d]; W: [2c, d] = W^{KV} | W^{Z}; B: [m', c].
    Returns (comp [n//m', c], raw C [n, c])."""
    H = np.asarray(H, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    c = W.shape[0] // 2
    C = H @ W[:c].T
    Z = H @ W[c:].T
    n_ent = H.shape[0] // m_prime
    comp = np.zeros((n_ent, c))
    for i in range(n_ent):
        r = slice(m_prime * i, m_prime * (i + 1))
        comp[i], _ = softmax_pool(C[r], Z[r], B)
    return comp, C


# ---------------------------------------------------------------------------
# lightning indexer and top-k selector
# ---------------------------------------------------------------------------

def visible_count(p, m, S):
    """Number of compressed entries visible at position p (R5): entries
    s with m*(s+1) <= p+1, i.e. s < floor((p+1)/m), capped at S."""
    return int(min(S, max(0, (p + 1) // m)))


def indexer_score(qI, wI, KI, m, q_pos):
    """Index scores (digest 模块 B eq 16; blog 第二阶段):
    I[t, s] = sum_h wI[t, h] * ReLU(qI[t, h] . KI[s]) for visible s, -inf
    otherwise (R5, R7, R8).

    qI [nq, hI, cI], wI [nq, hI], KI [S, cI], q_pos [nq] absolute positions."""
    qI = np.asarray(qI, dtype=np.float64)
    wI = np.asarray(wI, dtype=np.float64)
    KI = np.asarray(KI, dtype=np.float64)
    nq, S = qI.shape[0], KI.shape[0]
    out = np.full((nq, S), -np.inf)
    for t in range(nq):
        nv = visible_count(int(q_pos[t]), m, S)
        dots = qI[t] @ KI[:nv].T              # [hI, nv]
        out[t, :nv] = wI[t] @ np.maximum(dots, 0.0)
    return out


def indexer_score_fp4q(qI, wI, KI, m, q_pos):
    """Index scores of the FP4 lightning indexer (digest 模块 F: the indexer's
    attention runs in FP4): eq 16 over the query heads rounded to MXFP4 along
    c_I (R19b).  qI [nq, hI, cI] with cI a multiple of 32; KI [S, cI] are the
    decoded MXFP4 keys."""
    qI = np.asarray(qI, dtype=np.float64)
    codes, scales = _codecs.mxfp4_encode(qI)
    return indexer_score(_codecs.mxfp4_decode(codes, scales), wI, KI, m, q_pos)


def indexer_score_fp8q(qI, wI, KI, m, q_pos):
    """Index scores with the queries in FP8 (NEXT-3's FP8 variant of the
    digest 模块 F FP4 indexer): eq 16 over the query heads rounded to MXFP8
    along c_I (R19c); KI [S, cI] are the decoded MXFP4 keys."""
    qI = np.asarray(qI, dtype=np.float64)
    codes, scales = _codecs.mxfp8_encode(qI)
    return indexer_score(_codecs.mxfp8_decode(codes, scales), wI, KI, m, q_pos)


def rmsnorm(x, gamma, eps=1e-6):
    """RMSNorm over the last axis (digest 模块 D; R32)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(gamma, dtype=np.float64)


def rope_last(x, pos, theta=10000.0, rope_dims=64):
    """Partial RoPE (digest 模块 D; R33): the last rope_dims dims of x [..., c]
    rotated as interleaved pairs (2j, 2j+1) by pos * theta^(-2j/rope_dims);
    pos broadcasts over the leading axes of x (one position per row)."""
    x = np.array(x, dtype=np.float64)
    c = x.shape[-1]
    pos = np.asarray(pos, dtype=np.float64)[..., None]        # [..., 1]
    j = np.arange(rope_dims // 2, dtype=np.float64)
    ang = pos * theta ** (-2.0 * j / rope_dims)               # [..., rope_dims/2]
    cs, sn = np.cos(ang), np.sin(ang)
    a = x[..., c - rope_dims::2].copy()
    b = x[..., c - rope_dims + 1::2].copy()
    x[..., c - rope_dims::2] = a * cs - b * sn
    x[..., c - rope_dims + 1::2] = a * sn + b * cs
    return x


def q_norm_rope(q, gamma, q_pos, eps=1e-6, theta=10000.0, rope_dims=64):
    """Query preparation (R32, R33): q [nq, nh, c] at positions q_pos [nq]."""
    y = rmsnorm(q, gamma, eps)
    return rope_last(y, np.asarray(q_pos, dtype=np.float64)[:, None] * np.ones(y.shape[:-1]), theta, rope_dims)


def kv_norm_rope(rows, gamma, pos, eps=1e-6, theta=10000.0, rope_dims=64):
    """KV row preparation (R32-R34): rows [n, c] at positions pos [n]."""
    return rope_last(rmsnorm(rows, gamma, eps), pos, theta, rope_dims)


def entry_positions(m, s0, n):
    """Positions of compressed entries s0 .. s0+n-1 (R34): the newest pooled token."""
    return m * (np.arange(s0, s0 + n, dtype=np.int64) + 1) - 1


def out_rope(o, q_pos, theta=10000.0, rope_dims=64):
    """Output rotation (R35): o [nq, nh, c], last dims rotated by -q_pos."""
    o = np.asarray(o, dtype=np.float64)
    return rope_last(o, -np.asarray(q_pos, dtype=np.float64)[:, None] * np.ones(o.shape[:-1]), theta, rope_dims)


def _bf16(x):
    return _codecs.bf16_round(x)


def query_proj(h, W_DQ, W_UQ, W_IUQ, W_w, nh, c, hI, cI):
    """Low-rank query path (digest 模块 B eq 13-15, 18; R36): c^Q = h W^DQ^T
    (stored bf16), q = c^Q W^UQ^T, q^I = c^Q W^IUQ^T, w^I = h W^w^T.
    h [n, d]; weights in the [out, in] layout.  Returns q [n, nh, c],
    q^I [n, hI, cI] (both before their bf16 storage rounding) and w^I [n, hI]."""
    h = np.asarray(h, dtype=np.float64)
    cq = _bf16(h @ np.asarray(W_DQ, dtype=np.float64).T)
    q = cq @ np.asarray(W_UQ, dtype=np.float64).T
    qI = cq @ np.asarray(W_IUQ, dtype=np.float64).T
    wI = h @ np.asarray(W_w, dtype=np.float64).T
    n = h.shape[0]
    return q.reshape(n, nh, c), qI.reshape(n, hI, cI), wI


def output_proj(o, W_O1, W_O2, g):
    """Grouped output projection (digest 模块 B, grouped output projection; R36,
    R37): the nh head outputs o [n, nh, c] form g groups of consecutive heads;
    group j's flattened rows are projected by W_O1[j] [d_g, (nh/g) c] into
    columns [j d_g, (j+1) d_g) of z (stored bf16), then out = z W_O2^T with
    W_O2 [d, g d_g]."""
    o = np.asarray(o, dtype=np.float64)
    n, nh, c = o.shape
    W_O1 = np.asarray(W_O1, dtype=np.float64)
    hg = nh // g
    z = np.concatenate([o[:, j * hg:(j + 1) * hg, :].reshape(n, hg * c) @ W_O1[j].T for j in range(g)], axis=1)
    return _bf16(z) @ np.asarray(W_O2, dtype=np.float64).T


def topk_select(I, m, q_pos, k):
    """Top-k selector (digest 模块 B eq 17; blog 第二阶段 Top-k稀疏选择) with
    the tie and padding rule R9.  I [nq, S] -> idx [nq, k] int32."""
    I = np.asarray(I, dtype=np.float64)
    nq, S = I.shape
    idx = np.full((nq, k), -1, dtype=np.int32)
    for t in range(nq):
        nv = visible_count(int(q_pos[t]), m, S)
        s = np.arange(nv)
        order = np.lexsort((s, -I[t, :nv]))    # primary: score desc; secondary: index asc
        take = order[:min(k, nv)]
        idx[t, :take.size] = take
    return idx


# ---------------------------------------------------------------------------
# core attention
# ---------------------------------------------------------------------------

def core_attention(q, keys, scale, sink=None):
    """Shared-KV MQA of one query (digest 模块 B eq 18-19, 模块 D attention sink).

    q [nh, c]; keys [N, c] are both keys and values (R13).
    o_h = sum_x e^{l_x - M} k_x / (sum_x e^{l_x - M} + e^{z'_h - M}),
    l_x = scale * q_h . k_x, M = max(max_x l_x, z'_h)."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    nh, c = q.shape
    if keys.shape[0] == 0:
        return np.zeros((nh, c))                       # R16
    L = scale * (q @ keys.T)                            # [nh, N]
    M = L.max(axis=1)
    if sink is not None:
        z = np.asarray(sink, dtype=np.float64)
        M = np.maximum(M, z)
    E = np.exp(L - M[:, None])
    den = E.sum(axis=1)
    if sink is not None:
        den = den + np.exp(z - M)                      # R15
    return (E @ keys) / den[:, None]


def window_rows(kv_win, win_pos0, n_win, p):
    """Uncompressed rows of the sliding window of query p (R11), in position order."""
    if n_win <= 0:
        return kv_win[:0]
    lo = max(0, p - n_win + 1)
    if lo < win_pos0 or p >= win_pos0 + kv_win.shape[0]:
        raise ValueError("window of position %d not covered by kv_win" % p)
    return kv_win[lo - win_pos0:p - win_pos0 + 1]


def sparse_mqa(q, kv_comp, idx, kv_win, win_pos0, n_win, q_pos, sink, scale):
    """CSA core: shared-KV MQA over the selected compressed entries plus the
    sliding window (digest 模块 B eq 18-19, 模块 D sliding-window branch;
    blog 第三阶段; R10).  Index entries outside [0, S) are padding.

    q [nq, nh, c]; kv_comp [S, c]; idx [nq, k]; kv_win [W, c]."""
    q = np.asarray(q, dtype=np.float64)
    kv_comp = np.asarray(kv_comp, dtype=np.float64)
    kv_win = np.asarray(kv_win, dtype=np.float64)
    S = kv_comp.shape[0]
    out = np.zeros(q.shape)
    for t in range(q.shape[0]):
        sel = [int(s) for s in idx[t] if 0 <= s < S]
        keys = np.concatenate([kv_comp[sel], window_rows(kv_win, win_pos0, n_win, int(q_pos[t]))])
        out[t] = core_attention(q[t], keys, scale, sink)
    return out


def hca_dense(q, kv_comp, m_prime, kv_win, win_pos0, n_win, q_pos, sink, scale):
    """HCA core: shared-KV MQA over every visible compressed entry plus the
    window (digest 模块 C eq 24-26; blog 2.) HCA 融合与计算)."""
    q = np.asarray(q, dtype=np.float64)
    kv_comp = np.asarray(kv_comp, dtype=np.float64)
    kv_win = np.asarray(kv_win, dtype=np.float64)
    S = kv_comp.shape[0]
    out = np.zeros(q.shape)
    for t in range(q.shape[0]):
        p = int(q_pos[t])
        nv = visible_count(p, m_prime, S)
        keys = np.concatenate([kv_comp[:nv], window_rows(kv_win, win_pos0, n_win, p)])
        out[t] = core_attention(q[t], keys, scale, sink)
    return out
