"""Streaming (decode-time) cache maintenance for the CSA / HCA compressors and
the sliding window, in float64.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark use this module.  It shares no code with the HIP
library and never imports it.

Sources (by page title and section; the pages print no code):
  digest = ai-papers-daily page "DeepSeek-V4: Towards Highly Efficient
           Million-Token Context Intelligence", 模块 B (CSA compressor, eq 9-12),
           模块 C (HCA compressor, eq 20-23), 模块 F (on-disk KV cache: every
           compressed entry is persisted and a shared prefix reuses them as
           they are, while the incomplete trailing block is computed again;
           the uncompressed sliding-window rows, about eight times the size of
           the compressed ones, are either cached in full, checkpointed
           periodically or not cached at all and recomputed).
  blog   = jsqmd page "DeepSeek V4大模型算法解析", 二、核心算法 1.) CSA 第一阶段
           (each entry pools its own block and, through the second weight
           stream, the block before it).

Readings (each also listed in the design notes of the repository):
  R38 a streaming compressor keeps the projected rows [C^a | C^b | Z^a | Z^b]
      (CSA) or [C | Z] (HCA) of the tokens it still needs: for CSA those of
      the current block and of the previous one (the b-window of the next
      entry), for HCA those of the current block.  The token at position
      m (s + 1) - 1 completes block s and emits entry s, pooled over the same
      rows, biases and softmax as the batch compressor (R1-R3);
  R39 resuming after a persisted prefix of P tokens replays the hidden states
      of positions [tail_start(P), P): HCA from m floor(P/m); CSA from
      m (floor(P/m) - 1), since the next entry's b-window is the last complete
      block.  The replay writes no entry below floor(P/m): those are the
      persisted ones;
  R40 the window ring of capacity Wr >= n_win keeps the row of position x at
      rows x mod Wr and x mod Wr + Wr (a mirrored ring of 2 Wr rows), so the
      rows of positions [p - n_win + 1, p] are consecutive, starting at row
      x - pos0 with pos0 = floor((p - Wr + 1) / Wr) * Wr.  The attention calls
      read such a ring as an ordinary window buffer of 2 Wr rows whose row 0
      holds position pos0.
"""
import numpy as np

from .dsv4 import softmax_pool


def stream_init(overlap, m):
    """Empty compressor state: overlap 1 for CSA (b-window), 0 for HCA."""
    return {"overlap": int(overlap), "m": int(m), "rows": {}}


def stream_feed(state, H_new, pos0, W, B, emit_from=0):
    """Feed the hidden states of positions pos0 .. pos0 + n - 1, in order (R38).

    H_new: [n, d].  W: [4c, d] = W^{aKV} | W^{bKV} | W^{aZ} | W^{bZ} (CSA) or
    [2c, d] = W^{KV} | W^{Z} (HCA).  B: [2, m, c] (CSA: B^a, B^b) or [m, c].
    Returns (entries, raw): entries maps s -> pooled entry [c] for every block
    completed in this call with s >= emit_from; raw [n, c] are the C^a (CSA)
    or C (HCA) rows of the fed tokens, the sliding-window source."""
    H_new = np.asarray(H_new, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    m, ov = state["m"], state["overlap"]
    c = W.shape[0] // (4 if ov else 2)
    P = H_new @ W.T                         # eq 9-10 / eq 20-21, row by row
    rows = state["rows"]
    entries = {}
    for i in range(P.shape[0]):
        x = pos0 + i
        rows[x] = P[i]
        if (x + 1) % m:
            continue
        s = (x + 1) // m - 1                # this token completes block s
        if s >= emit_from:                  # persisted entries below emit_from only keep their rows
            need = list(range(m * s, m * s + m))
            need_b = list(range(m * (s - 1), m * s)) if ov and s >= 1 else []
            missing = [p for p in need + need_b if p not in rows]
            if missing:
                raise ValueError("entry %d needs the rows of positions %d..%d" % (s, missing[0], missing[-1]))
            if ov:
                C_rows = [rows[p][0:c] for p in need] + [rows[p][c:2 * c] for p in need_b]
                Z_rows = [rows[p][2 * c:3 * c] for p in need] + [rows[p][3 * c:4 * c] for p in need_b]
                B_rows = np.concatenate([B[0]] + ([B[1]] if need_b else []))
            else:
                C_rows = [rows[p][0:c] for p in need]
                Z_rows = [rows[p][c:2 * c] for p in need]
                B_rows = B
            entries[s], _ = softmax_pool(np.stack(C_rows), np.stack(Z_rows), B_rows)
        keep_from = m * s if ov else x + 1   # CSA keeps block s for the next b-window
        for p in [p for p in rows if p < keep_from]:
            del rows[p]
    return entries, P[:, :c].copy()


def tail_start(P, m, overlap):
    """First position whose hidden state a resume after P persisted tokens
    replays (R39)."""
    nb = P // m
    if overlap:
        return m * max(nb - 1, 0)
    return m * nb


def resume(H, P, W, B, m, overlap):
    """State after a persisted prefix of P tokens, rebuilt by replaying the
    tail of H (rows are positions 0 ..); emits nothing (R39)."""
    st = stream_init(overlap, m)
    t0 = tail_start(P, m, overlap)
    ent, _ = stream_feed(st, np.asarray(H)[t0:P], t0, W, B, emit_from=P // m)
    assert not ent
    return st


def ring_pos0(p, ring_w):
    """Position held by row 0 of a mirrored ring whose newest row is p (R40)."""
    return ((p - ring_w + 1) // ring_w) * ring_w


def ring_append(ring, ring_w, rows, pos0):
    """Write rows [n, c] of positions pos0 .. into the ring [2 ring_w, c] (R40)."""
    for i in range(len(rows)):
        x = pos0 + i
        ring[x % ring_w] = rows[i]
        ring[x % ring_w + ring_w] = rows[i]


def ring_window(ring, ring_w, p, n_win):
    """Rows of positions [max(0, p - n_win + 1), p] read from the ring as a
    window buffer whose row 0 holds ring_pos0(p, ring_w) (R40)."""
    assert n_win <= ring_w
    p0 = ring_pos0(p, ring_w)
    lo = max(0, p - n_win + 1)
    return ring[lo - p0:p + 1 - p0]
