"""Interleaved CSA + HCA layer pair over one chunk of a chunked prefill.

DeepSeek-V4 digest (ai-papers-daily page "DeepSeek-V4: Towards Highly
Efficient Million-Token Context Intelligence"): CSA and HCA layers alternate
layer by layer (核心思路); the compressed entries of a prefix are cached and
reused, and only complete blocks produce entries (模块 F).

One `step()` enqueues, on one stream, the calls of the pair:
  the three compressors of the chunk in one launch over the same tiles of H
       (CSA KV appended to the KV cache with its window rows to the CSA window
       buffer, CSA indexer keys appended, HCA entries appended with their
       window rows to the HCA window buffer), the KV rows RMS-normalised and
       rotated at their positions in the same call (kv_nr=dict(gamma=, eps=,
       theta=, rope_dims=); None: stored as compressed);
  CSA: index scores and top-k in one call (the score rows are not stored),
       sparse MQA;
  HCA: dense MQA;
  both attention calls rotate the output's RoPE dims back by the query
  position in their store (out_rope=(theta, rope_dims); None: not rotated).
indexer() and topk() are the same selection as two calls through a stored
score buffer.
Buffers are torch tensors owned by the caller; nothing is allocated in step().
"""
import math

from . import _lib as L


class PairLayer:
    def __init__(self, *, H, n_left, m, mp, c, cI, hI, nh, k, n_win,
                 W_kv, B_kv, W_ki, B_ki, W_hca, B_hca,
                 kv_cache, S0, ki_codes, ki_scales, hca_cache, Sh0, kv_win, hca_win, win_pos0,
                 q, qI, wI, q_hca, sink, sink_hca, q_pos0, kv_layout, key_layout, out_rope=(10000.0, 64),
                 kv_nr=dict(gamma=None, eps=1e-6, theta=10000.0, rope_dims=64)):
        import torch
        self.__dict__.update(locals())
        del self.__dict__["self"]
        self.n = H.shape[0] - n_left
        n = self.n
        self.scale = 1.0 / math.sqrt(c)
        self.S = S0 + n // m
        self.Sh = Sh0 + n // mp
        dev = H.device
        self.scores = torch.empty((1, n, self.S), dtype=torch.float32, device=dev)
        self.idx = torch.empty((1, n, k), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(q)
        self.out_hca = torch.empty_like(q_hca)
        nb = L.topk_workspace_size(1, n, self.S, k)
        self.ws_topk = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        nb = L.indexer_topk_workspace_size(L.BF16 if qI.dtype != torch.float32 else L.F32, key_layout, 1, n, hI, cI,
                                           self.S, k)
        self.ws_it = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        nb = max(L.attn_workspace_size(False, 1, n, nh, c, k + n_win),
                 L.attn_workspace_size(True, 1, n, nh, c, self.Sh + n_win))
        self.ws_attn = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        if kv_nr is not None:
            self.nr_kv = L.norm_rope(kv_nr["gamma"], eps=kv_nr["eps"], theta=kv_nr["theta"],
                                     rope_dims=kv_nr["rope_dims"])
            self.nr_hca = L.norm_rope(kv_nr["gamma"], eps=kv_nr["eps"], theta=kv_nr["theta"],
                                      rope_dims=kv_nr["rope_dims"])
            nb = L.compress_chunk_nr_workspace_size(n, m, c, mp, c)
            self.ws_nr = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        else:
            self.nr_kv = self.nr_hca = self.ws_nr = None
        rb = L.row_bytes(kv_layout, c)
        self.kv_new = kv_cache[S0:self.S]
        self.kv_win_new = kv_win[n_win:n_win + n]
        self.ki_new = ki_codes[S0:self.S]
        self.ki_sc_new = ki_scales[S0:self.S]
        self.hca_new = hca_cache[Sh0:self.Sh]
        self.hca_win_new = hca_win[n_win:n_win + n]
        assert kv_cache.shape[1] == rb and hca_cache.shape[1] == rb

    # the CSA and HCA halves are separate so that each can be timed
    def csa_compress(self, stream=None):
        L.csa_compress(self.H, self.W_kv, self.B_kv, self.m, self.c, self.kv_new, self.kv_layout,
                       n_left=self.n_left, block0=self.S0, raw_out=self.kv_win_new, raw_layout=self.kv_layout,
                       stream=stream)
        L.csa_compress(self.H, self.W_ki, self.B_ki, self.m, self.cI, self.ki_new, self.key_layout,
                       n_left=self.n_left, block0=self.S0, comp_scales=self.ki_sc_new, stream=stream)

    def compress(self, stream=None):
        """All three compressors of the chunk in one call (dsv4_compress_chunk, or
        dsv4_compress_chunk_nr with the KV norm + RoPE)."""
        kv = L.compressor(self.W_kv, self.B_kv, self.c, self.kv_new, self.kv_layout, raw_out=self.kv_win_new,
                          raw_layout=self.kv_layout)
        ki = L.compressor(self.W_ki, self.B_ki, self.cI, self.ki_new, self.key_layout, comp_scales=self.ki_sc_new)
        hc = L.compressor(self.W_hca, self.B_hca, self.c, self.hca_new, self.kv_layout, raw_out=self.hca_win_new,
                          raw_layout=self.kv_layout)
        L.compress_chunk(self.H, self.m, n_left=self.n_left, block0=self.S0, csa_kv=kv, csa_keys=ki,
                         m_prime=self.mp, hca=hc, kv_nr=self.nr_kv, hca_nr=self.nr_hca, ws=self.ws_nr, stream=stream)

    def indexer(self, stream=None):
        L.indexer_score(self.qI.view(1, self.n, self.hI, self.cI), self.wI.view(1, self.n, self.hI),
                        self.ki_codes[:self.S].view(1, self.S, -1), self.key_layout, self.m, self.q_pos0,
                        self.scores, k_scales=self.ki_scales[:self.S].view(1, self.S, -1), stream=stream)

    def indexer_fp4q(self, stream=None):
        """The same scores with the query heads rounded to MXFP4 (FP4 indexer)."""
        L.indexer_score_fp4q(self.qI.view(1, self.n, self.hI, self.cI), self.wI.view(1, self.n, self.hI),
                             self.ki_codes[:self.S].view(1, self.S, -1), self.ki_scales[:self.S].view(1, self.S, -1),
                             self.m, self.q_pos0, self.scores, stream=stream)

    def indexer_fp8q(self, stream=None):
        """The same scores with the query heads rounded to MXFP8."""
        L.indexer_score_fp8q(self.qI.view(1, self.n, self.hI, self.cI), self.wI.view(1, self.n, self.hI),
                             self.ki_codes[:self.S].view(1, self.S, -1), self.ki_scales[:self.S].view(1, self.S, -1),
                             self.m, self.q_pos0, self.scores, stream=stream)

    def topk(self, stream=None):
        L.topk_select(self.scores, self.m, self.q_pos0, self.k, self.idx, self.ws_topk, stream=stream)

    def indexer_topk(self, stream=None):
        """idx as indexer() then topk() give it, in one call (dsv4_indexer_topk)."""
        L.indexer_topk(self.qI.view(1, self.n, self.hI, self.cI), self.wI.view(1, self.n, self.hI),
                       self.ki_codes[:self.S].view(1, self.S, -1), self.key_layout, self.m, self.q_pos0, self.k,
                       self.idx, self.ws_it, k_scales=self.ki_scales[:self.S].view(1, self.S, -1), stream=stream)

    def sparse(self, stream=None):
        L.sparse_mqa_fwd(self.q.view(1, self.n, self.nh, self.c), self.kv_cache[:self.S].view(1, self.S, -1),
                         self.kv_layout, self.idx, self.kv_win.view(1, -1, self.kv_win.shape[1]), self.win_pos0,
                         self.n_win, self.q_pos0, self.sink, self.scale, self.out.view(1, self.n, self.nh, self.c),
                         self.ws_attn, out_rope=self.out_rope, stream=stream)

    def hca_compress(self, stream=None):
        L.hca_compress(self.H[self.n_left:], self.W_hca, self.B_hca, self.mp, self.c, self.hca_new,
                       self.kv_layout, raw_out=self.hca_win_new, raw_layout=self.kv_layout, stream=stream)

    def hca_dense(self, stream=None):
        L.hca_dense_fwd(self.q_hca.view(1, self.n, self.nh, self.c), self.hca_cache[:self.Sh].view(1, self.Sh, -1),
                        self.kv_layout, self.mp, self.hca_win.view(1, -1, self.hca_win.shape[1]), self.win_pos0,
                        self.n_win, self.q_pos0, self.sink_hca, self.scale,
                        self.out_hca.view(1, self.n, self.nh, self.c), self.ws_attn, out_rope=self.out_rope,
                        stream=stream)

    def step(self, stream=None):
        self.compress(stream)
        self.indexer_topk(stream)
        self.sparse(stream)
        self.hca_dense(stream)


def pair_from_arrays(inp, device="cuda"):
    """Upload the stored numpy arrays of a layer-pair workload and build the layer."""
    import numpy as np
    import torch

    def up(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(x).to(device)

    cfg = inp["cfg"]
    n, nh, c, hI, cI = cfg["n"], cfg["nh"], cfg["c"], cfg["hI"], cfg["cI"]
    return PairLayer(
        H=up(inp["H"]), n_left=cfg["n_left"], m=cfg["m"], mp=cfg["mp"], c=c, cI=cI, hI=hI, nh=nh, k=cfg["k"],
        n_win=cfg["n_win"], W_kv=up(inp["W_kv"]), B_kv=up(inp["B_kv"]), W_ki=up(inp["W_ki"]),
        B_ki=up(inp["B_ki"]), W_hca=up(inp["W_hca"]), B_hca=up(inp["B_hca"]),
        kv_cache=up(inp["kv_cache"]), S0=inp["S0"], ki_codes=up(inp["ki_codes"]), ki_scales=up(inp["ki_scales"]),
        hca_cache=up(inp["hca_cache"]), Sh0=inp["Sh0"], kv_win=up(inp["kv_win"]), hca_win=up(inp["hca_win"]),
        win_pos0=[int(inp["win_pos0"][0])], q=up(inp["q"]).view(n, nh, c), qI=up(inp["qI"]), wI=up(inp["wI"]),
        q_hca=up(inp["q_hca"]).view(n, nh, c), sink=up(inp["sink"]), sink_hca=up(inp["sink_hca"]),
        q_pos0=[int(inp["q_pos0"][0])], kv_layout=cfg["kv_layout"], key_layout=cfg["key_layout"])
