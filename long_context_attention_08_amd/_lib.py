"""ctypes binding of libdsv4attn (the C ABI in include/dsv4attn.h).

Argument marshalling only: every step runs in the HIP library.  torch supplies
device memory and the current stream.  Importing this module raises if the
built library is missing -- there is no fallback.  DSV4ATTN_LIB names another
build of the same C ABI to load instead (the host-sanitizer tests use it).
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("DSV4ATTN_LIB") or os.path.join(HERE, "libdsv4attn.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
ROW_F32, ROW_BF16, ROW_FP8_ROPE_BF16, ROW_MXFP4 = 0, 1, 2, 3

EXPORTS = [
    "dsv4_row_bytes", "dsv4_csa_compress", "dsv4_hca_compress", "dsv4_compress_chunk", "dsv4_compress_chunk_nr",
    "dsv4_compress_chunk_nr_workspace_size", "dsv4_indexer_score",
    "dsv4_indexer_score_fp4q", "dsv4_indexer_score_fp8q", "dsv4_indexer_topk_workspace_size", "dsv4_indexer_topk", "dsv4_q_norm_rope", "dsv4_kv_norm_rope", "dsv4_out_rope",
    "dsv4_gemm_bf16_nt", "dsv4_query_proj_workspace_size", "dsv4_query_proj",
    "dsv4_output_proj_workspace_size", "dsv4_output_proj",
    "dsv4_topk_workspace_size", "dsv4_topk_select", "dsv4_topk_select_noalloc", "dsv4_attn_workspace_size", "dsv4_attn_plan",
    "dsv4_sparse_mqa_fwd", "dsv4_hca_dense_fwd", "dsv4_sparse_mqa_fwd_rope", "dsv4_hca_dense_fwd_rope",
    "dsv4_status_string", "dsv4_last_error",
    "dsv4_stream_state_bytes", "dsv4_stream_state_reset", "dsv4_stream_workspace_size",
    "dsv4_stream_compress", "dsv4_swa_ring_pos0",
]

if not os.path.exists(LIB_PATH):
    raise ImportError("libdsv4attn.so is not built (run `python long_context_attention_08_amd/build.py`)")

lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _int, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_P64 = ctypes.POINTER(ctypes.c_int64)


def _sig(name, res, args):
    f = getattr(lib, name)
    f.restype = res
    f.argtypes = args
    return f


_sig("dsv4_row_bytes", _sz, [_int, _int])
_sig("dsv4_status_string", ctypes.c_char_p, [_int])
_sig("dsv4_last_error", ctypes.c_char_p, [])
_sig("dsv4_csa_compress", _int, [_vp, _i64, _i64, _i64, _int, _vp, _vp, _int, _int, _i64,
                                 _vp, _vp, _int, _vp, _int, _vp])
class Compressor(ctypes.Structure):
    """dsv4_compressor_t: one compressor's weights and outputs for dsv4_compress_chunk."""
    _fields_ = [("W", _vp), ("bias", _vp), ("c", _int), ("comp_out", _vp), ("comp_scales", _vp),
                ("comp_layout", _int), ("raw_out", _vp), ("raw_layout", _int)]


_sig("dsv4_compress_chunk", _int, [_vp, _i64, _i64, _i64, _int, _int, _i64, ctypes.POINTER(Compressor),
                                   ctypes.POINTER(Compressor), _int, ctypes.POINTER(Compressor), _vp])
_sig("dsv4_hca_compress", _int, [_vp, _i64, _i64, _int, _vp, _vp, _int, _int, _vp, _vp, _int, _vp, _int, _vp])
_sig("dsv4_indexer_score", _int, [_vp, _int, _vp, _vp, _vp, _int, _i64, _i64, _int, _int, _i64, _int,
                                  _P64, _vp, _vp])
_sig("dsv4_indexer_score_fp4q", _int, [_vp, _int, _vp, _vp, _vp, _i64, _i64, _int, _int, _i64, _int,
                                       _P64, _vp, _vp])
_sig("dsv4_indexer_score_fp8q", _int, [_vp, _int, _vp, _vp, _vp, _i64, _i64, _int, _int, _i64, _int,
                                       _P64, _vp, _vp])
_sig("dsv4_q_norm_rope", _int, [_vp, _int, _vp, _i64, _i64, _int, _int, _vp, _f32, _f32, _int, _P64, _vp])
_sig("dsv4_kv_norm_rope", _int, [_vp, _int, _i64, _i64, _int, _vp, _f32, _f32, _int, _P64, _i64, _vp, _int, _vp])
_sig("dsv4_out_rope", _int, [_vp, _int, _i64, _i64, _int, _int, _f32, _int, _P64, _vp])
_sig("dsv4_gemm_bf16_nt", _int, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _int, _i64, _i64, _i64, _i64, _i64,
                                 _i64, _vp])
_sig("dsv4_query_proj_workspace_size", _sz, [_i64, _int])
_sig("dsv4_query_proj", _int, [_vp, _i64, _int, _vp, _int, _vp, _int, _int, _vp, _int, _int, _vp,
                               _vp, _vp, _vp, _vp, _sz, _vp])
_sig("dsv4_output_proj_workspace_size", _sz, [_i64, _int, _int])
_sig("dsv4_output_proj", _int, [_vp, _i64, _int, _int, _int, _int, _vp, _vp, _int, _vp, _vp, _sz, _vp])
_sig("dsv4_indexer_topk_workspace_size", _sz, [_int, _int, _i64, _i64, _int, _int, _i64, _int])
_sig("dsv4_indexer_topk", _int, [_vp, _int, _vp, _vp, _vp, _int, _i64, _i64, _int, _int, _i64, _int, _P64, _int,
                                 _vp, _vp, _sz, _vp])
_sig("dsv4_topk_workspace_size", _sz, [_i64, _i64, _i64, _int])
_sig("dsv4_topk_select", _int, [_vp, _i64, _i64, _i64, _int, _P64, _int, _vp, _vp, _sz, _vp])
_sig("dsv4_topk_select_noalloc", _int, [_vp, _i64, _i64, _i64, _int, _P64, _int, _vp, _vp])
_sig("dsv4_attn_workspace_size", _sz, [_int, _i64, _i64, _int, _int, _i64])


class AttnPlan(ctypes.Structure):
    """dsv4_attn_plan_t"""
    _fields_ = [("path", ctypes.c_int), ("queries_per_block", ctypes.c_int), ("splits", ctypes.c_int),
                ("split_slots", ctypes.c_int), ("workspace_bytes", ctypes.c_size_t)]


_sig("dsv4_attn_plan", _int, [_int, _int, _int, _i64, _i64, _int, _int, _i64, _int, _int, _int, _P64,
                              ctypes.POINTER(AttnPlan)])
_sig("dsv4_sparse_mqa_fwd", _int, [_vp, _int, _i64, _i64, _int, _int, _vp, _int, _i64, _vp, _int,
                                   _vp, _i64, _P64, _int, _P64, _vp, _f32, _vp, _vp, _sz, _vp])
_sig("dsv4_hca_dense_fwd", _int, [_vp, _int, _i64, _i64, _int, _int, _vp, _int, _i64, _int,
                                  _vp, _i64, _P64, _int, _P64, _vp, _f32, _vp, _vp, _sz, _vp])
_sig("dsv4_sparse_mqa_fwd_rope", _int, [_vp, _int, _i64, _i64, _int, _int, _vp, _int, _i64, _vp, _int,
                                        _vp, _i64, _P64, _int, _P64, _vp, _f32, _f32, _int, _vp, _vp, _sz, _vp])
_sig("dsv4_hca_dense_fwd_rope", _int, [_vp, _int, _i64, _i64, _int, _int, _vp, _int, _i64, _int,
                                       _vp, _i64, _P64, _int, _P64, _vp, _f32, _f32, _int, _vp, _vp, _sz, _vp])



class NormRope(ctypes.Structure):
    """dsv4_norm_rope_t: RMSNorm and partial RoPE before a row is packed."""
    _fields_ = [("norm", _int), ("gamma", _vp), ("eps", _f32), ("rope_dims", _int), ("theta", _f32)]


_sig("dsv4_compress_chunk_nr_workspace_size", _sz, [_i64, _int, _int, _int, _int])
_sig("dsv4_compress_chunk_nr", _int, [_vp, _i64, _i64, _i64, _int, _int, _i64, ctypes.POINTER(Compressor),
                                      ctypes.POINTER(Compressor), _int, ctypes.POINTER(Compressor),
                                      ctypes.POINTER(NormRope), ctypes.POINTER(NormRope), _vp, _sz, _vp])


_sig("dsv4_stream_state_bytes", _sz, [_int, _int, _int])
_sig("dsv4_stream_state_reset", _int, [_vp, _i64, _int, _int, _int, _vp])
_sig("dsv4_stream_workspace_size", _sz, [_i64, _i64, _i64, _int, _int])
_sig("dsv4_stream_compress", _int, [_vp, _i64, _i64, _i64, _int, _vp, _vp, _int, _int, _int, _P64, _P64, _vp,
                                    _vp, _vp, _int, _i64, _vp, _i64, _int, ctypes.POINTER(NormRope),
                                    _vp, _sz, _vp])
_sig("dsv4_swa_ring_pos0", _i64, [_i64, _i64])

class Dsv4Error(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s (%d): %s" % (lib.dsv4_status_string(status).decode(), status, msg))
        self.status = status


def _check(status):
    if status != OK:
        raise Dsv4Error(status, lib.dsv4_last_error().decode())


def row_bytes(layout, c):
    return int(lib.dsv4_row_bytes(layout, c))


def _torch():
    import torch
    return torch


def _ptr(t):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor, got %r" % type(t))
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _act(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("activations must be float32 or bfloat16, got %s" % t.dtype)


def _host_i64(vals):
    arr = (ctypes.c_int64 * max(1, len(vals)))(*[int(v) for v in vals])
    return arr


def _stream(stream):
    if stream is not None:
        return stream
    return _torch().cuda.current_stream().cuda_stream


# --------------------------------------------------------------------- the six calls

def csa_compress(H, W, bias_ab, m, c, comp_out, comp_layout, *, n_left=0, block0=0,
                 comp_scales=None, raw_out=None, raw_layout=ROW_F32, stream=None):
    """CSA compressor.  H [n_left + n, d]; W [4c, d]; bias_ab [2, m, c] float32."""
    n = H.shape[0] - n_left
    _check(lib.dsv4_csa_compress(_ptr(H), n_left, n, H.shape[1], _act(H), _ptr(W), _ptr(bias_ab), m, c,
                                 block0, _ptr(comp_out), _ptr(comp_scales), comp_layout,
                                 _ptr(raw_out), raw_layout, _stream(stream)))


def hca_compress(H, W, bias, m_prime, c, comp_out, comp_layout, *, comp_scales=None,
                 raw_out=None, raw_layout=ROW_F32, stream=None):
    """HCA compressor.  H [n, d]; W [2c, d]; bias [m', c] float32."""
    _check(lib.dsv4_hca_compress(_ptr(H), H.shape[0], H.shape[1], _act(H), _ptr(W), _ptr(bias), m_prime, c,
                                 _ptr(comp_out), _ptr(comp_scales), comp_layout, _ptr(raw_out), raw_layout,
                                 _stream(stream)))


def compressor(W, bias, c, comp_out, comp_layout, *, comp_scales=None, raw_out=None, raw_layout=ROW_F32):
    """One compressor's weights and outputs for compress_chunk."""
    return Compressor(_ptr(W), _ptr(bias), c, _ptr(comp_out), _ptr(comp_scales), comp_layout, _ptr(raw_out),
                      raw_layout)


def norm_rope(gamma=None, *, eps=1e-6, theta=10000.0, rope_dims=64, norm=True):
    """A dsv4_norm_rope_t: RMSNorm (times gamma [c] float32, or 1) and RoPE of the last rope_dims dims."""
    return NormRope(1 if norm else 0, _ptr(gamma), eps, rope_dims, theta)


def compress_chunk(H, m, *, n_left=0, block0=0, csa_kv=None, csa_keys=None, m_prime=128, hca=None,
                   kv_nr=None, hca_nr=None, ws=None, stream=None):
    """The CSA KV, CSA indexer-key and HCA compressors of one chunk in one call
    (each a `compressor(...)` or None).  H [n_left + n, d]; the HCA compressor
    takes rows n_left.. of H.  kv_nr / hca_nr (`norm_rope(...)`): the KV RMSNorm
    and RoPE of the CSA KV / HCA rows in the same call (dsv4_compress_chunk_nr,
    ws of compress_chunk_nr_workspace_size)."""
    n = H.shape[0] - n_left
    ref = lambda j: ctypes.byref(j) if j is not None else None
    if kv_nr is None and hca_nr is None:
        _check(lib.dsv4_compress_chunk(_ptr(H), n_left, n, H.shape[1], _act(H), m, block0, ref(csa_kv),
                                       ref(csa_keys), m_prime, ref(hca), _stream(stream)))
        return
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.dsv4_compress_chunk_nr(_ptr(H), n_left, n, H.shape[1], _act(H), m, block0, ref(csa_kv),
                                      ref(csa_keys), m_prime, ref(hca), ref(kv_nr), ref(hca_nr), _ptr(ws), wsb,
                                      _stream(stream)))


def compress_chunk_nr_workspace_size(n, m, c_kv, m_prime, c_hca):
    return int(lib.dsv4_compress_chunk_nr_workspace_size(n, m, c_kv, m_prime, c_hca))


def indexer_score(qI, wI, keys, k_layout, m, q_pos0, scores, *, k_scales=None, S=None, stream=None):
    """Index scores.  qI [B, nq, hI, cI]; wI [B, nq, hI]; keys [B, S, ...]; scores [B, nq, S]."""
    B, nq, hI, cI = qI.shape
    S = scores.shape[2] if S is None else S
    _check(lib.dsv4_indexer_score(_ptr(qI), _act(qI), _ptr(wI), _ptr(keys), _ptr(k_scales), k_layout,
                                  B, nq, hI, cI, S, m, _host_i64(q_pos0), _ptr(scores), _stream(stream)))


def indexer_score_fp4q(qI, wI, k_codes, k_scales, m, q_pos0, scores, *, S=None, stream=None):
    """Index scores of the FP4 indexer: the query heads are rounded to MXFP4 and
    multiplied with the MXFP4 keys.  qI [B, nq, hI, cI]; wI [B, nq, hI];
    k_codes [B, S, cI/2]; k_scales [B, S, cI/32]; scores [B, nq, S]."""
    B, nq, hI, cI = qI.shape
    S = scores.shape[2] if S is None else S
    _check(lib.dsv4_indexer_score_fp4q(_ptr(qI), _act(qI), _ptr(wI), _ptr(k_codes), _ptr(k_scales),
                                       B, nq, hI, cI, S, m, _host_i64(q_pos0), _ptr(scores),
                                       _stream(stream)))



def indexer_score_fp8q(qI, wI, k_codes, k_scales, m, q_pos0, scores, *, S=None, stream=None):
    """Index scores with FP8 queries: the query heads are rounded to MXFP8
    (E4M3) and multiplied with the MXFP4 keys.  Shapes as indexer_score_fp4q."""
    B, nq, hI, cI = qI.shape
    S = scores.shape[2] if S is None else S
    _check(lib.dsv4_indexer_score_fp8q(_ptr(qI), _act(qI), _ptr(wI), _ptr(k_codes), _ptr(k_scales),
                                       B, nq, hI, cI, S, m, _host_i64(q_pos0), _ptr(scores),
                                       _stream(stream)))

def indexer_topk_workspace_size(q_dtype, k_layout, B, nq, hI, cI, S, k):
    return int(lib.dsv4_indexer_topk_workspace_size(q_dtype, k_layout, B, nq, hI, cI, S, k))


def indexer_topk(qI, wI, keys, k_layout, m, q_pos0, k, idx_out, ws=None, *, k_scales=None, S=None, stream=None):
    """Index scores and top-k in one call.  qI [B, nq, hI, cI]; wI [B, nq, hI];
    keys [B, S, ...]; idx_out [B, nq, k] int32 (what indexer_score followed by
    topk_select would give)."""
    B, nq, hI, cI = qI.shape
    S = keys.shape[1] if S is None else S
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.dsv4_indexer_topk(_ptr(qI), _act(qI), _ptr(wI), _ptr(keys), _ptr(k_scales), k_layout,
                                 B, nq, hI, cI, S, m, _host_i64(q_pos0), k, _ptr(idx_out), _ptr(ws), wsb,
                                 _stream(stream)))


def topk_workspace_size(B, nq, S, k):
    return int(lib.dsv4_topk_workspace_size(B, nq, S, k))


def topk_select(scores, m, q_pos0, k, idx_out, ws=None, *, stream=None):
    """Top-k.  scores [B, nq, S] float32 -> idx_out [B, nq, k] int32."""
    B, nq, S = scores.shape
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.dsv4_topk_select(_ptr(scores), B, nq, S, m, _host_i64(q_pos0), k, _ptr(idx_out),
                                _ptr(ws), wsb, _stream(stream)))


def topk_select_noalloc(scores, m, q_pos0, k, idx_out, *, stream=None):
    """Top-k without a workspace argument (the library's static per-GPU array)."""
    B, nq, S = scores.shape
    _check(lib.dsv4_topk_select_noalloc(_ptr(scores), B, nq, S, m, _host_i64(q_pos0), k, _ptr(idx_out),
                                        _stream(stream)))


def attn_workspace_size(dense, B, nq, nh, c, max_keys):
    return int(lib.dsv4_attn_workspace_size(1 if dense else 0, B, nq, nh, c, max_keys))


def attn_plan(dense, q_dtype, kv_layout, B, nq, nh, c, S, k, m_prime, n_win, q_pos0):
    """The launch plan of an attention call (host only): an AttnPlan."""
    p = AttnPlan()
    _check(lib.dsv4_attn_plan(1 if dense else 0, q_dtype, kv_layout, B, nq, nh, c, S, k, m_prime, n_win,
                              _host_i64(q_pos0), ctypes.byref(p)))
    return p


def sparse_mqa_fwd(q, kv_comp, kv_layout, idx, kv_win, win_pos0, n_win, q_pos0, sink, scale, out,
                   ws=None, *, S=None, W=None, out_rope=None, stream=None):
    """CSA core.  q [B, nq, nh, c]; kv_comp [B, S, row]; idx [B, nq, k]; kv_win [B, W, row].
    out_rope=(theta, rope_dims): the output rotation in the same launch
    (dsv4_sparse_mqa_fwd_rope)."""
    B, nq, nh, c = q.shape
    S = kv_comp.shape[1] if S is None else S
    W = kv_win.shape[1] if (W is None and kv_win is not None) else (W or 0)
    k = idx.shape[2] if idx is not None else 0
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    head = (_ptr(q), _act(q), B, nq, nh, c, _ptr(kv_comp), kv_layout, S, _ptr(idx), k, _ptr(kv_win), W,
            _host_i64(win_pos0), n_win, _host_i64(q_pos0), _ptr(sink), float(scale))
    tail = (_ptr(out), _ptr(ws), wsb, _stream(stream))
    if out_rope is None:
        _check(lib.dsv4_sparse_mqa_fwd(*head, *tail))
    else:
        _check(lib.dsv4_sparse_mqa_fwd_rope(*head, float(out_rope[0]), int(out_rope[1]), *tail))


def hca_dense_fwd(q, kv_comp, kv_layout, m_prime, kv_win, win_pos0, n_win, q_pos0, sink, scale, out,
                  ws=None, *, S=None, W=None, out_rope=None, stream=None):
    """HCA core.  q [B, nq, nh, c]; kv_comp [B, S, row]; kv_win [B, W, row].
    out_rope=(theta, rope_dims): the output rotation in the same launch
    (dsv4_hca_dense_fwd_rope)."""
    B, nq, nh, c = q.shape
    S = kv_comp.shape[1] if S is None else S
    W = kv_win.shape[1] if (W is None and kv_win is not None) else (W or 0)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    head = (_ptr(q), _act(q), B, nq, nh, c, _ptr(kv_comp), kv_layout, S, m_prime, _ptr(kv_win), W,
            _host_i64(win_pos0), n_win, _host_i64(q_pos0), _ptr(sink), float(scale))
    tail = (_ptr(out), _ptr(ws), wsb, _stream(stream))
    if out_rope is None:
        _check(lib.dsv4_hca_dense_fwd(*head, *tail))
    else:
        _check(lib.dsv4_hca_dense_fwd_rope(*head, float(out_rope[0]), int(out_rope[1]), *tail))


# --------------------------------------------------------------------- Q/KV norm and RoPE

def q_norm_rope(q, gamma, q_pos0, *, out=None, eps=1e-6, theta=10000.0, rope_dims=64, stream=None):
    """RMSNorm and partial RoPE of every query head.  q [B, nq, nh, c] float32 or
    bfloat16; out (default: q, in place) of the same shape and dtype."""
    B, nq, nh, c = q.shape
    out = q if out is None else out
    _check(lib.dsv4_q_norm_rope(_ptr(q), _act(q), _ptr(out), B, nq, nh, c, _ptr(gamma), eps, theta, rope_dims,
                                _host_i64(q_pos0), _stream(stream)))


def kv_norm_rope(rows, in_layout, c, gamma, pos0, pos_stride, rows_out, out_layout, *, eps=1e-6,
                 theta=10000.0, rope_dims=64, stream=None):
    """RMSNorm, partial RoPE and the storage pack of KV rows.  rows [B, n, row]
    in in_layout; row i of batch entry b sits at pos0[b] + pos_stride * i;
    rows_out [B, n, row] in out_layout."""
    B, n = rows.shape[0], rows.shape[1]
    _check(lib.dsv4_kv_norm_rope(_ptr(rows), in_layout, B, n, c, _ptr(gamma), eps, theta, rope_dims,
                                 _host_i64(pos0), pos_stride, _ptr(rows_out), out_layout, _stream(stream)))


def out_rope(o, q_pos0, *, theta=10000.0, rope_dims=64, stream=None):
    """Rotate the last rope_dims dims of every output row o[b, t, h] (in place)
    by -(q_pos0[b] + t)."""
    B, nq, nh, c = o.shape
    _check(lib.dsv4_out_rope(_ptr(o), _act(o), B, nq, nh, c, theta, rope_dims, _host_i64(q_pos0), _stream(stream)))


# --------------------------------------------------------------------- projections (bf16 GEMM)

def gemm_bf16_nt(A, B, C, *, batch=1, stride_a=0, stride_b=0, stride_c=0, M=None, N=None, K=None,
                 lda=None, ldb=None, ldc=None, stream=None):
    """C = A B^T (bf16 A [M, K], B [N, K], fp32 accumulation, C bf16 or fp32).
    Shapes default to the tensors' last two dims."""
    M = A.shape[-2] if M is None else M
    K = A.shape[-1] if K is None else K
    N = B.shape[-2] if N is None else N
    lda = A.shape[-1] if lda is None else lda
    ldb = B.shape[-1] if ldb is None else ldb
    ldc = C.shape[-1] if ldc is None else ldc
    _check(lib.dsv4_gemm_bf16_nt(_ptr(A), lda, stride_a, _ptr(B), ldb, stride_b, _ptr(C), _act(C), ldc, stride_c,
                                 M, N, K, batch, _stream(stream)))


def query_proj_workspace_size(n, d_c):
    return int(lib.dsv4_query_proj_workspace_size(n, d_c))


def query_proj(h, W_DQ, W_UQ, W_IUQ, W_w, *, nh, c, hI, cI, q=None, qI=None, wI=None, ws=None, stream=None):
    """Low-rank query path: q = (h W_DQ^T) W_UQ^T, q^I = (h W_DQ^T) W_IUQ^T,
    w^I = h W_w^T.  h [n, d] bf16; outputs q [n, nh, c] / q^I [n, hI, cI] bf16,
    w^I [n, hI] fp32 (any of them None to skip)."""
    n, d = h.shape
    d_c = W_DQ.shape[0]
    _check(lib.dsv4_query_proj(_ptr(h), n, d, _ptr(W_DQ), d_c, _ptr(W_UQ), nh, c, _ptr(W_IUQ), hI, cI, _ptr(W_w),
                               _ptr(q), _ptr(qI), _ptr(wI), _ptr(ws), 0 if ws is None else ws.numel(),
                               _stream(stream)))


def output_proj_workspace_size(n, g, d_g):
    return int(lib.dsv4_output_proj_workspace_size(n, g, d_g))


def output_proj(o, W_O1, W_O2, out, *, g, ws=None, stream=None):
    """Grouped output projection: o [n, nh, c] bf16, W_O1 [g, d_g, (nh/g) c],
    W_O2 [d, g d_g], out [n, d] bf16."""
    n, nh, c = o.shape
    d_g = W_O1.shape[1]
    d = W_O2.shape[0]
    _check(lib.dsv4_output_proj(_ptr(o), n, nh, c, g, d_g, _ptr(W_O1), _ptr(W_O2), d, _ptr(out), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(stream)))


# --------------------------------------------------------------------- streaming cache maintenance (decode)

def stream_state_bytes(overlap, m, c):
    """Bytes of one sequence's streaming-compressor state."""
    return int(lib.dsv4_stream_state_bytes(overlap, m, c))


def stream_state_reset(state, B, overlap, m, c, *, stream=None):
    """Mark every slot of B sequences' states empty."""
    _check(lib.dsv4_stream_state_reset(_ptr(state), B, overlap, m, c, _stream(stream)))


def stream_workspace_size(B, n_new, d, overlap, c):
    return int(lib.dsv4_stream_workspace_size(B, n_new, d, overlap, c))


def swa_ring_pos0(p_last, ring_w):
    """Window-buffer position of row 0 of a mirrored ring whose newest row is p_last."""
    return int(lib.dsv4_swa_ring_pos0(p_last, ring_w))


def stream_compress(H, W, bias, overlap, m, c, pos0, state, *, emit_from=None, cache=None, cache_scales=None,
                    cache_layout=ROW_F32, S=None, ring=None, ring_w=0, ring_layout=ROW_F32, norm=False,
                    gamma=None, eps=1e-6, rope_dims=0, theta=10000.0, ws=None, stream=None):
    """Feed H [B, n_new, d] (positions pos0[b] + i) to the streaming compressor
    of B sequences: completed entries go to cache [B, S, row], every token's
    C^a / C row to the mirrored ring [B, 2 ring_w, row]."""
    B, n_new, d = H.shape
    if S is None:
        S = cache.shape[1] if cache is not None else 0
    nr = None
    if norm or rope_dims:
        nr = ctypes.byref(NormRope(1 if norm else 0, _ptr(gamma), eps, rope_dims, theta))
    if ws is None:
        nbytes = stream_workspace_size(B, n_new, d, overlap, c)
        ws = _torch().empty(max(16, nbytes), dtype=_torch().uint8, device=H.device)
    _check(lib.dsv4_stream_compress(_ptr(H), B, n_new, d, _act(H), _ptr(W), _ptr(bias), overlap, m, c,
                                    _host_i64(pos0), None if emit_from is None else _host_i64(emit_from),
                                    _ptr(state), _ptr(cache), _ptr(cache_scales), cache_layout, S,
                                    _ptr(ring), ring_w, ring_layout, nr, _ptr(ws), ws.numel(), _stream(stream)))
