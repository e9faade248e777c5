"""Hybrid compressed attention (CSA + HCA) on MI355X: Python binding.

This module only marshals arguments to the C ABI of ``liblac.so``
(``include/lac.h``): tensor pointers, sizes, host position arrays and the
current HIP stream.  Every step of the computation runs in the library's
gfx950 kernels; if the library is missing, importing this module fails.

Tensors are PyTorch tensors on the GPU, row-major.  Storage formats follow
the tensor dtype: ``torch.float32`` -> LAC_F32, ``torch.bfloat16`` ->
LAC_BF16, ``torch.uint8`` rows of ``(D - r) + 2r`` bytes -> the mixed FP8
E4M3 / bf16 KV format.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Union

import torch

__all__ = [
    "LacError", "csa_compress", "hca_compress", "indexer_topk", "indexer_topk_workspace_size",
    "indexer_topk_noalloc", "indexer_topk_prepare", "LAC_TOPK_PREPARED",
    "csa_attend", "hca_attend", "attend_workspace_size", "time_next_launch", "lib",
    "grouped_output_projection", "grouped_projection_workspace_size",
    "LAC_F32", "LAC_BF16", "LAC_KV_E4M3_ROPE_BF16", "LAC_E4M3", "LAC_MXFP4", "LAC_SCORE_BF16",
    "LAC_Q_E4M3", "KERNELS",
    "CallList", "group",
]

LAC_F32, LAC_BF16, LAC_KV_E4M3_ROPE_BF16, LAC_E4M3, LAC_MXFP4 = 0, 1, 2, 3, 4
LAC_SCORE_BF16 = 0x100      # dtype flag of indexer_topk: scores rounded to bf16
LAC_TOPK_PREPARED = 0x200   # dtype flag of indexer_topk: workspace zeroed by indexer_topk_prepare
LAC_Q_E4M3 = 0x400          # dtype flag of indexer_topk: E4M3 q_idx with MXFP4 keys
KERNELS = {"compress": 0, "indexer_score": 1, "topk": 2, "attend": 3, "combine": 4,
           "project": 5}
STATUS = {0: "LAC_OK", 1: "LAC_ERR_INVALID", 2: "LAC_ERR_UNSUPPORTED", 3: "LAC_ERR_WORKSPACE",
          4: "LAC_ERR_DEVICE"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblac.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")

lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_COMPRESS_ARGS = [_vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _i64, _i64,
                  _i64, _vp]
lib.csa_compress.argtypes = _COMPRESS_ARGS
lib.csa_compress.restype = _i32
lib.hca_compress.argtypes = _COMPRESS_ARGS
lib.hca_compress.restype = _i32
lib.csa_compress_overlap.argtypes = _COMPRESS_ARGS[:9] + [_i32] + _COMPRESS_ARGS[9:]
lib.csa_compress_overlap.restype = _i32
_COMPRESS_NORM_ARGS = _COMPRESS_ARGS[:-1] + [_vp, _f32, _vp]
lib.csa_compress_rmsnorm.argtypes = _COMPRESS_NORM_ARGS
lib.csa_compress_rmsnorm.restype = _i32
lib.hca_compress_rmsnorm.argtypes = _COMPRESS_NORM_ARGS
lib.hca_compress_rmsnorm.restype = _i32
lib.indexer_topk_workspace_size.argtypes = [_i32, _i32, _i32, _i32]
lib.indexer_topk_workspace_size.restype = _sz
lib.indexer_topk.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _i32,
                             _vp, _vp, _vp, _sz, _vp]
lib.indexer_topk.restype = _i32
lib.indexer_topk_noalloc.argtypes = lib.indexer_topk.argtypes[:-3] + [_vp]
lib.indexer_topk_noalloc.restype = _i32
lib.indexer_topk_prepare.argtypes = [_i32, _i32, _i32, _i32, _vp, _sz, _vp]
lib.indexer_topk_prepare.restype = _i32
lib.attend_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]
lib.attend_workspace_size.restype = _sz
lib.csa_attend.argtypes = [_vp, _i32, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _i32, _vp, _f32,
                           _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _sz, _vp]
lib.csa_attend.restype = _i32
lib.hca_attend.argtypes = [_vp, _i32, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _f32, _i32,
                           _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _sz, _vp]
lib.hca_attend.restype = _i32
lib.csa_attend_rmsnorm.argtypes = lib.csa_attend.argtypes[:-1] + [_vp, _f32, _vp]
lib.csa_attend_rmsnorm.restype = _i32
lib.hca_attend_rmsnorm.argtypes = lib.hca_attend.argtypes[:-1] + [_vp, _f32, _vp]
lib.hca_attend_rmsnorm.restype = _i32
lib.grouped_projection_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
lib.grouped_projection_workspace_size.restype = _sz
lib.grouped_output_projection.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp,
                                          _vp, _sz, _vp]
lib.grouped_output_projection.restype = _i32
lib.lac_last_error.argtypes = []
lib.lac_last_error.restype = ctypes.c_char_p
lib.lac_time_next_launch.argtypes = [_i32, _vp, _vp]
lib.lac_time_next_launch.restype = _i32
lib.lac_group_begin.argtypes = [_vp]
lib.lac_group_begin.restype = _i32
lib.lac_group_end.argtypes = [_vp]
lib.lac_group_end.restype = _i32
lib.lac_group_cancel.argtypes = []
lib.lac_group_cancel.restype = _i32


class LacError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def _check(status: int):
    if status != 0:
        raise LacError(status, lib.lac_last_error().decode())


_recording = None


def _call(fn, args):
    """Calls an entry point, or (inside a CallList) records the call with its
    arguments already converted to their ctypes types."""
    if _recording is None:
        _check(fn(*args))
        return
    conv = []
    for t, a in zip(fn.argtypes, args):
        conv.append(a if a is None or isinstance(a, (ctypes.Array, ctypes._SimpleCData)) else t(a))
    _recording.append((fn, tuple(conv)))


class CallList:
    """A fixed sequence of library calls, marshalled once and replayed.

    Inside ``with CallList() as cl:`` the entry points of this module record
    their C call (tensor pointers, sizes, positions, the current stream)
    instead of making it; ``cl.run()`` then makes the recorded calls in order,
    one ctypes call each, with the same validation in the library.  The
    tensors behind the recorded pointers must stay alive and in place."""

    def __init__(self):
        self.calls = []

    def __enter__(self):
        global _recording
        _recording = self.calls
        return self

    def __exit__(self, *exc):
        global _recording
        _recording = None
        return False

    def run(self):
        for fn, a in self.calls:
            st = fn(*a)
            if st:
                raise LacError(st, lib.lac_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _positions(p: Union[None, int, Sequence[int], torch.Tensor], B: int):
    if p is None:
        return None
    if isinstance(p, torch.Tensor):
        p = p.tolist()
    if isinstance(p, int):
        p = [p] * B
    if len(p) != B:
        raise ValueError(f"expected {B} positions, got {len(p)}")
    return (ctypes.c_int64 * B)(*[int(v) for v in p])


def _fmt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LAC_F32
    if t.dtype == torch.bfloat16:
        return LAC_BF16
    if t.dtype == torch.uint8:
        return LAC_KV_E4M3_ROPE_BF16
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _rows(t: torch.Tensor, what: str):
    """Batch stride in rows of a [B, rows, width] tensor whose rows are dense."""
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{what} must be [B, rows, width] with dense rows")
    return t.stride(0) // t.shape[2]


def _need_dense(t: Optional[torch.Tensor], what: str):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


_group_keep = None


def _workspace(ws: Optional[torch.Tensor], need: int, device) -> torch.Tensor:
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        if _group_keep is not None:      # used only when the group is enqueued
            _group_keep.append(ws)
    return ws


class group:
    """Launch group (lac_group_begin / lac_group_end in include/lac.h).

    Inside ``with group():`` the compress and attention calls on the stream
    are validated and recorded; leaving the block enqueues them together
    (compress calls in one launch, attention calls in one attention launch
    and one combine launch).  The calls must be independent: none reads what
    another writes.  Workspaces the wrappers allocate are kept alive until
    the group is enqueued.  An exception inside the block cancels the group
    (nothing recorded is enqueued).  Inside a CallList the begin and end
    calls are recorded like any other."""

    def __init__(self, stream=None):
        self.stream = stream

    def __enter__(self):
        global _group_keep
        _call(lib.lac_group_begin, (_stream(self.stream),))
        if _recording is None:
            _group_keep = []
        return self

    def __exit__(self, exc_type, *rest):
        global _group_keep
        try:
            if exc_type is None:
                _call(lib.lac_group_end, (_stream(self.stream),))
            elif _recording is None:
                lib.lac_group_cancel()
        finally:
            _group_keep = None
        return False


# ---------------------------------------------------------------- compress
def _norm_gain(gain, D, device):
    if gain is None:
        return None
    if gain.dtype != torch.float32 or gain.numel() != D or gain.device != device or not gain.is_contiguous():
        raise TypeError(f"norm gain must be a contiguous float32 tensor of {D} values on {device}")
    return gain


def _out_fmt(out, D, rope_dims):
    """Compressed-row format of `out`: uint8 rows of D/2 + D/32 bytes with no
    rotated dims are MXFP4 (include/lac.h); other uint8 rows the mixed format."""
    if out.dtype == torch.uint8 and rope_dims == 0 and D % 32 == 0 and \
            out.shape[-1] == D // 2 + D // 32:
        return LAC_MXFP4
    return _fmt(out)


def _compress(fn, fn_norm, raw_kv, logits, out, m, rope_dims, rope_theta, pos0, T, norm_gain,
              norm_eps, stream):
    B, _, D = raw_kv.shape
    T = raw_kv.shape[1] if T is None else T
    if logits.dtype != raw_kv.dtype:
        raise TypeError("raw_kv and logits must share a dtype")
    args = [_ptr(raw_kv), _ptr(logits), _fmt(raw_kv), _ptr(out), _out_fmt(out, D, rope_dims), B, T, D, m,
            rope_dims, rope_theta, _positions(pos0, B), _rows(raw_kv, "raw_kv"),
            _rows(logits, "logits"), _rows(out, "out")]
    gain = _norm_gain(norm_gain, D, raw_kv.device)
    if gain is None:
        _call(fn, (*args, _stream(stream)))
    else:
        _call(fn_norm, (*args, _ptr(gain), norm_eps, _stream(stream)))
    return out


def csa_compress(raw_kv, logits, out, m=4, rope_dims=64, rope_theta=10000.0, pos0=None, T=None,
                 stream=None, norm_gain=None, norm_eps=1e-6, overlap=0):
    """Pool every m raw KV rows into one entry (see include/lac.h); with
    norm_gain [D] float32, each entry is RMSNorm'd before its rotation
    (csa_compress_rmsnorm).  With overlap > 0 each entry also pools the
    `overlap` tokens before its block (csa_compress_overlap): raw_kv and
    logits then start min(overlap, pos0[b]) rows before the first block, and
    T defaults to the rows after the largest such lead."""
    if overlap == 0:
        return _compress(lib.csa_compress, lib.csa_compress_rmsnorm, raw_kv, logits, out, m,
                         rope_dims, rope_theta, pos0, T, norm_gain, norm_eps, stream)
    if norm_gain is not None:
        raise ValueError("overlapping windows take no fused RMSNorm")
    B, rows, D = raw_kv.shape
    if logits.dtype != raw_kv.dtype:
        raise TypeError("raw_kv and logits must share a dtype")
    pos = _positions(pos0, B)
    if T is None:
        lead = max((min(overlap, max(0, int(pos[b]) if pos is not None else 0)) for b in range(B)),
                   default=0)
        T = rows - lead
    _call(lib.csa_compress_overlap, (_ptr(raw_kv), _ptr(logits), _fmt(raw_kv), _ptr(out),
                                     _out_fmt(out, D, rope_dims),
                                     B, T, D, m, overlap, rope_dims, rope_theta, pos,
                                     _rows(raw_kv, "raw_kv"), _rows(logits, "logits"),
                                     _rows(out, "out"), _stream(stream)))
    return out


def hca_compress(raw_kv, logits, out, m=128, rope_dims=64, rope_theta=10000.0, pos0=None, T=None,
                 stream=None, norm_gain=None, norm_eps=1e-6):
    """Pool every m' raw KV rows into one entry (see include/lac.h); with
    norm_gain, each entry is RMSNorm'd first (hca_compress_rmsnorm)."""
    return _compress(lib.hca_compress, lib.hca_compress_rmsnorm, raw_kv, logits, out, m,
                     rope_dims, rope_theta, pos0, T, norm_gain, norm_eps, stream)


# ---------------------------------------------------------------- indexer + top-k
def indexer_topk_workspace_size(B, Tq, N, k) -> int:
    return int(lib.indexer_topk_workspace_size(B, Tq, N, k))


def _indexer_dtype(q_idx, k_idx):
    dI = q_idx.shape[-1]
    if k_idx.dtype == torch.uint8 and k_idx.shape[-1] == dI // 2 + dI // 32 and dI % 32 == 0:
        if q_idx.dtype == torch.bfloat16:
            return LAC_MXFP4                   # MXFP4 key rows (include/lac.h)
        if q_idx.dtype == torch.uint8:
            return LAC_MXFP4 | LAC_Q_E4M3      # E4M3 queries, scaled FP4 products
    if q_idx.dtype == torch.uint8:
        if k_idx.dtype != torch.uint8:
            raise TypeError("E4M3 (uint8) q_idx needs E4M3 (uint8) k_idx")
        return LAC_E4M3
    if k_idx.dtype == torch.uint8:
        return LAC_KV_E4M3_ROPE_BF16
    return _fmt(q_idx)


def indexer_topk_prepare(B, Tq, N, k, workspace, stream=None):
    """Zero the counters of an indexer_topk workspace ahead of the call that
    passes prepared=True (include/lac.h); inside a group() it joins the
    group's compress launch."""
    _call(lib.indexer_topk_prepare, (B, Tq, N, k, _ptr(workspace), workspace.numel(),
                                     _stream(stream)))


def indexer_topk(q_idx, w, k_idx, m, k, q_pos0=None, topk_idx=None, topk_score=None,
                 workspace=None, stream=None, score_bf16=False, prepared=False):
    """Scores + top-k.  q_idx [B,Tq,H_I,d_I], w [B,Tq,H_I] f32, k_idx [B,N,d_I]
    (the dtype of q_idx; uint8 E4M3 codes with bf16 or uint8 E4M3 q_idx; or
    uint8 MXFP4 rows of d_I/2 + d_I/32 bytes with bf16 q_idx, or with uint8
    E4M3 q_idx at d_I = 128: the scaled FP4 matrix-core path, LAC_Q_E4M3).
    score_bf16: select on scores rounded to bf16 (include/lac.h).
    prepared: the workspace went through indexer_topk_prepare (LAC_TOPK_PREPARED).
    Returns topk_idx [B,Tq,k] int32 (ascending, -1 padded)."""
    B, Tq, HI, dI = q_idx.shape
    N = k_idx.shape[1]
    if prepared and workspace is None:
        raise ValueError("prepared=True needs the prepared workspace")
    dt = (_indexer_dtype(q_idx, k_idx) | (LAC_SCORE_BF16 if score_bf16 else 0)
          | (LAC_TOPK_PREPARED if prepared else 0))
    for t, nm in ((q_idx, "q_idx"), (w, "w"), (k_idx, "k_idx")):
        _need_dense(t, nm)
    if topk_idx is None:
        topk_idx = torch.empty((B, Tq, k), dtype=torch.int32, device=q_idx.device)
    workspace = _workspace(workspace, indexer_topk_workspace_size(B, Tq, N, k), q_idx.device)
    _call(lib.indexer_topk, (_ptr(q_idx), _ptr(w), _ptr(k_idx), dt, B, Tq, HI, dI, N,
                             _positions(q_pos0, B), m, k, _ptr(topk_idx), _ptr(topk_score),
                             _ptr(workspace), workspace.numel(), _stream(stream)))
    return topk_idx


def indexer_topk_noalloc(q_idx, w, k_idx, m, k, q_pos0=None, topk_idx=None, topk_score=None,
                         stream=None, score_bf16=False):
    """indexer_topk on the library's fixed per-device scratch (no workspace, no
    allocation in the call; see include/lac.h).  topk_idx must be given when
    the caller cannot allocate."""
    B, Tq, HI, dI = q_idx.shape
    N = k_idx.shape[1]
    dt = _indexer_dtype(q_idx, k_idx) | (LAC_SCORE_BF16 if score_bf16 else 0)
    for t, nm in ((q_idx, "q_idx"), (w, "w"), (k_idx, "k_idx")):
        _need_dense(t, nm)
    if topk_idx is None:
        topk_idx = torch.empty((B, Tq, k), dtype=torch.int32, device=q_idx.device)
    _call(lib.indexer_topk_noalloc, (_ptr(q_idx), _ptr(w), _ptr(k_idx), dt, B, Tq, HI, dI, N,
                                     _positions(q_pos0, B), m, k, _ptr(topk_idx),
                                     _ptr(topk_score), _stream(stream)))
    return topk_idx


# ---------------------------------------------------------------- attention
def attend_workspace_size(B, Tq, H, D, rope_dims, kv_dtype, n_entries, window) -> int:
    return int(lib.attend_workspace_size(B, Tq, H, D, rope_dims, kv_dtype, n_entries, window))


def _attend_common(q, kv, raw_kv, out, raw_pos0, q_pos0):
    B, Tq, H, D = q.shape
    for t, nm in ((q, "q"), (kv, "kv"), (raw_kv, "raw_kv")):
        _need_dense(t, nm)
    if out is None:
        out = torch.empty_like(q)
    T_raw = 0 if raw_kv is None else raw_kv.shape[1]
    return B, Tq, H, D, out, T_raw, _positions(raw_pos0, B), _positions(q_pos0, B)


def csa_attend(q, ckv, topk_idx, raw_kv, window, q_pos0=None, raw_pos0=None, rope_dims=64,
               rope_theta=10000.0, sink=None, softmax_scale=0.0, out=None, workspace=None,
               stream=None, q_norm_gain=None, norm_eps=1e-6):
    """Sparse MQA over the selected compressed entries + raw window (include/lac.h);
    with q_norm_gain [D] float32, each query head is RMSNorm'd first
    (csa_attend_rmsnorm)."""
    B, Tq, H, D, out, T_raw, rp, qp = _attend_common(q, ckv, raw_kv, out, raw_pos0, q_pos0)
    k = topk_idx.shape[-1]
    kvf = _fmt(ckv)
    workspace = _workspace(workspace, attend_workspace_size(B, Tq, H, D, rope_dims, kvf, k, window),
                           q.device)
    args = [_ptr(q), _fmt(q), _ptr(ckv), kvf, ckv.shape[1], _ptr(topk_idx), k, _ptr(raw_kv), T_raw,
            rp, window, _ptr(sink), softmax_scale, B, Tq, H, D, rope_dims, rope_theta, qp,
            _ptr(out), _ptr(workspace), workspace.numel()]
    gain = _norm_gain(q_norm_gain, D, q.device)
    if gain is None:
        _call(lib.csa_attend, (*args, _stream(stream)))
    else:
        _call(lib.csa_attend_rmsnorm, (*args, _ptr(gain), norm_eps, _stream(stream)))
    return out


def hca_attend(q, hkv, raw_kv, window, m=128, q_pos0=None, raw_pos0=None, rope_dims=64,
               rope_theta=10000.0, sink=None, softmax_scale=0.0, out=None, workspace=None,
               stream=None, q_norm_gain=None, norm_eps=1e-6):
    """Dense MQA over all visible compressed entries + raw window (include/lac.h);
    with q_norm_gain, each query head is RMSNorm'd first (hca_attend_rmsnorm)."""
    B, Tq, H, D, out, T_raw, rp, qp = _attend_common(q, hkv, raw_kv, out, raw_pos0, q_pos0)
    N = hkv.shape[1]
    kvf = _fmt(hkv)
    workspace = _workspace(workspace, attend_workspace_size(B, Tq, H, D, rope_dims, kvf, N, window),
                           q.device)
    args = [_ptr(q), _fmt(q), _ptr(hkv), kvf, N, m, _ptr(raw_kv), T_raw, rp, window, _ptr(sink),
            softmax_scale, B, Tq, H, D, rope_dims, rope_theta, qp, _ptr(out), _ptr(workspace),
            workspace.numel()]
    gain = _norm_gain(q_norm_gain, D, q.device)
    if gain is None:
        _call(lib.hca_attend, (*args, _stream(stream)))
    else:
        _call(lib.hca_attend_rmsnorm, (*args, _ptr(gain), norm_eps, _stream(stream)))
    return out


# ---------------------------------------------------------------- grouped output projection
def grouped_projection_workspace_size(T, H, D, G, d_g, d) -> int:
    return int(lib.grouped_projection_workspace_size(T, H, D, G, d_g, d))


def grouped_output_projection(attn, w1, w2, out=None, workspace=None, stream=None):
    """attn [..., H, D] bf16 (leading dims flattened to T tokens), w1 [G, d_g,
    (H/G)*D] bf16, w2 [d, G*d_g] bf16 -> out [T, d] bf16."""
    for t, what in ((attn, "attn"), (w1, "w1"), (w2, "w2")):
        _need_dense(t, what)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{what} must be bfloat16")
    H, D = attn.shape[-2], attn.shape[-1]
    T = attn.numel() // (H * D) if H * D else 0
    G, d_g = w1.shape[0], w1.shape[1]
    d = w2.shape[0]
    if w1.dim() != 3 or w2.dim() != 2 or w2.shape[1] != G * d_g:
        raise ValueError("w1 must be [G, d_g, (H/G)*D] and w2 [d, G*d_g]")
    if H % G or w1.shape[2] != (H // G) * D:
        raise ValueError("w1's last dim must be (H/G)*D")
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=attn.device)
    elif out.dtype != torch.bfloat16 or out.numel() != T * d or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor of T*d values")
    workspace = _workspace(workspace, grouped_projection_workspace_size(T, H, D, G, d_g, d),
                           attn.device)
    _call(lib.grouped_output_projection, (_ptr(attn), _ptr(w1), _ptr(w2), T, H, D, G, d_g, d,
                                          _ptr(out), _ptr(workspace), workspace.numel(),
                                          _stream(stream)))
    return out


def time_next_launch(kernel: str, start: "torch.cuda.Event", stop: "torch.cuda.Event"):
    """Arm the library's one-shot launch timer (lac_time_next_launch)."""
    _check(lib.lac_time_next_launch(KERNELS[kernel], start.cuda_event, stop.cuda_event))
