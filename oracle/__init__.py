"""CPU oracle for hybrid compressed attention (CSA + HCA).

TEST INFRASTRUCTURE ONLY: the slow, plain, double-precision definition that
the GPU library is checked against.  It lives in ``lac_oracle.c`` (plain C,
OpenMP over independent rows) and is reached through ctypes here.  Only the
tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package; the GPU library never does, and the two share no
code.

Inputs are the exact stored bytes (numpy arrays of float32, uint16 bfloat16
bit patterns, uint8 mixed FP8/bf16 rows, or float64), decoded by the oracle's
own decoders.  Storage codes: F32=0, BF16=1, MIXED=2 (E4M3 for the first D-r
dims, bf16 for the last r), F64=3.

Parity status of each function (what pins it is in ``tests/test_oracle_*.py``):
all functions here are pinned; see the module docstrings of those tests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32, BF16, MIXED, F64, MXFP4 = 0, 1, 2, 3, 4

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lac_oracle.c")
_LIB = os.path.join(_HERE, "liblac_oracle.so")
_lib = None


def build() -> str:
    """Compile the oracle with gcc (IEEE double, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-shared", "-fPIC",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.lo_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.lo_bf16_decode.restype = dbl
    lib.lo_bf16_encode.argtypes = [dbl]
    lib.lo_bf16_encode.restype = ctypes.c_uint16
    lib.lo_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.lo_e4m3_decode.restype = dbl
    lib.lo_e4m3_encode.argtypes = [dbl]
    lib.lo_e4m3_encode.restype = ctypes.c_uint8
    lib.lo_row_bytes.argtypes = [i32, i32, i32]
    lib.lo_row_bytes.restype = i64
    lib.lo_decode_rows.argtypes = [vp, i32, i64, i32, i32, vp]
    lib.lo_decode_rows.restype = None
    lib.lo_encode_rows.argtypes = [vp, i32, i64, i32, i32, vp]
    lib.lo_encode_rows.restype = None
    lib.lo_rope.argtypes = [vp, i32, i32, dbl, dbl]
    lib.lo_rope.restype = None
    lib.lo_compress.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, dbl, vp, i64, i64, vp, vp]
    lib.lo_compress.restype = i32
    lib.lo_compress2.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, dbl, vp, i64, i64, vp, dbl,
                                 vp, vp]
    lib.lo_compress2.restype = i32
    lib.lo_compress_overlap.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, dbl, vp, i64,
                                        i64, vp, vp]
    lib.lo_compress_overlap.restype = i32
    lib.lo_rmsnorm.argtypes = [vp, i32, vp, dbl]
    lib.lo_rmsnorm.restype = None
    lib.lo_index_scores.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, i32, vp, i32,
                                    vp, vp]
    lib.lo_index_scores.restype = i32
    lib.lo_index_scores2.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, vp, i32, vp,
                                     i32, vp, vp]
    lib.lo_index_scores2.restype = i32
    lib.lo_e2m1_decode.argtypes = [ctypes.c_uint8]
    lib.lo_e2m1_decode.restype = dbl
    lib.lo_e8m0_decode.argtypes = [ctypes.c_uint8]
    lib.lo_e8m0_decode.restype = dbl
    lib.lo_round_scores_bf16.argtypes = [vp, ctypes.c_int64]
    lib.lo_round_scores_bf16.restype = i32
    lib.lo_topk.argtypes = [vp, i32, i32, vp, i32, vp]
    lib.lo_topk.restype = i32
    lib.lo_attend.argtypes = [vp, i32, vp, i32, i32, i32, vp, i32, i32, vp, i32, vp, i32, vp,
                              dbl, i32, i32, i32, i32, i32, dbl, vp, vp, i32, vp]
    lib.lo_attend.restype = i32
    lib.lo_attend2.argtypes = [vp, i32, vp, i32, i32, i32, vp, i32, i32, vp, i32, vp, i32, vp,
                               dbl, i32, i32, i32, i32, i32, dbl, vp, vp, i32, vp, dbl, vp]
    lib.lo_attend2.restype = i32
    lib.lo_grouped_projection.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.lo_grouped_projection.restype = i32
    lib.lo_num_threads.argtypes = []
    lib.lo_num_threads.restype = i32
    _lib = lib
    return lib


def _p(a):
    if a is None:
        return None
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("oracle inputs must be C-contiguous")
    return a.ctypes.data


def _i64(v, n):
    if v is None:
        return np.zeros(n, np.int64)
    return np.ascontiguousarray(np.broadcast_to(np.asarray(v, np.int64), (n,)))


def num_threads() -> int:
    return _load().lo_num_threads()


# ---------------------------------------------------------------- formats
def bf16_decode(bits) -> np.ndarray:
    lib = _load()
    bits = np.asarray(bits, np.uint16)
    return np.array([lib.lo_bf16_decode(int(b)) for b in bits.ravel()]).reshape(bits.shape)


def bf16_encode(v) -> np.ndarray:
    lib = _load()
    v = np.asarray(v, np.float64)
    return np.array([lib.lo_bf16_encode(float(x)) for x in v.ravel()],
                    np.uint16).reshape(v.shape)


def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes, np.uint8)
    return np.array([lib.lo_e4m3_decode(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e4m3_encode(v) -> np.ndarray:
    lib = _load()
    v = np.asarray(v, np.float64)
    return np.array([lib.lo_e4m3_encode(float(x)) for x in v.ravel()],
                    np.uint8).reshape(v.shape)


def row_bytes(dtype: int, D: int, r: int) -> int:
    return int(_load().lo_row_bytes(dtype, D, r))


def decode_rows(src: np.ndarray, dtype: int, D: int, r: int) -> np.ndarray:
    """Stored rows (any numpy dtype holding the bytes) -> float64 [..., D]."""
    rb = row_bytes(dtype, D, r)
    src = np.ascontiguousarray(src)
    n = src.nbytes // rb
    out = np.empty((n, D), np.float64)
    _load().lo_decode_rows(_p(src), dtype, n, D, r, _p(out))
    return out


def encode_rows(v: np.ndarray, dtype: int, r: int) -> np.ndarray:
    """float64 [n, D] -> stored bytes, uint8 [n, row_bytes]."""
    v = np.ascontiguousarray(v, np.float64)
    D = v.shape[-1]
    n = v.size // D
    rb = row_bytes(dtype, D, r)
    out = np.empty((n, rb), np.uint8)
    _load().lo_encode_rows(_p(v), dtype, n, D, r, _p(out))
    return out


def rope(v: np.ndarray, r: int, theta: float, pos: float) -> np.ndarray:
    """Rotate the last r dims of one float64 vector at position pos (copy)."""
    v = np.array(v, np.float64, copy=True)
    _load().lo_rope(_p(v), v.shape[-1], r, float(theta), float(pos))
    return v


# ---------------------------------------------------------------- method
def rmsnorm(v, gain, eps):
    """RMSNorm of one float64 vector over all its dims, times gain (copy)."""
    v = np.array(v, np.float64, copy=True)
    g = np.ascontiguousarray(gain, np.float32)
    _load().lo_rmsnorm(_p(v), v.shape[-1], _p(g), float(eps))
    return v


def compress(x, z, in_dtype, B, T, D, m, r=0, theta=10000.0, pos0=None,
             x_bstride=None, z_bstride=None, want_weights=False, norm_gain=None, norm_eps=1e-6):
    """Block-softmax pooling (+ RMSNorm with norm_gain [D] when given) + rotation
    at the block start.  -> float64 [B, T//m, D] (and the weights [B, T//m, m, D]
    when want_weights)."""
    N = T // m
    out = np.empty((B, N, D), np.float64)
    alpha = np.empty((B, N, m, D), np.float64) if want_weights else None
    pos = _i64(pos0, B)        # held until the call returns
    gain = None if norm_gain is None else np.ascontiguousarray(norm_gain, np.float32)
    rc = _load().lo_compress2(_p(x), _p(z), in_dtype, B, T, D, m, r, float(theta),
                              _p(pos), T if x_bstride is None else x_bstride,
                              T if z_bstride is None else z_bstride, _p(gain), float(norm_eps),
                              _p(out), _p(alpha))
    if rc:
        raise ValueError(f"lo_compress rejected its arguments ({rc})")
    return (out, alpha) if want_weights else out


def compress_overlap(x, z, in_dtype, B, T, D, m, o, r=0, theta=10000.0, pos0=None,
                     x_bstride=None, z_bstride=None, want_weights=False):
    """CSA compression with overlapping windows: entry j pools positions
    [max(0, p_j - o), p_j + m) (p_j = pos0 + j*m), then is rotated at p_j.
    Row 0 of sequence b is at position pos0[b] - min(o, pos0[b]); T rows
    follow that lead.  -> float64 [B, T//m, D] (and the weights
    [B, T//m, m + o, D] when want_weights)."""
    N = T // m
    out = np.empty((B, N, D), np.float64)
    alpha = np.empty((B, N, m + o, D), np.float64) if want_weights else None
    pos = _i64(pos0, B)        # held until the call returns
    lead = np.minimum(pos, o)
    rows = T + int(lead.max()) if B else T
    rc = _load().lo_compress_overlap(_p(x), _p(z), in_dtype, B, T, D, m, o, r, float(theta),
                                     _p(pos), rows if x_bstride is None else x_bstride,
                                     rows if z_bstride is None else z_bstride, _p(out),
                                     _p(alpha))
    if rc:
        raise ValueError(f"lo_compress_overlap rejected its arguments ({rc})")
    return (out, alpha) if want_weights else out


def _rows(rows, B, Tq):
    if rows is None:
        rows = [(b, i) for b in range(B) for i in range(Tq)]
    return np.ascontiguousarray(np.asarray(rows, np.int32).reshape(-1, 2))


def index_scores(q, w, K, dtype, B, Tq, HI, dI, N, qpos0, m, rows=None, k_dtype=None,
                 score_bf16=False):
    """-> (scores float64 [n_rows, N] with -inf where not visible, nvis int32 [n_rows]).
    q is stored in dtype, K in k_dtype (default dtype; the mixed code with no
    rotated dims means E4M3 codes).  score_bf16: the scores rounded to bf16."""
    rows = _rows(rows, B, Tq)
    n = rows.shape[0]
    scores = np.empty((n, N), np.float64)
    nvis = np.empty(n, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    qpos = _i64(qpos0, B)      # held until the call returns
    rc = _load().lo_index_scores2(_p(q), dtype, _p(w), _p(K), dtype if k_dtype is None else k_dtype,
                                  B, Tq, HI, dI, N, _p(qpos), m, _p(rows), n, _p(scores), _p(nvis))
    if rc:
        raise ValueError(f"lo_index_scores rejected its arguments ({rc})")
    if score_bf16:
        _load().lo_round_scores_bf16(_p(scores), scores.size)
    return scores, nvis


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 codes (0..15) -> float64."""
    f = _load().lo_e2m1_decode
    return np.array([f(int(c)) for c in np.ravel(codes)], np.float64).reshape(np.shape(codes))


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 scale bytes -> float64 powers of two (255 -> NaN)."""
    f = _load().lo_e8m0_decode
    return np.array([f(int(c)) for c in np.ravel(codes)], np.float64).reshape(np.shape(codes))


def round_scores_bf16(scores):
    """Index scores rounded to bf16 (ties to even), in a new float64 array."""
    out = np.array(scores, np.float64, copy=True, order="C")
    _load().lo_round_scores_bf16(_p(out), out.size)
    return out


def topk(scores, nvis, k):
    """-> int32 [n_rows, k] (selection order, -1 padded)."""
    scores = np.ascontiguousarray(scores, np.float64)
    n, N = scores.shape
    nvis = np.ascontiguousarray(nvis, np.int32)
    idx = np.empty((n, k), np.int32)
    _load().lo_topk(_p(scores), n, N, _p(nvis), k, _p(idx))
    return idx


def attend(q, q_dtype, kv, kv_dtype, N, mode, idx, k, m, raw, T_raw, raw_pos0, W, sink,
           scale, B, Tq, H, D, r, theta, qpos0, rows=None, q_norm_gain=None, norm_eps=1e-6):
    """Core attention.  mode 0 = CSA (idx [n_rows, k]), mode 1 = HCA (m = m').
    With q_norm_gain [D], each query head vector is RMSNorm'd first.
    -> float64 [n_rows, H, D]."""
    rows = _rows(rows, B, Tq)
    n = rows.shape[0]
    out = np.empty((n, H, D), np.float64)
    if idx is not None:
        idx = np.ascontiguousarray(idx, np.int32)
    if sink is not None:
        sink = np.ascontiguousarray(sink, np.float64)
    rpos, qpos = _i64(raw_pos0, B), _i64(qpos0, B)   # held until the call returns
    gain = None if q_norm_gain is None else np.ascontiguousarray(q_norm_gain, np.float32)
    rc = _load().lo_attend2(_p(q), q_dtype, _p(kv), kv_dtype, N, mode, _p(idx), k, m, _p(raw),
                            T_raw, _p(rpos), W, _p(sink), float(scale), B, Tq, H, D,
                            r, float(theta), _p(qpos), _p(rows), n, _p(gain), float(norm_eps),
                            _p(out))
    if rc:
        raise ValueError(f"lo_attend rejected its arguments ({rc})")
    return out


def grouped_projection(attn, w1, w2, dtype, T, H, D, G, d_g, d, y_dtype=F64):
    """Grouped output projection (QbitAI rewrite, grouped output projection
    step): heads split into G groups of H/G consecutive heads, group g's
    concatenated outputs projected by W1[g] [d_g, (H/G)*D], the concatenation
    of the G results by W2 [d, G*d_g].  y_dtype=BF16 rounds the intermediate
    to bfloat16 between the products.  -> float64 [T, d]."""
    out = np.empty((T, d), np.float64)
    rc = _load().lo_grouped_projection(_p(attn), _p(w1), _p(w2), dtype, T, H, D, G, d_g, d,
                                       y_dtype, _p(out))
    if rc:
        raise ValueError(f"lo_grouped_projection rejected its arguments ({rc})")
    return out
