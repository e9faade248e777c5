"""The oracle's end-to-end chains (TEST INFRASTRUCTURE ONLY).

Compose the oracle's steps in the order the pages give them -- compress the
KV (and the indexer keys), store the compressed cache in its storage format,
score and select (CSA), attend -- and round to a storage format only where
the GPU library stores a tensor (compressed caches; bf16 outputs are compared
before the oracle's own rounding).  Inputs are host numpy views of the bytes
that ``synth`` produced.
"""
from __future__ import annotations

import numpy as np

from . import BF16, F32, MIXED, MXFP4, attend, compress, encode_rows, index_scores, topk

FMT = {"f32": F32, "bf16": BF16, "mixed": MIXED, "mxfp4": MXFP4}


def compress_store(x, z, in_fmt, out_fmt, B, T, D, m, r, theta, pos0, norm_gain=None,
                   norm_eps=1e-6):
    """Compress (RMSNorm'd with norm_gain when given) and encode into the
    storage format: uint8 [B, T//m, row_bytes]."""
    vals = compress(x, z, FMT[in_fmt], B, T, D, m, r, theta, pos0, norm_gain=norm_gain,
                    norm_eps=norm_eps)
    N = T // m
    return encode_rows(vals.reshape(B * N, D), FMT[out_fmt], r).reshape(B, N, -1)


def csa_select(qI, w, KI, fmt, B, Tq, HI, dI, N, q_pos0, m, k, rows=None, k_fmt=None):
    """Index scores and top-k: (idx [n_rows, k], scores [n_rows, N], nvis)."""
    s, nv = index_scores(qI, w, KI, FMT[fmt], B, Tq, HI, dI, N, q_pos0, m, rows,
                         k_dtype=FMT[fmt if k_fmt is None else k_fmt])
    return topk(s, nv, k), s, nv


def csa_prefill_tiny(inp, rows=None):
    """The whole CSA prefill chain of one float32 sequence."""
    B, T, D, m, r, th = inp["B"], inp["T"], inp["D"], inp["m"], inp["r"], inp["theta"]
    h = {k_: np.ascontiguousarray(v.numpy()) for k_, v in inp.items() if hasattr(v, "numpy")}
    ckv = compress_store(h["kv"], h["z"], "f32", "f32", B, T, D, m, r, th, inp["pos0"])
    KI = compress_store(h["kI_raw"], h["zI"], "f32", "f32", B, T, inp["dI"], m, 0, th,
                        inp["pos0"])
    N = T // m
    idx, scores, nv = csa_select(h["qI"], h["w"], KI, "f32", B, T, inp["HI"], inp["dI"], N,
                                 inp["q_pos0"], m, inp["k"], rows)
    y = attend(h["q"], F32, ckv, F32, N, 0, idx, inp["k"], m, h["kv"], T, inp["raw_pos0"],
               inp["W"], None, 0.0, B, T, inp["H"], D, r, th, inp["q_pos0"], rows)
    return dict(ckv=ckv, KI=KI, idx=idx, scores=scores, nvis=nv, y=y)
