"""Shared checks for the GPU-vs-oracle parity tests (test infrastructure).

Tolerances (written here once, used by every parity test):
  * compressed entries: |g - r| <= 2^-8 |r| + 1e-6 in bf16 dims,
    1e-5 |r| + 1e-6 in float32, and within one E4M3 code (value step) in FP8
    dims -- the storage rounding of the GPU's fp32 result may land on the
    other side of a rounding boundary from the oracle's double result;
  * top-k: identical sets except entries whose oracle score lies within
    1e-3 |s_k| + 1e-6 of the oracle's k-th score (near-ties);
  * attention outputs: per (b, t, h) row, max_c |g - r| / max_c |r| <= 1e-2
    (bf16 operands, fp32 accumulation), r the oracle's double result;
  * grouped projection outputs (bf16, against the oracle with the same
    bfloat16 rounding of the intermediate y):
        |g - r| <= 2^-8 |r| + (1 + 2^-8) F + A
    2^-8 |r|: the output's own rounding (bf16 keeps 8 significant bits, so
    rounding to nearest moves a value by at most 2^-8 of itself).  F: the
    GPU sums y in fp32 before rounding it, so where the exact y lies within
    that sum's error bound of a bf16 rounding midpoint it may round to the
    neighbouring value; F adds |W2[j, c]| * ulp(y_c) over those c.  A: the
    fp32 error bound of the second sum.  An fp32 sum of K exact bf16 products
    in MFMA steps of 16 is within (K/16 + 1) 2^-24 sum|terms| of the exact sum.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

ATTN_TOL = 1e-2
TIE_REL, TIE_ABS = 1e-3, 1e-6


def host(t: torch.Tensor):
    return synth.host_bytes(t)


def as_f64(t: torch.Tensor) -> np.ndarray:
    """GPU result -> float64 (through PyTorch's own conversion)."""
    return t.detach().float().cpu().double().numpy()


def check_compressed(gpu: torch.Tensor, ref: np.ndarray, fmt: str, D: int, r: int):
    """gpu: stored entries [..., row]; ref: oracle doubles [..., D]."""
    ref = ref.reshape(-1, D)
    if fmt == "f32":
        g = as_f64(gpu).reshape(-1, D)
        bad = np.abs(g - ref) > 1e-5 * np.abs(ref) + 1e-6
    elif fmt == "bf16":
        g = as_f64(gpu).reshape(-1, D)
        bad = np.abs(g - ref) > 2.0 ** -8 * np.abs(ref) + 1e-6
    elif fmt == "mxfp4":
        # within one E2M1 grid step of the exact value at the coarser of the
        # two blocks' scales (the GPU's fp32 pooled value can round to the
        # neighbouring code, or cross a power of two and take the next scale)
        rowb = D // 2 + D // 32
        raw = np.ascontiguousarray(gpu.detach().cpu().numpy().reshape(-1, rowb))
        g = oracle.decode_rows(raw, oracle.MXFP4, D, 0)
        mine = oracle.encode_rows(ref, oracle.MXFP4, 0)
        S = np.repeat(2.0 ** (np.maximum(raw[:, D // 2:], mine[:, D // 2:]).astype(np.int64) - 127),
                      32, axis=1)
        x = np.abs(ref) / S
        gap = np.where(x < 2, 0.5, np.where(x < 4, 1.0, 2.0))
        bad = np.abs(g - ref) > np.where(x <= 6, gap * S, np.abs(ref) - 6 * S + 2 * S) * (1 + 1e-9)
        same = (raw == mine).mean()
        assert same > 0.98, f"only {same:.3f} of the MXFP4 bytes equal the oracle's encoding"
    else:
        rowb = (D - r) + 2 * r
        raw = gpu.detach().cpu().numpy().reshape(-1, rowb)
        g = oracle.decode_rows(np.ascontiguousarray(raw), oracle.MIXED, D, r)
        fp8 = g[:, : D - r]
        ref8 = ref[:, : D - r]
        # one E4M3 step at the value's binade (2^-9 below 2^-6)
        step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref8), 2.0 ** -6))) - 3),
                          2.0 ** -9)
        bad8 = np.abs(fp8 - np.clip(ref8, -448, 448)) > step * (1 + 1e-9)
        badb = np.abs(g[:, D - r:] - ref[:, D - r:]) > 2.0 ** -8 * np.abs(ref[:, D - r:]) + 1e-6
        bad = np.concatenate([bad8, badb], axis=1)
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} compressed values out of tolerance"


def check_topk(gpu_idx: np.ndarray, o_idx: np.ndarray, o_scores: np.ndarray, nvis: np.ndarray,
               k: int):
    """Rows of GPU indices vs oracle indices under the near-tie rule.
    Returns the rows whose sets are identical."""
    same_rows = []
    for rr in range(gpu_idx.shape[0]):
        nv = int(nvis[rr])
        keff = min(k, nv)
        g = gpu_idx[rr]
        assert (g[keff:] == -1).all(), f"row {rr}: padding"
        gs = g[:keff]
        assert len(set(gs.tolist())) == keff, f"row {rr}: duplicates"
        assert ((gs >= 0) & (gs < nv)).all(), f"row {rr}: invisible index"
        osel = set(o_idx[rr, :keff].tolist())
        diff = set(gs.tolist()) ^ osel
        if diff:
            s = o_scores[rr, :nv]
            sk = np.sort(s)[::-1][keff - 1]
            for j in diff:
                assert abs(s[j] - sk) <= TIE_REL * abs(sk) + TIE_ABS, \
                    f"row {rr}: index {j} score {s[j]} vs k-th {sk}"
        else:
            same_rows.append(rr)
    return same_rows


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (the smallest normal spacing below 2^-126)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_topk_bf16(gpu_idx, gpu_score, o_idx, o_rounded, nvis, k):
    """Selection on bf16-rounded scores (LAC_SCORE_BF16).  The GPU rounds its
    fp32 sum, the oracle its double score, so a score can land one bf16 step
    apart; rows must then agree except for indices whose oracle score lies
    within one step of the k-th, and every returned score within one step of
    the oracle's rounded score.  Returns the rows whose sets are identical."""
    same_rows = []
    for rr in range(gpu_idx.shape[0]):
        nv = int(nvis[rr])
        keff = min(k, nv)
        g = gpu_idx[rr]
        assert (g[keff:] == -1).all(), f"row {rr}: padding"
        gs = g[:keff]
        assert len(set(gs.tolist())) == keff, f"row {rr}: duplicates"
        assert ((gs >= 0) & (gs < nv)).all(), f"row {rr}: invisible index"
        s = o_rounded[rr, :nv]
        assert (np.abs(gpu_score[rr, :keff] - s[gs]) <= bf16_ulp(s[gs])).all(), \
            f"row {rr}: returned scores off by more than one bf16 step"
        diff = set(gs.tolist()) ^ set(o_idx[rr, :keff].tolist())
        if diff:
            sk = np.sort(s)[::-1][keff - 1]
            for j in diff:
                assert abs(s[j] - sk) <= bf16_ulp(sk), f"row {rr}: index {j} score {s[j]} vs k-th {sk}"
        else:
            same_rows.append(rr)
    return same_rows


def check_attention(gpu: np.ndarray, ref: np.ndarray, what=""):
    """gpu, ref: [rows, H, D] float64."""
    num = np.abs(gpu - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    rel = np.where(den > 0, num / np.maximum(den, 1e-300), num)
    worst = float(rel.max()) if rel.size else 0.0
    if worst > ATTN_TOL:
        bad = np.argwhere(rel > ATTN_TOL)
        r, h = (int(v) for v in np.unravel_index(int(np.argmax(rel)), rel.shape))
        d = int(np.argmax(np.abs(gpu[r, h] - ref[r, h])))
        raise AssertionError(
            f"{what}: worst row relative error {worst:.3e} at (row {r}, head {h}, dim {d}): "
            f"gpu {gpu[r, h, d]:.6g} ref {ref[r, h, d]:.6g}, row max |ref| {den[r, h]:.4g}; "
            f"{len(bad)} (row, head) pairs over {ATTN_TOL}: first {bad[:12].tolist()}")
    return worst


def _sum_bound(K, abs_sum):
    return (K / 16 + 1) * 2.0 ** -24 * abs_sum


def check_projection(gpu: np.ndarray, ref: np.ndarray, attn, w1, w2, what: str):
    """gpu, ref: [rows, d] float64; attn [rows, H, D], w1 [G, d_g, K1], w2 [d, G*d_g]
    as float64 arrays (the stored bf16 values)."""
    rows = attn.shape[0]
    G, d_g, K1 = w1.shape
    x = attn.reshape(rows, G, K1)
    y = np.einsum("tgk,gjk->tgj", x, w1).reshape(rows, G * d_g)
    ya = np.einsum("tgk,gjk->tgj", np.abs(x), np.abs(w1)).reshape(rows, G * d_g)
    rho = _sum_bound(K1, ya)
    ay = np.maximum(np.abs(y), 2.0 ** -126)
    ulp = 2.0 ** (np.floor(np.log2(ay)) - 7)
    frac = np.abs(y) / ulp - np.floor(np.abs(y) / ulp)
    near = np.abs(frac - 0.5) * ulp <= rho
    F = (np.where(near, ulp, 0.0)) @ np.abs(w2).T
    A = _sum_bound(G * d_g, (np.abs(y) + np.where(near, ulp, 0.0)) @ np.abs(w2).T)
    bad = np.abs(gpu - ref) > 2.0 ** -8 * np.abs(ref) + (1 + 2.0 ** -8) * F + A
    scale = np.max(np.abs(ref), axis=1, keepdims=True)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} projection outputs out of "
                           f"tolerance, worst {np.max(np.abs(gpu - ref) / scale):.3g} of row max, "
                           f"{int(near.sum())} intermediates near a rounding midpoint")
