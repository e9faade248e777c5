"""Throughput of the hybrid compressed attention path on one MI355X.

Default workload (pair_decode_1m): one decode step of a CSA + HCA layer pair
for 4 sequences at position 2^20 -- compress the newest complete blocks (CSA
entry, indexer key, HCA entry), index 262144 compressed entries per sequence
and keep the top 2048, sparse CSA attention and dense HCA attention over
8192 entries, each with a 128-token raw window; 64 query heads, 512-dim KV
stored as FP8 E4M3 with the 64 rotated dims in bf16.  The metric is decode
tokens/s (4 per step) with the algorithmic HBM GB/s beside it.  Three
independent cache sets rotate so that a step never finds its 294 MB working
set in the 256 MB Infinity Cache.  The step's three compress calls run as one
launch group, and so do its two attention calls (lac.group);
pair_decode_1m_ungrouped makes the same calls one launch each.

Other workloads (--workload): pair_decode_1m_e4m3_indexer (the same step with
the indexer keys stored as E4M3, one byte per dim), pair_decode_1m_fp8_indexer
(E4M3 indexer queries and keys on the FP8 matrix cores),
pair_decode_1m_mxfp4_indexer (MXFP4 indexer keys, widened for bf16 queries),
pair_decode_1m_fp4_indexer (E4M3 queries against MXFP4 keys on the
block-scaled FP4 matrix cores), csa_decode_128k (32
sequences at 131072),
csa_chunk_prefill (4096 queries appended to 262144 tokens; TFLOP/s),
csa_chunk_prefill_1m (the same chunk ending at 2^20 tokens),
csa_chunk_prefill_fp8_indexer (the 262144-token chunk with E4M3 indexer
queries and keys), csa_chunk_prefill_fp4_indexer (E4M3 queries against MXFP4
keys),
hca_prefill_8k (8192 tokens; TFLOP/s), bulk_compress_1m and
bulk_compress_128k (building the compressed caches of whole contexts from raw
activations; GB/s), and the grouped output projection.

Each step's library calls are marshalled once per cache set (lac.CallList)
and replayed, so the host cost of a step is one ctypes call per entry point
plus the library's own validation and launches.

Prints one JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import contextlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

METRIC = "CSA+HCA decode tokens/s and HBM GB/s at 128K-1M ctx; prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0

# HBM bytes per launch of the indexer score kernel, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE (one pass each), scaled by what the same counters read for a 1 GiB
# device copy (FETCH x2.000, WRITE x1.000).  They hold only for the kernel
# sources they were taken on (score.hip and the device helpers it includes),
# identified by their SHA-256; after any change to them the roofline reports
# traffic as null until the counters are taken again.
SCORE_TRAFFIC_BYTES = {"pair_decode_1m": 273737728, "pair_decode_1m_ungrouped": 273737728,
                       "csa_decode_128k": 277470208, "csa_chunk_prefill": 1328329728,
                       "pair_decode_1m_fp8_indexer": 138900480,
                       "pair_decode_1m_mxfp4_indexer": 76721152,
                       "pair_decode_1m_fp4_indexer": 76252160,
                       "csa_chunk_prefill_fp8_indexer": 1278718976,
                       "csa_chunk_prefill_fp4_indexer": 1158550528}
SCORE_TRAFFIC_SOURCE_SHA256 = "f2fbdff8ead546bfc2485b2304e89ecc502bd8f3f22f65c2c57a140e80a3e770"
SCORE_SOURCES = ("score.hip", "lac_device.h")


def score_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for name in SCORE_SOURCES:
        with open(os.path.join(ROOT, "long_context_attention_compressor_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _score_traffic(workload):
    if score_source_sha256() != SCORE_TRAFFIC_SOURCE_SHA256:
        return None
    return SCORE_TRAFFIC_BYTES.get(workload)


# The same for the product kernel of the grouped output projection: bytes per
# launch averaged over its two launches (the per-group product and the output
# product), for the kernel source identified by its SHA-256.
PROJECT_TRAFFIC_BYTES = 688514801
PROJECT_TRAFFIC_SOURCE_SHA256 = "71f3771f1facab32cb70505661b95e4d60f0e51022455247a042c8dfb8bb7384"
PROJECT_SOURCES = ("project.hip", "lac_device.h")


def _project_traffic():
    import hashlib
    h = hashlib.sha256()
    for name in PROJECT_SOURCES:
        with open(os.path.join(ROOT, "long_context_attention_compressor_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return PROJECT_TRAFFIC_BYTES if h.hexdigest() == PROJECT_TRAFFIC_SOURCE_SHA256 else None


def _rows(t, r0, r1):
    return t[:, r0:r1]


# ---------------------------------------------------------------- workloads
class PairDecode:
    name = "pair_decode_1m"
    unit = "tokens/s"

    ki_fmt = "bf16"
    qi_fmt = "bf16"
    rmsnorm = False     # fused RMSNorm of the new compressed entries and the queries
    gain = None
    overlap = 0         # CSA compression windows reaching this many tokens back
    grouped = True      # the step's independent calls in launch groups (lac.group)

    def __init__(self, lac, synth, dev, sets, seed=4, B=4, ctx=1 << 20):
        self.lac, self.B, self.ctx = lac, B, ctx
        self.sets = [synth.pair_decode(seed=seed + 1000 * s, B=B, ctx=ctx, ki_fmt=self.ki_fmt,
                                       qi_fmt=self.qi_fmt, csa_overlap=self.overlap, device=dev)
                     for s in range(sets)]
        c = self.sets[0]
        self.c = c
        # RMSNorm gains (synthetic: 1), used when rmsnorm is set
        self.gain = torch.ones(c["D"], dtype=torch.float32, device=dev) if self.rmsnorm else None
        self.idx = torch.empty((B, 1, c["k"]), dtype=torch.int32, device=dev)
        self.out_csa = torch.empty_like(c["q_csa"])
        self.out_hca = torch.empty_like(c["q_hca"])
        self.ws_idx = torch.empty(lac.indexer_topk_workspace_size(B, 1, c["N"], c["k"]),
                                  dtype=torch.uint8, device=dev)
        self.ws_csa = torch.empty(lac.attend_workspace_size(B, 1, c["H"], c["D"], c["r"], 2, c["k"],
                                                            c["W"]), dtype=torch.uint8, device=dev)
        self.ws_hca = torch.empty(lac.attend_workspace_size(B, 1, c["H"], c["D"], c["r"], 2,
                                                            c["Nh"], c["W"]),
                                  dtype=torch.uint8, device=dev)

    timer_kernel = "indexer_score"

    def step(self, i):
        lac, c, s = self.lac, self.c, self.sets[i % len(self.sets)]
        N, Nh, m, mh, ctx = c["N"], c["Nh"], c["m"], c["m_hca"], self.ctx
        g = self.gain
        grp = lac.group if self.grouped else contextlib.nullcontext
        # compress the newest blocks: the CSA layer's KV entry and indexer key,
        # the HCA layer's entry; grouped, the indexer's workspace zeroing joins
        # their launch (independent calls: one launch)
        with grp():
            lac.csa_compress(s["new_kv_csa"], s["new_z_csa"], _rows(s["ckv"], N - 1, N), m=m,
                             rope_dims=c["r"], pos0=ctx - m, norm_gain=g, T=m,
                             overlap=self.overlap)
            lac.csa_compress(s["new_kI"], s["new_zI"], _rows(s["KI"], N - 1, N), m=m,
                             rope_dims=0, pos0=ctx - m)
            lac.hca_compress(s["new_kv_hca"], s["new_z_hca"], _rows(s["hkv"], Nh - 1, Nh),
                             m=mh, rope_dims=c["r"], pos0=ctx - mh, norm_gain=g)
            if self.grouped:
                lac.indexer_topk_prepare(self.B, 1, N, c["k"], self.ws_idx)
        # the CSA layer's selection
        lac.indexer_topk(s["qI"], s["w"], s["KI"], m=m, k=c["k"], q_pos0=ctx, topk_idx=self.idx,
                         workspace=self.ws_idx, prepared=self.grouped)
        # both layers' attention (independent: one attention and one combine
        # launch when grouped)
        with grp():
            lac.csa_attend(s["q_csa"], s["ckv"], self.idx, s["raw_csa"], c["W"], q_pos0=ctx,
                           raw_pos0=c["raw_pos0"], rope_dims=c["r"], out=self.out_csa,
                           workspace=self.ws_csa, q_norm_gain=g)
            lac.hca_attend(s["q_hca"], s["hkv"], s["raw_hca"], c["W"], m=mh, q_pos0=ctx,
                           raw_pos0=c["raw_pos0"], rope_dims=c["r"], out=self.out_hca,
                           workspace=self.ws_hca, q_norm_gain=g)

    def tokens_per_step(self):
        return self.B

    def bytes_per_step(self):
        c = self.c
        row = c["D"] - c["r"] + 2 * c["r"]
        kb = self.key_bytes_per_dim()
        qb = 1 if self.qi_fmt == "mixed" else 2                                   # query bytes/dim
        per_seq = (c["N"] * c["dI"] * kb + c["HI"] * c["dI"] * qb + c["HI"] * 4  # indexer
                   + c["k"] * row + c["Nh"] * row + 2 * c["W"] * row               # gathers
                   + 2 * c["H"] * c["D"] * 2 * 2)                                   # q, out
        compress = (((c["m"] + self.overlap) * c["D"] + c["m"] * c["dI"] + c["m_hca"] * c["D"])
                    * 2 * 2 + 2 * row + int(c["dI"] * kb))
        return self.B * (per_seq + compress)

    def key_bytes_per_dim(self):
        """Indexer key bytes per dim: bf16 2, E4M3 1, MXFP4 (codes + scales) 17/32."""
        return {"bf16": 2, "mixed": 1, "mxfp4": 17 / 32}[self.ki_fmt]

    def indexer_bytes_per_launch(self):
        c = self.c
        kb = self.key_bytes_per_dim()
        qb = 1 if self.qi_fmt == "mixed" else 2
        return self.B * int(c["N"] * c["dI"] * kb + c["HI"] * c["dI"] * qb + c["HI"] * 4)

    def config(self):
        c = self.c
        return {"workload": self.name, "batch": self.B, "ctx": self.ctx, "topk": c["k"],
                "window": c["W"], "heads": c["H"], "kv_dim": c["D"], "rope_dims": c["r"],
                "indexer": (f"{c['HI']}x{c['dI']} bf16" if self.ki_fmt == "bf16" else
                            f"{c['HI']}x{c['dI']}, bf16 queries, mxfp4 keys (e2m1 + e8m0 per 32)"
                            if self.ki_fmt == "mxfp4" and self.qi_fmt == "bf16" else
                            f"{c['HI']}x{c['dI']}, e4m3 queries, mxfp4 keys (scaled fp4 mfma)"
                            if self.ki_fmt == "mxfp4" else
                            f"{c['HI']}x{c['dI']}, bf16 queries, e4m3 keys" if self.qi_fmt == "bf16"
                            else f"{c['HI']}x{c['dI']}, e4m3 queries and keys (fp8 mfma)"),
                "csa_entries": c["N"],
                "hca_entries": c["Nh"], "kv_format": "e4m3 + bf16 rope dims (576 B/entry)",
                "rmsnorm": "q and new entries, fused" if self.rmsnorm else "none",
                "csa_window_overlap": self.overlap,
                "cache_sets": len(self.sets)}

    def cpu_sample(self, min_seconds=10.0, max_steps=48):
        """The oracle's whole decode step, one sequence at a time: sequences
        0..B-1 of cache sets 0, 1, ... in turn until min_seconds of oracle
        work (at most max_steps); only the oracle's calls are timed."""
        import numpy as np

        import oracle
        from oracle import chain
        import synth

        c, ctx = self.c, self.ctx
        N, Nh = c["N"], c["Nh"]
        g = None if self.gain is None else self.gain.cpu().numpy()
        el, steps = 0.0, 0
        while steps < max_steps and (el < min_seconds or steps == 0):
            s = self.sets[(steps // self.B) % len(self.sets)]
            b = steps % self.B
            h = {k_: synth.host_bytes(v[b:b + 1]) for k_, v in s.items()
                 if isinstance(v, torch.Tensor)}
            ckv = h["ckv"].reshape(1, N, -1).copy()
            KI = h["KI"].reshape(1, N, -1).copy()
            hkv = h["hkv"].reshape(1, Nh, -1).copy()
            t0 = time.perf_counter()
            if self.overlap:
                vals = oracle.compress_overlap(h["new_kv_csa"], h["new_z_csa"], oracle.BF16, 1,
                                               c["m"], c["D"], c["m"], self.overlap, c["r"], 1e4,
                                               ctx - c["m"])
                ckv[:, N - 1:] = oracle.encode_rows(vals.reshape(1, c["D"]), oracle.MIXED,
                                                    c["r"]).reshape(1, 1, -1)
            else:
                ckv[:, N - 1:] = chain.compress_store(h["new_kv_csa"], h["new_z_csa"], "bf16",
                                                      "mixed", 1, c["m"], c["D"], c["m"], c["r"],
                                                      1e4, ctx - c["m"], norm_gain=g)
            KI.view(np.uint8)[:, N - 1:] = chain.compress_store(
                h["new_kI"], h["new_zI"], "bf16", self.ki_fmt, 1, c["m"], c["dI"], c["m"], 0, 1e4,
                ctx - c["m"])
            hkv[:, Nh - 1:] = chain.compress_store(h["new_kv_hca"], h["new_z_hca"], "bf16",
                                                   "mixed", 1, c["m_hca"], c["D"], c["m_hca"],
                                                   c["r"], 1e4, ctx - c["m_hca"], norm_gain=g)
            idx, _, _ = chain.csa_select(h["qI"], h["w"], KI, self.qi_fmt, 1, 1, c["HI"], c["dI"],
                                         N, ctx, c["m"], c["k"], k_fmt=self.ki_fmt)
            oracle.attend(h["q_csa"], oracle.BF16, ckv, oracle.MIXED, N, 0, idx, c["k"], c["m"],
                          h["raw_csa"], c["W"], c["raw_pos0"], c["W"], None, 0.0, 1, 1, c["H"],
                          c["D"], c["r"], 1e4, ctx, q_norm_gain=g)
            oracle.attend(h["q_hca"], oracle.BF16, hkv, oracle.MIXED, Nh, 1, None, 0, c["m_hca"],
                          h["raw_hca"], c["W"], c["raw_pos0"], c["W"], None, 0.0, 1, 1, c["H"],
                          c["D"], c["r"], 1e4, ctx, q_norm_gain=g)
            el += time.perf_counter() - t0
            steps += 1
        return {"value": steps / el, "unit": self.unit, "seconds": el,
                "sample": f"{steps} single-sequence decode steps (compress newest blocks, index "
                          f"262144 entries, top-2048, CSA + HCA attention, 64 heads), sequences "
                          f"0-{self.B - 1} of the cache sets in turn"}


class PairDecodeUngrouped(PairDecode):
    """pair_decode_1m with every call launched on its own (no launch groups):
    seven launches of compress, attention and combine instead of three, and
    the indexer zeroing its workspace in a launch of its own."""
    name = "pair_decode_1m_ungrouped"
    grouped = False


class PairDecodeE4M3Indexer(PairDecode):
    """pair_decode_1m with the indexer keys stored as E4M3 (d_I bytes per key)."""
    name = "pair_decode_1m_e4m3_indexer"
    ki_fmt = "mixed"


class PairDecodeFp8Indexer(PairDecode):
    """pair_decode_1m with E4M3 indexer queries and keys, scored on the FP8
    matrix cores."""
    name = "pair_decode_1m_fp8_indexer"
    ki_fmt = "mixed"
    qi_fmt = "mixed"


class PairDecodeMxfp4Indexer(PairDecode):
    """pair_decode_1m with MXFP4 indexer keys (E2M1 codes and an E8M0 scale
    per 32 dims, 68 bytes per key); the step quantises the newest key."""
    name = "pair_decode_1m_mxfp4_indexer"
    ki_fmt = "mxfp4"


class PairDecodeFp4Indexer(PairDecode):
    """pair_decode_1m with E4M3 indexer queries against MXFP4 keys: codes
    and block scales go to the scaled FP4 matrix cores as stored."""
    name = "pair_decode_1m_fp4_indexer"
    ki_fmt = "mxfp4"
    qi_fmt = "mixed"


class PairDecodeRmsNorm(PairDecode):
    """pair_decode_1m with RMSNorm of the new compressed entries (in the compress
    epilogue) and of the queries (in the attention prologue)."""
    name = "pair_decode_1m_rmsnorm"
    rmsnorm = True


class PairDecodeOverlap(PairDecode):
    """pair_decode_1m with overlapping CSA compression windows: the new CSA
    entry pools its block and the 4 tokens before it."""
    name = "pair_decode_1m_overlap"
    overlap = 4


class CsaDecode(PairDecode):
    name = "csa_decode_128k"

    def __init__(self, lac, synth, dev, sets, seed=2, B=32, ctx=131072):
        self.lac, self.B, self.ctx = lac, B, ctx
        self.sets = [synth.csa_decode(seed=seed + 1000 * s, B=B, ctx=ctx, device=dev)
                     for s in range(sets)]
        c = self.c = self.sets[0]
        self.idx = torch.empty((B, 1, c["k"]), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(c["q"])
        self.ws_idx = torch.empty(lac.indexer_topk_workspace_size(B, 1, c["N"], c["k"]),
                                  dtype=torch.uint8, device=dev)
        self.ws = torch.empty(lac.attend_workspace_size(B, 1, c["H"], c["D"], c["r"], 1, c["k"],
                                                        c["W"]), dtype=torch.uint8, device=dev)

    def step(self, i):
        lac, c, s = self.lac, self.c, self.sets[i % len(self.sets)]
        lac.indexer_topk(s["qI"], s["w"], s["KI"], m=c["m"], k=c["k"], q_pos0=self.ctx,
                         topk_idx=self.idx, workspace=self.ws_idx)
        lac.csa_attend(s["q"], s["ckv"], self.idx, s["raw"], c["W"], q_pos0=self.ctx,
                       raw_pos0=c["raw_pos0"], rope_dims=c["r"], out=self.out, workspace=self.ws)

    def bytes_per_step(self):
        c = self.c
        return self.B * (c["N"] * c["dI"] * 2 + c["HI"] * c["dI"] * 2 + c["HI"] * 4
                         + (c["k"] + c["W"]) * c["D"] * 2 + 2 * c["H"] * c["D"] * 2)

    def config(self):
        c = self.c
        return {"workload": self.name, "batch": self.B, "ctx": self.ctx, "topk": c["k"],
                "window": c["W"], "heads": c["H"], "kv_dim": c["D"],
                "indexer": f"{c['HI']}x{c['dI']} bf16", "csa_entries": c["N"], "kv_format": "bf16",
                "cache_sets": len(self.sets)}

    def cpu_sample(self):
        import oracle
        from oracle import chain
        import synth

        c, s = self.c, self.sets[0]
        h = {k_: synth.host_bytes(v[:1]) for k_, v in s.items() if isinstance(v, torch.Tensor)}
        t0 = time.perf_counter()
        idx, _, _ = chain.csa_select(h["qI"], h["w"], h["KI"], "bf16", 1, 1, c["HI"], c["dI"],
                                     c["N"], self.ctx, c["m"], c["k"])
        oracle.attend(h["q"], oracle.BF16, h["ckv"], oracle.BF16, c["N"], 0, idx, c["k"], c["m"],
                      h["raw"], c["W"], c["raw_pos0"], c["W"], None, 0.0, 1, 1, c["H"], c["D"],
                      c["r"], 1e4, self.ctx)
        el = time.perf_counter() - t0
        return {"value": 1.0 / el, "unit": self.unit, "seconds": el,
                "sample": "the decode step of 1 of the 32 sequences, cache set 0"}


class ChunkPrefill:
    name = "csa_chunk_prefill"
    unit = "TFLOP/s"
    timer_kernel = "indexer_score"
    ctx = 262144
    idx_fmt = "bf16"        # indexer queries and keys; "mixed": E4M3 codes

    def __init__(self, lac, synth, dev, sets, seed=3):
        self.lac = lac
        c = self.c = synth.csa_chunk_prefill(seed=seed, ctx=self.ctx, idx_fmt=self.idx_fmt,
                                             device=dev)
        T = c["chunk"]
        self.idx = torch.empty((1, T, c["k"]), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(c["q"])
        self.ws_idx = torch.empty(lac.indexer_topk_workspace_size(1, T, c["N"], c["k"]),
                                  dtype=torch.uint8, device=dev)
        self.ws = torch.empty(lac.attend_workspace_size(1, T, c["H"], c["D"], c["r"], 1, c["k"],
                                                        c["W"]), dtype=torch.uint8, device=dev)
        self.sets = [c]

    def step(self, i):
        lac, c = self.lac, self.c
        n0, n1 = c["N_ctx"], c["N"]
        lac.csa_compress(c["raw"][:, c["W"] - 1:], c["z"], c["ckv"][:, n0:n1], m=c["m"],
                         rope_dims=c["r"], pos0=c["pos0"], T=c["chunk"])
        lac.csa_compress(c["kI_raw"], c["zI"], c["KI"][:, n0:n1], m=c["m"], rope_dims=0,
                         pos0=c["pos0"])
        lac.indexer_topk(c["qI"], c["w"], c["KI"], m=c["m"], k=c["k"], q_pos0=c["q_pos0"],
                         topk_idx=self.idx, workspace=self.ws_idx)
        lac.csa_attend(c["q"], c["ckv"], self.idx, c["raw"], c["W"], q_pos0=c["q_pos0"],
                       raw_pos0=c["raw_pos0"], rope_dims=c["r"], out=self.out, workspace=self.ws)

    def indexer_flops(self):
        c = self.c
        nv = sum(min(c["N"], (c["q_pos0"] + i) // c["m"]) for i in range(c["chunk"]))
        return nv * c["HI"] * c["dI"] * 2

    def flops_per_step(self):
        c = self.c
        att = 0
        for i in range(c["chunk"]):
            t = c["q_pos0"] + i
            nv = min(c["N"], t // c["m"])
            att += (min(c["k"], nv) + min(c["W"], t + 1)) * c["H"] * c["D"] * 4
        return self.indexer_flops() + att

    def tokens_per_step(self):
        return self.c["chunk"]

    def config(self):
        c = self.c
        return {"workload": self.name, "batch": 1, "ctx": c["q_pos0"], "chunk": c["chunk"],
                "topk": c["k"], "window": c["W"], "heads": c["H"], "kv_dim": c["D"],
                "indexer": (f"{c['HI']}x{c['dI']} bf16" if self.idx_fmt == "bf16" else
                            f"{c['HI']}x{c['dI']}, e4m3 queries and keys (scaled fp8 mfma)"
                            if self.idx_fmt == "mixed" else
                            f"{c['HI']}x{c['dI']}, e4m3 queries, mxfp4 keys (scaled fp4 mfma)"),
                "csa_entries": c["N"], "kv_format": "bf16"}

    def cpu_sample(self):
        import oracle
        from oracle import chain
        import synth

        c = self.c
        h = {k_: synth.host_bytes(v) for k_, v in c.items() if isinstance(v, torch.Tensor)}
        rows = [(0, i) for i in range(0, c["chunk"], 1024)]       # 4 of 4096 queries
        t0 = time.perf_counter()
        qf, kf = ("mixed", "mxfp4") if self.idx_fmt == "fp4" else (self.idx_fmt, self.idx_fmt)
        idx, _, _ = chain.csa_select(h["qI"], h["w"], h["KI"], qf, 1, c["chunk"], c["HI"],
                                     c["dI"], c["N"], c["q_pos0"], c["m"], c["k"], rows, k_fmt=kf)
        oracle.attend(h["q"], oracle.BF16, h["ckv"], oracle.BF16, c["N"], 0, idx, c["k"], c["m"],
                      h["raw"], c["T_raw"], c["raw_pos0"], c["W"], None, 0.0, 1, c["chunk"],
                      c["H"], c["D"], c["r"], 1e4, c["q_pos0"], rows)
        el = time.perf_counter() - t0
        fl = self.flops_per_step() * len(rows) / c["chunk"]
        return {"value": fl / el / 1e12, "unit": self.unit, "seconds": el,
                "sample": "indexer + top-k + attention for 4 of the 4096 queries (the chunk's "
                          "compression excluded), FLOPs scaled by 4/4096"}


class ChunkPrefill1M(ChunkPrefill):
    """csa_chunk_prefill with the chunk of 4096 queries ending at 2^20 tokens:
    262144 compressed entries per query row (4.3 GB of fp32 scores in the
    indexer workspace), each row's top 2048 by the one-workgroup-per-row
    selection."""
    name = "csa_chunk_prefill_1m"
    ctx = (1 << 20) - 4096


class ChunkPrefillFp8Indexer(ChunkPrefill):
    """csa_chunk_prefill with E4M3 indexer queries and keys: the score matrix
    on gfx950's block-scaled FP8 product (unit scales), the rest as in the
    bf16 workload; the score kernel is priced against the FP8 dense peak."""
    name = "csa_chunk_prefill_fp8_indexer"
    idx_fmt = "mixed"


class ChunkPrefillFp4Indexer(ChunkPrefill):
    """csa_chunk_prefill with E4M3 indexer queries against MXFP4 keys: the
    score matrix on gfx950's block-scaled FP4 product; the chunk's new keys
    are quantised by the compress call.  Priced against the FP8 dense peak
    (the products' E4M3 side)."""
    name = "csa_chunk_prefill_fp4_indexer"
    idx_fmt = "fp4"


class HcaPrefill(ChunkPrefill):
    name = "hca_prefill_8k"
    timer_kernel = "attend"

    def __init__(self, lac, synth, dev, sets, seed=1):
        self.lac = lac
        c = self.c = synth.hca_prefill(seed=seed, device=dev)
        self.hkv = torch.empty((1, c["T"] // c["m"], c["D"]), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty_like(c["q"])
        self.ws = torch.empty(lac.attend_workspace_size(1, c["T"], c["H"], c["D"], c["r"], 1,
                                                        c["T"] // c["m"], c["W"]),
                              dtype=torch.uint8, device=dev)
        self.sets = [c]

    def step(self, i):
        lac, c = self.lac, self.c
        lac.hca_compress(c["kv"], c["z"], self.hkv, m=c["m"], rope_dims=c["r"], pos0=0)
        lac.hca_attend(c["q"], self.hkv, c["kv"], c["W"], m=c["m"], q_pos0=0, raw_pos0=0,
                       rope_dims=c["r"], out=self.out, workspace=self.ws)

    def flops_per_step(self):
        c = self.c
        tot = 0
        for t in range(c["T"]):
            tot += (min(c["T"] // c["m"], t // c["m"]) + min(c["W"], t + 1)) * c["H"] * c["D"] * 4
        return tot

    def tokens_per_step(self):
        return self.c["T"]

    def config(self):
        c = self.c
        return {"workload": self.name, "batch": 1, "tokens": c["T"], "m_hca": c["m"],
                "window": c["W"], "heads": c["H"], "kv_dim": c["D"], "kv_format": "bf16"}

    def cpu_sample(self):
        import oracle
        from oracle import chain
        import synth

        c = self.c
        h = {k_: synth.host_bytes(v) for k_, v in c.items() if isinstance(v, torch.Tensor)}
        rows = [(0, t) for t in range(0, c["T"], 64)]
        t0 = time.perf_counter()
        hkv = chain.compress_store(h["kv"], h["z"], "bf16", "bf16", 1, c["T"], c["D"], c["m"],
                                   c["r"], 1e4, 0)
        oracle.attend(h["q"], oracle.BF16, hkv, oracle.BF16, c["T"] // c["m"], 1, None, 0,
                      c["m"], h["kv"], c["T"], 0, c["W"], None, 0.0, 1, c["T"], c["H"], c["D"],
                      c["r"], 1e4, 0, rows)
        el = time.perf_counter() - t0
        fl = self.flops_per_step() * len(rows) / c["T"]
        return {"value": fl / el / 1e12, "unit": self.unit, "seconds": el,
                "sample": "compression of all 8192 tokens + attention of 128 of the 8192 "
                          "queries, FLOPs scaled by 128/8192"}


class ProjectionPrefill:
    """The grouped output projection of a 4096-token prefill chunk: 64 heads of
    512 in 8 groups, each projected to 1024, then the 8192-wide concatenation
    to the model width 7168."""
    name = "grouped_projection_prefill"
    unit = "TFLOP/s"
    kernel = "gemm_nt_bf16_kernel (both products)"
    timer_kernel = "project"

    def __init__(self, lac, synth, dev, sets, seed=5):
        self.lac = lac
        c = self.c = synth.projection(seed=seed, device=dev)
        self.out = torch.empty((c["T"], c["d"]), dtype=torch.bfloat16, device=dev)
        self.ws = torch.empty(lac.grouped_projection_workspace_size(c["T"], c["H"], c["D"], c["G"], c["d_g"], c["d"]),
                              dtype=torch.uint8, device=dev)
        self.sets = [c]

    def step(self, i):
        c = self.c
        self.lac.grouped_output_projection(c["attn"], c["w1"], c["w2"], out=self.out,
                                           workspace=self.ws)

    def flops_per_token(self):
        c = self.c
        return 2 * c["H"] * c["D"] * c["d_g"] + 2 * c["G"] * c["d_g"] * c["d"]

    def flops_per_step(self):
        return self.c["T"] * self.flops_per_token()

    def tokens_per_step(self):
        return self.c["T"]

    def config(self):
        c = self.c
        return {"workload": self.name, "tokens": c["T"], "heads": c["H"], "head_dim": c["D"],
                "groups": c["G"], "d_g": c["d_g"], "d_model": c["d"], "dtype": "bf16"}

    def cpu_sample(self):
        import oracle
        import synth

        c = self.c
        n = 1024
        attn = synth.host_bytes(c["attn"][:n])
        w1, w2 = synth.host_bytes(c["w1"]), synth.host_bytes(c["w2"])
        t0 = time.perf_counter()
        oracle.grouped_projection(attn, w1, w2, oracle.BF16, n, c["H"], c["D"], c["G"],
                                  c["d_g"], c["d"], y_dtype=oracle.BF16)
        el = time.perf_counter() - t0
        return {"value": n * self.flops_per_token() / el / 1e12, "unit": self.unit,
                "seconds": el, "sample": f"{n} of the {c['T']} tokens"}


class ProjectionDecode(ProjectionPrefill):
    """The grouped output projection of one decode step of 4 sequences (4
    tokens): the weights (176 MB) stream from HBM once per call."""
    name = "grouped_projection_decode"
    unit = "tokens/s"
    kernel = "grouped_output_projection call (2 product + 2 sum launches)"

    def __init__(self, lac, synth, dev, sets, seed=6):
        self.lac = lac
        c = self.c = synth.projection(seed=seed, T=4, device=dev)
        self.out = torch.empty((c["T"], c["d"]), dtype=torch.bfloat16, device=dev)
        self.ws = torch.empty(lac.grouped_projection_workspace_size(c["T"], c["H"], c["D"], c["G"],
                                                                    c["d_g"], c["d"]),
                              dtype=torch.uint8, device=dev)
        self.sets = [c]

    def bytes_per_step(self):
        c = self.c
        K1 = c["H"] // c["G"] * c["D"]
        weights = (c["G"] * c["d_g"] * K1 + c["d"] * c["G"] * c["d_g"]) * 2
        acts = c["T"] * (c["H"] * c["D"] + c["G"] * c["d_g"] * 2 + c["d"]) * 2
        return weights + acts

    def cpu_sample(self):
        import oracle
        import synth

        c = self.c
        attn = synth.host_bytes(c["attn"])
        w1, w2 = synth.host_bytes(c["w1"]), synth.host_bytes(c["w2"])
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 10.0:
            oracle.grouped_projection(attn, w1, w2, oracle.BF16, c["T"], c["H"], c["D"], c["G"],
                                      c["d_g"], c["d"], y_dtype=oracle.BF16)
            reps += 1
        el = time.perf_counter() - t0
        return {"value": reps * c["T"] / el, "unit": self.unit, "seconds": el,
                "sample": f"{reps} whole calls of {c['T']} tokens"}


class BulkCompress1M:
    """Building the compressed caches of a 1M-token CSA + HCA layer pair from
    raw activations (4 sequences of 2^20 tokens): CSA entries (m = 4, E4M3 +
    bf16 rotated dims), indexer keys (m = 4, bf16) and HCA entries (m' = 128,
    E4M3 + bf16), each layer from its own raw KV and logits."""
    name = "bulk_compress_1m"
    unit = "GB/s"
    timer_kernel = "compress"
    kernel = "compress_kernel (CSA entries, m = 4)"

    def __init__(self, lac, synth, dev, sets, seed=4, B=4, T=1 << 20):
        self.lac = lac
        c = self.c = synth.bulk_compress(seed=seed, B=B, T=T, device=dev)
        self.r, self.m, self.mh = 64, 4, 128
        D, dI = c["D"], c["dI"]
        row = D - self.r + 2 * self.r
        self.ckv = torch.empty((B, T // self.m, row), dtype=torch.uint8, device=dev)
        self.KI = torch.empty((B, T // self.m, dI), dtype=torch.bfloat16, device=dev)
        self.hkv = torch.empty((B, T // self.mh, row), dtype=torch.uint8, device=dev)
        self.sets = [c]

    def step(self, i):
        lac, c = self.lac, self.c
        lac.csa_compress(c["kv"], c["z"], self.ckv, m=self.m, rope_dims=self.r, pos0=0)
        lac.csa_compress(c["kI_raw"], c["zI"], self.KI, m=self.m, rope_dims=0, pos0=0)
        lac.hca_compress(c["kv_hca"], c["z_hca"], self.hkv, m=self.mh, rope_dims=self.r, pos0=0)

    def tokens_per_step(self):
        return self.c["B"] * self.c["T"]

    def kernel_bytes(self):
        """Bytes of the timed launch (the CSA entries): raw KV and logits read,
        entries written."""
        c = self.c
        return c["B"] * c["T"] * c["D"] * 2 * 2 + self.ckv.numel()

    def bytes_per_step(self):
        c = self.c
        rd = c["B"] * c["T"] * (2 * c["D"] + 2 * c["dI"] + (2 * c["D"] if "kv_hca" in c else 0)) * 2
        wr = self.ckv.numel() + self.KI.numel() * 2 + (self.hkv.numel() if "kv_hca" in c else 0)
        return rd + wr

    def config(self):
        c = self.c
        return {"workload": self.name, "batch": c["B"], "tokens": c["T"], "kv_dim": c["D"],
                "indexer_dim": c["dI"], "m": self.m, "m_hca": self.mh, "rope_dims": self.r,
                "in_format": "bf16", "out_format": "csa/hca e4m3 + bf16 rope dims, keys bf16"}

    def cpu_sample(self):
        import oracle
        import synth

        c = self.c
        n = 4096                      # raw tokens of sequence 0 per layer
        h = {k_: synth.host_bytes(c[k_][0, :n]) for k_ in ("kv", "z", "kI_raw", "zI", "kv_hca",
                                                            "z_hca") if k_ in c}
        t0 = time.perf_counter()
        oracle.compress(h["kv"], h["z"], oracle.BF16, 1, n, c["D"], self.m, self.r)
        oracle.compress(h["kI_raw"], h["zI"], oracle.BF16, 1, n, c["dI"], self.m, 0)
        if "kv_hca" in h:
            oracle.compress(h["kv_hca"], h["z_hca"], oracle.BF16, 1, n, c["D"], self.mh, self.r)
        el = time.perf_counter() - t0
        frac = n / (c["B"] * c["T"])
        return {"value": self.bytes_per_step() * frac / el / 1e9, "unit": self.unit,
                "seconds": el, "sample": f"the first {n} tokens of sequence 0 (every cache), "
                                         "bytes scaled by the same fraction"}


class BulkCompress128K(BulkCompress1M):
    """Building the CSA caches of 32 sequences of 131072 tokens (bf16 entries
    and indexer keys) from raw activations."""
    name = "bulk_compress_128k"
    kernel = "compress_kernel (CSA entries, m = 4)"

    def __init__(self, lac, synth, dev, sets, seed=2, B=32, T=131072):
        self.lac = lac
        c = self.c = synth.bulk_compress(seed=seed, B=B, T=T, hca=False, device=dev)
        self.r, self.m, self.mh = 64, 4, 128
        self.ckv = torch.empty((B, T // self.m, c["D"]), dtype=torch.bfloat16, device=dev)
        self.KI = torch.empty((B, T // self.m, c["dI"]), dtype=torch.bfloat16, device=dev)
        self.sets = [c]

    def step(self, i):
        lac, c = self.lac, self.c
        lac.csa_compress(c["kv"], c["z"], self.ckv, m=self.m, rope_dims=self.r, pos0=0)
        lac.csa_compress(c["kI_raw"], c["zI"], self.KI, m=self.m, rope_dims=0, pos0=0)

    def kernel_bytes(self):
        c = self.c
        return c["B"] * c["T"] * c["D"] * 2 * 2 + self.ckv.numel() * 2

    def config(self):
        d = super().config()
        d["out_format"] = "bf16"
        d.pop("m_hca")
        return d


WORKLOADS = {w.name: w for w in (PairDecode, PairDecodeUngrouped, PairDecodeE4M3Indexer,
                                  PairDecodeFp8Indexer,
                                  PairDecodeMxfp4Indexer, PairDecodeFp4Indexer, ChunkPrefillFp8Indexer,
                                  ChunkPrefillFp4Indexer,
                                  PairDecodeRmsNorm, PairDecodeOverlap, CsaDecode,
                                  ChunkPrefill, ChunkPrefill1M, HcaPrefill,
                                  ProjectionPrefill, ProjectionDecode,
                                  BulkCompress1M, BulkCompress128K)}



TIMER_EVERY = 8      # timed steps per launch-timer sample


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="pair_decode_1m", choices=sorted(WORKLOADS))
    ap.add_argument("--sets", type=int, default=3, help="rotating cache sets (decode)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus 1 only)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 1 << 30, "launches": 5}))
        return

    import long_context_attention_compressor_amd as lac
    import synth

    wl = WORKLOADS[args.workload](lac, synth, dev, args.sets)
    # one marshalled call list per cache set (the binding records, not runs)
    lists = []
    for i in range(len(wl.sets)):
        with lac.CallList() as cl:
            wl.step(i)
        lists.append(cl)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        lists[i % len(lists)].run()
    torch.cuda.synchronize()
    # The dominant kernel is timed by the library's launch timer on every
    # TIMER_EVERY-th timed step: each armed step records two events around the
    # launch, which cost the 1M-token decode step about 7 us.
    n_timed = (args.steps + TIMER_EVERY - 1) // TIMER_EVERY
    timers = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_timed)]
    for a, b in timers:          # PyTorch creates the HIP events on their first record
        a.record()
        b.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % TIMER_EVERY == 0:
            lac.time_next_launch(wl.timer_kernel, *timers[i // TIMER_EVERY])
        lists[(args.warmup + i) % len(lists)].run()
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms = el * 1e3 / args.steps
    kern_ms = sum(a.elapsed_time(b) for a, b in timers) / n_timed

    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": wl.config()}
    if isinstance(wl, ProjectionDecode):
        # HBM-bound: the timed span brackets the whole call (4 launches)
        res["value"] = wl.tokens_per_step() / (ms / 1e3)
        res["unit"] = "tokens/s"
        ach = wl.bytes_per_step() / (kern_ms / 1e3) / 1e9
        res["hbm_gbps"] = wl.bytes_per_step() / (ms / 1e3) / 1e9
        res["roofline"] = {"bound": "hbm", "kernel": wl.kernel, "achieved": round(ach, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                           "traffic_unit": "B/call", "launch_ms": round(kern_ms, 5),
                           "step_frac": round(res["hbm_gbps"] / HBM_PEAK_GBS, 4)}
    elif isinstance(wl, BulkCompress1M):
        res["value"] = wl.bytes_per_step() / (ms / 1e3) / 1e9
        res["unit"] = "GB/s"
        res["tokens_per_s"] = wl.tokens_per_step() / (ms / 1e3)
        ach = wl.kernel_bytes() / (kern_ms / 1e3) / 1e9
        res["roofline"] = {"bound": "hbm", "kernel": wl.kernel, "achieved": round(ach, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                           "traffic_unit": "B/launch", "launch_ms": round(kern_ms, 5),
                           "step_frac": round(res["value"] / HBM_PEAK_GBS, 4)}
    elif wl.unit == "tokens/s":
        res["value"] = wl.tokens_per_step() / (ms / 1e3)
        res["unit"] = "tokens/s"
        res["hbm_gbps"] = wl.bytes_per_step() / (ms / 1e3) / 1e9
        ach = wl.indexer_bytes_per_launch() / (kern_ms / 1e3) / 1e9
        res["roofline"] = {"bound": "hbm", "kernel": "score_bf16_kernel (indexer scores)",
                           "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(ach / HBM_PEAK_GBS, 4),
                           "traffic": _score_traffic(wl.name), "traffic_unit": "B/launch",
                           "launch_ms": round(kern_ms, 5),
                           "step_frac": round(res["hbm_gbps"] / HBM_PEAK_GBS, 4)}
    else:
        fl = wl.flops_per_step()
        res["value"] = fl / (ms / 1e3) / 1e12
        res["unit"] = "TFLOP/s"
        launches = 1
        if isinstance(wl, ProjectionPrefill):
            # one timed span holds both products (the same kernel, launched twice)
            kfl, kname, traffic, launches = fl, wl.kernel, _project_traffic(), 2
        elif isinstance(wl, HcaPrefill):
            kfl, kname, traffic = fl, "attend_mfma_kernel (HCA attention)", None
        else:
            kfl, kname = wl.indexer_flops(), "score_prefill_kernel (indexer scores)"
            traffic = _score_traffic(wl.name)
        # the score kernel's own dtype sets its peak (E4M3 indexer: FP8 dense)
        kpeak = FP8_PEAK_TFLOPS if getattr(wl, "idx_fmt", "bf16") != "bf16" else BF16_PEAK_TFLOPS
        ach = kfl / (kern_ms / 1e3) / 1e12
        res["roofline"] = {"bound": "mfma", "kernel": kname, "achieved": round(ach, 2),
                           "peak": kpeak, "unit": "TFLOP/s",
                           "frac": round(ach / kpeak, 4), "traffic": traffic,
                           "traffic_unit": "B/launch",
                           "launch_ms": round(kern_ms / launches, 5),
                           "step_frac": round(res["value"] / BF16_PEAK_TFLOPS, 4)}
    res["host_enqueue_ms_per_step"] = round((t_enq - t0) * 1e3 / args.steps, 5)
    res["roofline"]["timed_launches"] = n_timed
    if not args.no_cpu:
        import oracle
        cb = wl.cpu_sample()
        res["cpu_baseline"] = {"value": cb["value"], "unit": cb["unit"],
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "sample": cb["sample"], "seconds": round(cb["seconds"], 2)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
