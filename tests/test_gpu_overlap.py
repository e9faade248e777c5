"""GPU parity of csa_compress_overlap against the oracle's overlapping CSA
windows (QbitAI rewrite: HCA's compression has none of the overlap CSA's
has; reading: entry j pools [max(0, p_j - o), p_j + m) and is rotated at
p_j).  Seeded inputs; windows clipped at position 0, sequences with
different leading rows, ragged block counts, windows split over several
lanes (m + o > 8), and every output format."""
import numpy as np
import pytest
import torch

import long_context_attention_compressor_amd as lac
import oracle
import synth
from parity import check_compressed, host

pytestmark = pytest.mark.gpu
DEV = "cuda"
FMTS = {"f32": torch.float32, "bf16": torch.bfloat16}


def _run(B, T, D, m, o, r, in_fmt, out_fmt, pos0, seed):
    print(f"compress overlap B={B} T={T} D={D} m={m} o={o} r={r} {in_fmt}->{out_fmt} "
          f"pos0={pos0}", flush=True)
    lead = max(min(o, p) for p in pos0)
    rows = T + lead
    x = synth.store(synth.normal(seed, "x", (B, rows, D)), in_fmt)
    z = synth.store(synth.normal(seed, "z", (B, rows, D)), in_fmt)
    N = T // m
    if out_fmt == "mixed":
        out = torch.full((B, N, D + r), 0x55, dtype=torch.uint8, device=DEV)
    else:
        out = torch.full((B, N, D), 7.0, dtype=FMTS[out_fmt], device=DEV)
    lac.csa_compress(x.to(DEV), z.to(DEV), out, m=m, rope_dims=r, pos0=pos0, T=T, overlap=o)
    torch.cuda.synchronize()
    ref = oracle.compress_overlap(host(x), host(z), synth.DTYPE_CODES[in_fmt], B, T, D, m, o, r,
                                  10000.0, pos0, x_bstride=rows, z_bstride=rows)
    check_compressed(out, ref, out_fmt, D, r)


@pytest.mark.parametrize("o", [1, 4, 7])
def test_f32_prefill_from_position_zero(o):
    _run(2, 64, 128, 4, o, 64, "f32", "f32", [0, 8], 10 + o)


def test_bf16_chunk_after_a_long_context():
    # a chunk whose first window reaches back into the context before it
    _run(1, 4 * 50 + 2, 512, 4, 4, 64, "bf16", "bf16", [262144], 20)


def test_bf16_to_mixed_decode_blocks_at_1m_positions():
    # the newest block of each sequence (one entry), from 8 raw rows
    _run(4, 4, 512, 4, 4, 64, "bf16", "mixed", [(1 << 20) - 4] * 4, 21)


def test_sequences_with_different_leading_rows():
    _run(3, 40, 256, 4, 6, 64, "bf16", "bf16", [0, 4, 100], 22)


@pytest.mark.parametrize("m,o", [(16, 16), (16, 13), (64, 64), (8, 120)])
def test_windows_split_over_several_lanes(m, o):
    _run(2, 3 * m + 5, 128, m, o, 32, "bf16", "mixed", [0, 4 * m], 30 + m + o)


def test_overlap_zero_is_plain_compression():
    B, T, D, m = 2, 48, 128, 4
    x = synth.store(synth.normal(40, "x", (B, T, D)), "bf16").to(DEV)
    z = synth.store(synth.normal(40, "z", (B, T, D)), "bf16").to(DEV)
    a = torch.empty((B, T // m, D), dtype=torch.bfloat16, device=DEV)
    b = torch.empty_like(a)
    lac.csa_compress(x, z, a, m=m, pos0=[0, 64])
    lac.lib.csa_compress_overlap  # the entry point exists
    lac.csa_compress(x, z, b, m=m, pos0=[0, 64], overlap=0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_refuses_an_overlap_out_of_range():
    x = torch.zeros((1, 300, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((1, 1, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(lac.LacError):
        lac.csa_compress(x, x, out, m=4, pos0=[400], T=4, overlap=253)
