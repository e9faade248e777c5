"""GPU parity of grouped_output_projection against the oracle (QbitAI rewrite,
grouped output projection step: heads in g groups, each group projected to
d_g, the concatenation projected back to d).  The oracle rounds the
intermediate to bfloat16 as the library stores it.  Shapes span several
256 x 256 output tiles with a ragged last row band, and the few-token path
(64 tokens or fewer: split contraction, fixed-order sums); the full-size case (4096
tokens, 64 heads of 512, 8 groups of 1024, d = 7168) is checked on sampled
tokens, which the oracle computes one by one (tokens are independent)."""
import numpy as np
import pytest
import torch

import long_context_attention_compressor_amd as lac
import oracle
import synth
from parity import as_f64, check_projection, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(T, H, D, G, d_g, d, seed, rows=None):
    print(f"projection T={T} H={H} D={D} G={G} d_g={d_g} d={d} seed={seed}", flush=True)
    inp = synth.projection(seed, T, H, D, G, d_g, d)
    out = lac.grouped_output_projection(inp["attn"].to(DEV), inp["w1"].to(DEV),
                                        inp["w2"].to(DEV))
    torch.cuda.synchronize()
    g = as_f64(out)
    if rows is None:
        rows = np.arange(T)
    rows = np.asarray(rows)
    attn = np.ascontiguousarray(host(inp["attn"])[rows])
    ref = oracle.grouped_projection(attn, host(inp["w1"]), host(inp["w2"]), oracle.BF16,
                                    len(rows), H, D, G, d_g, d, y_dtype=oracle.BF16)
    check_projection(g[rows], ref, as_f64(inp["attn"][torch.from_numpy(rows)]),
                     as_f64(inp["w1"]), as_f64(inp["w2"]), f"T={T} G={G}")


def test_several_tiles_with_a_ragged_row_band():
    _run(300, 8, 128, 2, 256, 512, 50)


def test_one_group_is_two_plain_products():
    _run(64, 4, 64, 1, 256, 256, 51)


def test_single_token():
    _run(1, 16, 128, 4, 512, 768, 52)


def test_eight_groups_of_the_512_wide_heads():
    _run(257, 64, 512, 8, 256, 1024, 53)


def test_full_size_prefill_chunk_on_sampled_tokens():
    T = 4096
    rows = np.array([0, 1, 255, 256, 1000, 2047, 2048, 3333, 4094, 4095])
    _run(T, 64, 512, 8, 1024, 7168, 54, rows)


def test_ragged_full_width_on_sampled_tokens():
    T = 777
    rows = np.array([0, 511, 512, 700, 767, 768, 776])
    _run(T, 64, 512, 8, 1024, 7168, 55, rows)


@pytest.mark.parametrize("T", [1, 4, 32, 33, 64])
def test_decode_token_counts_full_width(T):
    # 64 tokens or fewer take the split-contraction path (one or two token
    # tiles); every token is checked
    _run(T, 64, 512, 8, 1024, 7168, 60 + T)


def test_decode_path_small_groups():
    _run(5, 8, 128, 2, 256, 512, 70)


def test_first_token_count_on_the_tiled_path():
    _run(65, 16, 128, 4, 256, 512, 71)


def test_zero_tokens_is_a_no_op():
    attn = torch.zeros((0, 8, 64), dtype=torch.bfloat16, device=DEV)
    w1 = torch.zeros((2, 256, 256), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((256, 512), dtype=torch.bfloat16, device=DEV)
    out = lac.grouped_output_projection(attn, w1, w2)
    assert out.shape == (0, 256)


def test_unsupported_widths_are_refused():
    attn = torch.zeros((4, 8, 64), dtype=torch.bfloat16, device=DEV)
    w1 = torch.zeros((2, 100, 256), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((256, 200), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(lac.LacError):
        lac.grouped_output_projection(attn, w1, w2)


def test_small_workspace_is_refused():
    attn = torch.zeros((4, 8, 64), dtype=torch.bfloat16, device=DEV)
    w1 = torch.zeros((2, 256, 256), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((256, 512), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((4, 256), dtype=torch.bfloat16, device=DEV)
    need = lac.grouped_projection_workspace_size(4, 8, 64, 2, 256, 256)
    assert need >= 4 * 512 * 2
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    st = lac.lib.grouped_output_projection(attn.data_ptr(), w1.data_ptr(), w2.data_ptr(), 4, 8,
                                           64, 2, 256, 256, out.data_ptr(), ws.data_ptr(),
                                           need - 2, None)
    assert st == 3      # LAC_ERR_WORKSPACE
