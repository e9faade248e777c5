"""Seeded synthetic inputs for hybrid compressed attention.

This module draws random tensors and converts them to their stored formats
with PyTorch's own conversions (``.to(torch.bfloat16)``,
``.to(torch.float8_e4m3fn)``).  It holds none of the method's arithmetic and
imports neither the GPU library nor the oracle; both sides are fed the same
bytes from here.

Every tensor is drawn by name: its generator is seeded from
``crc32(f"{seed}/{name}")``, so the order in which tensors are drawn does not
matter and a tensor can be redrawn alone.  Drawing happens on ``device``
(CPU for the small cases, the GPU for the large workloads, where a host copy
of the sampled part is then handed to the oracle).

Stored formats:
  * ``f32``   float32
  * ``bf16``  bfloat16
  * ``mixed`` uint8 rows of ``(D - r) + 2 r`` bytes: the first ``D - r`` dims
    as FP8 E4M3 ("fn" variant) and the last ``r`` dims as bfloat16
"""
from __future__ import annotations

import zlib

import torch

F32, BF16, MIXED, MXFP4 = 0, 1, 2, 4
DTYPE_CODES = {"f32": F32, "bf16": BF16, "mixed": MIXED, "mxfp4": MXFP4}


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(zlib.crc32(f"{seed}/{name}".encode()) & 0x7FFFFFFFFFFFFFFF)
    return g


def normal(seed: int, name: str, shape, std: float = 1.0, device="cpu") -> torch.Tensor:
    """float32 draws from N(0, std^2)."""
    t = torch.randn(tuple(shape), generator=_gen(seed, name, device), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def uniform(seed: int, name: str, shape, device="cpu") -> torch.Tensor:
    """float32 draws from U(0, 1)."""
    return torch.rand(tuple(shape), generator=_gen(seed, name, device), device=device,
                      dtype=torch.float32)


def mxfp4_rows(seed: int, name: str, shape, d: int, scale_lo: int = 124, scale_hi: int = 130,
               device="cpu") -> torch.Tensor:
    """Random MXFP4 rows [*shape, d/2 + d/32] uint8: uniform code bytes (two
    E2M1 codes each), then scale bytes drawn from [scale_lo, scale_hi]."""
    g = _gen(seed, name, device)
    codes = torch.randint(0, 256, (*shape, d // 2), generator=g, device=device, dtype=torch.int32)
    scales = torch.randint(scale_lo, scale_hi + 1, (*shape, d // 32), generator=g, device=device,
                           dtype=torch.int32)
    return torch.cat([codes, scales], dim=-1).to(torch.uint8).contiguous()


def store(t: torch.Tensor, fmt: str, rope_dims: int = 0) -> torch.Tensor:
    """Convert float32 values to a stored format with PyTorch's conversions."""
    if fmt == "f32":
        return t.contiguous()
    if fmt == "bf16":
        return t.to(torch.bfloat16).contiguous()
    if fmt == "mixed":
        D = t.shape[-1]
        r = rope_dims
        lo = t[..., : D - r].to(torch.float8_e4m3fn).view(torch.uint8)
        hi = t[..., D - r:].to(torch.bfloat16).contiguous().view(torch.uint8)
        return torch.cat([lo, hi], dim=-1).contiguous()
    raise ValueError(fmt)


def row_bytes(fmt: str, D: int, r: int) -> int:
    return {"f32": 4 * D, "bf16": 2 * D, "mixed": (D - r) + 2 * r}[fmt]


def host_bytes(t: torch.Tensor):
    """A numpy view of a (CPU) tensor's bytes, for the oracle."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


# ---------------------------------------------------------------------------
# Workloads.  Sizes follow the five configurations the method is measured on;
# each builder can be shrunk (keyword overrides) for tests that the oracle
# finishes in seconds.  Positions: query i of sequence b is at q_pos0[b] + i,
# raw row i at raw_pos0[b] + i, compressed entry j covers [j*m, j*m + m - 1].
# ---------------------------------------------------------------------------

def csa_prefill_tiny(seed=0, T=256, D=128, m=4, r=64, HI=4, dI=32, H=8, k=16, W=8,
                     device="cpu"):
    """Tiny CSA prefill in float32: compress KV and indexer keys, index,
    select, attend every query of one sequence."""
    B = 1
    return dict(
        kind="csa_prefill", fmt="f32", B=B, T=T, D=D, m=m, r=r, HI=HI, dI=dI, H=H, k=k, W=W,
        theta=10000.0, q_pos0=0, raw_pos0=0, pos0=0,
        kv=normal(seed, "kv", (B, T, D), device=device),
        z=normal(seed, "z", (B, T, D), device=device),
        kI_raw=normal(seed, "kI_raw", (B, T, dI), device=device),
        zI=normal(seed, "zI", (B, T, dI), device=device),
        qI=normal(seed, "qI", (B, T, HI, dI), device=device),
        w=uniform(seed, "w", (B, T, HI), device=device),
        q=normal(seed, "q", (B, T, H, D), device=device),
    )


def hca_prefill(seed=1, T=8192, D=128, m=128, r=64, H=16, W=128, z_std=0.5, device="cpu"):
    """HCA prefill in bf16: compress with m' tokens per entry, then dense
    attention of every query over the visible entries plus the window."""
    B = 1
    return dict(
        kind="hca_prefill", fmt="bf16", B=B, T=T, D=D, m=m, r=r, H=H, W=W, theta=10000.0,
        q_pos0=0, raw_pos0=0, pos0=0,
        kv=store(normal(seed, "kv", (B, T, D), device=device), "bf16"),
        z=store(normal(seed, "z", (B, T, D), std=z_std, device=device), "bf16"),
        q=store(normal(seed, "q", (B, T, H, D), device=device), "bf16"),
    )


def csa_decode(seed=2, B=32, ctx=131072, D=512, m=4, r=64, HI=64, dI=128, H=64, k=2048,
               W=128, fmt="bf16", device="cpu"):
    """CSA decode: one query per sequence at position ctx, all ctx/m compressed
    entries visible.  The stored caches are drawn directly."""
    N = ctx // m
    return dict(
        kind="csa_decode", fmt=fmt, B=B, D=D, m=m, r=r, HI=HI, dI=dI, H=H, k=k, W=W, N=N,
        theta=10000.0, q_pos0=ctx, raw_pos0=ctx - W + 1, T_raw=W,
        ckv=store(normal(seed, "ckv", (B, N, D), device=device), fmt, r),
        KI=store(normal(seed, "KI", (B, N, dI), device=device), "bf16"),
        raw=store(normal(seed, "raw", (B, W, D), device=device), fmt, r),
        qI=store(normal(seed, "qI", (B, 1, HI, dI), device=device), "bf16"),
        w=uniform(seed, "w", (B, 1, HI), device=device),
        q=store(normal(seed, "q", (B, 1, H, D), device=device), "bf16"),
    )


def csa_chunk_prefill(seed=3, ctx=262144, chunk=4096, D=512, m=4, r=64, HI=64, dI=128, H=64,
                      k=2048, W=128, idx_fmt="bf16", device="cpu"):
    """CSA chunked prefill: a chunk of queries appended to a long context.  The
    cache rows of the context are drawn directly; the chunk's raw KV and
    indexer keys are compressed into the rows that follow.  Indexer queries
    and keys are bf16, or E4M3 codes with idx_fmt = "mixed"; with idx_fmt =
    "fp4" the queries are E4M3 codes and the keys MXFP4 rows (random codes,
    scales 2^-3..2^3)."""
    B = 1
    N_ctx = ctx // m
    N = (ctx + chunk) // m
    T_raw = chunk + W - 1
    ckv = torch.zeros((B, N, D), dtype=torch.bfloat16, device=device)
    ckv[:, :N_ctx] = store(normal(seed, "ckv", (B, N_ctx, D), device=device), "bf16")
    if idx_fmt == "fp4":
        KI = torch.zeros((B, N, dI // 2 + dI // 32), dtype=torch.uint8, device=device)
        KI[:, :N_ctx] = mxfp4_rows(seed, "KI", (B, N_ctx), dI, device=device)
    else:
        KI = torch.zeros((B, N, dI), dtype=torch.bfloat16 if idx_fmt == "bf16" else torch.uint8,
                         device=device)
        KI[:, :N_ctx] = store(normal(seed, "KI", (B, N_ctx, dI), device=device), idx_fmt)
    return dict(
        kind="csa_chunk_prefill", fmt="bf16", B=B, D=D, m=m, r=r, HI=HI, dI=dI, H=H, k=k, W=W,
        N=N, N_ctx=N_ctx, chunk=chunk, theta=10000.0, q_pos0=ctx, raw_pos0=ctx - W + 1,
        T_raw=T_raw, pos0=ctx,
        ckv=ckv, KI=KI,
        raw=store(normal(seed, "raw", (B, T_raw, D), device=device), "bf16"),
        z=store(normal(seed, "z", (B, chunk, D), device=device), "bf16"),
        kI_raw=store(normal(seed, "kI_raw", (B, chunk, dI), device=device), "bf16"),
        zI=store(normal(seed, "zI", (B, chunk, dI), device=device), "bf16"),
        qI=store(normal(seed, "qI", (B, chunk, HI, dI), device=device),
                 "mixed" if idx_fmt == "fp4" else idx_fmt),
        w=uniform(seed, "w", (B, chunk, HI), device=device),
        q=store(normal(seed, "q", (B, chunk, H, D), device=device), "bf16"),
        idx_fmt=idx_fmt,
    )


def pair_decode(seed=4, B=4, ctx=1 << 20, D=512, m=4, m_hca=128, r=64, HI=64, dI=128, H=64,
                k=2048, W=128, ki_fmt="bf16", csa_overlap=0, qi_fmt="bf16", device="cpu"):
    """Decode of a CSA + HCA layer pair at position ctx with the KV stored as
    FP8 E4M3 plus bf16 rotated dims.  The step also compresses the newest
    complete block of each layer (CSA entry, indexer key, HCA entry) from
    bf16 activations, so every stage of the path runs in one step.  The
    indexer keys are bf16, E4M3 with ki_fmt = "mixed" (no rotated dims), or
    MXFP4 rows with ki_fmt = "mxfp4" (random codes, scales 2^-3..2^3);
    indexer queries bf16 or E4M3 likewise with qi_fmt.
    With csa_overlap > 0 the newest CSA block comes with the csa_overlap raw
    rows before it (overlapping compression windows)."""
    N = ctx // m
    Nh = ctx // m_hca
    return dict(
        kind="pair_decode", fmt="mixed", B=B, D=D, m=m, m_hca=m_hca, r=r, HI=HI, dI=dI, H=H,
        k=k, W=W, N=N, Nh=Nh, theta=10000.0, q_pos0=ctx, raw_pos0=ctx - W + 1, T_raw=W,
        ckv=store(normal(seed, "ckv", (B, N, D), device=device), "mixed", r),
        KI=(mxfp4_rows(seed, "KI", (B, N), dI, device=device) if ki_fmt == "mxfp4" else
            store(normal(seed, "KI", (B, N, dI), device=device), ki_fmt)),
        hkv=store(normal(seed, "hkv", (B, Nh, D), device=device), "mixed", r),
        raw_csa=store(normal(seed, "raw_csa", (B, W, D), device=device), "mixed", r),
        raw_hca=store(normal(seed, "raw_hca", (B, W, D), device=device), "mixed", r),
        csa_overlap=csa_overlap,
        new_kv_csa=store(normal(seed, "new_kv_csa", (B, m + csa_overlap, D), device=device), "bf16"),
        new_z_csa=store(normal(seed, "new_z_csa", (B, m + csa_overlap, D), device=device), "bf16"),
        new_kI=store(normal(seed, "new_kI", (B, m, dI), device=device), "bf16"),
        new_zI=store(normal(seed, "new_zI", (B, m, dI), device=device), "bf16"),
        new_kv_hca=store(normal(seed, "new_kv_hca", (B, m_hca, D), device=device), "bf16"),
        new_z_hca=store(normal(seed, "new_z_hca", (B, m_hca, D), device=device), "bf16"),
        qI=store(normal(seed, "qI", (B, 1, HI, dI), device=device), qi_fmt),
        w=uniform(seed, "w", (B, 1, HI), device=device),
        q_csa=store(normal(seed, "q_csa", (B, 1, H, D), device=device), "bf16"),
        q_hca=store(normal(seed, "q_hca", (B, 1, H, D), device=device), "bf16"),
    )


def projection(seed=5, T=4096, H=64, D=512, G=8, d_g=1024, d=7168, device="cpu"):
    """Inputs of the grouped output projection: attention outputs [T, H, D]
    ~ N(0, 1) and weights scaled by 1/sqrt(fan-in) (W1 [G, d_g, (H/G)*D],
    W2 [d, G*d_g]) so that the intermediate and the output stay near unit
    scale; all bf16."""
    K1 = (H // G) * D
    return dict(
        kind="projection", T=T, H=H, D=D, G=G, d_g=d_g, d=d,
        attn=store(normal(seed, "attn", (T, H, D), device=device), "bf16"),
        w1=store(normal(seed, "w1", (G, d_g, K1), std=K1 ** -0.5, device=device), "bf16"),
        w2=store(normal(seed, "w2", (d, G * d_g), std=(G * d_g) ** -0.5, device=device), "bf16"),
    )


def bulk_compress(seed=4, B=4, T=1 << 20, D=512, dI=128, hca=True, device="cpu"):
    """Raw activations of whole contexts for building the compressed caches in
    bulk: the CSA layer's KV and logits [B, T, D] and raw indexer keys and
    logits [B, T, dI], and with hca the HCA layer's KV and logits [B, T, D];
    all N(0, 1) in bf16.  Drawn one sequence at a time (names carry the
    sequence) to bound the float32 temporaries."""
    names = [("kv", D), ("z", D), ("kI_raw", dI), ("zI", dI)]
    if hca:
        names += [("kv_hca", D), ("z_hca", D)]
    out = dict(kind="bulk_compress", B=B, T=T, D=D, dI=dI, pos0=0)
    for name, width in names:
        t = torch.empty((B, T, width), dtype=torch.bfloat16, device=device)
        for b in range(B):
            t[b] = normal(seed, f"{name}/{b}", (T, width), device=device).to(torch.bfloat16)
        out[name] = t
    return out
