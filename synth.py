"""Seeded synthetic inputs shaped like the workloads of the source pages.

This module only draws random numbers and lays them out; it holds none of the
quantization arithmetic.  Both sides of every parity check (the GPU library and
the CPU oracle) consume the exact same bytes produced here.

Each generator is deterministic in (recipe, shape, seed, device): the same
call on the same device type returns the same tensor.  torch's CPU and GPU
generators are different streams, so a recipe drawn on the GPU differs from
the same recipe drawn on the CPU; parity always compares outputs computed from
one drawn tensor.

Recipes (stand-ins for MoE expert weights and KV caches; no dataset or trained
checkpoint is involved):
  mxfp4_fp32   float32 N(0,1); row 0 all +0.0; last row multiplied by 1e-30.
  moe_mxfp4    bfloat16 z * 0.02 * r * gamma: r = 50 on 1% of rows (drawn
               without replacement), else 1; gamma = 2^u per 32-column block,
               u ~ U[-8, 8).
  moe_nvfp4    bfloat16; in each expert the first half of the rows ~ N(0,0.02),
               the second half ~ N(0,0.2) (fused gate/up halves).
  kv_cache     bfloat16 N(0,1) * 2^u with one u ~ U[-4, 4) per token (row).
  moe_sweep    bfloat16 N(0,0.02) with three disjoint sets of 32-column blocks,
               each 0.1% of all blocks: all +0.0; N(0,1) * 2^-130 (bfloat16
               subnormal magnitudes); one element set to +-1e4.
Products are formed in float32 in the order written, then rounded once to
bfloat16.  Zeros are written by fill, never by multiplying (so they are +0.0).
"""
from __future__ import annotations

import torch

# Workload shapes (leading dims..., last dim).
SHAPES = {
    "c1": (256, 1024),            # MXFP4 round trip, float32
    "c2": (32, 4096, 2048),       # MXFP4 MoE expert weights
    "c3": (64, 3072, 4096),       # NVFP4 fused gate/up expert weights
    "c4a": (16, 8192, 512),       # cache QDQ fp8, block 32 (SWA KV)
    "c4b": (16, 8192, 128),       # cache QDQ mxfp4, block 32 (index Q/K)
    "c4c": (16, 2048, 512),       # cache QDQ nvfp4, block 16 (compressed KV)
    "c5": (256, 2048, 7168),      # large sweep, processed in expert chunks
}
C5_CHUNK_EXPERTS = 36             # 36 * 2048 * 7168 * 2 B ~= 0.98 GiB per chunk

SEEDS = {"c1": 1, "c2": 2, "c3": 3, "c4a": 41, "c4b": 42, "c4c": 43, "c5": 5}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def mxfp4_fp32(shape=SHAPES["c1"], seed=SEEDS["c1"], device="cpu") -> torch.Tensor:
    g = _gen(device, seed)
    x = _normal(shape, g, device)
    x = x.reshape(-1, shape[-1])
    x[0].fill_(0.0)
    x[-1] = x[-1] * 1e-30
    return x.reshape(shape)


def moe_mxfp4(shape=SHAPES["c2"], seed=SEEDS["c2"], device="cpu") -> torch.Tensor:
    assert shape[-1] % 32 == 0
    g = _gen(device, seed)
    z = _normal(shape, g, device)
    K = shape[-1]
    rows = z.numel() // K
    r = torch.ones(rows, device=device, dtype=torch.float32)
    n_out = max(1, round(0.01 * rows))
    idx = torch.randperm(rows, generator=g, device=device)[:n_out]
    r[idx] = 50.0
    u = torch.rand(rows, K // 32, generator=g, device=device) * 16.0 - 8.0
    gamma = torch.exp2(u)
    x = z.reshape(rows, K // 32, 32) * 0.02
    x = x * r.reshape(rows, 1, 1)
    x = x * gamma.reshape(rows, K // 32, 1)
    return x.reshape(shape).to(torch.bfloat16)


def moe_nvfp4(shape=SHAPES["c3"], seed=SEEDS["c3"], device="cpu") -> torch.Tensor:
    g = _gen(device, seed)
    z = _normal(shape, g, device)
    N = shape[-2]
    sigma = torch.full((N, 1), 0.02, device=device)
    sigma[N // 2:] = 0.2
    return (z * sigma).to(torch.bfloat16)


def kv_cache(shape=SHAPES["c4a"], seed=SEEDS["c4a"], device="cpu") -> torch.Tensor:
    g = _gen(device, seed)
    z = _normal(shape, g, device)
    u = torch.rand(shape[:-1], generator=g, device=device) * 8.0 - 4.0
    return (z * torch.exp2(u).unsqueeze(-1)).to(torch.bfloat16)


def moe_sweep(shape, seed, device="cpu", special_frac=1e-3) -> torch.Tensor:
    """One chunk of the large sweep: [experts, N, K] bfloat16."""
    K = shape[-1]
    assert K % 32 == 0
    g = _gen(device, seed)
    x = (_normal(shape, g, device) * 0.02).to(torch.bfloat16)
    nblk = x.numel() // 32
    m = int(round(special_frac * nblk))
    if m == 0:
        return x
    pick = torch.randperm(nblk, generator=g, device=device)[: 3 * m]
    zero_b, sub_b, spike_b = pick[:m], pick[m:2 * m], pick[2 * m:]
    xb = x.view(nblk, 32)
    xb[zero_b] = 0.0
    tiny = (_normal((m, 32), g, device) * (2.0 ** -130)).to(torch.bfloat16)
    xb[sub_b] = tiny
    pos = torch.randint(0, 32, (m,), generator=g, device=device)
    sgn = torch.randint(0, 2, (m,), generator=g, device=device).float() * 2 - 1
    xb[spike_b, pos] = (sgn * 1e4).to(torch.bfloat16)
    return x


def c5_chunks(n_experts=SHAPES["c5"][0], per_chunk=C5_CHUNK_EXPERTS):
    """(chunk_id, first_expert, n_experts_in_chunk) for the large sweep."""
    out, e0, cid = [], 0, 0
    while e0 < n_experts:
        n = min(per_chunk, n_experts - e0)
        out.append((cid, e0, n))
        e0 += n
        cid += 1
    return out


def c5_chunk(cid: int, n_experts: int, device="cpu", N=None, K=None) -> torch.Tensor:
    N = N or SHAPES["c5"][1]
    K = K or SHAPES["c5"][2]
    return moe_sweep((n_experts, N, K), seed=SEEDS["c5"] * 1000 + cid,
                     device=device)
