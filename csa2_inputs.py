"""Seeded synthetic inputs for the CSA2 step (shared by tests, bench and smoke).

This module only draws random numbers and lays them out: it holds none of the
step's arithmetic, so both the GPU library's callers and the CPU oracle's
tests can take their inputs from it.  Every tensor comes from its own torch
generator seeded from (seed, tensor name, layer, sequence), so a single
sequence can be drawn again on its own.  Values drawn on a CUDA device differ
from values drawn on the CPU; a test draws once and copies to the host what
the oracle needs.

Workload shapes (five configurations, contexts inside the 4K..1M range the
pages discuss; no public benchmark defines shapes for this step):
  0  decode, 1 sequence, 4,096 entries, one Full layer
  1  decode, 8 sequences, 65,536 entries, one Full layer, latent and window
     rows scaled per channel by lognormal(0, 0.5)
  2  decode, 16 sequences, 131,072 entries, a 4-layer group run as
     Full + 3 Reuse and then Reindex + 3 Reuse on the same state
  3  decode, 4 sequences, 1,048,576 entries, hierarchical Full layer
  4  prefill, one sequence: a 262,144-token prefix (131,072 entries at
     ratio 2) plus a chunk of 4,096 query tokens (2,048 entries), 1 Full +
     5 Reuse layers
Values: latent and indexer key N(0,1) float32; indexer Q N(0,1) rounded to
E4M3 by torch; head weights 1; attention Q N(0,1)/sqrt(512) rounded to
bfloat16 by torch; window rows N(0,1) rounded to bfloat16.
"""

import math
import zlib

import torch

D_LATENT, D_INDEX, H_INDEX, H_ATTN = 512, 64, 4, 16
TOP_K, SWA_WINDOW, BLOCK, N_BLOCKS = 512, 128, 8, 2048

CONFIGS = {
    0: dict(kind="decode", batch=1, ctx=4096, lognormal=False, plans=[["F"]], index="flat"),
    1: dict(kind="decode", batch=8, ctx=65536, lognormal=True, plans=[["F"]], index="flat"),
    2: dict(kind="decode", batch=16, ctx=131072, lognormal=False,
            plans=[["F", "U", "U", "U"], ["R", "U", "U", "U"]], index="flat"),
    3: dict(kind="decode", batch=4, ctx=1048576, lognormal=False, plans=[["F"]], index="hier"),
    4: dict(kind="prefill", batch=1, prefix_tokens=262144, chunk=4096, ratio=2,
            plans=[["F", "U", "U", "U", "U", "U"]], index="flat"),
}


def seed_of(seed, name, layer=0, seq=0):
    """Deterministic 63-bit seed of one tensor."""
    return zlib.crc32(f"{seed}/{name}/{layer}/{seq}".encode()) * 1_000_003 + seed


def _gen(device, s):
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def normal(shape, seed, name, layer=0, seq=0, device="cpu"):
    """float32 N(0,1) tensor."""
    g = _gen(device, seed_of(seed, name, layer, seq))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def channel_sigma(seed, device="cpu"):
    """Per-channel factors exp(0.5 z), one per latent channel, shared by all
    positions and sequences."""
    return torch.exp(0.5 * normal((D_LATENT,), seed, "sigma", device=device))


def latent(n, seed, seq=0, lognormal=False, device="cpu", name="latent"):
    x = normal((n, D_LATENT), seed, name, seq=seq, device=device)
    if lognormal:
        x *= channel_sigma(seed, device)
    return x


def index_key(n, seed, seq=0, device="cpu", name="idxk"):
    return normal((n, D_INDEX), seed, name, seq=seq, device=device)


def index_query(shape_prefix, seed, layer=0, device="cpu", name="idxq"):
    """E4M3 codes (uint8) of N(0,1) draws, [*shape_prefix, 4, 64]."""
    x = normal(tuple(shape_prefix) + (H_INDEX, D_INDEX), seed, name, layer, device=device)
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def index_weight(shape_prefix, device="cpu"):
    return torch.ones(tuple(shape_prefix) + (H_INDEX,), dtype=torch.float32, device=device)


def attn_query(shape_prefix, seed, layer=0, device="cpu", name="q"):
    """bfloat16 [*shape_prefix, 16, 512] of N(0,1)/sqrt(512)."""
    x = normal(tuple(shape_prefix) + (H_ATTN, D_LATENT), seed, name, layer, device=device)
    return (x / math.sqrt(D_LATENT)).to(torch.bfloat16)


def window_rows(batch, rows, seed, layer=0, lognormal=False, device="cpu", name="swa"):
    """bfloat16 [batch, rows, 512] sliding-window rows."""
    x = normal((batch, rows, D_LATENT), seed, name, layer, device=device)
    if lognormal:
        x *= channel_sigma(seed, device)
    return x.to(torch.bfloat16)


def bf16_bits(t):
    """uint16 numpy view of a bfloat16 tensor (host copy)."""
    return t.detach().cpu().view(torch.int16).numpy().view("uint16")
