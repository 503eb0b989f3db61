"""Seeded synthetic inputs shaped like the IndexCache workloads.

This module only draws random tensors and stores them in the formats the
kernels read (bf16, or OCP fp8 e4m3 codes with one fp32 scale per 128-element
row block).  It holds none of the method's arithmetic, so both the HIP path and
the CPU oracle can take their inputs from it.

Recipe (one seed per tensor: 1_000_003*cfg + 1_009*layer + tensor_id, with
tensor ids q_idx 1, w 2, k_base 3, k_noise 4, q 5, kv 6):
  * indexer query q_idx ~ N(0,1) and head weights w ~ U(0,1) fp32 are drawn
    once per stack (layer 0 seeds) and shared by every layer;
  * indexer keys of layer l: k_l = 0.95*k_base + 0.31*N(0,1)_l, so keys of two
    layers correlate at 0.9025 and have variance ~1;
  * MLA query q ~ N(0,1) [B,T,Hq,576] and latent KV ~ N(0,1) [B,Lmax,576]
    are independent per layer;
  * bf16 tensors are the round-to-nearest-even bf16 of the fp32 draws; fp8
    tensors are quantised per row: scale = amax/448 (1.0 for an all-zero
    row), code = e4m3(x/scale) with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

TENSOR_IDS = dict(q_idx=1, w=2, k_base=3, k_noise=4, q=5, kv=6)
FP8_MAX = 448.0

# C3's pattern: F at layers 0,3,7,11,15,19,23,27,31,35,40,44 of 48.
_C3_F = (0, 3, 7, 11, 15, 19, 23, 27, 31, 35, 40, 44)
C3_PATTERN = "".join("F" if i in _C3_F else "S" for i in range(48))


@dataclasses.dataclass
class Shape:
    """One workload: a decode (T == 1) or prefill (T > 1) layer stack."""
    cfg_id: int
    name: str
    n_layers: int
    pattern: str
    B: int
    T: int
    ctx: int                 # context length of every sequence (ctx_len[b] = ctx)
    H: int                   # indexer heads
    D: int                   # indexer head dim
    idx_dtype: str           # "bf16" | "fp8"
    k: int                   # top-k
    Hq: int = 0              # MLA query heads (0: no attention in this workload)
    d_qk: int = 576
    d_v: int = 512
    scale: float = 1.0 / math.sqrt(192.0)
    Lmax: int = 0            # key-cache capacity (defaults to ctx)
    patterns: tuple = ()     # extra patterns this workload is run with

    def __post_init__(self):
        if self.Lmax == 0:
            self.Lmax = self.ctx


def tile_pattern(p: str, n: int) -> str:
    return (p * ((n + len(p) - 1) // len(p)))[:n]


CONFIGS = {
    0: Shape(0, "tiny decode stack", 4, "FSSS", B=1, T=1, ctx=4096, H=4, D=64,
             idx_dtype="bf16", k=256, Hq=16),
    1: Shape(1, "batched decode", 8, "FSSSFSSS", B=32, T=1, ctx=32768, H=64, D=128,
             idx_dtype="bf16", k=2048, Hq=128),
    2: Shape(2, "prefill chunk, indexer+top-k", 1, "F", B=1, T=8192, ctx=65536, H=64,
             D=128, idx_dtype="fp8", k=2048, Hq=0),
    3: Shape(3, "long-context decode", 48, C3_PATTERN, B=8, T=1, ctx=131072, H=64,
             D=128, idx_dtype="fp8", k=2048, Hq=128,
             patterns=("F" * 48, tile_pattern("FSSS", 48), C3_PATTERN)),
    4: Shape(4, "pattern sweep", 16, "F" * 16, B=4, T=1, ctx=196608, H=64, D=128,
             idx_dtype="fp8", k=2048, Hq=128,
             patterns=("F" * 16, tile_pattern("FS", 16), tile_pattern("FSSS", 16),
                       tile_pattern("FSSSSSSS", 16))),
}


def seed_of(cfg_id: int, layer: int, tensor: str) -> int:
    return 1_000_003 * cfg_id + 1_009 * layer + TENSOR_IDS[tensor]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn(shape, seed: int, device) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)


def rand(shape, seed: int, device) -> torch.Tensor:
    return torch.rand(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)


def quantize_fp8_rows(x: torch.Tensor):
    """fp32 [..., D] -> (e4m3 codes [..., D] as torch.float8_e4m3fn, fp32 scales [...])."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    codes = (x / scale[..., None]).to(torch.float8_e4m3fn)
    return codes, scale.contiguous()


def store(x: torch.Tensor, dtype: str):
    """Store an fp32 draw in the kernel's input format: (tensor, scale or None)."""
    if dtype == "bf16":
        return x.to(torch.bfloat16).contiguous(), None
    if dtype == "fp8":
        return quantize_fp8_rows(x)
    raise ValueError(dtype)


@dataclasses.dataclass
class IndexerQuery:
    q: torch.Tensor                 # [B,T,H,D] bf16 or float8_e4m3fn
    q_scale: Optional[torch.Tensor]  # [B,T,H] fp32 (fp8 only)
    w: torch.Tensor                 # [B,T,H] fp32


@dataclasses.dataclass
class IndexerKeys:
    k: torch.Tensor                 # [B,Lmax,D]
    k_scale: Optional[torch.Tensor]  # [B,Lmax] fp32 (fp8 only)


def make_indexer_query(s: Shape, device="cpu", w_low: float = 0.0) -> IndexerQuery:
    """q_idx ~ N(0,1), w ~ U(w_low, 1) (w_low < 0 gives weights of both signs)."""
    qf = randn((s.B, s.T, s.H, s.D), seed_of(s.cfg_id, 0, "q_idx"), device)
    q, qs = store(qf, s.idx_dtype)
    w = rand((s.B, s.T, s.H), seed_of(s.cfg_id, 0, "w"), device)
    if w_low != 0.0:
        w = w_low + (1.0 - w_low) * w
    return IndexerQuery(q, qs, w.contiguous())


def make_key_base(s: Shape, device="cpu") -> torch.Tensor:
    return randn((s.B, s.Lmax, s.D), seed_of(s.cfg_id, 0, "k_base"), device)


def make_indexer_keys(s: Shape, layer: int, k_base: torch.Tensor, device="cpu",
                      a: float = 0.95, b: float = 0.31) -> IndexerKeys:
    noise = randn((s.B, s.Lmax, s.D), seed_of(s.cfg_id, layer, "k_noise"), device)
    kf = a * k_base + b * noise if b != 0.0 else a * k_base
    del noise
    k, ks = store(kf, s.idx_dtype)
    return IndexerKeys(k, ks)


def calibration_segments(n_layers: int, early: int, transition: int) -> List[int]:
    """Key-cache segment of each layer for a stack with planted structure:
    layers 0..early-1 each have a segment of their own, layers early..
    transition-1 share one, layers transition.. share another."""
    return [l if l < early else (early if l < transition else early + 1)
            for l in range(n_layers)]


def make_segment_base(s: Shape, segment: int, device="cpu") -> torch.Tensor:
    """Key base of one segment (segment 0 is the stack's usual key base)."""
    return randn((s.B, s.Lmax, s.D), seed_of(s.cfg_id, segment, "k_base"), device)


def make_mla_layer(s: Shape, layer: int, device="cpu"):
    """(q [B,T,Hq,d_qk] bf16, kv [B,Lmax,d_qk] bf16) for one layer."""
    q = randn((s.B, s.T, s.Hq, s.d_qk), seed_of(s.cfg_id, layer, "q"), device).to(torch.bfloat16)
    kv = torch.empty((s.B, s.Lmax, s.d_qk), dtype=torch.bfloat16, device=device)
    g = _gen(seed_of(s.cfg_id, layer, "kv"), device)
    # draw sequence by sequence to bound the fp32 temporary
    for bb in range(s.B):
        kv[bb].copy_(torch.randn((s.Lmax, s.d_qk), generator=g, device=device,
                                 dtype=torch.float32))
    return q.contiguous(), kv


def ctx_lens(s: Shape, device="cpu", values: Optional[List[int]] = None) -> torch.Tensor:
    v = values if values is not None else [s.ctx] * s.B
    return torch.tensor(v, dtype=torch.int32, device=device)


def bits(t: torch.Tensor):
    """Raw bit patterns of a bf16 / fp8 tensor as a CPU numpy array."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)
