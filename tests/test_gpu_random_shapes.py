"""Seeded random shapes through the whole chain on the GPU (GPU).

Each case draws batch, query rows, context lengths (ragged, some shorter than
k), indexer heads and width, number format, k and attention heads from a
fixed-seed generator, then checks every stage against the oracle on the same
inputs: indexer scores within the format's tolerance, the GPU top-k bit-exact
on the GPU's own fp32 scores and within the k-th boundary rule against the
oracle's fp64 scores, and sparse attention over the GPU's index set within the
attention tolerance.  The shapes cover both indexer kernels (decode rows and
prefill chunks), both top-k launch shapes (one workgroup per row, chunked long
rows) and split and unsplit attention.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import dsa_sparse_attention_lightning_amd as dsa
from dsa_sparse_attention_lightning_amd import inputs as gen
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def draw(seed):
    r = np.random.default_rng(seed)
    T = int(r.choice([1, 1, 1, 2, 7, 33]))
    B = int(r.integers(1, 4))
    long_rows = T == 1 and r.random() < 0.4
    Lmax = int(r.integers(16384, 40000)) if long_rows else int(r.integers(T + 1, 6000))
    k = int(r.choice([16, 100, 512, 2048]))
    ctx = []
    for _ in range(B):
        lo = T if r.random() < 0.3 else max(T, Lmax // 2)
        ctx.append(int(r.integers(lo, Lmax + 1)))
    ctx[0] = Lmax                                  # at least one full row
    H = int(r.choice([1, 8, 32, 40, 64]))
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["bf16", "fp8"]))
    Hq = int(r.choice([16, 48, 128]))
    return dict(B=B, T=T, Lmax=Lmax, ctx=ctx, k=k, H=H, D=D, dtype=dtype, Hq=Hq)


CASES = [draw(1000 + i) for i in range(14)]


@pytest.mark.parametrize("c", CASES, ids=lambda c: "B{B}T{T}L{Lmax}k{k}H{H}D{D}{dtype}Hq{Hq}".format(**c))
def test_random_chain(c):
    say("random chain case", c)
    B, T, Lmax, ctx, k = c["B"], c["T"], c["Lmax"], c["ctx"], c["k"]
    s = gen.Shape(5000 + c["H"] + c["D"] + k, "case", 1, "F", B=B, T=T, ctx=Lmax, H=c["H"],
                  D=c["D"], idx_dtype=c["dtype"], k=k, Hq=c["Hq"])
    qi = gen.make_indexer_query(s, DEV, w_low=-0.3)
    ki = gen.make_indexer_keys(s, 1, gen.make_key_base(s, DEV), DEV)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    sc = dsa.indexer_scores(qi.q, qi.w, ki.k, ctx_t, qi.q_scale, ki.k_scale)
    idx = dsa.topk(sc, ctx_t, k)
    q, kv = gen.make_mla_layer(s, 1, DEV)
    out, lse = dsa.sparse_attn(q, kv, idx, ctx_t, s.scale)
    torch.cuda.synchronize()
    ref_sc = oracle.indexer_scores(parity.host_real(qi.q, qi.q_scale),
                                   qi.w.cpu().double().numpy(),
                                   parity.host_real(ki.k, ki.k_scale), ctx)
    gpu_sc = sc.cpu().numpy()
    parity.check_scores(gpu_sc.astype(np.float64), ref_sc, c["dtype"])
    gpu_idx = idx.cpu().numpy()
    parity.check_topk_exact(gpu_idx, gpu_sc, ctx, k)
    st = parity.check_topk_boundary(gpu_idx, ref_sc, ctx, k)
    ro, rl = oracle.sparse_attn(parity.host_real(q), parity.host_real(kv), gpu_idx, ctx,
                                s.scale, 512)
    err = parity.check_attn(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl)
    say("  boundary swaps", st["swaps"], "attention max abs err", err)
