"""Fused indexer + top-k for decode rows (GPU).

dsa_indexer_topk keeps the scores on chip and compacts candidates per
workgroup against a lower bound of the threshold bin (the row histogram as it
stands when the workgroup ends plus its own counts); the finishing kernel
takes the true threshold from the finished histogram.  Its selection must be
exactly the oracle's top-k over the same fp32 scores (the scores the separate
indexer kernel writes: the fused kernel computes them with the same
arithmetic), and so equal to the separate indexer + top-k path, on ragged
rows, rows with n <= k and n = k + 1, heavy ties (the candidate list then
overflows LDS and is finished from the slices in memory), both key dtypes and
head dims, rows with one tile per wave (no early hand-off: the first
workgroups count fewer than k keys and take all of theirs), and the largest
plan (1024 workgroups per row).
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


def make_case(B, H, D, Lmax, dtype, seed, keys="random", T=1):
    s = gen.Shape(seed, "fused", 1, "F", B=B, T=T, ctx=Lmax, H=H, D=D, idx_dtype=dtype, k=1)
    qi = gen.make_indexer_query(s, DEV, w_low=-0.3)
    ki = gen.make_indexer_keys(s, 1, gen.make_key_base(s, DEV), DEV)
    k, ks = ki.k, ki.k_scale
    if keys == "equal":      # every key the same row: every visible score equal
        k = k[:, :1].expand(-1, Lmax, -1).contiguous()
        ks = None if ks is None else ks[:, :1].expand(-1, Lmax).contiguous()
    elif keys == "few":      # five distinct key rows: five distinct scores per row
        sel = torch.arange(Lmax, device=DEV) % 5
        k = k[:, sel].contiguous()
        ks = None if ks is None else ks[:, sel].contiguous()
    return qi, k, ks


CASES = [
    # B, H, D, Lmax, ctx, k, dtype, keys
    (4, 64, 128, 20000, [20000, 13777, 2049, 1500], 2048, "fp8", "random"),  # n=k+1, n<k
    (3, 16, 64, 9000, [9000, 4097, 1], 512, "bf16", "random"),
    (2, 33, 64, 70000, [70000, 41234], 2048, "fp8", "random"),    # D = 64 fp8 tiles, H % 32
    (2, 64, 128, 40000, [40000, 39999], 1024, "bf16", "random"),  # 32-key bf16 tiles
    (8, 64, 128, 131072, [131072] * 8, 2048, "fp8", "random"),    # long-context decode
    (2, 64, 128, 65536, [65536, 30000], 2048, "fp8", "equal"),    # list overflows LDS
    (2, 64, 128, 65536, [65536, 20000], 2048, "bf16", "few"),     # heavy ties
    (1, 8, 128, 524288, [524288], 2048, "fp8", "random"),         # 256 workgroups per row
    (1, 4, 128, 8388608, [8388608], 2048, "fp8", "random"),       # 1024: the largest plan
    (1, 64, 128, 100, [100], 64, "fp8", "random"),                # one key tile
    (1, 64, 128, 65536, [65536], 16384, "fp8", "random"),         # k above the LDS list
    (2, 64, 64, 10000, [10000, 9000], 8192, "bf16", "random"),    # k close to n
]


@pytest.mark.parametrize("case", CASES,
                         ids=lambda c: f"B{c[0]}H{c[1]}D{c[2]}L{c[3]}k{c[5]}{c[6]}-{c[7]}")
def test_fused_equals_oracle_selection(case):
    B, H, D, Lmax, ctx, k, dtype, keys = case
    say("fused indexer + top-k case", case)
    qi, kc, ks = make_case(B, H, D, Lmax, dtype, seed=40 + H + D, keys=keys)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    got = dsa.indexer_topk(qi.q, qi.w, kc, ctx_t, k, qi.q_scale, ks)
    sc = dsa.indexer_scores(qi.q, qi.w, kc, ctx_t, qi.q_scale, ks)
    sep = dsa.topk(sc, ctx_t, k)
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    parity.check_topk_exact(g, sc.cpu().numpy(), ctx, k)
    assert np.array_equal(g, sep.cpu().numpy())


def test_fused_boundary_against_oracle_scores():
    """End to end: the fused set obeys the k-th boundary rule against the
    oracle's fp64 scores of the same inputs."""
    B, H, D, L, k = 2, 64, 128, 8192, 2048
    ctx = [8192, 6000]
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    for dtype in ("bf16", "fp8"):
        qi, kc, ks = make_case(B, H, D, L, dtype, seed=8)
        idx = dsa.indexer_topk(qi.q, qi.w, kc, ctx_t, k, qi.q_scale, ks)
        torch.cuda.synchronize()
        ref = oracle.indexer_scores(parity.host_real(qi.q, qi.q_scale),
                                    qi.w.cpu().double().numpy(), parity.host_real(kc, ks), ctx)
        st = parity.check_topk_boundary(idx.cpu().numpy(), ref, ctx, k)
        say(dtype, "boundary swaps", st)


def _zero_region(ws, rows):
    """The row histograms: what must be zero between calls."""
    return int(ws[: rows * 4096 * 4].count_nonzero().item()) == 0


def test_fused_workspace_reuse():
    """One workspace across many calls (different queries, ragged rows
    including n <= k), the separate top-k using the same workspace in
    between: every result equals the separate path's, and the part of the
    workspace that must start at zero is zero after every call.  (A read of
    the row histogram that saw a previous call's counts would raise the
    bound above the true one and drop selected keys.)"""
    B, H, D, L, k = 3, 64, 128, 65536, 2048
    ctx = [65536, 40000, 2000]
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    nbytes = max(dsa.indexer_topk_workspace_size(B, 1, H, D, L, k, "fp8"),
                 dsa.topk_workspace_size(B, 1, L, k))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    for seed in range(1, 9):
        qi, kc, ks = make_case(B, H, D, L, "fp8", seed=seed)
        got = dsa.indexer_topk(qi.q, qi.w, kc, ctx_t, k, qi.q_scale, ks, workspace=ws)
        sc = dsa.indexer_scores(qi.q, qi.w, kc, ctx_t, qi.q_scale, ks)
        sep = dsa.topk(sc, ctx_t, k, workspace=ws)
        again = dsa.indexer_topk(qi.q, qi.w, kc, ctx_t, k, qi.q_scale, ks, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, sep), f"seed {seed}"
        assert torch.equal(again, sep), f"seed {seed}, after the separate top-k"
        assert _zero_region(ws, B), f"seed {seed}: workspace not left zero"


PREFILL_CASES = [
    # B, T, H, D, Lmax, ctx, k, dtype, keys
    (2, 5, 64, 128, 1030, [1030, 517], 256, "fp8", "random"),
    (1, 64, 64, 128, 2080, [2080], 512, "bf16", "random"),
    (1, 300, 64, 128, 5000, [5000], 1024, "fp8", "random"),     # T not a multiple of 8
    (2, 17, 64, 64, 900, [900, 500], 128, "bf16", "random"),     # D = 64, ragged ctx
    (1, 40, 20, 128, 4000, [3000], 256, "bf16", "random"),       # ctx < Lmax, H < 32
    (1, 16, 64, 128, 40000, [40000], 2048, "fp8", "equal"),      # every key listed: past LDS
    (1, 24, 64, 128, 30000, [30000], 2048, "bf16", "few"),       # heavy ties
]


@pytest.mark.parametrize("case", PREFILL_CASES,
                         ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}D{c[3]}L{c[4]}k{c[6]}{c[7]}-{c[8]}")
def test_fused_prefill_equals_oracle_selection(case):
    """Prefill form (several query rows per sequence, running bound per row,
    candidate lists): exactly the oracle's top-k over the GPU's fp32 scores,
    and the separate kernels' selection."""
    B, T, H, D, Lmax, ctx, k, dtype, keys = case
    say("fused prefill indexer + top-k case", case)
    qi, kc, ks = make_case(B, H, D, Lmax, dtype, seed=60 + T + D, keys=keys, T=T)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    got = dsa.indexer_topk(qi.q, qi.w, kc, ctx_t, k, qi.q_scale, ks)
    sc = dsa.indexer_scores(qi.q, qi.w, kc, ctx_t, qi.q_scale, ks)
    sep = dsa.topk(sc, ctx_t, k)
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    parity.check_topk_exact(g, sc.cpu().numpy(), ctx, k)
    assert np.array_equal(g, sep.cpu().numpy())


def test_fused_prefill_chunk_equals_separate():
    """The 8192-query prefill chunk on a 65536-token context: the fused form's
    sets equal the separate kernels' for every row (the separate path is held
    to the oracle at this size by the full-size parity tests)."""
    B, T, H, D, L, k = 1, 8192, 64, 128, 65536, 2048
    qi, kc, ks = make_case(B, H, D, L, "fp8", seed=70, T=T)
    ctx_t = torch.tensor([L], dtype=torch.int32, device=DEV)
    got = dsa.indexer_topk(qi.q, qi.w, kc, ctx_t, k, qi.q_scale, ks)
    sc = dsa.indexer_scores(qi.q, qi.w, kc, ctx_t, qi.q_scale, ks)
    sep = dsa.topk(sc, ctx_t, k)
    torch.cuda.synchronize()
    assert torch.equal(got, sep)


@pytest.mark.parametrize("idx_dtype,D", [("fp8", 128), ("bf16", 64)])
def test_stack_fused_equals_unfused(idx_dtype, D):
    """The layer stack with the fused F layers and with scores through the
    score buffer: the same index sets and bit-identical attention outputs."""
    B, Lmax, H, k, Hq = 2, 20000, 64, 2048, 32
    pattern = "FSSF"
    ctx_t = torch.tensor([20000, 9000], dtype=torch.int32, device=DEV)
    s = gen.Shape(9100 + D, "fused stack", len(pattern), pattern, B=B, T=1, ctx=Lmax, H=H, D=D,
                  idx_dtype=idx_dtype, k=k, Hq=Hq)
    kb = gen.make_key_base(s, DEV)
    qi = gen.make_indexer_query(s, DEV, w_low=-0.2)
    layers = []
    for l in range(s.n_layers):
        ki = gen.make_indexer_keys(s, l, kb, DEV)
        q, kv = gen.make_mla_layer(s, l, DEV)
        layers.append(dict(q_idx=qi.q, q_idx_scale=qi.q_scale, w=qi.w, k_idx=ki.k,
                           k_idx_scale=ki.k_scale, q=q, kv=kv,
                           out=torch.empty((B, 1, Hq, s.d_v), dtype=torch.bfloat16, device=DEV),
                           lse=torch.empty((B, 1, Hq), dtype=torch.float32, device=DEV)))
    res = {}
    for unfused in (False, True):
        st = dsa.Stack(pattern, layers, ctx_t, B=B, T=1, H=H, D=D, Lmax=Lmax, k=k, Hq=Hq,
                       idx_dtype=idx_dtype, scale=s.scale, fused_topk=not unfused)
        assert st.fused == (not unfused)
        stats = st.run()
        torch.cuda.synchronize()
        assert stats["n_indexer_calls"] == 2 and stats["n_topk_calls"] == 2
        res[unfused] = (st.idx_buf.clone(), [L["out"].clone() for L in layers],
                        [L["lse"].clone() for L in layers])
    assert torch.equal(res[False][0], res[True][0])
    for l in range(len(pattern)):
        assert torch.equal(res[False][1][l], res[True][1][l]), f"layer {l} output"
        assert torch.equal(res[False][2][l], res[True][2][l]), f"layer {l} lse"
