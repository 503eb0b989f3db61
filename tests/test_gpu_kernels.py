"""Per-kernel parity of the HIP path against the fp64 oracle (GPU)."""
import math
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


def make_indexer(B, T, H, D, Lmax, dtype, seed, w_low=0.0):
    s = gen.Shape(seed, "case", 1, "F", B=B, T=T, ctx=Lmax, H=H, D=D, idx_dtype=dtype, k=1)
    qi = gen.make_indexer_query(s, DEV, w_low=w_low)
    kb = gen.make_key_base(s, DEV)
    ki = gen.make_indexer_keys(s, 1, kb, DEV)
    return qi, ki


INDEXER_CASES = [
    # B, T, H, D, Lmax, ctx, dtype
    (1, 1, 4, 64, 4096, [4096], "bf16"),                     # tiny decode shape
    (3, 1, 64, 128, 4100, [4100, 1000, 33], "bf16"),         # ragged ctx, ragged tail tile
    (2, 1, 64, 128, 3001, [3001, 1500], "fp8"),
    (2, 1, 40, 64, 777, [777, 700], "fp8"),                  # H not a multiple of 32
    (1, 1, 1, 128, 100, [100], "bf16"),                      # single head
    (2, 5, 64, 128, 1030, [1030, 517], "fp8"),               # prefill rows (T > 1)
    (1, 64, 64, 128, 2080, [2080], "bf16"),
    (1, 300, 64, 128, 5000, [5000], "fp8"),                  # prefill MFMA path, ragged T
    (2, 17, 64, 64, 900, [900, 500], "bf16"),                # prefill, D = 64, ragged ctx
    (1, 40, 20, 128, 4000, [3000], "bf16"),                  # prefill, ctx < Lmax, H < 32
]


@pytest.mark.parametrize("case", INDEXER_CASES, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}D{c[3]}L{c[4]}{c[6]}")
def test_indexer_scores(case):
    B, T, H, D, Lmax, ctx, dtype = case
    say("indexer case", case)
    qi, ki = make_indexer(B, T, H, D, Lmax, dtype, seed=11 + H + D, w_low=-0.5)
    ctx_t = gen.ctx_lens(gen.Shape(0, "", 1, "F", B, T, Lmax, H, D, dtype, 1), DEV, ctx)
    got = dsa.indexer_scores(qi.q, qi.w, ki.k, ctx_t, qi.q_scale, ki.k_scale)
    torch.cuda.synchronize()
    ref = oracle.indexer_scores(parity.host_real(qi.q, qi.q_scale), qi.w.cpu().double().numpy(),
                                parity.host_real(ki.k, ki.k_scale), ctx)
    parity.check_scores(got.cpu().numpy().astype(np.float64), ref, dtype)


@pytest.mark.parametrize("T,Lmax,dtype", [(1, 4100, "bf16"), (1, 1000, "fp8"), (5, 1000, "fp8"),
                                           (3, 4100, "bf16")])
def test_indexer_scores_tail_tile_stays_in_row(T, Lmax, dtype):
    """Lmax not a multiple of the key tile and ld = Lmax: the last tile's keys
    past Lmax must neither reach the next row's scores nor the memory after
    the last row (a canary after the output)."""
    B, H, D = 3, 64, 128
    say("tail tile case", T, Lmax, dtype)
    qi, ki = make_indexer(B, T, H, D, Lmax, dtype, seed=23 + T + Lmax)
    ctx = [Lmax, Lmax - 7, max(T, 40)]
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    ld = dsa.ld_for(Lmax)
    assert ld == Lmax
    n = B * T * ld
    buf = torch.full((n + 1024,), 7.0, dtype=torch.float32, device=DEV)
    out = buf[:n].view(B, T, ld)
    got = dsa.indexer_scores(qi.q, qi.w, ki.k, ctx_t, qi.q_scale, ki.k_scale, out=out)
    torch.cuda.synchronize()
    assert bool((buf[n:] == 7.0).all()), "scores written past the output"
    ref = oracle.indexer_scores(parity.host_real(qi.q, qi.q_scale), qi.w.cpu().double().numpy(),
                                parity.host_real(ki.k, ki.k_scale), ctx)
    parity.check_scores(got.cpu().numpy().astype(np.float64), ref, dtype)


def _rand_scores(B, T, L, seed, kind="normal"):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    if kind == "normal":
        x = torch.randn((B, T, L), generator=g, device=DEV)
    elif kind == "sampletop":  # every 16th position of the first 16384 far above the rest
        x = torch.rand((B, T, L), generator=g, device=DEV)
        m = min(1024, (L + 15) // 16)
        x[..., 0:16 * m:16] = 10.0 + torch.arange(m, device=DEV, dtype=torch.float32) / 1000.0
    elif kind == "few":        # heavy ties: 7 distinct values
        x = torch.randint(0, 7, (B, T, L), generator=g, device=DEV).float()
    elif kind == "equal":
        x = torch.full((B, T, L), 0.25, device=DEV)
    elif kind == "signed_zero":
        m = torch.randint(0, 2, (B, T, L), generator=g, device=DEV) == 1
        x = torch.where(m, torch.tensor(-0.0, device=DEV), torch.tensor(0.0, device=DEV))
    elif kind == "wide":
        x = torch.randn((B, T, L), generator=g, device=DEV) * 1e30
    elif kind.startswith("cluster"):
        # m scores in [1, 1.1) (one top-12-bit bin) over small noise, so the
        # threshold bin holds m keys: "clusterM", or "clustertieM" with the
        # cluster values on a grid of 101 (heavy ties inside the bin)
        tie = kind.startswith("clustertie")
        m = int(kind[len("clustertie" if tie else "cluster"):])
        r = np.random.default_rng(seed)
        x = r.standard_normal((B, T, L)) * 0.05
        for b in range(B):
            for t in range(T):
                at = r.choice(L, m, replace=False)
                v = r.integers(0, 101, m) / 1000.0 if tie else r.random(m) * 0.1
                x[b, t, at] = 1.0 + v
        x = torch.from_numpy(x.astype(np.float32)).to(DEV)
    else:
        raise ValueError(kind)
    ld = (L + 3) // 4 * 4          # rows padded to a multiple of 4 floats
    buf = torch.full((B, T, ld), float("nan"), device=DEV)
    buf[..., :L] = x
    return buf[..., :L]


TOPK_CASES = [
    # B, T, L, ctx, k, kind
    (1, 1, 4096, [4096], 256, "normal"),
    (2, 1, 131072, [131072, 90001], 2048, "normal"),
    (4, 1, 32768, [32768, 32767, 2048, 2047], 2048, "normal"),   # n == k and n < k rows
    (2, 1, 20000, [20000, 19999], 2048, "few"),                  # LDS list overflow path
    (1, 1, 5000, [5000], 300, "equal"),
    (1, 1, 3000, [3000], 64, "signed_zero"),
    (1, 1, 9000, [9000], 1000, "wide"),
    (1, 12, 4100, [4100], 1024, "normal"),                       # causal rows (T > 1)
    (3, 1, 70, [70, 13, 1], 16, "normal"),
    (2, 1, 40000, [40000, 39000], 2048, "equal"),                # chunked rows, list overflow
    (3, 1, 196608, [196608, 100000, 16385], 2048, "normal"),     # chunked, ragged rows
    (32, 1, 32768, [32768] * 32, 2048, "normal"),                # chunked, many rows
    # crowded threshold bin: refined by one wave (m <= 3072) or by the block
    (2, 1, 40000, [40000, 39000], 2048, "cluster2500"),          # chunked rows
    (2, 1, 40000, [40000, 39000], 2048, "clustertie3072"),
    (2, 1, 40000, [40000, 39000], 2048, "cluster5000"),
    # a list longer than one emission pass (8192 entries) but inside LDS
    (2, 1, 40000, [40000, 39000], 2048, "cluster11000"),
    (1, 4, 8192, [8192], 2048, "cluster3000"),                   # row kernel (T > 1)
    (1, 4, 8192, [8192], 2048, "clustertie2200"),
    (1, 4, 8192, [8192], 1000, "cluster6000"),
    # row kernel (more than 128 rows), rows held in registers (n <= 65536):
    # a bin bound taken from one sampled key per thread (positions 16 t),
    # which falls back to counting every key when the sample runs high
    # ("sampletop": the sampled positions hold the largest scores); rows up
    # to 65536, and rows on both sides of it
    (1, 130, 60000, [60000], 2048, "sampletop"),
    (1, 130, 65536, [65536], 2048, "normal"),
    (1, 130, 65600, [65600], 2048, "normal"),
]


@pytest.mark.parametrize("case", TOPK_CASES, ids=lambda c: f"B{c[0]}T{c[1]}L{c[2]}k{c[4]}{c[5]}")
def test_topk_exact(case):
    B, T, L, ctx, k, kind = case
    say("topk case", case)
    s = _rand_scores(B, T, L, seed=L + k, kind=kind)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    idx = dsa.topk(s, ctx_t, k)
    torch.cuda.synchronize()
    parity.check_topk_exact(idx.cpu().numpy(), s.cpu().numpy(), ctx, k)


def _rand_idx(B, T, ctx, k, seed, pad=0):
    """Distinct ascending visible positions per row, -1 padded (a valid top-k output)."""
    r = np.random.default_rng(seed)
    out = np.full((B, T, k), -1, np.int32)
    pos = oracle.query_positions(ctx, T)
    for b in range(B):
        for t in range(T):
            n = int(pos[b, t]) + 1
            m = max(0, min(k - pad, n))
            out[b, t, :m] = np.sort(r.choice(n, m, replace=False))
    return out


ATTN_CASES = [
    # B, T, Hq, Lmax, ctx, k, pad
    (1, 1, 16, 4096, [4096], 256, 0),
    (2, 1, 128, 8192, [8192, 5000], 2048, 0),
    (3, 1, 32, 1000, [1000, 40, 1], 100, 7),       # padded rows, ragged tile
    (1, 3, 64, 600, [600], 200, 0),                 # prefill rows
    (4, 1, 128, 2048, [2048] * 4, 1000, 0),
    (1, 256, 64, 4096, [4096], 2048, 5),            # one 2048-row slice per row
    (1, 64, 128, 4096, [4096], 3000, 0),            # k above the slice cap: two slices
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}k{c[5]}")
def test_sparse_attn(case):
    B, T, Hq, Lmax, ctx, k, pad = case
    say("attn case", case)
    s = gen.Shape(900 + Hq, "", 1, "F", B, T, Lmax, 1, 64, "bf16", k, Hq=Hq)
    q, kv = gen.make_mla_layer(s, 0, DEV)
    idx = _rand_idx(B, T, ctx, k, seed=Hq + k, pad=pad)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    out, lse = dsa.sparse_attn(q, kv, torch.from_numpy(idx).to(DEV), ctx_t, s.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attn(parity.host_real(q), parity.host_real(kv), idx, ctx, s.scale, 512)
    err = parity.check_attn(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl)
    say("  max abs err", err)


def test_sparse_equals_dense_when_k_covers_context():
    """k >= context: the sparse path over all positions equals dense attention."""
    B, T, Hq, L = 2, 1, 32, 700
    s = gen.Shape(77, "", 1, "F", B, T, L, 1, 64, "bf16", 1, Hq=Hq)
    q, kv = gen.make_mla_layer(s, 0, DEV)
    ctx = [700, 300]
    k = 800
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        idx[b, 0, :ctx[b]] = np.arange(ctx[b])
    out, lse = dsa.sparse_attn(q, kv, torch.from_numpy(idx).to(DEV),
                               torch.tensor(ctx, dtype=torch.int32, device=DEV), s.scale)
    torch.cuda.synchronize()
    do, dl = oracle.dense_attn(parity.host_real(q), parity.host_real(kv), ctx, s.scale, 512)
    parity.check_attn(out.float().cpu().numpy(), lse.cpu().numpy(), do, dl)


def test_sparse_attn_empty_rows():
    B, T, Hq, L, k = 2, 1, 16, 64, 40
    s = gen.Shape(78, "", 1, "F", B, T, L, 1, 64, "bf16", 1, Hq=Hq)
    q, kv = gen.make_mla_layer(s, 0, DEV)
    idx = np.full((B, T, k), -1, np.int32)
    idx[1, 0, :3] = [5, 9, 63]
    idx[0, 0, :2] = [70, 1000]      # beyond the context: ignored
    ctx = [64, 64]
    out, lse = dsa.sparse_attn(q, kv, torch.from_numpy(idx).to(DEV),
                               torch.tensor(ctx, dtype=torch.int32, device=DEV), s.scale)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    ro, rl = oracle.sparse_attn(parity.host_real(q), parity.host_real(kv), idx, ctx, s.scale, 512)
    parity.check_attn(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl)


def test_indexer_topk_end_to_end_boundary():
    """GPU scores -> GPU top-k against oracle fp64 scores -> oracle top-k."""
    B, T, H, D, L, k = 2, 1, 64, 128, 8192, 2048
    for dtype in ("bf16", "fp8"):
        qi, ki = make_indexer(B, T, H, D, L, dtype, seed=5)
        ctx = [8192, 6000]
        ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
        sc = dsa.indexer_scores(qi.q, qi.w, ki.k, ctx_t, qi.q_scale, ki.k_scale)
        idx = dsa.topk(sc, ctx_t, k)
        torch.cuda.synchronize()
        parity.check_topk_exact(idx.cpu().numpy(), sc.cpu().numpy(), ctx, k)
        ref = oracle.indexer_scores(parity.host_real(qi.q, qi.q_scale),
                                    qi.w.cpu().double().numpy(),
                                    parity.host_real(ki.k, ki.k_scale), ctx)
        st = parity.check_topk_boundary(idx.cpu().numpy(), ref, ctx, k)
        say(dtype, "boundary swaps", st)


def test_deterministic_reruns():
    B, T, H, D, L, k = 2, 1, 64, 128, 20000, 2048
    qi, ki = make_indexer(B, T, H, D, L, "fp8", seed=6)
    ctx_t = torch.tensor([L, L - 5], dtype=torch.int32, device=DEV)
    a = dsa.indexer_scores(qi.q, qi.w, ki.k, ctx_t, qi.q_scale, ki.k_scale).clone()
    b = dsa.indexer_scores(qi.q, qi.w, ki.k, ctx_t, qi.q_scale, ki.k_scale).clone()
    assert torch.equal(a, b)
    assert torch.equal(dsa.topk(a, ctx_t, k), dsa.topk(b, ctx_t, k))


def test_topk_workspace_reuse_left_zeroed():
    """The chunked top-k meets in a per-row histogram inside the workspace: a
    workspace reused across calls gives the same result as fresh ones and is
    zero again after each call."""
    B, T, L, k = 3, 1, 65536, 2048
    ctx = [65536, 50000, 3000]
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    nbytes = dsa.topk_workspace_size(B, T, L, k)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    for seed in (1, 2, 3):
        s = _rand_scores(B, T, L, seed=seed)
        idx = dsa.topk(s, ctx_t, k, workspace=ws)
        torch.cuda.synchronize()
        parity.check_topk_exact(idx.cpu().numpy(), s.cpu().numpy(), ctx, k)
        assert int(ws.count_nonzero().item()) == 0 or _hist_zero(ws, B)


def _hist_zero(ws, rows):
    return int(ws[: rows * 4096 * 4].count_nonzero().item()) == 0
