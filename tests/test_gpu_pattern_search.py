"""Pattern-search cost matrix on the GPU against the oracle (GPU).

The device builds every layer's own index set, runs the reuse attentions
and reduces the proxies; the oracle recomputes the matrix from the same
index sets (checked separately against its own top-k with the k-th boundary
rule).  The miss proxy is integer counting followed by one division, so it
must match bit for bit.

The output proxy compares the kernel's bf16 attention outputs, so its
tolerance follows the attention kernel's roundings (u = 2^-8, the unit
roundoff of bf16).  For one output element o_d = sum_j p_j v_jd / sum_j p_j
over the selected rows, with A_d = sum_j p_j |v_jd| / sum_j p_j:
  * the probabilities enter P.V rounded to bf16 while the row sum keeps them
    in fp32: error at most u A_d;
  * split-KV slices store their normalised partial outputs in bf16, and the
    merge weights sum to one: at most u sum_i w_i |o_i,d| <= u A_d;
  * the final output is rounded to bf16: at most u |o_d| <= u A_d;
  * the logits are fp32 sums of 576 exact bf16 products: each is off by at
    most delta = scale * 576 * 2^-24 * sum_c |q_c kv_jc|, which moves every
    p_j / sum p by a factor within exp(+-2 delta_max): at most
    (exp(2 delta_max) - 1) A_d.
So |gpu_d - o_d| <= c A_d with c = 3u + 4u^2 + exp(2 delta_max) - 1, and over a
whole output the error vector has norm E <= ||c A||.  With R = ||o_own|| and
N = ||o_reused - o_own||, a cost C = N^2 / R^2 computed from the GPU's outputs
lies in [(N - E_reused - E_own)_+^2 / (R + E_own)^2,
(N + E_reused + E_own)^2 / (R - E_own)^2]; the test asserts that interval.
"""
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
U_BF16 = 2.0 ** -8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def build_stack(n_layers, B, T, ctx, H, D, dtype, k, Hq, early, transition, seed):
    s = gen.Shape(seed, "search", n_layers, "F" * n_layers, B=B, T=T, ctx=max(ctx), H=H, D=D,
                  idx_dtype=dtype, k=k, Hq=Hq)
    qi = gen.make_indexer_query(s, DEV)
    seg = gen.calibration_segments(n_layers, early, transition)
    bases = {g: gen.make_segment_base(s, g, DEV) for g in sorted(set(seg))}
    layers = []
    for l in range(n_layers):
        ki = gen.make_indexer_keys(s, l, bases[seg[l]], DEV)
        L = dict(q_idx=qi.q, q_idx_scale=qi.q_scale, w=qi.w, k_idx=ki.k, k_idx_scale=ki.k_scale)
        if Hq:
            q, kv = gen.make_mla_layer(s, l, DEV)
            L.update(q=q, kv=kv,
                     out=torch.empty((B, T, Hq, s.d_v), dtype=torch.bfloat16, device=DEV),
                     lse=torch.empty((B, T, Hq), dtype=torch.float32, device=DEV))
        layers.append(L)
    return s, layers, seg, gen.ctx_lens(s, DEV, ctx)


def kw(s):
    return dict(B=s.B, T=s.T, H=s.H, D=s.D, Lmax=s.Lmax, k=s.k, Hq=s.Hq,
                idx_dtype=s.idx_dtype, scale=s.scale)


def gpu_sets(s, layers, ctx_t, ctx, check_against_oracle=True):
    """Each layer's own set through the standalone kernels (the cost builder
    runs the same kernels), checked against the oracle's top-k."""
    sets = []
    for L in layers:
        sc = dsa.indexer_scores(L["q_idx"], L["w"], L["k_idx"], ctx_t, L["q_idx_scale"],
                                L["k_idx_scale"])
        idx = dsa.topk(sc, ctx_t, s.k).cpu().numpy()
        if check_against_oracle:
            ref = oracle.indexer_scores(parity.host_real(L["q_idx"], L["q_idx_scale"]),
                                        L["w"].cpu().double().numpy(),
                                        parity.host_real(L["k_idx"], L["k_idx_scale"]), ctx)
            parity.check_topk_boundary(idx, ref, ctx, s.k)
        sets.append(idx)
    return sets


def error_norm(hl, idx, ctx, s):
    """Bound on the norm of (kernel output - exact output) for one layer's
    attention over the index set idx: || c * A || (see the module docstring)."""
    q, kv = hl["q"], hl["kv"]
    B, T, Hq, _ = q.shape
    pos = oracle.query_positions(ctx, T)
    _, lse = oracle.sparse_attn(q, kv, idx, ctx, s.scale, s.d_v)
    total = 0.0
    for b in range(B):
        for t in range(T):
            sel = np.asarray(idx[b, t], dtype=np.int64)
            sel = sel[(sel >= 0) & (sel <= pos[b, t]) & (sel < kv.shape[1])]
            if sel.size == 0:
                continue
            rows = kv[b, sel]
            logits = s.scale * (q[b, t] @ rows.T)                  # [Hq, n]
            w = np.exp(logits - lse[b, t][:, None])                 # softmax weights
            A = w @ np.abs(rows[:, :s.d_v])                         # [Hq, d_v]
            delta = s.scale * q.shape[-1] * 2.0 ** -24 * (np.abs(q[b, t]) @ np.abs(rows).T)
            c = 3 * U_BF16 + 4 * U_BF16 ** 2 + math.expm1(2 * float(delta.max()))
            total += float(np.sum((c * A) ** 2))
    return math.sqrt(total)


def host_layers(layers):
    return [dict(q=parity.host_real(L["q"]), kv=parity.host_real(L["kv"])) for L in layers]


CASES = [
    # n, B, T, ctx, H, D, dtype, k, Hq, early, transition
    (6, 2, 1, [900, 1300], 16, 64, "bf16", 128, 16, 2, 4),
    (5, 1, 3, [2100], 32, 128, "fp8", 256, 32, 1, 3),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"n{c[0]}B{c[1]}T{c[2]}{c[6]}k{c[7]}")
def test_output_cost_matrix(case):
    n, B, T, ctx, H, D, dtype, k, Hq, early, trans = case
    say("reuse costs (output proxy)", case)
    s, layers, _, ctx_t = build_stack(n, B, T, ctx, H, D, dtype, k, Hq, early, trans, seed=31)
    cost = dsa.reuse_costs(layers, ctx_t, proxy="output", **kw(s))
    torch.cuda.synchronize()
    got = cost.cpu().numpy()
    sets = gpu_sets(s, layers, ctx_t, ctx)
    hl = host_layers(layers)
    ref = oracle.reuse_costs(hl, ctx, k, s.scale, s.d_v, "output", idx_sets=sets)
    assert np.all(got[np.triu_indices(n)] == 0)
    own = [oracle.sparse_attn(hl[l]["q"], hl[l]["kv"], sets[l], ctx, s.scale, s.d_v)[0]
           for l in range(n)]
    err_own = [error_norm(hl[l], sets[l], ctx, s) for l in range(n)]
    checked = 0
    for l in range(n):
        R = float(np.linalg.norm(own[l]))
        for j in range(l):
            o = oracle.sparse_attn(hl[l]["q"], hl[l]["kv"], sets[j], ctx, s.scale, s.d_v)[0]
            N = float(np.linalg.norm(o - own[l]))
            E = error_norm(hl[l], sets[j], ctx, s) + err_own[l]
            lo = max(0.0, N - E) ** 2 / (R + err_own[l]) ** 2
            hi = (N + E) ** 2 / (R - err_own[l]) ** 2
            assert abs(ref[l, j] - N * N / (R * R)) <= 1e-9 * max(1.0, ref[l, j])
            assert lo <= got[l, j] <= hi, (l, j, got[l, j], ref[l, j], lo, hi)
            checked += 1
    say(f"{checked} output costs within their rounding bounds")
    # each layer's out holds its all-F output
    for l in range(n):
        o, z = oracle.sparse_attn(hl[l]["q"], hl[l]["kv"], sets[l], ctx, s.scale, s.d_v)
        parity.check_attn(layers[l]["out"].float().cpu().numpy(), layers[l]["lse"].cpu().numpy(),
                          o, z)
    low = np.tril_indices(n, -1)
    say("cost range", float(ref[low].min()), float(ref[low].max()))


@pytest.mark.parametrize("dtype,T,ctx,k", [("fp8", 1, [700, 3000, 2049], 2048),
                                           ("bf16", 5, [300, 4100], 512)],
                         ids=["decode-ragged-short-rows", "prefill-rows"])
def test_miss_cost_matrix_exact(dtype, T, ctx, k):
    """Rows with fewer visible positions than k (-1 padded) included."""
    n = 7
    say("reuse costs (miss proxy)", dtype, T, ctx, k)
    s, layers, _, ctx_t = build_stack(n, len(ctx), T, ctx, 64, 128, dtype, k, 0, 2, 4, seed=32)
    cost = dsa.reuse_costs(layers, ctx_t, proxy="miss", **kw(s))
    torch.cuda.synchronize()
    got = cost.cpu().numpy()
    sets = gpu_sets(s, layers, ctx_t, ctx)
    ref = oracle.reuse_costs([{}] * n, ctx, k, s.scale, s.d_v, "miss", idx_sets=sets)
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), (got, ref)


def test_search_finds_planted_layers():
    """A stack whose first two layers and the start of two later segments
    have unrelated key caches: four greedy steps convert exactly the other
    four layers, under both proxies, and the device-matrix search equals the
    oracle's search on the same matrix."""
    n = 8
    say("planted search")
    s, layers, seg, ctx_t = build_stack(n, 2, 1, [4096, 3000], 32, 128, "fp8", 256, 16, 2, 5,
                                        seed=33)
    starts = {l for l in range(n) if l == 0 or seg[l] != seg[l - 1]}
    assert starts == {0, 1, 2, 5}
    for proxy in ("output", "miss"):
        cost = dsa.reuse_costs(layers, ctx_t, proxy=proxy, **kw(s)).cpu().numpy()
        trace = dsa.greedy_search(cost, 4)
        assert trace == oracle.greedy_pattern_search(cost, 4)
        final = trace[-1][0]
        assert {l for l, c in enumerate(final) if c == "F"} == starts, (proxy, final)
        assert dsa.pattern_cost(cost, final) == trace[-1][1]
        say(proxy, [p for p, _ in trace])


def test_cost_matrix_is_deterministic():
    """Two calls on one reused workspace give the same bits (the workspace's
    top-k region is left zero-filled by every call)."""
    say("determinism")
    s, layers, _, ctx_t = build_stack(4, 2, 1, [1500, 1500], 16, 64, "bf16", 128, 16, 1, 2,
                                      seed=34)
    need = dsa.reuse_costs_workspace_size(proxy="output", n_layers=4, **kw(s))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    a = dsa.reuse_costs(layers, ctx_t, proxy="output", workspace=ws, **kw(s)).cpu().numpy()
    b = dsa.reuse_costs(layers, ctx_t, proxy="output", workspace=ws, **kw(s)).cpu().numpy()
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))
