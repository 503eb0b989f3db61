"""The IndexCache layer stack on the GPU against the fp64 oracle (tiny decode workload)."""
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


def build_layers(s: gen.Shape):
    qi = gen.make_indexer_query(s, DEV)
    kb = gen.make_key_base(s, DEV)
    layers = []
    for l in range(s.n_layers):
        ki = gen.make_indexer_keys(s, l, kb, DEV)
        q, kv = gen.make_mla_layer(s, l, DEV)
        layers.append(dict(q_idx=qi.q, q_idx_scale=qi.q_scale, w=qi.w, k_idx=ki.k,
                           k_idx_scale=ki.k_scale, q=q, kv=kv,
                           out=torch.empty((s.B, s.T, s.Hq, s.d_v), dtype=torch.bfloat16,
                                           device=DEV),
                           lse=torch.empty((s.B, s.T, s.Hq), dtype=torch.float32, device=DEV)))
    return layers


def shape_kwargs(s):
    return dict(B=s.B, T=s.T, H=s.H, D=s.D, Lmax=s.Lmax, k=s.k, Hq=s.Hq,
                idx_dtype=s.idx_dtype, scale=s.scale)


def oracle_layers(layers, s):
    out = []
    for L in layers:
        out.append(dict(q_idx=parity.host_real(L["q_idx"], L["q_idx_scale"]),
                        w=L["w"].cpu().double().numpy(),
                        k_idx=parity.host_real(L["k_idx"], L["k_idx_scale"]),
                        q=parity.host_real(L["q"]), kv=parity.host_real(L["kv"])))
    return out


@pytest.mark.parametrize("pattern", ["FSSS", "FFFF", "FSFS"])
def test_tiny_stack_against_oracle(pattern):
    s = gen.CONFIGS[0]
    say("stack C0 pattern", pattern)
    layers = build_layers(s)
    ctx_t = gen.ctx_lens(s, DEV)
    ctx = [s.ctx] * s.B
    st = dsa.Stack(pattern, layers, ctx_t, **shape_kwargs(s))
    stats = st.run()
    torch.cuda.synchronize()
    assert stats["n_indexer_calls"] == pattern.count("F")
    assert stats["n_topk_calls"] == pattern.count("F")
    assert stats["n_attn_calls"] == len(pattern)
    # GPU index set of every F layer through the standalone entry points
    gpu_idx = {}
    for l, c in enumerate(pattern):
        if c == "F":
            L = layers[l]
            sc = dsa.indexer_scores(L["q_idx"], L["w"], L["k_idx"], ctx_t, L["q_idx_scale"],
                                    L["k_idx_scale"])
            gpu_idx[l] = dsa.topk(sc, ctx_t, s.k).cpu().numpy()
    last_f = max(gpu_idx)
    assert np.array_equal(st.idx_buf.cpu().numpy(), gpu_idx[last_f])
    ol = oracle_layers(layers, s)
    ref = oracle.run_stack(pattern, ol, ctx, s.k, s.scale, s.d_v)
    assert ref["n_indexer_calls"] == stats["n_indexer_calls"]
    used = None
    for l, c in enumerate(pattern):
        if c == "F":
            used = gpu_idx[l]
            sc = oracle.indexer_scores(ol[l]["q_idx"], ol[l]["w"], ol[l]["k_idx"], ctx)
            parity.check_topk_boundary(used, sc, ctx, s.k)
        # attention of layer l on the index set the GPU used
        ro, rl = oracle.sparse_attn(ol[l]["q"], ol[l]["kv"], used, ctx, s.scale, s.d_v)
        parity.check_attn(layers[l]["out"].float().cpu().numpy(), layers[l]["lse"].cpu().numpy(),
                          ro, rl)
        # and end to end against the oracle's own stack
        parity.check_attn(layers[l]["out"].float().cpu().numpy(), None, ref["out"][l], None)


def test_shared_layers_match_all_f_on_identical_keys():
    """With the same keys in every layer, every pattern reproduces all-F outputs bit for bit."""
    s = gen.CONFIGS[0]
    layers = build_layers(s)
    for L in layers[1:]:
        L["k_idx"] = layers[0]["k_idx"]
    ctx_t = gen.ctx_lens(s, DEV)
    outs = {}
    for p in ("FFFF", "FSSS", "FSFS"):
        dsa.Stack(p, layers, ctx_t, **shape_kwargs(s)).run()
        torch.cuda.synchronize()
        outs[p] = [L["out"].clone() for L in layers]
    for p in ("FSSS", "FSFS"):
        for a, b in zip(outs[p], outs["FFFF"]):
            assert torch.equal(a, b)


@pytest.mark.parametrize("bad", ["SFFF", "FSX", "FSS", "FSSSS"])
def test_bad_pattern_rejected_before_launch(bad):
    s = gen.CONFIGS[0]
    layers = build_layers(s)
    st = dsa.Stack("FSSS", layers, gen.ctx_lens(s, DEV), **shape_kwargs(s))
    st.pattern = bad.encode()
    st.n_layers = 4
    with pytest.raises(dsa.DSAError) as e:
        st.run()
    assert e.value.status == 1


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate"])
@pytest.mark.parametrize("idx_dtype", ["fp8", "bf16"])
def test_stack_fused_histogram_ragged(idx_dtype, fused):
    """Long rows take the chunked top-k, whose first histogram the decode
    indexer builds inside the stack.  Rows with n <= k (every visible position
    kept) and consecutive F layers must leave that histogram clean: each F
    layer's set equals the standalone kernels' (indexer, then top-k with its
    own histogram pass), for every row, and a second run of the same stack
    reproduces it.  Both stack paths: the separate indexer (histogram built
    on the way) + top-k, and the fused indexer + top-k."""
    s = gen.Shape(90, "fused histogram", 3, "FFS", B=3, T=1, ctx=32768, H=16, D=128,
                  idx_dtype=idx_dtype, k=2048, Hq=0)
    say("stack with fused histogram,", idx_dtype)
    qi = gen.make_indexer_query(s, DEV)
    kb = gen.make_key_base(s, DEV)
    layers = []
    for l in range(s.n_layers):
        ki = gen.make_indexer_keys(s, l, kb, DEV)
        layers.append(dict(q_idx=qi.q, q_idx_scale=qi.q_scale, w=qi.w, k_idx=ki.k,
                           k_idx_scale=ki.k_scale))
    # ragged: one row with fewer visible positions than k, one just above k
    ctx_t = torch.tensor([1000, 2049, 32768], dtype=torch.int32, device=DEV)
    for run in range(2):
        for p in ("FFS", "FSF"):
            st = dsa.Stack(p, layers, ctx_t, B=s.B, T=1, H=s.H, D=s.D, Lmax=s.Lmax, k=s.k, Hq=0,
                           idx_dtype=s.idx_dtype, scale=s.scale, fused_topk=fused)
            assert st.fused == fused
            st.run()
            torch.cuda.synchronize()
            last_f = max(i for i, c in enumerate(p) if c == "F")
            L = layers[last_f]
            sc = dsa.indexer_scores(L["q_idx"], L["w"], L["k_idx"], ctx_t, L["q_idx_scale"],
                                    L["k_idx_scale"])
            want = dsa.topk(sc, ctx_t, s.k)
            torch.cuda.synchronize()
            got = st.idx_buf.cpu().numpy()
            assert np.array_equal(got, want.cpu().numpy()), (run, p)
            assert np.array_equal(got[0, 0, :1000], np.arange(1000)) and np.all(got[0, 0, 1000:] == -1)
            parity.check_topk_exact(got, sc.cpu().numpy(), [1000, 2049, 32768], s.k)
            say(f"  run {run} pattern {p}: ok")


@pytest.mark.parametrize("idx_dtype,D,k,Hq", [("bf16", 64, 128, 32), ("fp8", 128, 512, 16)],
                         ids=["bf16-k128-unsplit", "fp8-k512-split"])
def test_prefill_stack_against_oracle(idx_dtype, D, k, Hq):
    """A chunked-prefill stack under IndexCache: T query rows per sequence
    (causal, row t sees keys <= ctx - T + t), ragged contexts, the F/S branch,
    the prefill indexer kernel and sparse attention over per-row index sets
    (with and without split-KV), against the fp64 oracle's stack."""
    s = gen.Shape(91, "prefill stack", 4, "FSFS", B=2, T=24, ctx=1536, H=8, D=D,
                  idx_dtype=idx_dtype, k=k, Hq=Hq)
    say("prefill stack", idx_dtype, "k", k, "Hq", Hq)
    layers = build_layers(s)
    ctx = [1536, 1000]
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    st = dsa.Stack(s.pattern, layers, ctx_t, **shape_kwargs(s))
    stats = st.run()
    torch.cuda.synchronize()
    assert stats["n_indexer_calls"] == 2 and stats["n_attn_calls"] == 4
    ol = oracle_layers(layers, s)
    ref = oracle.run_stack(s.pattern, ol, ctx, s.k, s.scale, s.d_v)
    used = None
    for l, c in enumerate(s.pattern):
        if c == "F":
            L = layers[l]
            sc = dsa.indexer_scores(L["q_idx"], L["w"], L["k_idx"], ctx_t, L["q_idx_scale"],
                                    L["k_idx_scale"])
            used = dsa.topk(sc, ctx_t, s.k).cpu().numpy()
            osc = oracle.indexer_scores(ol[l]["q_idx"], ol[l]["w"], ol[l]["k_idx"], ctx)
            parity.check_scores(sc.cpu().numpy()[..., :s.Lmax].astype(np.float64), osc, idx_dtype)
            parity.check_topk_exact(used, sc.cpu().numpy(), ctx, s.k)
            parity.check_topk_boundary(used, osc, ctx, s.k)
        ro, rl = oracle.sparse_attn(ol[l]["q"], ol[l]["kv"], used, ctx, s.scale, s.d_v)
        parity.check_attn(layers[l]["out"].float().cpu().numpy(), layers[l]["lse"].cpu().numpy(),
                          ro, rl)
        parity.check_attn(layers[l]["out"].float().cpu().numpy(), None, ref["out"][l], None)
        say(f"  layer {l} {c}: ok")
    assert np.array_equal(st.idx_buf.cpu().numpy(), used)


def test_stack_replays_from_a_hip_graph():
    """A whole decode step of the stack (chunked top-k with the indexer-built
    histogram, split-KV attention) captured into one HIP graph and replayed:
    every replay, with eager work and synchronisations in between, must give
    the eager run's outputs and index set bit for bit.  The stack issues no
    memset nodes; its workspace is left zero-filled by every step, which is
    what makes the replays independent."""
    s = gen.Shape(95, "graph replay", 8, "FSSSFSSS", B=2, T=1, ctx=20000, H=32, D=128,
                  idx_dtype="fp8", k=1024, Hq=32)
    say("stack graph replay")
    layers = build_layers(s)
    ctx_t = torch.tensor([20000, 15001], dtype=torch.int32, device=DEV)
    st = dsa.Stack(s.pattern, layers, ctx_t, **shape_kwargs(s))
    st.run()
    torch.cuda.synchronize()
    want_out = [L["out"].clone() for L in layers]
    want_lse = [L["lse"].clone() for L in layers]
    want_idx = st.idx_buf.clone()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        st.run()                       # a warm-up on the capture stream
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        st.run()
    torch.cuda.synchronize()
    for rep in range(3):
        for L in layers:               # eager work between replays
            L["out"].zero_()
            L["lse"].fill_(7.0)
        st.idx_buf.fill_(-5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l, L in enumerate(layers):
            assert torch.equal(L["out"].view(torch.int16), want_out[l].view(torch.int16)), (rep, l)
            assert torch.equal(L["lse"], want_lse[l]), (rep, l)
        assert torch.equal(st.idx_buf, want_idx), rep
        say(f"  replay {rep}: identical")
