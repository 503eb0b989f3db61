"""Decode steps as a serving loop issues them (GPU).

Each step appends one new token per sequence to every layer's caches (latent
row bf16, indexer key bf16 or fp8 with its row scale) through the KV-append
entry point, then runs the IndexCache layer stack over the grown context.
After every step: the caches equal the oracle's append bit for bit, every F
layer's index set satisfies the top-k boundary rule against the oracle's fp64
scores on those caches, the shared index buffer holds the last F layer's set,
and every layer's attention output matches the oracle run over the index set
the GPU used.  The loop runs with the separate indexer and top-k kernels
and, for fp8 keys, also with the fused indexer + top-k.
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


def cache_bits(t):
    """Raw codes of a cache tensor (bf16 -> uint16, fp8 -> uint8)."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("idx_dtype,D,fused", [("fp8", 128, False), ("bf16", 64, False),
                                               ("fp8", 128, True)])
def test_append_then_stack_for_three_steps(idx_dtype, D, fused):
    B, Lmax, H, k, Hq = 2, 1200, 16, 128, 32
    pattern = "FSSF"
    ctx = [900, 517]
    fp8 = idx_dtype == "fp8"
    s = gen.Shape(7100 + D, "decode loop", len(pattern), pattern, B=B, T=1, ctx=Lmax, H=H,
                  D=D, idx_dtype=idx_dtype, k=k, Hq=Hq)
    kb = gen.make_key_base(s, DEV)
    layers = []
    for l in range(s.n_layers):
        ki = gen.make_indexer_keys(s, l, kb, DEV)
        _, kv = gen.make_mla_layer(s, l, DEV)
        layers.append(dict(k_idx=ki.k, k_idx_scale=ki.k_scale, kv=kv,
                           out=torch.empty((B, 1, Hq, s.d_v), dtype=torch.bfloat16, device=DEV),
                           lse=torch.empty((B, 1, Hq), dtype=torch.float32, device=DEV)))
    # host mirror of every layer's caches (the oracle appends into it)
    mirror = [[cache_bits(L["kv"]), cache_bits(L["k_idx"]),
               None if L["k_idx_scale"] is None else L["k_idx_scale"].cpu().numpy()]
              for L in layers]
    rng = np.random.default_rng(31 + D)
    for step in range(3):
        ctx = [c + 1 for c in ctx]
        ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
        say(f"{idx_dtype} step {step}: contexts {ctx}")
        # the new token's rows, appended to every layer's caches
        for l, L in enumerate(layers):
            kv_new = rng.standard_normal((B, 1, s.d_qk)).astype(np.float32)
            k_new = rng.standard_normal((B, 1, D)).astype(np.float32)
            dsa.kv_append(ctx_t, torch.from_numpy(kv_new).to(DEV), L["kv"],
                          torch.from_numpy(k_new).to(DEV), L["k_idx"], L["k_idx_scale"])
            mirror[l] = list(oracle.kv_append(mirror[l][0], mirror[l][1], mirror[l][2], kv_new,
                                              k_new, ctx, fp8))
        torch.cuda.synchronize()
        for l, L in enumerate(layers):
            assert np.array_equal(cache_bits(L["kv"]), mirror[l][0]), f"latent cache, layer {l}"
            assert np.array_equal(cache_bits(L["k_idx"]), mirror[l][1]), f"key cache, layer {l}"
            if fp8:
                assert np.array_equal(L["k_idx_scale"].cpu().numpy().view(np.uint32),
                                      mirror[l][2].view(np.uint32)), f"key scales, layer {l}"
        # this step's queries (indexer query and weights shared by the layers)
        sq = gen.Shape(7200 + 10 * step + D, "decode loop", len(pattern), pattern, B=B, T=1,
                       ctx=Lmax, H=H, D=D, idx_dtype=idx_dtype, k=k, Hq=Hq)
        qi = gen.make_indexer_query(sq, DEV, w_low=-0.2)
        for l, L in enumerate(layers):
            q, _ = gen.make_mla_layer(sq, l, DEV)
            L.update(q_idx=qi.q, q_idx_scale=qi.q_scale, w=qi.w, q=q)
        st = dsa.Stack(pattern, layers, ctx_t, B=B, T=1, H=H, D=D, Lmax=Lmax, k=k, Hq=Hq,
                       idx_dtype=idx_dtype, scale=s.scale, fused_topk=fused)
        assert st.fused == fused
        stats = st.run()
        torch.cuda.synchronize()
        assert stats["n_indexer_calls"] == pattern.count("F")
        used = None
        for l, c in enumerate(pattern):
            L = layers[l]
            q_idx = parity.host_real(L["q_idx"], L["q_idx_scale"])
            w = L["w"].cpu().double().numpy()
            k_idx = parity.host_real(L["k_idx"], L["k_idx_scale"])
            if c == "F":
                sc = dsa.indexer_scores(L["q_idx"], L["w"], L["k_idx"], ctx_t, L["q_idx_scale"],
                                        L["k_idx_scale"])
                used = dsa.topk(sc, ctx_t, k).cpu().numpy()
                parity.check_topk_boundary(used, oracle.indexer_scores(q_idx, w, k_idx, ctx),
                                           ctx, k)
            ro, rl = oracle.sparse_attn(parity.host_real(L["q"]), parity.host_real(L["kv"]),
                                        used, ctx, s.scale, s.d_v)
            err = parity.check_attn(L["out"].float().cpu().numpy(), L["lse"].cpu().numpy(),
                                    ro, rl)
            say(f"  layer {l} {c}: attention max abs err {err:.3g}")
        assert np.array_equal(st.idx_buf.cpu().numpy(), used)
