"""Chunked prefill under IndexCache, chunk after chunk (GPU).

A prompt is taken in chunks of T tokens: each chunk's latent rows and indexer
keys are appended to every layer's caches (KV-append entry point, T > 1),
then the chunk's T query rows run through the layer stack over the grown
context (query row t of a chunk sits at position ctx - T + t and sees the
earlier chunks and the rows of its own chunk up to itself).  After every
chunk: the caches equal the oracle's append bit for bit, every F layer's
index sets satisfy the top-k boundary rule against the oracle's fp64 scores
on those caches, S layers attend with the preceding F layer's sets, and every
layer's attention output matches the oracle over the index sets the GPU used.
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
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("idx_dtype,D,T,k", [("fp8", 128, 40, 128), ("bf16", 64, 24, 256)])
def test_prefill_chunks_append_then_stack(idx_dtype, D, T, k):
    B, Lmax, H, Hq = 2, 1400, 16, 32
    pattern = "FSSF"
    ctx = [300, 150]            # tokens already in the caches before the first chunk
    fp8 = idx_dtype == "fp8"
    s = gen.Shape(7400 + D, "chunked prefill", len(pattern), pattern, B=B, T=T, ctx=Lmax, H=H,
                  D=D, idx_dtype=idx_dtype, k=k, Hq=Hq)
    kb = gen.make_key_base(s, DEV)
    layers = []
    for l in range(s.n_layers):
        ki = gen.make_indexer_keys(s, l, kb, DEV)
        _, kv = gen.make_mla_layer(s, l, DEV)
        layers.append(dict(k_idx=ki.k, k_idx_scale=ki.k_scale, kv=kv,
                           out=torch.empty((B, T, Hq, s.d_v), dtype=torch.bfloat16, device=DEV),
                           lse=torch.empty((B, T, Hq), dtype=torch.float32, device=DEV)))
    mirror = [[cache_bits(L["kv"]), cache_bits(L["k_idx"]),
               None if L["k_idx_scale"] is None else L["k_idx_scale"].cpu().numpy()]
              for L in layers]
    rng = np.random.default_rng(47 + D)
    for chunk in range(3):
        ctx = [c + T for c in ctx]
        ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
        say(f"{idx_dtype} chunk {chunk}: {T} tokens, contexts now {ctx}")
        for l, L in enumerate(layers):
            kv_new = rng.standard_normal((B, T, s.d_qk)).astype(np.float32)
            k_new = rng.standard_normal((B, T, D)).astype(np.float32)
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
        sq = gen.Shape(7500 + 10 * chunk + D, "chunked prefill", len(pattern), pattern, B=B,
                       T=T, ctx=Lmax, H=H, D=D, idx_dtype=idx_dtype, k=k, Hq=Hq)
        qi = gen.make_indexer_query(sq, DEV, w_low=-0.2)
        for l, L in enumerate(layers):
            q, _ = gen.make_mla_layer(sq, l, DEV)
            L.update(q_idx=qi.q, q_idx_scale=qi.q_scale, w=qi.w, q=q)
        st = dsa.Stack(pattern, layers, ctx_t, B=B, T=T, H=H, D=D, Lmax=Lmax, k=k, Hq=Hq,
                       idx_dtype=idx_dtype, scale=s.scale)
        stats = st.run()
        torch.cuda.synchronize()
        assert stats["n_indexer_calls"] == pattern.count("F")
        used = None
        for l, c in enumerate(pattern):
            L = layers[l]
            if c == "F":
                sc = dsa.indexer_scores(L["q_idx"], L["w"], L["k_idx"], ctx_t, L["q_idx_scale"],
                                        L["k_idx_scale"])
                used = dsa.topk(sc, ctx_t, k).cpu().numpy()
                ref = oracle.indexer_scores(parity.host_real(L["q_idx"], L["q_idx_scale"]),
                                            L["w"].cpu().double().numpy(),
                                            parity.host_real(L["k_idx"], L["k_idx_scale"]), ctx)
                parity.check_topk_boundary(used, ref, ctx, k)
            ro, rl = oracle.sparse_attn(parity.host_real(L["q"]), parity.host_real(L["kv"]),
                                        used, ctx, s.scale, s.d_v)
            err = parity.check_attn(L["out"].float().cpu().numpy(), L["lse"].cpu().numpy(),
                                    ro, rl)
            say(f"  layer {l} {c}: attention max abs err {err:.3g}")
        assert np.array_equal(st.idx_buf.cpu().numpy(), used)
        # the earliest query row of the chunk sees fewer keys than the last
        pos = oracle.query_positions(ctx, T)
        assert np.all((used[:, 0] <= pos[:, :1]) | (used[:, 0] == -1))
