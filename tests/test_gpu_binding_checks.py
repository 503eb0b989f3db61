"""The Python binding rejects mis-shaped buffers and short workspaces before
anything is launched: the C ABI receives only pointers, so a buffer of the
wrong size would otherwise be read or written out of bounds (GPU; no kernel
runs in these tests)."""
import pytest
import torch

import dsa_sparse_attention_lightning_amd as dsa
from dsa_sparse_attention_lightning_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _attn_case(B=8, Hq=128, k=2048, Lmax=4096):
    q = torch.zeros((B, 1, Hq, 576), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((B, Lmax, 576), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((B, 1, k), dtype=torch.int32, device=DEV)
    ctx = torch.full((B,), Lmax, dtype=torch.int32, device=DEV)
    return q, kv, idx, ctx


def test_short_attention_workspace_is_rejected():
    q, kv, idx, ctx = _attn_case()
    need = dsa.sparse_attn_workspace_size(8, 1, 128, 2048)
    assert need > 0   # this shape is split over the GPU: partials need room
    ws = torch.zeros(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(dsa.DSAError) as e:
        dsa.sparse_attn(q, kv, idx, ctx, 0.07, workspace=ws)
    assert e.value.status == _lib.DSA_ERR_WORKSPACE


def test_short_topk_workspace_is_rejected():
    B, L, k = 2, 50000, 2048
    scores = torch.zeros((B, 1, L), dtype=torch.float32, device=DEV)
    ctx = torch.full((B,), L, dtype=torch.int32, device=DEV)
    need = dsa.topk_workspace_size(B, 1, L, k)
    ws = torch.zeros(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(dsa.DSAError) as e:
        dsa.topk(scores, ctx, k, workspace=ws)
    assert e.value.status == _lib.DSA_ERR_WORKSPACE


@pytest.mark.parametrize("bad", ["out", "lse", "ctx", "kv", "idx", "ws_dtype"])
def test_misshaped_attention_buffers_are_rejected(bad):
    q, kv, idx, ctx = _attn_case(B=2, Hq=32, k=256, Lmax=1000)
    out = torch.empty((2, 1, 32, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((2, 1, 32), dtype=torch.float32, device=DEV)
    ws = None
    if bad == "out":
        out = torch.empty((2, 1, 16, 512), dtype=torch.bfloat16, device=DEV)
    elif bad == "lse":
        lse = torch.empty((2, 32), dtype=torch.float32, device=DEV)
    elif bad == "ctx":
        ctx = ctx[:1].contiguous()
    elif bad == "kv":
        kv = kv[:1].contiguous()
    elif bad == "idx":
        idx = torch.zeros((1, 1, 256), dtype=torch.int32, device=DEV)
    elif bad == "ws_dtype":
        ws = torch.zeros(1 << 20, dtype=torch.float32, device=DEV)
    with pytest.raises(TypeError):
        dsa.sparse_attn(q, kv, idx, ctx, 0.07, out=out, lse=lse, workspace=ws)


@pytest.mark.parametrize("bad", ["w", "k_scale", "q_scale", "out", "ctx"])
def test_misshaped_indexer_buffers_are_rejected(bad):
    B, T, H, D, L = 2, 1, 8, 128, 300
    q = torch.zeros((B, T, H, D), dtype=torch.float8_e4m3fn, device=DEV)
    k = torch.zeros((B, L, D), dtype=torch.float8_e4m3fn, device=DEV)
    w = torch.zeros((B, T, H), dtype=torch.float32, device=DEV)
    qs = torch.ones((B, T, H), dtype=torch.float32, device=DEV)
    ks = torch.ones((B, L), dtype=torch.float32, device=DEV)
    ctx = torch.full((B,), L, dtype=torch.int32, device=DEV)
    out = torch.empty((B, T, dsa.ld_for(L)), dtype=torch.float32, device=DEV)
    if bad == "w":
        w = torch.zeros((B, T, H - 1), dtype=torch.float32, device=DEV)
    elif bad == "k_scale":
        ks = torch.ones((B, L - 1), dtype=torch.float32, device=DEV)
    elif bad == "q_scale":
        qs = None
    elif bad == "out":
        out = torch.empty((B, T, L - 1), dtype=torch.float32, device=DEV)
    elif bad == "ctx":
        ctx = torch.full((B + 1,), L, dtype=torch.int32, device=DEV)
    with pytest.raises(TypeError):
        dsa.indexer_scores(q, w, k, ctx, qs, ks, out=out)
    if bad != "out":
        with pytest.raises(TypeError):
            dsa.indexer_topk(q, w, k, ctx, 64, qs, ks)


def test_misshaped_stack_layer_is_rejected():
    B, H, D, L, k, Hq = 2, 8, 64, 600, 64, 16
    def layer(hq):
        return dict(q_idx=torch.zeros((B, 1, H, D), dtype=torch.bfloat16, device=DEV),
                    w=torch.zeros((B, 1, H), dtype=torch.float32, device=DEV),
                    k_idx=torch.zeros((B, L, D), dtype=torch.bfloat16, device=DEV),
                    q=torch.zeros((B, 1, hq, 576), dtype=torch.bfloat16, device=DEV),
                    kv=torch.zeros((B, L, 576), dtype=torch.bfloat16, device=DEV),
                    out=torch.empty((B, 1, Hq, 512), dtype=torch.bfloat16, device=DEV))
    ctx = torch.full((B,), L, dtype=torch.int32, device=DEV)
    layers = [layer(Hq), layer(Hq // 2)]
    with pytest.raises(TypeError):
        dsa.Stack("FS", layers, ctx, B=B, T=1, H=H, D=D, Lmax=L, k=k, Hq=Hq)
