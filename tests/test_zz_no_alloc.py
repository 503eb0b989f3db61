"""indexcache_run_stack_noalloc (the stack with the library's static scratch
instead of a caller's workspace) against indexcache_run_stack (GPU).

Both entry points run the same kernels on the same inputs, so every index
set, attention output and lse must be bit-identical.  Two calls in a row,
the second on a smaller stack, show that what the first left in the shared
scratch does not leak into the second; a stack too large for the scratch is
rejected before anything is launched."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import dsa_sparse_attention_lightning_amd as dsa
from dsa_sparse_attention_lightning_amd import _lib
from dsa_sparse_attention_lightning_amd import inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def build(seed, pattern, B, ctx, H, D, dtype, k, Hq):
    s = gen.Shape(seed, "noalloc", len(pattern), pattern, B=B, T=1, ctx=max(ctx), H=H, D=D,
                  idx_dtype=dtype, k=k, Hq=Hq)
    qi = gen.make_indexer_query(s, DEV)
    kb = gen.make_key_base(s, DEV)
    layers = []
    for l in range(s.n_layers):
        ki = gen.make_indexer_keys(s, l, kb, DEV)
        q, kv = gen.make_mla_layer(s, l, DEV)
        layers.append(dict(q_idx=qi.q, q_idx_scale=qi.q_scale, w=qi.w, k_idx=ki.k,
                           k_idx_scale=ki.k_scale, q=q, kv=kv,
                           out=torch.empty((B, 1, Hq, s.d_v), dtype=torch.bfloat16, device=DEV),
                           lse=torch.empty((B, 1, Hq), dtype=torch.float32, device=DEV)))
    return s, layers, gen.ctx_lens(s, DEV, ctx)


def snapshot(stack, layers):
    torch.cuda.synchronize()
    return ([L["out"].view(torch.int16).cpu().numpy().copy() for L in layers],
            [L["lse"].view(torch.int32).cpu().numpy().copy() for L in layers],
            stack.idx_buf.cpu().numpy().copy())


def scribble(layers, stack):
    for L in layers:
        L["out"].fill_(7.0)
        L["lse"].fill_(-3.0)
    stack.idx_buf.fill_(-5)


# pattern, B, ctx, H, D, dtype, k, Hq: the first has a split attention (partials
# in the scratch) and a chunked top-k (row histograms in the scratch); the
# second is smaller in every dimension.
CASES = [("FSSF", 8, [70000, 65000, 9000, 70000, 1, 300, 2049, 40000], 64, 128, "fp8", 2048,
          128),
         ("FS", 2, [3000, 2500], 16, 64, "bf16", 256, 32)]


@pytest.mark.parametrize("fused", [True, False], ids=["fused-topk", "separate-topk"])
def test_noalloc_matches_workspace_entry_point(fused):
    lib = dsa.library()
    for i, (pattern, B, ctx, H, D, dtype, k, Hq) in enumerate(CASES):
        say(f"call {i + 1}: {pattern} B={B} ctx={ctx} {dtype} k={k} Hq={Hq} fused={fused}")
        s, layers, ctx_t = build(9300 + i, pattern, B, ctx, H, D, dtype, k, Hq)
        st = dsa.Stack(pattern, layers, ctx_t, B=B, T=1, H=H, D=D, Lmax=s.Lmax, k=k, Hq=Hq,
                       idx_dtype=dtype, scale=s.scale, fused_topk=fused)
        assert 0 < st.ws_bytes <= _lib.DSA_NOALLOC_SCRATCH_BYTES
        ref_stats = st.run()
        want = snapshot(st, layers)
        scribble(layers, st)
        stats = _lib.StackStats()
        status = lib.indexcache_run_stack_noalloc(
            st.pattern, st.n_layers, st.layers, ctypes.byref(st.shape),
            ctx_t.data_ptr(), st.idx_buf.data_ptr(),
            None if st.score_buf is None else st.score_buf.data_ptr(), st.ld,
            ctypes.byref(stats), torch.cuda.current_stream().cuda_stream)
        _lib.check(status)
        got = snapshot(st, layers)
        assert (stats.n_indexer_calls, stats.n_topk_calls, stats.n_attn_calls) == (
            ref_stats["n_indexer_calls"], ref_stats["n_topk_calls"], ref_stats["n_attn_calls"])
        for l in range(len(layers)):
            assert np.array_equal(got[0][l], want[0][l]), f"layer {l} out differs"
            assert np.array_equal(got[1][l], want[1][l]), f"layer {l} lse differs"
        assert np.array_equal(got[2], want[2]), "index sets differ"
        # the binding's method is the same call
        scribble(layers, st)
        st.run_noalloc()
        again = snapshot(st, layers)
        for l in range(len(layers)):
            assert np.array_equal(again[0][l], want[0][l])
        assert np.array_equal(again[2], want[2])
        say(f"  call {i + 1} bit-identical ({len(layers)} layers, workspace {st.ws_bytes} B)")
        del st, layers


def test_noalloc_rejects_a_stack_beyond_its_scratch():
    """batch 512 x 64K context: the split partials alone exceed the scratch."""
    B, L, k, Hq = 512, 65536, 2048, 128
    s = _lib.StackShape(B, 1, 64, 128, L, k, Hq, 576, 512, _lib.DSA_FP8_E4M3, 0.07, 0)
    need = ctypes.c_size_t(0)
    lib = dsa.library()
    _lib.check(lib.indexcache_stack_workspace_size(ctypes.byref(s),
                                                   ctypes.byref(need)))
    assert need.value > _lib.DSA_NOALLOC_SCRATCH_BYTES
    # pointers are only validated (never dereferenced) before the size check fails
    fake = 1 << 20
    arr = (_lib.Layer * 1)(_lib.Layer(fake, fake, fake, fake, fake, fake, fake, fake, None))
    status = lib.indexcache_run_stack_noalloc(b"F", 1, arr, ctypes.byref(s), fake, fake, fake,
                                              L, None, None)
    assert status == _lib.DSA_ERR_WORKSPACE, lib.dsa_last_error()
    assert b"static scratch" in lib.dsa_last_error()
