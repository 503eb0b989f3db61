"""Pins that tie the fp64 oracle to facts fixed outside itself.

Every check takes the oracle module as an argument and raises AssertionError
on failure, so the same checks can be run against the real oracle (they must
pass) and against copies with a planted mistake (at least one must fail).
None of them re-types the oracle's formula: each compares against a closed
form, a brute-force enumeration, an independent library routine (torch fp64),
the number-format definition as decoded by torch, or an invariant.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch

RNG = np.random.default_rng


# ---------------------------------------------------------------- formats

def pin_e4m3_table(o):
    codes = np.arange(256, dtype=np.uint8)
    mine = o.e4m3fn_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(mine[fin], ref[fin])
    assert np.array_equal(np.signbit(mine[fin]), np.signbit(ref[fin]))


def pin_e4m3_values(o):
    # OCP E4M3: bias 7, max 448, min normal 2^-6, min subnormal 2^-9, 0x7F NaN.
    want = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0xB8: -1.0,
            0x40: 2.0, 0x3C: 1.5, 0x07: 7 * 2.0 ** -9, 0xFE: -448.0}
    got = o.e4m3fn_bits_to_f64(np.array(list(want), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(want.values())))
    assert np.isnan(o.e4m3fn_bits_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()


def pin_bf16_table(o):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = o.bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(mine[fin], ref[fin])


# ---------------------------------------------------------------- indexer

def pin_indexer_closed_form(o):
    r = RNG(1)
    L, D = 37, 8
    k = r.standard_normal((1, L, D))
    for j in range(D):
        q = np.zeros((1, 1, 1, D)); q[0, 0, 0, j] = 1.0
        s = o.indexer_scores(q, np.ones((1, 1, 1)), k, [L])
        assert np.array_equal(s[0, 0], np.maximum(k[0, :, j], 0.0))
    # two heads with weights of both signs: 2*relu(k[:,0]) - relu(k[:,1])
    q = np.zeros((1, 1, 2, D)); q[0, 0, 0, 0] = 1.0; q[0, 0, 1, 1] = 1.0
    w = np.array([[[2.0, -1.0]]])
    s = o.indexer_scores(q, w, k, [L])
    assert np.allclose(s[0, 0], 2 * np.maximum(k[0, :, 0], 0) - np.maximum(k[0, :, 1], 0),
                       rtol=0, atol=1e-15)


def pin_indexer_bruteforce(o):
    r = RNG(2)
    B, T, H, D, Lmax = 2, 3, 3, 4, 7
    q = r.standard_normal((B, T, H, D)); w = r.uniform(-1, 1, (B, T, H))
    k = r.standard_normal((B, Lmax, D)); ctx = [7, 5]
    s = o.indexer_scores(q, w, k, ctx)
    for b in range(B):
        for t in range(T):
            pos = ctx[b] - T + t
            for j in range(Lmax):
                if j > pos:
                    assert s[b, t, j] == -math.inf
                    continue
                acc = 0.0
                for h in range(H):
                    dot = math.fsum(q[b, t, h, d] * k[b, j, d] for d in range(D))
                    acc += w[b, t, h] * (dot if dot > 0 else 0.0)
                assert abs(s[b, t, j] - acc) <= 1e-12 * (1 + abs(acc))


def pin_indexer_library(o):
    r = RNG(3)
    B, T, H, D, L = 2, 4, 5, 16, 40
    q = r.standard_normal((B, T, H, D)); w = r.uniform(0, 1, (B, T, H))
    k = r.standard_normal((B, L, D)); ctx = [40, 33]
    s = o.indexer_scores(q, w, k, ctx)
    tq, tw, tk = (torch.from_numpy(x) for x in (q, w, k))
    ref = torch.einsum("bth,bths->bts", tw, torch.relu(torch.einsum("bthd,bsd->bths", tq, tk)))
    pos = torch.tensor(ctx)[:, None] - T + torch.arange(T)[None, :]
    mask = torch.arange(L)[None, None, :] > pos[:, :, None]
    ref = ref.masked_fill(mask, -math.inf).numpy()
    assert np.allclose(s, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isinf(s), np.isinf(ref))


def pin_indexer_invariants(o):
    r = RNG(4)
    B, T, H, D, L = 1, 2, 6, 8, 25
    q = r.standard_normal((B, T, H, D)); k = r.standard_normal((B, L, D))
    w1 = r.uniform(-1, 1, (B, T, H)); w2 = r.uniform(-1, 1, (B, T, H))
    ctx = [L]
    vis = np.isfinite(o.indexer_scores(q, w1, k, ctx))
    s1 = o.indexer_scores(q, w1, k, ctx)[vis]
    s2 = o.indexer_scores(q, w2, k, ctx)[vis]
    s12 = o.indexer_scores(q, w1 + w2, k, ctx)[vis]
    assert np.allclose(s12, s1 + s2, atol=1e-12)                    # linear in w
    assert np.allclose(o.indexer_scores(2.5 * q, w1, k, ctx)[vis], 2.5 * s1, atol=1e-12)
    # all dot products negative -> every visible score is exactly 0
    kpos = np.abs(k); qneg = -np.abs(q)
    s0 = o.indexer_scores(qneg, np.abs(w1), kpos, ctx)
    assert np.all(s0[np.isfinite(s0)] == 0.0)
    # causal: row t sees exactly pos+1 keys
    assert vis[0, 0].sum() == L - 1 and vis[0, 1].sum() == L


def pin_indexer_fp8_fold(o):
    """Block-scaled fp8 inputs: scores must equal s_k * sum_h (w*s_q) relu(q8.k8),
    with q8, k8 decoded by torch (the fold every fp8 kernel relies on)."""
    r = RNG(5)
    B, T, H, D, L = 1, 1, 4, 128, 50
    qf = torch.from_numpy(r.standard_normal((B, T, H, D)).astype(np.float32))
    kf = torch.from_numpy(r.standard_normal((B, L, D)).astype(np.float32))
    sq = qf.abs().amax(-1) / 448; sk = kf.abs().amax(-1) / 448
    q8 = (qf / sq[..., None]).to(torch.float8_e4m3fn)
    k8 = (kf / sk[..., None]).to(torch.float8_e4m3fn)
    w = r.uniform(0, 1, (B, T, H))
    qd = o.dequant_fp8_rows(q8.view(torch.uint8).numpy(), sq.numpy())
    kd = o.dequant_fp8_rows(k8.view(torch.uint8).numpy(), sk.numpy())
    s = o.indexer_scores(qd, w, kd, [L])[0, 0]
    dots = q8.to(torch.float64)[0, 0] @ k8.to(torch.float64)[0].T          # [H, L]
    ref = sk.double()[0] * ((torch.from_numpy(w[0, 0]) * sq.double()[0, 0]) @ torch.relu(dots))
    assert np.allclose(s, ref.numpy(), rtol=1e-12, atol=0)


# ---------------------------------------------------------------- top-k

def pin_topk_bruteforce(o):
    r = RNG(6)
    for _ in range(300):
        n = int(r.integers(1, 10)); k = int(r.integers(1, 6))
        row = r.integers(-3, 4, size=n).astype(np.float64)     # many ties
        nv = int(r.integers(1, n + 1))
        got = o.topk_row(row, nv, k)
        want = o.topk_row_bruteforce(row, nv, k)
        assert np.array_equal(got, want), (row, nv, k, got, want)


def pin_topk_library(o):
    r = RNG(7)
    for _ in range(20):
        n = int(r.integers(50, 400)); k = int(r.integers(1, 60))
        row = r.permutation(n).astype(np.float64) + r.uniform(0, 0.5, n)   # distinct
        got = o.topk_row(row, n, k)
        ref = torch.topk(torch.from_numpy(row), min(k, n)).indices.sort().values.numpy()
        assert np.array_equal(got[:min(k, n)], ref)
        assert np.all(got[min(k, n):] == -1)


def pin_topk_special(o):
    assert np.array_equal(o.topk_row(np.full(20, 3.0), 20, 5), np.arange(5))
    assert np.array_equal(o.topk_row(np.arange(6.0), 6, 9), [0, 1, 2, 3, 4, 5, -1, -1, -1])
    row = np.array([5.0, 1.0, 9.0, -np.inf, 100.0])       # position 4 not visible
    assert np.array_equal(o.topk_row(row, 3, 2), [0, 2])
    z = np.array([-0.0, 0.0, -0.0, 0.0])                   # -0 == +0: lower position wins
    assert np.array_equal(o.topk_row(z, 4, 2), [0, 1])
    got = o.topk_row(np.array([1.0, 7.0, 3.0, 7.0, 2.0]), 5, 3)
    assert np.array_equal(got, [1, 2, 3])                  # ascending order


# ---------------------------------------------------------------- attention

def _attn_case(r, B=2, T=2, Hq=3, L=19, dqk=24, dv=16):
    q = r.standard_normal((B, T, Hq, dqk)); kv = r.standard_normal((B, L, dqk))
    return q, kv


def pin_attn_dense_equiv(o):
    r = RNG(8)
    q, kv = _attn_case(r)
    B, T, Hq, dqk = q.shape; L = kv.shape[1]; dv = 16; scale = 0.37
    ctx = [19, 14]
    pos = np.asarray(ctx)[:, None] - T + np.arange(T)[None, :]
    kk = L + 3
    idx = np.full((B, T, kk), -1, np.int64)
    for b in range(B):
        for t in range(T):
            idx[b, t, :pos[b, t] + 1] = np.arange(pos[b, t] + 1)
    so, sl = o.sparse_attn(q, kv, idx, ctx, scale, dv)
    do, dl = o.dense_attn(q, kv, ctx, scale, dv)
    assert np.allclose(so, do, atol=1e-13) and np.allclose(sl, dl, atol=1e-13)
    for b in range(B):   # library: torch SDPA in fp64 with an explicit causal mask
        tq = torch.from_numpy(q[b]).transpose(0, 1)                  # [Hq, T, dqk]
        tk = torch.from_numpy(kv[b, :ctx[b]])[None].expand(Hq, -1, -1)
        tv = torch.from_numpy(kv[b, :ctx[b], :dv])[None].expand(Hq, -1, -1)
        mask = torch.arange(ctx[b])[None, :] <= torch.from_numpy(pos[b])[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                               scale=scale)
        assert np.allclose(so[b], ref.transpose(0, 1).numpy(), atol=1e-12)
        lref = torch.logsumexp((scale * tq @ tk.transpose(1, 2)).masked_fill(~mask, -math.inf), -1)
        assert np.allclose(sl[b], lref.transpose(0, 1).numpy(), atol=1e-12)


def pin_attn_single_row(o):
    r = RNG(9)
    q, kv = _attn_case(r, B=1, T=1)
    idx = np.array([[[-1, 7, -1, -1]]])
    out, lse = o.sparse_attn(q, kv, idx, [19], 0.5, 16)
    assert np.array_equal(out[0, 0], np.broadcast_to(kv[0, 7, :16], out[0, 0].shape))
    assert np.allclose(lse[0, 0], 0.5 * q[0, 0] @ kv[0, 7], atol=1e-13)


def pin_attn_zero_query(o):
    r = RNG(10)
    q, kv = _attn_case(r, B=1, T=1)
    q[:] = 0.0
    sel = [3, 11, 4, 18, 0]
    out, lse = o.sparse_attn(q, kv, np.array([[sel]]), [19], 0.9, 16)
    assert np.allclose(out[0, 0], kv[0, sel, :16].mean(0), atol=1e-14)
    assert np.allclose(lse, math.log(len(sel)), atol=1e-14)


def pin_attn_perm_and_padding(o):
    r = RNG(11)
    q, kv = _attn_case(r, B=1, T=1)
    a = np.array([[[2, 9, 5, 17, 1, 12]]])
    b = np.array([[[17, -1, 12, 1, 2, -1, 5, 9, 400, -7]]])   # shuffled, padded, out of range
    oa, la = o.sparse_attn(q, kv, a, [19], 0.3, 16)
    ob, lb = o.sparse_attn(q, kv, b, [19], 0.3, 16)
    assert np.allclose(oa, ob, atol=1e-14) and np.allclose(la, lb, atol=1e-14)
    oz, lz = o.sparse_attn(q, kv, np.full((1, 1, 4), -1), [19], 0.3, 16)
    assert np.all(oz == 0) and np.all(lz == -np.inf)


def pin_attn_bruteforce(o):
    r = RNG(12)
    Hq, dqk, dv, L = 2, 6, 4, 9
    q = r.standard_normal((1, 1, Hq, dqk)); kv = r.standard_normal((1, L, dqk))
    sel = [0, 4, 8, 2]
    out, lse = o.sparse_attn(q, kv, np.array([[sel]]), [L], 0.7, dv)
    for h in range(Hq):
        logit = [0.7 * math.fsum(q[0, 0, h, d] * kv[0, j, d] for d in range(dqk)) for j in sel]
        z = math.fsum(math.exp(x) for x in logit)
        for c in range(dv):
            want = math.fsum(math.exp(x) / z * kv[0, j, c] for x, j in zip(logit, sel))
            assert abs(out[0, 0, h, c] - want) < 1e-13
        assert abs(lse[0, 0, h] - math.log(z)) < 1e-13


# ---------------------------------------------------------------- stack

def _stack_layers(r, n_layers, B=2, T=1, H=3, D=8, L=30, Hq=2, dqk=12, shared_keys=False):
    q_idx = r.standard_normal((B, T, H, D)); w = r.uniform(0, 1, (B, T, H))
    base = r.standard_normal((B, L, D))
    layers = []
    for _ in range(n_layers):
        k_idx = base if shared_keys else 0.95 * base + 0.31 * r.standard_normal((B, L, D))
        layers.append(dict(q_idx=q_idx, w=w, k_idx=k_idx,
                           q=r.standard_normal((B, T, Hq, dqk)),
                           kv=r.standard_normal((B, L, dqk))))
    return layers


def pin_stack_semantics(o):
    r = RNG(13)
    pat = "FSSFSF"
    layers = _stack_layers(r, len(pat))
    ctx, k = [30, 21], 6
    res = o.run_stack(pat, layers, ctx, k, 0.4, 8)
    assert res["n_indexer_calls"] == pat.count("F")
    for l, c in enumerate(pat):
        own = o.topk_row  # the layer's own selection, computed through the brute-force definition
        for b in range(2):
            s = o.indexer_scores(layers[l]["q_idx"], layers[l]["w"], layers[l]["k_idx"], ctx)[b, 0]
            if c == "F":
                want = o.topk_row_bruteforce(s, ctx[b], k) if ctx[b] <= 12 else own(s, ctx[b], k)
                assert np.array_equal(res["idx"][l][b, 0], want)
        if c == "S":
            f = max(i for i in range(l) if pat[i] == "F")
            assert res["idx"][l].tobytes() == res["idx"][f].tobytes()
    allf = o.run_stack("F" * len(pat), layers, ctx, k, 0.4, 8)
    for l in range(len(pat)):            # F layers agree with the all-F run
        if pat[l] == "F":
            assert np.array_equal(allf["idx"][l], res["idx"][l])
            assert np.array_equal(allf["out"][l], res["out"][l])


def pin_stack_identical_keys(o):
    r = RNG(14)
    layers = _stack_layers(r, 8, shared_keys=True)
    base = o.run_stack("F" * 8, layers, [30, 25], 5, 0.4, 8)
    for p in ("FSSSFSSS", "FSFSFSFS", "FSSSSSSS"):
        res = o.run_stack(p, layers, [30, 25], 5, 0.4, 8)
        for l in range(8):
            assert np.array_equal(res["out"][l], base["out"][l])


def pin_stack_counts(o, cases):
    for c in cases:
        n = c["n_layers"]
        pat = (c["group"] * n)[:n]
        r = RNG(15)
        layers = _stack_layers(r, n, B=1, L=12, H=2, D=4, Hq=1, dqk=4)
        res = o.run_stack(pat, layers, [12], 3, 1.0, 2, attend=False)
        assert res["n_indexer_calls"] == c["expected_indexer_calls"]


# ---------------------------------------------------------------- cache append

def _finite_e4m3_values():
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = ~np.isnan(vals)
    return codes[fin], vals[fin]


def pin_e4m3_encode_roundtrip(o):
    # every finite code is reproduced from its own value (both zeros included)
    codes, vals = _finite_e4m3_values()
    got = o.e4m3fn_encode(vals.astype(np.float32))
    assert np.array_equal(got, codes)


def pin_e4m3_encode_bruteforce(o):
    # nearest code by exhaustive search over the 254 finite codes; a tie goes
    # to the code with the even mantissa (last bit 0)
    codes, vals = _finite_e4m3_values()
    r = RNG(11)
    x = np.concatenate([r.uniform(-460, 460, 3000), r.normal(0, 1, 3000),
                        r.normal(0, 2.0 ** -7, 2000),
                        (vals[:, None] + vals[None, :]).ravel()[:: 7] / 2.0]).astype(np.float32)
    x = x[np.abs(x.astype(np.float64)) < 464.0]
    got = o.e4m3fn_encode(x)
    xv = x.astype(np.float64)
    for xi, gi in zip(xv, got):
        d = np.abs(vals - xi)
        best = np.flatnonzero(d == d.min())
        best = best[np.signbit(vals[best]) == np.signbit(xi)] if len(best) > 1 else best
        if len(best) > 1:
            best = best[(codes[best] & 1) == 0]
        assert codes[best[0]] == gi, (xi, hex(codes[best[0]]), hex(gi))


def pin_e4m3_encode_library(o):
    # torch's float32 -> float8_e4m3fn conversion rounds to nearest even
    r = RNG(12)
    x = np.concatenate([r.uniform(-448, 448, 20000), r.normal(0, 3, 20000)]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(o.e4m3fn_encode(x), ref)


def pin_bf16_encode_library(o):
    r = RNG(13)
    x = np.concatenate([r.normal(0, 1, 50000), r.uniform(-1e4, 1e4, 50000)]).astype(np.float32)
    # exact ties: a float32 whose dropped 16 bits are exactly 0x8000
    base = r.normal(0, 100, 2000).astype(np.float32).view(np.uint32)
    ties = (base & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.bf16_encode(x), ref)


def pin_fp8_row_quantisation(o):
    r = RNG(14)
    v = r.normal(0, 2, (40, 128)).astype(np.float32)
    v[3] = 0.0
    codes, scale = o.quantize_fp8_rows_f32(v)
    dec = o.e4m3fn_bits_to_f64(codes)
    # the largest magnitude of each non-zero row maps to the largest code
    amax_col = np.argmax(np.abs(v), axis=1)
    nz = np.abs(v).max(axis=1) > 0
    assert np.all(np.abs(dec[np.arange(40), amax_col])[nz] == 448.0)
    assert scale[3] == 1.0 and np.all(codes[3] == 0)
    # reconstruction within half a step of the format (relative 2^-4 for
    # normals, absolute 2^-10 * scale for subnormals)
    err = np.abs(dec * scale[:, None] - v.astype(np.float64))
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)


def pin_kv_append(o):
    r = RNG(15)
    B, T, L, dqk, D = 3, 4, 20, 12, 8
    ctx = [20, 9, 4]
    kv = r.integers(0, 1 << 16, (B, L, dqk), dtype=np.uint32).astype(np.uint16)
    k8 = r.integers(0, 256, (B, L, D), dtype=np.uint32).astype(np.uint8)
    ks = r.uniform(0.1, 1, (B, L)).astype(np.float32)
    kv_new = r.normal(0, 1, (B, T, dqk)).astype(np.float32)
    k_new = r.normal(0, 1, (B, T, D)).astype(np.float32)
    kv2, k2, s2 = o.kv_append(kv, k8, ks, kv_new, k_new, ctx, True)
    for b in range(B):
        written = set(range(ctx[b] - T, ctx[b]))
        for p in range(L):
            if p in written:
                t = p - (ctx[b] - T)
                assert np.array_equal(kv2[b, p], torch.from_numpy(kv_new[b, t]).to(
                    torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
                ref = torch.from_numpy(k_new[b, t] / s2[b, p]).to(torch.float8_e4m3fn)
                assert np.array_equal(k2[b, p], ref.view(torch.uint8).numpy())
                assert s2[b, p] == np.float32(np.abs(k_new[b, t]).max() / np.float32(448.0))
            else:   # nothing else moves
                assert np.array_equal(kv2[b, p], kv[b, p]) and np.array_equal(k2[b, p], k8[b, p])
                assert s2[b, p] == ks[b, p]
    kb = r.integers(0, 1 << 16, (B, L, D), dtype=np.uint32).astype(np.uint16)
    _, kb2, none = o.kv_append(kv, kb, None, kv_new, k_new, ctx, False)
    assert none is None
    for b in range(B):
        p0 = ctx[b] - T
        assert np.array_equal(kb2[b, p0:ctx[b]], torch.from_numpy(k_new[b]).to(
            torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


# ---------------------------------------------------------------- pattern search

def _direct_pattern_cost(o, pattern, layers, ctx, k, scale, d_v, proxy):
    """A pattern's proxy loss measured the long way: run the stack with the
    pattern and with all-F and compare layer by layer."""
    n = len(pattern)
    run = o.run_stack(pattern, layers, ctx, k, scale, d_v)
    ref = o.run_stack("F" * n, layers, ctx, k, scale, d_v)
    total = 0.0
    for l in range(n):
        if proxy == "output":
            d = math.fsum(((run["out"][l] - ref["out"][l]) ** 2).ravel())
            z = math.fsum((ref["out"][l] ** 2).ravel())
            total += d / z
        else:
            a = run["idx"][l].reshape(-1, k)
            b = ref["idx"][l].reshape(-1, k)
            hit = sum(np.intersect1d(a[i][a[i] >= 0], b[i][b[i] >= 0]).size
                      for i in range(a.shape[0]))
            total += 1.0 - hit / int((b >= 0).sum())
    return total


def pin_search_cost_decomposition(o):
    """reuse_costs + pattern_cost equal the whole-stack difference against
    all-F for every pattern of a 5-layer stack, for both proxies."""
    r = RNG(21)
    layers = _stack_layers(r, 5, B=2, T=2, L=24, H=3, D=6, Hq=2, dqk=10)
    ctx, k, scale, dv = [24, 17], 5, 0.5, 6
    for proxy in ("output", "miss"):
        C = o.reuse_costs(layers, ctx, k, scale, dv, proxy)
        assert np.all(C[np.triu_indices(5)] == 0)
        for bits in itertools.product("FS", repeat=4):
            p = "F" + "".join(bits)
            want = _direct_pattern_cost(o, p, layers, ctx, k, scale, dv, proxy)
            got = o.pattern_cost(p, C)
            assert abs(got - want) <= 1e-12 * max(1.0, abs(want)), (proxy, p, got, want)


def pin_search_hand_trace(o):
    """A 4-layer cost matrix worked by hand.  Step 1: S at 1, 2, 3 costs 0.5,
    0.1, 0.2 -> FFSF.  Step 2: S at 1 makes layers 1 and 2 reuse layer 0
    (0.5 + 0.9); S at 3 makes layer 3 reuse layer 1 (0.1 + 0.7) -> FFSS, 0.8.
    Step 3: FSSS = 0.5 + 0.9 + 0.8."""
    C = np.zeros((4, 4))
    C[1, 0] = 0.5
    C[2, 0], C[2, 1] = 0.9, 0.1
    C[3, 0], C[3, 1], C[3, 2] = 0.8, 0.7, 0.2
    trace = o.greedy_pattern_search(C, 3)
    assert [p for p, _ in trace] == ["FFSF", "FFSS", "FSSS"]
    for (_, c), want in zip(trace, (0.1, 0.8, 2.2)):
        assert abs(c - want) <= 1e-12
    assert o.pattern_sources("FSSFSF") == [0, 0, 0, 3, 3, 5]


def pin_search_row_constant(o):
    """If reusing any earlier set costs layer l the same c_l, a pattern costs
    the sum of c over its S layers, so greedy takes the layers in increasing
    order of c_l (closed form: a sort), never layer 0."""
    r = RNG(22)
    n = 9
    c = r.permutation(np.linspace(0.1, 2.0, n))
    C = np.zeros((n, n))
    for l in range(n):
        C[l, :l] = c[l]
    trace = o.greedy_pattern_search(C, n - 1)
    order = [int(i) for i in np.argsort(c[1:]) + 1]
    for m, (p, cost) in enumerate(trace, start=1):
        assert p[0] == "F"
        assert {i for i, ch in enumerate(p) if ch == "S"} == set(order[:m])
        assert abs(cost - math.fsum(c[order[:m]])) <= 1e-12


def pin_search_bruteforce(o):
    """Against every pattern of a 7-layer stack with a random cost matrix:
    one step of greedy reaches the best single conversion (lowest layer on
    ties), later steps are never better than the best pattern with as many
    S layers, and each step flips exactly one F layer (never layer 0)."""
    r = RNG(23)
    n = 7
    C = np.tril(r.uniform(0, 1, (n, n)), -1)

    def cost(p):
        tot, src = 0.0, 0
        for l, ch in enumerate(p):
            src = l if ch == "F" else src
            tot += C[l, src]
        return tot

    pats = ["F" + "".join(b) for b in itertools.product("FS", repeat=n - 1)]
    trace = o.greedy_pattern_search(C, n - 1)
    prev = "F" * n
    for m, (p, c) in enumerate(trace, start=1):
        best = min(cost(q) for q in pats if q.count("S") == m)
        assert c >= best - 1e-12 and abs(c - cost(p)) <= 1e-12
        if m == 1:
            first = min((q for q in pats if q.count("S") == 1), key=lambda q: (cost(q), q.index("S")))
            assert p == first
        flips = [i for i in range(n) if prev[i] != p[i]]
        assert len(flips) == 1 and prev[flips[0]] == "F" and flips[0] > 0
        prev = p


def pin_search_identical_keys(o):
    """Layers sharing one key cache select the same sets: every reuse costs 0
    under both proxies and greedy converts layers 1, 2, ... in order."""
    r = RNG(24)
    layers = _stack_layers(r, 5, shared_keys=True)
    for proxy in ("output", "miss"):
        C = o.reuse_costs(layers, [30, 26], 5, 0.4, 8, proxy)
        assert np.all(C == 0)
        trace = o.greedy_pattern_search(C, 4)
        assert [p for p, _ in trace] == ["FSFFF", "FSSFF", "FSSSF", "FSSSS"]


# ---------------------------------------------------------------- overlap

def pin_overlap_hand_worked(o):
    """A = {3, 7, 9}, B = {1, 3, 9, 11}, both padded with -1: A and B share
    {3, 9}, so 2 of A's 3 positions are kept (2/3) and 2 of B's 4 (1/2).
    A set with nothing selected has no overlap to report (nan); an empty B
    keeps nothing (0); a set against itself keeps everything (1)."""
    a = np.array([3, 7, 9, -1, -1], dtype=np.int32)
    b = np.array([1, 3, 9, 11, -1], dtype=np.int32)
    assert abs(o.overlap_fraction(a, b) - 2 / 3) < 1e-15
    assert abs(o.overlap_fraction(b, a) - 1 / 2) < 1e-15
    assert abs(o.overlap_fraction(a[None, :], b[None, None, :]) - 2 / 3) < 1e-15
    none = np.full(5, -1, dtype=np.int32)
    assert math.isnan(o.overlap_fraction(none, b))
    assert o.overlap_fraction(a, none) == 0.0
    assert o.overlap_fraction(a, a) == 1.0
    assert o.overlap_fraction(np.array([5, -1]), np.array([-1, 6])) == 0.0
    try:
        o.overlap_fraction(np.stack([a, a]), np.stack([b, b]))
    except ValueError:
        pass
    else:
        raise AssertionError("two rows at once must be rejected")


def pin_overlap_bruteforce(o):
    """Random ascending, -1-padded selections (as the top-k emits them):
    count A's valid entries found anywhere among B's valid entries by
    scanning, one entry at a time."""
    r = RNG(31)
    for _ in range(200):
        k = int(r.integers(1, 12))
        L = int(r.integers(k, 40))
        sets = []
        for _ in range(2):
            n = int(r.integers(0, k + 1))
            x = np.full(k, -1, dtype=np.int32)
            x[:n] = np.sort(r.choice(L, size=n, replace=False))
            sets.append(x)
        a, b = sets
        valid_a = [int(x) for x in a if x != -1]
        found = 0
        for x in valid_a:
            for y in b:
                if y != -1 and int(y) == x:
                    found += 1
                    break
        got = o.overlap_fraction(a, b)
        if not valid_a:
            assert math.isnan(got)
        else:
            assert got == found / len(valid_a), (a, b, got)


ALL_PINS = [
    pin_e4m3_table, pin_e4m3_values, pin_bf16_table,
    pin_indexer_closed_form, pin_indexer_bruteforce, pin_indexer_library,
    pin_indexer_invariants, pin_indexer_fp8_fold,
    pin_topk_bruteforce, pin_topk_library, pin_topk_special,
    pin_attn_dense_equiv, pin_attn_single_row, pin_attn_zero_query,
    pin_attn_perm_and_padding, pin_attn_bruteforce,
    pin_stack_semantics, pin_stack_identical_keys,
    pin_e4m3_encode_roundtrip, pin_e4m3_encode_bruteforce, pin_e4m3_encode_library,
    pin_bf16_encode_library, pin_fp8_row_quantisation, pin_kv_append,
    pin_search_cost_decomposition, pin_search_hand_trace, pin_search_row_constant,
    pin_search_bruteforce, pin_search_identical_keys,
    pin_overlap_hand_worked, pin_overlap_bruteforce,
]
