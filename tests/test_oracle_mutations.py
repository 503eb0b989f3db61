"""Plant plausible mistakes in a private copy of the oracle; the pins must catch each (CPU)."""
import importlib.util
import math
import os

import numpy as np
import pytest

from tests import oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "dsa_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("oracle_mutant", SRC)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _indexer_row(relu=True, w_inside=False, mask_shift=0, drop_w=False):
    def f(q_bt, w_bt, k_b, pos, Lmax):
        out = np.full(Lmax, -np.inf)
        n = int(min(pos + 1 + mask_shift, Lmax))
        if n <= 0:
            return out
        dots = np.asarray(q_bt, np.float64) @ np.asarray(k_b[:n], np.float64).T
        w = np.ones_like(w_bt) if drop_w else np.asarray(w_bt, np.float64)
        if w_inside:
            out[:n] = np.maximum(w[:, None] * dots, 0.0).sum(0)
        else:
            out[:n] = w @ (np.maximum(dots, 0.0) if relu else dots)
        return out
    return f


def _e4m3(bias=7, sub_exp=-6):
    def f(bits):
        b = np.asarray(bits).astype(np.int64) & 0xFF
        sign = np.where((b & 0x80) != 0, -1.0, 1.0)
        e = (b >> 3) & 0xF
        m = (b & 0x7).astype(np.float64)
        mag = np.where(e == 0, (m / 8) * 2.0 ** sub_exp, (1 + m / 8) * np.exp2((e - bias).astype(float)))
        return np.where((e == 15) & (m == 7), np.nan, sign * mag)
    return f


def _topk(tie_high=False, descending=False, vis_shift=0):
    def f(scores_row, n_visible, k):
        n = int(max(0, min(n_visible + vis_shift, scores_row.shape[0])))
        out = np.full(k, -1, dtype=np.int32)
        if n == 0:
            return out
        s = np.asarray(scores_row[:n], np.float64)
        pos = -np.arange(n) if tie_high else np.arange(n)
        order = np.lexsort((pos, -s))
        take = np.sort(order[:min(k, n)])
        if descending:
            take = take[::-1]
        out[:take.shape[0]] = take
        return out
    return f


def _attend(no_scale=False, no_max_in_lse=False, value_slice_end=False):
    def f(q_h, rows, scale, d_v):
        Hq = q_h.shape[0]
        if rows.shape[0] == 0:
            return np.zeros((Hq, d_v)), np.full(Hq, -np.inf)
        logits = (1.0 if no_scale else scale) * (q_h @ rows.T)
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        z = p.sum(axis=1, keepdims=True)
        vals = rows[:, -d_v:] if value_slice_end else rows[:, :d_v]
        out = (p @ vals) / z
        lse = np.log(z)[:, 0] if no_max_in_lse else (m + np.log(z))[:, 0]
        return out, lse
    return f


def _sparse_attn_no_filter(o):
    def f(q, kv, idx, ctx_len, scale, d_v, rows=None):
        q = np.asarray(q, np.float64)
        B, T, Hq, _ = q.shape
        outs, lses = [], []
        for b in range(B):
            for t in range(T):
                sel = np.asarray(idx[b, t], dtype=np.int64)
                sel = sel[sel < kv.shape[1]]          # -1 now wraps to the last row
                oo, ll = o._softmax_attend(q[b, t], kv[b, sel], scale, d_v)
                outs.append(oo); lses.append(ll)
        return np.stack(outs).reshape(B, T, Hq, d_v), np.stack(lses).reshape(B, T, Hq)
    return f


def _stack_reuse_first_f(o):
    orig = o.run_stack

    def f(pattern, layers, ctx_len, k, scale, d_v, attend=True):
        res = orig(pattern, layers, ctx_len, k, scale, d_v, attend)
        first = res["idx"][0]
        res["idx"] = [first if c == "S" else i for c, i in zip(pattern, res["idx"])]
        if attend:
            res["out"] = [o.sparse_attn(layers[l]["q"], layers[l]["kv"], res["idx"][l], ctx_len,
                                        scale, d_v)[0] for l in range(len(pattern))]
        return res
    return f


def _bf16_truncate(o):
    def f(x):
        u = np.asarray(x, dtype=np.float32).view(np.uint32)
        return (u >> np.uint32(16)).astype(np.uint16)
    return f


def _e4m3_encode(o, half_up=False, normal_from=2.0 ** -6):
    def f(x):
        x = np.asarray(x, dtype=np.float32).astype(np.float64)
        if np.any(np.abs(x) >= 464.0):
            raise ValueError("out of range")
        rnd = (lambda v: np.floor(v + 0.5)) if half_up else np.rint
        sign = np.signbit(x).astype(np.int64)
        a = np.abs(x)
        _, ex = np.frexp(a)
        e = ex.astype(np.int64) - 1
        m = rnd((a / np.exp2(e.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
        e = np.where(m == 8, e + 1, e)
        m = np.where(m == 8, 0, m)
        normal = ((e + 7) << 3) | m
        sub = rnd(a * 2.0 ** 9).astype(np.int64)
        code = np.where(a >= normal_from, normal, sub)
        return ((sign << 7) | (code & 0x7F)).astype(np.uint8)
    return f


def _fp8_rows_scale(o, denom=447.0):
    def f(v):
        v32 = np.asarray(v, dtype=np.float32)
        amax = np.max(np.abs(v32), axis=-1)
        scale = np.where(amax > 0, amax / np.float32(denom), np.float32(1.0)).astype(np.float32)
        q = np.clip(v32 / scale[..., None], -463.0, 463.0).astype(np.float32)
        return o.e4m3fn_encode(q), scale
    return f


def _kv_append_shifted(o):
    def f(kv_cache, k_cache, k_scale, kv_new, k_new, ctx_len, fp8):
        kv_out, k_out = np.array(kv_cache, copy=True), np.array(k_cache, copy=True)
        s_out = None if k_scale is None else np.array(k_scale, copy=True)
        B, T = kv_new.shape[0], kv_new.shape[1]
        for b in range(B):
            for t in range(T):
                p = min(int(ctx_len[b]) - T + t + 1, kv_cache.shape[1] - 1)
                kv_out[b, p] = o.bf16_encode(kv_new[b, t])
                if fp8:
                    c, sc = o.quantize_fp8_rows_f32(k_new[b, t][None])
                    k_out[b, p], s_out[b, p] = c[0], sc[0]
                else:
                    k_out[b, p] = o.bf16_encode(k_new[b, t])
        return kv_out, k_out, s_out
    return f


def _greedy(o, pick_max=False, from_layer=1, tie_high=False):
    def f(C, n_shared):
        n = C.shape[0]
        pattern, trace = ["F"] * n, []
        for _ in range(n_shared):
            best, best_c = None, None
            for l in range(from_layer, n):
                if pattern[l] != "F":
                    continue
                cand = pattern.copy()
                cand[l] = "S"
                c = o.pattern_cost("".join(cand), C)
                better = best_c is None or (c > best_c if pick_max else
                                            (c <= best_c if tie_high else c < best_c))
                if better:
                    best, best_c = cand, c
            pattern = best
            trace.append(("".join(pattern), best_c))
        return trace
    return f


def _sources_previous_layer(o):
    def f(pattern):
        o.validate_pattern(pattern, len(pattern))
        return [l if c == "F" else max(l - 1, 0) for l, c in enumerate(pattern)]
    return f


def _reuse_costs_variant(o, unnormalised=False, transposed=False):
    orig = o.reuse_costs

    def f(layers, ctx_len, k, scale, d_v, proxy="output", idx_sets=None):
        if proxy != "output":
            return orig(layers, ctx_len, k, scale, d_v, proxy, idx_sets)
        n = len(layers)
        sets = [o.topk(o.indexer_scores(L["q_idx"], L["w"], L["k_idx"], ctx_len), ctx_len, k)
                for L in layers]
        C = np.zeros((n, n))
        for l in range(n):
            for j in range(l):
                a, b = (j, l) if transposed else (l, j)
                own = o.sparse_attn(layers[a]["q"], layers[a]["kv"], sets[a], ctx_len, scale, d_v)[0]
                o2 = o.sparse_attn(layers[a]["q"], layers[a]["kv"], sets[b], ctx_len, scale, d_v)[0]
                err = float(np.sum((o2 - own) ** 2))
                C[l, j] = err if unnormalised else err / float(np.sum(own ** 2))
        return C
    return f


def _overlap(o, denom="a", count_padding=False):
    def f(a, b):
        a, b = np.asarray(a).reshape(-1), np.asarray(b).reshape(-1)
        keep = (lambda x: True) if count_padding else (lambda x: x >= 0)
        sa = set(int(x) for x in a if keep(x))
        sb = set(int(x) for x in b if keep(x))
        n = {"a": len(sa), "b": len(sb), "union": len(sa | sb)}[denom]
        return math.nan if n == 0 else len(sa & sb) / n
    return f


MUTANTS = {
    "indexer_no_relu": ("indexer_scores_row", lambda o: _indexer_row(relu=False)),
    "indexer_w_inside_relu": ("indexer_scores_row", lambda o: _indexer_row(w_inside=True)),
    "indexer_mask_off_by_one": ("indexer_scores_row", lambda o: _indexer_row(mask_shift=-1)),
    "indexer_drops_w": ("indexer_scores_row", lambda o: _indexer_row(drop_w=True)),
    "e4m3_bias_8": ("e4m3fn_bits_to_f64", lambda o: _e4m3(bias=8)),
    "e4m3_subnormal_exp": ("e4m3fn_bits_to_f64", lambda o: _e4m3(sub_exp=-7)),
    "topk_ties_to_higher_pos": ("topk_row", lambda o: _topk(tie_high=True)),
    "topk_descending_output": ("topk_row", lambda o: _topk(descending=True)),
    "topk_visible_off_by_one": ("topk_row", lambda o: _topk(vis_shift=-1)),
    "attn_no_scale": ("_softmax_attend", lambda o: _attend(no_scale=True)),
    "attn_lse_without_max": ("_softmax_attend", lambda o: _attend(no_max_in_lse=True)),
    "attn_values_wrong_slice": ("_softmax_attend", lambda o: _attend(value_slice_end=True)),
    "attn_padding_not_ignored": ("sparse_attn", _sparse_attn_no_filter),
    "stack_reuses_first_f": ("run_stack", _stack_reuse_first_f),
    "bf16_encode_truncates": ("bf16_encode", _bf16_truncate),
    "e4m3_encode_ties_away": ("e4m3fn_encode", lambda o: _e4m3_encode(o, half_up=True)),
    "e4m3_encode_subnormal_edge": ("e4m3fn_encode", lambda o: _e4m3_encode(o, normal_from=2.0 ** -7)),
    "fp8_rows_scale_447": ("quantize_fp8_rows_f32", _fp8_rows_scale),
    "kv_append_row_off_by_one": ("kv_append", _kv_append_shifted),
    "greedy_picks_costliest": ("greedy_pattern_search", lambda o: _greedy(o, pick_max=True)),
    "greedy_may_share_layer0": ("greedy_pattern_search", lambda o: _greedy(o, from_layer=0)),
    "greedy_ties_to_higher_layer": ("greedy_pattern_search", lambda o: _greedy(o, tie_high=True)),
    "search_source_is_previous_layer": ("pattern_sources", _sources_previous_layer),
    "search_cost_unnormalised": ("reuse_costs", lambda o: _reuse_costs_variant(o, unnormalised=True)),
    "search_cost_transposed": ("reuse_costs", lambda o: _reuse_costs_variant(o, transposed=True)),
    "overlap_divides_by_reused_set": ("overlap_fraction", lambda o: _overlap(o, denom="b")),
    "overlap_counts_padding": ("overlap_fraction", lambda o: _overlap(o, count_padding=True)),
    "overlap_is_jaccard": ("overlap_fraction", lambda o: _overlap(o, denom="union")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches(name):
    attr, make = MUTANTS[name]
    o = fresh_oracle()
    setattr(o, attr, make(o))
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutation {name} escaped every pin"


def test_unmutated_copy_passes():
    o = fresh_oracle()
    for pin in P.ALL_PINS:
        pin(o)
    assert math.isfinite(1.0)
