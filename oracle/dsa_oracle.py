"""Plain CPU fp64 oracle for the IndexCache / DeepSeek-Sparse-Attention hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in the root
entry module and the cpu_baseline leg of the benchmark may import, call or run
anything in this package.  The product path (the HIP library and its Python
binding) never does, and shares no code with it: no kernels, headers, helpers,
tables or pre/post-processing.  Inputs arrive as raw codes (bf16 / fp8 bit
patterns) plus fp32 scales, exactly the bytes the GPU reads, and are decoded
here from the number formats' own definitions.

What is computed (sources are the web pages on "IndexCache: Accelerating Sparse
Attention via Cross-Layer Index Reuse", gist.science es/pt/it/de editions):

* indexer_scores  - the lightning indexer of DSA scores every previous token for
  each query (technical summary §1 on every gist.science edition).  The pages
  print no formula; the DSA lightning-indexer form is used:
  I[b,t,s] = sum_h w[b,t,h] * max(0, sum_d q[b,t,h,d] * k[b,s,d]) for s <= pos,
  -inf otherwise.
* topk            - the k most relevant previous tokens per query (technical
  summary §1).  Ties go to the lower position; the selected positions are
  returned in ascending order and padded with -1.
* sparse_attn     - core attention restricted to the selected tokens, O(Lk)
  (technical summary §1).  Absorbed-MLA form: one shared latent row of width
  d_qk per token serves every head; logits use all d_qk columns, values the
  first d_v columns.  Dense softmax over the valid selected rows.
* dense_attn      - full causal attention, O(L^2): the baseline DSA replaces
  (technical summary §1); used only as a test pin.
* kv_append       - the cache write that precedes the path in every step:
  each new token's latent row and indexer key row are stored at its position
  (pos = ctx_len[b] - T + t).  New rows arrive in fp32 and are encoded into
  the cache's format: bfloat16 with round-to-nearest-even for the latent cache
  and a bf16 key cache; for an fp8 key cache, one scale per row,
  scale = amax / 448 (1 if the row is zero), and every value / scale rounded
  to the nearest OCP E4M3FN code (ties to even).  The scale and the quotients
  are fp32 operations, the precision the device uses, so that both sides take
  the same code decisions.  The pages only say that the indices are computed
  from the cached keys; the fp8 block format follows the fp8 workload
  description the decode benchmark is quoted on.
* reuse_costs, pattern_cost, greedy_pattern_search - the training-free
  pattern search (technical summary §2, part A of "Dos Enfoques de
  Configuración" on the es edition, "Duas Abordagens de Otimização" on pt and
  "Due Approcci di Configurazione" on it, "A. Training-Free IndexCache" under
  "Methodik" on de): start from all layers F and convert one
  layer at a time to S, each time the layer whose conversion raises the loss
  least.  The pages measure the loss as LM loss on a calibration set; without
  a trained model a PROXY stands in for it: the cost of a pattern is the sum,
  over layers, of what layer l loses by attending with the index set of its
  source layer (the nearest preceding F layer) instead of its own, either the
  relative squared error of its attention output ("output") or the fraction
  of its own selected positions missing from the reused set ("miss").  The
  layers of the synthetic stack take independent inputs, so this sum is the
  whole-stack difference against all-F, layer by layer.
* overlap_fraction - the measured statistic the pages quote for adjacent
  layers (technical summary §1 on the pt/it/de editions: their top-k
  selections share 70% to 100% of tokens): the share of one row's own
  selection that another layer's set for the same row also holds.
* run_stack       - the IndexCache layer loop: F layers run the indexer and
  top-k and store the index set; S layers skip both and reuse the set of the
  nearest preceding F layer (technical summary §2, "Arquitectura del Método" /
  "Arquitetura" / "Architettura e Funzionamento" / "Methodik"), a single
  conditional branch in the inference loop.

Query row t of sequence b sits at absolute position pos = ctx_len[b] - T + t
and sees keys 0..pos inclusive (causal).

Parity pins: every function here is pinned in tests/test_oracle_*.py against
closed forms, brute force, library routines and invariants; none is "parity
unpinned".
"""
from __future__ import annotations

import itertools
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "e4m3fn_bits_to_f64",
    "dequant_fp8_rows",
    "query_positions",
    "indexer_scores",
    "indexer_scores_row",
    "topk",
    "topk_row",
    "topk_row_bruteforce",
    "sparse_attn",
    "dense_attn",
    "run_stack",
    "validate_pattern",
    "overlap_fraction",
    "reuse_costs",
    "pattern_sources",
    "pattern_cost",
    "greedy_pattern_search",
    "bf16_encode",
    "e4m3fn_encode",
    "quantize_fp8_rows_f32",
    "kv_append",
]


# --------------------------------------------------------------------------
# Number formats (decoded from their definitions, not from any library).
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.

    bfloat16 is the upper half of an IEEE-754 binary32: sign, 8 exponent bits
    (bias 127), 7 mantissa bits.  Widening is exact."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        bits = bits.astype(np.uint16)
    u32 = bits.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # NaN payloads widen to NaN
        return u32.view(np.float32).astype(np.float64)


def e4m3fn_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 ("fn": finite, no infinities) bit patterns -> float64.

    Layout s.eeee.mmm, exponent bias 7.  e == 0: subnormal (m/8) * 2^-6.
    e == 15 and m == 7: NaN (the only non-finite code).  Otherwise
    (1 + m/8) * 2^(e-7); the largest finite magnitude is 448."""
    b = np.asarray(bits).astype(np.int64) & 0xFF
    sign = np.where((b & 0x80) != 0, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    sub = (m / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, sub, normal)
    out = sign * mag
    out = np.where((e == 15) & (m == 7.0), np.nan, out)
    return out


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    The kept value is the float32 truncated to its upper 16 bits, plus one unit
    in the last kept place when the dropped 16 bits exceed half a unit, or
    equal it and the kept part is odd.  (NaN inputs are not expected.)"""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep = u >> np.uint64(16)
    drop = u & np.uint64(0xFFFF)
    up = (drop > 0x8000) | ((drop == 0x8000) & ((keep & np.uint64(1)) == 1))
    return (keep + up.astype(np.uint64)).astype(np.uint16)


def e4m3fn_encode(x: np.ndarray) -> np.ndarray:
    """float32 values with |x| < 464 -> OCP E4M3FN codes (uint8), round to
    nearest, ties to even.

    A magnitude a >= 2^-6 has a = f * 2^(e+1) with f in [0.5, 1) (frexp, exact):
    its code keeps round((a / 2^e - 1) * 8) as the 3-bit mantissa m, and a
    carry to m = 8 moves to the next exponent.  Below 2^-6 the codes are the
    subnormals m * 2^-9, m = round(a * 2^9) (m = 8 is the smallest normal).
    The sign of x (also of -0) is kept.  Magnitudes up to 464 round to 448,
    the largest finite code (0x7E)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)   # exact widening
    sign = np.signbit(x).astype(np.int64)
    a = np.abs(x)
    if np.any(a >= 464.0) or np.any(np.isnan(a)):
        raise ValueError("e4m3fn_encode: value out of the finite range")
    f, ex = np.frexp(a)
    e = ex.astype(np.int64) - 1                     # a in [2^e, 2^(e+1))
    m = np.rint((a / np.exp2(e.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    normal_code = ((e + 7) << 3) | m
    sub_code = np.rint(a * 2.0 ** 9).astype(np.int64)  # 0..8
    code = np.where(a >= 2.0 ** -6, normal_code, sub_code)
    return ((sign << 7) | code).astype(np.uint8)


def quantize_fp8_rows_f32(v: np.ndarray):
    """Per-row fp8 quantisation in fp32 arithmetic: scale = amax / 448 (1 for
    an all-zero row), codes = e4m3fn_encode(v / scale).  Returns (codes uint8,
    scale float32)."""
    v32 = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v32), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = (v32 / scale[..., None]).astype(np.float32)
    return e4m3fn_encode(q), scale


def kv_append(kv_cache: np.ndarray, k_cache: np.ndarray, k_scale, kv_new: np.ndarray,
              k_new: np.ndarray, ctx_len: Sequence[int], fp8: bool):
    """Write T new token rows per sequence into copies of the caches.

    kv_cache [B,Lmax,d_qk] bf16 bits; k_cache [B,Lmax,D] (fp8 codes uint8 with
    k_scale [B,Lmax] float32, or bf16 bits uint16 and k_scale None); kv_new
    [B,T,d_qk] and k_new [B,T,D] float32.  Row t of sequence b goes to
    position ctx_len[b] - T + t.  Returns (kv_cache, k_cache, k_scale)."""
    kv_out = np.array(kv_cache, copy=True)
    k_out = np.array(k_cache, copy=True)
    s_out = None if k_scale is None else np.array(k_scale, copy=True)
    B, T = kv_new.shape[0], kv_new.shape[1]
    pos = query_positions(ctx_len, T)
    for b in range(B):
        for t in range(T):
            p = int(pos[b, t])
            kv_out[b, p] = bf16_encode(kv_new[b, t])
            if fp8:
                codes, sc = quantize_fp8_rows_f32(k_new[b, t][None])
                k_out[b, p] = codes[0]
                s_out[b, p] = sc[0]
            else:
                k_out[b, p] = bf16_encode(k_new[b, t])
    return kv_out, k_out, s_out


def dequant_fp8_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Per-row block dequantisation: value = decode(code) * scale, one fp32
    scale per trailing-dimension row (a 128-element block when D = 128)."""
    vals = e4m3fn_bits_to_f64(codes)
    return vals * np.asarray(scales, dtype=np.float64)[..., None]


# --------------------------------------------------------------------------
# Indexer
# --------------------------------------------------------------------------

def query_positions(ctx_len: Sequence[int], T: int) -> np.ndarray:
    """pos[b, t] = ctx_len[b] - T + t: the absolute position of query row t."""
    ctx = np.asarray(ctx_len, dtype=np.int64)
    return ctx[:, None] - T + np.arange(T, dtype=np.int64)[None, :]


def indexer_scores_row(q_bt: np.ndarray, w_bt: np.ndarray, k_b: np.ndarray,
                       pos: int, Lmax: int) -> np.ndarray:
    """Scores of one query row against keys 0..Lmax-1 (fp64).

    q_bt [H, D], w_bt [H], k_b [L, D].  Keys after pos are -inf."""
    out = np.full(Lmax, -np.inf, dtype=np.float64)
    n = int(min(pos + 1, Lmax))
    if n <= 0:
        return out
    dots = np.asarray(q_bt, np.float64) @ np.asarray(k_b[:n], np.float64).T  # [H, n]
    out[:n] = np.asarray(w_bt, np.float64) @ np.maximum(dots, 0.0)
    return out


def indexer_scores(q: np.ndarray, w: np.ndarray, k: np.ndarray,
                   ctx_len: Sequence[int], rows: Optional[Sequence] = None) -> np.ndarray:
    """Lightning-indexer scores for every query row.

    q [B, T, H, D], w [B, T, H], k [B, Lmax, D] (all already real-valued),
    ctx_len [B].  Returns [B, T, Lmax] fp64 with -inf at s > pos(b, t).
    When `rows` is a list of (b, t) pairs only those rows are computed and a
    [len(rows), Lmax] array is returned (for large shapes)."""
    q = np.asarray(q, np.float64)
    w = np.asarray(w, np.float64)
    B, T, H, D = q.shape
    Lmax = k.shape[1]
    pos = query_positions(ctx_len, T)
    if rows is not None:
        return np.stack([indexer_scores_row(q[b, t], w[b, t], k[b], int(pos[b, t]), Lmax)
                         for (b, t) in rows]) if len(rows) else np.zeros((0, Lmax))
    out = np.empty((B, T, Lmax), dtype=np.float64)
    for b in range(B):
        for t in range(T):
            out[b, t] = indexer_scores_row(q[b, t], w[b, t], k[b], int(pos[b, t]), Lmax)
    return out


# --------------------------------------------------------------------------
# Top-k
# --------------------------------------------------------------------------

def topk_row(scores_row: np.ndarray, n_visible: int, k: int) -> np.ndarray:
    """The k highest-scoring positions among 0..n_visible-1.

    Order key: higher score first, then lower position (a full stable sort on
    (-score, position)).  Returned in ascending position order, padded with -1
    when fewer than k positions are visible."""
    n = int(max(0, min(n_visible, scores_row.shape[0])))
    out = np.full(k, -1, dtype=np.int32)
    if n == 0 or k <= 0:
        return out
    s = np.asarray(scores_row[:n], dtype=np.float64)
    order = np.lexsort((np.arange(n), -s))     # last key is primary
    take = np.sort(order[:min(k, n)])
    out[:take.shape[0]] = take
    return out


def topk(scores: np.ndarray, ctx_len: Sequence[int], k: int) -> np.ndarray:
    """Row-wise top-k over [B, T, Lmax] scores -> [B, T, k] int32."""
    B, T, Lmax = scores.shape
    pos = query_positions(ctx_len, T)
    out = np.empty((B, T, k), dtype=np.int32)
    for b in range(B):
        for t in range(T):
            out[b, t] = topk_row(scores[b, t], int(pos[b, t]) + 1, k)
    return out


def topk_row_bruteforce(scores_row: Sequence[float], n_visible: int, k: int) -> np.ndarray:
    """Exhaustive definition for tiny rows: the unique subset S of size
    min(k, n) such that every member beats every non-member under the order
    (higher score, then lower position).  Enumerates all subsets."""
    n = int(n_visible)
    m = min(k, n)

    def beats(i, j):
        si, sj = float(scores_row[i]), float(scores_row[j])
        return si > sj or (si == sj and i < j)

    found = None
    for S in itertools.combinations(range(n), m):
        rest = [j for j in range(n) if j not in S]
        if all(beats(i, j) for i in S for j in rest):
            assert found is None, "selection must be unique"
            found = S
    out = np.full(k, -1, dtype=np.int32)
    out[:m] = np.array(sorted(found), dtype=np.int32) if m else []
    return out


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def _softmax_attend(q_h: np.ndarray, rows: np.ndarray, scale: float, d_v: int):
    """q_h [Hq, d_qk], rows [n, d_qk] -> (out [Hq, d_v], lse [Hq])."""
    Hq = q_h.shape[0]
    if rows.shape[0] == 0:
        return np.zeros((Hq, d_v)), np.full(Hq, -np.inf)
    logits = scale * (q_h @ rows.T)                 # [Hq, n]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    z = p.sum(axis=1, keepdims=True)
    out = (p @ rows[:, :d_v]) / z
    lse = (m + np.log(z))[:, 0]
    return out, lse


def sparse_attn(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, ctx_len: Sequence[int],
                scale: float, d_v: int, rows: Optional[Sequence] = None):
    """Sparse MLA attention over the selected latent rows.

    q [B, T, Hq, d_qk], kv [B, Lmax, d_qk], idx [B, T, k] (int; entries outside
    0..pos(b,t) - e.g. the -1 padding - are ignored).  For each (b, t, h):
    logits_j = scale * q . kv[idx_j]; p = softmax over valid j;
    out = sum_j p_j kv[idx_j, :d_v]; lse = log sum_j exp(logits_j).
    No valid j: out = 0, lse = -inf.  Returns (out [B,T,Hq,d_v], lse [B,T,Hq]),
    or stacked per-row results for `rows` = [(b, t), ...]."""
    q = np.asarray(q, np.float64)
    B, T, Hq, _ = q.shape
    pos = query_positions(ctx_len, T)
    pairs = rows if rows is not None else [(b, t) for b in range(B) for t in range(T)]
    outs, lses = [], []
    for (b, t) in pairs:
        sel = np.asarray(idx[b, t], dtype=np.int64)
        valid = sel[(sel >= 0) & (sel <= pos[b, t]) & (sel < kv.shape[1])]
        r = np.asarray(kv[b, valid], dtype=np.float64)
        o, l = _softmax_attend(q[b, t], r, scale, d_v)
        outs.append(o)
        lses.append(l)
    if rows is not None:
        return np.stack(outs), np.stack(lses)
    return (np.stack(outs).reshape(B, T, Hq, d_v), np.stack(lses).reshape(B, T, Hq))


def dense_attn(q: np.ndarray, kv: np.ndarray, ctx_len: Sequence[int], scale: float, d_v: int):
    """Full causal attention over positions 0..pos (the O(L^2) baseline)."""
    q = np.asarray(q, np.float64)
    B, T, Hq, _ = q.shape
    pos = query_positions(ctx_len, T)
    out = np.zeros((B, T, Hq, d_v))
    lse = np.zeros((B, T, Hq))
    for b in range(B):
        for t in range(T):
            n = int(min(pos[b, t] + 1, kv.shape[1]))
            o, l = _softmax_attend(q[b, t], np.asarray(kv[b, :max(n, 0)], np.float64), scale, d_v)
            out[b, t], lse[b, t] = o, l
    return out, lse


# --------------------------------------------------------------------------
# IndexCache layer stack
# --------------------------------------------------------------------------

def validate_pattern(pattern: str, n_layers: int) -> None:
    """A pattern is one 'F' or 'S' per layer; an S layer inherits from the
    nearest preceding F layer, so the first layer must be F."""
    if len(pattern) != n_layers:
        raise ValueError(f"pattern length {len(pattern)} != n_layers {n_layers}")
    if any(c not in "FS" for c in pattern):
        raise ValueError("pattern may hold only 'F' and 'S'")
    if n_layers > 0 and pattern[0] != "F":
        raise ValueError("an S layer needs a preceding F layer: pattern must start with 'F'")


def run_stack(pattern: str, layers: List[Dict[str, np.ndarray]], ctx_len: Sequence[int],
              k: int, scale: float, d_v: int, attend: bool = True):
    """The IndexCache inference loop over real-valued per-layer inputs.

    layers[l] holds 'q_idx' [B,T,H,D], 'w' [B,T,H], 'k_idx' [B,Lmax,D] (needed
    on F layers only) and 'q' [B,T,Hq,d_qk], 'kv' [B,Lmax,d_qk].
    Returns dict(out=[...], lse=[...], idx=[...] (index set each layer used),
    n_indexer_calls=#F)."""
    validate_pattern(pattern, len(layers))
    idx = None
    calls = 0
    outs, lses, used = [], [], []
    for l, kind in enumerate(pattern):
        L = layers[l]
        if kind == "F":
            s = indexer_scores(L["q_idx"], L["w"], L["k_idx"], ctx_len)
            idx = topk(s, ctx_len, k)
            calls += 1
        used.append(idx)
        if attend:
            o, z = sparse_attn(L["q"], L["kv"], idx, ctx_len, scale, d_v)
            outs.append(o)
            lses.append(z)
    return dict(out=outs, lse=lses, idx=used, n_indexer_calls=calls)


def overlap_fraction(a: np.ndarray, b: np.ndarray) -> float:
    """Share of one query row's index set A that another layer's set B for the
    same row also holds: |A ∩ B| / |A|, the -1 padding of either set ignored
    (nan when A selects nothing).  The pages report how far the top-k
    selections of adjacent layers coincide (technical summary §1 on the
    pt/it/de editions: 70% to 100%); with A the set a layer's own indexer
    would select and B the set it reuses, this is the share of its own
    selection that reuse keeps.  a and b hold one row each (leading size-1
    dimensions are allowed): positions of different rows are not comparable."""
    rows = []
    for x in (a, b):
        x = np.asarray(x)
        if x.ndim == 0 or any(d != 1 for d in x.shape[:-1]):
            raise ValueError("overlap_fraction takes one row's index set per argument")
        rows.append(x.reshape(-1))
    sa = set(int(x) for x in rows[0] if x >= 0)
    sb = set(int(x) for x in rows[1] if x >= 0)
    if not sa:
        return math.nan
    return len(sa & sb) / len(sa)


# --------------------------------------------------------------------------
# Training-free pattern search (greedy F -> S conversion, proxy loss)
# --------------------------------------------------------------------------

PROXIES = ("output", "miss")


def reuse_costs(layers: List[Dict[str, np.ndarray]], ctx_len: Sequence[int], k: int,
                scale: float, d_v: int, proxy: str = "output", idx_sets=None) -> np.ndarray:
    """Cost matrix C [n, n]: C[l, j] for j < l is the proxy cost at layer l of
    attending with layer j's index set instead of its own; C[l, l] = 0 and the
    entries above the diagonal are 0 (never used: a source precedes its
    layer).

    own set T_l = topk(indexer_scores(layer l)) unless idx_sets[l] is given.
    "output": sum over (b, t, head, value) of (o_l[T_j] - o_l[T_l])^2 divided
              by the sum of o_l[T_l]^2 (0 / 0 = 0, x / 0 = inf), o_l[T] being
              layer l's sparse attention output over set T;
    "miss":   1 - (sum over rows of |T_j ∩ T_l|) / (sum over rows of |T_l|)
              (0 when no row selects anything)."""
    if proxy not in PROXIES:
        raise ValueError(f"proxy must be one of {PROXIES}")
    n = len(layers)
    sets = list(idx_sets) if idx_sets is not None else [
        topk(indexer_scores(L["q_idx"], L["w"], L["k_idx"], ctx_len), ctx_len, k)
        for L in layers]
    C = np.zeros((n, n))
    if proxy == "output":
        own = [sparse_attn(layers[l]["q"], layers[l]["kv"], sets[l], ctx_len, scale, d_v)[0]
               for l in range(n)]
        for l in range(n):
            ref = float(np.sum(own[l] ** 2))
            for j in range(l):
                o = sparse_attn(layers[l]["q"], layers[l]["kv"], sets[j], ctx_len, scale, d_v)[0]
                err = float(np.sum((o - own[l]) ** 2))
                C[l, j] = err / ref if ref > 0 else (0.0 if err == 0 else math.inf)
    else:
        for l in range(n):
            mine = sets[l].reshape(-1, sets[l].shape[-1])
            for j in range(l):
                theirs = sets[j].reshape(-1, sets[j].shape[-1])
                common = total = 0
                for r in range(mine.shape[0]):
                    a = set(int(x) for x in mine[r] if x >= 0)
                    common += len(a & set(int(x) for x in theirs[r] if x >= 0))
                    total += len(a)
                C[l, j] = 1.0 - common / total if total > 0 else 0.0
    return C


def pattern_sources(pattern: str) -> List[int]:
    """src[l] = l for an F layer, the nearest preceding F layer for an S layer."""
    validate_pattern(pattern, len(pattern))
    src, last = [], 0
    for l, c in enumerate(pattern):
        if c == "F":
            last = l
        src.append(last)
    return src


def pattern_cost(pattern: str, C: np.ndarray) -> float:
    """Proxy loss of a pattern: sum over layers, in layer order, of
    C[l, src(l)] (F layers add C[l, l] = 0)."""
    total = 0.0
    for l, j in enumerate(pattern_sources(pattern)):
        total += float(C[l, j])
    return total


def greedy_pattern_search(C: np.ndarray, n_shared: int):
    """Greedy F -> S conversion.  Starting from all-F, each step tries every
    F layer except layer 0 (an S layer needs a preceding F) as S and keeps the
    conversion with the lowest pattern_cost; equal costs go to the lower
    layer.  Returns [(pattern, cost)] after each of the n_shared steps."""
    n = C.shape[0]
    if not 0 <= n_shared <= n - 1:
        raise ValueError(f"n_shared must be in 0..{n - 1}")
    pattern = ["F"] * n
    trace = []
    for _ in range(n_shared):
        best, best_cost = None, None
        for l in range(1, n):
            if pattern[l] != "F":
                continue
            cand = pattern.copy()
            cand[l] = "S"
            c = pattern_cost("".join(cand), C)
            if best_cost is None or c < best_cost:
                best, best_cost = cand, c
        pattern = best
        trace.append(("".join(pattern), best_cost))
    return trace
