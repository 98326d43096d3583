"""Float64 CPU oracle for exact attention, paged decode and the partial-result merge.

TEST INFRASTRUCTURE. This module is the checker, not the product: only the test
suite, the smoke check and the benchmark's CPU-baseline leg import it. The
library's HIP path never calls it, and it never calls the library.

What it computes is the plain definition of attention, not the tiled method.
The pages agree that FlashAttention returns exactly the result of ordinary
attention up to floating-point reordering ("3.4 Attention Kernels", sections
"Why this matters" and "Common pitfalls"; "FlashAttention and Optimized
Kernels", section "It is exact"). So the reference is ordinary attention
("3.4 Attention Kernels", section "Naive attention and its memory traffic" and
its NumPy `naive_attention` under "Code"):

    S = scale * Q K^T           materialised, one query row against all its keys
    S_ij = -inf  where key j is invisible to query i under the causal mask
    P = exp(S - rowmax S)       materialised
    O = (P V) / rowsum P
    LSE = rowmax S + ln rowsum P   (the log-sum-exp the tiled kernel stores,
                                     "3.4 Attention Kernels", "FlashAttention: tiling")

Everything is evaluated in float64 on the (already dtype-rounded) inputs the
GPU receives; bf16/fp16/fp32 values are exact in float64.

Readings taken where the pages leave a point open:
  * Layout [batch, seq, heads, d] for Q/K/V/O ("3.4 Attention Kernels",
    "Paged and ragged layouts"), LSE as [batch, heads, seq].
  * Causal alignment is bottom-right: key j is visible to query i iff
    j <= i + (Nk - Nq), the alignment of the mask in the page's NumPy naive
    attention ("3.4 Attention Kernels", section "Code"); it equals top-left
    alignment when Nq == Nk.
  * Grouped-query heads are contiguous groups: query head h reads KV head
    h // (H // Hkv) ("3.4 Attention Kernels", "Decode attention and
    Flash-Decoding", the GQA paragraph).
  * A row with no visible key has O = 0 and LSE = -inf (the empty partial of
    the merge rule).
  * Paged KV: token t of sequence b lives in page block_table[b, t // page]
    at slot t % page; only the first seq_lens[b] tokens exist ("3.4 Attention
    Kernels", "Paged and ragged layouts": block table plus last-page length,
    expressed here as the sequence length).
  * A partial result over a key subset is stored as (o, lse) with
    o = acc / l and lse = m + ln l; this is the triple (m, l, acc) of the merge
    rule with m = lse, l = 1, acc = o, so the merge below is that rule.

Row blocks only bound memory: each query row is always evaluated against all
of its keys at once, so the blocking never enters the arithmetic of a row.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "attention",
    "attention_ragged_paged",
    "cascade_attention",
    "log_sum_exp",
    "decode_paged",
    "decode_paged_variant",
    "gather_paged_kv",
    "merge_partials",
    "online_softmax_row",
    "split_kv_partials",
    "causal_visible",
    "default_threads",
]


def default_threads() -> int:
    """Worker threads for the row-block loop (BLAS and ufuncs release the GIL)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _f64(x) -> np.ndarray:
    """float64 copy of an array; torch CPU tensors (bf16/fp16 included) are
    converted by torch itself, exactly, since numpy has no bfloat16."""
    if type(x).__module__.startswith("torch"):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# The definition, one (batch, head) and one block of query rows at a time.
# ---------------------------------------------------------------------------

def causal_visible(q_idx: np.ndarray, n_keys: int, offset: int) -> np.ndarray:
    """Boolean [len(q_idx), n_keys]: key j visible to query i iff j <= i + offset.

    offset = Nk - Nq: the bottom-right aligned causal mask, the diagonal
    ending at the last query and the last key, as the page's NumPy naive
    attention builds it ("3.4 Attention Kernels", section "Code").
    """
    keys = np.arange(n_keys)[None, :]
    return keys <= (q_idx[:, None] + offset)


def _scores(qb: np.ndarray, kh: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for a block of query rows against all keys."""
    return scale * (qb @ kh.T)


def _softmax_stats(s: np.ndarray):
    """Row max m, unnormalised weights P = exp(S - m) and row sum l.

    Rows whose scores are all -inf (no visible key) get m = -inf, P = 0, l = 0.
    Stable softmax, "3.4 Attention Kernels", section "Online softmax", first
    paragraph: subtracting the row max prevents overflow and changes nothing.
    """
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    p = np.exp(s - m_safe[:, None])
    p[~finite, :] = 0.0
    l = p.sum(axis=1)
    return m, p, l


def _lse_from_stats(m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """LSE = m + ln l (natural log, "3.4 Attention Kernels", section
    "FlashAttention: tiling"); -inf where the row saw no key (l = 0)."""
    with np.errstate(divide="ignore"):
        v = m + np.log(l)
    return np.where(l > 0, v, -np.inf)


def _rows_block(qh, kh, vh, scale, causal, q_idx, nq, want_o=True):
    """O (or None) and LSE for the query rows q_idx of one (batch, head)."""
    nk = kh.shape[0]
    s = _scores(qh[q_idx], kh, scale)
    if causal:
        s = np.where(causal_visible(q_idx, nk, nk - nq), s, -np.inf)
    m, p, l = _softmax_stats(s)
    lse = _lse_from_stats(m, l)
    if not want_o:
        return None, lse
    num = p @ vh
    o = np.zeros_like(num)
    nz = l > 0
    o[nz] = num[nz] / l[nz, None]
    return o, lse


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or (v is not None and v.ndim != 4):
        raise ValueError("expected [batch, seq, heads, d] arrays")
    B, _, H, d = q.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("K shape does not match Q")
    if v is not None and v.shape != k.shape:
        raise ValueError("V shape must equal K shape")
    hkv = k.shape[2]
    if hkv < 1 or H % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    return B, H, hkv


def attention(q, k, v, scale: float, causal: bool, rows=None,
              block_rows: int = 512, threads: int | None = None):
    """Exact attention by the definition, in float64.

    q: [B, Nq, H, d]; k, v: [B, Nk, Hkv, d]; H % Hkv == 0.
    rows: optional 1-D index array of query positions; when given, O and LSE
    are returned for those positions only (each row still sees all its keys).
    Returns O [B, R, H, d] and LSE [B, H, R] (R = Nq, or len(rows)).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, hkv = _check_shapes(q, k, v)
    nq, d = q.shape[1], q.shape[3]
    group = H // hkv
    sel = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = sel.shape[0]
    out = np.zeros((B, R, H, d))
    lse = np.full((B, H, R), -np.inf)

    jobs = [(b, h, r0) for b in range(B) for h in range(H)
            for r0 in range(0, R, block_rows)]

    def run(job):
        b, h, r0 = job
        hk = h // group
        idx = sel[r0:r0 + block_rows]
        o, l = _rows_block(q[b, :, h, :], k[b, :, hk, :], v[b, :, hk, :],
                           scale, causal, idx, nq)
        out[b, r0:r0 + len(idx), h, :] = o
        lse[b, h, r0:r0 + len(idx)] = l

    _run_jobs(run, jobs, threads)
    return out, lse


def log_sum_exp(q, k, scale: float, causal: bool, heads=None,
                block_rows: int = 256, threads: int | None = None):
    """LSE = rowmax S + ln rowsum exp(S - rowmax S) for every query row.

    Same definition as `attention` without the P V product. For causal rows
    the score block is formed only over keys that some row of the block can
    see; every key past that bound is masked (-inf, weight exactly 0) for
    every row of the block, so the value is unchanged.
    heads: optional list of query heads to evaluate (others stay -inf).
    Returns LSE [B, H, Nq].
    """
    q, k = _f64(q), _f64(k)
    B, H, hkv = _check_shapes(q, k, None)
    nq, nk = q.shape[1], k.shape[1]
    group = H // hkv
    hs = range(H) if heads is None else list(heads)
    lse = np.full((B, H, nq), -np.inf)
    jobs = [(b, h, r0) for b in range(B) for h in hs
            for r0 in range(0, nq, block_rows)]

    def run(job):
        b, h, r0 = job
        hk = h // group
        idx = np.arange(r0, min(r0 + block_rows, nq))
        kmax = nk
        if causal:
            kmax = int(min(nk, max(0, idx[-1] + (nk - nq) + 1)))
        kh = k[b, :kmax, hk, :]
        s = _scores(q[b, idx, h, :], kh, scale)
        if causal:
            s = np.where(causal_visible(idx, kmax, nk - nq), s, -np.inf)
        m, _, l = _softmax_stats(s)
        lse[b, h, r0:r0 + len(idx)] = _lse_from_stats(m, l)

    _run_jobs(run, jobs, threads)
    return lse


def _run_jobs(fn, jobs, threads):
    n = default_threads() if threads is None else max(1, threads)
    if n == 1 or len(jobs) <= 1:
        for j in jobs:
            fn(j)
        return
    with ThreadPoolExecutor(max_workers=n) as ex:
        for _ in ex.map(fn, jobs):
            pass


# ---------------------------------------------------------------------------
# Paged decode: one query token per sequence against its paged, ragged cache.
# ---------------------------------------------------------------------------

def gather_paged_kv(pool, block_table, seq_len: int, b: int):
    """Tokens 0..seq_len-1 of sequence b from a page pool [P, page, Hkv, d].

    Token t is slot t % page of page block_table[b, t // page]. Entries of
    the block table past the last used page are never read.
    """
    page = pool.shape[1]
    t = np.arange(int(seq_len))
    pages = np.asarray(block_table)[b, t // page]
    return _f64(pool[pages, t % page])  # [len, Hkv, d]


def decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale: float):
    """Decode attention over a paged KV cache, by the definition.

    q: [B, H, d]; k_pool, v_pool: [P, page, Hkv, d]; block_table: [B, max_pages]
    int; seq_lens: [B] int. One query per sequence, no mask beyond the length
    ("3.4 Attention Kernels", "Decode attention and Flash-Decoding").
    Returns O [B, H, d] and LSE [B, H]; a sequence of length 0 gives O = 0,
    LSE = -inf.
    """
    q = _f64(q)
    B, H, d = q.shape
    hkv = k_pool.shape[2]
    if H % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = H // hkv
    out = np.zeros((B, H, d))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        kb = gather_paged_kv(k_pool, block_table, L, b)
        vb = gather_paged_kv(v_pool, block_table, L, b)
        for h in range(H):
            hk = h // group
            o, l = _rows_block(q[b, h][None, :], kb[:, hk, :], vb[:, hk, :],
                               scale, False, np.zeros(1, np.int64), 1)
            out[b, h] = o[0]
            lse[b, h] = l[0]
    return out, lse


def _seq_rows(qo_indptr, b: int):
    """Query rows of sequence b in a ragged batch: qo_indptr[b] .. qo_indptr[b+1]-1."""
    return int(qo_indptr[b]), int(qo_indptr[b + 1])


def attention_ragged_paged(q, qo_indptr, k_pool, v_pool, block_table, kv_lens, scale: float,
                           causal: bool, threads: int | None = None):
    """Attention for a ragged batch of queries over a paged KV cache, by the
    definition, one sequence at a time.

    "3.4 Attention Kernels", section "Paged and ragged layouts: FlashInfer":
    the query rows of all sequences are concatenated and `qo_indptr` marks where
    each sequence starts; each sequence's keys and values are its kv_lens[b]
    cached tokens, gathered through its block table. The queries of a sequence
    are its newest positions, so with causal=True the bottom-right alignment of
    `attention` applies within each sequence (query i sees key j iff
    j <= i + kv_len - q_len).

    q: [total_q, H, d]; qo_indptr: [B+1]; k_pool, v_pool: [P, page, Hkv, d];
    block_table: [B, max_pages]; kv_lens: [B]. Returns O [total_q, H, d] and
    LSE [total_q, H] (float64). Rows of no sequence stay O = 0, LSE = -inf.
    """
    q = _f64(q)
    total_q, H, d = q.shape
    hkv = k_pool.shape[2]
    out = np.zeros((total_q, H, d))
    lse = np.full((total_q, H), -np.inf)
    for b in range(len(kv_lens)):
        r0, r1 = _seq_rows(qo_indptr, b)
        if r1 <= r0:
            continue
        L = int(kv_lens[b])
        kb = gather_paged_kv(k_pool, block_table, L, b) if L else np.zeros((0, hkv, d))
        vb = gather_paged_kv(v_pool, block_table, L, b) if L else np.zeros((0, hkv, d))
        o, l = attention(q[r0:r1][None], kb[None], vb[None], scale, causal, threads=threads)
        out[r0:r1] = o[0]
        lse[r0:r1] = l[0].T
    return out, lse


def _concat_keys(prefix: np.ndarray, own: np.ndarray) -> np.ndarray:
    """A sequence's keys (or values) in a cascade: the shared prefix first."""
    return np.concatenate([prefix, own], axis=0)


def cascade_attention(q, qo_indptr, k_pool, v_pool, prefix_pages, prefix_len: int,
                      block_table, kv_lens, scale: float, causal: bool,
                      threads: int | None = None):
    """Attention for sequences sharing one prefix, by the definition.

    "3.4 Attention Kernels", section "Paged and ragged layouts: FlashInfer"
    (cascade attention): sequence b's keys and values are the prefix_len
    shared prefix tokens (token t in page prefix_pages[t // page], slot
    t % page) followed by its own kv_lens[b] tokens from its block table. The
    result is plain attention over that concatenation, bottom-right causal
    when causal=True, i.e. what the cascade's merge of prefix and suffix parts
    must reproduce. Shapes and outputs as `attention_ragged_paged`.
    """
    q = _f64(q)
    total_q, H, d = q.shape
    hkv = k_pool.shape[2]
    table = np.asarray(prefix_pages).reshape(1, -1)
    pk = gather_paged_kv(k_pool, table, prefix_len, 0) if prefix_len else np.zeros((0, hkv, d))
    pv = gather_paged_kv(v_pool, table, prefix_len, 0) if prefix_len else np.zeros((0, hkv, d))
    out = np.zeros((total_q, H, d))
    lse = np.full((total_q, H), -np.inf)
    for b in range(len(kv_lens)):
        r0, r1 = _seq_rows(qo_indptr, b)
        if r1 <= r0:
            continue
        L = int(kv_lens[b])
        kb = gather_paged_kv(k_pool, block_table, L, b) if L else np.zeros((0, hkv, d))
        vb = gather_paged_kv(v_pool, block_table, L, b) if L else np.zeros((0, hkv, d))
        kk, vv = _concat_keys(pk, kb), _concat_keys(pv, vb)
        o, l = attention(q[r0:r1][None], kk[None], vv[None], scale, causal, threads=threads)
        out[r0:r1] = o[0]
        lse[r0:r1] = l[0].T
    return out, lse


def _window_start(seq_len: int, window: int) -> int:
    """First visible token of a sequence of seq_len tokens under a sliding
    window of the newest `window` tokens (0 = no window)."""
    return seq_len - window if (window > 0 and seq_len > window) else 0


def _soft_cap(x: np.ndarray, cap: float) -> np.ndarray:
    """Logit soft-capping of scaled scores: cap * tanh(x / cap)."""
    return cap * np.tanh(x / cap)


def decode_paged_variant(q, k_pool, v_pool, block_table, seq_lens, scale: float,
                         window: int = 0, softcap: float = 0.0):
    """Decode attention with a sliding window and/or logit soft-capping.

    "3.4 Attention Kernels", section "Paged and ragged layouts: FlashInfer",
    names both as attention variants without defining them; the readings here
    are:
      window > 0: only the newest `window` tokens t of sequence b are visible,
        seq_lens[b] - window <= t < seq_lens[b] (the query's own position is
        the newest token); window == 0: all tokens.
      softcap > 0: the scaled score x = scale * q.k becomes
        softcap * tanh(x / softcap) before the softmax; softcap == 0: unchanged.
    Then P = exp(x - max x), O = P V / sum P, LSE = max x + ln sum P over the
    visible tokens, as in `decode_paged`. Returns O [B, H, d], LSE [B, H].
    """
    q = _f64(q)
    B, H, d = q.shape
    hkv = k_pool.shape[2]
    if H % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = H // hkv
    out = np.zeros((B, H, d))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        first = _window_start(L, window)
        if L - first <= 0:
            continue
        kb = gather_paged_kv(k_pool, block_table, L, b)[first:]
        vb = gather_paged_kv(v_pool, block_table, L, b)[first:]
        for h in range(H):
            hk = h // group
            x = _scores(q[b, h][None, :], kb[:, hk, :], scale)   # [1, visible]
            if softcap > 0:
                x = _soft_cap(x, softcap)
            m, p, l = _softmax_stats(x)
            out[b, h] = (p @ vb[:, hk, :])[0] / l[0]
            lse[b, h] = _lse_from_stats(m, l)[0]
    return out, lse


# ---------------------------------------------------------------------------
# The merge rule for partial results over disjoint key sets.
# ---------------------------------------------------------------------------

def _merge_weights(lse_parts: np.ndarray, M: float) -> np.ndarray:
    """w_c = exp(lse_c - M); an empty part (lse = -inf) weighs 0."""
    w = np.exp(lse_parts - M)
    w[~np.isfinite(lse_parts)] = 0.0
    return w


def merge_partials(o_parts, lse_parts, num_parts=None):
    """Combine per-split partials (o_c, lse_c) into (O, LSE), in float64.

    "3.4 Attention Kernels", section "Online softmax" (the merge of two partial
    results on disjoint key sets), applied to all parts at once with a common
    reference max: M = max_c lse_c, w_c = exp(lse_c - M),
    O = sum_c w_c o_c / sum_c w_c, LSE = M + ln sum_c w_c.
    A part with lse = -inf is empty and contributes nothing; if every part is
    empty the result is O = 0, LSE = -inf.

    o_parts: [R, S, d]; lse_parts: [R, S]; num_parts: optional [R] int, the
    number of leading parts that are valid in each row (default: all S).
    """
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    R, S, d = o_parts.shape
    out = np.zeros((R, d))
    lse = np.full(R, -np.inf)
    for r in range(R):
        n = S if num_parts is None else int(num_parts[r])
        ls = lse_parts[r, :n]
        if n == 0 or not np.isfinite(ls).any():
            continue
        M = ls.max()
        w = _merge_weights(ls, M)
        z = w.sum()
        out[r] = (w[:, None] * o_parts[r, :n]).sum(axis=0) / z
        lse[r] = M + math.log(z)
    return out, lse


# ---------------------------------------------------------------------------
# The method's own steps, for pinning the pages' printed traces and for the
# split/merge invariants. These never stand in for the definition above.
# ---------------------------------------------------------------------------

def _rescale_factor(m_old: float, m_new: float) -> float:
    """alpha = e^(m_old - m_new); a state that has seen nothing (m_old = -inf)
    weighs 0."""
    return 0.0 if m_old == -np.inf else float(np.exp(m_old - m_new))


def online_softmax_row(scores, values, tile: int):
    """Softmax-weighted sum of `values` visited `tile` scores at a time.

    The running triple (m, l, acc) starts at (-inf, 0, 0). For each block, in
    the order "3.4 Attention Kernels", section "Online softmax" states it and
    "Multi-head attention to flash attention", section "Online Softmax
    Calculation" traces it:
        m' = max(m, max of the block's scores)
        factor = e^(m - m')            (0 when nothing has been seen yet)
        l   <- factor * l   + sum_j e^(s_j - m')
        acc <- factor * acc + sum_j e^(s_j - m') v_j
        m   <- m'
    and the result is acc / l.
    Returns (o, trace) with one dict per block holding the state after the
    rescale and after the block's contribution.
    """
    s = _f64(scores)
    vals = _f64(values)
    if vals.ndim == 1:
        vals = vals[:, None]
    n = s.shape[0]
    state = {"m": -np.inf, "l": 0.0, "acc": np.zeros(vals.shape[1])}
    trace = []
    for first in np.arange(0, n, tile):
        block = slice(int(first), int(min(first + tile, n)))
        m_next = max(state["m"], float(np.max(s[block])))
        alpha = _rescale_factor(state["m"], m_next)
        l_scaled = alpha * state["l"]
        acc_scaled = alpha * state["acc"]
        w = np.exp(s[block] - m_next)
        state = {"m": m_next, "l": l_scaled + float(np.sum(w)),
                 "acc": acc_scaled + w @ vals[block]}
        trace.append(dict(m=m_next, factor=alpha, l_rescaled=l_scaled,
                          acc_rescaled=acc_scaled.copy(), l=state["l"],
                          acc=state["acc"].copy()))
    return state["acc"] / state["l"], trace


def split_kv_partials(q_row, k_rows, v_rows, scale: float, n_splits: int):
    """Partials (o_c, lse_c) of one query over `n_splits` contiguous key chunks.

    The chunking is numpy.array_split's, as in the page's `flash_decoding`
    ("3.4 Attention Kernels", section "Code"); each chunk's partial is the
    definition restricted to that chunk. A chunk with no keys is the empty
    partial (o = 0, lse = -inf).
    q_row: [d]; k_rows, v_rows: [L, d]. Returns o [S, d], lse [S].
    """
    q_row, k_rows, v_rows = _f64(q_row), _f64(k_rows), _f64(v_rows)
    idx = np.array_split(np.arange(k_rows.shape[0]), n_splits)
    o = np.zeros((n_splits, q_row.shape[0]))
    lse = np.full(n_splits, -np.inf)
    for c, ids in enumerate(idx):
        if len(ids) == 0:
            continue
        oc, lc = _rows_block(q_row[None, :], k_rows[ids], v_rows[ids], scale,
                             False, np.zeros(1, np.int64), 1)
        o[c], lse[c] = oc[0], lc[0]
    return o, lse
