"""Pins for the float64 oracle, all on the CPU.

Each pin ties the oracle to something other than itself: a value the pages
print, a closed form, a 50-digit brute force, a library routine on a case
where it is known to agree, or an invariance the pages state. The mutation
tests at the end plant plausible mistakes in the oracle and check that some
pin catches each one.
"""

import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
from oracle import attention_ref as ref_mod

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------
# Pins. Each takes the oracle module so the mutation tests can rerun it.
# ---------------------------------------------------------------------------

def pin_lab_example(ref):
    """Printed batch == online result 53.6863940430, through the attention call.

    The scores are produced as q . k_j with one-hot keys and scale 1, the
    values sit in column 0 of V; d is padded to 64 with zeros.
    """
    g = _golden("online_softmax_lab.json")
    s = np.array(g["scores"])
    n, d = len(s), 64
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, :n] = s
    k = np.zeros((1, n, 1, d))
    k[0, np.arange(n), 0, np.arange(n)] = 1.0
    v = np.zeros((1, n, 1, d))
    v[0, :, 0, 0] = g["values"]
    o, lse = ref.attention(q, k, v, scale=1.0, causal=False)
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    assert abs(o[0, 0, 0, 0] - g["printed_result"]) <= tol
    assert np.all(o[0, 0, 0, 1:] == 0.0)
    # the recurrence in the page's tiling gives the same printed value
    o2, _ = ref.online_softmax_row(s, np.array(g["values"], float), g["tile"])
    assert abs(o2[0] - g["printed_result"]) <= tol
    # and so do split partials merged by the merge rule, for several splits
    for n_splits in (1, 2, 3, 4, 10, 16):
        po, pl = ref.split_kv_partials(q[0, 0, 0], k[0, :, 0], v[0, :, 0],
                                       1.0, n_splits)
        mo, ml = ref.merge_partials(po[None], pl[None])
        assert abs(mo[0, 0] - g["printed_result"]) <= tol
        assert abs(ml[0] - lse[0, 0, 0]) <= 1e-12


def pin_trace_example(ref):
    """The page's step-by-step state (m, l, acc) and final 5.551."""
    g = _golden("online_softmax_trace.json")
    qv = np.array(g["q"], float)
    keys = np.array(g["keys"], float)
    vals = np.array(g["values"], float)
    s = keys @ qv * g["scale"]
    o, tr = ref.online_softmax_row(s, vals, g["block"])
    ts, to = g["tolerance_state"], g["tolerance_output"]
    b1, b2 = tr
    assert abs(b1["m"] - g["after_block_1"]["m"]) <= ts
    assert abs(b1["l"] - g["after_block_1"]["l"]) <= ts
    assert abs(b1["acc"][0] - g["after_block_1"]["acc"]) <= ts
    assert abs(b2["factor"] - g["block_2_factor"]) <= ts
    assert abs(b2["l_rescaled"] - g["after_rescale"]["l"]) <= ts
    assert abs(b2["acc_rescaled"][0] - g["after_rescale"]["acc"]) <= ts
    assert abs(b2["m"] - g["after_block_2"]["m"]) <= ts
    assert abs(b2["l"] - g["after_block_2"]["l"]) <= ts
    assert abs(b2["acc"][0] - g["after_block_2"]["acc"]) <= ts
    assert abs(o[0] - g["printed_output"]) <= to
    # the same example through the attention call (d = 2, values in column 0)
    q = qv.reshape(1, 1, 1, 2)
    k = keys.reshape(1, 4, 1, 2)
    v = np.zeros((1, 4, 1, 2))
    v[0, :, 0, 0] = vals
    oa, la = ref.attention(q, k, v, scale=g["scale"], causal=False)
    assert abs(oa[0, 0, 0, 0] - g["printed_output"]) <= to
    # LSE of the trace: m + ln l of the final state
    assert abs(la[0, 0, 0] - (b2["m"] + math.log(b2["l"]))) <= 1e-12


def pin_rescale_factor(ref):
    """Running max 3 -> 5 multiplies the old state by e^-2."""
    g = _golden("rescale_factor.json")
    s = np.array([g["old_max"], 1.0, g["new_max"], 0.0])
    _, tr = ref.online_softmax_row(s, np.ones(4), tile=2)
    assert tr[0]["m"] == g["old_max"] and tr[1]["m"] == g["new_max"]
    assert abs(tr[1]["factor"] - g["factor"]) <= 1e-15


def pin_single_key(ref):
    """One visible key: O = v, LSE = scale * q . k."""
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 2, 3, 4, 16), _rand(rng, 2, 1, 2, 16), _rand(rng, 2, 1, 2, 16)
    o, lse = ref.attention(q, k, v, scale=0.3, causal=False)
    for b in range(2):
        for h in range(4):
            hk = h // 2
            np.testing.assert_allclose(o[b, :, h], np.repeat(v[b, :, hk], 3, 0),
                                       rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse[b, h], 0.3 * (q[b, :, h] @ k[b, 0, hk]),
                                       rtol=0, atol=1e-13)


def pin_causal_row0(ref):
    """Causal, Nq == Nk: row 0 sees only key 0, so O_0 = v_0, LSE_0 = s_00."""
    rng = np.random.default_rng(12)
    q, k, v = (_rand(rng, 1, 37, 3, 8) for _ in range(3))
    o, lse = ref.attention(q, k, v, scale=0.5, causal=True)
    np.testing.assert_allclose(o[0, 0], v[0, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, :, 0], 0.5 * np.einsum("hd,hd->h", q[0, 0], k[0, 0]),
                               rtol=0, atol=1e-13)


def pin_constant_v(ref):
    """Every value row equal to c gives O = c, causal or not."""
    rng = np.random.default_rng(13)
    q, k = _rand(rng, 2, 20, 2, 8), _rand(rng, 2, 29, 2, 8)
    c = _rand(rng, 8)
    v = np.broadcast_to(c, (2, 29, 2, 8)).copy()
    for causal in (False, True):
        o, _ = ref.attention(q, k, v, scale=1.0, causal=causal)
        np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-13)


def pin_zero_query(ref):
    """Q = 0 gives uniform weights over the visible keys.

    Non-causal: O = mean of V, LSE = ln Nk. Causal with bottom-right offset
    off = Nk - Nq: O_i = mean of v_0..v_{i+off}, LSE_i = ln(i + off + 1); rows
    with i + off < 0 have no key (O = 0, LSE = -inf).
    """
    rng = np.random.default_rng(14)
    for nq, nk in ((33, 33), (10, 25), (25, 10), (1, 7)):
        q = np.zeros((1, nq, 2, 4))
        k, v = _rand(rng, 1, nk, 1, 4), _rand(rng, 1, nk, 1, 4)
        o, lse = ref.attention(q, k, v, scale=1.0, causal=False)
        np.testing.assert_allclose(o[0, :, 0], np.broadcast_to(v[0, :, 0].mean(0), (nq, 4)),
                                   rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, math.log(nk), rtol=0, atol=1e-14)
        o, lse = ref.attention(q, k, v, scale=1.0, causal=True)
        off = nk - nq
        csum = np.cumsum(v[0, :, 0], axis=0)
        for i in range(nq):
            last = i + off
            if last < 0:
                assert np.all(o[0, i] == 0.0) and np.all(lse[0, :, i] == -np.inf)
                continue
            last = min(last, nk - 1)
            np.testing.assert_allclose(o[0, i, 1], csum[last] / (last + 1), rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[0, :, i], math.log(last + 1), rtol=0, atol=1e-14)


def pin_rows_sum_to_one(ref):
    """With V = I (Nk = d), O is the probability matrix: rows >= 0, sum to 1."""
    rng = np.random.default_rng(15)
    n = 24
    q, k = _rand(rng, 1, n, 1, n) * 3, _rand(rng, 1, n, 1, n)
    v = np.eye(n).reshape(1, n, 1, n)
    for causal in (False, True):
        o, _ = ref.attention(q, k, v, scale=1.0, causal=causal)
        p = o[0, :, 0, :]
        assert np.all(p >= 0)
        np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-14)
        if causal:
            assert np.all(np.triu(p, 1) == 0.0)


def _decimal_attention(q, k, v, scale, causal):
    """50-digit brute force of O and LSE for tiny [N, d] single-head inputs."""
    getcontext().prec = 50
    nq, nk, d = q.shape[0], k.shape[0], q.shape[1]
    D = Decimal
    sc = D(scale)
    out = np.zeros((nq, d))
    lse = np.full(nq, -np.inf)
    for i in range(nq):
        s = []
        for j in range(nk):
            if causal and j > i + (nk - nq):
                continue
            s.append((j, sc * sum(D(float(q[i, t])) * D(float(k[j, t])) for t in range(d))))
        if not s:
            continue
        z = sum(x.exp() for _, x in s)
        for t in range(d):
            out[i, t] = float(sum(x.exp() * D(float(v[j, t])) for j, x in s) / z)
        lse[i] = float(z.ln())
    return out, lse


def pin_brute_force(ref):
    """Exact (50-digit) evaluation on tiny inputs, incl. GQA and Nq != Nk."""
    rng = np.random.default_rng(16)
    for (nq, nk, h, hkv, d, causal) in ((5, 5, 2, 1, 3, True), (4, 6, 2, 2, 3, True),
                                        (6, 4, 1, 1, 2, True), (3, 7, 4, 2, 3, False)):
        q = _rand(rng, 1, nq, h, d) * 2
        k, v = _rand(rng, 1, nk, hkv, d), _rand(rng, 1, nk, hkv, d)
        o, lse = ref.attention(q, k, v, scale=0.7, causal=causal)
        for hh in range(h):
            hk = hh // (h // hkv)
            eo, el = _decimal_attention(q[0, :, hh], k[0, :, hk], v[0, :, hk], 0.7, causal)
            np.testing.assert_allclose(o[0, :, hh], eo, rtol=0, atol=1e-12)
            fin = np.isfinite(el)
            assert np.array_equal(fin, np.isfinite(lse[0, hh]))
            np.testing.assert_allclose(lse[0, hh][fin], el[fin], rtol=0, atol=1e-12)


def pin_torch_sdpa(ref):
    """PyTorch's math attention in float64 on the CPU, Nq == Nk (top-left ==
    bottom-right there), plus an explicit bottom-right mask for Nq < Nk."""
    rng = np.random.default_rng(17)
    q, k, v = (_rand(rng, 2, 40, 4, 16) for _ in range(3))
    for causal in (False, True):
        o, _ = ref.attention(q, k, v, scale=0.25, causal=causal)
        t = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q).transpose(1, 2), torch.from_numpy(k).transpose(1, 2),
            torch.from_numpy(v).transpose(1, 2), is_causal=causal, scale=0.25)
        np.testing.assert_allclose(o, t.transpose(1, 2).numpy(), rtol=0, atol=1e-12)
    q2 = _rand(rng, 1, 12, 2, 8)
    k2, v2 = _rand(rng, 1, 30, 2, 8), _rand(rng, 1, 30, 2, 8)
    mask = torch.ones(12, 30, dtype=torch.bool).tril(diagonal=30 - 12)
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q2).transpose(1, 2), torch.from_numpy(k2).transpose(1, 2),
        torch.from_numpy(v2).transpose(1, 2), attn_mask=mask, scale=0.5)
    o, _ = ref.attention(q2, k2, v2, scale=0.5, causal=True)
    np.testing.assert_allclose(o, t.transpose(1, 2).numpy(), rtol=0, atol=1e-12)


def pin_key_permutation(ref):
    """Non-causal attention does not depend on the order of the keys."""
    rng = np.random.default_rng(18)
    q, k, v = _rand(rng, 1, 9, 2, 8), _rand(rng, 1, 31, 2, 8), _rand(rng, 1, 31, 2, 8)
    perm = rng.permutation(31)
    o1, l1 = ref.attention(q, k, v, 0.4, False)
    o2, l2 = ref.attention(q, k[:, perm], v[:, perm], 0.4, False)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


def pin_gqa_equals_repeated_mha(ref):
    """Grouped heads equal ordinary heads with each KV head repeated g times."""
    rng = np.random.default_rng(19)
    q = _rand(rng, 2, 17, 8, 8)
    k, v = _rand(rng, 2, 23, 2, 8), _rand(rng, 2, 23, 2, 8)
    for causal in (False, True):
        o1, l1 = ref.attention(q, k, v, 0.5, causal)
        o2, l2 = ref.attention(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), 0.5, causal)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
        np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-14)


def pin_rows_subset(ref):
    """O/LSE for a subset of rows equal the same rows of the full result."""
    rng = np.random.default_rng(20)
    q, k, v = (_rand(rng, 1, 50, 2, 8) for _ in range(3))
    rows = np.array([0, 3, 17, 49, 25])
    of, lf = ref.attention(q, k, v, 0.5, True)
    os_, ls = ref.attention(q, k, v, 0.5, True, rows=rows)
    np.testing.assert_array_equal(os_, of[:, rows])
    np.testing.assert_array_equal(ls, lf[:, :, rows])
    lfast = ref.log_sum_exp(q, k, 0.5, True, block_rows=7)
    np.testing.assert_allclose(lfast, lf, rtol=0, atol=1e-13)
    q2, k2 = _rand(rng, 1, 20, 2, 8), _rand(rng, 1, 33, 1, 8)
    _, l2 = ref.attention(q2, k2, k2, 0.5, True)
    np.testing.assert_allclose(ref.log_sum_exp(q2, k2, 0.5, True, block_rows=6), l2,
                               rtol=0, atol=1e-13)


def pin_paged_decode(ref):
    """Paged decode == dense decode; page order and unused table entries do
    not matter; a zero-length sequence gives O = 0, LSE = -inf."""
    rng = np.random.default_rng(21)
    B, H, hkv, d, page = 4, 8, 2, 8, 16
    lens = np.array([1, 16, 37, 0])
    max_pages = 4
    n_pages = 20
    kp, vp = _rand(rng, n_pages, page, hkv, d), _rand(rng, n_pages, page, hkv, d)
    q = _rand(rng, B, H, d)
    perm = rng.permutation(n_pages)
    table = perm[:B * max_pages].reshape(B, max_pages).copy()
    used = -(-lens // page)
    for b in range(B):
        table[b, used[b]:] = 10**6  # never read
    o, lse = ref.decode_paged(q, kp, vp, table, lens, 0.3)
    for b in range(B):
        if lens[b] == 0:
            assert np.all(o[b] == 0) and np.all(lse[b] == -np.inf)
            continue
        t = np.arange(lens[b])
        kb = kp[table[b, t // page], t % page]  # [L, hkv, d]
        vb = vp[table[b, t // page], t % page]
        od, ld = ref.attention(q[b][None, None], kb[None], vb[None], 0.3, False)
        np.testing.assert_allclose(o[b], od[0, 0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[b], ld[0, :, 0], rtol=0, atol=1e-14)
    # same tokens stored in a contiguous identity layout give the same result
    kid = np.zeros((B * max_pages, page, hkv, d))
    vid = np.zeros_like(kid)
    ident = np.arange(B * max_pages).reshape(B, max_pages)
    for b in range(B):
        for p in range(used[b]):
            kid[ident[b, p]] = kp[table[b, p]]
            vid[ident[b, p]] = vp[table[b, p]]
    o2, l2 = ref.decode_paged(q, kid, vid, ident, lens, 0.3)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)


def _paged_case(rng, lens, B=3, H=4, hkv=2, d=8, page=16, extra_pages=3):
    max_pages = int(max(1, -(-max(lens) // page)))
    n_pages = B * max_pages + extra_pages
    kp, vp = _rand(rng, n_pages, page, hkv, d), _rand(rng, n_pages, page, hkv, d)
    q = _rand(rng, B, H, d)
    table = rng.permutation(n_pages)[:B * max_pages].reshape(B, max_pages).copy()
    return q, kp, vp, table, np.asarray(lens)


def _tokens(pool, table, b, t, page=16):
    return pool[table[b, t // page], t % page]


def pin_decode_window(ref):
    """Sliding window: the newest `window` tokens only. window >= len is the
    plain decode; window == 1 returns the newest token's value row with
    LSE = its scaled score; 1 < window < len equals dense attention over the
    explicitly sliced last `window` tokens; len 0 gives O = 0, LSE = -inf."""
    rng = np.random.default_rng(31)
    lens = [45, 16, 0]
    q, kp, vp, table, lens = _paged_case(rng, lens)
    scale = 0.4
    plain = ref.decode_paged(q, kp, vp, table, lens, scale)
    for w in (45, 46, 1000):
        o, l = ref.decode_paged_variant(q, kp, vp, table, lens, scale, window=w)
        np.testing.assert_allclose(o, plain[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(l, plain[1], rtol=0, atol=1e-14)
    o, l = ref.decode_paged_variant(q, kp, vp, table, lens, scale, window=1)
    for b in range(2):
        t = lens[b] - 1
        kl, vl = _tokens(kp, table, b, t), _tokens(vp, table, b, t)
        for h in range(4):
            np.testing.assert_array_equal(o[b, h], vl[h // 2])
            assert abs(l[b, h] - scale * float(q[b, h] @ kl[h // 2])) < 1e-13
    assert np.all(o[2] == 0) and np.all(l[2] == -np.inf)
    for w in (2, 7, 17, 30):
        o, l = ref.decode_paged_variant(q, kp, vp, table, lens, scale, window=w)
        for b in range(2):
            t = np.arange(max(0, lens[b] - w), lens[b])
            kb, vb = _tokens(kp, table, b, t), _tokens(vp, table, b, t)
            od, ld = ref.attention(q[b][None, None], kb[None], vb[None], scale, False)
            np.testing.assert_allclose(o[b], od[0, 0], rtol=0, atol=1e-13)
            np.testing.assert_allclose(l[b], ld[0, :, 0], rtol=0, atol=1e-13)


def pin_decode_softcap(ref):
    """Logit soft-capping cap*tanh(x/cap) of the scaled scores: a two-key
    closed form worked by hand; an enormous cap is the plain decode; with
    every score huge and positive all capped scores equal cap, so the weights
    are uniform, O is the mean value row and LSE = cap + ln(len)."""
    # two keys, d = 2, one head: raw dots 3 and -1, scale 0.5, cap 2
    q = np.array([[[1.0, 0.0]]])
    kp = np.zeros((1, 16, 1, 2))
    vp = np.zeros((1, 16, 1, 2))
    kp[0, 0, 0] = [3.0, 5.0]
    kp[0, 1, 0] = [-1.0, 2.0]
    vp[0, 0, 0] = [1.0, -2.0]
    vp[0, 1, 0] = [4.0, 0.5]
    c1, c2 = 2.0 * math.tanh(0.75), 2.0 * math.tanh(-0.25)
    w1, w2 = math.exp(c1), math.exp(c2)
    o, l = ref.decode_paged_variant(q, kp, vp, np.array([[0]]), np.array([2]), 0.5,
                                    softcap=2.0)
    np.testing.assert_allclose(o[0, 0], [(w1 * 1 + w2 * 4) / (w1 + w2),
                                         (w1 * -2 + w2 * 0.5) / (w1 + w2)], rtol=1e-14)
    assert abs(l[0, 0] - math.log(w1 + w2)) < 1e-14
    rng = np.random.default_rng(32)
    lens = [45, 16, 0]
    qq, kk, vv, table, lens = _paged_case(rng, lens)
    plain = ref.decode_paged(qq, kk, vv, table, lens, 0.3)
    o, l = ref.decode_paged_variant(qq, kk, vv, table, lens, 0.3, softcap=1e9)
    np.testing.assert_allclose(o, plain[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, plain[1], rtol=0, atol=1e-12)
    # all keys aligned with the query and huge: every capped score is 5
    kk2 = np.abs(kk) + 1.0
    qh = np.full_like(qq, 1e6)
    o, l = ref.decode_paged_variant(qh, kk2, vv, table, lens, 1.0, softcap=5.0)
    for b in range(2):
        t = np.arange(lens[b])
        vb = _tokens(vv, table, b, t)
        for h in range(4):
            np.testing.assert_allclose(o[b, h], vb[:, h // 2].mean(axis=0), rtol=0, atol=1e-12)
            assert abs(l[b, h] - (5.0 + math.log(lens[b]))) < 1e-12


def pin_ragged_paged(ref):
    """Ragged queries over paged K/V == dense attention on each sequence's
    own contiguous tensors (from which the pools were built), with bottom-right
    causal alignment when q_len < kv_len; a one-query sequence equals the
    paged decode; an empty sequence owns no rows; a zero-length cache gives
    O = 0, LSE = -inf."""
    rng = np.random.default_rng(33)
    H, hkv, d, page = 4, 2, 8, 16
    q_lens = [5, 1, 0, 40, 3]
    kv_lens = [5, 33, 7, 40, 0]
    seqs = [(_rand(rng, ql, H, d), _rand(rng, kl, hkv, d), _rand(rng, kl, hkv, d))
            for ql, kl in zip(q_lens, kv_lens)]
    B = len(q_lens)
    indptr = np.concatenate([[0], np.cumsum(q_lens)])
    q = np.concatenate([sq for sq, _, _ in seqs])
    need = [-(-kl // page) for kl in kv_lens]
    n_pages = sum(need) + 4
    perm = rng.permutation(n_pages)
    max_pages = max(max(need), 1)
    table = np.full((B, max_pages), 10**6)
    kp = _rand(rng, n_pages, page, hkv, d)
    vp = _rand(rng, n_pages, page, hkv, d)
    off = 0
    for b, (_, kk, vv) in enumerate(seqs):
        for p_ in range(need[b]):
            pg = perm[off]
            off += 1
            table[b, p_] = pg
            n = min(page, kv_lens[b] - p_ * page)
            kp[pg, :n] = kk[p_ * page:p_ * page + n]
            vp[pg, :n] = vv[p_ * page:p_ * page + n]
    for causal in (False, True):
        o, l = ref.attention_ragged_paged(q, indptr, kp, vp, table, np.array(kv_lens), 0.35,
                                          causal)
        for b, (sq, kk, vv) in enumerate(seqs):
            r0, r1 = indptr[b], indptr[b + 1]
            if r1 == r0:
                continue
            if kv_lens[b] == 0:
                assert np.all(o[r0:r1] == 0) and np.all(l[r0:r1] == -np.inf)
                continue
            od, ld = ref.attention(sq[None], kk[None], vv[None], 0.35, causal)
            np.testing.assert_allclose(o[r0:r1], od[0], rtol=0, atol=1e-13)
            np.testing.assert_allclose(l[r0:r1], ld[0].T, rtol=0, atol=1e-13)
        # bottom-right: the last query row of sequence 3 sees all 40 keys, its first only key 0
        r0 = indptr[3]
        if causal:
            assert abs(l[r0, 0] - 0.35 * float(seqs[3][0][0, 0] @ seqs[3][1][0, 0])) < 1e-13
        # the one-query sequence is a decode
        od, ld = ref.decode_paged(q[indptr[1]:indptr[2]], kp, vp, table[1:2],
                                  np.array(kv_lens[1:2]), 0.35)
        np.testing.assert_allclose(o[indptr[1]], od[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l[indptr[1]], ld[0], rtol=0, atol=1e-13)


def pin_cascade(ref):
    """Cascade: dense attention over [prefix ++ own tokens] built from the
    original contiguous tensors; equal to the ragged paged attention with the
    (page-aligned) prefix pages prepended to each block table; equal to the
    merge of the prefix-only (non-causal) and suffix-only parts; prefix 0 is
    the plain ragged attention."""
    rng = np.random.default_rng(34)
    H, hkv, d, page = 4, 2, 8, 16
    P = 32                      # page-aligned shared prefix
    q_lens, kv_lens = [3, 1, 6, 0], [5, 20, 6, 4]
    B = len(q_lens)
    pk, pv = _rand(rng, P, hkv, d), _rand(rng, P, hkv, d)
    own = [(_rand(rng, ql, H, d), _rand(rng, kl, hkv, d), _rand(rng, kl, hkv, d))
           for ql, kl in zip(q_lens, kv_lens)]
    n_pages = P // page + sum(-(-kl // page) for kl in kv_lens) + 2
    perm = rng.permutation(n_pages)
    kp, vp = _rand(rng, n_pages, page, hkv, d), _rand(rng, n_pages, page, hkv, d)
    prefix_pages = perm[:P // page]
    for i, pg in enumerate(prefix_pages):
        kp[pg], vp[pg] = pk[i * page:(i + 1) * page], pv[i * page:(i + 1) * page]
    max_pages = max(-(-kl // page) for kl in kv_lens)
    table = np.full((B, max_pages), 10**6)
    nxt = P // page
    for b, (_, kk, vv) in enumerate(own):
        for p_ in range(-(-kv_lens[b] // page)):
            pg = perm[nxt]
            nxt += 1
            table[b, p_] = pg
            n = min(page, kv_lens[b] - p_ * page)
            kp[pg, :n], vp[pg, :n] = kk[p_ * page:p_ * page + n], vv[p_ * page:p_ * page + n]
    indptr = np.concatenate([[0], np.cumsum(q_lens)])
    q = np.concatenate([x for x, _, _ in own])
    lens = np.array(kv_lens)
    for causal in (False, True):
        o, l = ref.cascade_attention(q, indptr, kp, vp, prefix_pages, P, table, lens, 0.3, causal)
        for b, (sq, kk, vv) in enumerate(own):
            if q_lens[b] == 0:
                continue
            od, ld = ref.attention(sq[None], np.concatenate([pk, kk])[None],
                                   np.concatenate([pv, vv])[None], 0.3, causal)
            np.testing.assert_allclose(o[indptr[b]:indptr[b + 1]], od[0], rtol=0, atol=1e-13)
            np.testing.assert_allclose(l[indptr[b]:indptr[b + 1]], ld[0].T, rtol=0, atol=1e-13)
        full = np.concatenate([np.tile(prefix_pages, (B, 1)), table], axis=1)
        o2, l2 = ref.attention_ragged_paged(q, indptr, kp, vp, full, lens + P, 0.3, causal)
        np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l2, l, rtol=0, atol=1e-13)
        op, lp = ref.attention_ragged_paged(q, np.array([0, len(q)]), kp, vp,
                                            prefix_pages[None], np.array([P]), 0.3, False)
        os_, ls_ = ref.attention_ragged_paged(q, indptr, kp, vp, table, lens, 0.3, causal)
        R = len(q) * H
        om, lm = ref.merge_partials(np.stack([op.reshape(R, d), os_.reshape(R, d)], axis=1),
                                    np.stack([lp.reshape(R), ls_.reshape(R)], axis=1))
        np.testing.assert_allclose(om.reshape(o.shape), o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lm.reshape(l.shape), l, rtol=0, atol=1e-13)
        o0, l0 = ref.cascade_attention(q, indptr, kp, vp, prefix_pages[:0], 0, table, lens, 0.3,
                                       causal)
        np.testing.assert_allclose(o0, os_, rtol=0, atol=1e-14)
        np.testing.assert_allclose(l0, ls_, rtol=0, atol=1e-14)


def pin_merge(ref):
    """The merge rule: split partials merged == unsplit, for 1..96 splits
    (more splits than keys gives empty parts); associative; order-free;
    empty parts are the identity; no overflow at large LSE."""
    rng = np.random.default_rng(22)
    L, d = 40, 6
    qv, kv, vv = _rand(rng, d) * 4, _rand(rng, L, d), _rand(rng, L, d)
    o_full, l_full = ref.attention(qv.reshape(1, 1, 1, d), kv.reshape(1, L, 1, d),
                                   vv.reshape(1, L, 1, d), 1.0, False)
    for n in (1, 2, 3, 7, 16, 40, 64, 96):
        po, pl = ref.split_kv_partials(qv, kv, vv, 1.0, n)
        mo, ml = ref.merge_partials(po[None], pl[None])
        np.testing.assert_allclose(mo[0], o_full[0, 0, 0], rtol=0, atol=1e-13)
        assert abs(ml[0] - l_full[0, 0, 0]) <= 1e-13
        perm = rng.permutation(n)
        mo2, ml2 = ref.merge_partials(po[perm][None], pl[perm][None])
        np.testing.assert_allclose(mo2, mo, rtol=0, atol=1e-13)
        assert abs(ml2[0] - ml[0]) <= 1e-13
    po, pl = ref.split_kv_partials(qv, kv, vv, 1.0, 3)
    ab_o, ab_l = ref.merge_partials(po[None, :2], pl[None, :2])
    left_o, left_l = ref.merge_partials(np.stack([ab_o[0], po[2]])[None],
                                        np.array([ab_l[0], pl[2]])[None])
    bc_o, bc_l = ref.merge_partials(po[None, 1:], pl[None, 1:])
    right_o, right_l = ref.merge_partials(np.stack([po[0], bc_o[0]])[None],
                                          np.array([pl[0], bc_l[0]])[None])
    np.testing.assert_allclose(left_o, right_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(left_l, right_l, rtol=0, atol=1e-13)
    # empty parts, an all-empty row, and num_parts
    o3 = np.concatenate([po, np.zeros((2, d))])[None]
    l3 = np.concatenate([pl, [-np.inf, -np.inf]])[None]
    mo3, ml3 = ref.merge_partials(o3, l3)
    mo4, ml4 = ref.merge_partials(po[None], pl[None])
    np.testing.assert_allclose(mo3, mo4, rtol=0, atol=1e-15)
    mo5, ml5 = ref.merge_partials(np.zeros((1, 2, d)), np.full((1, 2), -np.inf))
    assert np.all(mo5 == 0) and ml5[0] == -np.inf
    mo6, ml6 = ref.merge_partials(o3, np.concatenate([pl, [5.0, 6.0]])[None], num_parts=[3])
    np.testing.assert_allclose(mo6, mo4, rtol=0, atol=1e-15)
    # large LSE values: the common max keeps the weights finite
    big_o, big_l = ref.merge_partials(po[None], pl[None] + 5000.0)
    np.testing.assert_allclose(big_o, mo4, rtol=0, atol=1e-12)
    assert abs(big_l[0] - (ml4[0] + 5000.0)) <= 1e-9


def pin_large_scores(ref):
    """Queries scaled by 30 and 40 (scores in the hundreds): finite results,
    O inside the range of the values, LSE >= the row max score, and agreement
    with the 50-digit brute force on a small case."""
    rng = np.random.default_rng(23)
    for mult in (30.0, 40.0):
        q = _rand(rng, 1, 64, 2, 64) * mult
        k, v = _rand(rng, 1, 64, 2, 64), _rand(rng, 1, 64, 2, 64)
        for causal in (False, True):
            o, lse = ref.attention(q, k, v, 1 / 8, causal)
            assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
            assert np.all(o <= v.max(axis=1, keepdims=True) + 1e-12)
            assert np.all(o >= v.min(axis=1, keepdims=True) - 1e-12)
            s = np.einsum("ihd,jhd->hij", q[0], k[0]) / 8
            if causal:   # key j visible to query i iff j <= i (Nq == Nk)
                s = np.where(np.arange(64)[None, :, None] >= np.arange(64)[None, None, :],
                             s, -np.inf)
            assert np.all(lse[0] >= s.max(axis=2) - 1e-12)
        qs = q[0, :4, 0, :8]
        ks, vs = k[0, :5, 0, :8], v[0, :5, 0, :8]
        o, lse = ref.attention(qs[None, :, None], ks[None, :, None], vs[None, :, None], 1.0, True)
        eo, el = _decimal_attention(qs, ks, vs, 1.0, True)
        np.testing.assert_allclose(o[0, :, 0], eo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, 0], el, rtol=0, atol=1e-11)


PINS = [pin_lab_example, pin_trace_example, pin_rescale_factor, pin_single_key,
        pin_causal_row0, pin_constant_v, pin_zero_query, pin_rows_sum_to_one,
        pin_brute_force, pin_torch_sdpa, pin_key_permutation,
        pin_gqa_equals_repeated_mha, pin_rows_subset, pin_paged_decode,
        pin_decode_window, pin_decode_softcap, pin_ragged_paged, pin_cascade, pin_merge,
        pin_large_scores]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(ref_mod)


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant must be caught by at least one pin.
# ---------------------------------------------------------------------------

def _mut_causal_flipped(m):
    m.setattr(ref_mod, "causal_visible",
              lambda qi, n, off: np.arange(n)[None, :] >= (qi[:, None] - off))


def _mut_causal_off_by_one(m):
    m.setattr(ref_mod, "causal_visible",
              lambda qi, n, off: np.arange(n)[None, :] < (qi[:, None] + off))


def _mut_causal_top_left(m):
    m.setattr(ref_mod, "causal_visible",
              lambda qi, n, off: np.arange(n)[None, :] <= qi[:, None])


def _mut_no_scale(m):
    m.setattr(ref_mod, "_scores", lambda qb, kh, scale: qb @ kh.T)


def _mut_transposed_scores(m):
    def f(qb, kh, scale):
        s = scale * (qb @ kh.T)
        if s.shape[0] == s.shape[1]:
            s = s.T.copy()
        return s
    m.setattr(ref_mod, "_scores", f)


def _mut_no_max_subtraction(m):
    orig = ref_mod._softmax_stats

    def f(s):
        mm, p, l = orig(s)
        with np.errstate(over="ignore", invalid="ignore"):
            p2 = np.exp(s)
        return mm, p2, p2.sum(axis=1)
    m.setattr(ref_mod, "_softmax_stats", f)


def _mut_lse_base2(m):
    def f(mm, l):
        with np.errstate(divide="ignore"):
            return np.where(l > 0, mm + np.log2(l), -np.inf)
    m.setattr(ref_mod, "_lse_from_stats", f)


def _mut_lse_without_max(m):
    def f(mm, l):
        with np.errstate(divide="ignore"):
            return np.where(l > 0, np.log(l), -np.inf)
    m.setattr(ref_mod, "_lse_from_stats", f)


def _mut_dropped_sum_term(m):
    orig = ref_mod._softmax_stats

    def f(s):
        mm, p, l = orig(s)
        return mm, p, l - p[:, 0] if p.shape[1] > 1 else l
    m.setattr(ref_mod, "_softmax_stats", f)


def _mut_gqa_modulo(m):
    orig = ref_mod.attention

    def f(q, k, v, scale, causal, rows=None, block_rows=512, threads=None):
        q = np.asarray(q, float)
        H, hkv = q.shape[2], np.asarray(k).shape[2]
        idx = np.arange(H) % hkv
        return orig(q, np.asarray(k)[:, :, idx], np.asarray(v)[:, :, idx], scale, causal,
                    rows, block_rows, threads)
    m.setattr(ref_mod, "attention", f)


def _mut_merge_sign(m):
    def f(ls, M):
        w = np.exp(np.where(np.isfinite(ls), M - ls, 0.0))
        w[~np.isfinite(ls)] = 0.0
        return w
    m.setattr(ref_mod, "_merge_weights", f)


def _mut_merge_no_weights(m):
    def f(ls, M):
        return np.isfinite(ls).astype(float)
    m.setattr(ref_mod, "_merge_weights", f)


def _mut_online_no_rescale(m):
    # the running sums are never rescaled when the maximum grows
    m.setattr(ref_mod, "_rescale_factor", lambda m_old, m_new: 0.0 if m_old == -np.inf else 1.0)


def _mut_page_slot(m):
    def f(pool, block_table, seq_len, b):
        page = pool.shape[1]
        t = np.arange(int(seq_len))
        return np.asarray(pool[np.asarray(block_table)[b, t // page], (t + 1) % page], float)
    m.setattr(ref_mod, "gather_paged_kv", f)


def _mut_window_off_by_one(m):
    m.setattr(ref_mod, "_window_start",
              lambda L, w: L - w + 1 if (w > 0 and L > w) else 0)


def _mut_window_oldest(m):
    m.setattr(ref_mod, "_window_start", lambda L, w: 0)


def _mut_softcap_unscaled(m):
    m.setattr(ref_mod, "_soft_cap", lambda x, cap: np.tanh(x / cap))


def _mut_softcap_no_tanh(m):
    m.setattr(ref_mod, "_soft_cap", lambda x, cap: np.clip(x, -cap, cap))


def _mut_ragged_rows_shifted(m):
    m.setattr(ref_mod, "_seq_rows", lambda ind, b: (int(ind[b]) + (b > 0), int(ind[b + 1])))


def _mut_cascade_prefix_last(m):
    m.setattr(ref_mod, "_concat_keys", lambda prefix, own: np.concatenate([own, prefix], axis=0))


MUTANTS = [_mut_cascade_prefix_last, _mut_ragged_rows_shifted, _mut_window_off_by_one, _mut_window_oldest, _mut_softcap_unscaled,
           _mut_softcap_no_tanh, _mut_causal_flipped, _mut_causal_off_by_one, _mut_causal_top_left,
           _mut_no_scale, _mut_transposed_scores, _mut_no_max_subtraction,
           _mut_lse_base2, _mut_lse_without_max, _mut_dropped_sum_term, _mut_gqa_modulo,
           _mut_merge_sign, _mut_merge_no_weights,
           _mut_online_no_rescale, _mut_page_slot]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__[5:])
def test_planted_mistake_is_caught(mutant, monkeypatch):
    mutant(monkeypatch)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(ref_mod)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught {mutant.__name__}"
