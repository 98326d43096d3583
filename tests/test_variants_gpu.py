"""Parity of the decode variants (sliding window, logit soft-capping) with the
float64 oracle, through the C ABI.

Every case prints what it runs before touching the GPU. Tokens outside the
window hold NaN and their block-table entries point outside the pool: the
kernels must never use them.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_11_amd as fa
from exact_tiled_attention_11_amd import inputs
import oracle
from parity_utils import assert_lowp_acc, assert_lowp_out, assert_lse, assert_rounded_from, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = inputs.TORCH_DTYPES


def say(*a):
    print(*a, flush=True)


def hide_outside_window(pi, lens, window):
    """NaN in every token slot before each sequence's window; table entries of
    pages wholly before the window point outside the pool."""
    n_pages = pi.k_pool.shape[0]
    for b, L in enumerate(lens):
        first = L - window if (window > 0 and L > window) else 0
        for t0 in range(0, first, 16):
            pg = int(pi.block_table[b, t0 // 16])
            hi = min(16, first - t0)
            pi.k_pool[pg, :hi] = float("nan")
            pi.v_pool[pg, :hi] = float("nan")
        for p in range(first // 16):
            pi.block_table[b, p] = n_pages + 7


def to_dev(pi):
    return dict(q=pi.q.to(DEV), k=pi.k_pool.to(DEV), v=pi.v_pool.to(DEV),
                t=pi.block_table.to(DEV), s=pi.seq_lens.to(DEV))


def gpu_decode_ex(d, window, softcap, splits, out_dtype=None):
    say(f"  fa_decode_paged_ex B={d['q'].shape[0]} window={window} softcap={softcap} "
        f"splits={splits} out={out_dtype}")
    o, l = fa.decode_paged_ex(d["q"], d["k"], d["v"], d["t"], d["s"], window=window,
                              softcap=softcap, num_splits=splits, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, l


VAR = [
    # (H, Hkv, d, dtype, lens)
    (8, 8, 128, "bf16", [1, 15, 16, 17, 31, 33, 0, 300]),
    (8, 4, 64, "f16", [0, 1, 100, 2048, 2049, 5000]),
    (32, 8, 128, "bf16", [1, 2047, 4097, 9000, 16, 300]),
]
WINDOWS = [1, 16, 17, 100, 4096]


@pytest.mark.parametrize("case", VAR, ids=[f"h{c[0]}/{c[1]}-d{c[2]}-{c[3]}" for c in VAR])
@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("splits", [0, 1, 3, 16])
def test_decode_window(case, window, splits):
    H, Hkv, d, dt, lens = case
    pi = inputs.paged_decode_inputs(len(lens), H, Hkv, d, lens, seed=41, dtype=TD[dt])
    ro, rl = oracle.decode_paged_variant(pi.q, pi.k_pool, pi.v_pool, pi.block_table,
                                         pi.seq_lens, 1 / math.sqrt(d), window=window)
    hide_outside_window(pi, lens, window)
    say(f"decode window {case} window={window} splits={splits}")
    dev = to_dev(pi)
    o32, l32 = gpu_decode_ex(dev, window, 0.0, splits, torch.float32)
    o16, l16 = gpu_decode_ex(dev, window, 0.0, splits)
    assert_lowp_acc(f"win {case} {window}", np64(o32), ro)
    assert_lse(f"win {case} {window}", np64(l32), rl)
    assert_rounded_from(f"win {case} {window}", o16, o32)
    assert torch.equal(l16, l32)


SOFTCAP = [(5.0, 0, 1.0), (30.0, 0, 30.0), (30.0, 100, 30.0), (50.0, 4096, 8.0)]


@pytest.mark.parametrize("case", VAR, ids=[f"h{c[0]}/{c[1]}-d{c[2]}-{c[3]}" for c in VAR])
@pytest.mark.parametrize("cap,window,qs", SOFTCAP, ids=[f"cap{c}-w{w}-q{q}" for c, w, q in SOFTCAP])
@pytest.mark.parametrize("splits", [0, 3])
def test_decode_softcap(case, cap, window, qs, splits):
    H, Hkv, d, dt, lens = case
    pi = inputs.paged_decode_inputs(len(lens), H, Hkv, d, lens, seed=42, dtype=TD[dt])
    pi.q = (pi.q.float() * qs).to(pi.q.dtype)   # sharper scores so the cap matters
    ro, rl = oracle.decode_paged_variant(pi.q, pi.k_pool, pi.v_pool, pi.block_table,
                                         pi.seq_lens, 1 / math.sqrt(d), window=window,
                                         softcap=cap)
    hide_outside_window(pi, lens, window)
    say(f"decode softcap {case} cap={cap} window={window} qscale={qs} splits={splits}")
    dev = to_dev(pi)
    o32, l32 = gpu_decode_ex(dev, window, cap, splits, torch.float32)
    o16, _ = gpu_decode_ex(dev, window, cap, splits)
    assert_lowp_acc(f"cap {case} {cap}", np64(o32), ro)
    assert_lse(f"cap {case} {cap}", np64(l32), rl)
    assert_rounded_from(f"cap {case} {cap}", o16, o32)


def test_decode_ex_defaults_equal_plain_decode():
    lens = [3000, 17, 4096, 1, 0, 777]
    pi = inputs.paged_decode_inputs(len(lens), 32, 8, 128, lens, seed=43)
    dev = to_dev(pi)
    say("decode_ex defaults vs decode")
    for splits in (0, 1, 5):
        a = fa.decode_paged(dev["q"], dev["k"], dev["v"], dev["t"], dev["s"], num_splits=splits)
        b = fa.decode_paged_ex(dev["q"], dev["k"], dev["v"], dev["t"], dev["s"],
                               num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_window_softcap_b64_h32_kv8():
    """The paged-decode workload with a 4096-token window and cap 50."""
    p = inputs.WORKLOADS["paged_decode_bf16_b64_h32_kv8"].params
    lens = inputs.uniform_lengths(p["B"], p["len_lo"], p["len_hi"], p["seed"])
    pi = inputs.paged_decode_inputs(p["B"], p["H"], p["Hkv"], p["d"], lens, p["seed"],
                                    pool_factor=p["pool_factor"], max_pages=p["len_hi"] // 16)
    say("c4 window 4096 cap 50: oracle on all 64 sequences")
    ro, rl = oracle.decode_paged_variant(pi.q, pi.k_pool, pi.v_pool, pi.block_table,
                                         pi.seq_lens, 1 / math.sqrt(128), window=4096,
                                         softcap=50.0)
    dev = to_dev(pi)
    for splits in (0, 16, 64):
        o32, l32 = gpu_decode_ex(dev, 4096, 50.0, splits, torch.float32)
        o16, _ = gpu_decode_ex(dev, 4096, 50.0, splits)
        assert_lowp_acc("c4 win/cap", np64(o32), ro)
        assert_lowp_out("c4 win/cap", o16, ro)
        assert_lse("c4 win/cap", np64(l32), rl)
        assert_rounded_from("c4 win/cap", o16, o32)


# ---------------------------------------------------------------------------
# The decode step recorded as a HIP graph.
# ---------------------------------------------------------------------------

GRAPH = [
    # (H, Hkv, d, dtype, lens, window, softcap, splits)
    (32, 8, 128, "bf16", [1, 2047, 4097, 9000, 16, 300], 0, 0.0, 0),
    (32, 8, 128, "bf16", [1, 2047, 4097, 9000, 16, 300], 0, 0.0, 1),
    (8, 4, 64, "f16", [0, 1, 100, 2048, 2049, 5000], 1000, 30.0, 0),
]


@pytest.mark.parametrize("case", GRAPH, ids=[f"d{c[2]}-{c[3]}-w{c[5]}-cap{c[6]}-s{c[7]}"
                                            for c in GRAPH])
def test_decode_graph_replays_match_eager(case):
    H, Hkv, d, dt, lens, window, cap, splits = case
    B = len(lens)
    pi = inputs.paged_decode_inputs(B, H, Hkv, d, lens, seed=44, dtype=TD[dt],
                                    unreferenced="normal")
    dev = to_dev(pi)
    say(f"decode graph {case}: create")
    g = fa.DecodeGraph(dev["q"], dev["k"], dev["v"], dev["t"], dev["s"], window=window,
                       softcap=cap, num_splits=splits, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(45)
    for it in range(4):
        # a new step: new queries and shorter sequences, written into the bound buffers
        qn = torch.from_numpy(rng.standard_normal(tuple(dev["q"].shape)).astype(np.float32))
        dev["q"].copy_(qn.to(dev["q"].dtype))
        new_lens = torch.as_tensor([max(0, L - 7 * it) for L in lens], dtype=torch.int32)
        dev["s"].copy_(new_lens)
        torch.cuda.synchronize()
        say(f"  replay {it}: eager reference, then graph")
        eo, el = fa.decode_paged_ex(dev["q"], dev["k"], dev["v"], dev["t"], dev["s"],
                                    window=window, softcap=cap, num_splits=splits,
                                    out_dtype=torch.float32)
        torch.cuda.synchronize()
        go, gl = g.launch()
        torch.cuda.synchronize()
        assert torch.equal(go, eo) and torch.equal(gl, el), f"replay {it} differs from eager"
        if it == 3:
            ro, rl = oracle.decode_paged_variant(dev["q"].cpu(), pi.k_pool, pi.v_pool,
                                                 pi.block_table, new_lens, 1 / math.sqrt(d),
                                                 window=window, softcap=cap)
            assert_lowp_acc("graph", np64(go), ro)
            assert_lse("graph", np64(gl), rl)
    g.close()


# ---------------------------------------------------------------------------
# Ragged queries over a paged cache (fa_forward_paged).
# ---------------------------------------------------------------------------

def gpu_forward_paged(ri, causal, out_dtype=None, max_q_len=None):
    say(f"  fa_forward_paged total_q={ri.q.shape[0]} B={ri.kv_lens.shape[0]} causal={causal} "
        f"out={out_dtype}")
    o, l = fa.forward_paged(ri.q.to(DEV), ri.qo_indptr.to(DEV), ri.k_pool.to(DEV),
                            ri.v_pool.to(DEV), ri.block_table.to(DEV), ri.kv_lens.to(DEV),
                            ri.max_q_len if max_q_len is None else max_q_len, causal=causal,
                            out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, l


RAGGED = [
    # (H, Hkv, d, dtype, q_lens, kv_lens)
    (8, 2, 128, "bf16", [1, 1, 17, 300, 100, 0, 513, 7, 64],
     [1, 3000, 17, 300, 2100, 50, 513, 0, 64]),
    (8, 8, 64, "f16", [33, 1, 256, 257, 5], [33, 4097, 1000, 257, 700]),
    (32, 8, 128, "bf16", [1000, 1, 1, 2048], [1000, 5000, 1, 2500]),
]


@pytest.mark.parametrize("case", RAGGED, ids=[f"h{c[0]}/{c[1]}-d{c[2]}-{c[3]}-b{len(c[4])}"
                                             for c in RAGGED])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_paged_mixed_batch(case, causal):
    H, Hkv, d, dt, q_lens, kv_lens = case
    ri = inputs.ragged_paged_inputs(q_lens, kv_lens, H, Hkv, d, seed=51, dtype=TD[dt])
    # token slots past each sequence's end hold NaN: they must never be used
    for b, L in enumerate(kv_lens):
        if L % 16:
            pg = int(ri.block_table[b, L // 16])
            ri.k_pool[pg, L % 16:] = float("nan")
            ri.v_pool[pg, L % 16:] = float("nan")
    say(f"forward_paged {case} causal={causal}: oracle")
    ro, rl = oracle.attention_ragged_paged(ri.q, ri.qo_indptr, ri.k_pool, ri.v_pool,
                                           ri.block_table, ri.kv_lens, 1 / math.sqrt(d), causal)
    o32, l32 = gpu_forward_paged(ri, causal, torch.float32)
    o16, l16 = gpu_forward_paged(ri, causal)
    assert_lowp_acc(f"ragged {case}", np64(o32), ro)
    assert_lse(f"ragged {case}", np64(l32), rl)
    assert_rounded_from(f"ragged {case}", o16, o32)
    assert torch.equal(l16, l32)


def test_forward_paged_equals_dense_forward():
    """Contiguous pages in sequence order hold the dense K/V: the paged kernel
    gives the dense kernel's results bit for bit."""
    B, N, H, Hkv, d = 2, 1000, 8, 2, 128
    q, k, v = inputs.prefill_inputs(B, H, Hkv, N, N, d, torch.bfloat16, seed=52)
    pages = -(-N // 16)
    kp = torch.zeros((B * pages, 16, Hkv, d), dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    kp.view(B, pages * 16, Hkv, d)[:, :N] = k
    vp.view(B, pages * 16, Hkv, d)[:, :N] = v
    table = torch.arange(B * pages, dtype=torch.int32).reshape(B, pages)
    ri = inputs.RaggedPagedInputs(q.reshape(B * N, H, d).contiguous(),
                                  torch.tensor([0, N, 2 * N], dtype=torch.int32), kp, vp, table,
                                  torch.tensor([N, N], dtype=torch.int32), N)
    for causal in (False, True):
        say(f"forward_paged vs forward causal={causal}")
        od, ld = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
        op, lp = gpu_forward_paged(ri, causal)
        assert torch.equal(op.reshape(B, N, H, d), od)
        assert torch.equal(lp.reshape(B, N, H).permute(0, 2, 1), ld)


def test_forward_paged_contract_violations_give_nan():
    q_lens, kv_lens = [19, 19, 19, 20, 19], [100, 100, 100, 100, 100]
    ri = inputs.ragged_paged_inputs(q_lens, kv_lens, 8, 2, 128, seed=53)
    n_pages = ri.k_pool.shape[0]
    ri.block_table[1, 2] = n_pages          # page id outside the pool
    ri.kv_lens[2] = 10_000                  # longer than the block table allows
    ri.block_table[4, 5] = -7               # negative page id
    say("forward_paged contract violations")
    for causal in (False, True):
        # sequence 3 is longer than max_q_len = 19
        o, l = gpu_forward_paged(ri, causal, torch.float32, max_q_len=19)
        assert torch.isfinite(o[:19]).all() and torch.isfinite(l[:19]).all()
        for b in (1, 2, 3, 4):
            r0, r1 = int(ri.qo_indptr[b]), int(ri.qo_indptr[b + 1])
            assert torch.isnan(o[r0:r1]).all() and torch.isnan(l[r0:r1]).all()


def test_forward_paged_single_query_rows_are_the_decode():
    """One-query sequences of a ragged batch are computed by the decode
    kernel: bit for bit what fa_decode_paged gives for them with one chunk,
    and the other sequences as before."""
    q_lens, kv_lens = [1, 300, 1, 1, 2, 1], [4100, 300, 1, 0, 900, 77]
    H, Hkv, d = 32, 8, 128
    ri = inputs.ragged_paged_inputs(q_lens, kv_lens, H, Hkv, d, seed=54)
    for causal in (False, True):
        say(f"forward_paged one-query rows causal={causal}")
        o, l = gpu_forward_paged(ri, causal, torch.float32)
        rows = [int(ri.qo_indptr[b]) for b in range(len(q_lens)) if q_lens[b] == 1]
        seqs = [b for b in range(len(q_lens)) if q_lens[b] == 1]
        od, ld = fa.decode_paged(ri.q[rows].contiguous().to(DEV), ri.k_pool.to(DEV),
                                 ri.v_pool.to(DEV), ri.block_table[seqs].contiguous().to(DEV),
                                 ri.kv_lens[seqs].contiguous().to(DEV), num_splits=1,
                                 out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o[rows], od) and torch.equal(l[rows], ld)
        ro, rl = oracle.attention_ragged_paged(ri.q, ri.qo_indptr, ri.k_pool, ri.v_pool,
                                               ri.block_table, ri.kv_lens, 1 / math.sqrt(d),
                                               causal)
        assert_lowp_acc("one-query rows", np64(o), ro)
        assert_lse("one-query rows", np64(l), rl)


def test_forward_paged_graph_replays_match_eager():
    """A ragged batch with one-query sequences (two launches: the decode
    kernel for those rows, then the tiled kernel) recorded into a graph:
    every replay, with new queries written in between, equals an eager call
    bit for bit."""
    q_lens, kv_lens = [1, 300, 1, 1, 700, 1], [4100, 300, 1, 2000, 900, 77]
    H, Hkv, d = 32, 8, 128
    ri = inputs.ragged_paged_inputs(q_lens, kv_lens, H, Hkv, d, seed=56)
    args = [t.to(DEV) for t in (ri.q, ri.qo_indptr, ri.k_pool, ri.v_pool, ri.block_table,
                                ri.kv_lens)]
    o = torch.empty(tuple(ri.q.shape), dtype=torch.float32, device=DEV)
    lse = torch.empty((ri.q.shape[0], H), dtype=torch.float32, device=DEV)
    say("forward_paged graph: eager warm-up, capture")
    fa.forward_paged(*args, ri.max_q_len, causal=True, out_dtype=torch.float32, out=o, lse=lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.forward_paged(*args, ri.max_q_len, causal=True, out_dtype=torch.float32, out=o,
                         lse=lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(57)
    for it in range(4):
        qn = torch.from_numpy(rng.standard_normal(tuple(ri.q.shape)).astype(np.float32))
        args[0].copy_(qn.to(args[0].dtype))
        torch.cuda.synchronize()
        say(f"  replay {it}: eager reference, then graph")
        eo, el = fa.forward_paged(*args, ri.max_q_len, causal=True, out_dtype=torch.float32)
        torch.cuda.synchronize()
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eo) and torch.equal(lse, el), f"replay {it} differs from eager"
    ro, rl = oracle.attention_ragged_paged(args[0].cpu(), ri.qo_indptr, ri.k_pool, ri.v_pool,
                                           ri.block_table, ri.kv_lens, 1 / math.sqrt(d), True)
    assert_lowp_acc("forward_paged graph", np64(o), ro)
    assert_lse("forward_paged graph", np64(lse), rl)
    del g


def test_forward_paged_single_query_contract_violations_give_nan():
    q_lens, kv_lens = [1, 1, 1, 1, 3], [100, 100, 100, 100, 100]
    ri = inputs.ragged_paged_inputs(q_lens, kv_lens, 8, 2, 128, seed=55)
    ri.block_table[1, 3] = ri.k_pool.shape[0]   # page id outside the pool
    ri.kv_lens[2] = 10_000                      # longer than the block table allows
    ri.kv_lens[3] = -5
    say("forward_paged one-query contract violations")
    for causal in (False, True):
        o, l = gpu_forward_paged(ri, causal, torch.float32)
        assert torch.isfinite(o[0]).all() and torch.isfinite(l[0]).all()
        assert torch.isfinite(o[4:]).all() and torch.isfinite(l[4:]).all()
        for r in (1, 2, 3):
            assert torch.isnan(o[r]).all() and torch.isnan(l[r]).all()


# ---------------------------------------------------------------------------
# Cascade: a shared prefix attended once, merged with each sequence's suffix.
# ---------------------------------------------------------------------------

def cascade_case(prefix_len, q_lens, kv_lens, H, Hkv, d, dt, seed):
    """Ragged inputs whose pool also holds a shared prefix of prefix_len tokens
    in pages of its own; token slots after the prefix's last token hold NaN."""
    ri = inputs.ragged_paged_inputs(q_lens, kv_lens, H, Hkv, d, seed=seed, dtype=TD[dt],
                                    unreferenced="nan")
    n_pre = -(-prefix_len // 16)
    extra = inputs.normal((n_pre, 16, Hkv, d), seed * 7 + 1, TD[dt])
    extra_v = inputs.normal((n_pre, 16, Hkv, d), seed * 7 + 2, TD[dt])
    perm = np.random.default_rng(seed).permutation(n_pre)
    if prefix_len % 16:   # the page holding the prefix's last token
        extra[perm[-1], prefix_len % 16:] = float("nan")
        extra_v[perm[-1], prefix_len % 16:] = float("nan")
    base = ri.k_pool.shape[0]
    ri.k_pool = torch.cat([ri.k_pool, extra])
    ri.v_pool = torch.cat([ri.v_pool, extra_v])
    prefix_pages = torch.from_numpy((base + perm).astype(np.int32))
    for b, L in enumerate(kv_lens):
        if L % 16:
            pg = int(ri.block_table[b, L // 16])
            ri.k_pool[pg, L % 16:] = float("nan")
            ri.v_pool[pg, L % 16:] = float("nan")
    return ri, prefix_pages


def gpu_cascade(ri, prefix_pages, prefix_len, causal, splits=0, out_dtype=None):
    say(f"  fa_cascade total_q={ri.q.shape[0]} prefix={prefix_len} splits={splits} "
        f"causal={causal} out={out_dtype}")
    o, l = fa.cascade(ri.q.to(DEV), ri.qo_indptr.to(DEV), ri.k_pool.to(DEV), ri.v_pool.to(DEV),
                      prefix_pages.to(DEV), prefix_len, ri.block_table.to(DEV),
                      ri.kv_lens.to(DEV), ri.max_q_len, causal=causal, prefix_splits=splits,
                      out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, l


CASCADE = [
    # (prefix_len, H, Hkv, d, dtype, q_lens, kv_lens)
    (16, 8, 2, 128, "bf16", [1, 1, 5, 40], [1, 300, 5, 100]),
    (1000, 8, 8, 64, "f16", [1, 17, 1, 0], [2049, 17, 60, 9]),
    (5000, 32, 8, 128, "bf16", [1] * 12 + [300], [100 * (i + 1) for i in range(12)] + [300]),
]


@pytest.mark.parametrize("case", CASCADE, ids=[f"p{c[0]}-h{c[1]}/{c[2]}-d{c[3]}-{c[4]}"
                                              for c in CASCADE])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [0, 1, 7])
def test_cascade(case, causal, splits):
    P, H, Hkv, d, dt, q_lens, kv_lens = case
    ri, pp = cascade_case(P, q_lens, kv_lens, H, Hkv, d, dt, seed=71)
    say(f"cascade {case} causal={causal} splits={splits}: oracle")
    ro, rl = oracle.cascade_attention(ri.q, ri.qo_indptr, ri.k_pool, ri.v_pool, pp, P,
                                      ri.block_table, ri.kv_lens, 1 / math.sqrt(d), causal)
    o32, l32 = gpu_cascade(ri, pp, P, causal, splits, torch.float32)
    o16, l16 = gpu_cascade(ri, pp, P, causal, splits)
    assert_lowp_acc(f"cascade {case}", np64(o32), ro)
    assert_lse(f"cascade {case}", np64(l32), rl)
    assert_rounded_from(f"cascade {case}", o16, o32)
    assert torch.equal(l16, l32)


def test_cascade_without_prefix_is_forward_paged():
    ri, pp = cascade_case(0, [1, 7, 300], [500, 7, 300], 8, 2, 128, "bf16", seed=72)
    for causal in (False, True):
        say(f"cascade prefix 0 vs forward_paged causal={causal}")
        a = gpu_cascade(ri, pp, 0, causal)
        b = gpu_forward_paged(ri, causal)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_cascade_bad_prefix_page_gives_nan():
    ri, pp = cascade_case(64, [1, 3], [40, 40], 8, 2, 128, "bf16", seed=73)
    pp[1] = ri.k_pool.shape[0] + 3           # outside the pool
    say("cascade bad prefix page")
    o, l = gpu_cascade(ri, pp, 64, True, 0, torch.float32)
    assert torch.isnan(o).all() and torch.isnan(l).all()
