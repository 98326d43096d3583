"""Tensors past 2^31 bytes: the kernels address K/V tiles and pages by 32-bit
byte offsets (below 2^32, since the API limits a tensor to 2^31 elements) and
64-bit bases, and must find the far end of such tensors.

Dense: K and V of just under 2^31 elements (4 GiB each) with structured
contents whose attention output has a closed form. Head 0 has all scores 0, so
every row is the mean of the visible V rows, which step up by one every 2^20
keys (the sums stay exact in fp32). Head 1 has one key, the very last, with a
score of 16 sqrt(128) and all others 0, so the row that sees it returns its V
row and LSE equals that score.

Paged: a ragged batch whose pages sit at the top of a pool of just under 2^31
elements must give, bit for bit, what the same batch gives from a compact
pool; the compact run is checked against the float64 oracle.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_11_amd as fa
from exact_tiled_attention_11_amd import inputs
import oracle
from parity_utils import assert_lowp_acc, assert_lse, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"
ELEMS_MAX = (1 << 31) - 1


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dense_big():
    Hkv, d, Nq = 2, 128, 64
    Nk = ELEMS_MAX // (Hkv * d)            # 8,388,607 keys: 2^31 - 256 elements
    say(f"large dense: Nk={Nk}, K/V {Nk * Hkv * d * 2 / 2**30:.2f} GiB each")
    k = torch.zeros((1, Nk, Hkv, d), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((1, Nk, Hkv, d), dtype=torch.bfloat16, device=DEV)
    step = (torch.arange(Nk, device=DEV) >> 20).to(torch.bfloat16)
    v[0, :, 0, :] = step[:, None]
    k[0, Nk - 1, 1, :] = 16.0
    v_last = torch.arange(d, device=DEV, dtype=torch.float32) / 16
    v[0, Nk - 1, 1, :] = v_last.to(torch.bfloat16)
    q = torch.ones((1, Nq, Hkv, d), dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    yield dict(q=q, k=k, v=v, Nk=Nk, Nq=Nq, d=d, v_last=v_last.double().cpu().numpy())
    del q, k, v
    torch.cuda.empty_cache()


def expected_dense(Nk, Nq, d, v_last, causal):
    """Closed-form O [Nq, 2, d] and LSE [2, Nq] (float64)."""
    s_last = 16.0 * math.sqrt(d)            # scale 1/sqrt(d) times q.k = 16 d
    o = np.zeros((Nq, 2, d))
    lse = np.zeros((2, Nq))
    for i in range(Nq):
        n_vis = Nk - (Nq - 1 - i) if causal else Nk   # keys 0 .. n_vis - 1
        full, rest = divmod(n_vis, 1 << 20)
        total = (1 << 20) * full * (full - 1) / 2 + full * rest
        o[i, 0, :] = total / n_vis
        lse[0, i] = math.log(n_vis)
        if n_vis == Nk:                     # sees the last key
            o[i, 1, :] = v_last
            lse[1, i] = s_last + math.log1p((Nk - 1) * math.exp(-s_last))
        else:
            lse[1, i] = math.log(n_vis)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_dense_tensors_past_2_31_bytes(dense_big, causal):
    t = dense_big
    say(f"large dense causal={causal}: fa_forward")
    o, l = fa.forward(t["q"], t["k"], t["v"], causal=causal, out_dtype=torch.float32)
    o16, l16 = fa.forward(t["q"], t["k"], t["v"], causal=causal)
    torch.cuda.synchronize()
    eo, el = expected_dense(t["Nk"], t["Nq"], t["d"], t["v_last"], causal)
    go = np64(o)[0]
    gl = np64(l)[0]
    assert np.abs(go - eo).max() <= 1e-5 * max(1.0, np.abs(eo).max()), np.abs(go - eo).max()
    assert np.abs(gl - el).max() <= 1e-4, np.abs(gl - el).max()
    assert torch.equal(l16, l)
    assert torch.equal(o16, o.to(torch.bfloat16))


@pytest.fixture(scope="module")
def paged_big():
    H, Hkv, d = 32, 8, 128
    page_elems = 16 * Hkv * d
    big = ELEMS_MAX // page_elems           # 131,071 pages: 2^31 - 2^14 elements
    q_lens, kv_lens = [300, 1, 700, 1], [5000, 3000, 700, 9000]
    ri = inputs.ragged_paged_inputs(q_lens, kv_lens, H, Hkv, d, seed=71,
                                    dtype=torch.bfloat16, unreferenced="normal")
    pc = ri.k_pool.shape[0]
    say(f"large paged: pool of {big} pages ({big * page_elems * 2 / 2**30:.2f} GiB per "
        f"tensor), the batch's {pc} pages at its top")
    kb = torch.zeros((big, 16, Hkv, d), dtype=torch.bfloat16, device=DEV)
    vb = torch.zeros((big, 16, Hkv, d), dtype=torch.bfloat16, device=DEV)
    # compact page c -> big page big - 1 - c
    kb[big - pc:] = ri.k_pool.flip(0).to(DEV)
    vb[big - pc:] = ri.v_pool.flip(0).to(DEV)
    table = ri.block_table.clone()
    valid = (table >= 0) & (table < pc)
    table_big = torch.where(valid, big - 1 - table, torch.full_like(table, big - 1))
    torch.cuda.synchronize()
    compact = dict(q=ri.q.to(DEV), indptr=ri.qo_indptr.to(DEV), k=ri.k_pool.to(DEV),
                   v=ri.v_pool.to(DEV), t=ri.block_table.to(DEV), s=ri.kv_lens.to(DEV))
    bigd = dict(compact, k=kb, v=vb, t=table_big.to(DEV))
    yield dict(ri=ri, compact=compact, big=bigd, H=H, d=d, q_lens=q_lens)
    del kb, vb, compact, bigd
    torch.cuda.empty_cache()


def run_paged(x, ri, causal):
    o, l = fa.forward_paged(x["q"], x["indptr"], x["k"], x["v"], x["t"], x["s"], ri.max_q_len,
                            causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return o, l


@pytest.mark.parametrize("causal", [False, True])
def test_paged_pool_past_2_31_bytes(paged_big, causal):
    p, ri = paged_big, paged_big["ri"]
    say(f"large paged causal={causal}: compact pool, then the top of the large pool")
    oc, lc = run_paged(p["compact"], ri, causal)
    ob, lb = run_paged(p["big"], ri, causal)
    assert torch.equal(ob, oc) and torch.equal(lb, lc)
    ro, rl = oracle.attention_ragged_paged(ri.q, ri.qo_indptr, ri.k_pool, ri.v_pool,
                                           ri.block_table, ri.kv_lens, 1 / math.sqrt(p["d"]),
                                           causal)
    assert_lowp_acc(f"large paged causal={causal}", np64(oc), ro)
    assert_lse(f"large paged causal={causal}", np64(lc), rl)


def test_decode_pool_past_2_31_bytes(paged_big):
    p, ri = paged_big, paged_big["ri"]
    rows = [int(ri.qo_indptr[b]) for b in range(len(p["q_lens"]))]
    q = ri.q[rows].contiguous().to(DEV)
    say("large decode: compact pool, then the top of the large pool")
    for splits in (0, 1, 7):
        oc, lc = fa.decode_paged(q, p["compact"]["k"], p["compact"]["v"], p["compact"]["t"],
                                 p["compact"]["s"], num_splits=splits, out_dtype=torch.float32)
        ob, lb = fa.decode_paged(q, p["big"]["k"], p["big"]["v"], p["big"]["t"], p["big"]["s"],
                                 num_splits=splits, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(ob, oc) and torch.equal(lb, lc), splits
