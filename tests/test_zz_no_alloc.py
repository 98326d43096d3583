"""fa_decode_paged_noalloc against fa_decode_paged_ex through the C ABI.

The no-allocation entry point runs the same kernels with the partials in the
library's own per-device buffer instead of a caller workspace, so its outputs
must equal the workspace entry point's bit for bit (and hence meet the oracle
bounds that entry point's parity tests establish). Two calls in a row, the
second smaller than the first, show that the buffer's leftover contents from
one call never leak into the next.
"""

import ctypes
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
BF16 = 2


def say(*a):
    print(*a, flush=True)


def to_dev(pi):
    return dict(q=pi.q.to(DEV), k=pi.k_pool.to(DEV), v=pi.v_pool.to(DEV),
                t=pi.block_table.to(DEV), s=pi.seq_lens.to(DEV))


def call_both(d, window, softcap, splits, out_dtype):
    """The same decode through fa_decode_paged_ex (torch workspace) and through
    fa_decode_paged_noalloc with preallocated outputs."""
    B, H, hd = d["q"].shape
    e_o, e_l = fa.decode_paged_ex(d["q"], d["k"], d["v"], d["t"], d["s"], window=window,
                                  softcap=softcap, num_splits=splits, out_dtype=out_dtype)
    n_o = torch.full((B, H, hd), float("nan"), dtype=out_dtype, device=DEV)
    n_l = torch.full((B, H), float("nan"), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    r = fa.decode_paged_noalloc(d["q"], d["k"], d["v"], d["t"], d["s"], window=window,
                                softcap=softcap, num_splits=splits, out_dtype=out_dtype,
                                out=n_o, lse=n_l)
    torch.cuda.synchronize()
    assert r[0] is n_o and r[1] is n_l
    return (e_o, e_l), (n_o, n_l)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_equals_workspace_decode_twice_shrinking(out_dtype):
    # first call: 24 sequences up to 12000 tokens, 32/8 heads, automatic splits
    lens1 = inputs.uniform_lengths(24, 1, 12000, 201)
    pi1 = inputs.paged_decode_inputs(24, 32, 8, 128, lens1, seed=202)
    say(f"noalloc call 1: B=24 h32/kv8 d128 auto splits out={out_dtype}")
    d1 = to_dev(pi1)
    (eo, el), (no, nl) = call_both(d1, 0, 0.0, 0, out_dtype)
    assert torch.equal(no, eo) and torch.equal(nl, el)
    if out_dtype == torch.float32:
        ro, rl = oracle.decode_paged(pi1.q, pi1.k_pool, pi1.v_pool, pi1.block_table,
                                     pi1.seq_lens, 1 / math.sqrt(128))
        assert_lowp_acc("noalloc call 1", np64(no), ro)
        assert_lse("noalloc call 1", np64(nl), rl)
    # second call, right after: fewer and shorter sequences, other heads, a
    # window and a soft cap, a fixed split count; the buffer still holds the
    # first call's partials
    lens2 = [5, 700, 4000]
    pi2 = inputs.paged_decode_inputs(3, 12, 2, 64, lens2, seed=203)
    say(f"noalloc call 2: B=3 h12/kv2 d64 window 1000 cap 30 splits 5 out={out_dtype}")
    d2 = to_dev(pi2)
    (eo2, el2), (no2, nl2) = call_both(d2, 1000, 30.0, 5, out_dtype)
    assert torch.equal(no2, eo2) and torch.equal(nl2, el2)
    if out_dtype == torch.float32:
        ro2, rl2 = oracle.decode_paged_variant(pi2.q, pi2.k_pool, pi2.v_pool, pi2.block_table,
                                               pi2.seq_lens, 1 / math.sqrt(64), window=1000,
                                               softcap=30.0)
        assert_lowp_acc("noalloc call 2", np64(no2), ro2)
        assert_lse("noalloc call 2", np64(nl2), rl2)


def test_noalloc_paged_decode_workload_and_limit():
    """The 64-sequence, 32/8-head workload fits the buffer (8.5 MB of
    partials); a batch whose partials would not fit (64 fixed splits of 128
    query heads) is refused before any launch, with the outputs untouched."""
    p = inputs.WORKLOADS["paged_decode_bf16_b64_h32_kv8"].params
    lens = inputs.uniform_lengths(p["B"], p["len_lo"], p["len_hi"], p["seed"])
    pi = inputs.paged_decode_inputs(p["B"], p["H"], p["Hkv"], p["d"], lens, p["seed"],
                                    pool_factor=p["pool_factor"], max_pages=p["len_hi"] // 16)
    say("noalloc on the 64-sequence workload")
    d = to_dev(pi)
    (eo, el), (no, nl) = call_both(d, 0, 0.0, 0, torch.bfloat16)
    assert torch.equal(no, eo) and torch.equal(nl, el)
    # 128 query heads over 8 KV heads at 64 sequences, 64 chunks each: 270 MB
    B, H, Hkv = 64, 128, 8
    assert fa.decode_workspace_size(B, H, Hkv, 128, d["t"].shape[1], 0, 64) > 32 << 20
    q = torch.zeros((B, H, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.full((B, H, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H), 7.0, dtype=torch.float32, device=DEV)
    st = fa.lib().fa_decode_paged_noalloc(
        q.data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["t"].data_ptr(), d["s"].data_ptr(),
        out.data_ptr(), lse.data_ptr(), B, H, Hkv, 128, 16, d["t"].shape[1], d["k"].shape[0],
        1 / math.sqrt(128), 64, 0, 0.0, BF16, BF16,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 7, fa.status_string(st)
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
