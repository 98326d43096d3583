"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Every case prints what it runs before touching the GPU. Inputs come from the
seeded generators; expected values come only from the oracle or from closed
forms.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_11_amd as fa
from exact_tiled_attention_11_amd import inputs
import oracle
from parity_utils import (assert_f32, assert_lowp_acc, assert_lowp_out, assert_lse,
                          assert_lse_ulp, assert_rounded_from, np64)

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = inputs.TORCH_DTYPES


def say(*a):
    print(*a, flush=True)


def gpu_forward(q, k, v, causal, out_dtype=None, scale=None):
    say(f"  fa_forward q{tuple(q.shape)} k{tuple(k.shape)} {q.dtype} causal={causal} "
        f"out={out_dtype or q.dtype}")
    o, l = fa.forward(q, k, v, causal=causal, out_dtype=out_dtype, scale=scale)
    torch.cuda.synchronize()
    return o, l


def check_prefill(name, q, k, v, causal, ref_o, ref_l, rows=None, scale=None):
    """Run the GPU forward with native and fp32 output, compare with the oracle."""
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    sel = slice(None) if rows is None else torch.as_tensor(rows)
    if q.dtype == torch.float32:
        o, l = gpu_forward(qd, kd, vd, causal, scale=scale)
        assert_f32(name, np64(o[:, sel]), ref_o)
        assert_lse(name, np64(l[:, :, sel]), ref_l)
        return o, l
    o32, l32 = gpu_forward(qd, kd, vd, causal, out_dtype=torch.float32, scale=scale)
    o16, l16 = gpu_forward(qd, kd, vd, causal, scale=scale)
    assert_lowp_acc(name, np64(o32[:, sel]), ref_o)
    assert_rounded_from(name, o16, o32)
    assert_lowp_out(name, o16[:, sel], ref_o)
    assert_lse(name, np64(l32[:, :, sel]), ref_l)
    assert torch.equal(l16, l32), "LSE must not depend on the output type"
    return o32, l32


# ---------------------------------------------------------------------------
# The five target workloads.
# ---------------------------------------------------------------------------

def test_single_head_f32_n256():
    p = inputs.WORKLOADS["single_head_f32_n256"].params
    q, k, v = inputs.prefill_inputs(1, 1, 1, 256, 256, 64, torch.float32, p["seed"])
    say("single head fp32 256x256")
    ro, rl = oracle.attention(q, k, v, 1 / 8, False)
    check_prefill("single_head_f32", q, k, v, False, ro, rl)


MHA12 = [(dt, c, s) for dt in ("f16", "f32") for c in (False, True) for s in (1.0, 30.0)]


@pytest.mark.parametrize("dt,causal,qs", MHA12, ids=[f"{d}-{'causal' if c else 'full'}-q{int(s)}"
                                                     for d, c, s in MHA12])
def test_mha12_d64_n2048(dt, causal, qs):
    p = inputs.WORKLOADS["mha12_d64_n2048"].params
    q, k, v = inputs.prefill_inputs(1, 12, 12, 2048, 2048, 64, TD[dt], p["seed"], q_scale=qs)
    say(f"mha12 {dt} causal={causal} qscale={qs}")
    ro, rl = oracle.attention(q, k, v, 1 / 8, causal)
    check_prefill(f"mha12-{dt}-{causal}-{qs}", q, k, v, causal, ro, rl)


@pytest.fixture(scope="module")
def c3():
    p = inputs.WORKLOADS["causal_prefill_bf16_b4_h32_n8192"].params
    q, k, v = inputs.prefill_inputs(p["B"], p["H"], p["Hkv"], p["N"], p["N"], p["d"],
                                    torch.bfloat16, p["seed"])
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o32, l32 = gpu_forward(qd, kd, vd, True, out_dtype=torch.float32)
    o16, l16 = gpu_forward(qd, kd, vd, True)
    return dict(q=q, k=k, v=v, o32=o32, l32=l32, o16=o16, l16=l16, p=p)


def test_causal_prefill_b4_h32_n8192_sampled_rows(c3):
    rows = inputs.sample_rows(256, 8192, seed=c3["p"]["seed"])
    # plus the edges of the 256-row query blocks and 64-key tiles
    edges = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 4095, 4096, 8127, 8128, 8190, 8191]
    rows = np.unique(np.concatenate([rows, edges]))
    say(f"c3 oracle on {len(rows)} rows x 4 batches x 32 heads")
    ro, rl = oracle.attention(c3["q"], c3["k"], c3["v"], 1 / math.sqrt(128), True, rows=rows)
    sel = torch.as_tensor(rows)
    assert_lowp_acc("c3 rows", np64(c3["o32"][:, sel]), ro)
    assert_lowp_out("c3 rows", c3["o16"][:, sel], ro)
    assert_lse("c3 rows", np64(c3["l32"][:, :, sel]), rl)
    assert_rounded_from("c3", c3["o16"], c3["o32"])
    assert torch.equal(c3["l16"], c3["l32"])
    assert torch.isfinite(c3["o32"]).all() and torch.isfinite(c3["l32"]).all()


@pytest.mark.parametrize("b", range(4))
def test_causal_prefill_b4_h32_n8192_full_lse(c3, b):
    """Every LSE value of the workload: all 8192 rows of all 32 heads of batch b."""
    say(f"c3 full LSE of batch {b}, all 32 heads")
    rl = oracle.log_sum_exp(c3["q"][b:b + 1], c3["k"][b:b + 1], 1 / math.sqrt(128), True)
    assert_lse(f"c3 b{b}", np64(c3["l32"][b]), rl[0])


def test_causal_prefill_b4_h32_n8192_zero_query():
    """Q = 0: O_i is the mean of v_0..v_i and LSE_i = ln(i+1), at full size."""
    p = inputs.WORKLOADS["causal_prefill_bf16_b4_h32_n8192"].params
    _, _, v = inputs.prefill_inputs(p["B"], p["H"], p["Hkv"], p["N"], p["N"], p["d"],
                                    torch.bfloat16, p["seed"])
    q = torch.zeros_like(v)
    say("c3 zero-query closed form")
    o, l = gpu_forward(q.to(DEV), v.to(DEV), v.to(DEV), True, out_dtype=torch.float32)
    n = p["N"]
    for b in range(p["B"]):
        vb = np64(v[b])                                    # [N, H, d]
        expect = np.cumsum(vb, axis=0) / np.arange(1, n + 1)[:, None, None]
        assert_lowp_acc(f"c3 zero-q b{b}", np64(o[b]), expect)
    lexp = np.log(np.arange(1, n + 1, dtype=np.float64))
    assert_lse("c3 zero-q", np64(l), np.broadcast_to(lexp, l.shape))


@pytest.fixture(scope="module")
def c4():
    p = inputs.WORKLOADS["paged_decode_bf16_b64_h32_kv8"].params
    lens = inputs.uniform_lengths(p["B"], p["len_lo"], p["len_hi"], p["seed"])
    say(f"c4 inputs: sum(len)={int(lens.sum())}")
    pi = inputs.paged_decode_inputs(p["B"], p["H"], p["Hkv"], p["d"], lens, p["seed"],
                                    pool_factor=p["pool_factor"], max_pages=p["len_hi"] // 16)
    dev = dict(q=pi.q.to(DEV), k=pi.k_pool.to(DEV), v=pi.v_pool.to(DEV),
               t=pi.block_table.to(DEV), s=pi.seq_lens.to(DEV))
    say(f"c4 oracle on all {p['B']} sequences")
    ro, rl = oracle.decode_paged(pi.q, pi.k_pool, pi.v_pool, pi.block_table, pi.seq_lens,
                                 1 / math.sqrt(128))
    return dict(pi=pi, dev=dev, ro=ro, rl=rl, p=p)


def gpu_decode(d, splits, out_dtype=None):
    say(f"  fa_decode_paged B={d['q'].shape[0]} splits={splits} out={out_dtype}")
    o, l = fa.decode_paged(d["q"], d["k"], d["v"], d["t"], d["s"], num_splits=splits,
                           out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, l


@pytest.mark.parametrize("splits", [0, 1, 2, 4, 8, 16, 32, 64])
def test_paged_decode_b64_h32_kv8(c4, splits):
    """All 64 sequences x 32 heads against the oracle."""
    o32, l32 = gpu_decode(c4["dev"], splits, torch.float32)
    o16, l16 = gpu_decode(c4["dev"], splits)
    assert_lowp_acc(f"c4 s{splits}", np64(o32), c4["ro"])
    assert_lowp_out(f"c4 s{splits}", o16, c4["ro"])
    assert_lse(f"c4 s{splits}", np64(l32), c4["rl"])
    assert_rounded_from(f"c4 s{splits}", o16, o32)
    assert torch.equal(l16, l32)


@pytest.mark.parametrize("splits", [0, 16, 64])
def test_paged_decode_batch1_32k_worked_example(splits):
    """The pages' occupancy example ("3.4 Attention Kernels", "Worked example"):
    one sequence of 32768 tokens, 32 query heads over 8 KV heads, d = 128. The
    automatic plan cuts it into 32 chunks (256 workgroups), the fixed 16 is the
    page's own count, 64 the most the library allows."""
    lens = [32768]
    pi = inputs.paged_decode_inputs(1, 32, 8, 128, lens, seed=141)
    assert list(fa.decode_plan([32768], 8, pi.block_table.shape[1])) == [32]
    say(f"decode batch 1, 32k tokens, splits={splits}: oracle")
    ro, rl = oracle.decode_paged(pi.q, pi.k_pool, pi.v_pool, pi.block_table, pi.seq_lens,
                                 1 / math.sqrt(128))
    dev = dict(q=pi.q.to(DEV), k=pi.k_pool.to(DEV), v=pi.v_pool.to(DEV),
               t=pi.block_table.to(DEV), s=pi.seq_lens.to(DEV))
    o32, l32 = gpu_decode(dev, splits, torch.float32)
    o16, l16 = gpu_decode(dev, splits)
    assert_lowp_acc(f"b1 32k s{splits}", np64(o32), ro)
    assert_lowp_out(f"b1 32k s{splits}", o16, ro)
    assert_lse(f"b1 32k s{splits}", np64(l32), rl)
    assert_rounded_from(f"b1 32k s{splits}", o16, o32)


def test_paged_decode_b64_h32_kv8_repeatable(c4):
    a = gpu_decode(c4["dev"], 0)
    b = gpu_decode(c4["dev"], 0)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.fixture(scope="module")
def c5():
    p = inputs.WORKLOADS["long_causal_prefill_bf16_n65536"].params
    q, k, v = inputs.prefill_inputs(p["B"], p["H"], p["Hkv"], p["N"], p["N"], p["d"],
                                    torch.bfloat16, p["seed"], q_scale=p["q_scales"][0])
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o32, l32 = gpu_forward(qd, kd, vd, True, out_dtype=torch.float32)
    o16, l16 = gpu_forward(qd, kd, vd, True)
    return dict(q=q, k=k, v=v, o32=o32, l32=l32, o16=o16, l16=l16, p=p)


def test_long_causal_prefill_n65536_sampled_rows(c5):
    rows = inputs.sample_rows(c5["p"]["sample_rows"], c5["p"]["N"], seed=c5["p"]["seed"])
    say("c5 oracle on 256 rows x 16 heads")
    ro, rl = oracle.attention(c5["q"], c5["k"], c5["v"], 1 / math.sqrt(128), True, rows=rows)
    sel = torch.as_tensor(rows)
    assert_lowp_acc("c5 rows", np64(c5["o32"][:, sel]), ro)
    assert_lowp_out("c5 rows", c5["o16"][:, sel], ro)
    assert_lse("c5 rows", np64(c5["l32"][:, :, sel]), rl)
    assert_rounded_from("c5", c5["o16"], c5["o32"])
    assert torch.equal(c5["l16"], c5["l32"])
    assert torch.isfinite(c5["o32"]).all() and torch.isfinite(c5["l32"]).all()


@pytest.mark.parametrize("h", range(16))
def test_long_causal_prefill_n65536_full_lse(c5, h):
    say(f"c5 full LSE head {h}")
    rl = oracle.log_sum_exp(c5["q"][:, :, h:h + 1], c5["k"][:, :, h:h + 1],
                            1 / math.sqrt(128), True)
    assert_lse(f"c5 h{h}", np64(c5["l32"][0, h]), rl[0, 0])


# ---------------------------------------------------------------------------
# Edge cases of the forward.
# ---------------------------------------------------------------------------

EDGE = [
    # (B, H, Hkv, Nq, Nk, d, dtype, causal)
    (1, 1, 1, 1, 1, 64, "bf16", False),
    (1, 1, 1, 1, 1, 128, "f32", True),
    (2, 3, 3, 200, 200, 64, "bf16", True),      # ragged q and k tiles
    (2, 3, 3, 200, 200, 128, "f16", False),
    (1, 8, 2, 333, 333, 128, "bf16", True),     # GQA
    (1, 4, 1, 129, 1000, 64, "f32", True),      # Nq < Nk, bottom-right causal
    (1, 4, 4, 300, 70, 128, "bf16", True),      # Nq > Nk: first rows see no key
    (1, 2, 2, 77, 0, 64, "bf16", False),        # no keys at all
    (1, 2, 1, 64, 65, 128, "f32", False),
    (3, 2, 2, 5, 700, 128, "f16", True),        # few queries, long cache
    # group sizes that are not powers of two, and one KV head for all (MQA)
    (2, 6, 2, 200, 200, 128, "bf16", True),     # G = 3
    (1, 12, 2, 77, 300, 64, "f16", True),       # G = 6, Nq < Nk
    (1, 16, 1, 130, 130, 128, "bf16", False),   # G = 16
    (2, 32, 1, 70, 70, 128, "bf16", True),      # G = 32 (MQA)
    (1, 32, 1, 9, 400, 64, "f16", True),        # G = 32, a few newest queries
    (1, 6, 2, 100, 100, 64, "f32", True),       # G = 3, fp32 inputs
]


@pytest.mark.parametrize("case", EDGE, ids=[f"{c[0]}x{c[3]}x{c[4]}-h{c[1]}/{c[2]}-d{c[5]}-{c[6]}"
                                               f"-{'c' if c[7] else 'n'}" for c in EDGE])
def test_forward_edge(case):
    B, H, Hkv, Nq, Nk, d, dt, causal = case
    q, k, v = inputs.prefill_inputs(B, H, Hkv, Nq, Nk, d, TD[dt], seed=100 + EDGE.index(case))
    say(f"edge {case}")
    ro, rl = oracle.attention(q, k, v, 1 / math.sqrt(d), causal)
    check_prefill(f"edge {case}", q, k, v, causal, ro, rl)


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f16", 64), ("f32", 128)])
def test_forward_closed_forms(dt, d):
    """Single key, constant V, causal row 0, Q = 0 prefix means."""
    rng_q, rng_k, rng_v = inputs.prefill_inputs(2, 4, 2, 300, 300, d, TD[dt], seed=7)
    say(f"closed forms {dt} d={d}")
    # single key: O = v, LSE = scale q.k
    o, l = gpu_forward(rng_q.to(DEV), rng_k[:, :1].to(DEV).contiguous(),
                       rng_v[:, :1].to(DEV).contiguous(), False, out_dtype=torch.float32)
    vexp = np.repeat(np.repeat(np64(rng_v[:, :1]), 300, axis=1), 2, axis=2)
    tol = 1e-4 if dt == "f32" else 1e-2
    assert np.abs(np64(o) - vexp).max() <= tol
    # constant V rows: O = c
    c = rng_v[:, :1].expand(-1, 300, -1, -1).contiguous()
    o, _ = gpu_forward(rng_q.to(DEV), rng_k.to(DEV), c.to(DEV), True, out_dtype=torch.float32)
    cexp = np.repeat(np64(c), 2, axis=2)
    assert np.abs(np64(o) - cexp).max() <= tol
    # causal row 0 sees key 0 only
    o, l = gpu_forward(rng_q.to(DEV), rng_k.to(DEV), rng_v.to(DEV), True, out_dtype=torch.float32)
    v0 = np.repeat(np64(rng_v[:, 0]), 2, axis=1)
    assert np.abs(np64(o[:, 0]) - v0).max() <= tol
    # Q = 0, causal: prefix means, LSE = ln(i+1)
    z = torch.zeros_like(rng_q)
    o, l = gpu_forward(z.to(DEV), rng_k.to(DEV), rng_v.to(DEV), True, out_dtype=torch.float32)
    pm = np.cumsum(np64(rng_v), axis=1) / np.arange(1, 301)[None, :, None, None]
    assert np.abs(np64(o) - np.repeat(pm, 2, axis=2)).max() <= tol
    assert np.abs(np64(l) - np.log(np.arange(1, 301))).max() <= 1e-4


@pytest.mark.parametrize("growth", [-3.0, 0.5, 3.0, 7.9, 8.1, 20.0, 31.9, 32.1])
@pytest.mark.parametrize("dt,causal", [("bf16", True), ("f16", False)])
def test_forward_rising_scores(growth, dt, causal):
    """Row maxima that climb steadily across the key tiles: every score gets a
    ramp of `growth` log2 units per 64 keys on top of its random part. Slow
    ramps keep an old reference max for many tiles (probabilities up to 2^32
    with bf16 inputs, 2^8 with fp16), ramps near 32 (bf16) and 8 (fp16) sit at
    the rescale thresholds, fast ramps move the reference at every tile, a
    falling ramp puts the maximum first."""
    B, H, N, d = 1, 2, 1024, 128
    q, k, v = inputs.prefill_inputs(B, H, H, N, N, d, TD[dt], seed=21)
    scale = 1 / math.sqrt(d)
    beta = growth / (64 * scale * math.log2(math.e))
    q = q.clone()
    k = k.clone()
    q[..., 0] = 1.0
    k[..., 0] = (beta * torch.arange(N, dtype=torch.float32)).to(k.dtype)[None, :, None]
    say(f"rising scores growth={growth} {dt} causal={causal}")
    ro, rl = oracle.attention(q, k, v, scale, causal)
    check_prefill(f"rising {growth} {dt}", q, k, v, causal, ro, rl)


def test_forward_repeatable():
    q, k, v = inputs.prefill_inputs(2, 4, 4, 1000, 1000, 128, torch.bfloat16, seed=8)
    say("forward repeatability")
    a = gpu_forward(q.to(DEV), k.to(DEV), v.to(DEV), True)
    b = gpu_forward(q.to(DEV), k.to(DEV), v.to(DEV), True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---------------------------------------------------------------------------
# Edge cases of the paged decode and the merge.
# ---------------------------------------------------------------------------

DEC = [
    # (H, Hkv, d, dtype, lens)
    (8, 8, 128, "bf16", [1, 15, 16, 17, 31, 32, 33, 0]),
    (8, 4, 64, "f16", [0, 1, 100, 2048, 2049, 5000]),
    (32, 8, 128, "bf16", [1, 2047, 4097, 9000, 16, 300]),
    (16, 2, 128, "f16", [50, 3000, 1]),
    (4, 4, 64, "bf16", [7, 70, 700, 7000]),
    # group sizes that are not powers of two, and the 16-head limit
    (6, 2, 128, "bf16", [1, 500, 3001]),        # G = 3
    (12, 2, 64, "f16", [17, 1025, 4000]),       # G = 6
    (5, 1, 128, "bf16", [33, 2222]),            # G = 5
    (32, 2, 128, "bf16", [1, 999, 5000]),       # G = 16
]


@pytest.mark.parametrize("case", DEC, ids=[f"h{c[0]}/{c[1]}-d{c[2]}-{c[3]}" for c in DEC])
@pytest.mark.parametrize("splits", [0, 1, 3, 16])
def test_decode_edge(case, splits):
    H, Hkv, d, dt, lens = case
    B = len(lens)
    pi = inputs.paged_decode_inputs(B, H, Hkv, d, lens, seed=11, dtype=TD[dt])
    # token slots past each sequence's end hold NaN: they must never be used
    for b in range(B):
        L = lens[b]
        if L % 16:
            pi.k_pool[int(pi.block_table[b, L // 16]), L % 16:] = float("nan")
            pi.v_pool[int(pi.block_table[b, L // 16]), L % 16:] = float("nan")
    say(f"decode edge {case} splits={splits}")
    ro, rl = oracle.decode_paged(pi.q, pi.k_pool, pi.v_pool, pi.block_table, pi.seq_lens,
                                 1 / math.sqrt(d))
    dev = dict(q=pi.q.to(DEV), k=pi.k_pool.to(DEV), v=pi.v_pool.to(DEV),
               t=pi.block_table.to(DEV), s=pi.seq_lens.to(DEV))
    o32, l32 = gpu_decode(dev, splits, torch.float32)
    o16, _ = gpu_decode(dev, splits)
    assert_lowp_acc(f"dec {case}", np64(o32), ro)
    assert_lse(f"dec {case}", np64(l32), rl)
    assert_rounded_from(f"dec {case}", o16, o32)


def test_decode_page_order_does_not_matter():
    lens = [3000, 17, 4096, 1]
    pi = inputs.paged_decode_inputs(4, 32, 8, 128, lens, seed=12, unreferenced="normal")
    # the same tokens laid out in consecutive pages
    table = pi.block_table
    need = [-(-L // 16) for L in lens]
    order = torch.cat([table[b, :need[b]] for b in range(4)]).long()
    kc, vc = pi.k_pool[order].contiguous(), pi.v_pool[order].contiguous()
    tc = torch.full_like(table, -1)
    off = 0
    for b in range(4):
        tc[b, :need[b]] = torch.arange(off, off + need[b], dtype=torch.int32)
        off += need[b]
    say("decode page order")
    a = gpu_decode(dict(q=pi.q.to(DEV), k=pi.k_pool.to(DEV), v=pi.v_pool.to(DEV),
                        t=table.to(DEV), s=pi.seq_lens.to(DEV)), 0)
    b = gpu_decode(dict(q=pi.q.to(DEV), k=kc.to(DEV), v=vc.to(DEV), t=tc.to(DEV),
                        s=pi.seq_lens.to(DEV)), 0)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_contract_violations_give_nan():
    lens = [40, 40, 40]
    pi = inputs.paged_decode_inputs(3, 8, 2, 128, lens, seed=13)
    n_pages = pi.k_pool.shape[0]
    table = pi.block_table.clone()
    table[1, 1] = n_pages          # page id outside the pool
    seq = pi.seq_lens.clone()
    seq[2] = 10_000                # longer than the block table allows
    say("decode contract violations")
    for splits in (0, 2):
        o, l = gpu_decode(dict(q=pi.q.to(DEV), k=pi.k_pool.to(DEV), v=pi.v_pool.to(DEV),
                               t=table.to(DEV), s=seq.to(DEV)), splits, torch.float32)
        assert torch.isfinite(o[0]).all() and torch.isfinite(l[0]).all()
        assert torch.isnan(o[1]).all() and torch.isnan(l[1]).all()
        assert torch.isnan(o[2]).all() and torch.isnan(l[2]).all()


@pytest.mark.parametrize("R,S,d,out", [(37, 5, 128, "f32"), (8, 16, 64, "bf16"),
                                       (5, 1, 3, "f16"), (3, 1024, 130, "f32")])
def test_merge(R, S, d, out):
    rng = np.random.default_rng(R * S + d)
    o = rng.standard_normal((R, S, d)).astype(np.float32)
    l = (rng.standard_normal((R, S)) * 20).astype(np.float32)
    l[0, :] = -np.inf                          # an all-empty row
    if S > 1:
        l[1, 1:] = -np.inf                     # empty parts are the identity
        l[2, 0] = 3000.0                       # large values stay finite
    num = rng.integers(0, S + 1, size=R).astype(np.int32)
    say(f"merge R={R} S={S} d={d} out={out}")
    for use_num in (False, True):
        og, lg = fa.merge_partials(torch.from_numpy(o).to(DEV), torch.from_numpy(l).to(DEV),
                                   torch.from_numpy(num).to(DEV) if use_num else None,
                                   out_dtype=TD[out])
        torch.cuda.synchronize()
        ro, rl = oracle.merge_partials(o, l, num if use_num else None)
        tol = 1e-5 if out == "f32" else 1e-2
        err = np.abs(np64(og) - ro)
        assert err.max() <= tol * max(1.0, np.abs(ro).max()), err.max()
        assert_lse_ulp("merge", np64(lg), rl)
