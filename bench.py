#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X; prints ONE JSON line on stdout.

One step = one causal prefill forward (B=4, H=32, N=8192, d=128, bf16 in,
fp32 accumulate, bf16 O + fp32 LSE) followed by one split-KV paged decode
(64 sequences, 32 query / 8 KV heads, d=128, 16-token pages, lengths uniform
in [1024, 32768], automatic split count) including its merge of partials.
Inputs are seeded synthetic tensors, resident in HBM before timing starts.

`value` is the prefill throughput in TFLOP/s of algorithmic work
(4 d per visible query-key pair); the decode's KV GB/s is reported beside it.
Both parts are timed with HIP events on the stream the kernels run on.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 4096 dense bf16 FLOP/clk x 2.4 GHz
FP32_PEAK_TFLOPS = 157.3         # published fp32 peak (matrix and vector)
HBM_PEAK_GBPS = 8000.0
PREFILL = "causal_prefill_bf16_b4_h32_n8192"
DECODE = "paged_decode_bf16_b64_h32_kv8"
LONG = "long_causal_prefill_bf16_n65536"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter runs
    (profiles/traffic.json), or None once the kernel's sources have changed
    since the counters were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != sources_sha256(rec["sources"]):
        return None
    return rec


def causal_flops(B, H, N, d):
    return 4.0 * d * (N * (N + 1) / 2) * B * H


def cpu_baseline_prefill(q, k, v, d, target_s):
    """Time the float64 oracle as the parity tests call it: 256 evenly spaced
    causal query rows per head, one block of rows (its default block size),
    each row scored against every key of the sequence and the invisible ones
    masked. `value` counts the algorithmic work of those rows (4 d per visible
    query-key pair), the same measure as the GPU figure; `executed_tflops`
    counts what the oracle actually multiplies (4 d per key of the whole row,
    about twice as much for these rows)."""
    import numpy as np
    import oracle
    N = q.shape[1]
    rows = np.arange(N // 256 - 1, N, N // 256)            # 256 rows spread over the sequence
    per_head = sum(4.0 * d * (i + 1) for i in rows)
    per_head_exec = 4.0 * d * N * len(rows)
    done, heads, b = 0.0, 0, 0
    H = q.shape[2]
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < target_s and b < q.shape[0]:
        # one batch entry, all heads: one job per head on the oracle's thread pool
        oracle.attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], 1 / math.sqrt(d), True, rows=rows)
        done += per_head * H
        heads += H
        b += 1
    dt = time.perf_counter() - t0
    return dict(value=done / dt / 1e12, unit="TFLOP/s", cores=oracle.default_threads(),
                kind="oracle", executed_tflops=heads * per_head_exec / dt / 1e12,
                sample=f"{heads} (batch, head) pairs x 256 evenly spaced causal query rows of "
                       f"the {PREFILL} workload, float64, rows scored against all {N} keys "
                       f"and masked (the oracle's own form); value counts visible pairs only; "
                       f"{dt:.1f} s")


def cpu_baseline_decode(pi, d, target_s):
    import oracle
    hkv = pi.k_pool.shape[2]
    done_bytes, seqs = 0.0, 0
    t0 = time.perf_counter()
    B = pi.q.shape[0]
    while time.perf_counter() - t0 < target_s and seqs < B:
        b = seqs
        oracle.decode_paged(pi.q[b:b + 1], pi.k_pool, pi.v_pool, pi.block_table[b:b + 1],
                            pi.seq_lens[b:b + 1], 1 / math.sqrt(d))
        done_bytes += float(pi.seq_lens[b]) * hkv * d * 2 * 2
        seqs += 1
    dt = time.perf_counter() - t0
    return dict(value=done_bytes / dt / 1e9, unit="GB/s", cores=oracle.default_threads(),
                kind="oracle",
                sample=f"{seqs} of the {B} sequences of the {DECODE} workload, float64, "
                       f"{dt:.1f} s")


def time_steps(torch, fn, n):
    """Mean ms per call of n back-to-back calls on the current stream."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def bench_decode_variants(torch, fa, inputs, pi, dev, lens, dp, steps):
    """The decode with a 4096-token window and logit cap 50: GB/s of the KV
    bytes the window leaves visible."""
    import numpy as np
    window, cap = 4096, 50.0
    vis = np.minimum(lens, window).astype(np.float64)
    kv = float(vis.sum()) * dp["Hkv"] * dp["d"] * 2 * 2
    ws = torch.empty(fa.decode_workspace_size(dp["B"], dp["H"], dp["Hkv"], dp["d"],
                                              dev["t"].shape[1], window), dtype=torch.uint8,
                     device="cuda")
    od = torch.empty_like(dev["q"])
    ld = torch.empty((dp["B"], dp["H"]), dtype=torch.float32, device="cuda")

    def run():
        fa.decode_paged_ex(dev["q"], dev["k"], dev["v"], dev["t"], dev["s"], window=window,
                           softcap=cap, out=od, lse=ld, workspace=ws)
    for _ in range(3):
        run()
    ms = time_steps(torch, run, max(steps, 10))
    return {"workload": DECODE + " window=4096 softcap=50", "ms_mean": ms,
            "visible_kv_bytes": kv, "value": kv / (ms * 1e-3) / 1e9, "unit": "GB/s",
            "frac_hbm": kv / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}


def bench_small_configs(torch, fa, inputs, reps=50):
    """The two small forward workloads, timed like the others: one fp32 head of
    256 x 256 (d = 64), and 12 heads of 2048 tokens (d = 64) causal and not, in
    fp16 and fp32 with Q and 30 Q. TFLOP/s of algorithmic work (4 d per visible
    query-key pair) against the published peak of the input type."""
    out = {}
    cases = [("single_head_f32_n256", 1, 1, 256, 64, "f32", False, 1.0)]
    for dt in ("f16", "f32"):
        for causal in (False, True):
            for qs in (1.0, 30.0):
                cases.append((f"mha12_d64_n2048_{dt}_{'causal' if causal else 'full'}_q{int(qs)}",
                              1, 12, 2048, 64, dt, causal, qs))
    for name, B, H, N, d, dt, causal, qs in cases:
        wl = "single_head_f32_n256" if name.startswith("single") else "mha12_d64_n2048"
        seed = inputs.WORKLOADS[wl].params["seed"]
        q, k, v = inputs.prefill_inputs(B, H, H, N, N, d, inputs.TORCH_DTYPES[dt], seed,
                                        q_scale=qs)
        q, k, v = q.cuda(), k.cuda(), v.cuda()
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

        def run():
            fa.forward(q, k, v, causal=causal, out=o, lse=lse)
        for _ in range(3):
            run()
        ms = time_steps(torch, run, reps)
        fl = causal_flops(B, H, N, d) if causal else 4.0 * d * N * N * B * H
        peak = FP32_PEAK_TFLOPS if dt == "f32" else MFMA_BF16_PEAK_TFLOPS
        tf = fl / (ms * 1e-3) / 1e12
        out[name] = {"us_mean": ms * 1e3, "algorithmic_flop": fl, "value": tf,
                     "unit": "TFLOP/s", "peak": peak, "frac": tf / peak, "calls": reps,
                     "kernel": "fwd_kernel<fp32>" if dt == "f32" else "fwd16_kernel<f16, d=64>"}
    return out


def bench_decode_batch1(torch, fa, inputs, reps=20, copies=4):
    """The pages' occupancy example: one sequence of 32768 cached tokens, 32
    query heads over 8 KV heads, d = 128 (134 MB of K and V). Successive calls
    read `copies` different caches in turn (537 MB in all, more than the 256 MB
    last-level cache), so every call streams its KV from HBM."""
    import numpy as np
    H, Hkv, d, L = 32, 8, 128, 32768
    lens = np.array([L], dtype=np.int64)
    devs = []
    for c in range(copies):
        pi = inputs.paged_decode_inputs(1, H, Hkv, d, lens, seed=150 + c, pool_factor=1.0,
                                        unreferenced="normal")
        devs.append(dict(q=pi.q.cuda(), k=pi.k_pool.cuda(), v=pi.v_pool.cuda(),
                         t=pi.block_table.cuda(), s=pi.seq_lens.cuda()))
    kv = float(L) * Hkv * d * 2 * 2
    o = torch.empty((1, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, H), dtype=torch.float32, device="cuda")
    out = {"workload": "decode batch 1, 32768 tokens, h32/kv8, d128, bf16, 16-token pages",
           "kv_bytes": kv, "caches_rotated": copies}
    for splits in (0, 16, 32, 64):
        ws = torch.empty(fa.decode_workspace_size(1, H, Hkv, d, devs[0]["t"].shape[1], 0,
                                                  splits), dtype=torch.uint8, device="cuda")
        it = [0]

        def run():
            dv = devs[it[0] % copies]
            it[0] += 1
            fa.decode_paged(dv["q"], dv["k"], dv["v"], dv["t"], dv["s"], num_splits=splits,
                            out=o, lse=lse, workspace=ws)
        for _ in range(copies):
            run()
        ms = time_steps(torch, run, reps)
        gbs = kv / (ms * 1e-3) / 1e9
        key = "auto" if splits == 0 else f"splits_{splits}"
        out[key] = {"splits": int(fa.decode_plan([L], Hkv, devs[0]["t"].shape[1], 0, splits)[0]),
                    "us_mean": ms * 1e3,
                    "value": gbs, "unit": "GB/s", "frac_hbm": gbs / HBM_PEAK_GBPS}
    del devs
    torch.cuda.empty_cache()
    return out


def bench_decode_graph(torch, fa, inputs, dev, dp, n=200):
    """Launch overhead: eager decode step (decode + merge launches) against one
    graph replay, on the paged-decode workload and on a one-sequence step."""
    import numpy as np
    out = {}
    small_lens = np.array([1024], dtype=np.int64)
    spi = inputs.paged_decode_inputs(1, dp["H"], dp["Hkv"], dp["d"], small_lens, seed=7)
    sdev = dict(q=spi.q.cuda(), k=spi.k_pool.cuda(), v=spi.v_pool.cuda(),
                t=spi.block_table.cuda(), s=spi.seq_lens.cuda())
    for name, d in (("b64_h32_kv8_paged", dev), ("b1_len1024", sdev)):
        B, H, hd = d["q"].shape
        ws = torch.empty(fa.decode_workspace_size(B, H, d["k"].shape[2], hd, d["t"].shape[1]),
                         dtype=torch.uint8, device="cuda")
        o = torch.empty_like(d["q"])
        lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
        g = fa.DecodeGraph(d["q"], d["k"], d["v"], d["t"], d["s"], out=o, lse=lse, workspace=ws)

        def eager():
            fa.decode_paged(d["q"], d["k"], d["v"], d["t"], d["s"], out=o, lse=lse, workspace=ws)
        for _ in range(3):
            eager()
            g.launch()
        torch.cuda.synchronize()
        t_e = time_steps(torch, eager, n)
        t_g = time_steps(torch, g.launch, n)
        g.close()
        out[name] = {"eager_us_per_step": t_e * 1e3, "graph_us_per_step": t_g * 1e3,
                     "saved_us_per_step": (t_e - t_g) * 1e3, "steps": n}
        if name == "b1_len1024":
            # a model step: one decode per layer, 32 layers, replayed as one graph
            layers = 32
            cg = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for _ in range(3):
                    eager()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(cg):
                for _ in range(layers):
                    eager()
            torch.cuda.synchronize()

            def many():
                for _ in range(layers):
                    eager()
            reps = max(1, n // layers)
            t_me = time_steps(torch, many, reps)
            t_mg = time_steps(torch, cg.replay, reps)
            out["b1_len1024_x32_layers"] = {"eager_us_per_step": t_me * 1e3,
                                            "graph_us_per_step": t_mg * 1e3,
                                            "saved_us_per_step": (t_me - t_mg) * 1e3,
                                            "steps": reps, "layers": layers}
    return out


def ragged_flops(q_lens, kv_lens, H, d, causal=True):
    """4 d H x (visible query-key pairs); with causal, query i of a sequence sees
    min(kv, max(0, i + kv - q + 1)) keys (bottom-right alignment)."""
    pairs = 0.0
    for ql, kl in zip(q_lens, kv_lens):
        ql, kl = int(ql), int(kl)
        off = kl - ql
        if not causal:
            pairs += ql * kl
        elif off >= 0:
            pairs += ql * (off + 1) + ql * (ql - 1) / 2.0
        else:
            pairs += sum(min(kl, max(0, i + off + 1)) for i in range(ql))
    return 4.0 * d * H * pairs


def bench_long_prefill(torch, fa, inputs, reps=10):
    """The long-context causal prefill (one sequence of 65536 tokens, 16 heads,
    d = 128, bf16, Q scaled by 30), timed like the headline prefill."""
    p = inputs.WORKLOADS[LONG].params
    B, H, N, d = p["B"], p["H"], p["N"], p["d"]
    q, k, v = inputs.prefill_inputs(B, H, p["Hkv"], N, N, d, torch.bfloat16, p["seed"],
                                    q_scale=p["q_scales"][0])
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def run():
        fa.forward(q, k, v, causal=True, out=o, lse=lse)
    for _ in range(2):
        run()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    import numpy as np
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    fl = causal_flops(B, H, N, d)
    tf = fl / (ms.mean() * 1e-3) / 1e12
    tr = measured_traffic("long_prefill")
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return {"workload": LONG, "config": {k_: p[k_] for k_ in ("B", "H", "Hkv", "N", "d")} |
            {"causal": True, "q_scale": p["q_scales"][0]},
            "ms_mean": float(ms.mean()), "ms_median": float(np.median(ms)),
            "ms_min": float(ms.min()), "calls": reps,
            "algorithmic_flop": fl, "value": tf, "unit": "TFLOP/s", "bound": "mfma",
            "peak": MFMA_BF16_PEAK_TFLOPS, "frac": tf / MFMA_BF16_PEAK_TFLOPS,
            "traffic": tr["hbm_bytes_per_launch"] if tr else None}


def bench_forward_paged(torch, fa, inputs, reps=10):
    """Ragged queries over a paged cache: the causal-prefill shape with its K/V
    scattered over pages, and a continuous-batching step mixing prefill chunks
    with decode tokens."""
    import numpy as np
    out = {}
    lens = inputs.uniform_lengths(60, 1024, 8192, 62)
    cases = {
        "causal_prefill_b4_h32_n8192_paged": ([8192] * 4, [8192] * 4, 32, 32),
        "mixed_4x2048_prefill_60_decode_h32_kv8": ([2048] * 4 + [1] * 60,
                                                   [8192] * 4 + list(lens), 32, 8),
    }
    for name, (ql, kl, H, Hkv) in cases.items():
        ri = inputs.ragged_paged_inputs(ql, kl, H, Hkv, 128, seed=61, pool_factor=1.0,
                                        unreferenced="normal")
        args = [t.cuda() for t in (ri.q, ri.qo_indptr, ri.k_pool, ri.v_pool, ri.block_table,
                                   ri.kv_lens)]
        o = torch.empty_like(args[0])
        lse = torch.empty((args[0].shape[0], H), dtype=torch.float32, device="cuda")

        def run():
            fa.forward_paged(*args, ri.max_q_len, causal=True, out=o, lse=lse)
        for _ in range(2):
            run()
        ms = time_steps(torch, run, reps)
        fl = ragged_flops(ql, kl, H, 128)
        out[name] = {"ms_mean": ms, "algorithmic_flop": fl, "value": fl / (ms * 1e-3) / 1e12,
                     "unit": "TFLOP/s", "frac_mfma": fl / (ms * 1e-3) / 1e12 /
                     MFMA_BF16_PEAK_TFLOPS, "q_rows": int(sum(ql)), "kv_tokens": int(sum(kl))}
        del args, o, lse, ri
        torch.cuda.empty_cache()
    return out


def bench_cascade(torch, fa, inputs, reps=10):
    """64 decode requests sharing a 16384-token prefix (own suffixes of 16..512
    tokens): the cascade against the split-KV decode over block tables that
    list the prefix pages before each request's own pages."""
    import numpy as np
    B, H, Hkv, d, P = 64, 32, 8, 128, 16384
    own = inputs.uniform_lengths(B, 16, 512, 64)
    ri = inputs.ragged_paged_inputs([1] * B, own, H, Hkv, d, seed=65, pool_factor=1.0,
                                    unreferenced="normal")
    n_pre = P // 16
    pre_k = inputs.normal((n_pre, 16, Hkv, d), 66)
    pre_v = inputs.normal((n_pre, 16, Hkv, d), 67)
    base = ri.k_pool.shape[0]
    kp = torch.cat([ri.k_pool, pre_k]).cuda()
    vp = torch.cat([ri.v_pool, pre_v]).cuda()
    prefix_pages = torch.arange(base, base + n_pre, dtype=torch.int32)
    q, ind = ri.q.cuda(), ri.qo_indptr.cuda()
    bt, kl = ri.block_table.cuda(), ri.kv_lens.cuda()
    S = fa.cascade_num_splits(P, B, H, Hkv)
    ws = torch.empty(fa.cascade_workspace_size(B, H, d, S), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ppd = prefix_pages.cuda()

    def run_cascade():
        fa.cascade(q, ind, kp, vp, ppd, P, bt, kl, 1, causal=True, out=o, lse=lse, workspace=ws)
    full = torch.cat([prefix_pages.repeat(B, 1), ri.block_table], dim=1).cuda()
    full_lens = (ri.kv_lens + P).cuda()
    dws = torch.empty(fa.decode_workspace_size(B, H, Hkv, d, full.shape[1]), dtype=torch.uint8,
                      device="cuda")
    o2 = torch.empty_like(o)
    l2 = torch.empty_like(lse)

    def run_decode():
        fa.decode_paged(q, kp, vp, full, full_lens, out=o2, lse=l2, workspace=dws)
    for _ in range(2):
        run_cascade()
        run_decode()
    t_c = time_steps(torch, run_cascade, reps)
    t_d = time_steps(torch, run_decode, reps)
    diff = (o.float() - o2.float()).abs().max().item()
    kv_row = Hkv * d * 2 * 2
    return {"workload": "64 decode requests, shared prefix 16384 tokens, own 16..512 tokens, "
                        "h32/kv8 d128 bf16",
            "cascade_ms": t_c, "decode_over_full_tables_ms": t_d, "speedup": t_d / t_c,
            "prefix_splits": S, "max_abs_diff_bf16_out": diff,
            "kv_bytes_cascade": float(P + int(own.sum())) * kv_row,
            "kv_bytes_decode": float(B * P + int(own.sum())) * kv_row}


def stream_read_rate(torch, fa, nbytes=4 << 30, reps=20):
    """Read bandwidth of the library's plain streaming-read kernel over a buffer
    far larger than L2 and the last-level cache: what a memory-bound kernel
    can reach here, beside the published peak."""
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    fa.stream_read(buf, sink)
    ms = time_steps(torch, lambda: fa.stream_read(buf, sink), reps)
    del buf
    return dict(value=nbytes / (ms * 1e-3) / 1e9, unit="GB/s", bytes=nbytes, ms_mean=ms)


def copy_calibration(torch, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling HBM byte counters."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes,
                      "dispatches": reps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--parts",
                    default="prefill,decode,long,small,batch1,variants,graph,paged,cascade",
                    help="comma list: prefill, decode (the timed step), long (the 64K-token "
                         "causal prefill), small (the fp32 256-token head and the 12-head "
                         "2048-token fp16/fp32 runs), batch1 (one 32K-token decode), variants "
                         "(windowed and soft-capped decode), graph (graph-replayed decode "
                         "step), paged (ragged queries over a paged cache), cascade "
                         "(shared-prefix decode)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of each oracle baseline sample (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only; the library has no multi-GPU "
              "path, so --gpus must be 1 (the per-GPU share is the whole workload).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_tiled_attention_11_amd as fa
    from exact_tiled_attention_11_amd import inputs

    if args.copy_calibration:
        copy_calibration(torch)
        return

    parts = set(args.parts.split(","))
    dev = "cuda"
    pp = inputs.WORKLOADS[PREFILL].params
    dp = inputs.WORKLOADS[DECODE].params
    B, H, N, d = pp["B"], pp["H"], pp["N"], pp["d"]

    flops = causal_flops(B, H, N, d)
    if "prefill" in parts or args.cpu_seconds > 0:
        log(f"bench: generating {PREFILL} inputs")
        q, k, v = inputs.prefill_inputs(B, H, pp["Hkv"], N, N, d, torch.bfloat16, pp["seed"])
    if "prefill" in parts:
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        o = torch.empty_like(qd)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

    lens = inputs.uniform_lengths(dp["B"], dp["len_lo"], dp["len_hi"], dp["seed"])
    kv_bytes = float(lens.sum()) * dp["Hkv"] * dp["d"] * 2 * 2
    need_decode = bool(parts & {"decode", "variants", "graph"})
    if need_decode or args.cpu_seconds > 0:
        log(f"bench: generating {DECODE} inputs")
        pi = inputs.paged_decode_inputs(dp["B"], dp["H"], dp["Hkv"], dp["d"], lens, dp["seed"],
                                        pool_factor=dp["pool_factor"],
                                        max_pages=dp["len_hi"] // 16)
    if need_decode:
        dq, dk, dv = pi.q.to(dev), pi.k_pool.to(dev), pi.v_pool.to(dev)
        dt_, ds_ = pi.block_table.to(dev), pi.seq_lens.to(dev)
        od = torch.empty_like(dq)
        lsed = torch.empty((dp["B"], dp["H"]), dtype=torch.float32, device=dev)
        ws = torch.empty(fa.decode_workspace_size(dp["B"], dp["H"], dp["Hkv"], dp["d"],
                                                  dt_.shape[1]), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if "prefill" in parts:
            fa.forward(qd, kd, vd, causal=True, out=o, lse=lse)
        if ev is not None:
            ev[1].record()
        if "decode" in parts:
            fa.decode_paged(dq, dk, dv, dt_, ds_, out=od, lse=lsed, workspace=ws)
        if ev is not None:
            ev[2].record()

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    log(f"bench: prefill ms mean {pre_ms.mean():.3f} min {pre_ms.min():.3f}; "
        f"decode ms mean {dec_ms.mean():.3f} min {dec_ms.min():.3f}")

    next_rows = {}
    if need_decode:
        ddev = dict(q=dq, k=dk, v=dv, t=dt_, s=ds_)
        if "variants" in parts:
            log("bench: windowed / soft-capped decode")
            next_rows["decode_window_softcap"] = bench_decode_variants(
                torch, fa, inputs, pi, ddev, lens, dp, args.steps)
        if "graph" in parts:
            log("bench: graph-replayed decode step")
            next_rows["decode_graph"] = bench_decode_graph(torch, fa, inputs, ddev, dp)

    long_prefill = None
    if "long" in parts:
        log(f"bench: {LONG}")
        long_prefill = bench_long_prefill(torch, fa, inputs)
    small = None
    if "small" in parts:
        log("bench: single-head fp32 and 12-head d64 forward runs")
        small = bench_small_configs(torch, fa, inputs)
    batch1 = None
    if "batch1" in parts:
        log("bench: one-sequence 32K-token decode")
        batch1 = bench_decode_batch1(torch, fa, inputs)

    if "paged" in parts:
        log("bench: ragged queries over a paged cache")
        next_rows["forward_paged"] = bench_forward_paged(torch, fa, inputs)
    if "cascade" in parts:
        log("bench: cascade over a shared prefix")
        next_rows["cascade"] = bench_cascade(torch, fa, inputs)

    read_rate = None
    if "decode" in parts:
        log("bench: plain streaming-read rate")
        read_rate = stream_read_rate(torch, fa)

    pre_tflops = flops / (pre_ms.mean() * 1e-3) / 1e12 if "prefill" in parts else None
    dec_gbps = kv_bytes / (dec_ms.mean() * 1e-3) / 1e9 if "decode" in parts else None
    tr_pre, tr_dec = measured_traffic("prefill"), measured_traffic("decode")

    cpu = None
    cpu_dec = None
    if args.cpu_seconds > 0:
        log("bench: timing the CPU oracle baseline")
        cpu = cpu_baseline_prefill(q, k, v, d, args.cpu_seconds)
        cpu_dec = cpu_baseline_decode(pi, d, args.cpu_seconds / 2)

    line = {
        "metric": "prefill attn TFLOP/s (% MFMA peak); split-KV decode KV GB/s (% HBM peak)",
        "value": pre_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PREFILL + " + " + DECODE, "prefill": {k_: pp[k_] for k_ in
                   ("B", "H", "Hkv", "N", "d")} | {"causal": True},
                   "decode": {k_: dp[k_] for k_ in ("B", "H", "Hkv", "d", "page", "len_lo",
                                                      "len_hi")} | {"splits": "auto"}},
        "roofline": None if pre_tflops is None else {
            "bound": "mfma", "achieved": pre_tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": pre_tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": tr_pre["hbm_bytes_per_launch"] if tr_pre else None,
            "traffic_detail": tr_pre,
            "kernel": "fwd16_kernel<BF16, bf16 out, d=128, causal, 8 waves, paired query blocks>",
            "ms_mean": float(pre_ms.mean()), "ms_median": float(np.median(pre_ms)),
            "ms_min": float(pre_ms.min()),
            "algorithmic_flop_per_launch": flops},
        "decode": None if dec_gbps is None else {
            "value": dec_gbps, "unit": "GB/s", "bound": "hbm", "peak": HBM_PEAK_GBPS,
            "frac": dec_gbps / HBM_PEAK_GBPS, "ms_mean": float(dec_ms.mean()),
            "ms_median": float(np.median(dec_ms)), "ms_min": float(dec_ms.min()),
            "kv_bytes": kv_bytes,
            "timed": "decode kernel + merge kernel",
            "stream_read": read_rate,
            "frac_of_stream_read": dec_gbps / read_rate["value"] if read_rate else None,
            "traffic": tr_dec["hbm_bytes_per_launch"] if tr_dec else None,
            "traffic_detail": tr_dec},
        "long_prefill": long_prefill,
        "small_forward": small,
        "decode_batch1_32k": batch1,
        "cpu_baseline": cpu,
        "cpu_baseline_decode": cpu_dec,
        "next_rows": next_rows or None,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
