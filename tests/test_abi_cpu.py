"""The C ABI on a host without a GPU: the library loads, exports every entry
point the header declares, and rejects invalid calls before any HIP call."""

import ctypes
import os
import re

import pytest

import exact_tiled_attention_11_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, NULL, SHAPE, UNSUP, WS, HIP, ARG, SCRATCH = range(8)
F32, F16, BF16 = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"fa_forward", "fa_decode_paged", "fa_merge_partials"} <= set(names)
    lib = ctypes.CDLL(fa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in fa.h but not exported"


def test_binding_covers_every_declared_function():
    for n in declared_functions():
        assert n in fa._SIGNATURES, f"{n} has no ctypes signature"


def test_status_strings_and_version():
    for s in range(8):
        assert fa.status_string(s).startswith("FA_")
    assert fa.status_string(99) == "unknown fa_status"
    assert re.fullmatch(r"\d+\.\d+\.\d+", fa.version())


def fwd(B=1, H=1, Hkv=1, Nq=1, Nk=1, d=64, scale=0.125, causal=0, ind=BF16, outd=BF16,
        ptrs=(None,) * 5):
    return fa.lib().fa_forward(*ptrs, B, H, Hkv, Nq, Nk, d, scale, causal, ind, outd, None)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), SHAPE), (dict(Nq=-1), SHAPE), (dict(Nk=-1), SHAPE), (dict(H=0), SHAPE),
    (dict(Hkv=0), SHAPE), (dict(H=3, Hkv=2), SHAPE), (dict(d=96), UNSUP), (dict(d=256), UNSUP),
    (dict(ind=7), ARG), (dict(outd=-1), ARG), (dict(causal=2), ARG),
    (dict(scale=0.0), ARG), (dict(scale=-1.0), ARG), (dict(scale=float("inf")), ARG),
    (dict(scale=float("nan")), ARG), (dict(ind=BF16, outd=F16), UNSUP),
    (dict(ind=F32, outd=BF16), UNSUP),
    (dict(B=1 << 14, Nq=1 << 14, H=16, d=128), SHAPE),
    # 2^24 workgroups of 512 threads: more than 2^32 - 1 threads along x
    (dict(B=1 << 24, Nq=1, Nk=1, d=64), SHAPE),
    (dict(B=(1 << 24) - 1, Nq=1, Nk=1, d=64, ind=F32, outd=F32), NULL),
    (dict(B=1 << 24, Nq=1, Nk=1, d=64, ind=F32, outd=F32), SHAPE),
    (dict(), NULL), (dict(B=0), OK), (dict(Nq=0), OK),
])
def test_forward_validation(kw, status):
    assert fwd(**kw) == status


def test_forward_null_checks():
    p = [FAKE] * 5
    for i in range(5):
        q = list(p)
        q[i] = None
        expect = NULL
        assert fwd(ptrs=q) == expect
    # K and V may be NULL when there are no keys, Q/O/LSE may not
    assert fwd(Nk=0, ptrs=[None, None, None, FAKE, FAKE]) == NULL


def test_forward_alignment_check():
    odd = ctypes.c_void_p(0x1008)
    high = ctypes.c_void_p(1 << 48)   # aligned, but beyond the 48-bit address space
    p = [FAKE] * 5
    for bad in (odd, high):
        for i in (0, 1, 2, 3):
            q = list(p)
            q[i] = bad
            assert fwd(ptrs=q) == ARG


def dec(B=2, H=8, Hkv=2, d=128, page=16, max_pages=4, num_pages=8, scale=0.1, splits=0,
        dt=BF16, outd=BF16, ptrs=(None,) * 7, ws=None, ws_bytes=0):
    return fa.lib().fa_decode_paged(*ptrs, B, H, Hkv, d, page, max_pages, num_pages, scale,
                                    splits, dt, outd, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), SHAPE), (dict(H=0), SHAPE), (dict(H=6, Hkv=4), SHAPE),
    (dict(max_pages=0), SHAPE), (dict(num_pages=0), SHAPE), (dict(page=0), SHAPE),
    (dict(splits=-1), ARG), (dict(splits=65), ARG), (dict(dt=9), ARG),
    (dict(scale=0.0), ARG), (dict(d=96), UNSUP), (dict(page=8), UNSUP),
    (dict(page=32), UNSUP), (dict(dt=F32, outd=F32), UNSUP), (dict(H=51, Hkv=3), UNSUP),
    (dict(H=34, Hkv=2), UNSUP), (dict(H=32, Hkv=1), UNSUP), (dict(dt=F16, outd=BF16), UNSUP),
    (dict(H=48, Hkv=3), NULL), (dict(H=32, Hkv=2), NULL), (dict(H=18, Hkv=3), NULL),
    (dict(splits=64), NULL),
    (dict(B=70000), SHAPE), (dict(), NULL), (dict(B=0), OK),
])
def test_decode_validation(kw, status):
    assert dec(**kw) == status


def dec_ex(window=0, softcap=0.0, B=2, H=8, Hkv=2, d=128, page=16, max_pages=4, num_pages=8,
           scale=0.1, splits=0, dt=BF16, outd=BF16, ptrs=(None,) * 7, ws=None, ws_bytes=0):
    return fa.lib().fa_decode_paged_ex(*ptrs, B, H, Hkv, d, page, max_pages, num_pages, scale,
                                       splits, window, softcap, dt, outd, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(window=-1), ARG), (dict(softcap=-1.0), ARG), (dict(softcap=float("nan")), ARG),
    (dict(softcap=float("inf")), ARG), (dict(window=5, B=0), OK), (dict(softcap=30.0), NULL),
    (dict(window=4096, softcap=50.0, d=96), UNSUP), (dict(window=3, splits=65), ARG),
    (dict(B=-1, window=1), SHAPE), (dict(window=1, B=0), OK),
])
def test_decode_ex_validation(kw, status):
    assert dec_ex(**kw) == status


def test_decode_ex_workspace_checks():
    p = [FAKE] * 7
    need = fa.decode_workspace_size(2, 8, 2, 128, 200, 2000, 0)
    assert fa.decode_max_splits(2, 2, 200, 2000) == 2
    assert dec_ex(window=2000, max_pages=200, ptrs=p, ws=None, ws_bytes=need) == WS
    assert dec_ex(window=2000, max_pages=200, ptrs=p, ws=FAKE, ws_bytes=need - 1) == WS


def test_decode_graph_validation_before_any_hip_call():
    lib = fa.lib()
    p = [FAKE] * 7
    h = ctypes.c_void_p()

    def create(out, window=0, softcap=0.0, splits=0, ptrs=p, B=2, ws=None, ws_bytes=0):
        return lib.fa_decode_graph_create(out, *ptrs, B, 8, 2, 128, 16, 200, 8, 0.1, splits,
                                          window, softcap, BF16, BF16, ws, ws_bytes)
    assert create(None) == NULL
    assert create(ctypes.byref(h), window=-1) == ARG
    assert h.value is None
    assert create(ctypes.byref(h), softcap=float("nan")) == ARG
    assert create(ctypes.byref(h), splits=65) == ARG
    assert create(ctypes.byref(h), ptrs=[None] * 7) == NULL
    assert create(ctypes.byref(h), ws=None, ws_bytes=0) == WS
    assert lib.fa_decode_graph_launch(None, None) == NULL
    lib.fa_decode_graph_destroy(None)


def fwdp(B=2, H=8, Hkv=2, d=128, total_q=10, max_q=8, page=16, max_pages=4, num_pages=8,
         scale=0.1, causal=1, dt=BF16, outd=BF16, ptrs=(None,) * 8):
    return fa.lib().fa_forward_paged(*ptrs, B, H, Hkv, d, total_q, max_q, page, max_pages,
                                     num_pages, scale, causal, dt, outd, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), SHAPE), (dict(H=0), SHAPE), (dict(H=6, Hkv=4), SHAPE),
    (dict(total_q=-1), SHAPE), (dict(max_q=-1), SHAPE), (dict(max_pages=0), SHAPE),
    (dict(num_pages=0), SHAPE), (dict(page=0), SHAPE), (dict(dt=7), ARG), (dict(causal=2), ARG),
    (dict(scale=float("nan")), ARG), (dict(d=96), UNSUP), (dict(page=32), UNSUP),
    (dict(dt=F32, outd=F32), UNSUP), (dict(dt=F16, outd=BF16), UNSUP),
    (dict(total_q=1 << 24, H=64), SHAPE), (dict(), NULL), (dict(B=0), OK),
    (dict(total_q=0), OK), (dict(max_q=0), OK),
])
def test_forward_paged_validation(kw, status):
    assert fwdp(**kw) == status


def test_forward_paged_alignment_check():
    odd = ctypes.c_void_p(0x1002)
    for i in (0, 2, 3, 6):
        p = [FAKE] * 8
        p[i] = odd
        assert fwdp(ptrs=p) == ARG


def casc(prefix_len=100, prefix_splits=0, B=2, H=8, Hkv=2, d=128, total_q=10, max_q=8, page=16,
         max_pages=4, num_pages=8, scale=0.1, causal=1, dt=BF16, outd=BF16, ptrs=(None,) * 8,
         ws=None, ws_bytes=0):
    q, ind, k, v, pp, bt, kl, o = ptrs
    return fa.lib().fa_cascade(q, ind, k, v, pp, prefix_len, prefix_splits, bt, kl, o, None,
                               B, H, Hkv, d, total_q, max_q, page, max_pages, num_pages, scale,
                               causal, dt, outd, ws, ws_bytes, None)


def test_cascade_split_rule_and_workspace():
    # explicit count wins; automatic: enough workgroups, at least 512 prefix keys each, <= 64
    assert fa.cascade_num_splits(10000, 64, 32, 8, 5) == 5
    assert fa.cascade_num_splits(100, 64, 32, 8, 0) == 1
    assert fa.cascade_num_splits(16384, 64, 32, 8, 0) == 32
    assert fa.cascade_num_splits(10**6, 64, 32, 8, 0) == 64
    assert fa.cascade_num_splits(10**6, 65536, 32, 8, 0) == 1
    assert fa.cascade_num_splits(0, 64, 32, 8, 0) == 1
    assert fa.cascade_num_splits(-1, 64, 32, 8, 0) == -1
    assert fa.cascade_num_splits(100, 64, 32, 8, 65) == -1
    assert fa.cascade_num_splits(100, 64, 32, 6, 0) == -1
    ws = fa.cascade_workspace_size(10, 8, 128, 4)
    rows = 80
    assert ws == (rows * 4 * 128 * 4) + -(-rows * 4 * 4 // 256) * 256 + rows * 128 * 4 + rows * 4
    assert fa.cascade_workspace_size(10, 8, 128, 0) == 0
    assert fa.cascade_workspace_size(10, 8, 128, 65) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(prefix_len=-1), ARG), (dict(prefix_splits=-1), ARG), (dict(prefix_splits=65), ARG),
    (dict(B=-1), SHAPE), (dict(H=6, Hkv=4), SHAPE), (dict(total_q=-1), SHAPE), (dict(dt=7), ARG),
    (dict(causal=3), ARG), (dict(scale=0.0), ARG), (dict(d=80), UNSUP), (dict(page=8), UNSUP),
    (dict(dt=F32, outd=F32), UNSUP), (dict(total_q=0), OK), (dict(), NULL),
])
def test_cascade_validation(kw, status):
    assert casc(**kw) == status


def test_cascade_pointer_and_workspace_checks():
    p = [FAKE] * 8
    assert casc(ptrs=p) == NULL   # LSE is NULL in every call of this helper
    need = fa.cascade_workspace_size(10, 8, 128, fa.cascade_num_splits(100, 10, 8, 2, 0))
    lib = fa.lib()

    def call(prefix_len, ws, ws_bytes, pp=FAKE):
        return lib.fa_cascade(FAKE, FAKE, FAKE, FAKE, pp, prefix_len, 0, FAKE, FAKE, FAKE, FAKE,
                              2, 8, 2, 128, 10, 8, 16, 4, 8, 0.1, 1, BF16, BF16, ws, ws_bytes,
                              None)
    assert call(100, None, 0) == WS
    assert call(100, FAKE, need - 1) == WS
    assert call(100, FAKE, need, pp=None) == NULL
    odd = ctypes.c_void_p(0x1002)
    assert lib.fa_cascade(odd, FAKE, FAKE, FAKE, FAKE, 100, 0, FAKE, FAKE, FAKE, FAKE, 2, 8, 2,
                          128, 10, 8, 16, 4, 8, 0.1, 1, BF16, BF16, FAKE, need, None) == ARG


def test_decode_workspace_checks():
    p = [FAKE] * 7
    # B = 2, Hkv = 2: chunks of 1024 tokens. 4 pages of 16 tokens: one chunk at
    # most, no workspace needed; 200 pages: ceil(3200 / 1024) = 4 slots
    assert fa.decode_max_splits(2, 2, 4) == 1 and fa.decode_max_splits(2, 2, 200) == 4
    need = fa.decode_workspace_size(2, 8, 2, 128, 200, 0, 0)
    assert need > 0
    assert dec(max_pages=200, ptrs=p, ws=None, ws_bytes=need) == WS
    assert dec(max_pages=200, ptrs=p, ws=FAKE, ws_bytes=need - 1) == WS
    need4 = fa.decode_workspace_size(2, 8, 2, 128, 4, 0, 4)
    assert dec(ptrs=p, splits=4, ws=FAKE, ws_bytes=need4 - 4) == WS
    # a workspace that is large enough but not 16-byte aligned
    assert dec(max_pages=200, ptrs=p, ws=ctypes.c_void_p(0x1008), ws_bytes=need) == ARG


def plan_by_hand(lens, Hkv, max_pages, window=0, fixed=0):
    """The split plan written out from its definition."""
    L = max_pages * 16
    vis = [0 if (x < 0 or x > L) else (min(x, window) if window > 0 else x) for x in lens]
    P = max(1, len(lens)) * Hkv
    C = min(4096, max(1024, 4 * P))
    Lv = min(L, window) if window > 0 else L
    S = fixed if fixed > 0 else min(64, max(1, min(-(-Lv // C), -(-4096 // P))))
    if fixed > 0:
        return [fixed] * len(lens), S
    return [min(S, max(1, -(-v // C))) for v in vis], S


def test_split_plan_and_workspace_size():
    from exact_tiled_attention_11_amd import inputs
    # slots: min(ceil(L / C), ceil(4096 / P)), C = clamp(4 P, 1024, 4096), P = B Hkv
    assert [fa.decode_max_splits(1, 8, mp) for mp in (1, 64, 65, 2048, 4096, 8192)] == \
        [1, 1, 2, 32, 64, 64]
    assert [fa.decode_max_splits(B, 8, 2048) for B in (1, 8, 16, 24, 32, 64, 128, 256)] == \
        [32, 32, 32, 22, 16, 8, 4, 2]
    assert fa.decode_max_splits(64, 8, 2048, 4096) == 2
    assert fa.decode_max_splits(1, 8, 2048, 4096) == 4
    assert fa.decode_max_splits(1, 8, 2048, 100) == 1
    assert fa.decode_max_splits(64, 8, 2048, 0, 7) == 7
    assert fa.decode_max_splits(1, 8, 0) == -1 and fa.decode_max_splits(1, 8, 8, -1) == -1
    assert fa.decode_max_splits(1, 8, 8, 0, 65) == -1 and fa.decode_max_splits(1, 0, 8) == -1
    # one sequence of 32K tokens over 8 KV heads: chunks of 1024 tokens, 256 workgroups
    assert list(fa.decode_plan([32768], 8, 2048)) == [32]
    assert list(fa.decode_plan([32768], 1, 2048)) == [32]
    assert list(fa.decode_plan([32768] * 8, 8, 2048)) == [32] * 8
    assert list(fa.decode_plan([1000, 0, 1], 8, 2048)) == [1, 1, 1]
    # the 64-sequence workload: chunks of 2048 tokens, at most 8 per sequence
    lens = [int(x) for x in inputs.uniform_lengths(64, 1024, 32768, 104)]
    got = fa.decode_plan(lens, 8, 2048)
    want, S = plan_by_hand(lens, 8, 2048)
    assert list(got) == want and S == 8
    assert list(got) == [min(8, -(-x // 2048)) for x in lens]
    # with a 4096-token window: two chunks for every sequence that long
    got = fa.decode_plan(lens, 8, 2048, window=4096)
    assert list(got) == plan_by_hand(lens, 8, 2048, 4096)[0]
    assert list(got) == [min(2, -(-x // 2048)) for x in lens]
    # fixed counts, lengths outside the table (visible 0)
    assert list(fa.decode_plan(lens[:3], 8, 2048, 0, 5)) == [5, 5, 5]
    assert list(fa.decode_plan([-1, 10 ** 6, 5000], 2, 2048)) == [1, 1, 5]
    assert list(fa.decode_plan([], 8, 2048)) == []
    with pytest.raises(fa.FAError):
        fa.decode_plan([1], 0, 2048)
    # fp32 o-partials, then fp32 lse-partials at a 256-byte boundary
    assert fa.decode_workspace_size(64, 32, 8, 128, 2048) == \
        64 * 32 * 8 * 128 * 4 + 64 * 32 * 8 * 4
    assert fa.decode_workspace_size(1, 32, 8, 128, 2048) == 32 * 32 * 128 * 4 + 32 * 32 * 4
    assert fa.decode_workspace_size(1, 1, 1, 1, 1, 0, 1) == 256 + 4
    assert fa.decode_workspace_size(1, 1, 1, 1, 1, 0, -1) == 0
    assert fa.decode_workspace_size(1, 1, 1, 1, 1, 0, 65) == 0
    assert fa.decode_workspace_size(1, 1, 1, 1, 0, 0, 0) == 0
    assert fa.decode_workspace_size(1, 3, 2, 1, 1, 0, 0) == 0


@pytest.mark.parametrize("args,status", [
    ((-1, 2, 64, F32), SHAPE), ((4, 0, 64, F32), SHAPE), ((4, 1025, 64, F32), SHAPE),
    ((4, 2, 0, F32), SHAPE), ((4, 2, 1025, F32), SHAPE), ((4, 2, 64, 5), ARG),
    ((4, 2, 64, F32), NULL), ((0, 2, 64, F32), OK),
    # (R + 3) / 4 workgroups of 256 threads: beyond 2^32 - 1 threads along x
    (((1 << 26) - 3, 1, 1, F32), SHAPE), (((1 << 26) - 4, 1, 1, F32), NULL),
])
def test_merge_validation(args, status):
    R, S, d, outd = args
    assert fa.lib().fa_merge_partials(None, None, None, None, None, R, S, d, outd, None) == status


def test_product_path_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)


def test_stream_read_validation_before_any_hip_call():
    lib = fa.lib()
    assert lib.fa_stream_read(None, 0, None, None) == 0          # nothing to read
    assert lib.fa_stream_read(None, 16, FAKE, None) == NULL
    assert lib.fa_stream_read(FAKE, 16, None, None) == NULL
    assert lib.fa_stream_read(ctypes.c_void_p(0x1008), 16, FAKE, None) == ARG
    assert lib.fa_stream_read(FAKE, 24, FAKE, None) == ARG


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it says so and exits before any GPU work."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def dec_noalloc(B=2, H=8, Hkv=2, d=128, page=16, max_pages=4, num_pages=8, scale=0.1, splits=0,
                window=0, softcap=0.0, dt=BF16, outd=BF16, ptrs=(None,) * 7):
    return fa.lib().fa_decode_paged_noalloc(*ptrs, B, H, Hkv, d, page, max_pages, num_pages,
                                            scale, splits, window, softcap, dt, outd, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), SHAPE), (dict(splits=65), ARG), (dict(window=-1), ARG),
    (dict(softcap=float("nan")), ARG), (dict(d=96), UNSUP), (dict(H=34, Hkv=2), UNSUP),
    (dict(B=0), OK), (dict(), NULL),
])
def test_decode_noalloc_validation(kw, status):
    assert dec_noalloc(**kw) == status


def test_decode_noalloc_rejects_more_partials_than_its_scratch():
    p = [FAKE] * 7
    # 64 sequences of 128 query heads, 64 fixed splits: 270 MB of partials
    assert fa.decode_workspace_size(64, 128, 8, 128, 2048, 0, 64) > 32 << 20
    assert dec_noalloc(B=64, H=128, Hkv=8, max_pages=2048, num_pages=1 << 16, splits=64,
                       ptrs=p) == SCRATCH
