"""Comparison helpers for the GPU parity tests (the HIP path vs the oracle).

Tolerances: fp32 inputs, max |err| <= 1e-4; bf16/fp16 inputs with fp32
accumulation, max |err| <= 1e-2 and mean |err| <= 1e-3; LSE |err| <= 1e-4.

Low-precision OUTPUTS: a correctly rounded bf16 value can sit 2^-8 * 2^e away
from the exact value, more than 1e-2 once |O| >= 4. So a low-precision run is
checked three ways: the same inputs with fp32 output meet the bounds above;
the low-precision output is exactly the round-to-nearest-even of that fp32
output; and it lies within 1e-2 + half an ulp of the exact value.
"""

from __future__ import annotations

import numpy as np
import torch

F32_MAX = 1e-4
LOWP_MAX = 1e-2
LOWP_MEAN = 1e-3
LSE_MAX = 1e-4

_MANT = {torch.bfloat16: 7, torch.float16: 10}


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def report(name, got, ref):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    print(f"[{name}] max {err.max() if err.size else 0:.3e} mean {err.mean() if err.size else 0:.3e}",
          flush=True)
    return err


def assert_f32(name, got, ref, tol=F32_MAX):
    err = report(name, got, ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert err.max(initial=0) <= tol, f"{name}: max err {err.max():.3e} > {tol}"


def assert_lowp_acc(name, got_f32out, ref):
    err = report(name, got_f32out, ref)
    assert np.all(np.isfinite(got_f32out)), f"{name}: non-finite output"
    assert err.max(initial=0) <= LOWP_MAX, f"{name}: max err {err.max():.3e}"
    assert err.mean() <= LOWP_MEAN, f"{name}: mean err {err.mean():.3e}"


def assert_rounded_from(name, got_lowp: torch.Tensor, got_f32: torch.Tensor):
    """Low-precision output == RNE of the fp32 output of the same computation."""
    expect = got_f32.to(got_lowp.dtype)
    same = torch.equal(got_lowp.view(torch.int16), expect.view(torch.int16))
    assert same, f"{name}: low-precision output is not the rounded fp32 output"


def assert_lowp_out(name, got_lowp: torch.Tensor, ref):
    g = np64(got_lowp)
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 1e-30)))
    half_ulp = np.exp2(e - _MANT[got_lowp.dtype] - 1)
    err = np.abs(g - ref)
    bad = err > LOWP_MAX + half_ulp
    assert not bad.any(), f"{name}: {bad.sum()} values outside 1e-2 + half ulp"


def ulp_f32(x):
    """Spacing of float32 values at |x| (the distance to the next one up)."""
    a = np.abs(np.asarray(x, np.float64)).astype(np.float32)
    return (np.nextafter(a, np.float32(np.inf)) - a).astype(np.float64)


def assert_lse(name, got, ref, tol=LSE_MAX):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{name}: -inf rows differ"
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(got[fin])), f"{name}: non-finite LSE"
    err = report(name + " lse", got[fin], ref[fin])
    assert err.max(initial=0) <= tol, f"{name}: LSE err {err.max():.3e} > {tol}"


def assert_lse_ulp(name, got, ref, ulps=2):
    """LSE within max(1e-4, `ulps` float32 ulps of |LSE|) of the exact value,
    per element: an fp32 result of magnitude beyond a few thousand cannot
    hold 1e-4 absolute (ulp_f32(3000) is 2.4e-4), below that 1e-4 binds."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{name}: -inf rows differ"
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(got[fin])), f"{name}: non-finite LSE"
    err = report(name + " lse", got[fin], ref[fin])
    tol = np.maximum(LSE_MAX, ulps * ulp_f32(ref[fin]))
    bad = err > tol
    assert not bad.any(), f"{name}: {bad.sum()} LSE values beyond max(1e-4, {ulps} ulp)"
