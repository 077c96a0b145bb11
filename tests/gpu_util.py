"""Helpers for the GPU parity tests: device transfer of seeded inputs and the
tolerance rules.

Tolerances (stated in one place):
  * fp32 storage: |out - ref| <= 1e-5 elementwise (ref = float64 oracle).
  * bf16 storage: |out - ref| <= 1e-2 + 2^-8 |ref| elementwise.  2^-8 |x| is
    at least half a bf16 ulp of x, so this is 1e-2 of compute error on top of
    the error of merely storing the exact value in bf16 (which alone exceeds
    1e-2 once |ref| >= 4).  The plain max abs error, the count of elements
    above 1e-2 and the smallest |ref| among them are reported alongside.
  * LSE (fp32 in every variant): |out - ref| <= 1e-3.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads as W

BF16_ABS = 1e-2
BF16_REL = 2.0 ** -8
F32_ABS = 1e-5
LSE_ABS = 1e-3


def require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_31_amd as fa
    fa.lib()   # raises if libfattn.so is missing: no silent fallback
    return torch, fa


def bf16_to_dev(bits: np.ndarray, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def f32_to_dev(x: np.ndarray, torch):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_bf16_bits(t) -> np.ndarray:
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def dev_bf16_to_f64(t) -> np.ndarray:
    return W.bf16_bits_to_f32(dev_bf16_bits(t)).astype(np.float64)


def dev_to_f64(t) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def check_bf16(out: np.ndarray, ref: np.ndarray, what: str) -> dict:
    assert out.shape == ref.shape, (what, out.shape, ref.shape)
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    err = np.abs(out - ref)
    bound = BF16_ABS + BF16_REL * np.abs(ref)
    bad = err > bound
    over = err > BF16_ABS
    info = dict(max_abs=float(err.max()) if err.size else 0.0, n_over_1e2=int(over.sum()),
                max_ref=float(np.abs(ref).max()) if ref.size else 0.0,
                min_ref_over_1e2=float(np.abs(ref[over]).min()) if over.any() else None)
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; worst at {idx}: "
                             f"out={out[idx]!r} ref={ref[idx]!r} ({info})")
    return info


def check_f32(out: np.ndarray, ref: np.ndarray, what: str, tol: float = F32_ABS) -> float:
    assert out.shape == ref.shape, (what, out.shape, ref.shape)
    err = np.abs(out - ref)
    m = float(err.max()) if err.size else 0.0
    assert m <= tol, f"{what}: max abs error {m} > {tol}"
    return m


def check_lse(out: np.ndarray, ref: np.ndarray, what: str) -> float:
    return check_f32(out, ref, what + " (lse)", LSE_ABS)


def dev_inputs(inp: W.Inputs, torch):
    """q, k, v (and dO) as device tensors holding exactly the generated bits."""
    if inp.w.dtype == "bf16":
        q, k, v = (bf16_to_dev(getattr(inp, n + "_bits"), torch) for n in ("q", "k", "v"))
        do = bf16_to_dev(inp.do_bits, torch) if inp.do_bits is not None else None
    else:
        q, k, v = (f32_to_dev(getattr(inp, n), torch) for n in ("q", "k", "v"))
        do = f32_to_dev(inp.do, torch) if inp.do is not None else None
    return q, k, v, do


def fwd_launch_shape(B: int, H: int, Hkv: int, N: int, causal: bool = True, window: int = 0):
    """(waves per workgroup, query heads per workgroup, workgroups) that the
    bf16 forward picks for these sizes.  Mirrors the host rule in the
    forward's launcher: workgroups of 8 waves x 32 rows serve `hp` query heads
    of one kv head (4, 2 or 1 as the group size allows); the launch falls back
    to 4-wave workgroups when the 8-wave grid has fewer than 512 workgroups
    (two per CU) or for a local window of at most 2048 keys."""
    rep = H // Hkv

    def grid(waves):
        hp = 4 if rep % 4 == 0 and waves % 4 == 0 else 2 if rep % 2 == 0 and waves % 2 == 0 else 1
        rows_h = (waves // hp) * 32
        return hp, -(-N // rows_h) * B * H // hp

    local = causal and 0 < window < N
    hp8, items8 = grid(8)
    if (local and window <= 2048) or items8 < 512:
        return (4, *grid(4))
    return 8, hp8, items8
