"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module holds no arithmetic of the attention method.  It only draws
random tensors, rounds them to the storage format the HIP path consumes
(bf16, round-to-nearest-even, done with integer bit operations; or OCP FP8
e4m3 codes with a per-tensor scale), and decodes those back exactly.  Both sides of every parity check consume the very
same bits: the HIP path as bf16 device tensors, the oracle as float64 values
upcast exactly from them.

Workloads (the pages use random tensors only, so these are the whole inputs):

  C1  fp32, B=1 H=1 Hkv=1 N=256   d=64,  non-causal, seed 1
  C2  bf16, B=4 H=16 Hkv=16 N=2048 d=128, causal,    seed 2
  C3  bf16, B=1 H=32 Hkv=8 N=8192  d=128, causal,    seed 3, 1% of K rows x8
  C4  bf16, B=1 H=32 Hkv=8 N=32768 d=128, causal,    seed 4, 512 sampled rows
  C5  bf16, B=2 H=16 Hkv=16 N=4096 d=128, causal,    seed 5, backward with dO
  F3  fp8 (e4m3 codes + per-tensor scales) of C3's draws (seed 3, same outliers)

Draw order inside one generator: q, k, v, then dO (backward workloads only),
then the outlier key rows (C3 only), then sampled rows (C4 only).  Values are
iid N(0, 1) drawn as float32 by ``numpy.random.default_rng(seed)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np


# --------------------------------------------------------------------------
# bf16 storage format (bit operations only)
# --------------------------------------------------------------------------

def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    NaN maps to the canonical quiet NaN 0x7FC0; overflow past the largest
    finite bf16 rounds to infinity, as IEEE rounding does.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> the nearest bf16 value, returned as float32."""
    return bf16_bits_to_f32(bf16_rne_bits(x))


# --------------------------------------------------------------------------
# FP8 storage format: OCP 8-bit floating point, E4M3 variant
# --------------------------------------------------------------------------
# Sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 holds the
# subnormals m * 2^-9; there are no infinities and S.1111.111 is NaN, so the
# largest finite magnitude is 1.75 * 2^8 = 448.

def _e4m3_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            t[c] = np.nan
            continue
        v = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        t[c] = -v if c & 0x80 else v
    return t


E4M3_VALUES = _e4m3_table()
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """e4m3 codes (uint8) -> float64 values, exact."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_rne_codes(x: np.ndarray) -> np.ndarray:
    """float64 -> e4m3 codes, round to nearest, ties to even, magnitudes
    beyond 448 saturate to 448; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.minimum(np.abs(x), 2.0 * E4M3_MAX))
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    # subnormal range: multiples of 2^-9 (the count 8 is 2^-6, code 0x08)
    sub = np.rint(a * 2.0 ** 9).astype(np.int64)
    f, ex = np.frexp(np.where(a > 0, a, 1.0))         # a = f 2^ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1                       # a in [2^e, 2^(e+1))
    m = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = e + carry
    m = np.where(carry, 0, m)
    normal = ((e + 7) << 3) | m
    code = np.where(a < 2.0 ** -6, sub, normal)
    code = np.minimum(code, 0x7E)                     # saturate at 448
    code = np.where(nan, 0x7F, code | sign)
    return code.astype(np.uint8)


def fp8_quantize(x: np.ndarray) -> tuple[np.ndarray, float]:
    """Per-tensor scale descale = amax / 448 (rounded to float32) and the
    e4m3 codes of x / descale; the stored values are descale * e4m3(code)."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    descale = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
    return e4m3_rne_codes(np.asarray(x, dtype=np.float64) / descale), descale


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str  # "f32", "bf16" or "fp8": the storage type of q, k, v (and o, dO;
                # fp8 workloads produce a bf16 o)
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    causal: bool
    seed: int
    backward: bool = False
    outlier_frac: float = 0.0   # fraction of key rows per (b, kv head) scaled
    outlier_mult: float = 1.0   # ... by this factor
    n_sampled_rows: int = 0     # sampled (h, i) query rows for full-size checks
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    # ---- work and byte counts used by the benchmark -----------------------
    def causal_adjusted_flops(self) -> float:
        """Two contractions of 2*N*N*d flops per head; halved under causal
        masking (only the visible lower triangle is counted)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    def compulsory_bytes(self) -> int:
        """Bytes the forward must move at least once: Q, K, V in, O and LSE out."""
        e = 4 if self.dtype == "f32" else 2
        q = self.B * self.H * self.N * self.d * e
        kv = 2 * self.B * self.Hkv * self.N * self.d * e
        o = q
        lse = self.B * self.H * self.N * 4
        return q + kv + o + lse


C1 = Workload("C1", "f32", 1, 1, 1, 256, 64, False, 1,
              note="single-head non-causal fp32, 64x64 tiles")
C2 = Workload("C2", "bf16", 4, 16, 16, 2048, 128, True, 2,
              note="multi-head causal bf16")
C3 = Workload("C3", "bf16", 1, 32, 8, 8192, 128, True, 3,
              outlier_frac=0.01, outlier_mult=8.0,
              note="Llama-3.1-8B-shaped GQA causal, 1% of K rows x8")
C4 = Workload("C4", "bf16", 1, 32, 8, 32768, 128, True, 4,
              n_sampled_rows=512,
              note="long-context causal, 512 sampled rows")
C5 = Workload("C5", "bf16", 2, 16, 16, 4096, 128, True, 5, backward=True,
              note="backward with recomputation")

F3 = replace(C3, name="F3", dtype="fp8")

WORKLOADS = {w.name: w for w in (C1, C2, C3, C4, C5, F3)}


@dataclass
class Inputs:
    """Generated tensors.  For bf16 workloads the ``*_bits`` arrays hold the
    uint16 patterns and the float arrays hold the same values as float32."""
    w: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray | None = None
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None
    do_bits: np.ndarray | None = None
    outlier_rows: np.ndarray | None = None   # [B, Hkv, n_out] key indices
    sampled_rows: np.ndarray | None = None   # [n, 2] (h, i) pairs, b = 0
    # fp8 workloads: e4m3 codes and per-tensor scales; q, k, v then hold the
    # represented values descale * e4m3(code) as float64
    q_codes: np.ndarray | None = None
    k_codes: np.ndarray | None = None
    v_codes: np.ndarray | None = None
    descale: dict | None = None

    def f64(self, name: str) -> np.ndarray:
        return getattr(self, name).astype(np.float64)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def gen_inputs(w: Workload, seed: int | None = None) -> Inputs:
    """Draw the workload's tensors.  Layout: q, dO [B, H, N, d];
    k, v [B, Hkv, N, d]; all row-major."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = _normal(rng, (w.B, w.H, w.N, w.d))
    k = _normal(rng, (w.B, w.Hkv, w.N, w.d))
    v = _normal(rng, (w.B, w.Hkv, w.N, w.d))
    do = _normal(rng, (w.B, w.H, w.N, w.d)) if w.backward else None

    outliers = None
    if w.outlier_frac > 0.0:
        n_out = int(round(w.outlier_frac * w.N))
        outliers = np.empty((w.B, w.Hkv, n_out), dtype=np.int64)
        for b in range(w.B):
            for g in range(w.Hkv):
                idx = np.sort(rng.choice(w.N, size=n_out, replace=False))
                outliers[b, g] = idx
                k[b, g, idx, :] *= np.float32(w.outlier_mult)

    sampled = None
    if w.n_sampled_rows > 0:
        sampled = sample_rows(rng, w.H, w.N, w.n_sampled_rows)

    inp = Inputs(w, q, k, v, do, outlier_rows=outliers, sampled_rows=sampled)
    if w.dtype == "fp8":
        inp.descale = {}
        for name in ("q", "k", "v"):
            codes, ds = fp8_quantize(getattr(inp, name))
            setattr(inp, name + "_codes", codes)
            inp.descale[name] = ds
            setattr(inp, name, e4m3_decode(codes) * ds)
    if w.dtype == "bf16":
        # x8 is exact in bf16, so scaling before or after rounding is the same.
        for name in ("q", "k", "v", "do"):
            arr = getattr(inp, name)
            if arr is None:
                continue
            bits = bf16_rne_bits(arr)
            setattr(inp, name + "_bits", bits)
            setattr(inp, name, bf16_bits_to_f32(bits))
    return inp


def sample_rows(rng: np.random.Generator, H: int, N: int, n: int) -> np.ndarray:
    """n distinct (h, i) query rows; always includes i in {0, 127, 128, N-1}
    (on heads 0..3) when N allows, the rest drawn without replacement."""
    fixed = [i for i in (0, 127, 128, N - 1) if 0 <= i < N]
    fixed = sorted(set(fixed))
    pairs = [(hh % H, i) for hh, i in enumerate(fixed)]
    taken = {h * N + i for h, i in pairs}
    need = max(0, min(n, H * N) - len(pairs))
    while need > 0:
        cand = rng.choice(H * N, size=need, replace=False)
        for c in cand:
            c = int(c)
            if c not in taken:
                taken.add(c)
                pairs.append((c // N, c % N))
        need = max(0, min(n, H * N) - len(pairs))
    pairs = pairs[:n]
    return np.array(sorted(pairs), dtype=np.int64).reshape(-1, 2)


def small_case(name: str, dtype: str, B: int, H: int, Hkv: int, N: int, d: int,
               causal: bool, seed: int, backward: bool = False,
               outlier_frac: float = 0.0, outlier_mult: float = 1.0) -> Workload:
    """A reduced workload with the same structure, for element-by-element parity."""
    return Workload(name, dtype, B, H, Hkv, N, d, causal, seed, backward,
                    outlier_frac, outlier_mult)
