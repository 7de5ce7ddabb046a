"""Seeded synthetic inputs for the sparse gated-FFN forward.

This module only draws and rounds numbers: it holds none of the FFN's
arithmetic, so that both the HIP path and the CPU oracle can consume the same
inputs without sharing any of the computation they are compared on.

Workloads stand in for the activations of the ReLU-gated FFN described in
"Sparser, Faster, Lighter Transformer Language Models Review" (section 1-1 for
the block, section 5-1 / 5-3 for the few dozen active neurons per token and
the per-row spread of more than ten times the mean).  No trained weights or
datasets are involved.

Recipe (one numpy PCG64 stream per workload, fixed draw order):

1. ``x``  ~ N(0, 1), shape [M, K], float32.
2. ``s``  ~ LogNormal(0, sigma_s), shape [M]  (drawn only when sigma_s > 0).
   Each token row ``x[t, :K-1]`` is multiplied by ``s[t]``; the last column
   is then set to exactly 1 and acts as the bias input.
3. ``Wg_t``, ``Wu_t``, ``Wd`` ~ N(0, 1/K), each of shape [N, K], float32.
   ``Wg_t`` and ``Wu_t`` hold W_g and W_u transposed (row j is column j of
   the K->N projection); ``Wd`` is the N->K down projection in its natural
   row-major layout.
4. Per-column biases ``b_j`` are written into ``Wg_t[:, K-1]`` as ``-b_j``
   (the gate sees ``x[t, K-1] * Wg_t[j, K-1] = -b_j``).  A real ``b`` is
   chosen by bisection so that the expected fraction of positive gate
   pre-activations over the draw of W_g equals the target density:
   ``mean_t Q(b / sigma_t) = density`` with
   ``sigma_t**2 = sum_{k<K-1} x[t,k]**2 / K`` and ``Q`` the standard normal
   survival function.  ``b`` is generally not a bfloat16 value, and in the
   far tail one bfloat16 step moves the density by 10-25%, so each column
   takes one of the two bfloat16 neighbours ``b_lo <= b <= b_hi``: a
   fraction ``f`` of the columns, spread evenly over j, takes ``b_lo`` with
   ``f * D(b_lo) + (1 - f) * D(b_hi) = density`` (D the expected density of
   a single bias), so the expected mean density is the target.
5. All arrays are rounded float32 -> bfloat16 with round-to-nearest-even and
   handed out as raw ``uint16`` bit patterns.

``density`` may also be exactly 0.0 or 1.0: the bias is then -B or +B with
``B`` larger than twice any possible ``|sum_{k<K-1} x w|``, which fixes the
sign of every gate entry regardless of rounding order.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_inputs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and sparsity recipe of one FFN-block forward."""

    name: str
    M: int          # tokens
    K: int          # model dimension
    N: int          # expanded FFN dimension
    T: int          # TwELL tile width (columns of h_g per tile)
    C: int          # TwELL capacity per (token-row, tile)
    density: float  # target mean fraction of positive gate entries
    sigma_s: float  # log-normal sigma of the per-token scale (0 = none)
    seed: int = 0

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads of the hot path: a tiny CPU-checkable block, three blocks at
# 0.5B / 1B / 2B scale with 1% / 0.5% / 0.3% active gate entries, an
# overflow-stress block with a heavier per-token tail, and the pages' own
# block width for the break-even sweeps.
WORKLOADS = {
    "tiny": Workload("tiny", 64, 256, 1024, 128, 16, 0.05, 0.0),
    "ffn-0.5b": Workload("ffn-0.5b", 4096, 1024, 4096, 128, 8, 0.01, 0.5),
    "ffn-1b": Workload("ffn-1b", 8192, 1536, 6144, 128, 8, 0.005, 0.5),
    "ffn-2b": Workload("ffn-2b", 16384, 2048, 8192, 256, 16, 0.003, 0.5),
    "ffn-ovf": Workload("ffn-ovf", 16384, 2048, 8192, 128, 4, 0.005, 1.0),
    # the pages' own FFN block width (hidden 5632 over model width 2048) at
    # about 28 active neurons per token, the middle of their observed range
    "ffn-paper": Workload("ffn-paper", 4096, 2048, 5632, 128, 8, 0.005, 0.5),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even).

    Returns the upper 16 bits of the rounded float32 as uint16.  Inputs are
    finite (the generator never produces NaN or Inf).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_sf(z: np.ndarray) -> np.ndarray:
    from scipy.special import erfc

    return 0.5 * erfc(z / math.sqrt(2.0))


def _solve_bias(sigma_t: np.ndarray, density: float) -> float:
    """Bisection for b with mean_t Q(b / sigma_t) == density (float64)."""
    lo, hi = 0.0, 1.0
    f = lambda b: float(np.mean(_normal_sf(b / sigma_t))) - density
    while f(hi) > 0.0:
        hi *= 2.0
    if density >= 0.5:
        lo = -hi
        while f(lo) < 0.0:
            lo *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if f(mid) > 0.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _round_up_bf16(v: float) -> float:
    """Smallest bfloat16 value >= v (v > 0)."""
    b = int(f32_to_bf16_bits(np.array([v], dtype=np.float32))[0])
    r = float(bf16_bits_to_f32(np.array([b], dtype=np.uint16))[0])
    while r < v:
        b += 1
        r = float(bf16_bits_to_f32(np.array([b], dtype=np.uint16))[0])
    return r


def make_inputs(w: Workload) -> dict:
    """Draw the inputs of workload ``w``.

    Returns a dict with uint16 bf16-bit arrays ``x`` [M,K], ``wg_t``, ``wu_t``,
    ``wd`` [N,K], the per-column biases ``bias`` [N] written (negated) into
    ``wg_t[:, K-1]``, and the per-token scales ``s``.
    """
    if w.K < 2 or w.M < 0 or w.N < 1:
        raise ValueError("bad workload shape")
    rng = np.random.default_rng(w.seed)
    M, K, N = w.M, w.K, w.N
    x = rng.standard_normal((M, K), dtype=np.float32)
    if w.sigma_s > 0.0:
        s = rng.lognormal(0.0, w.sigma_s, size=M).astype(np.float32)
    else:
        s = np.ones(M, dtype=np.float32)
    x[:, : K - 1] *= s[:, None]
    x[:, K - 1] = 1.0
    scale = np.float32(1.0 / math.sqrt(K))
    wg = rng.standard_normal((N, K), dtype=np.float32) * scale
    wu = rng.standard_normal((N, K), dtype=np.float32) * scale
    wd = rng.standard_normal((N, K), dtype=np.float32) * scale

    xb = f32_to_bf16_bits(x)
    wgb = f32_to_bf16_bits(wg)
    xr = bf16_bits_to_f32(xb).astype(np.float64)
    if w.density <= 0.0 or w.density >= 1.0:
        wgr = bf16_bits_to_f32(wgb[:, : K - 1]).astype(np.float64)
        big = 2.0 * float(np.abs(xr[:, : K - 1]).sum(axis=1).max(initial=0.0)) * float(
            np.abs(wgr).max(initial=0.0)) + 1.0
        B = _round_up_bf16(big)
        bias = B if w.density <= 0.0 else -B
    elif M == 0:
        bias = 0.0
    else:
        sigma_t = np.sqrt((xr[:, : K - 1] ** 2).sum(axis=1) / K)
        sigma_t = np.maximum(sigma_t, 1e-30)
        bias = _solve_bias(sigma_t, w.density)
    b_lo, b_hi = _bf16_neighbours(bias)
    if b_lo == b_hi or M == 0 or w.density <= 0.0 or w.density >= 1.0:
        frac_lo = 1.0
    else:
        d_lo = float(np.mean(_normal_sf(b_lo / sigma_t)))
        d_hi = float(np.mean(_normal_sf(b_hi / sigma_t)))
        frac_lo = min(1.0, max(0.0, (w.density - d_hi) / (d_lo - d_hi)))
    j = np.arange(N, dtype=np.float64)
    take_lo = np.floor((j + 1) * frac_lo) > np.floor(j * frac_lo)
    col_bias = np.where(take_lo, b_lo, b_hi).astype(np.float32)
    wgb[:, K - 1] = f32_to_bf16_bits(-col_bias)
    return {
        "x": xb,
        "wg_t": wgb,
        "wu_t": f32_to_bf16_bits(wu),
        "wd": f32_to_bf16_bits(wd),
        "bias": -bf16_bits_to_f32(wgb[:, K - 1]).astype(np.float64),
        "s": s,
    }


def _bf16_neighbours(v: float):
    """The bfloat16 values just below and just above v (equal if v is one)."""
    b = int(f32_to_bf16_bits(np.array([v], dtype=np.float32))[0])
    r = float(bf16_bits_to_f32(np.array([b], dtype=np.uint16))[0])
    if r == v:
        return r, r
    step = 1 if (r < v) == (v >= 0) else -1
    o = float(bf16_bits_to_f32(np.array([b + step], dtype=np.uint16))[0])
    return min(r, o), max(r, o)
