"""Shared helpers of the GPU parity tests: tolerances and comparisons against the oracle.

Tolerances (fixed by the parity contract of this library):
  O    max|err| <= 1e-2 and mean|err| <= 1e-3 for 16-bit I/O with fp32
       accumulation.  A bf16 value |O_ref| >= 4 has a half-ulp of rounding
       alone of 2^-6 = 0.0156 > 1e-2, so there the bound is the rounding
       floor of the output format plus 1e-3: |err| <= ulp(O_ref)/2 + 1e-3.
  lse  max|err| <= 1e-3.
  dQ, dK, dV  relative Frobenius error ||G - G_ref|| / ||G_ref|| <= 2e-2 each.
  With dropout, O = k (sum_j z_j w_j V_j) / (sum_j w_j) with the keep factor
  k = 256 / (256 - t): every rounding error made before the final
  multiplication by k is multiplied by k, so the O bounds other than the
  output rounding floor are scaled by k (check_o's ``gain``); a relative
  Frobenius bound on the whole O, ||O - O_ref|| / ||O_ref|| <= 1e-2, holds
  with dropout as well and does not grow with k.  And k V_j is
  in general not a 16-bit number (without dropout a row with one visible
  key returns V_j exactly), so with dropout the mean bound also admits the
  mean half-ulp of the output format at O_ref.
"""
from __future__ import annotations

import math

import numpy as np
import torch

O_MAX = 1e-2
O_MEAN = 1e-3
LSE_MAX = 1e-3
GRAD_REL_FRO = 2e-2
# With dropout, also ||O - O_ref||_F / ||O_ref||_F <= 1e-2, a bound that does
# not grow with the keep factor: the rounding of the weights to 16 bits and
# of O itself are each at most 2^-8 relative.
O_REL_FRO_DROPOUT = 1e-2

# explicit mantissa widths of the 16-bit formats
_MANT = {torch.bfloat16: 7, torch.float16: 10, "bf16": 7, "fp16": 10}


def half_ulp(x: np.ndarray, dtype) -> np.ndarray:
    """Half the spacing of the 16-bit format at |x| (normal range)."""
    m = _MANT[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    return 0.5 * np.exp2(e - m)


def check_o(o_gpu: np.ndarray, o_ref: np.ndarray, dtype, what: str = "O", gain: float = 1.0):
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    big = np.abs(o_ref) >= 4.0
    bound = np.where(big, half_ulp(o_ref, dtype) + 1e-3 * gain, O_MAX * gain)
    worst = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{what}: {len(bad)} elements over bound; worst {worst:.3e} at "
                           f"{tuple(bad[0])} gpu={o_gpu[tuple(bad[0])]} ref={o_ref[tuple(bad[0])]}")
    mean_bound = O_MEAN * gain + (float(half_ulp(o_ref, dtype).mean()) if gain != 1.0 and err.size else 0.0)
    assert mean <= mean_bound, f"{what}: mean|err| {mean:.3e} > {mean_bound:.3e}"
    n_big = int(big.sum())
    if n_big:
        log(f"{what}: {n_big} elements with |O_ref| >= 4 held to half an output ulp + {1e-3 * gain:.1e} "
            f"(worst of them {float(err[big].max()):.3e})")
    if gain != 1.0 and err.size:
        # the same O without the growth by k: its error relative to its own size
        rel = rel_fro(o_gpu, o_ref)
        assert rel <= O_REL_FRO_DROPOUT, f"{what}: relative Frobenius error {rel:.3e} > {O_REL_FRO_DROPOUT}"
    return worst, mean


def check_lse(l_gpu: np.ndarray, l_ref: np.ndarray, what: str = "lse"):
    err = np.abs(l_gpu.astype(np.float64) - l_ref)
    worst = float(err.max()) if err.size else 0.0
    assert np.all(np.isfinite(l_gpu)), f"{what}: non-finite values"
    assert worst <= LSE_MAX, f"{what}: max|err| {worst:.3e} > {LSE_MAX}"
    return worst


def rel_fro(g: np.ndarray, g_ref: np.ndarray) -> float:
    den = float(np.linalg.norm(g_ref))
    num = float(np.linalg.norm(g.astype(np.float64) - g_ref))
    return num / den if den > 0 else num


def check_grad(g_gpu: np.ndarray, g_ref: np.ndarray, what: str):
    assert np.all(np.isfinite(g_gpu)), f"{what}: non-finite values"
    e = rel_fro(g_gpu, g_ref)
    assert e <= GRAD_REL_FRO, f"{what}: relative Frobenius error {e:.3e} > {GRAD_REL_FRO}"
    return e


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def sample_rows(n: int, count: int, seed: int, block: int = 128) -> np.ndarray:
    """Query rows to check at full size: both ends of the sequence, rows at
    every block boundary region near the ends, and a seeded random spread."""
    rng = np.random.default_rng(seed)
    fixed = {0, 1, 31, 32, 63, 64, n // 2, n - 65, n - 64, n - 33, n - 32, n - 2, n - 1}
    fixed |= {min(n - 1, block * i + o) for i in range(3) for o in (block - 1, block)}
    rnd = set(rng.choice(n, size=min(count, n), replace=False).tolist())
    return np.array(sorted(x for x in (fixed | rnd) if 0 <= x < n), dtype=np.int64)


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import exact_attention_66_amd as ea
    ea.load()  # raises if the library is missing: never silently skipped
    return ea


def log(msg: str):
    print(msg, flush=True)
