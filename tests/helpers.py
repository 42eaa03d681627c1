"""Shared helpers for the GPU parity tests: tolerance checks against the fp64 oracle.

Bars (written here once, used by every parity test):
  * cache contents: bit-exact (torch.equal on the raw bits);
  * fp32 attention: max |O_gpu - O_oracle| <= 1e-5;
  * bf16/fp16 attention (fp32 accumulation): max |O_gpu - O_oracle| <= 2e-2 and at least
    99.9% of rows (one (b, t, h) output vector of length D) agree on the argmax. Agreement is
    tie-aware: row r agrees iff O_gpu[r, argmax O_oracle[r]] == max O_gpu[r], because bf16
    output rounding creates exact ties that a first-index argmax would split arbitrarily.
    The argmax bar is a rate, so it is judged only over at least ARGMAX_MIN_ROWS rows (below
    that one disagreement in a few hundred rows would decide it); every test that calls
    check_attention with fewer rows still gets the max-abs bar, and the workload tests sample
    enough rows for the rate.
"""
from __future__ import annotations

import warnings

import numpy as np
import torch

FP32_ATOL = 1e-5
LOWP_ATOL = 2e-2
ARGMAX_MIN = 0.999
ARGMAX_MIN_ROWS = 2000


def f64(t) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def argmax_agreement(o_gpu: np.ndarray, o_ref: np.ndarray) -> tuple[float, float]:
    """(tie-aware, strict) fraction of rows whose argmax agrees; rows are the last axis."""
    g = o_gpu.reshape(-1, o_gpu.shape[-1])
    r = o_ref.reshape(-1, o_ref.shape[-1])
    ia = r.argmax(axis=1)
    tie_aware = g[np.arange(len(g)), ia] == g.max(axis=1)
    strict = g.argmax(axis=1) == ia
    return float(tie_aware.mean()), float(strict.mean())


def check_attention(o_gpu, o_ref: np.ndarray, dtype, what: str = "") -> dict:
    """Assert the parity bar for `dtype` ('f32': max-abs <= 1e-5; bf16/fp16: max-abs <= 2e-2
    and tie-aware argmax agreement >= 99.9% over rows)."""
    og = f64(o_gpu) if isinstance(o_gpu, torch.Tensor) else o_gpu
    assert og.shape == o_ref.shape, (og.shape, o_ref.shape)
    assert np.isfinite(og).all(), f"{what}: non-finite outputs"
    err = float(np.max(np.abs(og - o_ref))) if og.size else 0.0
    if dtype in ("f32", torch.float32):
        assert err <= FP32_ATOL, f"{what}: max abs err {err:.3g} > {FP32_ATOL}"
        return {"max_abs": err}
    tie, strict = argmax_agreement(og, o_ref)
    rows = og.size // og.shape[-1]
    assert err <= LOWP_ATOL, f"{what}: max abs err {err:.3g} > {LOWP_ATOL}"
    if rows >= ARGMAX_MIN_ROWS:
        assert tie >= ARGMAX_MIN, f"{what}: argmax agreement {tie:.5f} < {ARGMAX_MIN} over {rows} rows"
    return {"max_abs": err, "argmax": tie, "argmax_strict": strict, "rows": rows}


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Bit-for-bit equality (NaN payloads included)."""
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    ia = a.contiguous().view(torch.uint8)
    ib = b.contiguous().view(torch.uint8)
    return bool(torch.equal(ia, ib))


class AgreementReport(UserWarning):
    """Measured parity figures of a workload test, shown in pytest's warnings summary (which a
    quiet run still prints) so that a passing run records them too."""


def report(what: str, stats: dict) -> None:
    parts = [f"{k}={v:.6g}" if isinstance(v, float) else f"{k}={v}" for k, v in stats.items()]
    warnings.warn(f"{what}: " + " ".join(parts), AgreementReport, stacklevel=2)
