"""Shared comparison rules for GPU-vs-oracle parity tests.

Bar (bf16 inputs, fp32 accumulation): max|dO| <= 1e-2 * max|O| against the exact oracle and
mean|dO| <= 1e-3 against the oracle rounded to the output dtype (bf16 rounding of an output of
magnitude ~1 alone is ~1e-3 on average); LSE within 1e-2 (natural log). fp32 inputs:
max|dO| <= (1e-4 + 1e-6 max|LSE|) * max|O|, mean|dO| <= 1e-5 + 1e-7 max|LSE|, LSE within
1e-4 + 2e-6 |LSE|: the LSE is about the largest
scaled score, which the kernel forms in fp32, so its rounding grows with the score's magnitude
(an fp32 ulp at 256 is 3e-5); the exponent of every P carries that absolute rounding (about
6e-8, one ulp per unit, times the score), so the outputs' mean error grows with it too. Skip
decisions must agree exactly on every tile whose oracle
margin lies outside a band around ln(lambda); inside the band float rounding may flip the
decision, and such tiles are counted, not failed (their units are then compared against the
oracle evaluated with the kernel's decisions).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

MARGIN_BAND = 1e-3
TOL = {
    torch.bfloat16: dict(max_rel=1e-2, max_lse=0.0, mean_abs=1e-3, mean_lse=0.0, lse_abs=1e-2,
                         lse_rel=0.0),
    torch.float32: dict(max_rel=1e-4, max_lse=1e-6, mean_abs=1e-5, mean_lse=1e-7, lse_abs=1e-4,
                        lse_rel=2e-6),
}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def tau(lam: float) -> float:
    return -math.inf if lam == 0 else math.log(min(lam, 1.0))


def _round_to(x: np.ndarray, dtype) -> np.ndarray:
    return torch.as_tensor(x, dtype=torch.float64).to(dtype).to(torch.float64).numpy()


def assert_outputs_close(o_gpu: np.ndarray, o_ref: np.ndarray, dtype, what: str,
                         lse_ref: np.ndarray | None = None):
    """max|dO| against the exact oracle; mean|dO| against the oracle rounded to the output dtype
    (a bf16 output of magnitude ~1 carries ~1e-3 of rounding on its own, whatever computed it).
    lse_ref: the oracle's LSE of the same rows, whose largest magnitude sets the fp32 part of the
    mean bar that grows with the scores."""
    tol = TOL[dtype]
    lse_mag = 0.0
    if lse_ref is not None:
        fin = np.isfinite(lse_ref)
        lse_mag = float(np.abs(lse_ref[fin]).max()) if fin.any() else 0.0
    mean_tol = tol["mean_abs"] + tol["mean_lse"] * lse_mag
    max_tol = tol["max_rel"] + tol["max_lse"] * lse_mag
    err = np.abs(o_gpu - o_ref)
    scale = np.abs(o_ref).max()
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite output"
    assert err.max() <= max_tol * scale, \
        f"{what}: max|dO| {err.max():.3e} > {max_tol:.3e} * max|O| ({scale:.3e})"
    mean_err = np.abs(o_gpu - _round_to(o_ref, dtype)).mean()
    assert mean_err <= mean_tol, \
        f"{what}: mean|dO| {mean_err:.3e} > {mean_tol:.3e} (vs rounded oracle)"
    return float(err.max()), float(mean_err)


def assert_lse_close(lse_gpu: np.ndarray, lse_ref: np.ndarray, dtype, what: str):
    t = TOL[dtype]
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), f"{what}: LSE finiteness differs"
    if fin.any():
        d = np.abs(lse_gpu[fin] - lse_ref[fin])
        tol = t["lse_abs"] + t["lse_rel"] * np.abs(lse_ref[fin])
        worst = int(np.argmax(d - tol))
        assert (d <= tol).all(), \
            f"{what}: LSE differs by {d[worst]:.3e} (tolerance {tol[worst]:.3e} at |LSE| " \
            f"{abs(lse_ref[fin][worst]):.3e})"


def compare_tile_status(st_gpu: np.ndarray, st_ref: np.ndarray, margin_ref: np.ndarray,
                        lam: float, what: str, band_width: float = MARGIN_BAND,
                        margin_gpu: np.ndarray | None = None, stats: dict | None = None):
    """Exact agreement outside the margin band; returns (#mismatches inside the band, #band).

    With margin_gpu (the kernel's tile_margin output for the same tiles) the margins themselves
    must agree to within the band on every tile (the same non-finite tiles, |d margin| <=
    band_width elsewhere): a kernel whose margins drift from the oracle's by a systematic bias
    fails here even when the bias only ever flips tiles inside the band. stats (optional) gathers
    the largest margin difference seen under 'max_dmargin'."""
    st_gpu = np.asarray(st_gpu).ravel()
    st_ref = np.asarray(st_ref).ravel()
    margin_ref = np.asarray(margin_ref).ravel()
    t = tau(lam)
    band = np.isfinite(margin_ref) & (np.abs(margin_ref - t) < band_width) if math.isfinite(t) \
        else np.zeros_like(st_ref, dtype=bool)
    mism = st_gpu != st_ref
    bad = mism & ~band
    assert not bad.any(), f"{what}: {int(bad.sum())} tile decisions differ outside the band " \
                          f"(first at {int(np.argmax(bad))}: gpu {st_gpu[bad][0]} ref {st_ref[bad][0]})"
    assert int(mism.sum()) <= int(band.sum()), f"{what}: more flips than band tiles"
    if margin_gpu is not None:
        mg = np.asarray(margin_gpu, dtype=np.float64).ravel()
        fin = np.isfinite(margin_ref)
        assert np.array_equal(np.isfinite(mg), fin), \
            f"{what}: the kernel's margins are finite on other tiles than the oracle's"
        if fin.any():
            dm = np.abs(mg[fin] - margin_ref[fin])
            assert dm.max() <= band_width, \
                f"{what}: tile margin differs from the oracle's by {dm.max():.3e} " \
                f"(> {band_width:.1e}) at tile {int(np.flatnonzero(fin)[np.argmax(dm)])}"
            if stats is not None:
                stats["max_dmargin"] = max(stats.get("max_dmargin", 0.0), float(dm.max()))
    return int(mism.sum()), int(band.sum())


def oracle_scale(head_dim: int) -> float:
    """1/sqrt(d): the library's default softmax scale."""
    return 1.0 / math.sqrt(head_dim)
