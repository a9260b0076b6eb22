"""Threshold calibration sweep ("BLASST: Dynamic BLocked Attention Sparsity via Softmax
Thresholding" talk notes, threshold calibration: Algorithm 2 steps 1-3, Eq. 3).

Step 1 sweeps many candidate thresholds in one pass: a prefill call with lambda = 0 writes every
visited tile's margin, and since the margin does not depend on lambda, the skip fraction at any
candidate follows from the margins alone (blasst_sparsity_curve). Step 2 records the observed
sparsity per (threshold, sequence length). Step 3 fits lambda * L = a * exp(b * S)
(blasst_fit_calibration); the (a, b) it returns feed BLASST_TARGET_SPARSITY.

All arithmetic runs in the library (the attention call on the GPU, the curve and the fit in the
host entry points); this module only allocates the observation buffers and loops.
"""
from __future__ import annotations

import torch

from . import blasst_attn_prefill, blasst_fit_calibration, blasst_prefill_tiles, blasst_sparsity_curve


def prefill_margins(q, k, v, *, causal: bool, block_r: int = 0, stream=None):
    """One lambda = 0 prefill call that records (tile_margin, tile_status) of every unit."""
    B, Lq, Hq, _ = q.shape
    br, bc = blasst_prefill_tiles(q, k, block_r=block_r)
    shape = (B, Hq, -(-Lq // br), -(-k.shape[1] // bc))
    status = torch.full(shape, 255, dtype=torch.uint8, device=q.device)
    margin = torch.empty(shape, dtype=torch.float32, device=q.device)
    blasst_attn_prefill(q, k, v, causal=causal, lam=0.0, tile_status=status, tile_margin=margin,
                        block_r=block_r, stream=stream)
    return margin, status


def observations(margin, status, seq_len: int, factors):
    """(L, lambda, S) for the candidates lambda = c / L, c in factors (Eq. 3's a / L form)."""
    lams = [float(c) / seq_len for c in factors]
    sparsity, _ = blasst_sparsity_curve(margin, status, lams)
    return [(seq_len, lam, s) for lam, s in zip(lams, sparsity)]


def fit(points, s_min: float = 0.05, s_max: float = 0.95):
    """(a, b) fitted to the observations whose sparsity lies strictly inside (s_min, s_max): at
    the flat ends of a curve many thresholds share one sparsity and carry no information."""
    use = [p for p in points if s_min < p[2] < s_max]
    if len(use) < 2:
        raise ValueError("fewer than two observations inside the sparsity range")
    L, lam, S = zip(*use)
    return blasst_fit_calibration(L, lam, S)
