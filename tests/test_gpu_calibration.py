"""GPU checks of the calibration sweep (BLASST talk notes, threshold calibration, Algorithm 2):
the skip fraction the sweep reads off one lambda = 0 call's margins equals what calls made with
each candidate actually skip (outside the margin band), the margins themselves match the oracle,
the swept curve is monotone in lambda, and the library's fit of lambda * L = a exp(b S) over the
observations of several lengths equals the oracle's. (How sparsity at a fixed threshold moves
with length depends on the inputs, not on the method; the benchmark reports it.)"""
import math
import random

import numpy as np
import pytest
import torch

import oracle
import flashattention_softmax_threshold_amd as F
from flashattention_softmax_threshold_amd import calibration as C
from flashattention_softmax_threshold_amd.inputs import prefill_inputs

from parity import MARGIN_BAND, need_gpu, oracle_scale

pytestmark = pytest.mark.gpu


def _inputs(L, seed, Hq=8, Hkv=2, beta=32.0):
    return prefill_inputs(B=1, L=L, Hq=Hq, Hkv=Hkv, d=128, cluster_len=256, dtype=torch.bfloat16,
                          device="cuda", seed=seed, beta=beta, sinks=64)


def test_one_pass_curve_equals_calls_at_each_lambda():
    need_gpu()
    L = 2048
    q, k, v = _inputs(L, 7100)
    margin, status = C.prefill_margins(q, k, v, causal=True)
    m = margin.cpu().numpy().ravel()
    st = status.cpu().numpy().ravel()
    assert set(np.unique(st)) <= {0, 2}  # lambda = 0: every visited tile kept
    lams = [a / L for a in (1.0, 4.0, 16.0, 64.0, 256.0, 1024.0)]
    curve, vis = F.blasst_sparsity_curve(margin, status, lams)
    print(f"L={L}: visited {vis}, curve {[round(c, 4) for c in curve]}", flush=True)
    assert 0 < curve[0] <= curve[-1] < 1
    for lam, frac in zip(lams, curve):
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        F.blasst_attn_prefill(q, k, v, causal=True, lam=lam, counters=cnt)
        torch.cuda.synchronize()
        n_vis, n_skip = (int(x) for x in cnt.cpu().tolist())
        band = int(np.sum((st != 2) & (np.abs(m - math.log(lam)) < MARGIN_BAND)))
        assert n_vis == vis
        assert abs(n_skip - round(frac * vis)) <= band, (lam, n_skip, frac * vis, band)

    # The margins the sweep reads are the oracle's, on a sample of units.
    br, bc = F.blasst_prefill_tiles(q, k)
    units = random.Random(1).sample([(0, h, qb) for h in range(q.shape[2]) for qb in range(L // br)], 6)
    ref = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), causal=True, block_r=br, block_c=bc,
                         scale=oracle_scale(128), lam=0.0, units=units, threads=16)
    mm = margin.cpu().numpy()
    for (b, h, qb), u in ref.units.items():
        vis_t = u.tile_status != oracle.TILE_NOT_VISITED
        got = mm[b, h, qb, :len(u.tile_status)][vis_t]
        np.testing.assert_allclose(got, u.tile_margin[vis_t], atol=MARGIN_BAND, rtol=0)


def test_sweep_over_lengths_is_monotone_and_fit_matches_oracle():
    need_gpu()
    factors = [2.0 ** e for e in range(-2, 13)]
    points = []
    for L in (2048, 4096):
        q, k, v = _inputs(L, 7200 + L, beta=16.0)
        margin, status = C.prefill_margins(q, k, v, causal=True)
        obs = C.observations(margin, status, L, factors)
        s = [o[2] for o in obs]
        print(f"L={L}: sparsity at lambda = 2^e / L, e = -2..12: {[round(x, 3) for x in s]}",
              flush=True)
        assert all(x <= y for x, y in zip(s, s[1:]))  # the skipped set grows with lambda
        assert 0 <= s[0] and s[-1] < 1
        points += obs
        del q, k, v
    use = [p for p in points if 0.05 < p[2] < 0.95]
    a, b = C.fit(points)
    ao, bo = oracle.fit_calibration(*zip(*use))
    print(f"fitted lambda * L = {a:.4g} * exp({b:.4g} * S) from {len(use)} points", flush=True)
    assert a == pytest.approx(ao, rel=1e-9) and b == pytest.approx(bo, rel=1e-9)
