"""Pins for the fp64 oracle, checked against things other than the oracle itself.

Each test names what it pins and which plausible mistake it would catch:
  * the dense definition and lambda = 0 against SciPy's softmax / logsumexp and torch's
    scaled_dot_product_attention in float64 (catches a transposed operand, a wrong scale, a
    dropped rescale of l or O, an off-by-one causal mask, a wrong GQA head map);
  * the streaming loop at lambda > 0 against the closed form "softmax over the kept tiles,
    normalised with the global row max", whose kept set comes from prefix maxima of the tile
    maxima (catches a wrong running max, a wrong sign or direction in the test, a skipped tile
    that still adds to l or O);
  * a hand-derived worked example (tests/golden/hand_tiles.json) for the "every row" vote, the
    strict comparison and the ragged last tile;
  * invariants fixed by the pages: the test's left side lies in (0, 1], lambda = 0 skips nothing,
    the skipped count is monotone in lambda, and the approximation error is bounded by the
    skipped mass.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _masked_scores(q, k, row_keys, scale, row_first=None):
    s = scale * (q @ k.T)
    idx = np.arange(k.shape[0])[None, :]
    mask = idx >= np.asarray(row_keys)[:, None]
    if row_first is not None:
        mask |= idx < np.asarray(row_first)[:, None]
    s = np.where(mask, -np.inf, s)
    return s


def _library_attention(q, k, v, row_keys, scale, row_first=None):
    s = _masked_scores(q, k, row_keys, scale, row_first)
    return softmax(s, axis=1) @ v, logsumexp(s, axis=1)


def _clustered_rows(rng, n_rows, n_keys, d, d_v, beta, cluster=16):
    centres = rng.standard_normal((n_keys // cluster + 1, d)) * beta / math.sqrt(d)
    idx = np.arange(n_keys) // cluster
    k = 3 * centres[idx] + 0.5 * rng.standard_normal((n_keys, d))
    qi = rng.integers(0, n_keys, size=n_rows)
    q = centres[idx[qi]] + 0.5 * rng.standard_normal((n_rows, d))
    v = rng.standard_normal((n_keys, d_v))
    return q, k, v


def _closed_form(q, k, v, row_keys, scale, lam, block_c, k_begin=0, k_end=None, row_first=None):
    """Kept set from prefix maxima of tile maxima; output = softmax over the kept keys."""
    n_keys = k.shape[0] if k_end is None else k_end
    s = _masked_scores(q, k[:n_keys], row_keys, scale, row_first)[:, k_begin:n_keys]
    n = s.shape[1]
    tiles = [(a, min(a + block_c, n)) for a in range(0, n, block_c)]
    tmax = np.stack([s[:, a:e].max(axis=1) for a, e in tiles], axis=1)  # rows x tiles
    prefix = np.maximum.accumulate(tmax, axis=1)  # running max including the tile
    with np.errstate(invalid="ignore"):
        row_margin = np.where(np.isfinite(tmax), tmax - prefix, -np.inf)
    visited = np.isfinite(tmax).any(axis=0)
    margin = row_margin.max(axis=0)
    tau = -np.inf if lam == 0 else math.log(min(lam, 1.0))
    skipped = visited & (margin < tau)
    keep_cols = np.zeros(n, dtype=bool)
    for t, (a, e) in enumerate(tiles):
        if visited[t] and not skipped[t]:
            keep_cols[a:e] = True
    sk = np.where(keep_cols[None, :], s, -np.inf)
    o = softmax(sk, axis=1) @ v[k_begin:n_keys]
    return dict(o=o, lse=logsumexp(sk, axis=1), margin=margin, visited=visited, skipped=skipped,
                s=s, keep_cols=keep_cols)


# ------------------------------------------------------------------------------------------
# Dense definition and lambda = 0
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("n_keys,causal", [(1, False), (37, False), (130, True), (200, False)])
def test_dense_rows_match_scipy(n_keys, causal):
    rng = np.random.default_rng(n_keys)
    n_rows, d, dv = 9, 16, 12
    q = rng.standard_normal((n_rows, d))
    k = rng.standard_normal((n_keys, d))
    v = rng.standard_normal((n_keys, dv))
    row_keys = [max(1, n_keys - 3 * r) for r in range(n_rows)] if causal else [n_keys] * n_rows
    scale = 0.3
    o, lse = oracle.dense_rows(q, k, v, row_keys, scale)
    o_ref, lse_ref = _library_attention(q, k, v, row_keys, scale)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("block_c", [1, 7, 16, 64, 500])
def test_lambda_zero_equals_dense(block_c):
    rng = np.random.default_rng(block_c)
    q, k, v = _clustered_rows(rng, 11, 203, 24, 8, beta=6.0)
    row_keys = [203 - 17 * r for r in range(11)]
    r = oracle.blasst_rows(q, k, v, row_keys, 0, 203, block_c, 0.2, 0.0)
    o_ref, lse_ref = _library_attention(q, k, v, row_keys, 0.2)
    np.testing.assert_allclose(r["o"], o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse_ref, rtol=1e-12, atol=1e-12)
    assert r["skipped"] == 0
    assert r["visited"] == -(-203 // block_c)


def _sdpa(q, k, v, causal):
    """torch SDPA in float64 on [B, L, H, d] tensors (GQA by repeating KV heads)."""
    qt = torch.as_tensor(q, dtype=torch.float64).transpose(1, 2)
    kt = torch.as_tensor(k, dtype=torch.float64).transpose(1, 2)
    vt = torch.as_tensor(v, dtype=torch.float64).transpose(1, 2)
    grp = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(grp, dim=1)
    vt = vt.repeat_interleave(grp, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal)
    return o.transpose(1, 2).numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_lambda_zero_matches_torch_sdpa(causal):
    from flashattention_softmax_threshold_amd.inputs import prefill_inputs

    B, L, Hq, Hkv, d = 2, 150, 4, 2, 16
    q, k, v = prefill_inputs(B=B, L=L, Hq=Hq, Hkv=Hkv, d=d, cluster_len=32, dtype=torch.float32,
                             seed=3, beta=4.0, sinks=8)
    res = oracle.prefill(q, k, v, causal=causal, block_r=32, block_c=16, scale=1 / math.sqrt(d),
                         lam=0.0)
    ref = _sdpa(q.numpy(), k.numpy(), v.numpy(), causal)
    for (b, h, qb), u in res.units.items():
        r0 = qb * 32
        np.testing.assert_allclose(u.o, ref[b, r0:r0 + u.o.shape[0], h], rtol=1e-10, atol=1e-11)
        assert u.skipped == 0
    assert len(res.units) == B * Hq * (-(-L // 32))
    # Visited tiles: all 10 (ragged last) non-causal; causal block qb sees tiles up to its last row.
    for (b, h, qb), u in res.units.items():
        last_row = min((qb + 1) * 32, L) - 1
        expect = (last_row // 16 + 1) if causal else -(-L // 16)
        assert u.visited == expect


@pytest.mark.parametrize("lq,lkv", [(70, 150), (150, 37)])
def test_cross_length_prefill_lambda_zero_matches_torch_sdpa(lq, lkv):
    """Non-causal prefill with fewer or more queries than keys (cross attention): every query
    row sees all Lkv keys; the last key tile is ragged."""
    from flashattention_softmax_threshold_amd.inputs import prefill_inputs

    B, Hq, Hkv, d = 2, 4, 2, 16
    q, k, v = prefill_inputs(B=B, L=max(lq, lkv), Hq=Hq, Hkv=Hkv, d=d, cluster_len=32,
                             dtype=torch.float32, seed=4, beta=4.0)
    q, k, v = q[:, :lq], k[:, :lkv], v[:, :lkv]
    res = oracle.prefill(q, k, v, causal=False, block_r=32, block_c=16, scale=1 / math.sqrt(d),
                         lam=0.0)
    ref = _sdpa(q.numpy(), k.numpy(), v.numpy(), False)
    assert len(res.units) == B * Hq * (-(-lq // 32))
    for (b, h, qb), u in res.units.items():
        r0 = qb * 32
        np.testing.assert_allclose(u.o, ref[b, r0:r0 + u.o.shape[0], h], rtol=1e-10, atol=1e-11)
        assert u.visited == -(-lkv // 16) and u.skipped == 0


def test_decode_lambda_zero_matches_torch_sdpa_with_lengths_and_splits():
    from flashattention_softmax_threshold_amd.inputs import decode_inputs

    B, Hq, Hkv, L, d, dv = 3, 8, 2, 300, 16, 12
    kv_len = [300, 1, 129]
    q, k, v, kvl = decode_inputs(B=B, Hq=Hq, Hkv=Hkv, L=L, d_qk=d, d_v=dv, cluster_len=50,
                                 dtype=torch.float32, seed=5, beta=3.0, kv_len=kv_len)
    for splits in (1, 2, 5):
        res = oracle.decode(q, k, v, kv_len=kvl, block_r=4, block_c=32, num_splits=splits,
                            scale=0.25, lam=0.0)
        for (b, g, rb), u in res.units.items():
            n = kv_len[b]
            heads = range(g * 4 + rb * 4, g * 4 + rb * 4 + 4)
            for i, h in enumerate(heads):
                s = 0.25 * (k[b, :n, g].double() @ q[b, h].double())
                ref = torch.softmax(s, 0) @ v[b, :n, g].double()
                np.testing.assert_allclose(u.o[i], ref.numpy(), rtol=1e-11, atol=1e-12)
                np.testing.assert_allclose(u.lse[i], torch.logsumexp(s, 0).item(), rtol=1e-12)


def test_decode_empty_sequence_gives_zero_and_minus_inf():
    q = np.ones((1, 2, 4))
    k = np.ones((1, 10, 1, 4))
    v = np.ones((1, 10, 1, 3))
    for splits in (1, 3):
        res = oracle.decode(q, k, v, kv_len=[0], block_r=2, block_c=4, num_splits=splits,
                            scale=1.0, lam=0.1)
        u = res.units[(0, 0, 0)]
        assert np.all(u.o == 0) and np.all(np.isneginf(u.lse))
        assert u.visited == 0 and u.skipped == 0


# ------------------------------------------------------------------------------------------
# lambda > 0: closed form, invariants, worked example
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(6))
def test_streaming_matches_closed_form(seed):
    rng = np.random.default_rng(100 + seed)
    n_rows = int(rng.integers(1, 9))
    n_keys = int(rng.integers(40, 400))
    block_c = int(rng.choice([8, 16, 33]))
    q, k, v = _clustered_rows(rng, n_rows, n_keys, 16, 6, beta=float(rng.choice([4.0, 8.0])))
    row_keys = sorted(rng.integers(1, n_keys + 1, size=n_rows).tolist())
    scale = 0.25
    total_skips = 0
    for lam in (0.0, 1e-4, 1e-2, 0.3, 1.0):
        r = oracle.blasst_rows(q, k, v, row_keys, 0, n_keys, block_c, scale, lam)
        cf = _closed_form(q, k, v, row_keys, scale, lam, block_c)
        vis = cf["visited"]
        np.testing.assert_array_equal(r["tile_status"][vis] == oracle.TILE_SKIPPED,
                                      cf["skipped"][vis])
        assert np.all(r["tile_status"][~vis] == oracle.TILE_NOT_VISITED)
        np.testing.assert_allclose(r["tile_margin"][vis], cf["margin"][vis], rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["o"], cf["o"], rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(r["lse"], cf["lse"], rtol=1e-12, atol=1e-12)
        assert r["visited"] == int(vis.sum())
        assert r["skipped"] == int(cf["skipped"].sum())
        total_skips += r["skipped"]
    assert total_skips > 0  # the case exercises the skip branch


def test_worked_example_from_golden_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "hand_tiles.json")))
    k = np.array(fx["k"])
    v = np.array(fx["v"])
    for case in fx["cases"]:
        q = np.array(case["rows"])
        row_keys = case.get("row_keys", [len(k)] * len(q))
        lam = 0.0 if case.get("lambda_zero") else math.exp(case["ln_lambda"])
        r = oracle.blasst_rows(q, k, v, row_keys, 0, len(k), fx["block_c"], fx["scale"], lam)
        assert r["tile_status"].tolist() == case["status"], case
        np.testing.assert_allclose(r["tile_margin"], case["margin"], atol=1e-12)
        # Output: plain softmax over the keys of the kept tiles, written out with math.exp.
        kept = [j for j in range(len(k)) if case["status"][j // fx["block_c"]] == 0]
        for i, row in enumerate(q):
            ks = [j for j in kept if j < row_keys[i]]
            w = [math.exp(row[0] * k[j][0]) for j in ks]
            expect = [sum(wj * v[j][c] for wj, j in zip(w, ks)) / sum(w) for c in range(2)]
            np.testing.assert_allclose(r["o"][i], expect, rtol=1e-13)
            assert abs(r["lse"][i] - math.log(sum(w))) < 1e-13


def test_margin_in_range_and_first_tile_kept():
    rng = np.random.default_rng(7)
    q, k, v = _clustered_rows(rng, 5, 333, 16, 4, beta=8.0)
    r = oracle.blasst_rows(q, k, v, [333] * 5, 0, 333, 16, 0.25, 0.5)
    m = r["tile_margin"]
    assert np.all(m <= 0)  # exp(margin) lies in (0, 1]
    assert np.all(np.exp(m) > 0)
    assert m[0] == 0 and r["tile_status"][0] == oracle.TILE_KEPT


def test_skipped_set_monotone_in_lambda_and_fixed_by_margin():
    rng = np.random.default_rng(11)
    q, k, v = _clustered_rows(rng, 4, 512, 16, 4, beta=8.0)
    lams = [0.0, 1e-6, 1e-4, 1e-3, 1e-2, 0.1, 0.5, 1.0]
    prev = None
    margins = None
    for lam in lams:
        r = oracle.blasst_rows(q, k, v, [512] * 4, 0, 512, 32, 0.25, lam)
        sk = r["tile_status"] == oracle.TILE_SKIPPED
        if margins is None:
            margins = r["tile_margin"]
        np.testing.assert_array_equal(r["tile_margin"], margins)  # margin does not depend on lambda
        tau = -np.inf if lam == 0 else math.log(lam)
        np.testing.assert_array_equal(sk, margins < tau)
        if prev is not None:
            assert np.all(sk >= prev)
        prev = sk
    assert prev.sum() > 0


def test_lambda_one_uses_strict_comparison_and_lambda_above_one_is_clamped():
    # All keys identical: every tile margin is exactly 0, so "0 < ln(1) = 0" is false and nothing
    # is skipped; a "<=" test would skip every tile after the first.
    n = 70
    q = np.ones((3, 4))
    k = np.ones((n, 4))
    v = np.arange(n, dtype=float)[:, None] * np.ones((1, 2))
    for lam in (1.0, 7.5):
        r = oracle.blasst_rows(q, k, v, [n] * 3, 0, n, 16, 1.0, lam)
        assert r["skipped"] == 0
        np.testing.assert_allclose(r["o"], np.full((3, 2), (n - 1) / 2.0), rtol=1e-14)
    r1 = oracle.blasst_rows(*_clustered_rows(np.random.default_rng(1), 3, 200, 8, 2, 8.0),
                            [200] * 3, 0, 200, 16, 0.3, 1.0)
    r2 = oracle.blasst_rows(*_clustered_rows(np.random.default_rng(1), 3, 200, 8, 2, 8.0),
                            [200] * 3, 0, 200, 16, 0.3, 40.0)
    np.testing.assert_array_equal(r1["tile_status"], r2["tile_status"])
    np.testing.assert_array_equal(r1["o"], r2["o"])


@pytest.mark.parametrize("lam", [-1e-9, float("nan"), float("inf")])
def test_invalid_lambda_rejected(lam):
    with pytest.raises(oracle.OracleError):
        oracle.blasst_rows(np.ones((1, 2)), np.ones((4, 2)), np.ones((4, 2)), [4], 0, 4, 2, 1.0, lam)


def test_error_bounded_by_skipped_mass():
    """|O_blasst - O_dense| <= 2 max|V| W / l_kept <= 2 max|V| W, with W the skipped weight
    sum_{skipped k} exp(s_k - M) (M the global row max); each skipped weight is below lambda, the
    Skip-Softmax page's upper-bound argument."""
    rng = np.random.default_rng(21)
    q, k, v = _clustered_rows(rng, 6, 640, 16, 5, beta=6.0)
    row_keys = [640] * 6
    o_dense, _ = _library_attention(q, k, v, row_keys, 0.25)
    s = _masked_scores(q, k, row_keys, 0.25)
    M = s.max(axis=1, keepdims=True)
    checked = 0
    for lam in (1e-4, 1e-3, 1e-2, 0.1, 0.5):
        r = oracle.blasst_rows(q, k, v, row_keys, 0, 640, 32, 0.25, lam)
        skip_cols = np.repeat(r["tile_status"] == oracle.TILE_SKIPPED, 32)[:640]
        w = np.exp(s - M)
        W = (w * skip_cols[None, :]).sum(axis=1)
        l_kept = (w * ~skip_cols[None, :]).sum(axis=1)
        err = np.abs(r["o"] - o_dense).max(axis=1)
        vmax = np.abs(v).max()
        assert np.all(err <= 2 * vmax * W / l_kept + 1e-12)
        assert np.all(l_kept >= 1.0 - 1e-12)  # the tile holding a row's global max is kept
        assert np.all((w * skip_cols[None, :]) < lam)  # every skipped weight is below lambda
        checked += int(skip_cols.sum() > 0)
    assert checked >= 3


def test_split_ranges_and_combine():
    """Splits restart the running state; merged by log-sum-exp they reproduce the unsplit dense
    result at lambda = 0, and each non-empty split keeps its first tile."""
    rng = np.random.default_rng(33)
    q, k, v = _clustered_rows(rng, 4, 500, 16, 6, beta=8.0)
    assert oracle.split_ranges(500, 500, 32, 4) == [(0, 128), (128, 256), (256, 384), (384, 500)]
    assert oracle.split_ranges(100, 500, 32, 4) == [(0, 100), (100, 100), (100, 100), (100, 100)]
    parts = [oracle.blasst_rows(q, k, v, [500] * 4, a, e, 32, 0.25, 0.0)
             for a, e in oracle.split_ranges(500, 500, 32, 4)]
    o, lse = oracle.combine(np.stack([p["o"] for p in parts]), np.stack([p["lse"] for p in parts]))
    o_ref, lse_ref = _library_attention(q, k, v, [500] * 4, 0.25)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)
    for lam in (0.01, 0.5):
        for a, e in oracle.split_ranges(500, 500, 32, 4):
            p = oracle.blasst_rows(q, k, v, [500] * 4, a, e, 32, 0.25, lam)
            assert p["tile_status"][0] == oracle.TILE_KEPT
            cf = _closed_form(q, k, v, [500] * 4, 0.25, lam, 32, k_begin=a, k_end=e)
            np.testing.assert_allclose(p["o"], cf["o"], rtol=1e-10, atol=1e-11)


def test_split_ranges_with_a_window_explicit_values():
    """Split ranges of a windowed decode, worked by hand from the reading taken for windows (the
    splits cut the at most ceil(W / B_c) + 1 tiles a window of W keys can touch, from the tile
    holding the first visible key kv_len - W, in equal runs of whole tiles, clipped to the
    sequence)."""
    # kv_len 1000, W 300, B_c 64: first key 700 is in tile 10 (key 640); span min(16, 5 + 1) = 6
    # tiles, 3 per split.
    assert oracle.split_ranges(1000, 1000, 64, 2, window=300) == [(640, 832), (832, 1000)]
    # kv_len 450 of a 1000-key cache, W 300, 3 splits: first key 150 -> tile 2 (key 128); 2 tiles
    # per split; the last split ends at the sequence.
    assert oracle.split_ranges(450, 1000, 64, 3, window=300) == [(128, 256), (256, 384),
                                                                 (384, 450)]
    # A window longer than the sequence: the unwindowed ranges exactly.
    assert oracle.split_ranges(100, 1000, 64, 2, window=5000) == [(0, 100), (100, 100)]
    assert oracle.split_ranges(100, 1000, 64, 2, window=5000) == oracle.split_ranges(100, 1000,
                                                                                     64, 2)
    # One tile's worth of window ending on a tile boundary: a single tile, then one key more
    # reaches into the next tile (span 2 tiles, one per split).
    assert oracle.split_ranges(640, 640, 64, 1, window=64) == [(576, 640)]
    assert oracle.split_ranges(641, 641, 64, 2, window=64) == [(576, 640), (640, 641)]
    # A one-key window at the start of a tile; more splits than tiles leave empty splits.
    assert oracle.split_ranges(129, 129, 64, 3, window=1) == [(128, 129), (129, 129), (129, 129)]
    assert oracle.window_first_key(1000, 300) == 700
    assert oracle.window_first_key(200, 300) == 0
    assert oracle.window_first_key(200, 0) == 0


def test_decode_units_and_splits_follow_closed_form():
    from flashattention_softmax_threshold_amd.inputs import decode_inputs

    B, Hq, Hkv, L, d = 2, 8, 2, 512, 16
    q, k, v, kvl = decode_inputs(B=B, Hq=Hq, Hkv=Hkv, L=L, d_qk=d, d_v=d, cluster_len=64,
                                 dtype=torch.float32, seed=9, beta=8.0, share=True,
                                 kv_len=[512, 300])
    any_skip = 0
    for splits in (1, 3):
        res = oracle.decode(q, k, v, kv_len=kvl, block_r=4, block_c=32, num_splits=splits,
                            scale=0.25, lam=0.05)
        for (b, g, rb), u in res.units.items():
            n = int(kvl[b])
            qq = q[b, g * 4:(g + 1) * 4].double().numpy()
            kk = k[b, :n, g].double().numpy()
            vv = v[b, :n, g].double().numpy()
            os_, ls_ = [], []
            for a, e in oracle.split_ranges(n, 512, 32, splits):
                if a == e:
                    continue
                cf = _closed_form(qq, kk, vv, [n] * 4, 0.25, 0.05, 32, k_begin=a, k_end=e)
                os_.append(cf["o"])
                ls_.append(cf["lse"])
                any_skip += int(cf["skipped"].sum())
            w = np.exp(np.array(ls_) - np.max(ls_, axis=0))
            o_ref = (w[:, :, None] * np.array(os_)).sum(0) / w.sum(0)[:, None]
            np.testing.assert_allclose(u.o, o_ref, rtol=1e-10, atol=1e-11)
    assert any_skip > 0


def test_forced_decisions_mode():
    """Imposing decisions: the test's own decisions change nothing; 'keep all' is the dense
    result; any other set gives the softmax over exactly the kept tiles."""
    rng = np.random.default_rng(44)
    q, k, v = _clustered_rows(rng, 5, 300, 16, 4, beta=8.0)
    rk = [300] * 5
    base = oracle.blasst_rows(q, k, v, rk, 0, 300, 32, 0.25, 0.05)
    same = oracle.blasst_rows(q, k, v, rk, 0, 300, 32, 0.25, 0.05, forced=base["tile_status"])
    np.testing.assert_array_equal(same["o"], base["o"])
    keep_all = oracle.blasst_rows(q, k, v, rk, 0, 300, 32, 0.25, 0.05,
                                  forced=np.zeros(10, dtype=np.uint8))
    o_ref, _ = _library_attention(q, k, v, rk, 0.25)
    np.testing.assert_allclose(keep_all["o"], o_ref, rtol=1e-11, atol=1e-12)
    pattern = np.array([0, 1, 1, 0, 1, 0, 0, 1, 1, 0], dtype=np.uint8)
    r = oracle.blasst_rows(q, k, v, rk, 0, 300, 32, 0.25, 0.05, forced=pattern)
    cols = np.repeat(pattern == 0, 32)[:300]
    s = _masked_scores(q, k, rk, 0.25)
    o_cf = softmax(np.where(cols[None, :], s, -np.inf), axis=1) @ v
    np.testing.assert_allclose(r["o"], o_cf, rtol=1e-10, atol=1e-11)
    assert r["skipped"] == int(pattern.sum())


# ------------------------------------------------------------------------------------------
# Calibration (BLASST talk notes, threshold calibration: Algorithm 2, Eq. 3)
# ------------------------------------------------------------------------------------------
def test_fit_calibration_hand_example():
    # ln(lambda L) = 1, 2, 4 at S = 0, 0.5, 1. By hand: mean S = 1/2, mean y = 7/3,
    # Sxy = (-1/2)(-4/3) + (1/2)(5/3) = 3/2, Sxx = 1/2, so b = 3 and ln a = 7/3 - 3/2 = 5/6.
    a, b = oracle.fit_calibration([1, 1, 1], [math.e, math.e ** 2, math.e ** 4], [0, 0.5, 1])
    assert b == pytest.approx(3.0, abs=1e-12)
    assert a == pytest.approx(math.exp(5 / 6), rel=1e-12)


def test_fit_calibration_recovers_the_wan_coefficients_from_model_points():
    # Points generated by the page's model lambda * L = a * exp(b * S) with the Wan 2.2
    # coefficients ("Skip-Softmax calibration config") at several lengths and sparsities.
    g = json.load(open(os.path.join(GOLDEN, "wan22_calibration.json")))
    a0, b0 = g["a"], g["b"]
    L, lam, S = [], [], []
    for n in (4096, 16384, 75600):
        for s in (0.3, 0.5, 0.7, 0.9):
            L.append(n)
            S.append(s)
            lam.append(a0 * math.exp(b0 * s) / n)
    a, b = oracle.fit_calibration(L, lam, S)
    assert a == pytest.approx(a0, rel=1e-9)
    assert b == pytest.approx(b0, rel=1e-9)


def test_sparsity_curve_from_one_pass_equals_separate_runs():
    # Algorithm 2 step 1 sweeps many thresholds in one pass. The margins of a lambda = 0 run must
    # give, for every candidate, exactly the skip fraction of a run made with that candidate.
    torch.manual_seed(3)
    L, Hq, Hkv, d = 320, 2, 1, 16
    idx = torch.arange(L) // 32
    cen = torch.randn(L // 32 + 1, d, dtype=torch.float64) * 8 / math.sqrt(d)
    k = (3 * cen[idx] + 0.5 * torch.randn(L, d, dtype=torch.float64))[None, :, None, :]
    q = (cen[idx] + 0.5 * torch.randn(Hq, L, d, dtype=torch.float64)).permute(1, 0, 2)[None]
    v = torch.randn(1, L, Hkv, d, dtype=torch.float64)
    kw = dict(causal=True, block_r=32, block_c=32, scale=1 / math.sqrt(d))
    base = oracle.prefill(q, k, v, lam=0.0, **kw)
    margins = np.concatenate([u.tile_margin for u in base.units.values()])
    status = np.concatenate([u.tile_status for u in base.units.values()])
    lams = [0.0, 1e-4, 1e-3, 1e-2, 0.05, 0.2, 0.6, 1.0, 3.0]
    curve, n_vis = oracle.sparsity_curve(margins, status, lams)
    assert n_vis == sum(int(u.visited) for u in base.units.values())
    for lam, frac in zip(lams, curve):
        r = oracle.prefill(q, k, v, lam=lam, **kw)
        vis = sum(int(u.visited) for u in r.units.values())
        sk = sum(int(u.skipped) for u in r.units.values())
        assert vis == n_vis
        assert frac == sk / vis, (lam, frac, sk / vis)
    assert curve == sorted(curve) and 0 < curve[-2] < 1


# ------------------------------------------------------------------------------------------
# Sliding window (the talk notes' Q&A: windowed attention as structured sparsity): a row sees
# keys [row_first, row_keys). Tiles before every row's window are not visited.
# ------------------------------------------------------------------------------------------
def test_window_dense_rows_match_scipy():
    rng = np.random.default_rng(71)
    n_rows, n_keys, d, dv = 7, 90, 16, 12
    q = rng.standard_normal((n_rows, d))
    k = rng.standard_normal((n_keys, d))
    v = rng.standard_normal((n_keys, dv))
    row_keys = [90, 90, 60, 41, 41, 5, 90]
    row_first = [0, 30, 59, 1, 40, 0, 89]
    o, lse = oracle.dense_rows(q, k, v, row_keys, 0.3, row_first=row_first)
    o_ref, lse_ref = _library_attention(q, k, v, row_keys, 0.3, row_first)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", range(6))
def test_window_streaming_matches_closed_form(seed):
    rng = np.random.default_rng(300 + seed)
    n_rows = int(rng.integers(1, 7))
    n_keys = int(rng.integers(60, 300))
    block_c = int(rng.choice([8, 16, 33]))
    q, k, v = _clustered_rows(rng, n_rows, n_keys, 16, 6, beta=8.0)
    row_keys = sorted(rng.integers(n_keys // 2, n_keys + 1, size=n_rows).tolist())
    width = int(rng.integers(5, n_keys // 2))
    row_first = [max(0, e - width) for e in row_keys]
    for lam in (0.0, 1e-3, 0.1, 1.0):
        r = oracle.blasst_rows(q, k, v, row_keys, 0, n_keys, block_c, 0.25, lam,
                               row_first=row_first)
        cf = _closed_form(q, k, v, row_keys, 0.25, lam, block_c, row_first=row_first)
        vis = cf["visited"]
        first_tile = min(row_first) // block_c
        assert not vis[:first_tile].any()  # tiles before every window are not visited
        np.testing.assert_array_equal(r["tile_status"][vis] == oracle.TILE_SKIPPED,
                                      cf["skipped"][vis])
        assert np.all(r["tile_status"][~vis] == oracle.TILE_NOT_VISITED)
        np.testing.assert_allclose(r["tile_margin"][vis], cf["margin"][vis], rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["o"], cf["o"], rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(r["lse"], cf["lse"], rtol=1e-12, atol=1e-12)


def test_window_prefill_lambda_zero_matches_torch_sdpa_with_band_mask():
    from flashattention_softmax_threshold_amd.inputs import prefill_inputs

    B, L, Hq, Hkv, d, W = 1, 150, 4, 2, 16, 40
    q, k, v = prefill_inputs(B=B, L=L, Hq=Hq, Hkv=Hkv, d=d, cluster_len=32, dtype=torch.float32,
                             seed=9, beta=4.0, sinks=8)
    res = oracle.prefill(q, k, v, causal=True, block_r=32, block_c=16, scale=1 / math.sqrt(d),
                         lam=0.0, window=W)
    i = torch.arange(L)
    allowed = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    qt, kt, vt = (torch.as_tensor(x.numpy(), dtype=torch.float64).transpose(1, 2) for x in (q, k, v))
    kt, vt = kt.repeat_interleave(Hq // Hkv, dim=1), vt.repeat_interleave(Hq // Hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed)
    ref = ref.transpose(1, 2).numpy()
    for (b, h, qb), u in res.units.items():
        r0 = qb * 32
        r1 = r0 + u.o.shape[0]
        np.testing.assert_allclose(u.o, ref[b, r0:r1, h], rtol=1e-10, atol=1e-11)
        # Visited: the tiles meeting [r0 - W + 1, r1 - 1].
        assert u.visited == (r1 - 1) // 16 - max(0, r0 - W + 1) // 16 + 1
        assert np.all(u.tile_status[:max(0, r0 - W + 1) // 16] == oracle.TILE_NOT_VISITED)


def test_window_decode_lambda_zero_matches_softmax_with_lengths_and_splits():
    from flashattention_softmax_threshold_amd.inputs import decode_inputs

    B, Hq, Hkv, L, d, dv, W = 3, 8, 2, 300, 16, 12, 70
    kv_len = [300, 50, 129]
    q, k, v, kvl = decode_inputs(B=B, Hq=Hq, Hkv=Hkv, L=L, d_qk=d, d_v=dv, cluster_len=50,
                                 dtype=torch.float32, seed=15, beta=3.0, kv_len=kv_len)
    for splits in (1, 2, 5):
        res = oracle.decode(q, k, v, kv_len=kvl, block_r=4, block_c=32, num_splits=splits,
                            scale=0.25, lam=0.0, window=W)
        for (b, g, rb), u in res.units.items():
            n = kv_len[b]
            a = max(0, n - W)
            for i, h in enumerate(range(g * 4, g * 4 + 4)):
                s = 0.25 * (k[b, a:n, g].double() @ q[b, h].double())
                ref = torch.softmax(s, 0) @ v[b, a:n, g].double()
                np.testing.assert_allclose(u.o[i], ref.numpy(), rtol=1e-11, atol=1e-12)
                np.testing.assert_allclose(u.lse[i], torch.logsumexp(s, 0).item(), rtol=1e-12)
            assert u.visited == (n - 1) // 32 - a // 32 + 1
            assert np.all(u.tile_status[:a // 32] == oracle.TILE_NOT_VISITED)


def test_window_covering_everything_equals_no_window():
    from flashattention_softmax_threshold_amd.inputs import decode_inputs, prefill_inputs

    q, k, v = prefill_inputs(B=1, L=100, Hq=2, Hkv=1, d=16, cluster_len=20, dtype=torch.float32,
                             seed=4, beta=8.0, sinks=4)
    kw = dict(causal=True, block_r=32, block_c=16, scale=0.25, lam=0.05)
    a, b = oracle.prefill(q, k, v, **kw), oracle.prefill(q, k, v, window=100, **kw)
    qd, kd, vd, kvl = decode_inputs(B=2, Hq=4, Hkv=1, L=200, d_qk=16, d_v=16, cluster_len=40,
                                    dtype=torch.float32, seed=6, beta=8.0, kv_len=[200, 77])
    kwd = dict(kv_len=kvl, block_r=4, block_c=32, num_splits=1, scale=0.25, lam=0.05)
    c, e = oracle.decode(qd, kd, vd, **kwd), oracle.decode(qd, kd, vd, window=200, **kwd)
    for x, y in ((a, b), (c, e)):
        assert x.units.keys() == y.units.keys() and x.skipped > 0
        for key in x.units:
            ux, uy = x.units[key], y.units[key]
            assert np.array_equal(ux.o, uy.o) and np.array_equal(ux.lse, uy.lse)
            assert np.array_equal(ux.tile_status, uy.tile_status)
            assert ux.visited == uy.visited and ux.skipped == uy.skipped
