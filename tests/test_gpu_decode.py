"""GPU parity of blasst_attn_decode (GQA / MQA / MLA-shaped) against the fp64 oracle."""
import random

import numpy as np
import pytest
import torch

import oracle
import flashattention_softmax_threshold_amd as F
from flashattention_softmax_threshold_amd.inputs import decode_inputs, paged_layout

from parity import (MARGIN_BAND, assert_lse_close, assert_outputs_close, compare_tile_status, need_gpu,
                    oracle_scale)

pytestmark = pytest.mark.gpu


def _run_gpu(q, k, v, kv_len, *, lam, num_splits=0, block_r=0, block_table=None,
             max_kv_len=None, window=0):
    B, Hq, Dqk = q.shape
    br, bc, S = F.blasst_decode_plan(q, k, v, block_r=block_r, num_splits=num_splits,
                                     block_table=block_table, max_kv_len=max_kv_len,
                                     window=window)
    Hkv = k.shape[2]
    n_rb = -(-(Hq // Hkv) // br)
    nt = -(-(k.shape[1] if max_kv_len is None else max_kv_len) // bc)
    ts = torch.full((B, Hkv, n_rb, max(nt, 1)), 255, dtype=torch.uint8, device=q.device)
    tm = torch.zeros((B, Hkv, n_rb, max(nt, 1)), dtype=torch.float32, device=q.device)
    lse = torch.zeros((B, Hq), dtype=torch.float32, device=q.device)
    cnt = torch.zeros(2, dtype=torch.int64, device=q.device)
    o = F.blasst_attn_decode(q, k, v, kv_len=kv_len, lam=lam, lse=lse, counters=cnt,
                             tile_status=ts, tile_margin=tm, block_r=block_r,
                             num_splits=num_splits, block_table=block_table,
                             max_kv_len=max_kv_len, window=window)
    torch.cuda.synchronize()
    return dict(o=o, lse=lse, status=ts.cpu().numpy(), margin=tm.cpu().numpy(),
                counters=cnt.cpu().tolist(), br=br, bc=bc, splits=S)


def _check(res, ref, q, k, v, lam, what, kv_len, window=0):
    """Decisions agree outside the margin band; a unit with in-band flips is compared against
    the oracle evaluated with the GPU's decisions."""
    o_gpu = res["o"].float().cpu().numpy().astype(np.float64)
    lse_gpu = res["lse"].cpu().numpy().astype(np.float64)
    G = q.shape[1] // res["status"].shape[1]
    br = res["br"]
    band_mism = band = 0
    flipped = {}
    bw = MARGIN_BAND
    stats = {}
    for (b, g, rb), u in ref.units.items():
        nt = len(u.tile_status)
        st = res["status"][b, g, rb]
        m, n = compare_tile_status(st[:nt], u.tile_status, u.tile_margin, lam,
                                   f"{what} unit {(b, g, rb)}", bw,
                                   margin_gpu=res["margin"][b, g, rb][:nt], stats=stats)
        band_mism += m
        band += n
        assert np.all(st[nt:] == 2), f"{what}: tiles past kv_len must be 'not visited'"
        if m:
            flipped[(b, g, rb)] = st[:nt].copy()
    print(f"{what}: {len(ref.units)} units, {band} tiles in the margin band (+-{bw:.1e}), "
          f"{band_mism} decided the other way, max |d margin| {stats.get('max_dmargin', 0):.2e}",
          flush=True)
    units = dict(ref.units)
    if flipped:
        forced = oracle.decode(q, k, v, kv_len=kv_len, block_r=br, block_c=res["bc"],
                               num_splits=res["splits"], scale=oracle_scale(q.shape[2]), lam=lam,
                               units=list(flipped), forced=flipped, threads=16, window=window)
        units.update(forced.units)
    og, orf, lg, lr = [], [], [], []
    for (b, g, rb), u in units.items():
        h0 = g * G + rb * br
        rows = u.o.shape[0]
        og.append(o_gpu[b, h0:h0 + rows])
        orf.append(u.o)
        lg.append(lse_gpu[b, h0:h0 + rows])
        lr.append(u.lse)
    assert_outputs_close(np.concatenate(og), np.concatenate(orf), q.dtype, what,
                         lse_ref=np.concatenate(lr))
    assert_lse_close(np.concatenate(lg), np.concatenate(lr), q.dtype, what)
    return band_mism


def _case(B, Hq, Hkv, L, D, kv_len, lams, splits, beta, share, seed, block_r=0, Dv=None,
          cluster_len=100, window=0):
    need_gpu()
    Dv = D if Dv is None else Dv
    mla = Dv != D
    q, k, v, kvl = decode_inputs(B=B, Hq=Hq, Hkv=Hkv, L=L, d_qk=D, d_v=Dv, cluster_len=cluster_len,
                                 dtype=torch.bfloat16, seed=seed, beta=beta, share=share,
                                 v_aliases_k=mla, kv_len=kv_len)
    # Head-major cache storage on the device, as the generator lays it out.
    kd = k.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    if mla:
        vd = kd[..., :Dv]
    else:
        vd = v.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    qd, kvd = q.cuda(), kvl.cuda()
    skipped = 0
    for S in splits:
        for lam in lams:
            what = (f"decode B{B} H{Hq}/{Hkv} L{L} d{D}/{Dv} S={S} beta={beta} lam={lam} "
                    f"window={window}")
            print(what, flush=True)
            res = _run_gpu(qd, kd, vd, kvd, lam=lam, num_splits=S, block_r=block_r, window=window)
            ref = oracle.decode(q, k, v, kv_len=kvl, block_r=res["br"], block_c=res["bc"],
                                num_splits=res["splits"], scale=oracle_scale(D), lam=lam,
                                threads=8, window=window)
            band_mism = _check(res, ref, q, k, v, lam, what, kvl, window)
            assert res["counters"][0] == ref.visited
            assert abs(res["counters"][1] - ref.skipped) <= band_mism
            skipped += ref.skipped
    return skipped


def test_gqa_small_lengths_and_splits():
    L = 1000
    kv_len = [1000, 1, 577]
    lams = [0.0, 16 / L, 64 / L, 1.0]
    _case(3, 8, 2, L, 128, kv_len, lams[:2], (1, 3), 1.0, False, seed=21)
    assert _case(3, 8, 2, L, 128, kv_len, lams, (1, 3, 7), 16.0, False, seed=22) > 0


def test_gqa_empty_sequence_d64_and_odd_group():
    # kv_len 0 gives o = 0, lse = -inf; head dim 64; 3 query heads per KV head (padded rows).
    _case(2, 6, 2, 300, 64, [0, 300], [0.0, 0.05], (1, 2), 8.0, True, seed=23)
    assert _case(2, 6, 2, 300, 128, [129, 300], [0.0, 0.2], (1,), 8.0, True, seed=24) > 0


def test_mqa_two_row_blocks():
    assert _case(2, 32, 1, 700, 128, None, [0.0, 0.02], (1, 2), 16.0, True, seed=25) > 0


def test_gqa_decode_full_size_sampled():
    """GQA decode at full size: 64 sequences x 32/8 heads, KV length 32768, d 128."""
    need_gpu()
    B, Hq, Hkv, L = 64, 32, 8, 32768
    q, k, v, kvl = decode_inputs(B=B, Hq=Hq, Hkv=Hkv, L=L, d_qk=128, d_v=128, cluster_len=512,
                                 dtype=torch.bfloat16, device="cuda", seed=3000, beta=16.0)
    rng = random.Random(3)
    units = [(0, 0, 0), (63, 7, 0)] + rng.sample(
        [(b, g, 0) for b in range(1, 63) for g in range(Hkv)], 62)
    for a in (4, 16, 64):
        lam = a / L
        what = f"C3 lam={a}/L"
        print(what, flush=True)
        res = _run_gpu(q, k, v, kvl, lam=lam)
        ref = oracle.decode(q, k, v, kv_len=kvl, block_r=res["br"], block_c=res["bc"],
                            num_splits=res["splits"], scale=oracle_scale(128), lam=lam,
                            units=units, threads=16)
        _check(res, ref, q, k, v, lam, what, kvl)
        st = res["status"]
        assert res["counters"][0] == int((st != 2).sum())
        assert res["counters"][1] == int((st == 1).sum())
        assert ref.skipped > 0


@pytest.mark.parametrize("Hq,Hkv,D,splits", [(32, 8, 128, 0), (16, 2, 64, 3), (4, 4, 128, 1)])
def test_layouts_equal_heads_major_bitwise(Hq, Hkv, D, splits):
    """The decode kernels address Q, K, V and O through their strides only: K and V stored
    token-major ([B, L, Hkv, D] contiguous), the query sliced from a packed [B, Hq + 2 Hkv, D]
    projection and O written into a wider buffer give the same bits as the heads-major cache."""
    need_gpu()
    B, L = 3, 1500
    q, k, v, kvl = decode_inputs(B=B, Hq=Hq, Hkv=Hkv, L=L, d_qk=D, d_v=D, cluster_len=64,
                                 dtype=torch.bfloat16, seed=3500 + Hq + D, beta=16.0, share=True,
                                 kv_len=[1500, 999, 64])
    qd, kvd = q.cuda(), kvl.cuda()
    kh = k.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    vh = v.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    kt, vt = kh.contiguous(), vh.contiguous()
    packed = torch.cat([qd, torch.zeros((B, 2 * Hkv, D), dtype=qd.dtype, device="cuda")], dim=1)
    qp = packed[:, :Hq]
    o_wide = torch.full((B, Hq, D + 64), 3.0, dtype=torch.bfloat16, device="cuda")
    lam = 16.0 / L

    def run(qq, kk, vv, o):
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        F.blasst_attn_decode(qq, kk, vv, kv_len=kvd, lam=lam, o=o, lse=lse, counters=cnt,
                             num_splits=splits)
        torch.cuda.synchronize()
        return o, lse, cnt

    ref = run(qd, kh, vh, torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda"))
    assert not kh.is_contiguous() and kt.is_contiguous() and not qp.is_contiguous()
    got = run(qp, kt, vt, o_wide[:, :, :D])
    print(f"decode layouts Hq{Hq} Hkv{Hkv} d{D} splits {splits}: counters {ref[2].tolist()}",
          flush=True)
    for what, a_, b_ in zip(("o", "lse", "counters"), ref, got):
        assert torch.equal(a_, b_), f"{what} differs from the heads-major call"
    assert torch.all(o_wide[:, :, D:] == 3.0), "columns past d_v were written"


@pytest.mark.parametrize("block_r", [0, 64])
def test_mla_small_lengths_and_splits(block_r):
    """MLA shape: 128 query heads on one latent KV head, d_qk 576, V = the first 512 columns;
    one unit of 128 heads (the default) or two of 64."""
    L = 700
    lams = [0.0, 16 / L, 1.0]
    _case(2, 128, 1, L, 576, [700, 321], lams[:2], (1, 3), 1.0, True, seed=31, Dv=512,
          cluster_len=128, block_r=block_r)
    assert _case(2, 128, 1, L, 576, [700, 130], lams, (1, 4), 16.0, True, seed=32, Dv=512,
                 cluster_len=128, block_r=block_r) > 0


@pytest.mark.parametrize("Hq,block_r", [(16, 0), (40, 0), (100, 64), (100, 0), (72, 0),
                                        (65, 0), (200, 0)])
def test_mla_partial_head_blocks(Hq, block_r):
    """MLA with head counts that leave row groups empty or partial. 64-head kernel: 16 (the
    second 32-head group of the only block empty), 40 (half full), 100 with blocks of 64 (a
    partial second block, heads 64..99): every wave's P.V covers both row groups of its block.
    128-head kernel: 100 (the last wave's rows 96..127 partly empty), 72 (waves 2 and 3
    with 8 and no valid rows), 65 (one valid row in wave 2), 200 (a second block of 72 heads). Invalid rows must neither
    leak into valid ones nor be written, and must not take part in the vote."""
    L = 600
    lams = [0.0, 16 / L, 1.0]
    assert _case(2, Hq, 1, L, 576, [600, 257], lams, (1, 3), 16.0, True, seed=3300 + Hq, Dv=512,
                 cluster_len=128, block_r=block_r) > 0


def test_gqa_sliding_window_lengths_and_splits():
    """Sliding windows of one key, shorter than a tile, and a few tiles not a multiple of the
    tile, on ragged lengths (one sequence shorter than the window), unsplit and split."""
    L = 1300
    kv_len = [1300, 1, 200, 1029]
    for w, seed in ((1, 41), (50, 42), (333, 43)):
        n = _case(4, 8, 2, L, 128, kv_len, [0.0, 16 / w, 1.0], (1, 2, 0), 16.0, False, seed=seed,
                  window=w)
        assert n > 0 or w == 1


@pytest.mark.parametrize("block_r", [0, 64])
def test_mla_sliding_window_and_splits(block_r):
    L = 900
    assert _case(2, 128, 1, L, 576, [900, 300], [0.0, 16 / 400, 1.0], (1, 3), 16.0, True,
                 seed=44, Dv=512, cluster_len=128, window=400, block_r=block_r) > 0


def test_paged_gqa_sliding_window_equals_contiguous_bitwise():
    _paged_vs_contiguous(B=2, Hq=8, Hkv=2, L=1000, D=128, Dv=128, kv_len=[1000, 450],
                         page_sizes=(16, 128), lams=(0.0, 16 / 300), splits=(1, 2), beta=16.0,
                         share=True, seed=8400, window=300)


def test_mla_decode_full_size_sampled():
    """MLA-shaped decode at full size: 32 sequences x 128 heads, KV 65536, d_qk 576 / d_v 512."""
    need_gpu()
    B, Hq, L = 32, 128, 65536
    q, k, v, kvl = decode_inputs(B=B, Hq=Hq, Hkv=1, L=L, d_qk=576, d_v=512, cluster_len=1024,
                                 dtype=torch.bfloat16, device="cuda", seed=5000, beta=16.0,
                                 share=True, v_aliases_k=True)
    units = None  # all 64 (sequence, row block) units, every split
    for a in (4, 64):
        lam = a / L
        what = f"MLA lam={a}/L"
        print(what, flush=True)
        res = _run_gpu(q, k, v, kvl, lam=lam)
        ref = oracle.decode(q, k, v, kv_len=kvl, block_r=res["br"], block_c=res["bc"],
                            num_splits=res["splits"], scale=oracle_scale(576), lam=lam,
                            units=units, threads=16)
        _check(res, ref, q, k, v, lam, what, kvl)
        st = res["status"]
        assert res["counters"][0] == int((st != 2).sum())
        assert res["counters"][1] == int((st == 1).sum())


# ------------------------------------------------------------------------------------------
# Paged KV cache ("The Hitchhiker's Guide -- Phase 08", paged attention: a block table maps a
# sequence position to a physical block). Paging changes only where a key row is read, so every
# output must equal the contiguous call on the same keys bit for bit.
# ------------------------------------------------------------------------------------------
def _paged_vs_contiguous(B, Hq, Hkv, L, D, Dv, kv_len, page_sizes, lams, splits, beta, share, seed,
                         cluster_len=100, window=0, heads_major=False, block_r=0):
    need_gpu()
    mla = Dv != D
    q, k, v, kvl = decode_inputs(B=B, Hq=Hq, Hkv=Hkv, L=L, d_qk=D, d_v=Dv, cluster_len=cluster_len,
                                 dtype=torch.bfloat16, device="cuda", seed=seed, beta=beta,
                                 share=share, v_aliases_k=mla, kv_len=kv_len)
    for ps in page_sizes:
        kp, vp, table = paged_layout(k, v, ps, seed=seed + ps, kv_len=kvl, heads_major=heads_major)
        for S in splits:
            for lam in lams:
                what = f"paged decode B{B} H{Hq}/{Hkv} L{L} d{D}/{Dv} page {ps} S={S} lam={lam}"
                print(what, flush=True)
                ref = _run_gpu(q, k, v, kvl, lam=lam, num_splits=S, window=window,
                               block_r=block_r)
                got = _run_gpu(q, kp, vp, kvl, lam=lam, num_splits=S, block_table=table,
                               max_kv_len=L, window=window, block_r=block_r)
                assert got["splits"] == ref["splits"]
                assert torch.equal(got["o"], ref["o"]), what
                assert np.array_equal(got["lse"].cpu().numpy(), ref["lse"].cpu().numpy()), what
                assert np.array_equal(got["status"], ref["status"]), what
                assert np.array_equal(got["margin"], ref["margin"]), what
                assert got["counters"] == ref["counters"], what
    return q, kp, vp, table, kvl, k, v


def test_paged_gqa_equals_contiguous_bitwise():
    _paged_vs_contiguous(B=3, Hq=16, Hkv=4, L=1100, D=128, Dv=128, kv_len=[1100, 517, 0],
                         page_sizes=(1, 16, 64, 256), lams=(0.0, 16 / 1100), splits=(1, 3),
                         beta=16.0, share=True, seed=8100)


def test_paged_gqa_heads_major_pages_equal_contiguous_bitwise():
    # Pages stored [head, row, dim]: the same pools described by other strides.
    _paged_vs_contiguous(B=2, Hq=16, Hkv=4, L=900, D=128, Dv=128, kv_len=[900, 300],
                         page_sizes=(16, 64), lams=(0.0, 16 / 900), splits=(1, 2), beta=16.0,
                         share=True, seed=8500, heads_major=True)


def test_paged_gqa_against_oracle():
    q, kp, vp, table, kvl, k, v = _paged_vs_contiguous(
        B=2, Hq=8, Hkv=2, L=700, D=128, Dv=128, kv_len=[700, 333], page_sizes=(32,),
        lams=(16 / 700,), splits=(2,), beta=16.0, share=True, seed=8200)
    lam = 16 / 700
    res = _run_gpu(q, kp, vp, kvl, lam=lam, num_splits=2, block_table=table, max_kv_len=700)
    kc, vc, qc, kvc = k.cpu(), v.cpu(), q.cpu(), kvl.cpu()
    ref = oracle.decode(qc, kc, vc, kv_len=kvc, block_r=res["br"], block_c=res["bc"],
                        num_splits=res["splits"], scale=oracle_scale(128), lam=lam, threads=8)
    band_mism = _check(res, ref, qc, kc, vc, lam, "paged decode vs oracle", kvc)
    assert res["counters"][0] == ref.visited
    assert abs(res["counters"][1] - ref.skipped) <= band_mism


@pytest.mark.parametrize("block_r", [0, 64])
def test_paged_mla_equals_contiguous_bitwise(block_r):
    _paged_vs_contiguous(B=2, Hq=128, Hkv=1, L=700, D=576, Dv=512, kv_len=[700, 129],
                         page_sizes=(16, 64), lams=(0.0, 16 / 700), splits=(1, 2), beta=4.0,
                         share=True, seed=8300, cluster_len=128, block_r=block_r)
