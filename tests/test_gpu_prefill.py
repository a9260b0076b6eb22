"""GPU parity of blasst_attn_prefill against the fp64 oracle, element by element."""
import random

import numpy as np
import pytest
import torch

import oracle
import flashattention_softmax_threshold_amd as F
from flashattention_softmax_threshold_amd.inputs import prefill_inputs

from parity import (MARGIN_BAND, assert_lse_close, assert_outputs_close, compare_tile_status, need_gpu,
                    oracle_scale)

pytestmark = pytest.mark.gpu


def _run_gpu(q, k, v, *, causal, lam, block_r=0, window=0):
    B, Lq, Hq, D = q.shape
    br, bc = F.blasst_prefill_tiles(q, k, block_r=block_r)
    nqb, nkt = -(-Lq // br), -(-k.shape[1] // bc)
    ts = torch.full((B, Hq, nqb, nkt), 255, dtype=torch.uint8, device=q.device)
    tm = torch.zeros((B, Hq, nqb, nkt), dtype=torch.float32, device=q.device)
    lse = torch.zeros((B, Hq, Lq), dtype=torch.float32, device=q.device)
    cnt = torch.zeros(2, dtype=torch.int64, device=q.device)
    o = F.blasst_attn_prefill(q, k, v, causal=causal, lam=lam, lse=lse, counters=cnt,
                              tile_status=ts, tile_margin=tm, block_r=block_r, window=window)
    torch.cuda.synchronize()
    return dict(o=o, lse=lse, status=ts.cpu().numpy(), margin=tm.cpu().numpy(),
                counters=cnt.cpu().tolist(), br=br, bc=bc)


def _check_units(res, ref, q, k, v, causal, lam, what, window=0):
    """Compare the oracle's units with the GPU outputs of the same units.

    Tile decisions must agree outside the margin band. A unit whose decisions differ inside the
    band is compared against the oracle evaluated with the GPU's decisions."""
    o_gpu = res["o"].float().cpu().numpy().astype(np.float64)
    lse_gpu = res["lse"].cpu().numpy().astype(np.float64)
    br = res["br"]
    band_mism = band = 0
    flipped = {}
    bw = MARGIN_BAND
    stats = {}
    for (b, h, qb), u in ref.units.items():
        nt = len(u.tile_status)
        st = res["status"][b, h, qb, :nt]
        m, n = compare_tile_status(st, u.tile_status, u.tile_margin, lam,
                                   f"{what} unit {(b, h, qb)}", bw,
                                   margin_gpu=res["margin"][b, h, qb, :nt], stats=stats)
        band_mism += m
        band += n
        if m:
            flipped[(b, h, qb)] = st.copy()
    print(f"{what}: {len(ref.units)} units, {band} tiles in the margin band (+-{bw:.1e}), "
          f"{band_mism} decided the other way, max |d margin| {stats.get('max_dmargin', 0):.2e}",
          flush=True)
    units = dict(ref.units)
    if flipped:
        forced = oracle.prefill(q, k, v, causal=causal, block_r=br, block_c=res["bc"],
                                scale=oracle_scale(q.shape[3]), lam=lam, units=list(flipped),
                                forced=flipped, threads=16, window=window)
        units.update(forced.units)
    og, orf, lg, lr = [], [], [], []
    for (b, h, qb), u in units.items():
        r0 = qb * br
        rows = u.o.shape[0]
        og.append(o_gpu[b, r0:r0 + rows, h])
        orf.append(u.o)
        lg.append(lse_gpu[b, h, r0:r0 + rows])
        lr.append(u.lse)
    o_g, o_r = np.concatenate(og), np.concatenate(orf)
    err = assert_outputs_close(o_g, o_r, q.dtype, what, lse_ref=np.concatenate(lr))
    assert_lse_close(np.concatenate(lg), np.concatenate(lr), q.dtype, what)
    return err, band_mism, band


def _case(B, L, Hq, Hkv, D, dtype, causal, block_r, beta, lams, seed, cluster_len=64, sinks=0,
          window=0):
    need_gpu()
    q, k, v = prefill_inputs(B=B, L=L, Hq=Hq, Hkv=Hkv, d=D, cluster_len=cluster_len, dtype=dtype,
                             seed=seed, beta=beta, sinks=sinks)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    skipped_any = False
    for lam in lams:
        what = (f"prefill B{B} L{L} H{Hq}/{Hkv} d{D} {dtype} causal={causal} br={block_r} "
                f"beta={beta} lam={lam} window={window}")
        print(what, flush=True)
        res = _run_gpu(qd, kd, vd, causal=causal, lam=lam, block_r=block_r, window=window)
        ref = oracle.prefill(q, k, v, causal=causal, block_r=res["br"], block_c=res["bc"],
                             scale=oracle_scale(D), lam=lam, threads=8, window=window)
        _, band_mism, _ = _check_units(res, ref, q, k, v, causal, lam, what, window)
        # Counters: the oracle's totals, up to decisions inside the margin band.
        assert res["counters"][0] == ref.visited
        assert abs(res["counters"][1] - ref.skipped) <= band_mism
        skipped_any |= ref.skipped > 0
    return skipped_any


def test_tiny_fp32_mha_all_lambdas():
    """The tiny fp32 workload: B1 H2 L512 d64, tile 64x64, lambda in {0, 1e-3, 1e-2, 1e-1}."""
    lams = [0.0, 1e-3, 1e-2, 1e-1]
    _case(1, 512, 2, 2, 64, torch.float32, False, 64, 1.0, lams, seed=1000)
    assert _case(1, 512, 2, 2, 64, torch.float32, False, 64, 8.0, lams, seed=1001)


@pytest.mark.parametrize("dtype,D,block_r,lq,lkv", [
    (torch.bfloat16, 128, 128, 300, 1000),
    (torch.bfloat16, 128, 128, 1000, 77),
    (torch.bfloat16, 64, 64, 129, 700),
    (torch.float32, 64, 64, 200, 513),
])
def test_cross_length_non_causal(dtype, D, block_r, lq, lkv):
    """Non-causal prefill with Lq != Lkv (cross attention), including a key range shorter than
    one query block (q, k and v are the leading rows of longer generated tensors)."""
    need_gpu()
    B, Hq, Hkv = 2, 8, 2
    q, k, v = prefill_inputs(B=B, L=max(lq, lkv), Hq=Hq, Hkv=Hkv, d=D, cluster_len=64,
                             dtype=dtype, seed=5100 + lq, beta=16.0)
    q, k, v = q[:, :lq], k[:, :lkv], v[:, :lkv]
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    skipped = 0
    for lam in (0.0, 16 / lkv, 1.0):
        what = f"cross prefill {dtype} d{D} br{block_r} Lq{lq} Lkv{lkv} lam={lam}"
        print(what, flush=True)
        res = _run_gpu(qd, kd, vd, causal=False, lam=lam, block_r=block_r)
        ref = oracle.prefill(q, k, v, causal=False, block_r=res["br"], block_c=res["bc"],
                             scale=oracle_scale(D), lam=lam, threads=8)
        _, band_mism, _ = _check_units(res, ref, q, k, v, False, lam, what)
        assert res["counters"][0] == ref.visited
        assert abs(res["counters"][1] - ref.skipped) <= band_mism
        skipped += ref.skipped
    assert skipped > 0


@pytest.mark.parametrize("dtype,D,causal,Hq,Hkv", [
    (torch.bfloat16, 128, True, 8, 2),
    (torch.bfloat16, 128, False, 3, 1),
    (torch.bfloat16, 64, True, 4, 4),
    (torch.float32, 64, False, 4, 2),
])
def test_packed_qkv_and_heads_major_layouts_equal_contiguous_bitwise(dtype, D, causal, Hq, Hkv):
    """The kernels address Q, K, V and O through their batch, row and head strides only: q, k
    and v sliced out of one packed [B, L, Hq + 2 Hkv, D] projection, K and V stored heads-major
    ([B, H, L, D] storage) and O written heads-major give the same bits as contiguous tensors."""
    need_gpu()
    B, L = 2, 333
    q, k, v = prefill_inputs(B=B, L=L, Hq=Hq, Hkv=Hkv, d=D, cluster_len=64, dtype=dtype,
                             device="cuda", seed=5600 + D + Hq, beta=16.0, sinks=8)
    packed = torch.cat([q, k, v], dim=2)
    qp, kp, vp = packed[:, :, :Hq], packed[:, :, Hq:Hq + Hkv], packed[:, :, Hq + Hkv:]
    kh = k.transpose(1, 2).contiguous().transpose(1, 2)
    vh = v.transpose(1, 2).contiguous().transpose(1, 2)
    assert not qp.is_contiguous() and (Hkv == 1 or not kh.is_contiguous())
    lam = 16.0 / L

    def run(qq, kk, vv, o):
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        F.blasst_attn_prefill(qq, kk, vv, causal=causal, lam=lam, o=o, lse=lse, counters=cnt)
        torch.cuda.synchronize()
        return o, lse, cnt

    ref = run(q, k, v, torch.empty_like(q))
    o_heads_major = torch.empty((B, Hq, L, D), dtype=dtype, device="cuda").transpose(1, 2)
    for name, args in (("packed qkv", (qp, kp, vp, torch.empty_like(q))),
                       ("heads-major k/v and o", (q, kh, vh, o_heads_major))):
        print(f"layout {name} {dtype} d{D} causal={causal} Hq{Hq} Hkv{Hkv}", flush=True)
        got = run(*args)
        for what, a_, b_ in zip(("o", "lse", "counters"), ref, got):
            assert torch.equal(a_, b_), f"{name}: {what} differs from the contiguous call"


@pytest.mark.parametrize("causal", [True, False])
def test_fp32_four_wave_query_blocks(causal):
    """fp32 with B_r = 128 (the generic kernel with four waves per workgroup) on ragged lengths."""
    need_gpu()
    L, D = 300, 64
    q, k, v = prefill_inputs(B=2, L=L, Hq=4, Hkv=2, d=D, cluster_len=64, dtype=torch.float32,
                             seed=5700 + causal, beta=16.0, sinks=8)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for lam in (0.0, 16 / L, 0.3):
        what = f"fp32 B_r 128 causal={causal} lam={lam}"
        print(what, flush=True)
        res = _run_gpu(qd, kd, vd, causal=causal, lam=lam, block_r=128)
        assert res["br"] == 128
        ref = oracle.prefill(q, k, v, causal=causal, block_r=128, block_c=res["bc"],
                             scale=oracle_scale(D), lam=lam, threads=8)
        _, band_mism, _ = _check_units(res, ref, q, k, v, causal, lam, what)
        assert res["counters"][0] == ref.visited
        assert abs(res["counters"][1] - ref.skipped) <= band_mism


def test_bf16_row_stride_beyond_32_bit_tile_offsets():
    """A K row stride of 2^25 elements puts 64 rows of a tile past a 32-bit byte offset, which
    the B_r = 128 MFMA kernel keeps per lane; such a call runs on the generic kernel (64-bit
    addresses) and still matches the oracle. The K storage spans about 9 GB."""
    need_gpu()
    B, L, Hq, Hkv, D = 1, 130, 2, 1, 64
    S = 1 << 25
    q, k, v = prefill_inputs(B=B, L=L, Hq=Hq, Hkv=Hkv, d=D, cluster_len=32, dtype=torch.bfloat16,
                             seed=5800, beta=16.0, sinks=4)
    big = torch.empty(((L - 1) * S + D,), dtype=torch.bfloat16, device="cuda")
    kd = big.as_strided((B, L, Hkv, D), (L * S, S, D, 1))
    kd.copy_(k)
    qd, vd = q.cuda(), v.cuda()
    assert kd.stride(1) == S and torch.equal(kd.cpu(), k)
    try:
        for causal in (True, False):
            for lam in (0.0, 16 / L):
                what = f"bf16 row stride 2^25 causal={causal} lam={lam}"
                print(what, flush=True)
                res = _run_gpu(qd, kd, vd, causal=causal, lam=lam)
                ref = oracle.prefill(q, k, v, causal=causal, block_r=res["br"], block_c=res["bc"],
                                     scale=oracle_scale(D), lam=lam, threads=8)
                _, band_mism, _ = _check_units(res, ref, q, k, v, causal, lam, what)
                assert res["counters"][0] == ref.visited
                assert abs(res["counters"][1] - ref.skipped) <= band_mism
    finally:
        del kd, big
        torch.cuda.empty_cache()


@pytest.mark.parametrize("block_r", [128, 64, 32])
def test_bf16_causal_gqa_ragged(block_r):
    L = 700
    lams = [0.0, 4 / L, 64 / L, 1.0, 5.0]
    _case(2, L, 8, 2, 128, torch.bfloat16, True, block_r, 1.0, lams[:2], seed=7, sinks=16)
    assert _case(2, L, 8, 2, 128, torch.bfloat16, True, block_r, 32.0, lams, seed=8,
                 cluster_len=128, sinks=16)


@pytest.mark.parametrize("L,Hq,Hkv,D", [(300, 3, 3, 128), (513, 3, 1, 128), (640, 2, 2, 64),
                                         (129, 1, 1, 128)])
def test_bf16_noncausal_query_block_pairs(L, Hq, Hkv, D):
    """Non-causal calls whose query heads do not pair up run two neighbouring 128-row query
    blocks of one head per workgroup; an odd block count leaves the last pair's second unit
    empty (it must record nothing), an even one fills every pair."""
    assert _case(2, L, Hq, Hkv, D, torch.bfloat16, False, 128, 16.0, [0.0, 16 / L, 1.0],
                 seed=5200 + L + Hq, cluster_len=64)


def test_bf16_noncausal_d64_and_fp32_causal_d128():
    assert _case(1, 333, 4, 4, 64, torch.bfloat16, False, 128, 16.0, [0.0, 0.01, 0.3], seed=9)
    assert _case(1, 200, 2, 1, 128, torch.float32, True, 64, 16.0, [0.0, 0.05], seed=10)


def test_edge_lengths():
    # A single key, fewer rows than a block, lengths one past a tile.
    _case(1, 1, 2, 1, 128, torch.bfloat16, False, 128, 8.0, [0.0, 0.5], seed=11)
    _case(3, 65, 2, 2, 64, torch.bfloat16, True, 64, 8.0, [0.0, 0.5], seed=12)
    _case(1, 129, 4, 2, 128, torch.float32, False, 32, 8.0, [0.0, 1.0], seed=13)


@pytest.mark.parametrize("L", [128, 191, 192, 193, 256, 320, 321])
def test_two_unit_full_tile_loop_boundaries(L):
    """Two units per workgroup (paired GQA heads, causal; neighbouring query blocks, non-causal)
    run the steps whose copies are all full key tiles in a loop of their own, then the rest:
    lengths at and around multiples of the 64-key tile change how many steps each loop takes
    (none, one pair, several, with and without a partial last tile), also under a window."""
    lams = [0.0, 16 / L, 1.0]
    _case(1, L, 4, 2, 128, torch.bfloat16, True, 128, 16.0, lams, seed=6100 + L,
          cluster_len=64, sinks=8)
    _case(2, L, 3, 3, 64, torch.bfloat16, False, 128, 16.0, lams, seed=6200 + L, cluster_len=64)
    _case(1, L, 4, 2, 128, torch.bfloat16, True, 128, 16.0, lams[:2], seed=6300 + L,
          cluster_len=64, window=130)


def _sampled_full_size(q, k, v, causal, lam, units, what, window=0):
    res = _run_gpu(q, k, v, causal=causal, lam=lam, window=window)
    ref = oracle.prefill(q, k, v, causal=causal, block_r=res["br"], block_c=res["bc"],
                         scale=oracle_scale(q.shape[3]), lam=lam, units=units, threads=16,
                         window=window)
    err, band_mism, band = _check_units(res, ref, q, k, v, causal, lam, what, window)
    # Whole-call counters agree with the whole-call tile map the kernel wrote.
    st = res["status"]
    assert res["counters"][0] == int((st != 2).sum())
    assert res["counters"][1] == int((st == 1).sum())
    return res, ref


@pytest.mark.parametrize("beta", [1.0, 32.0])
def test_causal_gqa_8k_full_size_sampled(beta):
    """Causal GQA prefill at full size (B1, 32/8 heads, L 8192, d 128, tile 128x64)."""
    need_gpu()
    L = 8192
    q, k, v = prefill_inputs(B=1, L=L, Hq=32, Hkv=8, d=128, cluster_len=256,
                             dtype=torch.bfloat16, device="cuda", seed=2000, beta=beta, sinks=64)
    rng = random.Random(5)
    units = [(0, 0, 0), (0, 31, 63), (0, 5, 63)] + rng.sample(
        [(0, h, qb) for h in range(32) for qb in range(64)], 61)
    for a in (4, 16, 64):
        what = f"C2 beta={beta} lam={a}/L"
        print(what, flush=True)
        res, ref = _sampled_full_size(q, k, v, True, a / L, units, what)
        if beta > 1:
            assert ref.skipped > 0


@pytest.mark.parametrize("block_r", [128, 64])
def test_bf16_causal_gqa_sliding_window(block_r):
    """Causal sliding windows: one key (the diagonal only), shorter than a tile, a few tiles
    and not a multiple of the tile, on ragged lengths. (Windows shorter than a tile leave every
    visited tile holding some row's own maximum, so only the longest one skips.)"""
    L = 1000
    for w, seed in ((1, 20), (40, 21), (333, 22)):
        skipped = _case(2, L, 8, 2, 128, torch.bfloat16, True, block_r, 32.0, [0.0, 16 / w, 1.0],
                        seed=seed, cluster_len=128, sinks=16, window=w)
        assert skipped or w < 64


def test_fp32_causal_sliding_window():
    assert _case(1, 400, 2, 1, 64, torch.float32, True, 64, 16.0, [0.0, 0.5], seed=23,
                 cluster_len=32, window=250)


def test_causal_gqa_8k_sliding_window_full_size_sampled():
    """The full-size causal GQA workload with a 2048-key window."""
    need_gpu()
    L, W = 8192, 2048
    q, k, v = prefill_inputs(B=1, L=L, Hq=32, Hkv=8, d=128, cluster_len=256,
                             dtype=torch.bfloat16, device="cuda", seed=2000, beta=32.0, sinks=64)
    units = [(0, 0, 0), (0, 31, 63), (0, 5, 20), (0, 12, 16), (0, 20, 40)]
    for a in (16, 64):
        what = f"C2 window={W} lam={a}/W"
        print(what, flush=True)
        res, ref = _sampled_full_size(q, k, v, True, a / W, units, what, window=W)
        assert ref.skipped > 0


@pytest.mark.parametrize("beta", [1.0, 4.0])
def test_video_dit_full_size_sampled(beta):
    """Video-DiT self-attention at full size (40 heads, L 75600 = 21 frames x 3600, d 128)."""
    need_gpu()
    L = 75600
    q, k, v = prefill_inputs(B=1, L=L, Hq=40, Hkv=40, d=128, cluster_len=60,
                             dtype=torch.bfloat16, device="cuda", seed=4000, beta=beta,
                             frame_len=3600, patch_len=60)
    a, b = 2822.6209952221557, 4.388250623520793
    rng = random.Random(6)
    units = [(0, 0, 0), (0, 39, 590), (0, 17, 300), (0, 3, 77)] + rng.sample(
        [(0, h, qb) for h in range(40) for qb in range(591)], 60)
    for s in (0.5, 0.7):
        lam = F.blasst_resolve_lambda(F.BLASST_TARGET_SPARSITY, L, target_sparsity=s, a=a, b=b)
        what = f"C4 beta={beta} s={s} lam={lam:.4f}"
        print(what, flush=True)
        _sampled_full_size(q, k, v, False, lam, units, what)
