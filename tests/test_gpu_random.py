"""Seeded random configurations through the C ABI against the fp64 oracle.

Each case draws its shape, lengths, thresholds, window, split count and cache layout from a fixed
seed, so a failure names a reproducible case. The shapes stay small (the oracle evaluates every
unit); the comparison and its tolerances are those of the other parity tests: decisions exact
outside the margin band, outputs, LSE and counters against the oracle.
"""
import math
import random

import pytest
import torch

import oracle
from flashattention_softmax_threshold_amd.inputs import decode_inputs, paged_layout

from parity import need_gpu, oracle_scale
import test_gpu_decode as dec
import test_gpu_prefill as pre

pytestmark = pytest.mark.gpu


def _prefill_case(seed):
    rng = random.Random(seed)
    dtype = rng.choice([torch.bfloat16, torch.bfloat16, torch.float32])
    D = rng.choice([64, 128])
    Hkv = rng.choice([1, 2, 4])
    Hq = Hkv * rng.choice([1, 2, 3, 4])
    L = rng.randrange(1, 700)
    causal = rng.random() < 0.7
    window = rng.choice([0, 0, rng.randrange(1, 400)]) if causal else 0
    block_r = rng.choice([128, 64, 32]) if dtype == torch.bfloat16 else rng.choice([64, 32])
    beta = rng.choice([1.0, 8.0, 32.0])
    lam = rng.choice([0.0, 4.0 / max(L, 1), 64.0 / max(L, 1), 0.3, 1.0])
    return dict(B=rng.choice([1, 2]), L=L, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, causal=causal,
                window=window, block_r=block_r, beta=beta, lam=lam,
                cluster_len=rng.choice([16, 64, 128]), sinks=rng.choice([0, 8]))


@pytest.mark.parametrize("seed", range(100))
def test_random_prefill(seed):
    need_gpu()
    c = _prefill_case(9000 + seed)
    what = f"random prefill seed={9000 + seed} {c}"
    print(what, flush=True)
    pre._case(c["B"], c["L"], c["Hq"], c["Hkv"], c["D"], c["dtype"], c["causal"], c["block_r"],
              c["beta"], [c["lam"]], seed=9000 + seed, cluster_len=c["cluster_len"],
              sinks=c["sinks"], window=c["window"])


def _decode_case(seed):
    rng = random.Random(seed)
    mla = rng.random() < 0.3
    if mla:
        Hkv, Hq, D, Dv = 1, rng.choice([16, 40, 64, 100, 128]), 576, 512
    else:
        Hkv = rng.choice([1, 2, 4])
        Hq = Hkv * rng.choice([1, 3, 4, 8, 16])
        D = Dv = rng.choice([64, 128])
    B = rng.choice([1, 2, 3])
    L = rng.randrange(1, 3000)
    kv_len = [L] + [rng.randrange(0, L + 1) for _ in range(B - 1)]
    rng.shuffle(kv_len)
    window = rng.choice([0, 0, rng.randrange(1, 500)])
    splits = rng.choice([0, 1, 2, 5])
    page = rng.choice([0, 0, 1, 16, 64])
    beta = rng.choice([1.0, 8.0, 16.0])
    lam = rng.choice([0.0, 16.0 / L, 0.05, 1.0])
    return dict(B=B, Hq=Hq, Hkv=Hkv, L=L, D=D, Dv=Dv, kv_len=kv_len, window=window, splits=splits,
                page=page, beta=beta, lam=lam, share=rng.random() < 0.5,
                heads_major=rng.random() < 0.5)


@pytest.mark.parametrize("seed", range(100))
def test_random_decode(seed):
    need_gpu()
    c = _decode_case(9100 + seed)
    what = f"random decode seed={9100 + seed} {c}"
    print(what, flush=True)
    mla = c["Dv"] != c["D"]
    q, k, v, kvl = decode_inputs(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], L=c["L"], d_qk=c["D"],
                                 d_v=c["Dv"], cluster_len=64, dtype=torch.bfloat16, seed=9100 + seed,
                                 beta=c["beta"], share=c["share"], v_aliases_k=mla,
                                 kv_len=c["kv_len"])
    kd = k.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    vd = kd[..., :c["Dv"]] if mla else v.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    qd, kvd = q.cuda(), kvl.cuda()
    extra = {}
    if c["page"]:
        kd, vd, table = paged_layout(kd, vd, c["page"], seed=seed, kv_len=kvd,
                                     heads_major=c["heads_major"])
        extra = dict(block_table=table, max_kv_len=c["L"])
    res = dec._run_gpu(qd, kd, vd, kvd, lam=c["lam"], num_splits=c["splits"],
                       window=c["window"], **extra)
    ref = oracle.decode(q, k, v, kv_len=kvl, block_r=res["br"], block_c=res["bc"],
                        num_splits=res["splits"], scale=oracle_scale(c["D"]), lam=c["lam"],
                        threads=8, window=c["window"])
    band_mism = dec._check(res, ref, q, k, v, c["lam"], what, kvl, c["window"])
    assert res["counters"][0] == ref.visited
    assert abs(res["counters"][1] - ref.skipped) <= band_mism
    assert not math.isnan(float(res["o"].float().abs().max()))
