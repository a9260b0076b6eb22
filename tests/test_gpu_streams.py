"""Stream and graph behaviour of the C ABI: every kernel of a call (prefill; decode with its split
merge; MLA-shaped decode) is launched on the stream the caller passes, and a HIP graph that
captured the calls replays to the eager results.

Side stream: the call's query is written on that stream behind a spin kernel, so a kernel
launched anywhere else would read the query before it is written. Graph: each replay follows
eager work of the program's own and a synchronisation, with the outputs cleared eagerly, and is
compared bitwise with the eager call (same kernels, same inputs)."""
import pytest
import torch

import flashattention_softmax_threshold_amd as F
from flashattention_softmax_threshold_amd.inputs import decode_inputs, prefill_inputs

from parity import need_gpu

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 20_000_000  # a bounded spin ahead of the producer on the side stream


def _prefill_case(name):
    if name == "bf16_causal_gqa":
        B, L, Hq, Hkv, D, dtype, causal = 1, 1000, 8, 2, 128, torch.bfloat16, True
    elif name == "bf16_noncausal_query_pairs":
        B, L, Hq, Hkv, D, dtype, causal = 1, 513, 3, 1, 128, torch.bfloat16, False
    else:  # fp32
        B, L, Hq, Hkv, D, dtype, causal = 2, 300, 2, 2, 64, torch.float32, True
    q, k, v = prefill_inputs(B=B, L=L, Hq=Hq, Hkv=Hkv, d=D, cluster_len=64, dtype=dtype,
                             device="cuda", seed=8100 + L, beta=8.0, sinks=8)
    lam = 16.0 / L
    outs = dict(o=torch.empty_like(q),
                lse=torch.empty((B, Hq, L), dtype=torch.float32, device="cuda"),
                cnt=torch.zeros(2, dtype=torch.int64, device="cuda"))

    def call(qq):
        F.blasst_attn_prefill(qq, k, v, causal=causal, lam=lam, o=outs["o"], lse=outs["lse"],
                              counters=outs["cnt"])
    return q, outs, call


def _decode_case(name):
    if name == "gqa_split":
        B, Hq, Hkv, L, D, Dv, splits, kvl = 3, 32, 8, 3000, 128, 128, 4, [3000, 1700, 0]
    else:  # mla_split
        B, Hq, Hkv, L, D, Dv, splits, kvl = 2, 128, 1, 1500, 576, 512, 3, [1500, 777]
    mla = Dv != D
    q, k, v, kv_len = decode_inputs(B=B, Hq=Hq, Hkv=Hkv, L=L, d_qk=D, d_v=Dv, cluster_len=64,
                                    dtype=torch.bfloat16, seed=8200 + L, beta=16.0, share=True,
                                    v_aliases_k=mla, kv_len=kvl)
    kd = k.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    vd = kd[..., :Dv] if mla else v.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    qd, kvd = q.cuda(), kv_len.cuda()
    ws = torch.empty(max(F.blasst_decode_workspace_size(qd, kd, vd, num_splits=splits), 1),
                     dtype=torch.uint8, device="cuda")
    lam = 16.0 / L
    outs = dict(o=torch.empty((B, Hq, Dv), dtype=torch.bfloat16, device="cuda"),
                lse=torch.empty((B, Hq), dtype=torch.float32, device="cuda"),
                cnt=torch.zeros(2, dtype=torch.int64, device="cuda"))

    def call(qq):
        F.blasst_attn_decode(qq, kd, vd, kv_len=kvd, lam=lam, o=outs["o"], lse=outs["lse"],
                             counters=outs["cnt"], num_splits=splits, workspace=ws,
                             max_kv_len=L)
    return qd, outs, call


CASES = [("prefill", "bf16_causal_gqa"), ("prefill", "bf16_noncausal_query_pairs"),
         ("prefill", "fp32"), ("decode", "gqa_split"), ("decode", "mla_split")]


def _make(kind, name):
    return _prefill_case(name) if kind == "prefill" else _decode_case(name)


def _snapshot(outs):
    return {n: t.clone() for n, t in outs.items()}


def _clear(outs):
    outs["o"].fill_(float("nan"))
    outs["lse"].fill_(float("nan"))
    outs["cnt"].zero_()


def _assert_same(outs, ref, what):
    for n in ("o", "lse", "cnt"):
        assert torch.equal(outs[n], ref[n]), f"{what}: {n} differs"


@pytest.mark.parametrize("kind,name", CASES)
def test_side_stream_runs_after_its_producer(kind, name):
    need_gpu()
    print(f"side stream {kind} {name}", flush=True)
    q, outs, call = _make(kind, name)
    call(q)
    torch.cuda.synchronize()
    ref = _snapshot(outs)
    assert ref["cnt"][0].item() > 0
    q_side = torch.zeros_like(q)
    _clear(outs)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(SPIN_CYCLES)
        q_side.copy_(q)
        call(q_side)
    s.synchronize()
    _assert_same(outs, ref, f"{kind} {name} on a side stream")


@pytest.mark.parametrize("kind,name", CASES)
def test_graph_replays_match_eager(kind, name):
    need_gpu()
    print(f"graph {kind} {name}", flush=True)
    q, outs, call = _make(kind, name)
    call(q)
    torch.cuda.synchronize()
    ref = _snapshot(outs)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _clear(outs)
        call(q)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    _assert_same(outs, ref, f"{kind} {name} warm-up")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(q)
    a = torch.randn(256, 256, device="cuda")
    for rep in range(3):
        _clear(outs)
        a = torch.tanh(a @ a.t() / 256.0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _assert_same(outs, ref, f"{kind} {name} replay {rep}")
