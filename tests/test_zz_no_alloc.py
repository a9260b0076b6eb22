"""blasst_attn_decode_noalloc (split partials in the library's per-GPU scratch array) against
blasst_attn_decode with a caller workspace: same outputs, LSE and counters, bit for bit, over
calls in a row whose second is smaller (the scratch keeps the first call's partials)."""
import ctypes

import pytest
import torch

import flashattention_softmax_threshold_amd as F
from flashattention_softmax_threshold_amd.inputs import decode_inputs

from parity import need_gpu

pytestmark = pytest.mark.gpu


def _call_both(q, k, v, kvl, lam, splits):
    """The same decode through both entry points, on the raw C ABI for the no-allocation one."""
    B, Hq = q.shape[0], q.shape[1]
    dv = v.shape[3]
    outs = []
    for noalloc in (False, True):
        o = torch.full((B, Hq, dv), float("nan"), dtype=q.dtype, device="cuda")
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        if noalloc:
            a = F._decode_args(q, k, v, o, kv_len=kvl, lam=lam, softmax_scale=0.0, lse=lse,
                               counters=cnt, tile_status=None, tile_margin=None, block_r=0,
                               block_c=0, num_splits=splits)
            st = F.load_library().blasst_attn_decode_noalloc(
                ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            assert st == F.BLASST_OK, F.blasst_status_string(st)
        else:
            need = F.blasst_decode_workspace_size(q, k, v, num_splits=splits)
            ws = torch.full((max(need, 4) // 4,), float("nan"), dtype=torch.float32,
                            device="cuda")  # partials must all be written: start from NaN
            F.blasst_attn_decode(q, k, v, kv_len=kvl, lam=lam, o=o, lse=lse, counters=cnt,
                                 num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        outs.append((o, lse, cnt))
    return outs


@pytest.mark.parametrize("shape", ["gqa", "mla"])
def test_noalloc_decode_equals_workspace_decode_on_two_calls(shape):
    need_gpu()
    if shape == "gqa":
        cases = [dict(B=3, Hq=8, Hkv=2, L=5000, d_qk=128, d_v=128, kv=[5000, 3333, 64], S=5),
                 dict(B=1, Hq=8, Hkv=2, L=700, d_qk=128, d_v=128, kv=[700], S=3)]
    else:
        cases = [dict(B=2, Hq=128, Hkv=1, L=3000, d_qk=576, d_v=512, kv=[3000, 1777], S=4),
                 dict(B=1, Hq=128, Hkv=1, L=1000, d_qk=576, d_v=512, kv=[1000], S=2)]
    for i, c in enumerate(cases):
        print(f"noalloc {shape} call {i}: {c}", flush=True)
        q, k, v, kvl = decode_inputs(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], L=c["L"],
                                     d_qk=c["d_qk"], d_v=c["d_v"], cluster_len=100,
                                     dtype=torch.bfloat16, device="cuda", seed=7100 + i,
                                     beta=16.0, kv_len=c["kv"], share=shape == "mla",
                                     v_aliases_k=shape == "mla")
        assert F.blasst_decode_plan(q, k, v, num_splits=c["S"])[2] == c["S"] > 1
        assert 0 < F.blasst_decode_workspace_size(q, k, v, num_splits=c["S"]) \
            <= F.NOALLOC_SCRATCH_BYTES
        for lam in (0.0, 16.0 / c["L"]):
            (o1, l1, c1), (o2, l2, c2) = _call_both(q, k, v, kvl, lam, c["S"])
            assert torch.isfinite(o1.float()).all()
            assert torch.equal(o1, o2), f"{shape} call {i} lam {lam}: O differs"
            assert torch.equal(l1, l2), f"{shape} call {i} lam {lam}: LSE differs"
            assert torch.equal(c1, c2), f"{shape} call {i} lam {lam}: counters differ"


def test_noalloc_binding_unsplit_call():
    """A call that needs no partials (one split) takes no scratch and equals the usual call."""
    need_gpu()
    q, k, v, kvl = decode_inputs(B=2, Hq=8, Hkv=2, L=600, d_qk=128, d_v=128, cluster_len=100,
                                 dtype=torch.bfloat16, device="cuda", seed=7200, beta=16.0,
                                 kv_len=[600, 333])
    o1 = F.blasst_attn_decode(q, k, v, kv_len=kvl, lam=0.01, num_splits=1)
    o2 = torch.empty_like(o1)
    F.blasst_attn_decode_noalloc(q, k, v, o=o2, kv_len=kvl, lam=0.01, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
