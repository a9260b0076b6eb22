"""Host-side checks of the C ABI (no GPU needed): the library loads and exports every entry point
the public header declares, the threshold resolution and the timestep gate match the values the
Skip-Softmax page prints, launch planning resolves its defaults, and bad arguments are refused
before anything is launched."""
import ctypes
import json
import math
import os
import re

import pytest
import torch

import flashattention_softmax_threshold_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "blasst.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(blasst_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert set(declared) == set(F.EXPORTED)
    lib = ctypes.CDLL(F.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(7):
        assert F.blasst_status_string(code).startswith("BLASST_")


def test_resolve_lambda_modes():
    # Threshold: lambda itself, independent of the length.
    assert F.blasst_resolve_lambda(F.BLASST_THRESHOLD, 4096, threshold=1e-3) == 1e-3
    assert F.blasst_resolve_lambda(F.BLASST_THRESHOLD, 75600, threshold=1e-3) == 1e-3
    assert F.blasst_resolve_lambda(F.BLASST_THRESHOLD, 10, threshold=0.0) == 0.0
    # Scale factor: divided by the call's max_kv_len (lambda = a / L).
    assert F.blasst_resolve_lambda(F.BLASST_SCALE_FACTOR, 8192, scale_factor=16.0) == 16.0 / 8192
    assert F.blasst_resolve_lambda(F.BLASST_DENSE, 8192) == 0.0


def test_resolve_lambda_target_sparsity_wan_calibration():
    fx = json.load(open(os.path.join(GOLDEN, "wan22_calibration.json")))
    a, b = fx["a"], fx["b"]
    for s, L in ((fx["target_sparsity"], 75600), (0.5, 75600), (0.0, 1024), (1.0, 65536)):
        lam = F.blasst_resolve_lambda(F.BLASST_TARGET_SPARSITY, L, target_sparsity=s, a=a, b=b)
        assert lam == pytest.approx(a * math.exp(b * s) / L, rel=1e-15)
    # The two operating points of the video-DiT workload.
    assert F.blasst_resolve_lambda(F.BLASST_TARGET_SPARSITY, 75600, target_sparsity=0.5, a=a,
                                   b=b) == pytest.approx(0.334986486358622, rel=1e-13)
    assert F.blasst_resolve_lambda(F.BLASST_TARGET_SPARSITY, 75600, target_sparsity=0.7, a=a,
                                   b=b) == pytest.approx(0.805723246153606, rel=1e-13)


@pytest.mark.parametrize("kw,code", [
    (dict(mode=F.BLASST_THRESHOLD, threshold=-1e-3), F.BLASST_ERR_INVALID_ARG),
    (dict(mode=F.BLASST_THRESHOLD, threshold=float("nan")), F.BLASST_ERR_INVALID_ARG),
    (dict(mode=F.BLASST_THRESHOLD, threshold=float("inf")), F.BLASST_ERR_INVALID_ARG),
    (dict(mode=F.BLASST_SCALE_FACTOR, scale_factor=4.0, L=0), F.BLASST_ERR_INVALID_ARG),
    (dict(mode=F.BLASST_SCALE_FACTOR, scale_factor=-4.0), F.BLASST_ERR_INVALID_ARG),
    (dict(mode=F.BLASST_TARGET_SPARSITY, target_sparsity=0.5), F.BLASST_ERR_NO_CALIBRATION),
    (dict(mode=F.BLASST_TARGET_SPARSITY, target_sparsity=1.5, a=1.0, b=1.0), F.BLASST_ERR_INVALID_ARG),
    (dict(mode=F.BLASST_TARGET_SPARSITY, target_sparsity=0.5, threshold=0.1, a=1.0, b=1.0),
     F.BLASST_ERR_CONFLICT),
    (dict(mode=7), F.BLASST_ERR_INVALID_ARG),
])
def test_resolve_lambda_errors(kw, code):
    kw = dict(kw)
    mode = kw.pop("mode")
    L = kw.pop("L", 1000)
    with pytest.raises(F.BlasstError) as e:
        F.blasst_resolve_lambda(mode, L, **kw)
    assert e.value.status == code


def _minimax_schedule(shift, n):
    us = [1.0 - i / n for i in range(n + 1)]
    return [shift * u / (1 + (shift - 1) * u) for u in us][:n]


def test_timestep_gate_reproduces_minimax_table():
    fx = json.load(open(os.path.join(GOLDEN, "minimax_timestep_table.json")))
    ts = _minimax_schedule(fx["shift"], fx["num_inference_steps"])
    assert [round(t, 3) for t in ts[:5]] == fx["first_values"]
    assert sum(t > 0.9 for t in ts) == fx["steps_above_0_9"]
    for row in fx["rows"]:
        active = [F.blasst_timestep_gate(row["disabled_until_timestep"], t) for t in ts]
        assert active.count(False) == row["dense_steps"], row
        assert active.count(True) == row["skip_softmax_steps"], row
        # Once active, stays active (t only decreases).
        first = active.index(True) if True in active else len(active)
        assert all(active[first:])


def test_timestep_gate_sentinel_and_unpublished_t():
    assert F.blasst_timestep_gate(0.0, None) is True      # gate off: t is never read
    assert F.blasst_timestep_gate(0.0, 0.999) is True
    assert F.blasst_timestep_gate(1.0, None) is False     # positive cutoff, no t: dense
    assert F.blasst_timestep_gate(1.0, 1.0) is True       # cutoff 1.0 with t: no dense step
    with pytest.raises(F.BlasstError):
        F.blasst_timestep_gate(-0.5, 0.3)
    with pytest.raises(F.BlasstError):
        F.blasst_timestep_gate(0.5, float("nan"))


def _meta(shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device="meta")


def test_prefill_tile_defaults_and_unsupported():
    q, k = _meta((1, 100, 8, 128)), _meta((1, 100, 2, 128))
    assert F.blasst_prefill_tiles(q, k) == (128, 64)
    assert F.blasst_prefill_tiles(q, k, block_r=64) == (64, 64)
    q32, k32 = _meta((1, 100, 2, 64), torch.float32), _meta((1, 100, 2, 64), torch.float32)
    assert F.blasst_prefill_tiles(q32, k32) == (64, 64)
    for br, bc in ((96, 64), (128, 128)):
        with pytest.raises(F.BlasstError) as e:
            F.blasst_prefill_tiles(q, k, block_r=br, block_c=bc)
        assert e.value.status == F.BLASST_ERR_UNSUPPORTED


def test_decode_plan_defaults():
    q, k = _meta((64, 32, 128)), _meta((64, 32768, 8, 128))
    assert F.blasst_decode_plan(q, k, k) == (4, 64, 1)  # 512 units: no split needed
    assert F.blasst_decode_workspace_size(q, k, k) == 0
    q1, k1 = _meta((2, 32, 128)), _meta((2, 32768, 8, 128))
    br, bc, s = F.blasst_decode_plan(q1, k1, k1)
    assert (br, bc) == (4, 64) and s > 1
    assert F.blasst_decode_workspace_size(q1, k1, k1) >= 2 * 32 * s * 129 * 4
    # MQA: 32 query heads on one KV head -> blocks of 16 rows.
    qm, km = _meta((4, 32, 128)), _meta((4, 1000, 1, 128))
    assert F.blasst_decode_plan(qm, km, km)[0] == 16
    with pytest.raises(F.BlasstError) as e:
        F.blasst_decode_plan(_meta((4, 32, 96)), _meta((4, 1000, 1, 96)), _meta((4, 1000, 1, 96)))
    assert e.value.status == F.BLASST_ERR_UNSUPPORTED


def _prefill_struct(**over):
    a = F._PrefillArgs()
    a.dtype = F.BLASST_BF16
    a.batch, a.heads_q, a.heads_kv, a.len_q, a.len_kv, a.head_dim = 1, 4, 2, 100, 100, 128
    a.q = a.k = a.v = a.o = 1 << 20
    for name in ("q_stride", "k_stride", "v_stride", "o_stride"):
        getattr(a, name)[:] = [100 * 4 * 128, 4 * 128, 128]
    a.lam = 0.01
    for key, val in over.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("over,code", [
    (dict(heads_kv=3), F.BLASST_ERR_INVALID_ARG),
    (dict(causal=1, len_kv=50), F.BLASST_ERR_INVALID_ARG),
    (dict(lam=-0.1), F.BLASST_ERR_INVALID_ARG),
    (dict(lam=float("nan")), F.BLASST_ERR_INVALID_ARG),
    (dict(softmax_scale=float("inf")), F.BLASST_ERR_INVALID_ARG),
    (dict(head_dim=96), F.BLASST_ERR_UNSUPPORTED),
    (dict(q=0), F.BLASST_ERR_INVALID_ARG),
    (dict(o=(1 << 20) + 8), F.BLASST_ERR_INVALID_ARG),
    (dict(len_kv=0), F.BLASST_ERR_INVALID_ARG),
    (dict(dtype=5), F.BLASST_ERR_UNSUPPORTED),
    (dict(causal=1, window=-1), F.BLASST_ERR_INVALID_ARG),
    (dict(causal=0, window=16), F.BLASST_ERR_UNSUPPORTED),  # windows are causal only
])
def test_prefill_rejects_bad_arguments_before_launch(over, code):
    a = _prefill_struct(**over)
    assert F.load_library().blasst_attn_prefill(ctypes.byref(a), None) == code


def test_prefill_rejects_misaligned_stride():
    a = _prefill_struct()
    a.k_stride[1] = 4 * 128 + 3
    assert F.load_library().blasst_attn_prefill(ctypes.byref(a), None) == F.BLASST_ERR_INVALID_ARG


def test_prefill_empty_inputs_are_a_no_op():
    for over in (dict(batch=0), dict(len_q=0, len_kv=0, causal=0)):
        a = _prefill_struct(**over)
        if "len_kv" in over:
            a.len_kv = 0
            a.len_q = 0
        assert F.load_library().blasst_attn_prefill(ctypes.byref(a), None) == F.BLASST_OK


def test_decode_rejects_bad_arguments_before_launch():
    lib = F.load_library()
    a = F._DecodeArgs()
    a.dtype = F.BLASST_BF16
    a.batch, a.heads_q, a.heads_kv, a.max_kv_len, a.head_dim_qk, a.head_dim_v = 2, 8, 2, 300, 128, 128
    a.q = a.k = a.v = a.o = 1 << 20
    a.q_stride[:] = [8 * 128, 128]
    a.k_stride[:] = [300 * 2 * 128, 2 * 128, 128]
    a.v_stride[:] = [300 * 2 * 128, 2 * 128, 128]
    a.o_stride[:] = [8 * 128, 128]
    a.lam = -1.0
    assert lib.blasst_attn_decode(ctypes.byref(a), None, 0, None) == F.BLASST_ERR_INVALID_ARG
    a.lam = 0.01
    a.num_splits = 3
    assert lib.blasst_attn_decode(ctypes.byref(a), None, 0, None) == F.BLASST_ERR_WORKSPACE
    a.num_splits = -1
    assert lib.blasst_attn_decode(ctypes.byref(a), None, 0, None) == F.BLASST_ERR_INVALID_ARG
    a.num_splits = 1
    a.heads_kv = 3
    assert lib.blasst_attn_decode(ctypes.byref(a), None, 0, None) == F.BLASST_ERR_INVALID_ARG
    a.heads_kv = 2
    # Paged cache: the page size must be a power of two in [1, 4096] and the pages must cover
    # max_kv_len (every case below is refused before anything is launched).
    a.block_table = 1 << 21
    for page_size, pages in ((48, 8), (0, 8), (8192, 1), (64, 4), (64, 0)):
        a.page_size, a.pages_per_seq = page_size, pages
        assert lib.blasst_attn_decode(ctypes.byref(a), None, 0, None) == F.BLASST_ERR_INVALID_ARG, \
            (page_size, pages)
    a.block_table, a.page_size, a.pages_per_seq = None, 0, 0
    a.window = -5
    assert lib.blasst_attn_decode(ctypes.byref(a), None, 0, None) == F.BLASST_ERR_INVALID_ARG


def test_decode_plan_with_window_splits_the_window_span():
    # MLA shape with the 64-head kernel, 32 sequences x 2 row blocks = 64 units: without a window
    # the 1024 tiles of 64K keys get 8 splits of 128 tiles; a 4096-key window touches at most 65
    # tiles, cut 8 ways (ceil(65 / 8) = 9 tiles per split), and a short window with few tiles is
    # not split.
    q, k = _meta((32, 128, 576)), _meta((32, 65536, 1, 576))
    v = k[..., :512]
    assert F.blasst_decode_plan(q, k, v, block_r=64) == (64, 64, 8)
    assert F.blasst_decode_plan(q, k, v, block_r=64, window=4096) == (64, 64, 8)
    assert F.blasst_decode_plan(q, k, v, block_r=64, window=300) == (64, 64, 1)
    assert F.blasst_decode_workspace_size(q, k, v, block_r=64, window=300) == 0
    # The default for 128 heads: one unit of 128 heads per sequence and split (32 units), split
    # until the 256 CUs each hold one workgroup (8 splits), the same window rules.
    assert F.blasst_decode_plan(q, k, v) == (128, 64, 8)
    assert F.blasst_decode_plan(q, k, v, window=4096) == (128, 64, 8)
    assert F.blasst_decode_plan(q, k, v, window=300) == (128, 64, 1)


def test_mla_plan_row_blocks():
    # 64 or fewer heads: the 64-head kernel; more: up to 128 per unit; other sizes unsupported.
    v_of = lambda k: k[..., :512]  # noqa: E731
    for hq, want in ((16, 16), (64, 64), (96, 96), (128, 128), (256, 128)):
        q, k = _meta((2, hq, 576)), _meta((2, 4096, 1, 576))
        assert F.blasst_decode_plan(q, k, v_of(k))[0] == want, hq
    q, k = _meta((2, 128, 576)), _meta((2, 4096, 1, 576))
    assert F.blasst_decode_plan(q, k, v_of(k), block_r=64)[0] == 64
    with pytest.raises(F.BlasstError) as e:
        F.blasst_decode_plan(q, k, v_of(k), block_r=32)
    assert e.value.status == F.BLASST_ERR_UNSUPPORTED


# ------------------------------------------------------------------------------------------
# Calibration entry points (host only) against the oracle's restatement
# ------------------------------------------------------------------------------------------
def test_sparsity_curve_matches_oracle():
    import numpy as np

    import oracle

    rng = np.random.default_rng(5)
    n = 5000
    margins = -np.abs(rng.standard_normal(n) * 4).astype(np.float32)
    margins[:50] = 0.0                               # tiles that set a new maximum
    margins[50:60] = np.float32(math.log(0.25))      # exactly at a candidate's ln(lambda)
    margins[60:70] = -np.inf                         # no row saw a key
    status = rng.integers(0, 3, n).astype(np.uint8)  # 2 = not visited
    lams = [0.0, 1e-3, 0.01, 0.25, 0.5, 1.0, 2.0]
    got, vis = F.blasst_sparsity_curve(margins, status, lams)
    # The oracle compares in float64 against ln(lambda) exactly like the library does.
    want, vis_o = oracle.sparsity_curve(margins, status, lams)
    assert vis == vis_o == int((status != 2).sum())
    assert got == want
    assert got[0] == 0.0 and got[-1] == got[-2]      # lambda = 0 skips nothing; lambda > 1 clamps


def test_fit_calibration_matches_oracle_and_refuses_bad_input():
    import numpy as np

    import oracle

    rng = np.random.default_rng(9)
    L = rng.choice([4096, 8192, 32768], 40).astype(float)
    S = rng.uniform(0.2, 0.9, 40)
    lam = 300 * np.exp(5 * S) / L * np.exp(rng.normal(0, 0.1, 40))
    a, b = F.blasst_fit_calibration(L, lam, S)
    ao, bo = oracle.fit_calibration(L, lam, S)
    assert a == pytest.approx(ao, rel=1e-10) and b == pytest.approx(bo, rel=1e-10)
    with pytest.raises(F.BlasstError):
        F.blasst_fit_calibration([1000], [1e-3], [0.5])                   # one point
    with pytest.raises(F.BlasstError):
        F.blasst_fit_calibration([1000, 2000], [1e-3, 1e-3], [0.5, 0.5])  # S all equal
    with pytest.raises(F.BlasstError):
        F.blasst_fit_calibration([1000, 2000], [0.0, 1e-3], [0.4, 0.5])   # lambda 0
    with pytest.raises(F.BlasstError):
        F.blasst_sparsity_curve([0.0], [7], [0.5])                          # unknown status
    with pytest.raises(F.BlasstError):
        F.blasst_sparsity_curve([0.0], [0], [-1.0])                         # negative lambda


def test_generator_sinks_on_a_sequence_shorter_than_the_sink_count():
    """The seeded clustered generator with more sink keys than keys: every key is a sink
    (3 x the mean centre, no noise), and longer sequences keep exactly `sinks` of them."""
    import torch
    from flashattention_softmax_threshold_amd.inputs import prefill_inputs

    q, k, v = prefill_inputs(B=2, L=5, Hq=4, Hkv=2, d=16, cluster_len=16, dtype=torch.float32,
                             seed=11, beta=4.0, sinks=8)
    assert q.shape == (2, 5, 4, 16) and k.shape == (2, 5, 2, 16) and v.shape == (2, 5, 2, 16)
    assert torch.equal(k, k[:, :1].expand_as(k))
    q, k, v = prefill_inputs(B=1, L=40, Hq=2, Hkv=1, d=16, cluster_len=16, dtype=torch.float32,
                             seed=11, beta=4.0, sinks=8)
    assert torch.equal(k[:, :8], k[:, :1].expand(1, 8, 1, 16))
    assert not torch.equal(k[:, 8], k[:, 0])


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU; a request for more exits with a message before any GPU
    work."""
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_unloadable_library_raises_instead_of_falling_back(tmp_path):
    """The binding has no other path: a library file that does not load is an error."""
    bogus = tmp_path / "libblasst.so"
    bogus.write_text("not a shared library")
    saved_path, saved_lib = F.LIB_PATH, F._lib
    try:
        F.LIB_PATH, F._lib = str(bogus), None
        with pytest.raises(OSError):
            F.load_library()
        q = torch.zeros((1, 4, 1, 64), dtype=torch.bfloat16)
        with pytest.raises((OSError, TypeError, ValueError)):
            F.blasst_attn_prefill(q, q, q)
    finally:
        F.LIB_PATH, F._lib = saved_path, saved_lib


def _expect(exc, match, fn, *args, **kw):
    with pytest.raises(exc, match=match):
        fn(*args, **kw)


def test_prefill_binding_checks_every_tensor_before_the_call():
    """Every buffer the prefill kernels address through a raw pointer is checked for shape,
    dtype, device and layout in the binding, before the library is called (meta tensors: no
    memory, no GPU). A call whose tensors all pass reaches the last check, the GPU device."""
    B, L, Hq, Hkv, D = 2, 300, 8, 2, 128
    q, k, v = _meta((B, L, Hq, D)), _meta((B, L, Hkv, D)), _meta((B, L, Hkv, D))
    nqb, nkt = -(-L // 128), -(-L // 64)
    ok = dict(o=_meta((B, L, Hq, D)), lse=_meta((B, Hq, L), torch.float32),
              counters=_meta((2,), torch.int64),
              tile_status=_meta((B, Hq, nqb, nkt), torch.uint8),
              tile_margin=_meta((B, Hq, nqb, nkt), torch.float32))
    _expect(ValueError, "GPU device", F.blasst_attn_prefill, q, k, v, causal=True, **ok)
    bad = [
        (ValueError, "same shape", (q, k, _meta((B, L, Hkv, 64))), {}),
        (ValueError, "batch or head dim", (q, _meta((1, L, Hkv, D)), _meta((1, L, Hkv, D))), {}),
        (TypeError, "share a dtype", (q, k, _meta((B, L, Hkv, D), torch.float32)), {}),
        (ValueError, "o must have shape", (q, k, v), dict(o=_meta((B, L, Hq, 64)))),
        (TypeError, "o must be", (q, k, v), dict(o=_meta((B, L, Hq, D), torch.float32))),
        (ValueError, "lse must have shape", (q, k, v), dict(lse=_meta((B, L, Hq), torch.float32))),
        (TypeError, "lse must be", (q, k, v), dict(lse=_meta((B, Hq, L)))),
        (ValueError, "lse must be contiguous", (q, k, v),
         dict(lse=_meta((B, L, Hq), torch.float32).transpose(1, 2))),
        (TypeError, "counters must be", (q, k, v), dict(counters=_meta((2,), torch.int32))),
        (ValueError, "2 elements", (q, k, v), dict(counters=_meta((3,), torch.int64))),
        (ValueError, "tile_status must have shape", (q, k, v),
         dict(tile_status=_meta((B, Hq, nqb, nkt + 1), torch.uint8))),
        (TypeError, "tile_margin must be", (q, k, v),
         dict(tile_margin=_meta((B, Hq, nqb, nkt), torch.float64))),
        (ValueError, "is on", (q, k, v), dict(counters=torch.zeros(2, dtype=torch.int64))),
    ]
    for exc, match, args, kw in bad:
        _expect(exc, match, F.blasst_attn_prefill, *args, causal=True, **kw)


def test_decode_binding_checks_every_tensor_before_the_call():
    """The same for decode: k / v / q agreement, kv_len, output, LSE, counters, tile arrays,
    block table and workspace."""
    B, Hq, Hkv, L, D = 3, 32, 8, 1000, 128
    q, k, v = _meta((B, Hq, D)), _meta((B, L, Hkv, D)), _meta((B, L, Hkv, D))
    kvl = _meta((B,), torch.int32)
    br, bc, _ = F.blasst_decode_plan(q, k, v)
    st = (B, Hkv, -(-(Hq // Hkv) // br), -(-L // bc))
    ok = dict(kv_len=kvl, o=_meta((B, Hq, D)), lse=_meta((B, Hq), torch.float32),
              counters=_meta((2,), torch.int64), tile_status=_meta(st, torch.uint8),
              tile_margin=_meta(st, torch.float32), workspace=_meta((1 << 20,), torch.uint8))
    _expect(ValueError, "GPU device", F.blasst_attn_decode, q, k, v, **ok)
    bad = [
        (ValueError, "differ in their first three", (q, k, _meta((B, L + 1, Hkv, D))), {}),
        (ValueError, "head dim", (q, _meta((B, L, Hkv, 64)), _meta((B, L, Hkv, 64))), {}),
        (ValueError, "not a multiple", (q, _meta((B, L, 3, D)), _meta((B, L, 3, D))), {}),
        (ValueError, "batch", (q, _meta((B - 1, L, Hkv, D)), _meta((B - 1, L, Hkv, D))), {}),
        (ValueError, "3 elements", (q, k, v), dict(kv_len=_meta((B - 1,), torch.int32))),
        (TypeError, "kv_len must be int32", (q, k, v), dict(kv_len=_meta((B,), torch.int64))),
        (ValueError, "o must have shape", (q, k, v), dict(o=_meta((B, Hq, 64)))),
        (ValueError, "lse must have shape", (q, k, v), dict(lse=_meta((B, Hq + 1), torch.float32))),
        (TypeError, "counters must be", (q, k, v), dict(counters=_meta((2,), torch.float32))),
        (ValueError, "tile_status must have shape", (q, k, v),
         dict(tile_status=_meta((B, Hkv, 1, 15), torch.uint8))),
        (TypeError, "block_table", (q, _meta((64, 16, Hkv, D)), _meta((64, 16, Hkv, D))),
         dict(block_table=_meta((B, 63), torch.int64))),
        (ValueError, "workspace must be contiguous", (q, k, v),
         dict(workspace=_meta((64, 64), torch.uint8).t())),
    ]
    for exc, match, args, kw in bad:
        _expect(exc, match, F.blasst_attn_decode, *args, **kw)


def test_noalloc_decode_refuses_partials_beyond_its_scratch_before_any_device_call():
    """blasst_attn_decode_noalloc checks on the host that the split partials fit its scratch array
    (BLASST_NOALLOC_SCRATCH_BYTES per GPU) and refuses a larger plan before touching the device."""
    a = F._DecodeArgs()
    a.dtype = F.BLASST_BF16
    a.batch, a.heads_q, a.heads_kv, a.max_kv_len = 128, 128, 1, 65536
    a.head_dim_qk, a.head_dim_v = 576, 512
    a.q = a.o = 1 << 20
    a.k = a.v = 1 << 21
    a.q_stride[:] = [128 * 576, 576]
    a.k_stride[:] = [65536 * 576, 576, 576]
    a.v_stride[:] = [65536 * 576, 576, 576]
    a.o_stride[:] = [128 * 512, 512]
    a.num_splits = 8
    lib = F.load_library()
    assert lib.blasst_decode_workspace_size(ctypes.byref(a)) > F.NOALLOC_SCRATCH_BYTES
    assert lib.blasst_attn_decode_noalloc(ctypes.byref(a), None) == F.BLASST_ERR_WORKSPACE
    a.lam = float("nan")
    assert lib.blasst_attn_decode_noalloc(ctypes.byref(a), None) == F.BLASST_ERR_INVALID_ARG
    assert lib.blasst_attn_decode_noalloc(None, None) == F.BLASST_ERR_INVALID_ARG
    text = open(os.path.join(ROOT, "include", "blasst.h")).read()
    m = re.search(r"#define BLASST_NOALLOC_SCRATCH_BYTES \((\d+)u \* (\d+)u \* (\d+)u\)", text)
    assert m and int(m[1]) * int(m[2]) * int(m[3]) == F.NOALLOC_SCRATCH_BYTES
