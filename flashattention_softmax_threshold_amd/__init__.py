"""BLASST skip-softmax attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libblasst.so`` whose C ABI is declared in ``include/blasst.h``.
Every step of the attention pass runs in the library's HIP kernels; this module only marshals
arguments (PyTorch supplies device memory and the stream). There is no fallback: if the library
cannot be loaded or a call fails, an exception is raised.

Functions keep the C names: ``blasst_resolve_lambda``, ``blasst_timestep_gate``,
``blasst_prefill_tiles``, ``blasst_attn_prefill``, ``blasst_decode_plan``,
``blasst_decode_workspace_size``, ``blasst_attn_decode``, ``blasst_status_string``.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libblasst.so")

# Status codes (blasst_status).
BLASST_OK = 0
BLASST_ERR_INVALID_ARG = 1
BLASST_ERR_UNSUPPORTED = 2
BLASST_ERR_NO_CALIBRATION = 3
BLASST_ERR_CONFLICT = 4
BLASST_ERR_HIP = 5
BLASST_ERR_WORKSPACE = 6

# Threshold modes (blasst_mode).
BLASST_DENSE = 0
BLASST_THRESHOLD = 1
BLASST_SCALE_FACTOR = 2
BLASST_TARGET_SPARSITY = 3

# Data types (blasst_dtype).
BLASST_F32 = 0
BLASST_BF16 = 1

TILE_KEPT = 0
TILE_SKIPPED = 1
TILE_NOT_VISITED = 2

EXPORTED = (
    "blasst_status_string", "blasst_resolve_lambda", "blasst_timestep_gate",
    "blasst_sparsity_curve", "blasst_fit_calibration",
    "blasst_prefill_tiles", "blasst_attn_prefill", "blasst_decode_plan",
    "blasst_decode_workspace_size", "blasst_attn_decode", "blasst_attn_decode_noalloc",
)

# Bytes of the scratch array blasst_attn_decode_noalloc keeps per GPU (BLASST_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024


class BlasstError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {blasst_status_string(status)}")


class _LambdaSpec(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int),
        ("threshold", ctypes.c_double),
        ("scale_factor", ctypes.c_double),
        ("target_sparsity", ctypes.c_double),
        ("has_calibration", ctypes.c_int32),
        ("a", ctypes.c_double),
        ("b", ctypes.c_double),
    ]


class _PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("len_q", ctypes.c_int32), ("len_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("softmax_scale", ctypes.c_float),
        ("lam", ctypes.c_double),
        ("lse", ctypes.c_void_p), ("counters", ctypes.c_void_p),
        ("tile_status", ctypes.c_void_p), ("tile_margin", ctypes.c_void_p),
        ("block_r", ctypes.c_int32), ("block_c", ctypes.c_int32),
        ("window", ctypes.c_int32),
    ]


class _DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32), ("head_dim_qk", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 2), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 2),
        ("kv_len", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("lam", ctypes.c_double),
        ("lse", ctypes.c_void_p), ("counters", ctypes.c_void_p),
        ("tile_status", ctypes.c_void_p), ("tile_margin", ctypes.c_void_p),
        ("block_r", ctypes.c_int32), ("block_c", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
        ("pages_per_seq", ctypes.c_int32),
        ("window", ctypes.c_int32),
    ]


_lock = threading.Lock()
_lib = None


def load_library():
    """Load libblasst.so (building it with hipcc first if it is not there)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            from . import build as _build

            _build.build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I32 = ctypes.c_int32
        lib.blasst_status_string.argtypes = [ctypes.c_int]
        lib.blasst_status_string.restype = ctypes.c_char_p
        lib.blasst_resolve_lambda.argtypes = [ctypes.POINTER(_LambdaSpec), ctypes.c_int64,
                                              ctypes.POINTER(ctypes.c_double)]
        lib.blasst_resolve_lambda.restype = ctypes.c_int
        lib.blasst_timestep_gate.argtypes = [ctypes.c_double, I32, ctypes.c_double,
                                             ctypes.POINTER(I32)]
        lib.blasst_timestep_gate.restype = ctypes.c_int
        D = ctypes.POINTER(ctypes.c_double)
        lib.blasst_sparsity_curve.argtypes = [P, P, ctypes.c_int64, D, I32, D,
                                              ctypes.POINTER(ctypes.c_int64)]
        lib.blasst_sparsity_curve.restype = ctypes.c_int
        lib.blasst_fit_calibration.argtypes = [D, D, D, I32, D, D]
        lib.blasst_fit_calibration.restype = ctypes.c_int
        lib.blasst_prefill_tiles.argtypes = [ctypes.POINTER(_PrefillArgs), ctypes.POINTER(I32),
                                             ctypes.POINTER(I32)]
        lib.blasst_prefill_tiles.restype = ctypes.c_int
        lib.blasst_attn_prefill.argtypes = [ctypes.POINTER(_PrefillArgs), P]
        lib.blasst_attn_prefill.restype = ctypes.c_int
        lib.blasst_decode_plan.argtypes = [ctypes.POINTER(_DecodeArgs), ctypes.POINTER(I32),
                                           ctypes.POINTER(I32), ctypes.POINTER(I32)]
        lib.blasst_decode_plan.restype = ctypes.c_int
        lib.blasst_decode_workspace_size.argtypes = [ctypes.POINTER(_DecodeArgs)]
        lib.blasst_decode_workspace_size.restype = ctypes.c_size_t
        lib.blasst_attn_decode.argtypes = [ctypes.POINTER(_DecodeArgs), P, ctypes.c_size_t, P]
        lib.blasst_attn_decode.restype = ctypes.c_int
        lib.blasst_attn_decode_noalloc.argtypes = [ctypes.POINTER(_DecodeArgs), P]
        lib.blasst_attn_decode_noalloc.restype = ctypes.c_int
        _lib = lib
        return lib


def _check(status: int, where: str):
    if status != BLASST_OK:
        raise BlasstError(status, where)


def blasst_status_string(status: int) -> str:
    return load_library().blasst_status_string(int(status)).decode()


def blasst_resolve_lambda(mode: int, max_kv_len: int, *, threshold: float = 0.0,
                          scale_factor: float = 0.0, target_sparsity: float = 0.0,
                          a: float | None = None, b: float | None = None) -> float:
    """lambda from a user control (see blasst.h). Raises BlasstError on a bad spec."""
    spec = _LambdaSpec(int(mode), float(threshold), float(scale_factor), float(target_sparsity),
                       1 if (a is not None and b is not None) else 0,
                       float(a) if a is not None else 0.0, float(b) if b is not None else 0.0)
    out = ctypes.c_double(0.0)
    _check(load_library().blasst_resolve_lambda(ctypes.byref(spec), int(max_kv_len),
                                                ctypes.byref(out)), "blasst_resolve_lambda")
    return out.value


def blasst_timestep_gate(disabled_until_timestep: float, t: float | None) -> bool:
    """True when skipping is active for a step with published timestep t (None = unpublished)."""
    act = ctypes.c_int32(0)
    _check(load_library().blasst_timestep_gate(float(disabled_until_timestep),
                                               0 if t is None else 1,
                                               float("nan") if t is None else float(t),
                                               ctypes.byref(act)), "blasst_timestep_gate")
    return bool(act.value)


def blasst_sparsity_curve(tile_margin, tile_status, lambdas):
    """Skip fraction at each candidate lambda from one call's tile_margin / tile_status outputs
    (torch tensors or arrays, any device; copied to the host). Returns (sparsity list, visited)."""
    import numpy as np

    def host(x, dt):
        if hasattr(x, "detach"):
            x = x.detach().cpu().numpy()
        return np.ascontiguousarray(np.asarray(x), dtype=dt).ravel()

    m = host(tile_margin, np.float32)
    st = host(tile_status, np.uint8)
    if m.size != st.size:
        raise ValueError("tile_margin and tile_status differ in size")
    lam = host(lambdas, np.float64)
    out = np.zeros(lam.size, dtype=np.float64)
    vis = ctypes.c_int64(0)
    dp = ctypes.POINTER(ctypes.c_double)
    _check(load_library().blasst_sparsity_curve(
        m.ctypes.data_as(ctypes.c_void_p), st.ctypes.data_as(ctypes.c_void_p), int(m.size),
        lam.ctypes.data_as(dp), int(lam.size), out.ctypes.data_as(dp), ctypes.byref(vis)),
        "blasst_sparsity_curve")
    return out.tolist(), int(vis.value)


def blasst_fit_calibration(seq_len, lam, sparsity):
    """(a, b) of lambda * L = a * exp(b * S) fitted to observations (sequences of equal length)."""
    import numpy as np

    L = np.ascontiguousarray(seq_len, dtype=np.float64).ravel()
    la = np.ascontiguousarray(lam, dtype=np.float64).ravel()
    S = np.ascontiguousarray(sparsity, dtype=np.float64).ravel()
    if not (L.size == la.size == S.size):
        raise ValueError("observation arrays differ in size")
    a, b = ctypes.c_double(0.0), ctypes.c_double(0.0)
    dp = ctypes.POINTER(ctypes.c_double)
    _check(load_library().blasst_fit_calibration(
        L.ctypes.data_as(dp), la.ctypes.data_as(dp), S.ctypes.data_as(dp), int(L.size),
        ctypes.byref(a), ctypes.byref(b)), "blasst_fit_calibration")
    return a.value, b.value


# ------------------------------------------------------------------------------------------
# Tensor helpers
# ------------------------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return BLASST_BF16
    if t.dtype == torch.float32:
        return BLASST_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _prefill_args(q, k, v, o, *, causal, lam, softmax_scale, lse, counters, tile_status,
                  tile_margin, block_r, block_c, window=0) -> _PrefillArgs:
    B, Lq, Hq, D = q.shape
    Lkv, Hkv = k.shape[1], k.shape[2]
    a = _PrefillArgs()
    a.dtype = _dtype_code(q)
    a.batch, a.heads_q, a.heads_kv, a.len_q, a.len_kv, a.head_dim = B, Hq, Hkv, Lq, Lkv, D
    a.causal = 1 if causal else 0
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.o = o.data_ptr() if o is not None else 0
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", o)):
        st = t.stride() if t is not None else (0, 0, 0, 1)
        getattr(a, name)[:] = [st[0], st[1], st[2]]
    a.softmax_scale = float(softmax_scale)
    a.lam = float(lam)
    a.lse = lse.data_ptr() if lse is not None else 0
    a.counters = counters.data_ptr() if counters is not None else 0
    a.tile_status = tile_status.data_ptr() if tile_status is not None else 0
    a.tile_margin = tile_margin.data_ptr() if tile_margin is not None else 0
    a.block_r, a.block_c = int(block_r), int(block_c)
    a.window = int(window)
    return a


def blasst_prefill_tiles(q, k, *, block_r: int = 0, block_c: int = 0):
    """(block_r, block_c) a prefill call on these tensors uses."""
    a = _prefill_args(q, k, k, None, causal=False, lam=0.0, softmax_scale=0.0, lse=None,
                      counters=None, tile_status=None, tile_margin=None, block_r=block_r,
                      block_c=block_c)
    br, bc = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load_library().blasst_prefill_tiles(ctypes.byref(a), ctypes.byref(br), ctypes.byref(bc)),
           "blasst_prefill_tiles")
    return br.value, bc.value


def _check_tensor(t, name, ndim, device):
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.numel() and t.stride(-1) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")


def _check_out(t, name, shape, dtype, device, contiguous):
    """An optional output buffer the kernels write through a raw pointer: exact shape, dtype and
    device, and (when the kernels index it densely) contiguous."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not contiguous and t.numel() and t.stride(-1) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")


def _check_counters(counters, device):
    """Two uint64 the kernels add to atomically (int64 storage is accepted: same bytes)."""
    import torch

    if counters is None:
        return
    if counters.dtype not in (torch.int64, getattr(torch, "uint64", torch.int64)):
        raise TypeError(f"counters must be int64 or uint64, got {counters.dtype}")
    if counters.numel() != 2 or not counters.is_contiguous():
        raise ValueError(f"counters must be a contiguous tensor of 2 elements, got "
                         f"{tuple(counters.shape)}")
    if counters.device != device:
        raise ValueError(f"counters is on {counters.device}, expected {device}")


def _check_on_gpu(device):
    if device.type != "cuda":
        raise ValueError(f"tensors are on {device}; the library runs on a GPU device only")


def blasst_attn_prefill(q, k, v, *, causal: bool = False, lam: float = 0.0,
                        softmax_scale: float = 0.0, o=None, lse=None, counters=None,
                        tile_status=None, tile_margin=None, block_r: int = 0, block_c: int = 0,
                        window: int = 0, stream=None):
    """BLASST prefill on q [B, Lq, Hq, D], k/v [B, Lkv, Hkv, D]; returns o [B, Lq, Hq, D].

    lse: optional fp32 [B, Hq, Lq]; counters: optional uint64 (int64) [2] accumulated (visited,
    skipped); tile_status (uint8) / tile_margin (fp32): optional [B, Hq, n_qblocks, n_kvtiles].
    window: causal sliding window in keys (0 = none).
    """
    import torch

    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(t, name, 4, dev)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    _dtype_code(q)
    B, Lq, Hq, D = q.shape
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} must have the same shape")
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)} in batch or head dim")
    _check_out(o, "o", q.shape, q.dtype, dev, contiguous=False)
    _check_out(lse, "lse", (B, Hq, Lq), torch.float32, dev, contiguous=True)
    _check_counters(counters, dev)
    if tile_status is not None or tile_margin is not None:
        br, bc = blasst_prefill_tiles(q, k, block_r=block_r, block_c=block_c)
        shape = (B, Hq, -(-Lq // br), -(-k.shape[1] // bc))
        _check_out(tile_status, "tile_status", shape, torch.uint8, dev, contiguous=True)
        _check_out(tile_margin, "tile_margin", shape, torch.float32, dev, contiguous=True)
    _check_on_gpu(dev)
    if o is None:
        o = torch.empty(q.shape, dtype=q.dtype, device=dev)
    a = _prefill_args(q, k, v, o, causal=causal, lam=lam, softmax_scale=softmax_scale, lse=lse,
                      counters=counters, tile_status=tile_status, tile_margin=tile_margin,
                      block_r=block_r, block_c=block_c, window=window)
    _check(load_library().blasst_attn_prefill(ctypes.byref(a), _stream_handle(stream)),
           "blasst_attn_prefill")
    return o


def _decode_args(q, k, v, o, *, kv_len, lam, softmax_scale, lse, counters, tile_status,
                 tile_margin, block_r, block_c, num_splits, block_table=None,
                 max_kv_len=None, window=0) -> _DecodeArgs:
    B, Hq, Dqk = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    if block_table is not None:  # k, v are page pools [pages, page_size, Hkv, d]
        L = block_table.shape[1] * k.shape[1]
    if max_kv_len is not None:
        L = int(max_kv_len)
    Dv = v.shape[3]
    a = _DecodeArgs()
    a.dtype = _dtype_code(q)
    a.batch, a.heads_q, a.heads_kv, a.max_kv_len = B, Hq, Hkv, L
    a.head_dim_qk, a.head_dim_v = Dqk, Dv
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.o = o.data_ptr() if o is not None else 0
    a.q_stride[:] = [q.stride(0), q.stride(1)]
    a.k_stride[:] = [k.stride(0), k.stride(1), k.stride(2)]
    a.v_stride[:] = [v.stride(0), v.stride(1), v.stride(2)]
    a.o_stride[:] = [o.stride(0), o.stride(1)] if o is not None else [0, 0]
    a.kv_len = kv_len.data_ptr() if kv_len is not None else 0
    a.softmax_scale = float(softmax_scale)
    a.lam = float(lam)
    a.lse = lse.data_ptr() if lse is not None else 0
    a.counters = counters.data_ptr() if counters is not None else 0
    a.tile_status = tile_status.data_ptr() if tile_status is not None else 0
    a.tile_margin = tile_margin.data_ptr() if tile_margin is not None else 0
    a.block_r, a.block_c, a.num_splits = int(block_r), int(block_c), int(num_splits)
    if block_table is not None:
        a.block_table = block_table.data_ptr()
        a.page_size = int(k.shape[1])
        a.pages_per_seq = int(block_table.shape[1])
    a.window = int(window)
    return a


def _decode_max_len(k, block_table, max_kv_len):
    """max_kv_len of a decode call: the given value, else the cache length (contiguous: k's
    row count; paged: pages_per_seq * page_size)."""
    if max_kv_len is not None:
        return int(max_kv_len)
    if block_table is not None:
        return int(block_table.shape[1]) * int(k.shape[1])
    return int(k.shape[1])


def _check_decode_inputs(q, k, v, kv_len, block_table):
    """Shapes the decode kernels index through raw pointers: k and v agree with each other and
    with q (batch, head dim, KV heads dividing the query heads); kv_len holds one int32 per
    sequence; a block table has one row per sequence."""
    import torch

    B, Hq, Dqk = q.shape
    if tuple(k.shape[:3]) != tuple(v.shape[:3]):
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} differ in their first three "
                         f"dims")
    if k.shape[3] != Dqk:
        raise ValueError(f"k head dim {k.shape[3]} does not match q's {Dqk}")
    if v.shape[3] > k.shape[3] and v.data_ptr() == k.data_ptr():
        raise ValueError("v aliasing k cannot be wider than k")
    if k.shape[2] == 0 or Hq % k.shape[2] != 0:
        raise ValueError(f"{Hq} query heads are not a multiple of {k.shape[2]} KV heads")
    if block_table is None:
        if k.shape[0] != B:
            raise ValueError(f"k has batch {k.shape[0]}, q has {B}")
    else:
        if (block_table.dtype != torch.int32 or block_table.device != q.device
                or block_table.dim() != 2 or not block_table.is_contiguous()
                or block_table.shape[0] != B):
            raise TypeError("block_table must be a contiguous int32 [B, pages_per_seq] on the "
                            "device")
    if kv_len is not None:
        if kv_len.dtype != torch.int32 or kv_len.device != q.device:
            raise TypeError("kv_len must be int32 on the same device")
        if kv_len.numel() != B or not kv_len.is_contiguous():
            raise ValueError(f"kv_len must be a contiguous tensor of {B} elements, got "
                             f"{tuple(kv_len.shape)}")


def blasst_decode_plan(q, k, v, *, block_r: int = 0, block_c: int = 0, num_splits: int = 0,
                       block_table=None, max_kv_len=None, window: int = 0):
    """(block_r, block_c, num_splits) a decode call on these tensors uses."""
    a = _decode_args(q, k, v, None, kv_len=None, lam=0.0, softmax_scale=0.0, lse=None,
                     counters=None, tile_status=None, tile_margin=None, block_r=block_r,
                     block_c=block_c, num_splits=num_splits, block_table=block_table,
                     max_kv_len=max_kv_len, window=window)
    br, bc, s = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load_library().blasst_decode_plan(ctypes.byref(a), ctypes.byref(br), ctypes.byref(bc),
                                             ctypes.byref(s)), "blasst_decode_plan")
    return br.value, bc.value, s.value


def blasst_decode_workspace_size(q, k, v, *, block_r: int = 0, block_c: int = 0,
                                 num_splits: int = 0, block_table=None, max_kv_len=None,
                                 window: int = 0) -> int:
    a = _decode_args(q, k, v, None, kv_len=None, lam=0.0, softmax_scale=0.0, lse=None,
                     counters=None, tile_status=None, tile_margin=None, block_r=block_r,
                     block_c=block_c, num_splits=num_splits, block_table=block_table,
                     max_kv_len=max_kv_len, window=window)
    return int(load_library().blasst_decode_workspace_size(ctypes.byref(a)))


def blasst_attn_decode(q, k, v, *, kv_len=None, lam: float = 0.0, softmax_scale: float = 0.0,
                       o=None, lse=None, counters=None, tile_status=None, tile_margin=None,
                       block_r: int = 0, block_c: int = 0, num_splits: int = 0, workspace=None,
                       block_table=None, max_kv_len=None, window: int = 0, stream=None):
    """BLASST decode: q [B, Hq, Dqk], k [B, L, Hkv, Dqk], v [B, L, Hkv, Dv] (v may be a view of
    k's first Dv columns: MLA shape); kv_len optional int32 [B] on the device. Returns o.

    Paged cache: block_table int32 [B, pages_per_seq] on the device, k / v page pools
    [pages, page_size, Hkv, d]; max_kv_len defaults to pages_per_seq * page_size.
    window: sliding window in keys (the query sees the last window keys; 0 = none)."""
    import torch

    dev = q.device
    _check_tensor(q, "q", 3, dev)
    _check_tensor(k, "k", 4, dev)
    _check_tensor(v, "v", 4, dev)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    _check_decode_inputs(q, k, v, kv_len, block_table)
    B, Hq = q.shape[0], q.shape[1]
    _check_out(o, "o", (B, Hq, v.shape[3]), q.dtype, dev, contiguous=False)
    _check_out(lse, "lse", (B, Hq), torch.float32, dev, contiguous=True)
    _check_counters(counters, dev)
    if tile_status is not None or tile_margin is not None:
        br, bc, _ = blasst_decode_plan(q, k, v, block_r=block_r, block_c=block_c,
                                       num_splits=num_splits, block_table=block_table,
                                       max_kv_len=max_kv_len, window=window)
        Hkv = k.shape[2]
        L = _decode_max_len(k, block_table, max_kv_len)
        shape = (B, Hkv, -(-(Hq // Hkv) // br), -(-L // bc))
        _check_out(tile_status, "tile_status", shape, torch.uint8, dev, contiguous=True)
        _check_out(tile_margin, "tile_margin", shape, torch.float32, dev, contiguous=True)
    if workspace is not None and workspace is not _NOALLOC:
        if workspace.device != dev:
            raise ValueError(f"workspace is on {workspace.device}, expected {dev}")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
    _check_on_gpu(dev)
    if o is None:
        o = torch.empty((q.shape[0], q.shape[1], v.shape[3]), dtype=q.dtype, device=dev)
    a = _decode_args(q, k, v, o, kv_len=kv_len, lam=lam, softmax_scale=softmax_scale, lse=lse,
                     counters=counters, tile_status=tile_status, tile_margin=tile_margin,
                     block_r=block_r, block_c=block_c, num_splits=num_splits,
                     block_table=block_table, max_kv_len=max_kv_len, window=window)
    lib = load_library()
    if workspace is _NOALLOC:
        _check(lib.blasst_attn_decode_noalloc(ctypes.byref(a), _stream_handle(stream)),
               "blasst_attn_decode_noalloc")
        return o
    need = int(lib.blasst_decode_workspace_size(ctypes.byref(a)))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.blasst_attn_decode(ctypes.byref(a), ws_ptr, ws_bytes, _stream_handle(stream)),
           "blasst_attn_decode")
    return o


_NOALLOC = object()


def blasst_attn_decode_noalloc(q, k, v, *, o, kv_len=None, lam: float = 0.0,
                               softmax_scale: float = 0.0, lse=None, counters=None,
                               tile_status=None, tile_margin=None, block_r: int = 0,
                               block_c: int = 0, num_splits: int = 0, block_table=None,
                               max_kv_len=None, window: int = 0, stream=None):
    """blasst_attn_decode with the split partials in the library's per-GPU scratch array: the
    call allocates nothing (o must be given). Calls that overlap in time on one GPU race."""
    if o is None:
        raise ValueError("blasst_attn_decode_noalloc writes into a caller-provided o")
    return blasst_attn_decode(q, k, v, kv_len=kv_len, lam=lam, softmax_scale=softmax_scale, o=o,
                              lse=lse, counters=counters, tile_status=tile_status,
                              tile_margin=tile_margin, block_r=block_r, block_c=block_c,
                              num_splits=num_splits, workspace=_NOALLOC, block_table=block_table,
                              max_kv_len=max_kv_len, window=window, stream=stream)
