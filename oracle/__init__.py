"""fp64 CPU oracle for the BLASST skip-softmax attention forward pass.

TEST INFRASTRUCTURE ONLY: the plain, slow reference the GPU library is checked against. Only the
test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it.
It shares no code with the GPU library and the GPU library never calls it.

The arithmetic lives in ``blasst_oracle.c`` (double precision, row-major, one unit of work per
call). This module only slices tensors into units, converts the exact input values to float64 and
marshals arguments; the unit and split bookkeeping below restates the tiling of "The Hitchhiker's
Guide -- Phase 08", Section 1 ("FlashAttention Tiling Strategy": B_r query rows against B_c keys)
and the per-tile test of the "Skip-Softmax" design page ("Algorithm").

Unit definitions (the kernel takes the same ones):
  * prefill: unit (b, h, qb) = query rows [qb*B_r, min((qb+1)*B_r, Lq)) of head h in batch b,
    against the keys of KV head g = h // (Hq // Hkv); causal means position p sees keys 0..p.
  * decode: unit (b, g, rb) = query heads g*G + [rb*B_r, min((rb+1)*B_r, G)) of batch b, where
    G = Hq // Hkv, against keys [0, kv_len[b]) of KV head g. With S splits the key tiles are cut
    into S equal runs of ceil(ceil(max_kv_len / B_c) / S) tiles; each run restarts the running
    state and the runs are merged by log-sum-exp.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "blasst_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

TILE_KEPT = 0
TILE_SKIPPED = 1
TILE_NOT_VISITED = 2

_lock = threading.Lock()
_lib = None


def build() -> str:
    """Compile the oracle shared library with gcc (no GPU code involved)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-fopenmp", "-shared", "-fPIC",
                           _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Unit(ctypes.Structure):
    _fields_ = [
        ("n_rows", ctypes.c_int),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("row_first", ctypes.c_void_p),
        ("row_keys", ctypes.c_void_p),
        ("k_begin", ctypes.c_int),
        ("k_end", ctypes.c_int),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("tile_status", ctypes.c_void_p),
        ("tile_margin", ctypes.c_void_p),
        ("max_tiles", ctypes.c_int),
        ("forced", ctypes.c_void_p),
        ("visited", ctypes.c_longlong),
        ("skipped", ctypes.c_longlong),
        ("status", ctypes.c_int),
    ]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or \
                    os.path.getmtime(_SRC) > os.path.getmtime(_LIB_PATH):
                build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I = ctypes.c_int
            D = ctypes.c_double
            lib.oracle_dense_rows.argtypes = [I, I, I, I, P, P, P, P, P, D, P, P]
            lib.oracle_dense_rows.restype = I
            lib.oracle_blasst_rows.argtypes = [I, I, I, P, P, P, P, P, I, I, I, D, D, P, P, P,
                                               P, P, P, P, P, I, P]
            lib.oracle_blasst_rows.restype = I
            lib.oracle_combine.argtypes = [I, I, I, P, P, P, P]
            lib.oracle_combine.restype = I
            lib.oracle_blasst_batch.argtypes = [I, P, I, I, I, D, D, I]
            lib.oracle_blasst_batch.restype = I
            lib.oracle_dense_batch.argtypes = [I, P, I, I, D, I]
            lib.oracle_dense_batch.restype = I
            _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Exact float64 copy (C-contiguous) of a numpy array or a CPU torch tensor."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # only reached when a torch tensor was passed

        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with oracle status {rc}")


# ----------------------------------------------------------------------------------------------
# Row-block level entry points
# ----------------------------------------------------------------------------------------------
def _rows_i32(x):
    return None if x is None else np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def dense_rows(q, k, v, row_keys, scale: float, row_first=None):
    """Dense softmax attention of a block of rows (q: R x d_qk, k: N x d_qk, v: N x d_v).

    Row r attends to keys [row_first[r], row_keys[r]) (row_first None: from 0). Returns
    (O [R, d_v], LSE [R]) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    rk = _rows_i32(row_keys)
    rf = _rows_i32(row_first)
    R, dqk = q.shape
    N, dv = v.shape
    o = np.zeros((R, dv))
    lse = np.zeros(R)
    _check(_load().oracle_dense_rows(R, N, dqk, dv, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(rf) if rf is not None else None, _ptr(rk),
                                     float(scale), _ptr(o), _ptr(lse)), "oracle_dense_rows")
    return o, lse


def blasst_rows(q, k, v, row_keys, k_begin: int, k_end: int, block_c: int, scale: float,
                lam: float, forced=None, row_first=None):
    """Tiled BLASST loop of one row block over keys [k_begin, k_end) (see blasst_oracle.c);
    row r sees keys [row_first[r], row_keys[r]) (row_first None: from 0).

    Returns a dict with o, lse, m (final running max), l (final running sum), visited, skipped,
    tile_status and tile_margin (one entry per tile of the range). ``forced``: optional per-tile
    decisions (TILE_SKIPPED = skip) imposed instead of the test.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    rk = _rows_i32(row_keys)
    rf = _rows_i32(row_first)
    R, dqk = q.shape
    dv = v.shape[1]
    n_tiles = max(0, -(-(k_end - k_begin) // block_c))
    o = np.zeros((R, dv))
    lse = np.zeros(R)
    m = np.zeros(R)
    l = np.zeros(R)
    ts = np.zeros(max(n_tiles, 1), dtype=np.uint8)
    tm = np.zeros(max(n_tiles, 1))
    vis = ctypes.c_longlong(0)
    sk = ctypes.c_longlong(0)
    fz = None
    if forced is not None:
        fz = np.ascontiguousarray(np.asarray(forced, dtype=np.uint8)[:n_tiles])
        if fz.shape[0] < n_tiles:
            raise ValueError("forced decisions must cover every tile of the range")
    rc = _load().oracle_blasst_rows(R, dqk, dv, _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(rf) if rf is not None else None, _ptr(rk), int(k_begin),
                                    int(k_end), int(block_c), float(scale), float(lam), _ptr(o),
                                    _ptr(lse), _ptr(m), _ptr(l), ctypes.byref(vis),
                                    ctypes.byref(sk), _ptr(ts), _ptr(tm), n_tiles,
                                    _ptr(fz) if fz is not None else None)
    _check(rc, "oracle_blasst_rows")
    return dict(o=o, lse=lse, m=m, l=l, visited=vis.value, skipped=sk.value,
                tile_status=ts[:n_tiles].copy(), tile_margin=tm[:n_tiles].copy())


def combine(o_parts, lse_parts):
    """Log-sum-exp merge of partial results (o_parts: S x R x d_v, lse_parts: S x R)."""
    op = _f64(o_parts)
    lp = _f64(lse_parts)
    S, R, dv = op.shape
    o = np.zeros((R, dv))
    lse = np.zeros(R)
    _check(_load().oracle_combine(S, R, dv, _ptr(op), _ptr(lp), _ptr(o), _ptr(lse)),
           "oracle_combine")
    return o, lse


# ----------------------------------------------------------------------------------------------
# Whole-call entry points (prefill and decode), evaluated unit by unit
# ----------------------------------------------------------------------------------------------
@dataclass
class UnitResult:
    o: np.ndarray          # [rows, d_v] float64
    lse: np.ndarray        # [rows] float64 (natural log)
    visited: int
    skipped: int
    tile_status: np.ndarray  # [tiles] uint8, per split concatenated
    tile_margin: np.ndarray  # [tiles] float64


@dataclass
class CallResult:
    units: dict = field(default_factory=dict)  # unit key -> UnitResult

    @property
    def visited(self) -> int:
        return sum(u.visited for u in self.units.values())

    @property
    def skipped(self) -> int:
        return sum(u.skipped for u in self.units.values())


class _Batch:
    """Collects units whose float64 inputs stay alive until the C batch driver has run."""

    def __init__(self, d_qk, d_v, block_c, scale, lam, threads, dense=False):
        self.d_qk, self.d_v, self.block_c = d_qk, d_v, block_c
        self.scale, self.lam, self.threads, self.dense = scale, lam, threads, dense
        self.keep = []
        self.entries = []  # (key, split index, arrays)
        self.bytes = 0

    def add(self, key, split, q, k, v, row_keys, k_begin, k_end, forced=None, row_first=None):
        R = q.shape[0]
        n_tiles = max(0, -(-(k_end - k_begin) // self.block_c))
        if forced is not None:
            forced = np.ascontiguousarray(np.asarray(forced, dtype=np.uint8)[:n_tiles])
            if forced.shape[0] < n_tiles:
                raise ValueError("forced decisions must cover every tile of the range")
        o = np.zeros((R, self.d_v))
        lse = np.zeros(R)
        ts = np.zeros(max(n_tiles, 1), dtype=np.uint8)
        tm = np.zeros(max(n_tiles, 1))
        rk = _rows_i32(row_keys)
        rf = _rows_i32(row_first)
        self.keep.append((q, k, v, rk, rf, forced))
        self.entries.append((key, split, R, q, k, v, rf, rk, k_begin, k_end, o, lse, ts, tm,
                             n_tiles, forced))

    def run(self, sink):
        if not self.entries:
            return
        units = (_Unit * len(self.entries))()
        for i, e in enumerate(self.entries):
            key, split, R, q, k, v, rf, rk, kb, ke, o, lse, ts, tm, nt, fz = e
            u = units[i]
            u.n_rows, u.q, u.k, u.v, u.row_keys = R, q.ctypes.data, k.ctypes.data, v.ctypes.data, rk.ctypes.data
            u.row_first = rf.ctypes.data if rf is not None else None
            u.k_begin, u.k_end = kb, ke
            u.o, u.lse = o.ctypes.data, lse.ctypes.data
            u.tile_status, u.tile_margin, u.max_tiles = ts.ctypes.data, tm.ctypes.data, nt
            u.forced = fz.ctypes.data if fz is not None else None
        lib = _load()
        if self.dense:
            rc = lib.oracle_dense_batch(len(self.entries), ctypes.cast(units, ctypes.c_void_p),
                                        self.d_qk, self.d_v, float(self.scale), int(self.threads))
        else:
            rc = lib.oracle_blasst_batch(len(self.entries), ctypes.cast(units, ctypes.c_void_p),
                                         self.d_qk, self.d_v, int(self.block_c), float(self.scale),
                                         float(self.lam), int(self.threads))
        _check(rc, "oracle batch")
        for i, e in enumerate(self.entries):
            key, split, R, q, k, v, rf, rk, kb, ke, o, lse, ts, tm, nt, _ = e
            sink(key, split, UnitResult(o, lse, units[i].visited, units[i].skipped,
                                        ts[:nt].copy(), tm[:nt].copy()))
        self.keep.clear()
        self.entries.clear()


def _as_shape(x):
    return tuple(int(s) for s in x.shape)


def prefill(q, k, v, *, causal: bool, block_r: int, block_c: int, scale: float, lam: float,
            units=None, threads: int = 0, dense: bool = False, forced=None,
            budget_bytes: int = 1 << 30, window: int = 0) -> CallResult:
    """Oracle of a prefill call. q: [B, Lq, Hq, d_qk], k: [B, Lkv, Hkv, d_qk], v: [B, Lkv, Hkv, d_v].

    window > 0 (causal only): query position i sees keys i - window + 1 .. i (a sliding window
    of window keys ending at the row); tiles before every row's window are not visited.

    units: iterable of (b, h, qb) or None for every unit. dense=True evaluates the dense
    definition instead of the tiled loop (tile fields are then empty). forced: optional dict
    unit -> per-tile decisions imposed instead of the test (see blasst_rows).
    """
    B, Lq, Hq, dqk = _as_shape(q)
    _, Lkv, Hkv, _ = _as_shape(k)
    dv = _as_shape(v)[3]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if causal and Lq != Lkv:
        raise ValueError("causal prefill needs Lq == Lkv")
    if window < 0 or (window and not causal):
        raise ValueError("a sliding window needs causal prefill and window > 0")
    grp = Hq // Hkv
    n_qb = -(-Lq // block_r)
    if units is None:
        units = [(b, h, qb) for b in range(B) for h in range(Hq) for qb in range(n_qb)]
    units = sorted(set(tuple(int(x) for x in u) for u in units), key=lambda u: (u[0], u[1] // grp, u[1], u[2]))
    result = CallResult()

    def sink(key, split, ur):
        result.units[key] = ur

    batch = _Batch(dqk, dv, block_c, scale, lam, threads, dense=dense)
    cache_key, kf, vf = None, None, None
    for (b, h, qb) in units:
        g = h // grp
        if cache_key != (b, g):
            if batch.bytes > budget_bytes:
                batch.run(sink)
                batch.bytes = 0
            kf = _f64(k[b, :, g, :])
            vf = _f64(v[b, :, g, :])
            cache_key = (b, g)
            batch.bytes += kf.nbytes + vf.nbytes
        r0, r1 = qb * block_r, min((qb + 1) * block_r, Lq)
        qf = _f64(q[b, r0:r1, h, :])
        if causal:
            row_keys = [min(p + 1, Lkv) for p in range(r0, r1)]
        else:
            row_keys = [Lkv] * (r1 - r0)
        row_first = [max(0, p - window + 1) for p in range(r0, r1)] if window else None
        batch.add((b, h, qb), 0, qf, kf, vf, row_keys, 0, Lkv,
                  forced.get((b, h, qb)) if forced else None, row_first)
    batch.run(sink)
    return result


def window_first_key(kv_len: int, window: int) -> int:
    """First key a decode query at position kv_len - 1 sees: kv_len - window, or 0 (no window)."""
    return max(0, kv_len - window) if window else 0


def split_ranges(kv_len: int, max_kv_len: int, block_c: int, num_splits: int, window: int = 0):
    """Key ranges of the splits of one sequence: equal runs of whole tiles. Without a window the
    runs cut the tiles of max_kv_len from tile 0; with one they cut the at most
    ceil(window / block_c) + 1 tiles a window can touch, from the tile holding the sequence's
    first visible key."""
    n_tiles = -(-max_kv_len // block_c)
    span = min(n_tiles, -(-window // block_c) + 1) if window else n_tiles
    per = -(-span // num_splits) if span else 0
    base = window_first_key(kv_len, window) // block_c * block_c
    out = []
    for s in range(num_splits):
        a = min(base + s * per * block_c, kv_len)
        e = min(base + (s + 1) * per * block_c, kv_len)
        out.append((a, e))
    return out


def decode(q, k, v, *, kv_len=None, block_r: int, block_c: int, num_splits: int = 1,
           scale: float, lam: float, units=None, threads: int = 0, dense: bool = False,
           forced=None, budget_bytes: int = 1 << 30, window: int = 0) -> CallResult:
    """Oracle of a decode call (one query token per sequence).

    q: [B, Hq, d_qk], k: [B, L, Hkv, d_qk], v: [B, L, Hkv, d_v]; kv_len: per-sequence lengths
    (None = all L). units: iterable of (b, g, rb) or None for all. Each unit's splits are merged
    by log-sum-exp; visited/skipped cover all of its splits and the tile arrays are indexed by
    absolute tile (ceil(max(kv_len) / block_c) entries; tiles no split visits are "not
    visited"). forced: optional dict unit -> decisions for the unit's tiles 0, 1, ... (absolute
    tile index), imposed instead of the test. window > 0: the query (at position kv_len - 1)
    sees only keys kv_len - window .. kv_len - 1 (see split_ranges for the splits).
    """
    B, Hq, dqk = _as_shape(q)
    _, L, Hkv, _ = _as_shape(k)
    dv = _as_shape(v)[3]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    grp = Hq // Hkv
    if kv_len is None:
        kv_len = [L] * B
    kv_len = [int(x) for x in (kv_len.tolist() if hasattr(kv_len, "tolist") else kv_len)]
    max_len = max(kv_len) if kv_len else 0
    n_rb = -(-grp // block_r)
    if units is None:
        units = [(b, g, rb) for b in range(B) for g in range(Hkv) for rb in range(n_rb)]
    units = sorted(set(tuple(int(x) for x in u) for u in units))
    if window < 0:
        raise ValueError("window must be >= 0")
    parts: dict = {}
    starts: dict = {}  # unit -> first absolute tile of each split's range

    def sink(key, split, ur):
        parts.setdefault(key, {})[split] = ur

    batch = _Batch(dqk, dv, block_c, scale, lam, threads, dense=dense)
    cache_key, kf, vf = None, None, None
    for (b, g, rb) in units:
        if cache_key != (b, g):
            if batch.bytes > budget_bytes:
                batch.run(sink)
                batch.bytes = 0
            kf = _f64(k[b, :kv_len[b], g, :]) if kv_len[b] > 0 else np.zeros((1, dqk))
            vf = _f64(v[b, :kv_len[b], g, :]) if kv_len[b] > 0 else np.zeros((1, dv))
            cache_key = (b, g)
            batch.bytes += kf.nbytes + vf.nbytes
        h0 = g * grp + rb * block_r
        h1 = min(g * grp + (rb + 1) * block_r, (g + 1) * grp)
        qf = _f64(q[b, h0:h1, :])
        first = window_first_key(kv_len[b], window)
        if dense or num_splits == 1:
            ranges = [(first // block_c * block_c, kv_len[b])]
        else:
            ranges = split_ranges(kv_len[b], max_len, block_c, num_splits, window)
        fu = forced.get((b, g, rb)) if forced else None
        for s, (a, e) in enumerate(ranges):
            fs = None if fu is None else np.asarray(fu)[a // block_c:]
            batch.add((b, g, rb), s, qf, kf, vf, [kv_len[b]] * (h1 - h0), a, e, fs,
                      [first] * (h1 - h0) if window else None)
        starts.setdefault((b, g, rb), [a // block_c for a, _ in ranges])
    batch.run(sink)

    n_all = -(-max_len // block_c)
    result = CallResult()
    for key, sp in parts.items():
        idx = sorted(sp)
        ts = np.full(n_all, TILE_NOT_VISITED, dtype=np.uint8)
        tm = np.full(n_all, -np.inf)
        for i in idx:
            t0 = starts[key][i]
            nt = len(sp[i].tile_status)
            ts[t0:t0 + nt] = sp[i].tile_status
            tm[t0:t0 + nt] = sp[i].tile_margin
        if len(idx) == 1:
            o, lse = sp[idx[0]].o, sp[idx[0]].lse
        else:
            o, lse = combine(np.stack([sp[i].o for i in idx]), np.stack([sp[i].lse for i in idx]))
        result.units[key] = UnitResult(o, lse, sum(sp[i].visited for i in idx),
                                       sum(sp[i].skipped for i in idx), ts, tm)
    return result


def default_scale(d_qk: int) -> float:
    """1/sqrt(d_qk), the scaling of the attention definition in "The Hitchhiker's Guide"."""
    return 1.0 / math.sqrt(d_qk)


# ------------------------------------------------------------------------------------------
# Calibration ("BLASST: Dynamic BLocked Attention Sparsity via Softmax Thresholding" talk notes,
# threshold calibration, Algorithm 2 steps 1-3 and Eq. 3). Plain numpy restatements.
# ------------------------------------------------------------------------------------------

def sparsity_curve(tile_margin, tile_status, lambdas):
    """Skip fraction at each lambda from one run's per-tile margins (natural log).

    A visited tile (status 0 or 1) is skipped at threshold lambda exactly when its margin is below
    ln(min(lambda, 1)); lambda = 0 skips nothing. Returns (list of fractions, visited count)."""
    m = np.asarray(tile_margin, dtype=np.float64).ravel()
    st = np.asarray(tile_status).ravel()
    vis = st != 2
    n_vis = int(vis.sum())
    out = []
    for lam in np.asarray(lambdas, dtype=np.float64).ravel():
        lam = min(float(lam), 1.0)
        tau = math.log(lam) if lam > 0.0 else -math.inf
        n_skip = int(np.sum(vis & (m < tau)))
        out.append(n_skip / n_vis if n_vis else 0.0)
    return out, n_vis


def fit_calibration(seq_len, lam, sparsity):
    """(a, b) of the model lambda * L = a * exp(b * S): least squares of ln(lambda L) = ln a + b S."""
    L = np.asarray(seq_len, dtype=np.float64).ravel()
    la = np.asarray(lam, dtype=np.float64).ravel()
    S = np.asarray(sparsity, dtype=np.float64).ravel()
    y = np.log(la * L)
    X = np.stack([np.ones_like(S), S], axis=1)
    (ln_a, b), *_ = np.linalg.lstsq(X, y, rcond=None)
    return float(math.exp(ln_a)), float(b)
