"""Seeded synthetic inputs shaped like the workloads of the BLASST pages.

This module only draws random numbers; it holds none of the attention arithmetic, and both the
GPU library's tests/benchmark and the CPU oracle take their inputs from it.

Recipe (clustered attention). Keys come in runs of ``cluster_len`` consecutive tokens that share a
centre u_c ~ beta * N(0, I_d) / sqrt(d); a key is K_t = 3 u_c + 0.5 * N(0, 1) per coordinate, a
prefill query is Q_t = u_c + 0.5 * N(0, 1) per coordinate, and V ~ N(0, 1). Centres are drawn per
(sequence, KV head); the query heads that share a KV head use that head's centres. ``beta = 1`` is
the recipe read literally; a larger centre gain beta spreads the scores so that some tiles fall
below the threshold (at beta = 1 they almost never do). Extras:

* ``sinks``: the first ``sinks`` keys are attention sinks, K = 3 * mean_c u_c (no noise).
* video DiT: a token's centre is u_frame(f) + u_patch(f, p), with frames of ``frame_len`` tokens
  and patches of ``patch_len`` consecutive tokens inside a frame.
* decode: the one query token of a head is the sum of 1-3 distinct centres of its sequence and KV
  head, chosen uniformly, plus 0.5 * N(0, I_d). With ``share`` every query head of a KV head draws
  the same centres (their noise stays independent).

Values are drawn in float32 and rounded to the target dtype (round-to-nearest-even for bf16).
Prefill tensors are [B, L, H, d] (row-major). Decode caches are stored head-major, [B, Hkv, L, d]
per sequence, and returned as [B, L, Hkv, d] views, so the strides carry the layout.
"""
from __future__ import annotations

import math

import torch


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device):
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)


def prefill_inputs(*, B: int, L: int, Hq: int, Hkv: int, d: int, cluster_len: int,
                   dtype=torch.bfloat16, device="cpu", seed: int = 0, beta: float = 1.0,
                   sinks: int = 0, frame_len: int | None = None, patch_len: int | None = None,
                   d_v: int | None = None):
    """Clustered (Q, K, V) for a prefill call, each [B, L, H, d] in ``dtype`` on ``device``."""
    d_v = d if d_v is None else d_v
    g = _gen(device, seed)
    scale = beta / math.sqrt(d)
    if frame_len is not None:
        n_frames = -(-L // frame_len)
        n_patch = -(-frame_len // patch_len)
        u_frame = _randn((B, Hkv, n_frames, d), g, device) * scale
        u_patch = _randn((B, Hkv, n_frames, n_patch, d), g, device) * scale
        t = torch.arange(L, device=device)
        f = t // frame_len
        p = (t % frame_len) // patch_len
        centre = u_frame[:, :, f, :] + u_patch[:, :, f, p, :]  # [B, Hkv, L, d]
        centres_all = None
    else:
        n_cl = -(-L // cluster_len)
        centres_all = _randn((B, Hkv, n_cl, d), g, device) * scale
        idx = torch.arange(L, device=device) // cluster_len
        centre = centres_all[:, :, idx, :]  # [B, Hkv, L, d]
    k = 3.0 * centre + 0.5 * _randn((B, Hkv, L, d), g, device)
    if sinks:
        if centres_all is None:
            raise ValueError("sinks are defined for the plain clustered recipe")
        sink = 3.0 * centres_all.mean(dim=2, keepdim=True)  # [B, Hkv, 1, d]
        ns = min(sinks, L)  # a sequence shorter than the sink count is all sinks
        k[:, :, :ns, :] = sink.expand(B, Hkv, ns, d)
    grp = Hq // Hkv
    q_centre = centre.repeat_interleave(grp, dim=1)  # [B, Hq, L, d]
    q = q_centre + 0.5 * _randn((B, Hq, L, d), g, device)
    v = _randn((B, Hkv, L, d_v), g, device)
    to = lambda x: x.transpose(1, 2).contiguous().to(dtype)  # noqa: E731  [B, L, H, d]
    return to(q), to(k), to(v)


def decode_inputs(*, B: int, Hq: int, Hkv: int, L: int, d_qk: int, d_v: int, cluster_len: int,
                  dtype=torch.bfloat16, device="cpu", seed: int = 0, beta: float = 1.0,
                  share: bool = False, v_aliases_k: bool = False, kv_len=None):
    """Clustered decode inputs.

    Returns (q [B, Hq, d_qk], k [B, L, Hkv, d_qk] view of [B, Hkv, L, d_qk] storage,
    v [B, L, Hkv, d_v] (a view of k's first d_v columns when ``v_aliases_k``), kv_len int32 [B]).
    """
    g = _gen(device, seed)
    scale = beta / math.sqrt(d_qk)
    n_cl = -(-L // cluster_len)
    centres = _randn((B, Hkv, n_cl, d_qk), g, device) * scale
    idx = torch.arange(L, device=device) // cluster_len
    k_store = torch.empty((B, Hkv, L, d_qk), dtype=dtype, device=device)
    # Fill per sequence to bound the float32 temporaries at full size.
    for b in range(B):
        kb = 3.0 * centres[b][:, idx, :] + 0.5 * _randn((Hkv, L, d_qk), g, device)
        k_store[b] = kb.to(dtype)
        del kb
    grp = Hq // Hkv
    # Query: sum of 1..3 distinct centres of its (sequence, KV head) + noise.
    n_draw_rows = Hkv if share else Hq
    counts = torch.randint(1, 4, (B, n_draw_rows), generator=g, device=device)
    keys = torch.rand((B, n_draw_rows, n_cl), generator=g, device=device)
    order = keys.argsort(dim=-1)  # a uniform random permutation of the centres per row
    rank = torch.empty_like(order)
    rank.scatter_(-1, order, torch.arange(n_cl, device=device).expand_as(order))
    chosen = (rank < counts.unsqueeze(-1)).to(torch.float32)  # first `count` of the permutation
    if share:
        chosen = chosen.repeat_interleave(grp, dim=1)  # [B, Hq, n_cl]
    head_centres = centres.repeat_interleave(grp, dim=1)  # [B, Hq, n_cl, d]
    q = (chosen.unsqueeze(-1) * head_centres).sum(dim=2) + 0.5 * _randn((B, Hq, d_qk), g, device)
    q = q.to(dtype).contiguous()
    k = k_store.transpose(1, 2)  # [B, L, Hkv, d_qk] view
    if v_aliases_k:
        v = k[..., :d_v]
    else:
        v_store = torch.empty((B, Hkv, L, d_v), dtype=dtype, device=device)
        for b in range(B):
            v_store[b] = _randn((Hkv, L, d_v), g, device).to(dtype)
        v = v_store.transpose(1, 2)
    if kv_len is None:
        kv = torch.full((B,), L, dtype=torch.int32, device=device)
    else:
        kv = torch.as_tensor(kv_len, dtype=torch.int32, device=device)
    return q, k, v, kv


def paged_layout(k, v, page_size: int, *, seed: int = 0, spare_pages: int = 3, kv_len=None,
                 heads_major: bool = False):
    """Scatter a per-sequence cache into shuffled pages of a shared pool (layout only).

    k [B, L, Hkv, d_qk], v [B, L, Hkv, d_v] (v may be a view of k's first d_v columns) ->
    (k_pool [P, page_size, Hkv, d_qk], v_pool, block_table int32 [B, ceil(L / page_size)]) with
    k_pool[block_table[b, t // page_size], t % page_size] == k[b, t] for the keys each sequence
    uses (all L, or kv_len[b]); pages are drawn in a random order, with `spare_pages` pool pages
    that no sequence uses, so neighbouring keys of a sequence sit in unrelated pages. When v
    aliases k's first columns, v_pool is the same view of k_pool. heads_major: each page is
    stored [Hkv, page_size, d] (one head's rows of a page contiguous); the pools are returned as
    [P, page_size, Hkv, d] views of that storage either way.
    """
    B, L, Hkv, dq = k.shape
    dv = v.shape[3]
    pps = -(-L // page_size)
    n_pages = B * pps + spare_pages
    g = _gen("cpu", seed)
    perm = torch.randperm(n_pages, generator=g)
    table = perm[: B * pps].view(B, pps).to(torch.int32)
    aliases = v.data_ptr() == k.data_ptr() and v.stride() == k.stride() and dv < dq
    def pool(d, dtype, device):
        if heads_major:
            return torch.zeros((n_pages, Hkv, page_size, d), dtype=dtype,
                               device=device).transpose(1, 2)
        return torch.zeros((n_pages, page_size, Hkv, d), dtype=dtype, device=device)

    k_pool = pool(dq, k.dtype, k.device)
    v_pool = k_pool[..., :dv] if aliases else pool(dv, v.dtype, v.device)
    if kv_len is None and L % page_size == 0:  # every page full: one scatter per pool
        src = k.reshape(B * pps, page_size, Hkv, dq)
        k_pool[table.view(-1).to(k.device)] = src
        if not aliases:
            v_pool[table.view(-1).to(v.device)] = v.reshape(B * pps, page_size, Hkv, dv)
        return k_pool, v_pool, table.to(k.device)
    lens = [L] * B if kv_len is None else [int(x) for x in torch.as_tensor(kv_len).cpu().tolist()]
    for b in range(B):
        for pg in range(-(-lens[b] // page_size)):
            t0, t1 = pg * page_size, min((pg + 1) * page_size, lens[b])
            dst = int(table[b, pg])
            k_pool[dst, : t1 - t0] = k[b, t0:t1]
            if not aliases:
                v_pool[dst, : t1 - t0] = v[b, t0:t1]
    return k_pool, v_pool, table.to(k.device)
