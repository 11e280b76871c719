"""Plain fp64 CPU reference of paged prefill attention.

Test infrastructure: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline of ``bench.py`` use this module; the library never calls it.

What it computes: the prefill path of the dispatch page ("Layer 3: Attention
prefill/decode dispatch", ``dispatch_prefill``): attention for a batch of
variable-length sequences that each bring several query tokens, whose keys
and values live in a paged cache reached through per-sequence block tables,
with cumulative query / key offsets, a causal flag, a left / right window and
a logit soft cap.  The page passes these arguments to a flash-attention call
with block tables and does not define them; the flash-attention conventions
are taken:

* Sequence b owns the query rows cu_q[b] .. cu_q[b+1] - 1 (nq_b of them) and
  the keys 0 .. nk_b - 1, nk_b = cu_k[b+1] - cu_k[b].  Key t of sequence b is
  slot t % bs of physical block block_tables[b, t // bs]; the cache layout is
  the page's [num_blocks, num_kv_heads, block_size, head_dim].
* The queries are the last nq_b positions of the sequence: query i sits at
  position p = nk_b - nq_b + i (the causal mask is aligned to the bottom
  right, so a decode step is the case nq_b = 1).
* Key t is visible to the query at p iff (not causal or t <= p) and
  (window_left < 0 or t >= p - window_left) and (window_right < 0 or
  t <= p + window_right).
* logit = scale * q . k; with a soft cap c > 0 it becomes c * tanh(logit / c);
  softmax over the visible keys; out = sum of the weights times v.  A query
  with no visible key (only possible when nk_b < nq_b under the causal mask,
  or through the window) gets an all-zero output row.
* GQA: query head h reads KV head h // (num_heads / num_kv_heads).

Everything is float64 NumPy; storage words are decoded with the decode
oracle's ``decode_storage``.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from oracle.pa_oracle import decode_storage


def gather_sequence_nhd(key_cache: np.ndarray, value_cache: np.ndarray,
                        table_row: np.ndarray, num_keys: int):
    """Keys and values [num_keys, Hkv, D] of one sequence from a decoded
    [num_blocks, Hkv, bs, D] cache, key t from block table_row[t // bs]."""
    bs = key_cache.shape[2]
    t = np.arange(num_keys)
    phys = np.asarray(table_row)[t // bs]
    slot = t % bs
    k = key_cache[phys, :, slot, :]      # [num_keys, Hkv, D]
    v = value_cache[phys, :, slot, :]
    return k, v


def visible_keys(num_q: int, num_k: int, causal: bool, window_left: int,
                 window_right: int) -> np.ndarray:
    """bool [num_q, num_k]: key t visible to query i (position num_k - num_q + i)."""
    p = (num_k - num_q + np.arange(num_q))[:, None]
    t = np.arange(num_k)[None, :]
    vis = np.ones((num_q, num_k), dtype=bool)
    if causal:
        vis &= t <= p
    if window_left >= 0:
        vis &= t >= p - window_left
    if window_right >= 0:
        vis &= t <= p + window_right
    return vis


def prefill_sequence(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                     visible: np.ndarray, soft_cap: float = 0.0) -> np.ndarray:
    """Attention output [nq, H, D] of one sequence (q [nq, H, D], k / v
    [nk, Hkv, D], visible [nq, nk])."""
    nq, num_heads, _ = q.shape
    num_kv_heads = k.shape[1]
    group = num_heads // num_kv_heads
    out = np.zeros(q.shape, dtype=np.float64)
    for h in range(num_heads):
        kv = h // group
        s = scale * (q[:, h, :] @ k[:, kv, :].T)          # [nq, nk]
        if soft_cap > 0.0:
            s = soft_cap * np.tanh(s / soft_cap)
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        has = np.isfinite(m[:, 0])
        w = np.zeros_like(s)
        w[has] = np.exp(s[has] - m[has])
        w[has] /= w[has].sum(axis=1, keepdims=True)
        out[:, h, :] = w @ v[:, kv, :]
    return out


def paged_prefill(query_raw: np.ndarray, key_cache_raw: np.ndarray,
                  value_cache_raw: np.ndarray, block_tables: np.ndarray,
                  cu_seq_q: np.ndarray, cu_seq_k: np.ndarray, scale: float, *,
                  causal: bool = True, window_left: int = -1, window_right: int = -1,
                  soft_cap: float = 0.0, kind: str = "bf16",
                  seqs: Optional[list] = None) -> np.ndarray:
    """Reference output [total_q, H, D] (float64) of a paged prefill batch.

    ``query_raw`` [total_q, H, D] and the caches [num_blocks, Hkv, bs, D] hold
    storage words of ``kind`` (see ``decode_storage``).  Rows of sequences not
    in ``seqs`` (default: all) are left zero."""
    q_all = decode_storage(query_raw, kind)
    kc = decode_storage(key_cache_raw, kind)
    vc = decode_storage(value_cache_raw, kind)
    cu_q = np.asarray(cu_seq_q, dtype=np.int64)
    cu_k = np.asarray(cu_seq_k, dtype=np.int64)
    num_seqs = len(cu_q) - 1
    out = np.zeros(q_all.shape, dtype=np.float64)
    for b in (range(num_seqs) if seqs is None else seqs):
        nq = int(cu_q[b + 1] - cu_q[b])
        nk = int(cu_k[b + 1] - cu_k[b])
        if nq == 0:
            continue
        q = q_all[cu_q[b]:cu_q[b + 1]]
        if nk == 0:
            continue
        k, v = gather_sequence_nhd(kc, vc, block_tables[b], nk)
        vis = visible_keys(nq, nk, causal, window_left, window_right)
        out[cu_q[b]:cu_q[b + 1]] = prefill_sequence(q, k, v, scale, vis, soft_cap)
    return out
