"""Pins for the paged-prefill oracle (``oracle/prefill_oracle.py``): each check
compares it with something other than itself --

  * dense attention written with ``scipy.special.softmax`` over contiguous
    K / V and a visibility mask built element by element with loops, after
    packing the dense K / V into a shuffled paged [num_blocks, Hkv, bs, D]
    pool with packing code written here;
  * the textbook causal attention of a sequence that is all queries
    (nq = nk: query i sees keys 0..i), written as a running loop;
  * the decode oracle: a prefill of one query per sequence is a decode step
    (same data repacked into the decode layout by code written here), with
    and without a sliding window and a soft cap;
  * closed forms (q = 0: the mean of the visible values) and invariants
    (block-table permutation; without a causal mask or window, a query's
    output does not depend on the other queries; fully masked rows are 0).
Each ``pin_*`` raises AssertionError on a mismatch; ``test_prefill_oracle.py``
runs them, and against broken copies of the oracle."""

from __future__ import annotations

import numpy as np
import scipy.special
import torch

from oracle import pa_oracle as O
from oracle import prefill_oracle as P
from tests.oracle_pins import RAW_VIEW, X_OF_KIND, random_storage


def pack_nhd(k_dense, v_dense, lens, block_size, pool_blocks, rng):
    """Dense per-sequence raw K / V ([L, Hkv, D] each) scattered element by
    element into a shuffled [pool_blocks, Hkv, bs, D] pool; returns the pools
    and the block tables."""
    hkv, d = k_dense[0].shape[1], k_dense[0].shape[2]
    dtype = k_dense[0].dtype
    kc = np.zeros((pool_blocks, hkv, block_size, d), dtype=dtype)
    vc = np.zeros_like(kc)
    need = [(L + block_size - 1) // block_size for L in lens]
    perm = rng.permutation(pool_blocks)
    max_blocks = max(1, max(need))
    tables = np.zeros((len(lens), max_blocks), dtype=np.int32)
    off = 0
    for s, L in enumerate(lens):
        for j in range(need[s]):
            tables[s, j] = perm[off + j]
        off += need[s]
        for t in range(L):
            blk, slot = tables[s, t // block_size], t % block_size
            for h in range(hkv):
                kc[blk, h, slot, :] = k_dense[s][t, h, :]
                vc[blk, h, slot, :] = v_dense[s][t, h, :]
    return kc, vc, tables


def explicit_mask(nq, nk, causal, wl, wr):
    m = np.zeros((nq, nk), dtype=bool)
    for i in range(nq):
        p = nk - nq + i
        for t in range(nk):
            ok = True
            if causal and t > p:
                ok = False
            if wl >= 0 and t < p - wl:
                ok = False
            if wr >= 0 and t > p + wr:
                ok = False
            m[i, t] = ok
    return m


def dense_reference(q, k, v, scale, mask, cap=0.0):
    """q [nq, H, D], k / v [nk, Hkv, D] float64 -> [nq, H, D]."""
    nq, h_all, d = q.shape
    group = h_all // k.shape[1]
    out = np.zeros((nq, h_all, d))
    for h in range(h_all):
        kv = h // group
        for i in range(nq):
            if not mask[i].any():
                continue
            s = scale * (k[:, kv, :] @ q[i, h, :])
            if cap > 0.0:
                s = cap * np.tanh(s / cap)
            w = scipy.special.softmax(s[mask[i]])
            out[i, h] = w @ v[mask[i], kv, :]
    return out


def build_prefill_case(qlens, klens, hkv, group, head_size, block_size, kind, seed=0):
    gen = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    h_all = hkv * group
    q_raw, q_val = random_storage(gen, (sum(qlens), h_all, head_size), kind)
    k_raw, k_val, v_raw, v_val = [], [], [], []
    for L in klens:
        kr, kv_ = random_storage(gen, (L, hkv, head_size), kind)
        vr, vv = random_storage(gen, (L, hkv, head_size), kind)
        k_raw.append(kr); k_val.append(kv_); v_raw.append(vr); v_val.append(vv)
    pool = sum((L + block_size - 1) // block_size for L in klens) + 3
    kc, vc, tables = pack_nhd(k_raw, v_raw, klens, block_size, pool, rng)
    cu_q = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(klens)]).astype(np.int32)
    return dict(q_raw=q_raw, q=q_val, k=k_val, v=v_val, kc=kc, vc=vc, tables=tables,
                cu_q=cu_q, cu_k=cu_k, kind=kind, qlens=list(qlens), klens=list(klens))


def _close(a, b, tol, what):
    err = np.max(np.abs(a - b), initial=0.0)
    assert err <= tol, f"{what}: max |diff| {err:.3e} > {tol:.1e}"


def _oracle(c, scale, **kw):
    return P.paged_prefill(c["q_raw"], c["kc"], c["vc"], c["tables"], c["cu_q"], c["cu_k"],
                           scale, kind=c["kind"], **kw)


def pin_prefill_dense():
    cases = [((1, 5, 7), (1, 37, 40), 2, 1, 64, 16, "bf16"),
             ((16, 3), (16, 70), 1, 3, 64, 32, "f16"),
             ((33,), (100,), 2, 2, 128, 16, "f32"),
             ((4, 6), (2, 6), 1, 2, 64, 16, "bf16")]      # nk < nq: masked rows
    opts = [dict(causal=True), dict(causal=False), dict(causal=True, window_left=9),
            dict(causal=False, window_left=3, window_right=5),
            dict(causal=True, soft_cap=2.0), dict(causal=False, window_right=0)]
    for n, (ql, kl, hkv, g, d, bs, kind) in enumerate(cases):
        c = build_prefill_case(ql, kl, hkv, g, d, bs, kind, seed=n)
        scale = 1.0 / np.sqrt(d)
        for o in opts:
            got = _oracle(c, scale, **o)
            for b in range(len(ql)):
                mask = explicit_mask(ql[b], kl[b], o.get("causal", True),
                                     o.get("window_left", -1), o.get("window_right", -1))
                want = dense_reference(c["q"][c["cu_q"][b]:c["cu_q"][b + 1]], c["k"][b], c["v"][b],
                                       scale, mask, o.get("soft_cap", 0.0))
                _close(got[c["cu_q"][b]:c["cu_q"][b + 1]], want, 1e-12, f"dense case {n} {o} seq {b}")


def pin_prefill_causal_square():
    """nq = nk with the causal mask: query i attends to keys 0..i."""
    c = build_prefill_case((50,), (50,), 2, 2, 64, 16, "f16", seed=11)
    scale = 0.2
    got = _oracle(c, scale, causal=True)
    q, k, v = c["q"], c["k"][0], c["v"][0]
    for i in range(50):
        for h in range(4):
            kv = h // 2
            s = np.array([scale * np.dot(q[i, h], k[t, kv]) for t in range(i + 1)])
            w = scipy.special.softmax(s)
            want = sum(w[t] * v[t, kv] for t in range(i + 1))
            _close(got[i, h], want, 1e-12, f"causal square row {i} head {h}")


def to_decode_layout(nhd_raw, kind):
    """[NB, Hkv, bs, D] raw -> decode K layout [NB, Hkv, D/x, bs, x] and V [NB, Hkv, D, bs]."""
    nb, hkv, bs, d = nhd_raw.shape
    x = X_OF_KIND[kind]
    k = np.zeros((nb, hkv, d // x, bs, x), dtype=nhd_raw.dtype)
    v = np.zeros((nb, hkv, d, bs), dtype=nhd_raw.dtype)
    for c_ in range(d // x):
        for j in range(x):
            k[:, :, c_, :, j] = nhd_raw[:, :, :, c_ * x + j]
    for dd in range(d):
        v[:, :, dd, :] = nhd_raw[:, :, :, dd]
    return k, v


def pin_prefill_one_query_is_decode():
    klens = (1, 16, 17, 600, 1100)
    c = build_prefill_case((1,) * len(klens), klens, 2, 3, 64, 16, "bf16", seed=21)
    kdec, _ = to_decode_layout(c["kc"], "bf16")
    _, vdec = to_decode_layout(c["vc"], "bf16")
    scale = 0.125
    for wl, cap in ((-1, 0.0), (0, 0.0), (100, 0.0), (-1, 5.0), (500, 30.0)):
        got = _oracle(c, scale, causal=True, window_left=wl, soft_cap=cap)
        ref = O.paged_attention(c["q_raw"], kdec, vdec, c["tables"], np.array(klens), scale,
                                q_kind="bf16", kv_kind="bf16", window_left=wl, soft_cap=cap)
        _close(got, ref["out_v1"], 1e-11, f"one query = decode (W={wl}, cap={cap})")


def pin_prefill_zero_query():
    c = build_prefill_case((6, 3), (20, 9), 2, 2, 64, 16, "f16", seed=31)
    c["q_raw"] = np.zeros_like(c["q_raw"])
    got = _oracle(c, 0.3, causal=True, window_left=4)
    for b in range(2):
        nq, nk = c["qlens"][b], c["klens"][b]
        mask = explicit_mask(nq, nk, True, 4, -1)
        for i in range(nq):
            for h in range(4):
                want = c["v"][b][mask[i], h // 2, :].mean(axis=0)
                _close(got[c["cu_q"][b] + i, h], want, 1e-12, "q = 0 mean")


def pin_prefill_invariants():
    c = build_prefill_case((5, 2), (40, 33), 1, 2, 64, 16, "bf16", seed=41)
    base = _oracle(c, 0.25, causal=True)
    # Block-table permutation: move every block to another slot of the pool.
    rng = np.random.default_rng(5)
    perm = rng.permutation(c["kc"].shape[0])
    c2 = dict(c)
    c2["kc"] = np.empty_like(c["kc"]); c2["vc"] = np.empty_like(c["vc"])
    c2["kc"][perm] = c["kc"]; c2["vc"][perm] = c["vc"]
    c2["tables"] = perm[c["tables"]].astype(np.int32)
    assert np.array_equal(_oracle(c2, 0.25, causal=True), base), "block permutation"
    # Without causal mask / window, each query alone gives the same row.
    full = _oracle(c, 0.25, causal=False)
    for b in range(2):
        for i in range(c["qlens"][b]):
            r = c["cu_q"][b] + i
            one = dict(c)
            one["q_raw"] = c["q_raw"][r:r + 1]
            one["tables"] = c["tables"][b:b + 1]
            one["cu_q"] = np.array([0, 1], dtype=np.int32)
            one["cu_k"] = np.array([0, c["klens"][b]], dtype=np.int32)
            _close(_oracle(one, 0.25, causal=False)[0], full[r], 1e-13, "query independence")
    # nk < nq under the causal mask: the first nq - nk rows see nothing.
    c3 = build_prefill_case((6,), (2,), 1, 1, 64, 16, "f32", seed=43)
    got = _oracle(c3, 0.5, causal=True)
    assert np.all(got[:4] == 0.0) and np.all(np.abs(got[4:]).sum(axis=-1) > 0), "masked rows"


def run_all_prefill_pins():
    pin_prefill_dense()
    pin_prefill_causal_square()
    pin_prefill_one_query_is_decode()
    pin_prefill_zero_query()
    pin_prefill_invariants()
