"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Every check here compares the oracle with an independent source of truth:
  * a dense attention written with ``scipy.special.softmax`` on contiguous K/V
    (a textbook routine), after packing the dense K/V into the paged layout
    with packing code written here, separately from the oracle's gather;
  * ``scipy.special.logsumexp`` for the per-partition statistics;
  * closed forms (q = 0 gives uniform weights; q = 0 with ALiBi gives a
    geometric distribution whose sums and means are known exactly);
  * torch's own dtype conversions for bf16 / fp16 / fp8-e4m3fn storage, and
    the special values of the OCP FP8 definition;
  * invariants the pages state (v2 with one partition equals v1; the
    log-sum-exp merge equals the full softmax for any partition size;
    block-table permutation does not change the result);
  * the dispatch rule's worked example printed on the dispatch page
    (``tests/golden/dispatch_rule_bi_v100.txt``).
Each ``pin_*`` function raises AssertionError on a mismatch.  They are run by
``test_oracle_pins.py`` and, against deliberately broken copies of the
oracle, by ``test_oracle_mutations.py``.
"""

from __future__ import annotations

import math
import os

import numpy as np
import scipy.special
import torch

from oracle import pa_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

X_OF_KIND = {"f32": 4, "f16": 8, "bf16": 8, "fp8_e4m3": 16}
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "fp8_e4m3": torch.float8_e4m3fn}
RAW_VIEW = {"f32": (torch.float32, np.float32), "f16": (torch.int16, np.uint16),
            "bf16": (torch.int16, np.uint16), "fp8_e4m3": (torch.uint8, np.uint8)}


# --------------------------------------------------------------------------
# Test-side data construction (independent of the oracle)
# --------------------------------------------------------------------------

def random_storage(gen: torch.Generator, shape, kind: str, std: float = 1.0):
    """Random values representable in ``kind``: (raw storage ndarray, float64 values)."""
    t = torch.randn(*shape, generator=gen, dtype=torch.float32) * std
    if kind == "fp8_e4m3":
        t = t.clamp(-448.0, 448.0)
    stored = t.to(TORCH_DTYPE[kind])
    values = stored.to(torch.float32).to(torch.float64).numpy()
    tview, npview = RAW_VIEW[kind]
    raw = stored.view(tview).numpy().view(npview) if kind != "f32" else stored.numpy()
    return raw.copy(), values


def pack_paged(k_dense_raw, v_dense_raw, lens, block_size, x, pool_blocks, rng,
               fill=0):
    """Scatter dense per-sequence K/V into a shuffled paged pool.

    k_dense_raw[b] / v_dense_raw[b]: [L_b, Hkv, D] raw storage.
    Returns key_cache [NB, Hkv, D/x, bs, x], value_cache [NB, Hkv, D, bs],
    block_tables [B, max_blocks].  Written element by element so that it
    shares nothing with the oracle's transpose/reshape gather.
    """
    hkv, head_size = k_dense_raw[0].shape[1:]
    dtype = k_dense_raw[0].dtype
    need = [(L + block_size - 1) // block_size for L in lens]
    assert sum(need) <= pool_blocks
    perm = rng.permutation(pool_blocks)
    max_blocks = max(1, max(need))
    tables = np.zeros((len(lens), max_blocks), dtype=np.int32)
    kc = np.full((pool_blocks, hkv, head_size // x, block_size, x), fill, dtype=dtype)
    vc = np.full((pool_blocks, hkv, head_size, block_size), fill, dtype=dtype)
    nxt = 0
    for b, L in enumerate(lens):
        for i in range(need[b]):
            tables[b, i] = perm[nxt]
            nxt += 1
        for t in range(L):
            phys = tables[b, t // block_size]
            slot = t % block_size
            for d in range(head_size):
                kc[phys, :, d // x, slot, d % x] = k_dense_raw[b][t, :, d]
                vc[phys, :, d, slot] = v_dense_raw[b][t, :, d]
    return kc, vc, tables


def dense_attention(q, k, v, scale, slopes=None, cap=0.0):
    """softmax(scale * q K^T + slope * t) V on contiguous K/V [L, Hkv, D];
    with cap > 0 the scaled dot products pass through cap * tanh(. / cap)
    first (that formula itself is pinned by pin_soft_cap_forms)."""
    num_heads = q.shape[0]
    group = num_heads // k.shape[1]
    out = np.empty((num_heads, v.shape[2]))
    for h in range(num_heads):
        logits = scale * (k[:, h // group, :] @ q[h])
        if cap > 0.0:
            logits = cap * np.tanh(logits / cap)
        if slopes is not None:
            logits = logits + slopes[h] * np.arange(k.shape[0])
        out[h] = scipy.special.softmax(logits) @ v[:, h // group, :]
    return out


def dense_logits(q, k, scale, slopes=None):
    num_heads = q.shape[0]
    group = num_heads // k.shape[1]
    s = np.empty((num_heads, k.shape[0]))
    for h in range(num_heads):
        s[h] = scale * (k[:, h // group, :] @ q[h])
        if slopes is not None:
            s[h] += slopes[h] * np.arange(k.shape[0])
    return s


def build_case(lens, hkv, group, head_size, block_size, kv_kind, q_kind=None,
               seed=0, pool_extra=3):
    """A small batch: dense values, their paged packing, and metadata."""
    if q_kind is None:
        q_kind = "bf16" if kv_kind == "fp8_e4m3" else kv_kind
    gen = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    num_heads = hkv * group
    q_raw, q_val = random_storage(gen, (len(lens), num_heads, head_size), q_kind)
    kd_raw, kd_val, vd_raw, vd_val = [], [], [], []
    for L in lens:
        a, b = random_storage(gen, (L, hkv, head_size), kv_kind)
        c, d = random_storage(gen, (L, hkv, head_size), kv_kind)
        kd_raw.append(a); kd_val.append(b); vd_raw.append(c); vd_val.append(d)
    pool = sum((L + block_size - 1) // block_size for L in lens) + pool_extra
    kc, vc, tables = pack_paged(kd_raw, vd_raw, lens, block_size, X_OF_KIND[kv_kind], pool, rng)
    return dict(q_raw=q_raw, q=q_val, k=kd_val, v=vd_val, kc=kc, vc=vc,
                tables=tables, lens=np.array(lens), q_kind=q_kind, kv_kind=kv_kind)


def run_oracle(case, scale, slopes=None, k_scale=1.0, v_scale=1.0, **kw):
    return O.paged_attention(case["q_raw"], case["kc"], case["vc"], case["tables"],
                             case["lens"], scale, q_kind=case["q_kind"],
                             kv_kind=case["kv_kind"], k_scale=k_scale, v_scale=v_scale,
                             alibi_slopes=slopes, **kw)


def _close(a, b, tol, what):
    a = np.asarray(a); b = np.asarray(b)
    err = np.abs(a - b).max(initial=0.0)
    ref = max(np.abs(b).max(initial=0.0), 1.0)
    assert err <= tol * ref, f"{what}: max abs err {err:.3e} > {tol:.1e} * {ref:.3e}"


# --------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------

def pin_fp8_special_values():
    """OCP E4M3FN special values and the full table against torch's decode."""
    t = O.fp8_e4m3fn_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9
    assert t[0x38] == 1.0 and t[0x40] == 2.0 and t[0xB8] == -1.0
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    assert int(np.isfinite(t).sum()) == 254
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must be strictly increasing"
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).to(torch.float64).numpy()
    finite = np.isfinite(ref)
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    assert np.array_equal(t[finite], ref[finite])
    assert np.array_equal(O.decode_storage(np.arange(256, dtype=np.uint8), "fp8_e4m3")[finite],
                          ref[finite])


def pin_storage_decode():
    """bf16 / fp16 / f32 bit patterns decode as torch decodes them."""
    gen = torch.Generator().manual_seed(7)
    bits = torch.randint(0, 1 << 16, (4096,), generator=gen, dtype=torch.int32).to(torch.int16)
    raw = bits.numpy().view(np.uint16)
    for kind, dt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        ref = bits.view(dt).to(torch.float32).to(torch.float64).numpy()
        got = O.decode_storage(raw, kind)
        same = (got == ref) | (np.isnan(got) & np.isnan(ref))
        assert same.all(), f"{kind} decode mismatch"
    assert O.decode_storage(np.array([0x3F80, 0xC000, 0x7F80], np.uint16), "bf16").tolist() == \
        [1.0, -2.0, math.inf]
    assert O.decode_storage(np.array([0x3C00, 0xC000, 0x0001], np.uint16), "f16").tolist() == \
        [1.0, -2.0, 2.0 ** -24]
    f = np.array([1.5, -3.25], np.float32)
    assert O.decode_storage(f, "f32").tolist() == [1.5, -3.25]


def pin_brute_force(lens, hkv, group, head_size, block_size, kv_kind,
                    alibi=False, k_scale=1.0, v_scale=1.0, seed=0):
    """Oracle on the paged layout == dense softmax attention on contiguous K/V."""
    case = build_case(lens, hkv, group, head_size, block_size, kv_kind, seed=seed)
    num_heads = hkv * group
    scale = 1.0 / math.sqrt(head_size)
    slopes = np.array([2.0 ** (-8.0 * (h + 1) / num_heads) for h in range(num_heads)]) if alibi else None
    res = run_oracle(case, scale, slopes, k_scale, v_scale)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(res["out_v1"][b] == 0) and np.all(res["out_v2"][b] == 0)
            continue
        ref = dense_attention(case["q"][b], case["k"][b] * k_scale,
                              case["v"][b] * v_scale, scale, slopes)
        _close(res["out_v1"][b], ref, 1e-12, f"v1 out seq {b} L={L}")
        _close(res["out_v2"][b], ref, 1e-12, f"v2 out seq {b} L={L}")


def pin_partition_statistics(lens=(1, 100, 513, 1100), hkv=2, group=3, head_size=64,
                             block_size=16, kv_kind="f32", alibi=True):
    """Per partition: m_p = max s, m_p + log S_p = logsumexp(s), O_p = softmax over T_p."""
    case = build_case(list(lens), hkv, group, head_size, block_size, kv_kind, seed=11)
    num_heads = hkv * group
    scale = 0.125
    slopes = np.linspace(0.01, 0.3, num_heads) if alibi else None
    max_p = O.num_partitions(max(lens)) + 2
    res = run_oracle(case, scale, slopes, max_num_partitions=max_p)
    ps = O.PARTITION_SIZE
    for b, L in enumerate(lens):
        s = dense_logits(case["q"][b], case["k"][b], scale, slopes)
        n_part = (L + ps - 1) // ps
        for p in range(max_p):
            ml = res["max_logits"][b, :, p]
            es = res["exp_sums"][b, :, p]
            to = res["tmp_out"][b, :, p, :]
            if p >= n_part:
                assert np.all(ml == -np.inf) and np.all(es == 0) and np.all(to == 0), \
                    "padding partition must be -inf / 0 / 0"
                continue
            sp = s[:, p * ps:min((p + 1) * ps, L)]
            _close(ml, sp.max(axis=1), 1e-12, "max_logits")
            _close(ml + np.log(es), scipy.special.logsumexp(sp, axis=1), 1e-12, "logsumexp")
            grp = num_heads // hkv
            for h in range(num_heads):
                vseg = case["v"][b][p * ps:min((p + 1) * ps, L), h // grp, :]
                _close(to[h], scipy.special.softmax(sp[h]) @ vseg, 1e-12, "tmp_out")


def pin_uniform_closed_form():
    """q = 0, no ALiBi: every logit is 0, so m_p = 0, S_p = |T_p|, O_p and out are means."""
    lens = [5, 512, 700, 1030]
    case = build_case(lens, 2, 2, 64, 16, "f32", seed=3)
    case["q_raw"][:] = 0.0
    res = run_oracle(case, 0.125, max_num_partitions=4)
    ps = O.PARTITION_SIZE
    for b, L in enumerate(lens):
        n_part = (L + ps - 1) // ps
        for p in range(n_part):
            n = min((p + 1) * ps, L) - p * ps
            assert np.all(res["max_logits"][b, :, p] == 0.0)
            assert np.all(res["exp_sums"][b, :, p] == float(n))
            seg_mean = case["v"][b][p * ps:p * ps + n].mean(axis=0)       # [Hkv, D]
            _close(res["tmp_out"][b, :, p, :], np.repeat(seg_mean, 2, axis=0), 1e-12, "O_p mean")
        full_mean = case["v"][b].mean(axis=0)
        _close(res["out_v1"][b], np.repeat(full_mean, 2, axis=0), 1e-12, "out mean")
        _close(res["out_v2"][b], np.repeat(full_mean, 2, axis=0), 1e-12, "out mean v2")


def pin_alibi_closed_form():
    """q = 0 with ALiBi slope a and V_t = t: the weights are geometric.

    Per partition of n tokens ending at e: m_p = a (e - 1) and
    S_p = (1 - r^n) / (1 - r) with r = exp(-a).  For the whole sequence the
    mean of k = L - 1 - t under weights r^k is r/(1-r) - L r^L / (1 - r^L),
    so out = (L - 1) - that mean in every dimension.
    """
    lens = [1, 300, 1500]
    hkv, group, head_size, bs = 2, 2, 64, 16
    case = build_case(lens, hkv, group, head_size, bs, "f32", seed=5)
    case["q_raw"][:] = 0.0
    # V_t = t in every head and dim, written straight into the paged pool.
    for b, L in enumerate(lens):
        for t in range(L):
            case["vc"][case["tables"][b, t // bs], :, :, t % bs] = float(t)
    slopes = np.array([0.5, 0.05, 0.005, 0.0005])
    res = run_oracle(case, 0.125, slopes, max_num_partitions=3)
    ps = O.PARTITION_SIZE
    for b, L in enumerate(lens):
        n_part = (L + ps - 1) // ps
        for p in range(n_part):
            e = min((p + 1) * ps, L)
            n = e - p * ps
            for h, a in enumerate(slopes):
                r = math.exp(-a)
                m = res["max_logits"][b, h, p]
                assert abs(m - a * (e - 1)) <= 1e-12 * max(1.0, a * e), "ALiBi max logit"
                s_ref = (1.0 - r ** n) / (1.0 - r)
                assert abs(res["exp_sums"][b, h, p] - s_ref) <= 1e-12 * s_ref, "ALiBi exp sum"
        for h, a in enumerate(slopes):
            r = math.exp(-a)
            mean_k = r / (1 - r) - L * r ** L / (1 - r ** L) if L > 1 else 0.0
            expect = (L - 1) - mean_k
            got = res["out_v1"][b, h]
            assert np.all(np.abs(got - expect) <= 1e-9 * max(1.0, L)), \
                f"ALiBi geometric mean: {got[0]} vs {expect}"
            assert np.all(np.abs(res["out_v2"][b, h] - expect) <= 1e-9 * max(1.0, L))


def pin_single_token():
    """L = 1: out = V_0, S = 1, m = scale * q.k_0 + 0 (ALiBi at t = 0 adds nothing)."""
    case = build_case([1, 1], 2, 4, 128, 32, "bf16", seed=9)
    slopes = np.linspace(0.1, 0.8, 8)
    res = run_oracle(case, 0.1, slopes, max_num_partitions=2)
    for b in range(2):
        for h in range(8):
            g = h // 4
            _close(res["out_v1"][b, h], case["v"][b][0, g], 1e-15, "L=1 out")
            assert res["exp_sums"][b, h, 0] == 1.0
            m = 0.1 * float(case["q"][b][h] @ case["k"][b][0, g])
            assert abs(res["max_logits"][b, h, 0] - m) <= 1e-12 * max(1.0, abs(m))
            assert res["max_logits"][b, h, 1] == -np.inf and res["exp_sums"][b, h, 1] == 0


def pin_partition_size_independence():
    """The merged output is the full softmax for every partition size."""
    lens = [1100]
    case = build_case(lens, 2, 2, 64, 16, "f32", seed=13)
    ref = dense_attention(case["q"][0], case["k"][0], case["v"][0], 0.125)
    for ps in (16, 64, 256, 512, 1024, 1100):
        res = run_oracle(case, 0.125, partition_size=ps)
        _close(res["out_v2"][0], ref, 1e-12, f"partition size {ps}")


def pin_v2_single_partition_equals_v1():
    """With one partition the v2 partial output and the merge both equal v1."""
    case = build_case([17, 512], 2, 2, 64, 16, "f32", seed=17)
    res = run_oracle(case, 0.125, max_num_partitions=1)
    for b in range(2):
        ref = dense_attention(case["q"][b], case["k"][b], case["v"][b], 0.125)
        _close(res["tmp_out"][b, :, 0, :], ref, 1e-12, "tmp_out with one partition")
        _close(res["out_v1"][b], res["out_v2"][b], 1e-14, "v1 vs v2")


def pin_block_table_permutation():
    """Relabelling physical blocks (pool and table together) changes nothing."""
    case = build_case([37, 700], 2, 2, 64, 16, "f32", seed=19, pool_extra=17)
    res0 = run_oracle(case, 0.125)
    rng = np.random.default_rng(1)
    nb = case["kc"].shape[0]
    perm = rng.permutation(nb)            # new position of old block i is perm[i]
    kc2 = np.empty_like(case["kc"]); vc2 = np.empty_like(case["vc"])
    kc2[perm] = case["kc"]; vc2[perm] = case["vc"]
    case2 = dict(case, kc=kc2, vc=vc2, tables=perm[case["tables"]].astype(np.int32))
    res1 = run_oracle(case2, 0.125)
    for key in ("out_v1", "out_v2", "max_logits", "exp_sums", "tmp_out"):
        assert np.array_equal(res0[key], res1[key]), key


def pin_convexity_and_dominant_key():
    """out lies in the per-dim hull of V; a key aligned with q dominates."""
    case = build_case([300], 1, 2, 64, 16, "f32", seed=23)
    res = run_oracle(case, 0.125)
    v = case["v"][0][:, 0, :]
    for h in range(2):
        assert np.all(res["out_v1"][0, h] <= v.max(axis=0) + 1e-12)
        assert np.all(res["out_v1"][0, h] >= v.min(axis=0) - 1e-12)
    # Make token 123's key a large multiple of head 0's query.
    tstar, bs = 123, 16
    q0 = case["q"][0][0]
    phys = case["tables"][0, tstar // bs]
    case["kc"][phys, 0, :, tstar % bs, :] = (q0 * 400.0).astype(np.float32).reshape(16, 4)
    res = run_oracle(case, 0.125)
    _close(res["out_v1"][0, 0], v[tstar], 1e-9, "dominant key")


def pin_empty_sequence():
    """seq_len = 0: zero output and padding statistics."""
    case = build_case([0, 20], 1, 1, 64, 16, "f32", seed=29)
    res = run_oracle(case, 0.125, max_num_partitions=2)
    assert np.all(res["out_v1"][0] == 0) and np.all(res["out_v2"][0] == 0)
    assert np.all(res["max_logits"][0] == -np.inf) and np.all(res["exp_sums"][0] == 0)


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


def pin_dispatch_golden():
    """The dispatch page's worked example of ``should_use_paged_v2``."""
    for seq_len, hkv, sms, want in read_golden("dispatch_rule_bi_v100.txt"):
        got = O.page_should_use_v2(int(seq_len), int(hkv), int(sms))
        assert got == (want == "v2"), (seq_len, hkv, sms, want)


def pin_partition_count_golden():
    """ceil(L / 512): the V2 page's code; 100000 tokens give 196 partitions."""
    for seq_len, parts in read_golden("partition_count.txt"):
        assert O.num_partitions(int(seq_len)) == int(parts), (seq_len, parts)


def pin_sliding_window(lens=(1, 16, 17, 600, 1100), hkv=2, group=3, head_size=64,
                       block_size=16, kv_kind="bf16", alibi=True, cap=0.0, seed=11):
    """Sliding window W: the oracle on the paged layout equals dense attention
    over the last W + 1 keys of the contiguous K/V (a window is a contiguous
    key range; ALiBi's absolute offset cancels in the softmax); W = 0 returns
    the last value row; W >= L - 1 and W = -1 give exactly the unwindowed
    result; partitions with no visible key are padding (-inf, 0, 0) and the
    visible ones hold the log-sum-exp statistics of their visible keys."""
    case = build_case(list(lens), hkv, group, head_size, block_size, kv_kind, seed=seed)
    num_heads = hkv * group
    scale = 1.0 / math.sqrt(head_size)
    slopes = (np.array([2.0 ** (-8.0 * (h + 1) / num_heads) for h in range(num_heads)])
              if alibi else None)
    full = run_oracle(case, scale, slopes, soft_cap=cap)
    for w in (0, 1, 15, 16, 17, 100, 511, 512, 513, 1099, 5000):
        res = run_oracle(case, scale, slopes, window_left=w, soft_cap=cap)
        for b, L in enumerate(lens):
            lo = max(0, L - 1 - w)
            q = case["q"][b]
            ref = dense_attention(q, case["k"][b][lo:], case["v"][b][lo:], scale,
                                  None if slopes is None else slopes, cap=cap)
            _close(res["out_v1"][b], ref, 1e-12, f"window {w} L {L} v1")
            _close(res["out_v2"][b], ref, 1e-12, f"window {w} L {L} v2")
            if w == 0:
                group_of = np.arange(num_heads) // group
                _close(res["out_v1"][b], case["v"][b][L - 1][group_of], 1e-12, "window 0")
            if w >= L - 1:
                for key in ("out_v1", "out_v2", "max_logits", "exp_sums", "tmp_out"):
                    assert np.array_equal(res[key][b], full[key][b]), (key, w, L)
            # statistics per partition over the visible keys only
            logits = dense_logits(q, case["k"][b], scale, slopes)
            if cap > 0.0:
                raw = dense_logits(q, case["k"][b], scale, None)
                logits = logits - raw + cap * np.tanh(raw / cap)
            for p in range(O.num_partitions(L)):
                a, e = p * 512, min((p + 1) * 512, L)
                vis = logits[:, max(a, lo):e]
                if vis.shape[1] == 0:
                    assert np.all(np.isneginf(res["max_logits"][b, :, p]))
                    assert np.all(res["exp_sums"][b, :, p] == 0.0)
                    assert np.all(res["tmp_out"][b, :, p] == 0.0)
                else:
                    _close(res["max_logits"][b, :, p], vis.max(axis=1), 1e-12, "window max")
                    _close(np.log(res["exp_sums"][b, :, p]) + res["max_logits"][b, :, p],
                           scipy.special.logsumexp(vis, axis=1), 1e-12, "window logsumexp")
    # W = -1 is no window at all
    none = run_oracle(case, scale, slopes, window_left=-1, soft_cap=cap)
    for key in ("out_v1", "max_logits", "exp_sums"):
        assert np.array_equal(none[key], full[key]), key


def pin_soft_cap_forms():
    """The soft cap c * tanh(s / c) on the scaled logits, before ALiBi:
    small logits follow the series s - s^3 / (3 c^2) (placement of c and of
    the scale); large logits stay inside (-c, c) with their order kept; the
    ALiBi bias is added after the cap (logits minus the bias lie in (-c, c)
    even with steep slopes); a huge cap changes nothing; q = 0 still gives
    the plain mean of V."""
    case = build_case([40], 1, 2, 64, 16, "f32", seed=21)
    q, k = case["q"][0], case["k"][0]
    scale = 1.0 / 8.0
    # series regime: scale the query down so |s| <= ~2e-3
    small = O.sequence_logits(q * 1e-3, k, scale, None, -1, 0.5)
    s = dense_logits(q * 1e-3, k, scale)
    assert np.abs(s).max() < 5e-3
    _close(small, s - s ** 3 / (3 * 0.5 ** 2), 1e-11, "soft cap series")
    # saturation regime
    big = O.sequence_logits(q * 50.0, k, scale, None, -1, 2.0)
    sb = dense_logits(q * 50.0, k, scale)
    assert np.all(np.abs(big) <= 2.0)      # tanh saturates to exactly 1 in fp64
    assert np.abs(sb).max() > 20.0 and np.abs(big).max() > 1.99
    for h in range(big.shape[0]):
        assert np.all(np.diff(big[h][np.argsort(sb[h])]) >= 0.0), "the cap must keep the order"
    # ALiBi after the cap
    slopes = np.array([3.0, 5.0])
    with_bias = O.sequence_logits(q, k, scale, slopes, -1, 1.0)
    unbiased = with_bias - slopes[:, None] * np.arange(k.shape[0])[None, :]
    assert np.all(np.abs(unbiased) <= 1.0)
    # a huge cap is no cap
    _close(O.sequence_logits(q, k, scale, slopes, -1, 1e9), O.sequence_logits(q, k, scale, slopes),
           1e-12, "huge cap")
    # q = 0: every logit is 0 -> the mean of V
    case0 = build_case([300], 1, 1, 64, 16, "f32", seed=22)
    case0["q_raw"] = np.zeros_like(case0["q_raw"])
    res = run_oracle(case0, 0.125, soft_cap=3.0)
    _close(res["out_v1"][0, 0], case0["v"][0][:, 0, :].mean(axis=0), 1e-12, "cap q=0 mean")


def pin_window_and_cap_brute_force():
    """Window and soft cap together on every storage kind: paged oracle ==
    dense attention over the visible keys."""
    for kind, bs, group in (("fp8_e4m3", 32, 8), ("f16", 16, 4), ("f32", 16, 1)):
        pin_sliding_window(lens=(33, 700), hkv=1, group=group, head_size=128 if kind == "fp8_e4m3" else 64,
                           block_size=bs, kv_kind=kind, alibi=kind != "f16", cap=20.0, seed=31)


BRUTE_FORCE_SMALL = [
    # lens, hkv, group, D, bs, kind, alibi, k_scale, v_scale
    ([1, 15, 16, 17], 1, 1, 64, 16, "f32", False, 1.0, 1.0),
    ([511, 512, 513], 2, 2, 64, 16, "bf16", True, 1.0, 1.0),
    ([1100, 33], 1, 7, 128, 16, "f16", False, 1.0, 1.0),
    ([700, 31, 32, 33], 2, 8, 128, 32, "fp8_e4m3", True, 0.37, 1.9),
    ([600, 5], 2, 1, 128, 32, "bf16", True, 1.0, 1.0),
]


def run_all_pins():
    """Every pin, at the sizes used by the mutation check."""
    pin_fp8_special_values()
    pin_storage_decode()
    for args in BRUTE_FORCE_SMALL:
        pin_brute_force(*args)
    pin_partition_statistics()
    pin_uniform_closed_form()
    pin_alibi_closed_form()
    pin_single_token()
    pin_partition_size_independence()
    pin_v2_single_partition_equals_v1()
    pin_block_table_permutation()
    pin_convexity_and_dominant_key()
    pin_empty_sequence()
    pin_sliding_window()
    pin_sliding_window(lens=(513, 1100), alibi=False, cap=5.0)
    pin_soft_cap_forms()
    pin_dispatch_golden()
    pin_partition_count_golden()
