"""GPU parity of the decode options (sliding window, logit soft cap): the HIP
path through the *_ex entry points against the fp64 oracle's reading of the
dispatch page's window_left / softcap fields, on every kernel family, on the
full-size decode workloads, and on the properties the reading fixes exactly:
a window that covers the sequence changes nothing, keys before the window
are never read (stale block-table entries, NaN in the first block), and the
auto rule sees the window-clipped length."""

import ctypes
import dataclasses

import numpy as np
import pytest
import torch

from paged_kv_cache_297_amd import binding as B
from paged_kv_cache_297_amd import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

PART = W.PARTITION_SIZE


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()


def _check(wl, paths, window_left, soft_cap, seqs=None):
    ref = H.oracle(wl, seqs, window_left=window_left, soft_cap=soft_cap)
    seqs = list(range(wl.num_seqs)) if seqs is None else seqs
    for path in paths:
        H.say(f"  {wl.name} path={path} W={window_left} cap={soft_cap} seqs={len(seqs)}")
        res = H.run(wl, path, window_left=window_left, soft_cap=soft_cap)
        H.check_against_oracle(wl, res, ref, seqs, path, window_left=window_left,
                               soft_cap=soft_cap)


# --------------------------------------------------------------------------
# Every kernel family, windows around block and partition edges, caps
# --------------------------------------------------------------------------

#: (kv cache, dtype, query heads per KV head, head size, block size): VALU
#: f32 / 16-bit / fp8 and MFMA 16-bit / fp8 instances.
FAMILIES = [
    ("auto", torch.float32, 1, 64, 16),
    ("auto", torch.float32, 4, 128, 32),
    ("auto", torch.bfloat16, 2, 128, 16),
    ("auto", torch.float16, 3, 64, 32),
    ("auto", torch.float16, 8, 64, 32),
    ("auto", torch.bfloat16, 16, 128, 16),
    ("fp8_e4m3", torch.bfloat16, 3, 128, 16),
    ("fp8_e4m3", torch.float16, 8, 128, 32),
    ("fp8_e4m3", torch.bfloat16, 6, 64, 16),
]

LENS = [0, 1, 16, 17, 100, 511, 512, 513, 700, 1100, 1600, 2100]

#: (window_left, soft cap): W = 0 keeps the last key alone; 15 / 16 / 31 /
#: 32 straddle block edges, 511 / 512 / 513 partition edges; -1 with a cap
#: is the cap alone; 5000 covers every sequence.
OPTIONS = [(0, 0.0), (1, 30.0), (15, 0.0), (16, 5.0), (31, 0.0), (32, 30.0), (100, 0.0),
           (511, 30.0), (512, 0.0), (513, 50.0), (1500, 0.0), (-1, 30.0), (-1, 5.0),
           (5000, 5.0)]


def _family_id(f):
    kv, dt, g, d, bs = f
    return f"{kv}-{str(dt).split('.')[-1]}-G{g}-D{d}-bs{bs}"


@pytest.mark.parametrize("fam", FAMILIES, ids=_family_id)
def test_window_and_cap_matrix(fam):
    kv, dt, group, d, bs = fam
    i = FAMILIES.index(fam)
    hkv = 2
    wl = W.make_workload(2, lens=LENS, H=hkv * group, Hkv=hkv, D=d, bs=bs, dtype=dt, kv=kv,
                         alibi=(i % 2 == 0), seed=7000 + i)
    for w_left, cap in OPTIONS:
        _check(wl, ["v1", "v2", "auto"], w_left, cap)


# --------------------------------------------------------------------------
# Exact properties
# --------------------------------------------------------------------------

def _bitwise_equal(a, b, what):
    for key in a:
        x, y = a[key], b[key]
        same = np.array_equal(x, y, equal_nan=True)
        assert same, f"{what}: {key} differs (max |diff| {np.nanmax(np.abs(x - y)):.3e})"


@pytest.mark.parametrize("fam", [FAMILIES[0], FAMILIES[3], FAMILIES[5], FAMILIES[7]],
                         ids=_family_id)
def test_window_covering_the_sequence_is_no_window(fam):
    """W >= L - 1 for every sequence: bitwise the plain call (v1, v2, auto)."""
    kv, dt, group, d, bs = fam
    wl = W.make_workload(2, lens=LENS, H=2 * group, Hkv=2, D=d, bs=bs, dtype=dt, kv=kv,
                         alibi=True, seed=7100)
    for path in ("v1", "v2", "auto"):
        plain = H.run(wl, path)
        for w_left in (wl.max_seq_len - 1, wl.max_seq_len, 2 ** 31 - 1):
            H.say(f"  {wl.name} path={path} W={w_left}")
            _bitwise_equal(H.run(wl, path, window_left=w_left), plain, f"{path} W={w_left}")


def test_ex_with_null_or_off_options_is_the_plain_call():
    wl = W.make_workload(2, lens=LENS, H=8, Hkv=2, D=128, bs=16, dtype=torch.bfloat16,
                         alibi=True, seed=7200)
    lib = B.load_library()
    for mode in ("v2", "auto"):
        plain = H.run(wl, mode)
        for opts in (None, B.DecodeOptions(-1, 0.0)):
            out, es, ml, to = wl.alloc_outputs()
            for t in (out, es, ml, to):
                t.fill_(float("nan"))
            args = B._v2_args(out, es, ml, to, wl.query, wl.key_cache, wl.value_cache,
                              wl.num_kv_heads, wl.scale, wl.block_tables, wl.seq_lens,
                              wl.block_size, wl.max_seq_len, wl.alibi_slopes, "auto", 1.0, 1.0,
                              None)
            ptr = None if opts is None else ctypes.addressof(opts)
            st = getattr(lib, f"paged_attention_{mode}_ex")(*args[:-1], ptr, args[-1])
            assert st == B.PA_OK
            torch.cuda.synchronize()
            got = {"out": out.float().cpu().numpy(), "exp_sums": es.cpu().numpy(),
                   "max_logits": ml.cpu().numpy(), "tmp_out": to.float().cpu().numpy()}
            want = {k: plain[k].astype(np.float32) for k in got}
            _bitwise_equal(got, want, f"{mode}_ex opts={opts}")


def _stale_tables(wl, window_left):
    """The block table with every entry of a block wholly before the window
    replaced by an index outside [0, num_blocks)."""
    tables = wl.block_tables.clone()
    nb = wl.key_cache.shape[0]
    host = tables.cpu()
    for s, L in enumerate(wl.lens.tolist()):
        lo = H.window_first_token(int(L), window_left) if L > 0 else 0
        for j in range(lo // wl.block_size):
            host[s, j] = -1 if j % 2 == 0 else nb + 7
    return host.to(tables.device)


@pytest.mark.parametrize("fam", FAMILIES, ids=_family_id)
def test_blocks_before_the_window_are_not_read(fam):
    """Stale (out-of-range) table entries before the window: a read would
    make the head NaN; the result is bitwise the one with the real table."""
    kv, dt, group, d, bs = fam
    wl = W.make_workload(2, lens=LENS, H=2 * group, Hkv=2, D=d, bs=bs, dtype=dt, kv=kv,
                         alibi=False, seed=7300)
    for w_left in (0, 40, 600):
        stale = _stale_tables(wl, w_left)
        for path in ("v1", "v2", "auto"):
            H.say(f"  {wl.name} path={path} W={w_left} stale entries")
            clean = H.run(wl, path, window_left=w_left)
            got = H.run(wl, path, window_left=w_left, block_tables=stale)
            assert np.isfinite(got["out"]).all()
            _bitwise_equal(got, clean, f"{path} W={w_left}")


def _nan_before_window(wl, window_left):
    """A copy of the workload whose K and V of the keys before the window,
    in the block holding the window's first key, are NaN."""
    kc, vc = wl.key_cache.clone(), wl.value_cache.clone()
    nan = 0x7F if wl.kv_cache_dtype == "fp8_e4m3" else float("nan")
    tables = wl.block_tables.cpu()
    for s, L in enumerate(wl.lens.tolist()):
        if L == 0:
            continue
        lo = H.window_first_token(int(L), window_left)
        if lo % wl.block_size == 0:
            continue
        phys = int(tables[s, lo // wl.block_size])
        kc[phys, :, :, :lo % wl.block_size, :] = nan
        vc[phys, :, :, :lo % wl.block_size] = nan
    return dataclasses.replace(wl, key_cache=kc, value_cache=vc)


@pytest.mark.parametrize("fam", FAMILIES, ids=_family_id)
def test_keys_before_the_window_carry_no_weight(fam):
    """NaN keys and values just before the window (same block as its first
    key): masked, so the result is bitwise the clean one."""
    kv, dt, group, d, bs = fam
    wl = W.make_workload(2, lens=LENS, H=2 * group, Hkv=2, D=d, bs=bs, dtype=dt, kv=kv,
                         alibi=True, seed=7400)
    for w_left, cap in ((5, 0.0), (100, 30.0), (530, 0.0)):
        dirty = _nan_before_window(wl, w_left)
        for path in ("v1", "v2"):
            H.say(f"  {wl.name} path={path} W={w_left} NaN before the window")
            clean = H.run(wl, path, window_left=w_left, soft_cap=cap)
            got = H.run(dirty, path, window_left=w_left, soft_cap=cap)
            _bitwise_equal(got, clean, f"{path} W={w_left}")


def test_partitions_before_the_window():
    """v2: a partition with no key in the window stores max_logit -inf,
    exp_sum 0 and leaves its tmp_out row alone; one partition in the window
    writes out from Phase 1 already."""
    wl = W.make_workload(2, lens=[2100, 1030, 600], H=8, Hkv=2, D=128, bs=16,
                         dtype=torch.bfloat16, seed=7500)
    w_left = 600
    res = H.run(wl, "v2", window_left=w_left)
    for s, L in enumerate(wl.lens.tolist()):
        lo = H.window_first_token(L, w_left) // PART
        n = (L + PART - 1) // PART
        assert np.all(np.isneginf(res["max_logits"][s, :, :lo]))
        assert np.all(res["exp_sums"][s, :, :lo] == 0.0)
        assert np.all(np.isnan(res["tmp_out"][s, :, :lo]))    # poison kept
        assert np.all(np.isfinite(res["max_logits"][s, :, lo:n]))
        assert np.all(np.isneginf(res["max_logits"][s, :, n:]))
    ref = H.oracle(wl, window_left=w_left)
    H.check_against_oracle(wl, res, ref, range(wl.num_seqs), "v2", window_left=w_left)


def test_two_phase_ex_is_v2_ex():
    """partition_ex(V2) then reduce_ex with the same options == v2_ex, bitwise."""
    wl = W.make_workload(4, lens=[3000, 700, 1, 5000], H=8, Hkv=8, D=128, bs=16,
                         dtype=torch.bfloat16, seed=7600)
    for w_left, cap in ((1200, 30.0), (-1, 30.0), (0, 0.0)):
        whole = H.run(wl, "v2", window_left=w_left, soft_cap=cap)
        out, es, ml, to = wl.alloc_outputs()
        for t in (out, es, ml, to):
            t.fill_(float("nan"))
        args = (out, es, ml, to, wl.query, wl.key_cache, wl.value_cache, wl.num_kv_heads,
                wl.scale, wl.block_tables, wl.seq_lens, wl.block_size, wl.max_seq_len)
        B.paged_attention_partition("v2", *args, alibi_slopes=wl.alibi_slopes,
                                    window_left=w_left, logits_soft_cap=cap)
        B.paged_attention_reduce("v2", out, es, ml, to, wl.seq_lens, wl.num_kv_heads,
                                 wl.max_seq_len, window_left=w_left)
        torch.cuda.synchronize()
        got = {"out": out.float().cpu().numpy().astype(np.float64),
               "exp_sums": es.cpu().numpy().astype(np.float64),
               "max_logits": ml.cpu().numpy().astype(np.float64),
               "tmp_out": to.float().cpu().numpy().astype(np.float64)}
        _bitwise_equal(got, whole, f"two-phase W={w_left} cap={cap}")


def test_auto_rule_sees_the_window_clipped_length():
    """A batch that fills the CUs (small-batch clause off).  A window that
    clips the long sequences below the v2 threshold turns the whole call
    into plain v1 (statistics untouched); a wider one keeps the long
    sequences on v2 and the short ones on v1, in one launch."""
    cu = B.device_cu_count()
    hkv = 32
    n = (4 * cu + hkv - 1) // hkv
    thresh = 512 * (2 * cu // hkv)          # v2 iff the clipped length exceeds this
    long_len = thresh + 3000
    lens = [long_len if s % 8 == 0 else 600 + 37 * s for s in range(n)]
    wl = W.make_workload(4, lens=lens, seed=7700)
    sample = [0, 1, 2, 8, n - 1]

    w_v1 = thresh - 1                        # clipped length thresh: v1 everywhere
    assert not any(H.uses_v2(wl, s, w_v1) for s in range(n))
    assert H.uses_v2(wl, 0)                  # without the window: v2
    res = H.run(wl, "auto", window_left=w_v1)
    assert np.all(np.isnan(res["exp_sums"])) and np.all(np.isnan(res["tmp_out"]))
    ref = H.oracle(wl, sample, window_left=w_v1)
    H.check_against_oracle(wl, res, ref, sample, "auto", window_left=w_v1)

    w_mix = thresh + 600                     # long: clipped thresh + 601 -> v2
    assert H.uses_v2(wl, 0, w_mix) and not H.uses_v2(wl, 1, w_mix)
    res = H.run(wl, "auto", window_left=w_mix, soft_cap=30.0)
    assert np.all(np.isnan(res["exp_sums"][1]))   # v1 sequence: statistics untouched
    ref = H.oracle(wl, sample, window_left=w_mix, soft_cap=30.0)
    H.check_against_oracle(wl, res, ref, sample, "auto", window_left=w_mix, soft_cap=30.0)


# --------------------------------------------------------------------------
# Full-size decode workloads with the options on
# --------------------------------------------------------------------------

def test_gqa_bf16_window_cap():
    wl = W.make_workload(2)
    _check(wl, ["auto", "v2", "v1"], 1023, 50.0)


def test_long_fp16_window():
    wl = W.make_workload(3)
    _check(wl, ["v2", "auto", "v1"], 8191, 0.0, seqs=[0, 3])


def test_ragged_alibi_window_cap():
    wl = W.make_workload(4)
    order = np.argsort(wl.lens)
    seqs = sorted(set(order[-3:].tolist() + order[:2].tolist() + [7, 100]))
    _check(wl, ["auto", "v2"], 1000, 30.0, seqs=seqs)


def test_fp8_kv_window_cap():
    wl = W.make_workload(5)
    _check(wl, ["auto", "v2"], 4095, 30.0, seqs=[0, 31])
