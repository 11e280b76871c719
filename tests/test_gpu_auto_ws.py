"""GPU parity of paged_attention_auto_ws (the auto decode scheduled for
balance when the caller gives a counters buffer: the work list or the
balanced split by batch shape): every full-size decode workload and the
kernel families against the fp64 oracle, with and without the decode
options and in both cache layouts; the counters are left at zero, repeated
calls are bitwise stable, and without counters the call is paged_attention_auto."""

import numpy as np
import pytest
import torch

from paged_kv_cache_297_amd import binding as B
from paged_kv_cache_297_amd import workloads as W
from tests import gpu_helpers as H
from tests.test_gpu_window import FAMILIES, _family_id

pytestmark = pytest.mark.gpu

LENS = [0, 1, 17, 511, 513, 1100, 1600, 2100, 3000, 5000, 9000, 700, 20000, 4097]


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()


def _check(wl, window_left=-1, soft_cap=0.0, seqs=None, partials="f32", kv_layout="decode",
           caches=None):
    ref = H.oracle(wl, seqs, window_left=window_left, soft_cap=soft_cap)
    seqs = list(range(wl.num_seqs)) if seqs is None else seqs
    H.say(f"  {wl.name} auto_ws W={window_left} cap={soft_cap} seqs={len(seqs)} {partials} "
          f"{kv_layout}")
    res = H.run(wl, "auto_ws", window_left=window_left, soft_cap=soft_cap, partials=partials,
                kv_layout=kv_layout, caches=caches)
    H.check_against_oracle(wl, res, ref, seqs, "auto_ws", window_left=window_left,
                           soft_cap=soft_cap)
    return res


@pytest.mark.parametrize("fam", FAMILIES, ids=_family_id)
def test_auto_ws_families(fam):
    kv, dt, group, d, bs = fam
    i = FAMILIES.index(fam)
    wl = W.make_workload(2, lens=LENS, H=2 * group, Hkv=2, D=d, bs=bs, dtype=dt, kv=kv,
                         alibi=(i % 2 == 1), seed=9500 + i)
    _check(wl)
    _check(wl, 600, 30.0)


@pytest.mark.parametrize("number", [1, 2, 3, 4, 5])
def test_auto_ws_workloads(number):
    wl = W.make_workload(number)
    seqs = None
    if number == 4:
        # The oracle on the longest, the shortest and two fixed sequences.
        order = np.argsort(wl.lens)
        seqs = sorted(set(order[-3:].tolist() + order[:2].tolist() + [7, 100]))
    elif number in (3, 5):
        seqs = [0, wl.num_seqs - 1]
    _check(wl, seqs=seqs)


def test_auto_ws_block_rows_layout():
    wl = W.make_workload(2, lens=LENS, H=14, Hkv=2, D=128, bs=16, dtype=torch.bfloat16,
                         seed=9600)
    caches = W.to_block_rows(wl.key_cache, wl.value_cache)
    _check(wl, kv_layout="block_rows", caches=caches)


def test_auto_ws_repeated_calls_are_bitwise():
    wl = W.make_workload(2)
    a = H.run(wl, "auto_ws")["out"]
    b = H.run(wl, "auto_ws")["out"]
    assert np.array_equal(a, b, equal_nan=True)


def test_auto_ws_without_counters_is_auto():
    wl = W.make_workload(2, lens=LENS, H=8, Hkv=2, D=128, bs=16, dtype=torch.bfloat16, seed=9700)
    out, es, ml, to = wl.alloc_outputs()
    args = (wl.query, wl.key_cache, wl.value_cache, wl.num_kv_heads, wl.scale,
            wl.block_tables, wl.seq_lens, wl.block_size, wl.max_seq_len)
    B.paged_attention_auto_ws(out, es, ml, to, None, *args)
    torch.cuda.synchronize()
    ref = H.run(wl, "auto")
    assert np.array_equal(out.float().cpu().numpy(), ref["out"], equal_nan=True)
