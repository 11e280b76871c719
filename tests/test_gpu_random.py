"""Seeded random decode configurations against the fp64 oracle.

Each case draws its storage kind (fp32, fp16, bf16, fp8 E4M3FN under a bf16 or
fp16 query), query heads per KV head, KV heads, head size, block size, a
ragged batch of lengths (empty sequences, partition edges, short and long
ones), ALiBi, a sliding window, a logit soft cap, the cache layout and the
path (v1, v2, auto, split), and checks every output the path defines against
the oracle on the same bytes; a second sweep draws larger batches for the
scheduled paths (work list, auto_ws).  Odd cases are NaN-poisoned: unused block-table
entries point at an all-NaN block and the slots past each sequence's end hold
NaN, which no output may see.  The draws are seeded, so every case is the
same on every run."""

import numpy as np
import pytest
import torch

from paged_kv_cache_297_amd import binding as B
from paged_kv_cache_297_amd import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

CASES = 64

KINDS = {
    "f32": (torch.float32, "auto"),
    "f16": (torch.float16, "auto"),
    "bf16": (torch.bfloat16, "auto"),
    "fp8-bf16": (torch.bfloat16, "fp8_e4m3"),
    "fp8-f16": (torch.float16, "fp8_e4m3"),
}


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()


def _draw(case: int) -> dict:
    rng = np.random.default_rng(20000 + case)
    kind = str(rng.choice(list(KINDS)))
    n = int(rng.integers(1, 9))
    lens = []
    for _ in range(n):
        r = rng.random()
        if r < 0.1:
            lens.append(0)
        elif r < 0.35:
            lens.append(int(512 * rng.integers(1, 6) + rng.integers(-1, 2)))  # partition edges
        elif r < 0.6:
            lens.append(int(rng.integers(1, 64)))
        else:
            lens.append(int(rng.integers(64, 3500)))
    if max(lens) == 0:
        lens[0] = 777
    sixteen = kind in ("f16", "bf16")
    return dict(
        kind=kind,
        lens=lens,
        group=int(rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16])),
        hkv=int(rng.choice([1, 2, 4])),
        d=int(rng.choice([64, 128])),
        bs=int(rng.choice([16, 32])),
        alibi=bool(rng.random() < 0.3),
        window=int(rng.choice([-1, -1, -1, 0, 31, 700, 2000])),
        cap=float(rng.choice([0.0, 0.0, 0.0, 5.0, 30.0])),
        layout="block_rows" if sixteen and rng.random() < 0.35 else "decode",
        path=str(rng.choice(["v1", "v2", "auto", "split"])),
        poison=bool(case % 2),
    )


def _case_id(case: int) -> str:
    c = _draw(case)
    return (f"{case}-{c['kind']}-G{c['group']}x{c['hkv']}-D{c['d']}-bs{c['bs']}-"
            f"{c['layout']}-{c['path']}")


@pytest.mark.parametrize("case", range(CASES), ids=_case_id)
def test_random_config(case):
    c = _draw(case)
    dtype, kv = KINDS[c["kind"]]
    wl = W.make_workload(2, lens=c["lens"], H=c["hkv"] * c["group"], Hkv=c["hkv"], D=c["d"],
                         bs=c["bs"], dtype=dtype, kv=kv, alibi=c["alibi"], seed=21000 + case,
                         poison=c["poison"])
    caches = W.to_block_rows(wl.key_cache, wl.value_cache) if c["layout"] == "block_rows" else None
    H.say(f"  random case {_case_id(case)} lens={c['lens']} W={c['window']} cap={c['cap']} "
          f"alibi={c['alibi']}")
    res = H.run(wl, c["path"], window_left=c["window"], soft_cap=c["cap"], caches=caches,
                kv_layout=c["layout"])
    ref = H.oracle(wl, window_left=c["window"], soft_cap=c["cap"])
    H.check_against_oracle(wl, res, ref, range(wl.num_seqs), c["path"],
                           window_left=c["window"], soft_cap=c["cap"])


# --------------------------------------------------------------------------
# The scheduled paths (work list, and auto_ws, which takes the work list or
# the balanced split by batch shape) over larger ragged batches, so that
# items are cut into pieces that different workers merge.
# --------------------------------------------------------------------------

SCHED_CASES = 40


def _draw_sched(case: int) -> dict:
    rng = np.random.default_rng(30000 + case)
    kind = str(rng.choice(list(KINDS)))
    n = int(rng.integers(1, 41))
    lens = []
    for _ in range(n):
        r = rng.random()
        if r < 0.08:
            lens.append(0)
        elif r < 0.3:
            lens.append(int(512 * rng.integers(1, 12) + rng.integers(-1, 2)))
        elif r < 0.45:
            lens.append(int(rng.integers(1, 64)))
        else:
            lens.append(int(rng.integers(64, 9000)))
    if max(lens) == 0:
        lens[0] = 4321
    sixteen = kind in ("f16", "bf16")
    path = str(rng.choice(["worklist", "auto_ws"]))
    return dict(
        kind=kind,
        lens=lens,
        group=int(rng.choice([1, 2, 4, 5, 7, 8, 16])),
        hkv=int(rng.choice([1, 2, 4, 8])),
        d=int(rng.choice([64, 128])),
        bs=int(rng.choice([16, 32])),
        alibi=bool(rng.random() < 0.3),
        window=int(rng.choice([-1, -1, -1, 700, 3000])),
        cap=float(rng.choice([0.0, 0.0, 0.0, 5.0, 30.0])),
        layout="block_rows" if sixteen and path == "auto_ws" and rng.random() < 0.3 else "decode",
        path=path,
        poison=bool(case % 2),
    )


def _sched_id(case: int) -> str:
    c = _draw_sched(case)
    return (f"{case}-{c['kind']}-B{len(c['lens'])}-G{c['group']}x{c['hkv']}-D{c['d']}-"
            f"bs{c['bs']}-{c['layout']}-{c['path']}")


@pytest.mark.parametrize("case", range(SCHED_CASES), ids=_sched_id)
def test_random_scheduled(case):
    c = _draw_sched(case)
    dtype, kv = KINDS[c["kind"]]
    wl = W.make_workload(2, lens=c["lens"], H=c["hkv"] * c["group"], Hkv=c["hkv"], D=c["d"],
                         bs=c["bs"], dtype=dtype, kv=kv, alibi=c["alibi"], seed=31000 + case,
                         poison=c["poison"])
    caches = W.to_block_rows(wl.key_cache, wl.value_cache) if c["layout"] == "block_rows" else None
    H.say(f"  scheduled case {_sched_id(case)} W={c['window']} cap={c['cap']} alibi={c['alibi']}")
    res = H.run(wl, c["path"], window_left=c["window"], soft_cap=c["cap"], caches=caches,
                kv_layout=c["layout"])
    ref = H.oracle(wl, window_left=c["window"], soft_cap=c["cap"])
    H.check_against_oracle(wl, res, ref, range(wl.num_seqs), c["path"],
                           window_left=c["window"], soft_cap=c["cap"])
