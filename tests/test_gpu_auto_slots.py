"""GPU parity of auto's persistent slot form (paged_attention_auto on batches
with many (sequence, KV head) items on the narrow-group kernel): piece j of
an item stores its partials in partition slot j, the slots past the last
piece padded, and the reduce kernel merges every sequence of two or more
partitions.  Checked against the fp64 oracle on lengths around the partition
boundaries (cut and whole items, one-partition items, empty and invalid
lengths), for the kernel families that take it, with ALiBi and a soft cap,
against the v2 path, and bitwise over repeats."""

import numpy as np
import pytest
import torch

from paged_kv_cache_297_amd import binding as B
from paged_kv_cache_297_amd import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()


#: Lengths that put partition boundaries, one-partition items and long items
#: next to one another; the rest of the batch is drawn (1 .. 3000).
EDGE = [1, 2, 511, 512, 513, 1023, 1024, 1025, 1536, 2047, 2048, 2049, 2560, 3000, 0, 4096]


def _batch(number, heads, seed, **over):
    """A workload of family ``number`` with enough items for the slot form
    (at least 2 x 4 per CU), the lengths above and one sequence long enough
    that the auto rule does not run the whole batch as plain v1 (KV heads x
    its partitions > 2 x CUs)."""
    cu = B.device_cu_count()
    hkv = over.get("Hkv", heads)
    n = max(len(EDGE) + 1, -(-2 * 4 * cu // heads))
    rng = np.random.default_rng(seed)
    lens = EDGE + [512 * (2 * cu // hkv + 2) + 17]
    lens += [int(x) for x in rng.integers(1, 3001, size=n - len(lens))]
    rng.shuffle(lens)
    return W.make_workload(number, lens=lens, seed=seed, **over)


FAMILIES = [
    ("bf16-alibi-D128", 4, 32, dict(H=32, Hkv=32)),
    ("f16-D128-bs16", 3, 16, dict(H=32, Hkv=16)),                              # G = 2
    ("bf16-D64-bs32", 4, 16, dict(H=64, Hkv=16, D=64, bs=32, alibi=False)),   # G = 4
    ("fp8-D128-bs32", 5, 16, dict(H=16, Hkv=16)),                              # G = 1, fp8
    ("f32-D64", 1, 8, dict(H=16, Hkv=8)),                                      # G = 2, fp32
]


@pytest.mark.parametrize("name,number,heads,over", FAMILIES, ids=[f[0] for f in FAMILIES])
def test_slot_form_matches_oracle(name, number, heads, over):
    wl = _batch(number, heads, 7000 + [f[0] for f in FAMILIES].index(name), **over)
    assert H.auto_slots(wl), f"{name}: the batch should take the slot form"
    H.say(f"  slots {name}: B={wl.num_seqs} H={wl.num_heads} Hkv={wl.num_kv_heads}")
    res = H.run(wl, "auto")
    ref = H.oracle(wl)
    H.check_against_oracle(wl, res, ref, range(wl.num_seqs), "auto")
    for s in np.flatnonzero(wl.lens == 0):
        assert np.all(res["out"][s] == 0.0)


def test_slot_form_with_soft_cap_and_against_v2():
    wl = _batch(4, 32, 7100, H=32, Hkv=32)
    assert H.auto_slots(wl, soft_cap=30.0)
    got = H.run(wl, "auto", soft_cap=30.0)
    ref = H.oracle(wl, soft_cap=30.0)
    H.check_against_oracle(wl, got, ref, range(wl.num_seqs), "auto", soft_cap=30.0)
    a = H.run(wl, "auto")["out"]
    v2 = H.run(wl, "v2")["out"]
    H.check_close(a, v2, H.TOL[wl.kv_kind], "slot form vs v2")


def test_slot_form_repeat_is_bitwise_and_partials_dtype():
    wl = _batch(4, 32, 7200, H=32, Hkv=32)
    a = H.run(wl, "auto")["out"]
    b = H.run(wl, "auto")["out"]
    assert np.array_equal(a, b)
    c = H.run(wl, "auto", partials="out")
    H.check_against_oracle(wl, c, H.oracle(wl), range(wl.num_seqs), "auto")


def test_slot_form_invalid_length_gives_nan():
    wl = _batch(4, 32, 7300, H=32, Hkv=32)
    bad = wl.seq_lens.clone()
    long_seq = int(np.argmax(wl.lens))
    picks = [s for s in range(wl.num_seqs) if s != long_seq][:2]
    bad[picks[0]] = wl.max_seq_len + 5
    bad[picks[1]] = -1
    res = H.run(W.Workload(**{**wl.__dict__, "seq_lens": bad}), "auto")
    assert np.all(np.isnan(res["out"][picks[0]])) and np.all(np.isnan(res["out"][picks[1]]))
    keep = [s for s in range(wl.num_seqs) if s not in picks]
    assert np.all(np.isfinite(res["out"][keep]))


def test_not_taken_with_window_or_few_items():
    wl = _batch(4, 32, 7400, H=32, Hkv=32)
    assert not H.auto_slots(wl, window_left=1000)
    small = W.make_workload(4, num_seqs=8, seed=7401)
    assert not H.auto_slots(small)


# --------------------------------------------------------------------------
# Seeded random batches large enough for the slot form: kernel families
# (dtype, fp8 cache, head group 1 / 2 / 4, head size, block size), ragged
# lengths with partition-boundary values, empty sequences, ALiBi, a soft cap
# and NaN-poisoned unused cache slots, against the oracle on every sequence.
# --------------------------------------------------------------------------

RANDOM_CASES = 8
RANDOM_KINDS = {"bf16": (torch.bfloat16, "auto"), "f16": (torch.float16, "auto"),
                "f32": (torch.float32, "auto"), "fp8-bf16": (torch.bfloat16, "fp8_e4m3")}


def _draw(case: int) -> dict:
    rng = np.random.default_rng(40000 + case)
    kind = str(rng.choice(sorted(RANDOM_KINDS)))
    group = int(rng.choice([1, 2, 4]))
    hkv = int(rng.choice([8, 16, 32]))
    return dict(kind=kind, group=group, hkv=hkv, d=int(rng.choice([64, 128])),
                bs=int(rng.choice([16, 32])), alibi=bool(rng.random() < 0.4),
                cap=float(rng.choice([0.0, 0.0, 20.0])), poison=bool(case % 2),
                seed=int(rng.integers(1 << 30)))


def _draw_id(case: int) -> str:
    c = _draw(case)
    return f"{case}-{c['kind']}-G{c['group']}x{c['hkv']}-D{c['d']}-bs{c['bs']}"


@pytest.mark.parametrize("case", range(RANDOM_CASES), ids=_draw_id)
def test_slot_form_random(case):
    c = _draw(case)
    dtype, kv = RANDOM_KINDS[c["kind"]]
    cu = B.device_cu_count()
    rng = np.random.default_rng(c["seed"])
    n = -(-2 * 4 * cu // c["hkv"])
    lens = []
    for _ in range(n):
        r = rng.random()
        if r < 0.05:
            lens.append(0)
        elif r < 0.3:
            lens.append(int(512 * rng.integers(1, 8) + rng.integers(-1, 2)))
        else:
            lens.append(int(rng.integers(1, 4000)))
    lens[int(rng.integers(n))] = 512 * (2 * cu // c["hkv"] + 2) + int(rng.integers(0, 512))
    wl = W.make_workload(2, lens=lens, H=c["hkv"] * c["group"], Hkv=c["hkv"], D=c["d"],
                         bs=c["bs"], dtype=dtype, kv=kv, alibi=c["alibi"], seed=c["seed"] % 100000,
                         poison=c["poison"])
    assert H.auto_slots(wl, soft_cap=c["cap"]), _draw_id(case)
    H.say(f"  slot form random {_draw_id(case)} B={wl.num_seqs} cap={c['cap']} alibi={c['alibi']}")
    res = H.run(wl, "auto", soft_cap=c["cap"])
    ref = H.oracle(wl, soft_cap=c["cap"])
    H.check_against_oracle(wl, res, ref, range(wl.num_seqs), "auto", soft_cap=c["cap"])
