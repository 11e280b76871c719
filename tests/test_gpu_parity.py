"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same bytes, on the five decode workloads (full size; the oracle checks every
sequence where it finishes in seconds and a sample elsewhere) and on a matrix
of small ragged cases covering every kernel instance family."""

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
    B.load_library()  # raises if the HIP library is not built


def _run_and_check(wl, paths, seqs=None):
    ref = H.oracle(wl, seqs)
    seqs = list(range(wl.num_seqs)) if seqs is None else seqs
    for path in paths:
        H.say(f"  {wl.name} path={path} seqs={len(seqs)}")
        res = H.run(wl, path)
        H.check_against_oracle(wl, res, ref, seqs, path)


def test_tiny_fp32():
    wl = W.make_workload(1)
    _run_and_check(wl, ["v1", "v2", "auto"])


def test_gqa_bf16_full():
    wl = W.make_workload(2)
    _run_and_check(wl, ["v2", "auto", "v1"])


def test_long_fp16():
    wl = W.make_workload(3)
    _run_and_check(wl, ["v2", "auto", "v1"], seqs=[0, 3])


def test_ragged_alibi_bf16():
    wl = W.make_workload(4)
    order = np.argsort(wl.lens)
    rng = np.random.default_rng(4)
    seqs = sorted(set(order[-3:].tolist() + order[:2].tolist()
                      + rng.choice(wl.num_seqs, 4, replace=False).tolist()))
    _run_and_check(wl, ["auto", "v2", "v1"], seqs=seqs)


def test_fp8_kv():
    wl = W.make_workload(5)
    _run_and_check(wl, ["v2", "auto"], seqs=[0, 31])


# --------------------------------------------------------------------------
# Small ragged cases over the kernel families
# --------------------------------------------------------------------------

RAGGED = [1, 15, 16, 17, 31, 33, 511, 512, 513, 1025, 1600]

MATRIX = []
for kv, dt in (("auto", torch.float32), ("auto", torch.float16), ("auto", torch.bfloat16),
               ("fp8_e4m3", torch.bfloat16), ("fp8_e4m3", torch.float16)):
    for group in (1, 2, 3, 4, 7, 8, 16):
        for d in (64, 128):
            for bs in (16, 32):
                MATRIX.append((kv, dt, group, d, bs))


def _matrix_id(case):
    kv, dt, group, d, bs = case
    return f"{kv}-{str(dt).split('.')[-1]}-G{group}-D{d}-bs{bs}"


@pytest.mark.parametrize("case", MATRIX, ids=_matrix_id)
def test_kernel_matrix(case):
    kv, dt, group, d, bs = case
    hkv = 2
    i = MATRIX.index(case)
    wl = W.make_workload(2, lens=RAGGED, H=hkv * group, Hkv=hkv, D=d, bs=bs, dtype=dt, kv=kv,
                         alibi=(i % 3 == 0), seed=5000 + i)
    _run_and_check(wl, ["v2", "v1"])


def test_auto_mixed_dispatch_small():
    """A batch large enough that AUTO sends short sequences down v1 and long
    ones down v2 in the same launch."""
    cu = B.device_cu_count()
    hkv = 32
    n = (4 * cu + hkv - 1) // hkv          # small-batch clause off
    long_len = 512 * (2 * cu // hkv + 1)   # Hkv * partitions > 2 * CUs
    lens = [long_len if s % 8 == 0 else 600 + 37 * s for s in range(n)]
    wl = W.make_workload(4, lens=lens)
    assert H.uses_v2(wl, 0) and not H.uses_v2(wl, 1)
    _run_and_check(wl, ["auto"], seqs=[0, 1, 2, 8, n - 1])


@pytest.mark.parametrize("number,group,alibi", [(4, 1, True), (2, 8, False)],
                         ids=["valu-alibi", "mfma"])
def test_many_partitions(number, group, alibi):
    """A 262221-key sequence (513 partitions: the reduce merges them over
    several rounds; the split path caps it at 64 pieces) next to a short one,
    on the VALU and the MFMA kernel, with ALiBi slopes on positions up to
    2.6e5 for the first."""
    lens = [262221, 1000]
    wl = W.make_workload(number, lens=lens, H=group, Hkv=1, D=128, bs=16, alibi=alibi,
                         seed=9100 + group)
    assert wl.max_num_partitions == 513
    _run_and_check(wl, ["v2", "auto", "split"])
